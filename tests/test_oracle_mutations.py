"""Plants plausible mistakes into copies of the oracle's C source, on the CPU,
and checks that the pin tests catch every one of them.

Each mutant is a small textual change (a dropped term, a wrong sign, index
or constant, a swapped rounding rule; a list of edits where one mistake spans
two lines).  It is compiled with the oracle's own
flags into a temporary library, every oracle call is routed through it, and
the battery below -- a subset of the pin tests, run unchanged -- must report
at least one failure.  The unmodified source must pass the same battery.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild

import test_oracle_attention as ta
import test_oracle_codecs as tc
import test_oracle_norm_rope as tn
import test_oracle_quant as tq

MUTANTS = {
    "kmean_divides_by_padded_rows": ("total[d] / (float)N", "total[d] / (float)(T * BK)"),
    "kmean_drops_last_tile": ("for (int64_t j = 0; j < T; ++j) {\n                int64_t n_end",
                              "for (int64_t j = 0; j < T - 1; ++j) {\n                int64_t n_end"),
    "kquant_no_mean_subtraction": ("float kc = in_val(K, sb, sn, sh, b, (int)n, h, d) - mean[d];\n                        float m",
                                   "float kc = in_val(K, sb, sn, sh, b, (int)n, h, d);\n                        float m"),
    "int8_truncates": ("float r = rintf(y);", "float r = truncf(y);"),
    "int8_inverse_uses_128": ("        *sc = a / 127.0f;\n                float inv = 127.0f / a;\n                for (int64_t n",
                              "        *sc = a / 127.0f;\n                float inv = 128.0f / a;\n                for (int64_t n"),
    "qgroup_128_rows": ("q_scale[bh * G + r / QG]", "q_scale[bh * G + (r / BQ) * 4]"),
    "kscale_wrong_tile": ("k_scale[bh * T + j]", "k_scale[bh * T + (j > 0 ? j - 1 : 0)]"),
    "vscale_fnuz_240": ("inv[d] = 448.0f / a[d];", "inv[d] = 240.0f / a[d];"),
    "e4m3_ties_odd": ("code = (lo % 2 == 0) ? lo : hi;", "code = (lo % 2 == 0) ? hi : lo;"),
    "e4m3_no_midpoint_round": ("if (a < midpoint)", "if (a < e4m3_pos[hi])"),
    "missing_log2e": ("const float c = sm_scale * log2e;", "const float c = sm_scale;"),
    "alpha_sign": ("float alpha = exp2f(m - m_new);", "float alpha = exp2f(m_new - m);"),
    "d_not_rescaled": ("dsum = dsum * alpha;", "dsum = dsum * 1.0f;"),
    "ro_not_rescaled": ("RO[e] = RO[e] * alpha;", "RO[e] = RO[e] * 1.0f;"),
    "p_unscaled": ("p[cc] = 448.0f * exp2f(x);", "p[cc] = exp2f(x);"),
    "no_tail_mask": [("if (j * BK + cc < N) {\n                    float x", "if (1) {\n                    float x"),
                     ("                if (n < N) {\n                    const int8_t* k",
                      "                if (1) {\n                    const int8_t* k")],
    "d_sums_fp8": ("dsum = dsum + p[cc];", "dsum = dsum + oracle_e4m3_decode(oracle_e4m3_encode(p[cc]));"),
    "pv_wrong_key_row": ("vdec[v8[(bh * Nk + n) * HD + e]]", "vdec[v8[(bh * Nk + j * BK) * HD + e]]"),
    "pv_transposed": ("vdec[v8[(bh * Nk + n) * HD + e]]", "vdec[v8[(bh * Nk + j * BK + e % BK) * HD + cc * 2]]"),
    "no_v_scale": ("float o = (RO[e] * rcp) * vs[e];", "float o = (RO[e] * rcp) * vs[0];"),
    "bf16_truncates": ("u += 0x7fffu + lsb;", "u += 0u * lsb;"),
    "norm_divides_by_64": ("float ms = ss / 128.0f;", "float ms = ss / 64.0f;"),
    "norm_no_sqrt": ("float w = sqrtf(t);", "float w = t;"),
    "norm_no_eps": ("float t = ms + eps;", "float t = ms;"),
    "norm_no_weight": ("float xg = xr * g[d];", "float xg = xr;"),
    "norm_sums_abs": ("float sq = x[d] * x[d];", "float sq = fabsf(x[d]);"),
    "norm_not_rounded": ("y[d] = oracle_bf16_to_f32(oracle_f32_to_bf16(xg));", "y[d] = xg;"),
    "rope_sign": ("o[i] = oracle_f32_to_bf16(ac - bs);", "o[i] = oracle_f32_to_bf16(ac + bs);"),
    "rope_pairs_mirror": ("float ac = y[i] * c, bs = y[i + HD / 2] * s;", "float ac = y[i] * c, bs = y[HD - 1 - i] * s;"),
    "rope_first_token_row": ("const float* crow = cs + (int64_t)n * (HD / 2);", "const float* crow = cs;"),
    "rope_cos_sin_swapped": ("float c = crow[i], s = srow[i];", "float c = srow[i], s = crow[i];"),
    "qk_skips_last_dim": ("for (int d = 0; d < HD; ++d)\n                        s += (int32_t)q[d] * (int32_t)k[d];\n                    t[cc]",
                          "for (int d = 0; d < HD - 1; ++d)\n                        s += (int32_t)q[d] * (int32_t)k[d];\n                    t[cc]"),
}


def _battery():
    """(name, callable) pairs, each taking the oracle module."""
    return [
        ("codec_torch", tc.test_e4m3_encode_matches_torch_rne),
        ("codec_ties", tc.test_e4m3_ties_go_to_even_code),
        ("bf16_torch", tc.test_bf16_encode_matches_torch),
        ("kmean_f64_200", lambda o: tq.test_k_mean_close_to_float64(o, 200)),
        ("kmean_shift", lambda o: tq.test_k_mean_exact_shift(o, 64)),
        ("kquant_tiny", lambda o: tq.test_k_quant_range_grouping_and_error(o, "tiny")),
        ("kquant_ties", tq.test_k_quant_ties_to_even),
        ("qquant_tiny", lambda o: tq.test_q_quant_range_grouping_and_error(o, "tiny")),
        ("qquant_ties", tq.test_q_quant_ties_to_even),
        ("vquant_tiny", lambda o: tq.test_v_quant_range_grouping_and_error(o, "tiny")),
        ("f64_tiny", lambda o: ta.test_oracle_close_to_float64_tile_boundaries(o, 200)),
        ("f64_n65", lambda o: ta.test_oracle_close_to_float64_tile_boundaries(o, 65)),
        ("f64_n256", lambda o: ta.test_oracle_close_to_float64_tile_boundaries(o, 256)),
        ("v_ones", lambda o: ta.test_v_ones_rows_sum_to_one(o, 200)),
        ("q_zero", ta.test_q_zero_gives_mean_of_dequantized_v),
        ("dominant_key", ta.test_one_dominant_key),
        ("small_weights", ta.test_small_weights_survive_fp8),
        ("qk_s32", lambda o: ta.test_qk_s32_matches_int64_matmul(o, "tiny")),
        ("nr_pow2", tn.test_power_of_two_rows_give_the_weight),
        ("nr_eps", tn.test_large_epsilon_on_tiny_rows),
        ("nr_turns", tn.test_quarter_and_half_turns),
        ("nr_angles", tn.test_random_angles_against_float64_rotation),
        ("nr_f64", lambda o: tn.test_against_float64_rmsnorm_and_rotation(o, 1e-6)),
        ("nr_rounded", tn.test_normalised_row_is_rounded_before_rotation),
    ]


def _run_battery():
    failed = []
    for name, fn in _battery():
        try:
            fn(oracle)
        except AssertionError:
            failed.append(name)
    return failed


def _build_variant(src_text: str, out_dir: str, tag: str) -> str:
    src = os.path.join(out_dir, tag + ".c")
    lib = os.path.join(out_dir, "lib" + tag + ".so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *obuild.CFLAGS, src, "-o", lib, "-lm"], check=True)
    return lib


@pytest.fixture(scope="module")
def source_text():
    with open(obuild.SRC) as f:
        return f.read()


def test_unmodified_source_passes_battery(source_text, tmp_path):
    lib = _build_variant(source_text, str(tmp_path), "clean")
    with oracle.use_library(lib):
        assert _run_battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(source_text, tmp_path, name):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    mutated = source_text
    for old, new in edits:
        assert mutated.count(old) >= 1, "mutation anchor not found: %s" % name
        mutated = mutated.replace(old, new, 1)
    lib = _build_variant(mutated, str(tmp_path), name)
    with oracle.use_library(lib):
        failed = _run_battery()
    assert failed, "planted mistake %s passed every pin" % name
