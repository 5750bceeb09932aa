"""Pins for the oracle's attention (per-tile online softmax, FP8 PV, epilogue).

  * reference64 (unquantized float64 attention) is itself pinned to PyTorch's
    scaled_dot_product_attention in float64 and to softmax invariants.
  * The oracle must stay close to reference64 (cosine >= 0.999 and a small
    relative error) on the small workloads and every tile-boundary length.
  * Closed forms: V == 1 gives rows of weights summing to 1; Q == 0 gives the
    plain mean of the dequantized V; one dominant key gives that key's V row.
  * Exact shift invariance from K-mean subtraction on grid data; padding
    independence; determinism; int32 QK sums against an int64 matmul.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import reference64

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _dec_bits(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# -------------------------------------------------------- reference64 pins --

def test_reference64_matches_torch_sdpa():
    inp = workloads.generate(workloads.sweep(129))
    ours = reference64.attention64(inp.q, inp.k, inp.v, SM)
    q, k, v = (t.to(torch.float64).permute(0, 2, 1, 3).contiguous() for t in (inp.q, inp.k, inp.v))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=SM)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_reference64_invariants():
    inp = workloads.generate(workloads.tiny())
    q = inp.q.to(torch.float64).numpy()
    k = inp.k.to(torch.float64).numpy()
    w = reference64.softmax_weights(q[0, 3, 1], k[0, :, 1], SM)
    assert abs(w.sum() - 1.0) < 1e-12 and np.all(w > 0)
    base = reference64.attention64(inp.q, inp.k, inp.v, SM)
    shifted = reference64.attention64(inp.q, torch.as_tensor(k + 5.0 * np.arange(128) / 128.0), inp.v, SM)
    assert np.max(np.abs(base - shifted)) < 1e-12


# ------------------------------------------------ oracle vs float64 answer --

def _check_close_to_f64(oracle_mod, inp, rows_per_head=None, seed=0):
    qz = oracle_mod.quantize(inp.q, inp.k, inp.v)
    B, N, H = qz.B, qz.N, qz.H
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        for h in range(H):
            rr = np.arange(N) if rows_per_head is None else np.sort(rng.choice(N, rows_per_head, replace=False))
            rows += [(b, h, r) for r in rr]
    rows = np.array(rows)
    bits, _ = oracle_mod.attn_rows(qz, rows, SM)
    got = _dec_bits(bits).astype(np.float64)
    q = inp.q.to(torch.float64).numpy()
    k = inp.k.to(torch.float64).numpy()
    v = inp.v.to(torch.float64).numpy()
    ref = np.stack([reference64.softmax_weights(q[b, r, h], k[b, :, h], SM) @ v[b, :, h] for b, h, r in rows])
    cos = _cos(got, ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    return cos, rel


@pytest.mark.parametrize("n", list(workloads.SWEEP_NS) + [200])
def test_oracle_close_to_float64_tile_boundaries(oracle_mod, n):
    w = workloads.tiny() if n == 200 else workloads.sweep(n)
    cos, rel = _check_close_to_f64(oracle_mod, workloads.generate(w))
    assert cos >= 0.999, cos
    assert rel <= 0.045, rel


def test_oracle_close_to_float64_mid(oracle_mod):
    # The 1% outlier K channels (x8) set each 64-row K scale, so the other
    # channels quantize with a coarser step: the method itself loses accuracy
    # here (measured cosine 0.9982).  The same shape without outliers must
    # reach the 0.999 bar, which shows the loss comes from the outliers.
    cos, rel = _check_close_to_f64(oracle_mod, workloads.generate(workloads.mid()), rows_per_head=96, seed=1)
    assert cos >= 0.997, cos
    assert rel <= 0.07, rel
    plain = workloads.Workload("mid_no_outliers", 1, 4096, 8, seed=1)
    cos, rel = _check_close_to_f64(oracle_mod, workloads.generate(plain), rows_per_head=96, seed=1)
    assert cos >= 0.999, cos
    assert rel <= 0.045, rel


# ------------------------------------------------------------ closed forms --

@pytest.mark.parametrize("n", [200, 256])
def test_v_ones_rows_sum_to_one(oracle_mod, n):
    w = workloads.Workload("v1", 1, n, 2, seed=31)
    inp = workloads.generate(w)
    v = torch.ones_like(inp.v)
    qz, bits, _ = oracle_mod.attention(inp.q, inp.k, v, SM)
    assert np.all(qz.v8[:, :, :n] == 0x7E) and np.all(qz.v_scale == np.float32(1.0) / np.float32(448.0))
    o = _dec_bits(bits).astype(np.float64)
    bound = 2.0 ** -4 + n * 2.0 ** -10 / 448.0 + 2.0 ** -8
    assert np.max(np.abs(o - 1.0)) <= bound
    assert abs(np.mean(o) - 1.0) < 2.0 ** -7
    # d sums the FP32 probabilities while PV uses their FP8 codes, so the
    # rows are not all exactly 1 (they would be if d summed the FP8 codes)
    assert np.mean(o != 1.0) > 0.2


def test_q_zero_gives_mean_of_dequantized_v(oracle_mod):
    w = workloads.Workload("q0", 1, 300, 2, seed=32)
    inp = workloads.generate(w)
    q = torch.zeros_like(inp.q)
    qz, bits, f32 = oracle_mod.attention(q, inp.k, inp.v, SM)
    assert np.all(qz.q_scale == 0)
    dec = oracle_mod.e4m3_decode(qz.v8.ravel()).reshape(qz.v8.shape).astype(np.float64)
    mean = dec[:, :, :300].mean(axis=2) * qz.v_scale.astype(np.float64)          # [B,H,D]
    o = _dec_bits(bits).astype(np.float64)                                          # [B,N,H,D]
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(mean), 1e-30))) - 7)
    assert np.all(np.abs(o - mean[:, None]) <= 2 * ulp[:, None] + 1e-30)


def test_one_dominant_key(oracle_mod):
    g = torch.Generator().manual_seed(33)
    n, nstar = 150, 97
    k = torch.randn((1, n, 1, 128), generator=g)
    v = torch.randn((1, n, 1, 128), generator=g)
    q = torch.randn((1, n, 1, 128), generator=g) * 0.05
    q[0, 10, 0] = 8.0 * k[0, nstar, 0]
    qz, bits, f32 = oracle_mod.attention(_bf16(q), _bf16(k), _bf16(v), SM)
    dec = oracle_mod.e4m3_decode(qz.v8[0, 0, nstar]).astype(np.float64) * qz.v_scale[0, 0]
    o = _dec_bits(bits[0, 10, 0]).astype(np.float64)
    assert np.all(np.abs(o - dec) <= np.abs(dec) * 2.0 ** -8 + 1e-6)


def test_small_weights_survive_fp8(oracle_mod):
    # Key 0 dominates the others by about 12 in log2 units, so each other key
    # has weight ~2^-12.  Carried at x448, those probabilities are normal E4M3
    # numbers (~0.11); unscaled they would round to zero.  V is 0 on key 0 and
    # 1 elsewhere, so the output is exactly the mass of the small weights.
    n = 64
    k = torch.zeros((1, n, 1, 128))
    k[0, 0, 0, 0] = 4.0
    q = torch.zeros((1, n, 1, 128))
    q[0, :, 0, 0] = 23.5
    v = torch.ones((1, n, 1, 128))
    v[0, 0] = 0.0
    qz, bits, _ = oracle_mod.attention(_bf16(q), _bf16(k), _bf16(v), SM)
    got = _dec_bits(bits).astype(np.float64)
    ref = reference64.attention64(_bf16(q), _bf16(k), _bf16(v), SM)
    assert 0.01 < ref[0, 0, 0, 0] < 0.03
    assert np.all(np.abs(got - ref) <= 0.08 * ref)


def test_exact_shift_invariance_on_grid(oracle_mod):
    g = torch.Generator().manual_seed(34)
    n = 128
    k = torch.randint(-64, 65, (1, n, 2, 128), generator=g).to(torch.float32) / 16.0
    q = torch.randn((1, n, 2, 128), generator=g)
    v = torch.randn((1, n, 2, 128), generator=g)
    c = torch.randint(-4, 5, (2, 128), generator=g).to(torch.float32)
    _, b0, _ = oracle_mod.attention(_bf16(q), _bf16(k), _bf16(v), SM)
    _, b1, _ = oracle_mod.attention(_bf16(q), _bf16(k + c), _bf16(v), SM)
    assert np.array_equal(b0, b1)


def test_general_shift_changes_output_by_rounding_only(oracle_mod):
    inp = workloads.generate(workloads.sweep(192))
    k2 = (inp.k.to(torch.float32) + 1.5).to(torch.bfloat16)
    _, b0, _ = oracle_mod.attention(inp.q, inp.k, inp.v, SM)
    _, b1, _ = oracle_mod.attention(inp.q, k2, inp.v, SM)
    assert _cos(_dec_bits(b0), _dec_bits(b1)) > 0.999


# ---------------------------------------------------- structural properties --

def test_padding_independence_and_determinism(oracle_mod):
    inp = workloads.generate(workloads.sweep(129))
    q2 = workloads.with_padding_rows(inp.q, 30)
    k2 = workloads.with_padding_rows(inp.k, 30, fill_seed=1)
    v2 = workloads.with_padding_rows(inp.v, 30, fill_seed=2)
    _, a, _ = oracle_mod.attention(inp.q, inp.k, inp.v, SM)
    _, b, _ = oracle_mod.attention(q2, k2, v2, SM)
    _, c, _ = oracle_mod.attention(inp.q, inp.k, inp.v, SM)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_rows_subset_matches_full(oracle_mod):
    inp = workloads.generate(workloads.tiny())
    qz, full, _ = oracle_mod.attention(inp.q, inp.k, inp.v, SM)
    rows = np.array([(0, 1, 199), (0, 0, 0), (0, 1, 64), (0, 0, 131)])
    bits, _ = oracle_mod.attn_rows(qz, rows, SM)
    for i, (b, h, r) in enumerate(rows):
        assert np.array_equal(bits[i], full[b, r, h])


@pytest.mark.parametrize("name", ["tiny", "sweep_n65", "sweep_n129"])
def test_qk_s32_matches_int64_matmul(oracle_mod, name):
    inp = workloads.generate(workloads.by_name(name))
    qz = oracle_mod.quantize(inp.q, inp.k, inp.v)
    s = oracle_mod.qk_s32(qz)
    ref = np.einsum("bhqd,bhkd->bhqk", qz.q_i8.astype(np.int64), qz.k_i8.astype(np.int64))
    assert np.array_equal(s.astype(np.int64), ref)
    assert np.abs(ref).max() < 2 ** 24


def test_sm_scale_enters_scores(oracle_mod):
    inp = workloads.generate(workloads.sweep(64))
    qz = oracle_mod.quantize(inp.q, inp.k, inp.v)
    rows = np.array([(0, 0, 5), (0, 2, 40)])
    a, _ = oracle_mod.attn_rows(qz, rows, SM)
    b, _ = oracle_mod.attn_rows(qz, rows, 0.25 * SM)
    assert not np.array_equal(a, b)
    # a huge scale makes the row one-hot on its arg-max key
    c, _ = oracle_mod.attn_rows(qz, rows, 1e4)
    s = oracle_mod.qk_s32(qz, 0, 64)
    for i, (b_, h, r) in enumerate(rows):
        logits = s[b_, h, r, :64].astype(np.float64) * qz.k_scale[b_, h, 0]
        n_star = int(np.argmax(logits))
        dec = oracle_mod.e4m3_decode(qz.v8[b_, h, n_star]).astype(np.float64) * qz.v_scale[b_, h]
        assert np.all(np.abs(_dec_bits(c[i]) - dec) <= np.abs(dec) * 2.0 ** -8 + 1e-6)
