"""Pins for the oracle's prepass steps: K mean, Q/K INT8 and V FP8 quantization.

What pins each step (none of these re-types the oracle's formulas):
  * K mean: float64 mean within the summation error bound; an exact shift
    test on grid-valued data where every binary32 operation is exact.
  * INT8 Q/K: the code range is attained in every group of the stated size
    (and not in every smaller sub-block, which pins the grouping); the
    reconstruction error is at most half a quantization step; exact
    power-of-two scaling invariance; ties go to even (vs torch.round);
    zero and padded groups; padding and stride independence.
  * FP8 V: 448 attained per channel over all rows (and not in every tile,
    which pins per-channel-over-N); relative reconstruction error within half
    an E4M3 step; power-of-two invariance; zero channels.
"""
import numpy as np
import pytest
import torch

import workloads


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _f64(x):
    return x.to(torch.float64).numpy()


# ------------------------------------------------------------------ K mean --

@pytest.mark.parametrize("n", [1, 63, 64, 65, 200, 1000])
def test_k_mean_close_to_float64(oracle_mod, n):
    w = workloads.Workload("t", 1, n, 3, seed=40 + n)
    inp = workloads.generate(w)
    km = oracle_mod.k_mean(inp.k)
    k64 = _f64(inp.k)
    ref = k64.mean(axis=1)                                   # [B,H,D]
    T = -(-n // 64)
    bound = (n + T + 2) * 2.0 ** -24 * np.abs(k64).sum(axis=1) / n + np.abs(ref) * 2.0 ** -23
    assert np.all(np.abs(km - ref) <= bound)


def _grid_k(n, h, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randint(-128, 129, (1, n, h, 128), generator=g).to(torch.float32) / 16.0   # [-8, 8] step 1/16
    return k


@pytest.mark.parametrize("n", [64, 128, 256])
def test_k_mean_exact_shift(oracle_mod, n):
    k = _grid_k(n, 2, seed=n)
    g = torch.Generator().manual_seed(99)
    c = torch.randint(-4, 5, (2, 128), generator=g).to(torch.float32)
    km0 = oracle_mod.k_mean(_bf16(k))
    km1 = oracle_mod.k_mean(_bf16(k + c))
    assert np.array_equal(km1, km0 + c.numpy()[None])
    # on grid data every step is exact, so the mean equals the float64 mean
    assert np.array_equal(km0.astype(np.float64), k.to(torch.float64).numpy().mean(axis=1))
    qk0 = oracle_mod.quant_k(_bf16(k), km0)
    qk1 = oracle_mod.quant_k(_bf16(k + c), km1)
    assert np.array_equal(qk0[0], qk1[0]) and np.array_equal(qk0[1], qk1[1])


# ------------------------------------------------------------ INT8 K quant --

def _kc64(k_bf16, km):
    return _f64(k_bf16) - km[:, None, :, :].astype(np.float64)  # [B,N,H,D]


@pytest.mark.parametrize("name", ["tiny", "sweep_n65", "sweep_n129", "mid"])
def test_k_quant_range_grouping_and_error(oracle_mod, name):
    w = workloads.by_name(name)
    inp = workloads.generate(w)
    km = oracle_mod.k_mean(inp.k)
    k_i8, k_scale = oracle_mod.quant_k(inp.k, km)
    B, N, H = w.B, w.N, w.H
    T = -(-N // 64)
    assert k_i8.shape == (B, H, T * 64, 128) and k_scale.shape == (B, H, T)
    kc = _kc64(inp.k, km)
    codes = k_i8.astype(np.int32)
    half_max = []
    for b in range(B):
        for h in range(H):
            for j in range(T):
                rows = slice(64 * j, min(64 * j + 64, N))
                blk = codes[b, h, 64 * j:64 * j + 64]
                assert np.abs(blk).max() == 127                         # range attained per 64-row tile
                assert np.all(blk[rows.stop - 64 * j:] == 0)            # padded rows are zero
                for hh in range(2):
                    part = blk[32 * hh:32 * hh + 32][: max(0, rows.stop - 64 * j - 32 * hh)]
                    if part.size:
                        half_max.append(np.abs(part).max())
                x = kc[b, rows, h, :]
                s = np.float64(k_scale[b, h, j])
                err = np.abs(x - blk[:rows.stop - 64 * j] * s)
                assert np.all(err <= s * (0.5 + 2.0 ** -20) + np.abs(x) * 2.0 ** -23)
    # grouping is per 64 rows, not per 32: some 32-row half does not reach 127
    assert min(half_max) < 127


def test_k_quant_power_of_two_invariance(oracle_mod):
    inp = workloads.generate(workloads.tiny())
    km = oracle_mod.k_mean(inp.k)
    c0, s0 = oracle_mod.quant_k(inp.k, km)
    for e in (-3, 5):
        k2 = (inp.k.to(torch.float32) * 2.0 ** e).to(torch.bfloat16)
        km2 = oracle_mod.k_mean(k2)
        assert np.array_equal(km2, km * np.float32(2.0 ** e))
        c2, s2 = oracle_mod.quant_k(k2, km2)
        assert np.array_equal(c0, c2)
        assert np.array_equal(s2, s0 * np.float32(2.0 ** e))


def test_k_quant_ties_to_even(oracle_mod):
    # channel values are +-(integer + 1/2) in mirrored row pairs, so the mean
    # is exactly 0; one element is 127, so scale = 1 and codes = rne(value).
    g = torch.Generator().manual_seed(5)
    half = torch.randint(-126, 126, (1, 32, 1, 128), generator=g).to(torch.float32) + 0.5
    k = torch.cat([half, -half], dim=1)
    k[0, 0, 0, 0] = 127.0
    k[0, 32, 0, 0] = -127.0
    km = oracle_mod.k_mean(_bf16(k))
    assert np.all(km == 0)
    codes, scale = oracle_mod.quant_k(_bf16(k), km)
    assert scale[0, 0, 0] == 1.0
    ref = torch.round(k).to(torch.int8).numpy()               # round half to even
    assert np.array_equal(codes[0, 0, :64], ref[0, :, 0, :])


def test_k_quant_zero_tile(oracle_mod):
    k = torch.full((1, 64, 1, 128), 0.75)
    k[0, :, 0, 5] = -2.0
    km = oracle_mod.k_mean(_bf16(k))
    codes, scale = oracle_mod.quant_k(_bf16(k), km)
    assert scale[0, 0, 0] == 0.0 and not codes.any()


# ------------------------------------------------------------ INT8 Q quant --

@pytest.mark.parametrize("name", ["tiny", "sweep_n127", "sweep_n129", "mid"])
def test_q_quant_range_grouping_and_error(oracle_mod, name):
    w = workloads.by_name(name)
    inp = workloads.generate(w)
    q_i8, q_scale = oracle_mod.quant_q(inp.q)
    B, N, H = w.B, w.N, w.H
    Nq = -(-N // 128) * 128
    assert q_i8.shape == (B, H, Nq, 128) and q_scale.shape == (B, H, Nq // 32)
    q64 = _f64(inp.q)
    codes = q_i8.astype(np.int32)
    sub_max = []
    for b in range(B):
        for h in range(H):
            for g in range(Nq // 32):
                r0, r1 = 32 * g, min(32 * g + 32, N)
                blk = codes[b, h, 32 * g:32 * g + 32]
                if r0 >= N:
                    assert q_scale[b, h, g] == 0 and not blk.any()      # empty group
                    continue
                assert np.abs(blk).max() == 127
                assert not blk[r1 - r0:].any()
                for qq in range(4):                                      # 8-row sub-blocks
                    part = blk[8 * qq:8 * qq + 8][: max(0, r1 - r0 - 8 * qq)]
                    if part.size:
                        sub_max.append(np.abs(part).max())
                s = np.float64(q_scale[b, h, g])
                x = q64[b, r0:r1, h, :]
                assert np.all(np.abs(x - blk[:r1 - r0] * s) <= s * (0.5 + 2.0 ** -20) + np.abs(x) * 2.0 ** -23)
    assert min(sub_max) < 127


def test_q_quant_grouping_is_32_rows(oracle_mod):
    # a single large value in row 40 must affect only group 1 (rows 32..63)
    g = torch.Generator().manual_seed(8)
    q = torch.randn((1, 128, 1, 128), generator=g)
    q[0, 40, 0, 7] = 50.0
    q_i8, q_scale = oracle_mod.quant_q(_bf16(q))
    assert q_scale[0, 0, 1] == np.float32(50.0) / np.float32(127.0)
    assert q_scale[0, 0, 0] < 0.1 and q_scale[0, 0, 2] < 0.1 and q_scale[0, 0, 3] < 0.1


def test_q_quant_power_of_two_invariance(oracle_mod):
    inp = workloads.generate(workloads.sweep(129))
    c0, s0 = oracle_mod.quant_q(inp.q)
    q2 = (inp.q.to(torch.float32) * 0.125).to(torch.bfloat16)
    c2, s2 = oracle_mod.quant_q(q2)
    assert np.array_equal(c0, c2) and np.array_equal(s2, s0 * np.float32(0.125))


def test_q_quant_ties_to_even(oracle_mod):
    g = torch.Generator().manual_seed(6)
    q = torch.randint(-126, 126, (1, 32, 1, 128), generator=g).to(torch.float32) + 0.5
    q[0, 3, 0, 3] = -127.0
    codes, scale = oracle_mod.quant_q(_bf16(q))
    assert scale[0, 0, 0] == 1.0
    assert np.array_equal(codes[0, 0, :32], torch.round(q).to(torch.int8).numpy()[0, :, 0, :])


def test_q_quant_tiny_group_is_zero(oracle_mod):
    q = torch.zeros((1, 32, 1, 128))
    q[0, 1, 0, 1] = 2.0 ** -110           # below the 2^-100 floor
    codes, scale = oracle_mod.quant_q(_bf16(q))
    assert scale[0, 0, 0] == 0 and not codes.any()
    q[0, 1, 0, 1] = 2.0 ** -90            # above it
    codes, scale = oracle_mod.quant_q(_bf16(q))
    assert codes[0, 0, 1, 1] == 127 and scale[0, 0, 0] == np.float32(2.0 ** -90) / np.float32(127)


# ------------------------------------------------------------- FP8 V quant --

@pytest.mark.parametrize("name", ["tiny", "sweep_n65", "mid"])
def test_v_quant_range_grouping_and_error(oracle_mod, name):
    w = workloads.by_name(name)
    inp = workloads.generate(w)
    v8, v_scale = oracle_mod.quant_v(inp.v)
    B, N, H = w.B, w.N, w.H
    Nk = -(-N // 64) * 64
    assert v8.shape == (B, H, Nk, 128) and v_scale.shape == (B, H, 128)
    dec = oracle_mod.e4m3_decode(v8.ravel()).reshape(v8.shape).astype(np.float64)
    assert not v8[:, :, N:].any()                                          # padded rows 0x00
    amax_dec = np.abs(dec[:, :, :N]).max(axis=2)                           # [B,H,D]
    assert np.all(amax_dec == 448.0)                                       # per channel over all N
    if N > 64:
        tile_max = np.abs(dec[:, :, :64]).max(axis=2)
        assert np.any(tile_max < 448.0)                                    # not per tile
    v64 = np.transpose(_f64(inp.v), (0, 2, 1, 3))                          # [B,H,N,D]
    s = v_scale.astype(np.float64)[:, :, None, :]
    y = v64 / s                                                            # the value being encoded
    rec = dec[:, :, :N] * s
    normal = np.abs(y) >= 2.0 ** -6
    err = np.abs(v64 - rec)
    assert np.all(err[normal] <= (np.abs(v64) * (2.0 ** -4 + 2.0 ** -20))[normal])
    assert np.all(err[~normal] <= (s * (2.0 ** -10 + 2.0 ** -20) + 0 * v64)[~normal])


def test_v_quant_power_of_two_invariance(oracle_mod):
    inp = workloads.generate(workloads.tiny())
    c0, s0 = oracle_mod.quant_v(inp.v)
    v2 = (inp.v.to(torch.float32) * 16.0).to(torch.bfloat16)
    c2, s2 = oracle_mod.quant_v(v2)
    assert np.array_equal(c0, c2) and np.array_equal(s2, s0 * np.float32(16.0))


def test_v_quant_zero_channel_and_sign(oracle_mod):
    g = torch.Generator().manual_seed(11)
    v = torch.randn((1, 70, 1, 128), generator=g)
    v[0, :, 0, 9] = 0.0
    v[0, :, 0, 10] = -0.0
    v8, vs = oracle_mod.quant_v(_bf16(v))
    assert vs[0, 0, 9] == 0 and vs[0, 0, 10] == 0
    assert not v8[0, 0, :, 9].any() and not v8[0, 0, :, 10].any()
    neg = v[0, :, 0, :].numpy() < 0
    assert np.all((v8[0, 0, :70][neg] & 0x80) == 0x80)


# ------------------------------------------------- layout independence pins --

def test_padding_and_stride_independence(oracle_mod):
    w = workloads.Workload("p", 1, 129, 3, seed=21, layout="projection")
    inp = workloads.generate(w)
    q2 = workloads.with_padding_rows(inp.q.contiguous(), 40)
    k2 = workloads.with_padding_rows(inp.k.contiguous(), 40, fill_seed=7)
    v2 = workloads.with_padding_rows(inp.v.contiguous(), 40, fill_seed=8)
    a = oracle_mod.quantize(inp.q, inp.k, inp.v)
    b = oracle_mod.quantize(q2, k2, v2)
    for f in ("k_mean", "q_i8", "q_scale", "k_i8", "k_scale", "v8", "v_scale"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
