"""Pins for the oracle's optional step 0: per-head RMSNorm of Q/K rows, then
split-half rotary embedding ("Sage2 Blackwell Mainloop", Completed P1 And P2).

What pins it (none of these re-types the oracle's formulas):
  * rows of +-2^k: every binary32 step is exact, so the output is +-weight;
  * a large epsilon on tiny rows leaves r = 1, so the output is bf16(x * w);
  * power-of-two scaling of a row leaves the output unchanged;
  * rotation by a quarter and a half turn (cos, sin in {0, +-1}) moves and
    negates channels exactly, and channel i pairs with i + 64;
  * per-token, per-frequency random angles against a float64 rotation of the
    oracle's own normalised row, within the binary32 and BF16 rounding bound
    (pins the table row/column and the signs);
  * the whole step against float64 RMSNorm + rotation within two BF16 steps;
  * a constructed row where rounding the normalised row to BF16 before the
    rotation changes the result (pins that rounding).
"""
import numpy as np
import pytest
import torch

import workloads

HD = 128


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _bits_of(x):
    """BF16 bit patterns of a float array (values already BF16-representable)."""
    return _bf16(np.asarray(x, np.float32)).view(torch.int16).numpy().view(np.uint16)


def _weights(seed):
    g = torch.Generator().manual_seed(seed)
    return _bf16(1.0 + 0.3 * torch.randn(HD, generator=g)).to(torch.float32).numpy()


def _tables(N, c, s):
    return np.full((N, HD // 2), c, np.float32), np.full((N, HD // 2), s, np.float32)


def test_power_of_two_rows_give_the_weight(oracle_mod):
    rng = np.random.default_rng(1)
    N, H = 7, 3
    k = rng.integers(-6, 7, size=(1, N, H, 1)).astype(np.float64)
    signs = rng.choice([-1.0, 1.0], size=(1, N, H, HD))
    x = _bf16(signs * 2.0 ** k)
    g = _weights(2)
    cos, sin = _tables(N, 1.0, 0.0)
    out = oracle_mod.norm_rope(x, g, cos, sin, 2.0 ** -60)
    assert np.array_equal(out, _bits_of(signs * g[None, None, None, :]))


def test_large_epsilon_on_tiny_rows(oracle_mod):
    g = torch.Generator().manual_seed(3)
    x = _bf16(torch.randn(1, 5, 2, HD, generator=g) * 2.0 ** -30)
    w = _weights(4)
    cos, sin = _tables(5, 1.0, 0.0)
    out = oracle_mod.norm_rope(x, w, cos, sin, 1.0)
    xf = x.to(torch.float32).numpy()
    expect = oracle_mod.bf16_encode(xf * w).reshape(xf.shape)   # r = 1 exactly
    assert np.array_equal(out, expect)


def test_power_of_two_scaling_invariance(oracle_mod):
    inp = workloads.generate(workloads.Workload("t", 1, 70, 3, seed=11))
    p = workloads.norm_rope_params(70)
    base = oracle_mod.norm_rope(inp.q, p.q_weight, p.cos, p.sin, 1e-30)
    for e in (-8, 3, 20):
        scaled = (inp.q.to(torch.float32) * 2.0 ** e).to(torch.bfloat16)
        assert np.array_equal(oracle_mod.norm_rope(scaled, p.q_weight, p.cos, p.sin, 1e-30), base)


def test_quarter_and_half_turns(oracle_mod):
    inp = workloads.generate(workloads.Workload("t", 2, 33, 2, seed=12))
    w = _weights(5)
    y = oracle_mod.bf16_decode(oracle_mod.norm_rope(inp.k, w, *_tables(33, 1.0, 0.0), 1e-6))
    q = oracle_mod.bf16_decode(oracle_mod.norm_rope(inp.k, w, *_tables(33, 0.0, 1.0), 1e-6))
    assert np.array_equal(q[..., :64], -y[..., 64:])
    assert np.array_equal(q[..., 64:], y[..., :64])
    hneg = oracle_mod.bf16_decode(oracle_mod.norm_rope(inp.k, w, *_tables(33, -1.0, 0.0), 1e-6))
    assert np.array_equal(hneg, -y)


def test_random_angles_against_float64_rotation(oracle_mod):
    N = 50
    inp = workloads.generate(workloads.Workload("t", 1, N, 4, seed=13))
    w = _weights(6)
    rng = np.random.default_rng(7)
    ang = rng.uniform(-np.pi, np.pi, size=(N, HD // 2))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    y = oracle_mod.bf16_decode(oracle_mod.norm_rope(inp.q, w, *_tables(N, 1.0, 0.0), 1e-6)).astype(np.float64)
    o = oracle_mod.bf16_decode(oracle_mod.norm_rope(inp.q, w, cos, sin, 1e-6)).astype(np.float64)
    c = cos.astype(np.float64)[None, :, None, :]
    s = sin.astype(np.float64)[None, :, None, :]
    a, b = y[..., :64], y[..., 64:]
    ref = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    mag = np.concatenate([np.abs(a * c) + np.abs(b * s), np.abs(b * c) + np.abs(a * s)], axis=-1)
    bound = mag * 2.0 ** -23 + np.abs(ref) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(o - ref) <= bound)


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_against_float64_rmsnorm_and_rotation(oracle_mod, eps):
    N = 64
    inp = workloads.generate(workloads.Workload("t", 1, N, 3, seed=14))
    p = workloads.norm_rope_params(N)
    o = oracle_mod.bf16_decode(oracle_mod.norm_rope(inp.k, p.k_weight, p.cos, p.sin, eps)).astype(np.float64)
    x = inp.k.to(torch.float64).numpy()
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    y = x * r * p.k_weight.double().numpy()
    c = p.cos.double().numpy()[None, :, None, :]
    s = p.sin.double().numpy()[None, :, None, :]
    a, b = y[..., :64], y[..., 64:]
    ref = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    mag = np.concatenate([np.abs(a * c) + np.abs(b * s), np.abs(b * c) + np.abs(a * s)], axis=-1)
    assert np.all(np.abs(o - ref) <= mag * 2.0 ** -7 + 1e-30)


def test_normalised_row_is_rounded_before_rotation(oracle_mod):
    # Every |x| = 1, so ss = 128 and r = 1 exactly.  Weight 1 + 2^-9 on channel 0
    # gives an unrounded y_0 = 1 + 2^-9, which BF16 rounds to 1; weight 2^-8 on
    # channel 64 gives y_64 = 2^-8.  With c = 1, s = -1: rounded first,
    # o_0 = bf16(1 + 2^-8) = 1 (tie to even); unrounded it would be
    # bf16(1 + 3 * 2^-9) = 1 + 2^-7.  Likewise o_64 = bf16(2^-8 - y_0) is
    # -(1 - 2^-8) when rounded first, and -1 (a tie, to even) when not.
    x = _bf16(np.ones((1, 1, 1, HD)))
    w = np.ones(HD, np.float32)
    w[0] = np.float32(1.0 + 2.0 ** -9)
    w[64] = np.float32(2.0 ** -8)
    cos, sin = _tables(1, 1.0, -1.0)
    o = oracle_mod.bf16_decode(oracle_mod.norm_rope(x, w, cos, sin, 2.0 ** -60))
    assert o[0, 0, 0, 0] == 1.0
    assert o[0, 0, 0, 64] == -(1.0 - 2.0 ** -8)
