"""Pins for the oracle's number codecs (BF16 and OCP FP8 E4M3FN).

Each codec is pinned against an independent implementation (PyTorch's CPU
casts, a library routine) and against closed-form facts of the formats.
"""
import numpy as np
import pytest
import torch


def _e4m3_values_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_e4m3_decode_all_codes_match_torch(oracle_mod):
    ours = oracle_mod.e4m3_decode(np.arange(256))
    ref = _e4m3_values_torch()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert set(np.nonzero(nan_ours)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours].view(np.uint32), ref[~nan_ours].view(np.uint32))


def test_e4m3_closed_form_facts(oracle_mod):
    v = oracle_mod.e4m3_decode(np.arange(256))
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite magnitude
    assert v[0x01] == 2.0 ** -9                              # smallest subnormal
    assert v[0x08] == 2.0 ** -6                              # smallest normal
    assert v[0x38] == 1.0                                    # exponent bias 7
    assert np.all(np.diff(v[:127]) > 0)                      # monotone on 0x00..0x7E
    assert np.signbit(v[0x80]) and v[0x80] == 0.0            # negative zero


def test_e4m3_roundtrip_all_finite_codes(oracle_mod):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle_mod.e4m3_decode(codes)
    assert np.array_equal(oracle_mod.e4m3_encode(vals), codes)


def _midpoints_and_neighbours():
    pos = _e4m3_values_torch()[:127].astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)     # exact in binary32
    xs = [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
          pos.astype(np.float32)]
    xs = np.concatenate(xs)
    return np.concatenate([xs, -xs])


def test_e4m3_encode_matches_torch_rne(oracle_mod):
    rng = np.random.default_rng(7)
    rand_bits = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    rand = rand_bits.view(np.float32)
    rand = rand[np.isfinite(rand) & (np.abs(rand) < 464.0)]
    uni = rng.uniform(-463.9, 463.9, size=200_000).astype(np.float32)
    tiny = (rng.uniform(-1, 1, size=100_000) * 2.0 ** -6).astype(np.float32)
    x = np.concatenate([_midpoints_and_neighbours(), rand, uni, tiny,
                        np.array([0.0, -0.0], np.float32)])
    ours = oracle_mod.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, "first mismatches: %s" % [(float(x[i]), int(ours[i]), int(ref[i])) for i in bad[:5]]


def test_e4m3_ties_go_to_even_code(oracle_mod):
    pos = oracle_mod.e4m3_decode(np.arange(127)).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    codes = oracle_mod.e4m3_encode(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect.astype(np.uint8))


def test_e4m3_saturates_and_nan(oracle_mod):
    x = np.array([448.0, 460.0, 464.0, 470.0, 1e6, np.inf, -1e6, -np.inf, np.nan], np.float32)
    assert oracle_mod.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]


def test_bf16_encode_matches_torch(oracle_mod):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=500_000, dtype=np.uint64).astype(np.uint32)
    bits[::3] = (bits[::3] & 0xFFFF0000) | 0x8000          # exact ties
    bits[1::7] = (bits[1::7] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = oracle_mod.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_exact(oracle_mod):
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))
