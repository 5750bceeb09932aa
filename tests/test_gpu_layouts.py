"""GPU parity on seeded random shapes and memory layouts.

Each case draws B (1..3), H (1..6) and N (1..520, so one to nine 64-key
tiles with any ragged tail; every fourth case below 70) and places Q, K, V and the output independently in one of three
memory layouts behind the same [B, N, H, 128] view: token-major (contiguous
NHD), head-major (contiguous BHND, seen through a permuted view) and pitched
(token and head strides with gaps, every gap filled with a large value that
would show in the result if it were read).  The oracle gets the same values
as contiguous CPU tensors, so the comparison also checks the kernels' stride
handling.  Two-call cases check every quantized byte and scale bit for bit;
all cases compare every output row at the output bar of the parity suite.
"""
import sys

import numpy as np
import pytest
import torch

import layouts

pytestmark = pytest.mark.gpu

HD = 128
MAX_ABS = 2e-2
MIN_COS = 0.9999
MIN_BIT_EQUAL = 0.95
GAP_FILL = 30000.0
CASES = 12


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_exact_attention_amd as s
    s._load()
    return s


def _draw_values(rng_seed, B, N, H):
    """Q, V ~ N(0,1); K ~ N(0,1) plus a per-(head, channel) offset 3*N(0,1)."""
    g = torch.Generator(device="cpu").manual_seed(rng_seed)
    shape = (B, N, H, HD)
    q = torch.randn(shape, generator=g).to(torch.bfloat16)
    k = (torch.randn(shape, generator=g) + 3.0 * torch.randn((H, HD), generator=g)).to(torch.bfloat16)
    v = torch.randn(shape, generator=g).to(torch.bfloat16)
    return q, k, v


class _Placed:
    """A [B, N, H, 128] view in a chosen memory layout: the backing buffer on
    the CPU and the geometry to view it on any device."""

    def __init__(self, kind, shape, rng):
        B, N, H, D = shape
        self.kind = kind
        self.size = shape
        if kind == "nhd":
            self.stride = (N * H * D, H * D, D, 1)
            self.offset = 0
            numel = B * N * H * D
        elif kind == "hnd":
            self.stride = (H * N * D, D, N * D, 1)
            self.offset = 0
            numel = B * H * N * D
        else:  # pitched: gaps between heads, between tokens and between batch entries
            sh = D + 8 * int(rng.integers(0, 3))
            sn = H * sh + 8 * int(rng.integers(1, 5))
            sb = N * sn + 8 * int(rng.integers(0, 3))
            self.stride = (sb, sn, sh, 1)
            self.offset = 8 * int(rng.integers(0, 4))
            numel = self.offset + B * sb
        self.buf = torch.full((numel,), GAP_FILL, dtype=torch.bfloat16)

    def view(self, device="cpu"):
        base = self.buf if device == "cpu" else self.buf.to(device)
        self.base = base
        return torch.as_strided(base, self.size, self.stride, self.offset)


def _case(i):
    rng = np.random.default_rng(9000 + i)
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 7))
    N = int(rng.integers(1, 521)) if i % 4 else int(rng.integers(1, 70))
    kinds = [str(x) for x in rng.choice(["nhd", "hnd", "pitched"], size=4)]
    sm_scale = None if i % 3 == 0 else float(rng.uniform(0.03, 0.4))
    two_call = i % 2 == 1
    return rng, B, N, H, kinds, sm_scale, two_call


@pytest.mark.parametrize("i", range(CASES))
def test_seeded_shapes_and_layouts(sage, i):
    import oracle
    rng, B, N, H, kinds, sm_scale, two_call = _case(i)
    _log("layout case %d: B=%d N=%d H=%d q/k/v/o=%s sm_scale=%s %s"
         % (i, B, N, H, "/".join(kinds), sm_scale, "two-call" if two_call else "one-call"))
    q, k, v = _draw_values(100 + i, B, N, H)
    placed = [_Placed(kind, (B, N, H, HD), rng) for kind in kinds]
    for p, x in zip(placed[:3], (q, k, v)):
        p.view().copy_(x)
    qg, kg, vg, og = (p.view("cuda") for p in placed)
    if two_call:
        qz = sage.quantize_qkv(qg, kg, vg)
        sage.attn_fwd_quantized(qz, sm_scale=sm_scale, out=og)
    else:
        sage.attn_fwd(qg, kg, vg, sm_scale=sm_scale, out=og)
    torch.cuda.synchronize()

    ref = oracle.quantize(q, k, v)
    if two_call:
        assert np.array_equal(qz.k_mean.cpu().numpy().view(np.uint32), ref.k_mean.view(np.uint32))
        assert np.array_equal(qz.q_scale.cpu().numpy().view(np.uint32), ref.q_scale.view(np.uint32))
        assert np.array_equal(qz.k_scale.cpu().numpy().view(np.uint32), ref.k_scale.view(np.uint32))
        assert np.array_equal(qz.v_scale.cpu().numpy().view(np.uint32), ref.v_scale.view(np.uint32))
        assert np.array_equal(layouts.q_logical(qz.q_i8.cpu().numpy(), B, H, N), ref.q_i8)
        assert np.array_equal(layouts.k_logical(qz.k_i8.cpu().numpy(), B, H, N), ref.k_i8)
        assert np.array_equal(layouts.v_logical(qz.v_fp8.cpu().numpy(), B, H, N), ref.v8)

    bb, hh, rr = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), rr.ravel()], axis=1)
    ref_bits, _ = oracle.attn_rows(ref, rows, sm_scale)
    out = og.cpu()                                   # the strided view, element by element
    got_bits = out.view(torch.int16).numpy().view(np.uint16)[rows[:, 0], rows[:, 2], rows[:, 1]]
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = (ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    max_abs = float(np.max(np.abs(got - want)))
    cos = float(got.ravel() @ want.ravel() / (np.linalg.norm(got) * np.linalg.norm(want)))
    exact = float(np.mean(got_bits == ref_bits))
    _log("layout case %d: max_abs=%.3g cos=%.7f bit-equal=%.3f" % (i, max_abs, cos, exact))
    assert max_abs <= MAX_ABS
    assert cos >= MIN_COS
    assert exact >= MIN_BIT_EQUAL

    # the output's gaps are untouched
    if kinds[3] == "pitched":
        whole = placed[3].base.cpu()
        mask = torch.ones(whole.numel(), dtype=torch.bool)
        idx = torch.as_strided(torch.arange(whole.numel()), og.shape, og.stride(), og.storage_offset())
        mask[idx.reshape(-1)] = False
        assert torch.all(whole[mask] == GAP_FILL)
