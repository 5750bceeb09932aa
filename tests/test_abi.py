"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/sage_mi355x.h declares, sizes and carves workspaces,
and rejects invalid arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import layouts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_mi355x.h")


@pytest.fixture(scope="module")
def sage():
    import quantized_exact_attention_amd as s
    from quantized_exact_attention_amd import build
    build.build(force=False)
    s._load()
    return s


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(sage_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_api():
    names = _declared_functions()
    for n in ("sage_quantize_qkv", "sage_attn_fwd", "sage_attn_fwd_quantized", "sage_workspace_bytes",
              "sage_quantized_carve", "sage_debug_qk_s32"):
        assert n in names


def test_library_exports_every_declared_symbol(sage):
    lib = ctypes.CDLL(sage.library_path())
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert missing == []
    assert sage._load().sage_abi_version() == 3


def test_workspace_bytes(sage):
    assert sage.workspace_bytes(1, 200, 2) > 0
    assert sage.workspace_bytes(0, 200, 2) == 0
    lib = sage._load()
    assert lib.sage_workspace_bytes(sage._Shape(1, 200, 2, 64)) == 0          # D must be 128
    assert lib.sage_workspace_bytes(sage._Shape(1, (1 << 24) + 1, 1, 128)) == 0
    assert lib.sage_workspace_bytes(sage._Shape(1, 1 << 24, 1 << 13, 128)) == 0     # grid of 2^31 tiles
    assert lib.sage_workspace_bytes(sage._Shape(1, 1 << 24, (1 << 13) - 1, 128)) > 0
    # canonical: three quantized tensors plus scales and prepass scratch
    n = sage.workspace_bytes(1, 37810, 56)
    assert 3 * 56 * 37824 * 128 < n < 3 * 56 * 37888 * 128 + 2 * 56 * 591 * 128 * 4 + (1 << 20)


def test_carve_layout(sage):
    lib = sage._load()
    shape = sage._Shape(2, 200, 3, 128)
    need = lib.sage_workspace_bytes(shape)
    qz = sage._Quantized()
    base = 0x7f0000000000                           # never dereferenced: carving is host arithmetic
    assert lib.sage_quantized_carve(shape, base, need, ctypes.byref(qz)) == 0
    ptrs = [qz.q_i8, qz.q_scale, qz.k_i8, qz.k_scale, qz.k_mean, qz.v_fp8, qz.v_scale,
            qz.k_tile_sum, qz.v_tile_amax, qz.v_inv, qz.k_scale_max]
    assert all(p % 256 == 0 for p in ptrs)
    assert ptrs == sorted(ptrs) and ptrs[0] == base
    sizes = [2 * 3 * 256 * 128, 2 * 3 * 8 * 4, 2 * 3 * 256 * 128, 2 * 3 * 4 * 4, 2 * 3 * 128 * 4,
             2 * 3 * 256 * 128, 2 * 3 * 128 * 4, 2 * 3 * 4 * 128 * 4, 2 * 3 * 4 * 128 * 4, 2 * 3 * 128 * 4,
             2 * 3 * 4]
    for p, q, s in zip(ptrs, ptrs[1:] + [base + need], sizes):
        assert q - p >= s                              # regions do not overlap
    assert base + need - ptrs[-1] >= sizes[-1]


def test_carve_rejects(sage):
    lib = sage._load()
    shape = sage._Shape(1, 200, 2, 128)
    need = lib.sage_workspace_bytes(shape)
    qz = sage._Quantized()
    assert lib.sage_quantized_carve(shape, None, need, ctypes.byref(qz)) == 3
    assert lib.sage_quantized_carve(shape, 0x1000 + 16, need, ctypes.byref(qz)) == 3
    assert b"256-byte" in lib.sage_last_error_message()
    assert lib.sage_quantized_carve(shape, 0x1000, need - 1, ctypes.byref(qz)) == 3
    assert lib.sage_quantized_carve(sage._Shape(1, 0, 2, 128), 0x1000, need, ctypes.byref(qz)) == 1
    assert lib.sage_quantized_carve(shape, 0x1000, need, None) == 1


def _carved(sage, B=1, N=200, H=2):
    lib = sage._load()
    shape = sage._Shape(B, N, H, 128)
    qz = sage._Quantized()
    assert lib.sage_quantized_carve(shape, 0x7f0000000000, lib.sage_workspace_bytes(shape), ctypes.byref(qz)) == 0
    return qz


def test_validation_happens_before_launch(sage):
    """Every invalid call returns a status without touching a device."""
    lib = sage._load()
    qz = _carved(sage)
    good = sage._In(0x7e0000000000, 200 * 2 * 128, 2 * 128, 128)
    null = sage._In(None, 0, 0, 0)
    misaligned = sage._In(0x7e0000000000 + 8, 200 * 256, 256, 128)
    odd_stride = sage._In(0x7e0000000000, 200 * 256, 250, 128)
    neg_stride = sage._In(0x7e0000000000, 200 * 256, -256, 128)
    out_good = sage._Out(0x7d0000000000, 200 * 256, 256, 128)
    B = ctypes.byref
    assert lib.sage_quantize_qkv(B(null), B(good), B(good), B(qz), None) == 1
    assert lib.sage_quantize_qkv(B(good), B(misaligned), B(good), B(qz), None) == 2
    assert lib.sage_quantize_qkv(B(good), B(good), B(odd_stride), B(qz), None) == 2
    assert lib.sage_quantize_qkv(B(good), B(neg_stride), B(good), B(qz), None) == 2
    bad_shape = _carved(sage)
    bad_shape.shape.D = 64
    assert lib.sage_quantize_qkv(B(good), B(good), B(good), B(bad_shape), None) == 1
    missing = _carved(sage)
    missing.v_fp8 = None
    assert lib.sage_attn_fwd_quantized(B(missing), ctypes.c_float(0.088), B(out_good), None) == 1
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.sage_attn_fwd_quantized(B(qz), ctypes.c_float(s), B(out_good), None) == 1
    assert lib.sage_attn_fwd_quantized(B(qz), ctypes.c_float(0.088), B(sage._Out(None, 0, 0, 0)), None) == 1
    assert lib.sage_attn_fwd_quantized(B(qz), ctypes.c_float(0.088),
                                       B(sage._Out(0x7d0000000000 + 4, 0, 256, 128)), None) == 2
    shape = sage._Shape(1, 200, 2, 128)
    need = lib.sage_workspace_bytes(shape)
    assert lib.sage_attn_fwd(B(good), B(good), B(good), shape, ctypes.c_float(0.088), B(out_good),
                             0x7c0000000000, need - 256, None) == 3
    big = _carved(sage, 1, 5000, 1)
    assert lib.sage_debug_qk_s32(B(big), 0x7b0000000000, None) == 2
    assert lib.sage_debug_cvt_e4m3(None, 0x1000, 4, None) == 1
    assert lib.sage_debug_cvt_e4m3(0x1000, 0x1000, -1, None) == 1
    assert lib.sage_debug_cvt_e4m3(0x1000, 0x1000, 0, None) == 0                # empty: nothing to do
    assert lib.sage_status_string(3) == b"workspace missing, misaligned or too small"
    for kind, wps, blocks, iters, ptr in [(3, 3, 1, 10, 0x1000), (0, 0, 1, 10, 0x1000), (0, 5, 1, 10, 0x1000),
                                          (0, 3, 0, 10, 0x1000), (0, 3, 1, 0, 0x1000), (0, 3, 1, 10, None)]:
        assert lib.sage_debug_issue_probe(kind, wps, blocks, iters, ptr, None) == 1


def test_noalloc_validation_happens_before_any_device_call(sage):
    """The allocation-free entry point checks the shape against its fixed
    workspace array, and its arguments, before it touches a device (these
    calls run on a machine without a GPU)."""
    lib = sage._load()
    B = ctypes.byref
    good = sage._In(0x7e0000000000, 200 * 2 * 128, 2 * 128, 128)
    out_good = sage._Out(0x7d0000000000, 200 * 256, 256, 128)
    small = sage._Shape(1, 200, 2, 128)
    assert lib.sage_workspace_bytes(small) <= sage.NOALLOC_SCRATCH_BYTES
    # the array holds a 4096-token, 8-head case but not the long-context one
    assert lib.sage_workspace_bytes(sage._Shape(1, 4096, 8, 128)) <= sage.NOALLOC_SCRATCH_BYTES
    big = sage._Shape(1, 37810, 56, 128)
    assert lib.sage_workspace_bytes(big) > sage.NOALLOC_SCRATCH_BYTES
    st = lib.sage_attn_fwd_noalloc(B(good), B(good), B(good), big, ctypes.c_float(0.088), B(out_good), None)
    assert st == 2
    msg = lib.sage_last_error_message().decode()
    assert "allocation-free" in msg and str(sage.NOALLOC_SCRATCH_BYTES) in msg
    assert lib.sage_attn_fwd_noalloc(B(good), B(good), B(good), sage._Shape(1, 200, 2, 64), ctypes.c_float(0.088),
                                     B(out_good), None) == 1
    assert lib.sage_attn_fwd_noalloc(B(sage._In(None, 0, 0, 0)), B(good), B(good), small, ctypes.c_float(0.088),
                                     B(out_good), None) == 1
    assert lib.sage_attn_fwd_noalloc(B(good), B(good), B(good), small, ctypes.c_float(0.0), B(out_good), None) == 1
    assert lib.sage_attn_fwd_noalloc(B(good), B(good), B(good), small, ctypes.c_float(0.088),
                                     B(sage._Out(None, 0, 0, 0)), None) == 1


def test_layout_unpack_roundtrip():
    """The test-side unpackers are bijections onto the logical index space."""
    B, H, N = 1, 2, 200
    Nq, Nk, T = 256, 256, 4
    idx = np.arange(B * H * Nq * 128, dtype=np.int64)
    for f, rows in ((layouts.q_logical, Nq), (layouts.k_logical, Nk), (layouts.v_logical, Nk)):
        out = f(np.arange(B * H * rows * 128, dtype=np.int64), B, H, N)
        assert out.shape == (B, H, rows, 128)
        assert np.array_equal(np.sort(out.ravel()), np.arange(B * H * rows * 128))
    # spot checks against the header's formulas
    q = layouts.q_logical(idx, B, H, N)
    g, kk, l, i = 3, 2, 37, 9
    assert q[0, 1, 32 * g + l % 32, 32 * kk + 16 * (l // 32) + i] == ((1 * 8 + g) * 4096 + (kk * 64 + l) * 16 + i)
    k = layouts.k_logical(idx, B, H, N)
    t, half = 2, 1
    assert k[0, 0, 64 * t + 32 * half + l % 32, 32 * kk + 16 * (l // 32) + i] == \
        (t * 8192 + ((half * 4 + kk) * 64 + l) * 16 + i)
    v = layouts.v_logical(idx, B, H, N)
    db = 3
    assert v[0, 1, 64 * t + 32 * half + 8 * (i // 4) + 4 * (l // 32) + i % 4, 32 * db + l % 32] == \
        ((1 * T + t) * 8192 + ((db * 2 + half) * 64 + l) * 16 + i)


def test_range_validation_happens_before_launch(sage):
    """Empty or out-of-bounds query/head ranges are rejected on the host."""
    lib = sage._load()
    qz = _carved(sage, N=200, H=2)
    out = sage._Out(0x7f0000000000, 200 * 2 * 128, 2 * 128, 128)
    bad = [(0, 0, 0, 2), (-1, 10, 0, 2), (150, 51, 0, 2), (0, 200, 0, 3), (0, 200, 2, 1), (0, 200, -1, 2),
           (0, 200, 0, 0)]
    for r in bad:
        rr = sage._Range(*r)
        assert lib.sage_attn_fwd_quantized_range(ctypes.byref(qz), ctypes.c_float(0.088), ctypes.byref(rr),
                                                 ctypes.byref(out), None) == 1, r
        assert b"range" in lib.sage_last_error_message()
    assert lib.sage_attn_fwd_quantized_range(ctypes.byref(qz), ctypes.c_float(0.088), None,
                                             ctypes.byref(out), None) == 1


def test_norm_rope_validation_happens_before_launch(sage):
    """The RMSNorm + RoPE prepass rejects a missing descriptor, missing or
    misaligned weights and tables, and a bad epsilon, without a launch."""
    lib = sage._load()
    qz = _carved(sage)
    good = sage._In(0x7e0000000000, 200 * 2 * 128, 2 * 128, 128)
    B = ctypes.byref
    w, c, s = 0x7a0000000000, 0x7a0000100000, 0x7a0000200000
    assert lib.sage_quantize_qkv_norm_rope(B(good), B(good), B(good), None, B(qz), None) == 1
    assert b"descriptor" in lib.sage_last_error_message()
    for nr, code in ((sage._NormRope(None, w, c, s, 1e-6), 1), (sage._NormRope(w, w, None, s, 1e-6), 1),
                     (sage._NormRope(w + 4, w, c, s, 1e-6), 2), (sage._NormRope(w, w, c, s + 8, 1e-6), 2),
                     (sage._NormRope(w, w, c, s, 0.0), 1), (sage._NormRope(w, w, c, s, -1e-6), 1),
                     (sage._NormRope(w, w, c, s, float("nan")), 1), (sage._NormRope(w, w, c, s, float("inf")), 1)):
        assert lib.sage_quantize_qkv_norm_rope(B(good), B(good), B(good), B(nr), B(qz), None) == code
    ok = sage._NormRope(w, w, c, s, 1e-6)
    null = sage._In(None, 0, 0, 0)
    assert lib.sage_quantize_qkv_norm_rope(B(null), B(good), B(good), B(ok), B(qz), None) == 1
    bad_shape = _carved(sage)
    bad_shape.shape.D = 64
    assert lib.sage_quantize_qkv_norm_rope(B(good), B(good), B(good), B(ok), B(bad_shape), None) == 1
    # the one-call form checks the same descriptor, then the workspace
    shape = sage._Shape(1, 200, 2, 128)
    need = lib.sage_workspace_bytes(shape)
    out = sage._Out(0x7d0000000000, 200 * 256, 256, 128)
    assert lib.sage_attn_fwd_norm_rope(B(good), B(good), B(good), shape, None, ctypes.c_float(0.088), B(out),
                                       0x7c0000000000, need, None) == 1
    assert lib.sage_attn_fwd_norm_rope(B(good), B(good), B(good), shape, B(sage._NormRope(w, w, c, s, 0.0)),
                                       ctypes.c_float(0.088), B(out), 0x7c0000000000, need, None) == 1
    assert lib.sage_attn_fwd_norm_rope(B(good), B(good), B(good), shape, B(ok), ctypes.c_float(0.088), B(out),
                                       0x7c0000000000, need - 256, None) == 3


def test_error_messages_are_per_thread(sage):
    """The last-error text is thread-local: concurrent failing calls on two
    host threads each read back their own message."""
    import threading
    lib = sage._load()
    results = {}
    barrier = threading.Barrier(2)

    def worker(name, shape):
        qz = sage._Quantized()
        for _ in range(200):
            barrier.wait()
            st = lib.sage_quantized_carve(shape, 0x7f0000000000, 1 << 40, ctypes.byref(qz))
            barrier.wait()
            results.setdefault(name, set()).add((st, lib.sage_last_error_message()))

    t1 = threading.Thread(target=worker, args=("d", sage._Shape(1, 200, 2, 64)))         # bad head dim
    t2 = threading.Thread(target=worker, args=("n", sage._Shape(1, 0, 2, 128)))          # empty sequence
    t1.start(); t2.start(); t1.join(); t2.join()
    assert len(results["d"]) == 1 and len(results["n"]) == 1
    (sd, md), = results["d"]
    (sn, mn), = results["n"]
    assert sd == sn == 1
    assert b"D=64" in md and b"N=0" in mn
