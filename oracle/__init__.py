"""CPU oracle of SageAttention2-style quantized non-causal attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.  The arithmetic lives
in ``sage_oracle.c`` (plain C, one binary32 operation per statement, no FMA
contraction); this module only marshals arrays into it.  ``reference64`` holds
the unquantized float64 softmax attention used as a self-check.

Inputs are BF16 tensors viewed as [B, N, H, D=128] with unit stride along D
(torch CPU bfloat16 tensors, or numpy uint16 arrays of BF16 bit patterns); any
strides along B, N and H are honoured, so projection-strided views work as is.
"""
import contextlib
import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

HD = 128
_lib = None


def _configure(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_float
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_k_mean.argtypes = [P, I64, I64, I64, I, I, I, P]
    lib.oracle_quant_k.argtypes = [P, I64, I64, I64, I, I, I, P, P, P]
    lib.oracle_quant_q.argtypes = [P, I64, I64, I64, I, I, I, P, P]
    lib.oracle_quant_v.argtypes = [P, I64, I64, I64, I, I, I, P, P]
    lib.oracle_norm_rope.argtypes = [P, I64, I64, I64, I, I, I, P, P, P, ctypes.c_float, P]
    lib.oracle_qk_s32.argtypes = [P, P, I, I, I, I64, I64, P]
    lib.oracle_attn_rows.argtypes = [P, P, P, P, P, P, I, I, I, ctypes.c_float, P, I64, P, P]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_e4m3_encode_n.argtypes = [P, P, I64]
    lib.oracle_f32_to_bf16_n.argtypes = [P, P, I64]
    for name in ("oracle_norm_rope", "oracle_k_mean", "oracle_quant_k", "oracle_quant_q", "oracle_quant_v",
                 "oracle_qk_s32", "oracle_attn_rows", "oracle_e4m3_encode_n",
                 "oracle_f32_to_bf16_n"):
        getattr(lib, name).restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        _lib = _configure(ctypes.CDLL(path))
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call through another build of the C
    source (used by the test that plants mistakes into copies of it)."""
    global _lib
    saved = _load()
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class _View:
    """A [B, N, H, 128] BF16 view: base pointer, element strides, keep-alive."""

    def __init__(self, x):
        try:
            import torch
        except ImportError:  # pragma: no cover
            torch = None
        if torch is not None and isinstance(x, torch.Tensor):
            if x.device.type != "cpu" or x.dtype != torch.bfloat16:
                raise ValueError("oracle inputs must be CPU bfloat16 tensors")
            if x.dim() != 4 or x.shape[3] != HD or x.stride(3) != 1:
                raise ValueError("expected [B,N,H,128] with unit stride along D")
            self.ptr = x.data_ptr()
            self.strides = tuple(int(s) for s in x.stride()[:3])
            self.shape = tuple(int(s) for s in x.shape)
            self.keep = x
        else:
            a = np.asarray(x)
            if a.dtype != np.uint16 or a.ndim != 4 or a.shape[3] != HD or a.strides[3] != 2:
                raise ValueError("expected uint16 BF16 bits [B,N,H,128] with unit stride along D")
            self.ptr = a.ctypes.data
            self.strides = tuple(s // 2 for s in a.strides[:3])
            self.shape = a.shape
            self.keep = a
        self.B, self.N, self.H, _ = self.shape


def ceil_div(a: int, b: int) -> int:
    return (a + b - 1) // b


@dataclass
class Quantized:
    """Oracle quantized operands in plain logical layouts (see sage_oracle.c)."""
    B: int
    N: int
    H: int
    k_mean: np.ndarray   # float32 [B,H,128]
    q_i8: np.ndarray     # int8   [B,H,Nq,128]
    q_scale: np.ndarray  # float32 [B,H,Nq/32]
    k_i8: np.ndarray     # int8   [B,H,Nk,128]
    k_scale: np.ndarray  # float32 [B,H,Nk/64]
    v8: np.ndarray       # uint8  [B,H,Nk,128]  (E4M3 bytes)
    v_scale: np.ndarray  # float32 [B,H,128]


def k_mean(K) -> np.ndarray:
    v = _View(K)
    out = np.zeros((v.B, v.H, HD), np.float32)
    _load().oracle_k_mean(v.ptr, *v.strides, v.B, v.N, v.H, _ptr(out))
    return out


def quant_k(K, km: np.ndarray):
    v = _View(K)
    T = ceil_div(v.N, 64)
    km = np.ascontiguousarray(km, np.float32)
    k_i8 = np.zeros((v.B, v.H, T * 64, HD), np.int8)
    k_scale = np.zeros((v.B, v.H, T), np.float32)
    _load().oracle_quant_k(v.ptr, *v.strides, v.B, v.N, v.H, _ptr(km), _ptr(k_i8), _ptr(k_scale))
    return k_i8, k_scale


def quant_q(Q):
    v = _View(Q)
    Nq = ceil_div(v.N, 128) * 128
    q_i8 = np.zeros((v.B, v.H, Nq, HD), np.int8)
    q_scale = np.zeros((v.B, v.H, Nq // 32), np.float32)
    _load().oracle_quant_q(v.ptr, *v.strides, v.B, v.N, v.H, _ptr(q_i8), _ptr(q_scale))
    return q_i8, q_scale


def quant_v(V):
    v = _View(V)
    Nk = ceil_div(v.N, 64) * 64
    v8 = np.zeros((v.B, v.H, Nk, HD), np.uint8)
    v_scale = np.zeros((v.B, v.H, HD), np.float32)
    _load().oracle_quant_v(v.ptr, *v.strides, v.B, v.N, v.H, _ptr(v8), _ptr(v_scale))
    return v8, v_scale


def quantize(Q, K, V) -> Quantized:
    """Steps 1-4: K mean, Q/K INT8 and V FP8 quantization."""
    vq, vk, vv = _View(Q), _View(K), _View(V)
    if not (vq.shape == vk.shape == vv.shape):
        raise ValueError("Q, K, V shapes differ")
    km = k_mean(K)
    q_i8, q_scale = quant_q(Q)
    k_i8, k_scale = quant_k(K, km)
    v8, v_scale = quant_v(V)
    return Quantized(vq.B, vq.N, vq.H, km, q_i8, q_scale, k_i8, k_scale, v8, v_scale)


def norm_rope(X, weight, cos, sin, eps: float) -> np.ndarray:
    """Step 0: per-head RMSNorm (FP32 weight [128]) then split-half RoPE with the
    FP32 angle tables cos, sin [N, 64]; returns BF16 bits [B, N, H, 128]."""
    v = _View(X)
    g = np.ascontiguousarray(np.asarray(weight, np.float32).reshape(HD))
    c = np.ascontiguousarray(np.asarray(cos, np.float32))
    s = np.ascontiguousarray(np.asarray(sin, np.float32))
    if c.shape != (v.N, HD // 2) or s.shape != (v.N, HD // 2):
        raise ValueError("angle tables must be [N, 64]")
    out = np.zeros((v.B, v.N, v.H, HD), np.uint16)
    _load().oracle_norm_rope(v.ptr, *v.strides, v.B, v.N, v.H, _ptr(g), _ptr(c), _ptr(s),
                             ctypes.c_float(eps), _ptr(out))
    return out


def quantize_norm_rope(Q, K, V, q_weight, k_weight, cos, sin, eps: float) -> Quantized:
    """Step 0 on Q and K, then steps 1-4 on the results (V unchanged)."""
    return quantize(norm_rope(Q, q_weight, cos, sin, eps), norm_rope(K, k_weight, cos, sin, eps), V)


def qk_s32(qz: Quantized, r0: int = 0, r1: int = None) -> np.ndarray:
    """Exact int32 Q.K^T for query rows [r0, r1) against all Nk keys: [B,H,r1-r0,Nk]."""
    if r1 is None:
        r1 = qz.q_i8.shape[2]
    Nk = qz.k_i8.shape[2]
    out = np.zeros((qz.B, qz.H, r1 - r0, Nk), np.int32)
    _load().oracle_qk_s32(_ptr(qz.q_i8), _ptr(qz.k_i8), qz.B, qz.N, qz.H, r0, r1, _ptr(out))
    return out


def default_sm_scale() -> float:
    """1/sqrt(128) rounded to binary32: the plain softmax-attention scale."""
    return float(np.float32(1.0 / np.sqrt(np.float64(HD))))


def attn_rows(qz: Quantized, rows, sm_scale: float = None):
    """Steps 5-9 for the given (b, h, r) rows.

    Returns (bits, f32): BF16 bit patterns uint16 [n,128] and the FP32 value
    before BF16 rounding, float32 [n,128].
    """
    if sm_scale is None:
        sm_scale = default_sm_scale()
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    if rows.size and (rows[:, 2].max() >= qz.N or rows.min() < 0
                      or rows[:, 0].max() >= qz.B or rows[:, 1].max() >= qz.H):
        raise ValueError("row index out of range")
    n = rows.shape[0]
    bits = np.zeros((n, HD), np.uint16)
    f32 = np.zeros((n, HD), np.float32)
    _load().oracle_attn_rows(_ptr(qz.q_i8), _ptr(qz.q_scale), _ptr(qz.k_i8), _ptr(qz.k_scale),
                             _ptr(qz.v8), _ptr(qz.v_scale), qz.B, qz.N, qz.H,
                             ctypes.c_float(sm_scale), _ptr(rows), n, _ptr(bits), _ptr(f32))
    return bits, f32


def attention(Q, K, V, sm_scale: float = None):
    """Whole path on every row: returns (qz, bits [B,N,H,128] uint16, f32 [B,N,H,128])."""
    qz = quantize(Q, K, V)
    B, N, H = qz.B, qz.N, qz.H
    bb, hh, rr = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), rr.ravel()], axis=1)
    bits, f32 = attn_rows(qz, rows, sm_scale)
    bits = bits.reshape(B, H, N, HD).transpose(0, 2, 1, 3).copy()
    f32 = f32.reshape(B, H, N, HD).transpose(0, 2, 1, 3).copy()
    return qz, bits, f32


# ----------------------------------------------------------------- codecs --

def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, np.float32).ravel())
    y = np.zeros(x.shape, np.uint8)
    _load().oracle_e4m3_encode_n(_ptr(x), _ptr(y), x.size)
    return y


def e4m3_decode(b) -> np.ndarray:
    lib = _load()
    b = np.asarray(b, np.uint8).ravel()
    return np.array([lib.oracle_e4m3_decode(int(v)) for v in b], np.float32)


def bf16_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, np.float32).ravel())
    y = np.zeros(x.shape, np.uint16)
    _load().oracle_f32_to_bf16_n(_ptr(x), _ptr(y), x.size)
    return y


def bf16_decode(bits) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact)."""
    b = np.asarray(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
