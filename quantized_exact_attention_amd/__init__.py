"""SageAttention2-style quantized non-causal attention for AMD MI355X (gfx950).

A thin binding over the C ABI in include/sage_mi355x.h (libsage_mi355x.so):
it only marshals torch device tensors into pointers, strides and the current
HIP stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback -- if the library is missing, every call raises.

    import quantized_exact_attention_amd as sage
    o = sage.attn_fwd(q, k, v)        # q, k, v: BF16 [B, N, H, 128] on the GPU
"""
import ctypes
import math
import os

from . import build as _build

__all__ = [
    "SageError", "library_path", "workspace_bytes", "Quantized", "quantize_qkv", "quantize_qkv_norm_rope",
    "attn_fwd_quantized", "attn_fwd", "attn_fwd_noalloc", "attn_fwd_norm_rope", "debug_qk_s32", "debug_cvt_e4m3", "debug_issue_probe",
    "default_sm_scale",
]

HEAD_DIM = 128
ABI_VERSION = 3   # SAGE_ABI_VERSION of include/sage_mi355x.h that these structures follow
NOALLOC_SCRATCH_BYTES = 64 << 20   # SAGE_NOALLOC_SCRATCH_BYTES: the allocation-free path's workspace


class SageError(RuntimeError):
    """A failed library call (status code and the library's message)."""


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32)]


class _In(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_n", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class _Range(ctypes.Structure):
    _fields_ = [("q_start", ctypes.c_int32), ("q_count", ctypes.c_int32),
                ("head_start", ctypes.c_int32), ("head_count", ctypes.c_int32)]


class _Out(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_n", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class _Quantized(ctypes.Structure):
    _fields_ = [("shape", _Shape),
                ("q_i8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("k_i8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_mean", ctypes.c_void_p),
                ("v_fp8", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_tile_sum", ctypes.c_void_p), ("v_tile_amax", ctypes.c_void_p), ("v_inv", ctypes.c_void_p),
                ("k_scale_max", ctypes.c_void_p)]


class _NormRope(ctypes.Structure):
    _fields_ = [("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p),
                ("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("eps", ctypes.c_float)]


_lib = None


def library_path() -> str:
    return _build.LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        raise SageError("libsage_mi355x.so is not built (%s); run __graft_entry__.build() "
                        "or python -m quantized_exact_attention_amd.build" % _build.LIB)
    lib = ctypes.CDLL(_build.LIB)
    P = ctypes.c_void_p
    st = ctypes.c_int
    lib.sage_workspace_bytes.argtypes = [_Shape]
    lib.sage_workspace_bytes.restype = ctypes.c_size_t
    lib.sage_quantized_carve.argtypes = [_Shape, P, ctypes.c_size_t, ctypes.POINTER(_Quantized)]
    lib.sage_quantized_carve.restype = st
    lib.sage_quantize_qkv.argtypes = [ctypes.POINTER(_In)] * 3 + [ctypes.POINTER(_Quantized), P]
    lib.sage_quantize_qkv.restype = st
    lib.sage_quantize_qkv_norm_rope.argtypes = [ctypes.POINTER(_In)] * 3 + [ctypes.POINTER(_NormRope),
                                                                           ctypes.POINTER(_Quantized), P]
    lib.sage_quantize_qkv_norm_rope.restype = st
    lib.sage_attn_fwd_quantized.argtypes = [ctypes.POINTER(_Quantized), ctypes.c_float, ctypes.POINTER(_Out), P]
    lib.sage_attn_fwd_quantized.restype = st
    lib.sage_attn_fwd_quantized_range.argtypes = [ctypes.POINTER(_Quantized), ctypes.c_float,
                                                  ctypes.POINTER(_Range), ctypes.POINTER(_Out), P]
    lib.sage_attn_fwd_quantized_range.restype = st
    lib.sage_attn_fwd.argtypes = [ctypes.POINTER(_In)] * 3 + [_Shape, ctypes.c_float, ctypes.POINTER(_Out),
                                                              P, ctypes.c_size_t, P]
    lib.sage_attn_fwd.restype = st
    lib.sage_attn_fwd_noalloc.argtypes = [ctypes.POINTER(_In)] * 3 + [_Shape, ctypes.c_float,
                                                                      ctypes.POINTER(_Out), P]
    lib.sage_attn_fwd_noalloc.restype = st
    lib.sage_attn_fwd_norm_rope.argtypes = [ctypes.POINTER(_In)] * 3 + [_Shape, ctypes.POINTER(_NormRope),
                                                                        ctypes.c_float, ctypes.POINTER(_Out),
                                                                        P, ctypes.c_size_t, P]
    lib.sage_attn_fwd_norm_rope.restype = st
    lib.sage_status_string.argtypes = [st]
    lib.sage_status_string.restype = ctypes.c_char_p
    lib.sage_last_error_message.argtypes = []
    lib.sage_last_error_message.restype = ctypes.c_char_p
    lib.sage_abi_version.restype = ctypes.c_int32
    lib.sage_debug_qk_s32.argtypes = [ctypes.POINTER(_Quantized), P, P]
    lib.sage_debug_qk_s32.restype = st
    lib.sage_debug_cvt_e4m3.argtypes = [P, P, ctypes.c_int64, P]
    lib.sage_debug_cvt_e4m3.restype = st
    lib.sage_debug_issue_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P]
    lib.sage_debug_issue_probe.restype = st
    if lib.sage_abi_version() != ABI_VERSION:
        raise SageError("%s has ABI version %d, this binding needs %d (rebuild the library)"
                        % (_build.LIB, lib.sage_abi_version(), ABI_VERSION))
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = _load()
        raise SageError("%s: %s" % (lib.sage_status_string(status).decode(),
                                    lib.sage_last_error_message().decode()))


def _torch():
    import torch
    return torch


def _stream_ptr(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def default_sm_scale() -> float:
    """1/sqrt(128) rounded to binary32."""
    return float(ctypes.c_float(1.0 / math.sqrt(HEAD_DIM)).value)


def _in_desc(x, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise SageError("%s must be a GPU tensor" % name)
    if x.dtype != torch.bfloat16 or x.dim() != 4 or x.shape[3] != HEAD_DIM or x.stride(3) != 1:
        raise SageError("%s must be BF16 [B, N, H, 128] with unit stride along the last dimension" % name)
    return _In(x.data_ptr(), x.stride(0), x.stride(1), x.stride(2))


def _out_desc(o, shape):
    torch = _torch()
    if not isinstance(o, torch.Tensor) or o.device.type != "cuda" or o.dtype != torch.bfloat16 \
            or o.dim() != 4 or o.shape[3] != HEAD_DIM or o.stride(3) != 1:
        raise SageError("out must be a BF16 GPU tensor [B, N, H, 128] with unit stride along the last dimension")
    if tuple(o.shape) != tuple(shape):
        raise SageError("out has shape %s, expected %s" % (tuple(o.shape), tuple(shape)))
    return _Out(o.data_ptr(), o.stride(0), o.stride(1), o.stride(2))


def workspace_bytes(B: int, N: int, H: int) -> int:
    return int(_load().sage_workspace_bytes(_Shape(B, N, H, HEAD_DIM)))


def _workspace(B, N, H, device):
    torch = _torch()
    n = workspace_bytes(B, N, H)
    if n == 0:
        raise SageError("invalid shape B=%d N=%d H=%d" % (B, N, H))
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws, off, n


class Quantized:
    """Quantized operands inside one workspace tensor (layouts: include/sage_mi355x.h)."""

    def __init__(self, B, N, H, device, workspace=None):
        torch = _torch()
        if workspace is None:
            self._ws, off, n = _workspace(B, N, H, device)
        else:
            n = workspace_bytes(B, N, H)
            if workspace.numel() * workspace.element_size() < n:
                raise SageError("workspace too small: needs %d bytes" % n)
            self._ws, off = workspace, 0
        self.c = _Quantized()
        _check(_load().sage_quantized_carve(_Shape(B, N, H, HEAD_DIM), self._ws.data_ptr() + off, n,
                                            ctypes.byref(self.c)))
        self.B, self.N, self.H = B, N, H
        self.T = (N + 63) // 64
        self.Nq = (N + 127) // 128 * 128
        self.G = self.Nq // 32
        self.device = device

    def _view(self, field, dtype, count):
        torch = _torch()
        base = self._ws.data_ptr()
        start = getattr(self.c, field) - base
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self._ws[start:start + nbytes].view(dtype)

    # raw views, in the library's layouts
    @property
    def q_i8(self):
        return self._view("q_i8", _torch().int8, self.B * self.H * self.Nq * HEAD_DIM)

    @property
    def q_scale(self):
        return self._view("q_scale", _torch().float32, self.B * self.H * self.G).view(self.B, self.H, self.G)

    @property
    def k_i8(self):
        return self._view("k_i8", _torch().int8, self.B * self.H * self.T * 64 * HEAD_DIM)

    @property
    def k_scale(self):
        return self._view("k_scale", _torch().float32, self.B * self.H * self.T).view(self.B, self.H, self.T)

    @property
    def k_scale_max(self):
        return self._view("k_scale_max", _torch().float32, self.B * self.H).view(self.B, self.H)

    @property
    def k_mean(self):
        return self._view("k_mean", _torch().float32, self.B * self.H * HEAD_DIM).view(self.B, self.H, HEAD_DIM)

    @property
    def v_fp8(self):
        return self._view("v_fp8", _torch().uint8, self.B * self.H * self.T * 64 * HEAD_DIM)

    @property
    def v_scale(self):
        return self._view("v_scale", _torch().float32, self.B * self.H * HEAD_DIM).view(self.B, self.H, HEAD_DIM)


def _target(q, k, v, workspace, into):
    if not (q.shape == k.shape == v.shape):
        raise SageError("q, k, v shapes differ")
    B, N, H, _ = q.shape
    if into is not None:
        if (into.B, into.N, into.H) != (B, N, H):
            raise SageError("into has shape %s, inputs %s" % ((into.B, into.N, into.H), (B, N, H)))
        return into
    return Quantized(B, N, H, q.device, workspace)


def quantize_qkv(q, k, v, workspace=None, into: Quantized = None) -> Quantized:
    """The prepass: K mean, INT8 Q/K and FP8 V with their scales.

    With ``into``, the operands are rewritten in that object's workspace
    (same shape required) and nothing is allocated."""
    dq, dk, dv = _in_desc(q, "q"), _in_desc(k, "k"), _in_desc(v, "v")
    qz = _target(q, k, v, workspace, into)
    _check(_load().sage_quantize_qkv(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                     ctypes.byref(qz.c), _stream_ptr(q)))
    qz._inputs = (q, k, v)
    return qz


def _f32_desc(x, shape, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.float32 \
            or tuple(x.shape) != tuple(shape) or not x.is_contiguous():
        raise SageError("%s must be a contiguous FP32 GPU tensor of shape %s" % (name, tuple(shape)))
    return x.data_ptr()


def quantize_qkv_norm_rope(q, k, v, q_weight, k_weight, cos, sin, eps: float = 1e-6,
                           workspace=None, into: Quantized = None) -> Quantized:
    """The prepass on RMSNorm + split-half RoPE of Q and K (V as is).

    q_weight, k_weight: FP32 [128]; cos, sin: FP32 [N, 64] (row n = token n).
    The normalised and rotated rows are recomputed where the prepass reads Q
    and K and never stored; the result equals quantize_qkv on them."""
    dq, dk, dv = _in_desc(q, "q"), _in_desc(k, "k"), _in_desc(v, "v")
    N = q.shape[1]
    nr = _NormRope(_f32_desc(q_weight, (HEAD_DIM,), "q_weight"), _f32_desc(k_weight, (HEAD_DIM,), "k_weight"),
                   _f32_desc(cos, (N, HEAD_DIM // 2), "cos"), _f32_desc(sin, (N, HEAD_DIM // 2), "sin"), eps)
    qz = _target(q, k, v, workspace, into)
    _check(_load().sage_quantize_qkv_norm_rope(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                               ctypes.byref(nr), ctypes.byref(qz.c), _stream_ptr(q)))
    qz._inputs = (q, k, v, q_weight, k_weight, cos, sin)
    return qz


def attn_fwd_quantized(qz: Quantized, sm_scale: float = None, out=None):
    """The fused mainloop on already-quantized operands; returns BF16 [B, N, H, 128]."""
    torch = _torch()
    if sm_scale is None:
        sm_scale = default_sm_scale()
    if out is None:
        out = torch.empty((qz.B, qz.N, qz.H, HEAD_DIM), dtype=torch.bfloat16, device=qz.device)
    do = _out_desc(out, (qz.B, qz.N, qz.H, HEAD_DIM))
    _check(_load().sage_attn_fwd_quantized(ctypes.byref(qz.c), ctypes.c_float(sm_scale), ctypes.byref(do),
                                           _stream_ptr(out)))
    return out


def attn_fwd_quantized_range(qz: Quantized, q_start: int, q_count: int, head_start: int, head_count: int,
                             sm_scale: float = None, out=None):
    """The mainloop for query rows [q_start, q_start + q_count) and heads
    [head_start, head_start + head_count); returns (or fills) the BF16
    [B, q_count, head_count, 128] view of those rows."""
    torch = _torch()
    if sm_scale is None:
        sm_scale = default_sm_scale()
    if out is None:
        out = torch.empty((qz.B, q_count, head_count, HEAD_DIM), dtype=torch.bfloat16, device=qz.device)
    do = _out_desc(out, (qz.B, q_count, head_count, HEAD_DIM))
    r = _Range(q_start, q_count, head_start, head_count)
    _check(_load().sage_attn_fwd_quantized_range(ctypes.byref(qz.c), ctypes.c_float(sm_scale), ctypes.byref(r),
                                                 ctypes.byref(do), _stream_ptr(out)))
    return out


def _one_call(q, k, v, sm_scale, out, workspace, nr):
    torch = _torch()
    dq, dk, dv = _in_desc(q, "q"), _in_desc(k, "k"), _in_desc(v, "v")
    if not (q.shape == k.shape == v.shape):
        raise SageError("q, k, v shapes differ")
    B, N, H, _ = q.shape
    if sm_scale is None:
        sm_scale = default_sm_scale()
    if out is None:
        out = torch.empty((B, N, H, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    do = _out_desc(out, (B, N, H, HEAD_DIM))
    if workspace is None:
        ws, off, n = _workspace(B, N, H, q.device)
    else:
        ws, off, n = workspace, 0, workspace.numel() * workspace.element_size()
    args = (ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _Shape(B, N, H, HEAD_DIM))
    tail = (ctypes.c_float(sm_scale), ctypes.byref(do), ws.data_ptr() + off, n, _stream_ptr(q))
    if nr is None:
        _check(_load().sage_attn_fwd(*args, *tail))
    else:
        _check(_load().sage_attn_fwd_norm_rope(*args, ctypes.byref(nr), *tail))
    return out


def attn_fwd(q, k, v, sm_scale: float = None, out=None, workspace=None):
    """Whole path (prepass + mainloop) in one call; returns BF16 [B, N, H, 128]."""
    return _one_call(q, k, v, sm_scale, out, workspace, None)


def attn_fwd_noalloc(q, k, v, sm_scale: float = None, out=None):
    """attn_fwd with the library's own fixed-size device workspace
    (NOALLOC_SCRATCH_BYTES per GPU) instead of a caller workspace; the library
    call allocates nothing (only `out`, when not given, is allocated here)."""
    torch = _torch()
    dq, dk, dv = _in_desc(q, "q"), _in_desc(k, "k"), _in_desc(v, "v")
    if not (q.shape == k.shape == v.shape):
        raise SageError("q, k, v shapes differ")
    B, N, H, _ = q.shape
    if sm_scale is None:
        sm_scale = default_sm_scale()
    if out is None:
        out = torch.empty((B, N, H, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    do = _out_desc(out, (B, N, H, HEAD_DIM))
    _check(_load().sage_attn_fwd_noalloc(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                         _Shape(B, N, H, HEAD_DIM), ctypes.c_float(sm_scale), ctypes.byref(do),
                                         _stream_ptr(q)))
    return out


def attn_fwd_norm_rope(q, k, v, q_weight, k_weight, cos, sin, eps: float = 1e-6, sm_scale: float = None,
                       out=None, workspace=None):
    """attn_fwd on RMSNorm + split-half RoPE of Q and K (as quantize_qkv_norm_rope):
    K is normalised in the prepass, Q in the mainloop prologue."""
    N = q.shape[1]
    nr = _NormRope(_f32_desc(q_weight, (HEAD_DIM,), "q_weight"), _f32_desc(k_weight, (HEAD_DIM,), "k_weight"),
                   _f32_desc(cos, (N, HEAD_DIM // 2), "cos"), _f32_desc(sin, (N, HEAD_DIM // 2), "sin"), eps)
    return _one_call(q, k, v, sm_scale, out, workspace, nr)


def debug_qk_s32(qz: Quantized):
    """int32 Q.K^T from the mainloop's tile routine: [B, H, Nq, 64*T] (N <= 4096)."""
    torch = _torch()
    s = torch.empty((qz.B, qz.H, qz.Nq, qz.T * 64), dtype=torch.int32, device=qz.device)
    _check(_load().sage_debug_qk_s32(ctypes.byref(qz.c), s.data_ptr(), _stream_ptr(s)))
    return s


def debug_issue_probe(kind: int, waves_per_simd: int, blocks: int, iters: int, device=None):
    """Cycle counts of the mainloop's tile-step instruction streams
    (sage_debug_issue_probe): an int64 GPU tensor [blocks, 4*waves_per_simd]."""
    torch = _torch()
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    ticks = torch.zeros((blocks, 4 * waves_per_simd), dtype=torch.int64, device=device)
    _check(_load().sage_debug_issue_probe(kind, waves_per_simd, blocks, iters, ticks.data_ptr(), _stream_ptr(ticks)))
    return ticks


def debug_cvt_e4m3(x):
    """The kernels' FP32 -> E4M3FN conversion applied to a float32 GPU tensor."""
    torch = _torch()
    if x.device.type != "cuda" or x.dtype != torch.float32:
        raise SageError("x must be a float32 GPU tensor")
    x = x.contiguous()
    y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_load().sage_debug_cvt_e4m3(x.data_ptr(), y.data_ptr(), x.numel(), _stream_ptr(x)))
    return y
