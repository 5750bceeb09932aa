"""Unquantized softmax attention in float64 -- a self-check of the oracle.

TEST INFRASTRUCTURE ONLY.  The plain definition written out: for each batch b
and head h, O[b,:,h,:] = softmax(Q K^T * sm_scale) V over all N keys (no
mask: non-causal), from the exact values of the BF16 inputs.  This is what the
quantized method approximates; it carries no quantization, so the oracle's
output must stay close to it (cosine similarity), not equal.
"""
import numpy as np


def _as_f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype == np.uint16:  # BF16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def softmax_weights(q_row: np.ndarray, k: np.ndarray, sm_scale: float) -> np.ndarray:
    """Softmax weights of one query row over the key rows k [N,D] (float64)."""
    s = (k @ q_row) * sm_scale
    s = s - s.max()
    w = np.exp(s)
    return w / w.sum()


def attention64(Q, K, V, sm_scale: float) -> np.ndarray:
    """[B,N,H,D] float64 output of softmax(Q K^T * sm_scale) V per (b, h)."""
    q, k, v = _as_f64(Q), _as_f64(K), _as_f64(V)
    B, N, H, D = q.shape
    out = np.zeros((B, N, H, D), np.float64)
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h, :] @ k[b, :, h, :].T) * sm_scale      # [N, N]
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w = w / w.sum(axis=1, keepdims=True)
            out[b, :, h, :] = w @ v[b, :, h, :]
    return out
