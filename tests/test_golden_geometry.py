"""The tiling numbers the pages print for their 37,810-token workload
(tests/golden/canonical_geometry.txt), checked against the oracle's own
tiling and the library's workspace carve (host arithmetic only)."""
import ctypes
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "canonical_geometry.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = int(v)
    return vals


def test_oracle_tiling_matches_the_pages():
    g = _golden()
    N, H = g["tokens"], g["heads"]
    gen = torch.Generator().manual_seed(5)
    x = torch.randn(1, N, 1, g["head_dim"], generator=gen).to(torch.bfloat16)
    qz = oracle.quantize(x, x, x)                     # one head: tiling does not depend on H
    T = qz.k_scale.shape[-1]
    assert T == g["kv_tiles_64"]
    assert qz.k_i8.shape[2] == 64 * T and N - 64 * (T - 1) == 50
    assert qz.q_i8.shape[2] == 128 * g["q_blocks_128"]
    assert qz.q_scale.shape[-1] == 4 * g["q_blocks_128"]
    assert H * T == g["ctas_q64"]
    assert H * g["q_blocks_128"] == g["ctas_q128"]
    # the padded rows hold zero bytes and do not change the scales
    assert not np.any(qz.k_i8[0, 0, N:]) and not np.any(qz.q_i8[0, 0, N:])


def test_library_carve_matches_the_pages():
    import quantized_exact_attention_amd as sage
    from quantized_exact_attention_amd import build
    build.build(force=False)
    g = _golden()
    lib = sage._load()
    shape = sage._Shape(1, g["tokens"], g["heads"], g["head_dim"])
    qz = sage._Quantized()
    base = 0x7f0000000000                             # never dereferenced
    assert lib.sage_quantized_carve(shape, base, lib.sage_workspace_bytes(shape), ctypes.byref(qz)) == 0
    H, T, blocks = g["heads"], g["kv_tiles_64"], g["q_blocks_128"]
    assert qz.q_scale - qz.q_i8 >= H * blocks * 128 * 128          # INT8 Q, 128-row blocks
    assert qz.k_scale - qz.k_i8 >= H * T * 64 * 128                # INT8 K, 64-row tiles
    assert qz.k_mean - qz.k_scale >= H * T * 4                     # one K scale per tile
    assert qz.k_i8 - qz.q_scale >= H * blocks * 4 * 4              # one Q scale per 32 rows
