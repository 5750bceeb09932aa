"""A plain C program (tests/c_consumer/sage_c_consumer.c) drives the library
through its C ABI alone: host-side validation on the CPU; on the GPU, the
one-call path and the two-call path on seeded inputs against the oracle
(same bar as the Python binding's parity tests)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c_consumer"))
import build as c_build  # noqa: E402


@pytest.fixture(scope="module")
def consumer():
    import quantized_exact_attention_amd as sage
    sage._load()                     # the library must be built
    return c_build.build(force=False)


def test_c_consumer_validation(consumer):
    res = subprocess.run([consumer, "errors"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["run", "run2"])
@pytest.mark.parametrize("B,N,H", [(1, 200, 2), (2, 129, 3)])
def test_c_consumer_matches_oracle(consumer, tmp_path, B, N, H, mode):
    """mode "run": the one-call sage_attn_fwd; "run2": carve, sage_quantize_qkv
    and sage_attn_fwd_quantized."""
    import torch
    import oracle
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("c consumer %s: B=%d N=%d H=%d" % (mode, B, N, H), flush=True)
    inp = workloads.generate(workloads.Workload("c", B, N, H, seed=300 + N))
    bits = [t.contiguous().view(torch.int16).numpy().view(np.uint16) for t in (inp.q, inp.k, inp.v)]
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    np.concatenate([b.ravel() for b in bits]).tofile(src)
    res = subprocess.run([consumer, mode, str(src), str(dst), str(B), str(N), str(H)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    got = oracle.bf16_decode(np.fromfile(dst, np.uint16).reshape(B, N, H, 128)).astype(np.float64)
    _, ref_bits, _ = oracle.attention(inp.q, inp.k, inp.v)
    ref = oracle.bf16_decode(ref_bits).astype(np.float64)
    max_abs = float(np.max(np.abs(got - ref)))
    cos = float(got.ravel() @ ref.ravel() / (np.linalg.norm(got) * np.linalg.norm(ref)))
    assert max_abs <= 2e-2 and cos >= 0.9999, (max_abs, cos)
