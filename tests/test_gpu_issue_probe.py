"""The issue probe behind the benchmark's vector roofline (sage_debug_issue_probe).

Its matrix-only stream is one tile's 4 FP8 32x32x64 and 8 INT8 32x32x32
instructions, which the matrix pipe executes in 64 and 32 cycles: one wave
alone on its SIMD must come to 512 cycles per tile, which also shows that the
counter the probe reads counts shader cycles.  The vector streams must take
longer with the matrix work added than without it, and more waves per SIMD
must not make a tile slower per SIMD.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_exact_attention_amd as s
    s._load()
    return s


def _cycles_per_tile(sage, kind, wps, iters=1000):
    t = sage.debug_issue_probe(kind, wps, 1, iters)
    torch.cuda.synchronize()
    return float(t.max().item()) / (iters * wps)


def test_matrix_stream_is_512_cycles_per_tile(sage):
    c = _cycles_per_tile(sage, 2, 1)
    print("matrix stream, one wave per SIMD: %.1f cycles per tile" % c, flush=True)
    assert 505.0 < c < 530.0


def test_vector_streams_are_ordered(sage):
    v3 = _cycles_per_tile(sage, 0, 3)
    vm3 = _cycles_per_tile(sage, 1, 3)
    v1 = _cycles_per_tile(sage, 0, 1)
    print("vector mix: %.1f (1 wave), %.1f (3 waves); with matrix work %.1f (3 waves)" % (v1, v3, vm3), flush=True)
    assert 160 * 2.0 < v3 < v1          # at least two cycles per instruction; more waves fill the pipe better
    assert vm3 > v3 and vm3 < v3 + 512.0
