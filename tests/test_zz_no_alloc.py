"""The allocation-free entry point (sage_attn_fwd_noalloc) against the
workspace one (sage_attn_fwd), through the C ABI, on the GPU.

Both run the same kernels on the same inputs, so their outputs must be
identical byte for byte.  Two calls in a row on the library's one workspace
array, the second with a smaller input, show that nothing left in the array
by a call changes the next one.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_exact_attention_amd as s
    s._load()
    return s


def _case(B, N, H, seed):
    inp = workloads.generate(workloads.Workload("noalloc", B, N, H, seed=seed))
    return inp.q.cuda(), inp.k.cuda(), inp.v.cuda()


def test_noalloc_equals_workspace_path_on_two_calls(sage):
    shapes = [(2, 1000, 4, 81), (1, 200, 2, 82)]           # the second call is smaller
    outs = []
    for B, N, H, seed in shapes:
        assert sage.workspace_bytes(B, N, H) <= sage.NOALLOC_SCRATCH_BYTES
        q, k, v = _case(B, N, H, seed)
        got = sage.attn_fwd_noalloc(q, k, v)
        ref = sage.attn_fwd(q, k, v)
        torch.cuda.synchronize()
        g = got.view(torch.int16).cpu().numpy()
        r = ref.view(torch.int16).cpu().numpy()
        print("noalloc B=%d N=%d H=%d: %d of %d outputs differ" % (B, N, H, int(np.sum(g != r)), g.size), flush=True)
        assert np.array_equal(g, r)
        outs.append(g)
    assert outs[0].shape != outs[1].shape


def test_noalloc_rejects_a_shape_beyond_its_array(sage):
    # a long-sequence, 56-head view of one row (zero strides): never read, the
    # shape check comes first
    big = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device="cuda").expand(1, 37810, 56, 128)
    out = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device="cuda").expand(1, 37810, 56, 128)
    with pytest.raises(sage.SageError, match="allocation-free"):
        sage.attn_fwd_noalloc(big, big, big, out=out)
