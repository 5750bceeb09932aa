"""The entry points allocate, copy and synchronise nothing and launch only on
the caller's stream, so a caller can capture them in a HIP graph.

Each test captures one form of the path with torch.cuda.graph (the binding
passes the capturing stream to the library and allocates its workspace and
output from the graph's pool), replays the graph several times with eager
work and synchronisations in between, and requires every replay to equal the
eager result byte for byte -- also after new inputs are copied into the
captured input tensors.  Forms: the two calls bench.py times
(sage_quantize_qkv + sage_attn_fwd_quantized), the one-call sage_attn_fwd and
the one-call sage_attn_fwd_norm_rope.
"""
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

B, N, H = 2, 1000, 3        # 16 KV tiles (the last with 40 keys), 8 Q blocks per head, ragged last block


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


def _inputs(seed):
    inp = workloads.generate(workloads.Workload("graph", B, N, H, seed=seed))
    return inp.q.cuda(), inp.k.cuda(), inp.v.cuda()


def _bits(t):
    return t.view(torch.int16)


def _eager_work():
    # unrelated eager work between replays: a float32 matrix product and a reduction
    x = torch.randn(512, 512, device="cuda")
    y = x @ x
    torch.cuda.synchronize()
    return float(y.abs().sum())


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _check_replays(run, label):
    q, k, v = _inputs(seed=501)
    statics = [t.clone() for t in (q, k, v)]
    g, out_g = _capture(lambda: run(*statics))
    want = run(q, k, v)
    torch.cuda.synchronize()
    for i in range(3):
        g.replay()
        _eager_work()
        assert torch.equal(_bits(out_g), _bits(want)), "%s: replay %d differs from the eager call" % (label, i)
    # new inputs into the captured tensors: the replay must follow them
    q2, k2, v2 = _inputs(seed=502)
    for s, t in zip(statics, (q2, k2, v2)):
        s.copy_(t)
    want2 = run(q2, k2, v2)
    torch.cuda.synchronize()
    assert not torch.equal(_bits(want2), _bits(want))
    for i in range(2):
        _eager_work()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_g), _bits(want2)), "%s: replay %d on new inputs differs" % (label, i)
    _log("graph %s: 5 replays equal to the eager calls" % label)


def test_graph_two_call_path(sage):
    keep = []       # the quantized operands' workspaces stay alive with the graph

    def two_call(q, k, v):
        qz = sage.quantize_qkv(q, k, v)
        keep.append(qz)
        return sage.attn_fwd_quantized(qz)

    _check_replays(two_call, "two-call")


def test_graph_one_call_path(sage):
    _check_replays(lambda q, k, v: sage.attn_fwd(q, k, v), "one-call")


def test_graph_one_call_norm_rope(sage):
    p = workloads.norm_rope_params(N, seed=17)
    nrp = [t.cuda() for t in (p.q_weight, p.k_weight, p.cos, p.sin)]
    _check_replays(lambda q, k, v: sage.attn_fwd_norm_rope(q, k, v, *nrp, p.eps), "one-call norm+rope")
