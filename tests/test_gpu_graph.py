"""The forward and the backward captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: the library enqueues kernels only (no allocation, no memset, no host
synchronisation), so a captured call must give, on every replay, exactly what the same call
gives eagerly. Between replays the test writes new inputs into the captured tensors and runs
the eager reference on them, with synchronisations in between."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_common import dev, to_dev
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def inputs(seed, **kw):
    # bf16, heads of 128 (the matrix-core path), a ragged tail, an initial state (kw: other
    # dtypes and head dims)
    inp = make_inputs(dataclasses.replace(WORKLOADS["stateful_32k"], **kw), T=1000, B=1)
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    # fresh values per replay: permute tokens of the seeded inputs and scale the state
    perm = torch.from_numpy(rng.permutation(q.shape[1])).to(dev())
    s = float(rng.uniform(0.5, 1.5))
    return q[:, perm].contiguous(), k[:, perm].contiguous(), v[:, perm].contiguous(), \
        g[:, perm].contiguous(), beta[:, perm].contiguous(), (h0 * s).contiguous()


@pytest.mark.parametrize("kw", [{}, {"io": "f32"}, {"io": "f32", "dk": 64, "dv": 64}],
                         ids=["bf16_d128", "f32_d128", "f32_d64_padded"])
def test_forward_graph_replays_match_eager_calls(kw):
    q, k, v, g, beta, h0 = inputs(0, **kw)
    o = torch.empty_like(v)
    hT = torch.empty(h0.shape, dtype=torch.float32, device=dev())
    ws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(gdn.problem(q, v)), dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture, as torch asks
        gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, o=o, hT=hT, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, o=o, hT=hT, ws=ws)
    for r in range(REPLAYS):
        new = inputs(10 + r, **kw)
        for dst, src in zip((q, k, v, g, beta, h0), new):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_ref, hT_ref = gdn.gdn_chunk_fwd(*new)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d: o differs from the eager call" % r
        assert torch.equal(hT, hT_ref), "replay %d: hT differs from the eager call" % r


def test_backward_graph_replays_match_eager_calls():
    q, k, v, g, beta, h0 = inputs(1)
    torch.manual_seed(3)
    d_o = torch.randn(v.shape, device=dev()).to(torch.bfloat16)
    p = gdn.problem(q, v)
    ws = gdn.workspace(gdn.gdn_chunk_bwd_workspace(p), dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grads = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o, ws=ws)
    for r in range(REPLAYS):
        new = inputs(20 + r)
        for dst, src in zip((q, k, v, g, beta, h0), new):
            dst.copy_(src)
        d_o.copy_(torch.randn(v.shape, device=dev()).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = gdn.gdn_chunk_bwd(*new, d_o)
        torch.cuda.synchronize()
        for nm, x, y in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), grads, ref):
            assert torch.equal(x, y), "replay %d: %s differs from the eager call" % (r, nm)
