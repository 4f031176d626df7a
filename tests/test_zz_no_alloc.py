"""The forward entry point that allocates nothing (gdn_chunk_fwd_noalloc): its chunk
records sit in the library's static device scratch instead of a caller workspace. Its
outputs must equal gdn_chunk_fwd's bit for bit (same kernels, same arithmetic), on two
calls in a row, the second with a smaller problem, so that records the first call left
in the shared scratch cannot leak into the second."""
import ctypes
import dataclasses

import pytest
import torch

from gpu_common import dev, sync, to_dev, workload_inputs
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _run_both(inp, with_state=True):
    q, k, v, g, beta, h0, vl = to_dev(inp)
    o_ref, hT_ref = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, vl, want_state=with_state)
    o = torch.empty_like(v)
    hT = torch.empty_like(hT_ref) if with_state else None
    gdn.gdn_chunk_fwd_noalloc(q, k, v, g, beta, h0, o, hT, vl)
    sync()
    return (o, hT), (o_ref, hT_ref)


def test_noalloc_equals_workspace_forward_twice_second_smaller():
    # first call: the stateless 8K workload (32 heads of 128, 52 MiB of chunk records)
    (o, _), (o_ref, _) = _run_both(workload_inputs("stateless_8k"), with_state=False)
    assert torch.equal(o, o_ref)
    # second call, smaller and different: padded ragged rows with an initial state
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="noalloc_small", B=2, T=700, Hqk=2, H=4,
                            seed=991, valid_len=517)
    (o2, hT2), (o2_ref, hT2_ref) = _run_both(make_inputs(w))
    assert torch.equal(o2, o2_ref) and torch.equal(hT2, hT2_ref)
    # and the fp32 path (fp32 records in the same scratch)
    w3 = dataclasses.replace(WORKLOADS["stateful_32k"], name="noalloc_f32", B=1, T=300, Hqk=2, H=4, dk=128, dv=32,
                             io="f32", seed=992)
    (o3, hT3), (o3_ref, hT3_ref) = _run_both(make_inputs(w3))
    assert torch.equal(o3, o3_ref) and torch.equal(hT3, hT3_ref)


def test_noalloc_narrow_heads_equal_the_workspace_forward():
    """Heads under 128 run here, as in gdn_chunk_fwd, on padded copies of q and k (in the
    static array beside the records): bit for bit, fp32 and bf16."""
    for io in ("f32", "bf16"):
        w = dataclasses.replace(WORKLOADS["stateful_32k"], name="noalloc_narrow_" + io, B=1, T=300, Hqk=2, H=4,
                                dk=32, dv=32, io=io, seed=993)
        (o, hT), (o_ref, hT_ref) = _run_both(make_inputs(w))
        assert torch.equal(o, o_ref) and torch.equal(hT, hT_ref), io


def test_noalloc_rejects_problems_beyond_the_scratch():
    inp = workload_inputs("stateful_32k")   # 208 MiB of records
    q, k, v, g, beta, h0, _ = to_dev(inp)
    o = torch.empty_like(v)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd_noalloc(q, k, v, g, beta, h0, o)
    assert e.value.status == gdn.GDN_EWORKSPACE
