"""Tokens that take no part in the recurrence must never reach it: padded tokens
(t >= valid_len), the rows of a ragged last chunk past the end of the tensors, and
tokens of a packed tensor outside the sequence being read. The header's contract is
that they count as zero q, k, v (beta = g = 0); the tail-padding case of the pages is
hyper-parallel issue #320 (test report for PR #1114), section 5.2.

Every test fills those positions with NaN and asserts the outputs equal, bit for bit,
the run with finite values there (or with no such tokens at all). Finite pads alone
cannot show a leak: a finite garbage row is multiplied by zero masks, while a NaN row
turns every product it enters into NaN."""
import numpy as np
import pytest
import torch

from gpu_common import dev, sync, to_dev, workload_inputs
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs
import dataclasses

pytestmark = pytest.mark.gpu


def _nan_after(x, n, b=None):
    y = x.clone()
    if b is None:
        y[:, n:] = float("nan")
    else:
        y[b, n:] = float("nan")
    return y


def test_padded_8k_nan_pads_give_the_same_bits():
    """The padded 8K workload (two rows of 7777 valid tokens in 8192) with q, k, v, g and
    beta set to NaN at every padded token: the same bits as the finite-pad run, pads +0.0."""
    inp = workload_inputs("padded_8k")
    n = int(inp.valid_len[0])
    q, k, v, g, beta, _, vl = to_dev(inp)
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, None, vl)
    qn, kn, vn, gn, bn = (_nan_after(x, n) for x in (q, k, v, g, beta))
    o2, hT2 = gdn.gdn_chunk_fwd(qn, kn, vn, gn, bn, None, vl)
    sync()
    assert torch.equal(o, o2), "NaN pads changed the valid outputs"
    assert torch.equal(hT, hT2), "NaN pads changed the final state"
    assert int(torch.count_nonzero(o2[:, n:].contiguous().view(torch.int16))) == 0


@pytest.mark.parametrize("io,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 32)])
def test_padded_rows_nan_pads_small(io, d):
    """Both kernel paths, rows with different valid lengths (one ending inside a chunk,
    one with none valid), NaN at every padded token."""
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="nanpad", B=3, T=300, Hqk=2, H=4, dk=d, dv=d,
                            io=io, seed=901)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    lens = [300, 131, 0]
    vl = torch.tensor(lens, dtype=torch.int32, device=dev())
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, vl)
    xs = [x.clone() for x in (q, k, v, g, beta)]
    for b, n in enumerate(lens):
        for x in xs:
            x[b, n:] = float("nan")
    o2, hT2 = gdn.gdn_chunk_fwd(*xs, h0, vl)
    sync()
    assert torch.equal(o, o2) and torch.equal(hT, hT2)


@pytest.mark.parametrize("T,io", [(1000, "bf16"), (63, "bf16"), (4097, "bf16"), (1000, "f32"), (63, "f32")])
def test_ragged_tensor_end_followed_by_nan_memory(T, io):
    """A B = 1 problem whose T ends inside a chunk, passed as a view of the start of a
    longer buffer filled with NaN: the rows the last chunk covers past T must read as
    zero, not as the memory behind the tensor."""
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="ragged_view", B=1, T=T, Hqk=2, H=4, seed=902, io=io)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0)
    extra = 200

    def in_nan_buffer(x):
        buf = torch.full((1, T + extra) + tuple(x.shape[2:]), float("nan"), dtype=x.dtype, device=x.device)
        buf[:, :T] = x
        view = buf[:, :T]
        assert view.is_contiguous()
        return view

    o2, hT2 = gdn.gdn_chunk_fwd(*(in_nan_buffer(x) for x in (q, k, v, g, beta)), h0)
    sync()
    assert torch.equal(o, o2) and torch.equal(hT, hT2)


def test_varlen_nan_outside_sequences_and_between_chunks():
    """Packed sequences whose last chunks end inside a 64-token chunk, followed in the
    packed tensor by the next sequence and, after the last one, by NaN tokens that belong
    to no sequence: each sequence equals its own plain run bit for bit."""
    lens = [100, 64, 1, 250, 77]
    T_used = sum(lens)
    T = T_used + 150
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="varlen_nan", B=1, T=T, Hqk=2, H=4, seed=903)
    inp = make_inputs(w)
    q, k, v, g, beta, _, _ = to_dev(inp)
    xs = [_nan_after(x, T_used) for x in (q, k, v, g, beta)]
    cu_np = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(cu_np).to(dev())
    h0 = 0.1 * torch.randn((len(lens), 4, 128, 128), device=dev())
    o, hT = gdn.gdn_chunk_fwd_varlen(*xs, cu, max(lens), h0)
    sync()
    assert not torch.any(torch.isnan(o[:, :T_used].float()))
    for b in range(len(lens)):
        s, e = int(cu_np[b]), int(cu_np[b + 1])
        ob, hb = gdn.gdn_chunk_fwd(*(x[:, s:e].contiguous() for x in (q, k, v, g, beta)), h0[b:b + 1].contiguous())
        sync()
        assert torch.equal(o[:, s:e], ob), b
        assert torch.equal(hT[b:b + 1], hb), b


def test_segment_calls_nan_pads_give_the_same_bits():
    """The segment summary and apply on padded rows with NaN at the pads: M, S, outputs
    and final state equal the finite-pad run bit for bit."""
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="seg_nanpad", B=2, T=512, Hqk=2, H=4, seed=904)
    inp = make_inputs(w)
    q, k, v, g, beta, _, _ = to_dev(inp)
    lens = [400, 129]
    vl = torch.tensor(lens, dtype=torch.int32, device=dev())

    def run(xs):
        M, S, ws = gdn.gdn_segment_summary(*xs, 128, valid_len=vl)
        H_in, _, _ = gdn.gdn_summary_combine(M, S, None)
        o, hT = gdn.gdn_apply_initial_state(*xs, H_in, 128, ws, valid_len=vl)
        sync()
        return M, S, o, hT

    ref = run((q, k, v, g, beta))
    xs = [x.clone() for x in (q, k, v, g, beta)]
    for b, n in enumerate(lens):
        for x in xs:
            x[b, n:] = float("nan")
    got = run(xs)
    for nm, a, b_ in zip(("M", "S", "o", "hT"), ref, got):
        assert torch.equal(a, b_), nm
