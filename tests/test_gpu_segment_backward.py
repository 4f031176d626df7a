"""GPU parity of the backward through the segment calls (gdn_apply_initial_state_bwd,
gdn_summary_combine_bwd, gdn_segment_summary_bwd) against oracle/segment_backward.py on the
same seeded inputs, and of their composition against the backward of the unsplit forward
(the fp64 oracle, and gdn_chunk_bwd on the GPU). The state gradient passes backwards across
the segment boundaries the way hyper-parallel PR #1035's p2p mode passes it across ranks."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import backward, segment_backward as sb
from gpu_common import TOL_BF16, TOL_F32, dev, np_f64, sync, to_dev, workload_inputs
from helpers import rel_l2
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, slow_decay

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta")


def check(x, ref, tol, what):
    xn = np_f64(x) if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    err = rel_l2(xn, ref)
    print("%s rel-L2 %.3e (bound %.0e)" % (what, err, tol))
    assert np.all(np.isfinite(xn)), what
    assert err <= tol, "%s rel-L2 %.3e > %.0e" % (what, err, tol)


def output_grad(inp, seed):
    """A seeded output gradient in the io dtype: the device tensor and the values the GPU
    sees, as fp64 for the oracle."""
    rng = np.random.default_rng(seed)
    d_o = rng.standard_normal(inp.v.shape).astype(np.float32)
    if inp.w.io == "bf16":
        bits = f32_to_bf16_bits(d_o)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev()), bf16_bits_to_f32(bits).astype(np.float64)
    return torch.from_numpy(d_o).to(dev()), d_o.astype(np.float64)


CASES = [
    # name, io, dk, dv, B, T, Hqk, H, seg_len, valid
    ("bf16_d128", "bf16", 128, 128, 1, 256, 1, 2, 64, None),
    ("bf16_d128_padded", "bf16", 128, 128, 2, 192, 2, 4, 64, 101),
    ("f32_dk16_dv32", "f32", 16, 32, 1, 256, 2, 4, 128, None),
]


def call_tol(case):
    """The apply and summary backward of bf16 heads of 128 run the chunked matrix-core backward
    (bf16 operands, fp32 accumulation): the pages' bf16 bound on gradients (issue #320,
    section 4.2). Every other shape runs fp32 arithmetic: 1e-4. The combine is fp32 always."""
    _, io, dk, dv = case[:4]
    return TOL_BF16 if (io == "bf16" and dk == 128 and dv == 128) else TOL_F32


def case_inputs(case, seed):
    name, io, dk, dv, B, T, Hqk, H, L, valid = case
    w = dataclasses.replace(slow_decay(WORKLOADS["stateful_32k"], seed=seed, seg_len=L), name="segbwd_" + name, B=B,
                            T=T, Hqk=Hqk, H=H, dk=dk, dv=dv, io=io, valid_len=valid)
    return make_inputs(w)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_each_backward_call_matches_the_oracle(case):
    L = case[8]
    inp = case_inputs(case, 700)
    q, k, v, g, beta, h0, vl = to_dev(inp)
    qf, kf, vf, gf, bf, h0f = inp.f64()
    d_o_t, d_o = output_grad(inp, 701)
    rng = np.random.default_rng(702)
    dhT = (0.1 * rng.standard_normal(h0f.shape)).astype(np.float32)
    # forward through the segment calls on the GPU; the oracle backward uses the GPU's own
    # H_in, so each call is checked on exactly the inputs it received
    M, S, ws = gdn.gdn_segment_summary(q, k, v, g, beta, L, valid_len=vl)
    H_in, _, _ = gdn.gdn_summary_combine(M, S, h0)
    sync()
    Hf, Mf = np_f64(H_in), np_f64(M)
    # 1. apply
    got = gdn.gdn_apply_initial_state_bwd(q, k, v, g, beta, H_in, L, d_o_t, torch.from_numpy(dhT).to(dev()), vl)
    sync()
    ref = sb.apply_initial_state_bwd(qf, kf, vf, gf, bf, Hf, L, d_o, dhT.astype(np.float64), inp.valid_len)
    tol = call_tol(case)
    for nm, x, r in zip(NAMES + ("dH_in",), got, ref):
        check(x, r, tol, case[0] + " apply " + nm)
    dH_in = got[5]
    # 2. combine
    dM, dS, dh0 = gdn.gdn_summary_combine_bwd(M, H_in, dH_in)
    sync()
    rM, rS, rh0 = sb.summary_combine_bwd(Mf, Hf, np_f64(dH_in))
    for nm, x, r in (("dM", dM, rM), ("dS", dS, rS), ("dh0", dh0, rh0)):
        check(x, r, TOL_F32, case[0] + " combine " + nm)
    # 3. summaries (written, not accumulated)
    got = gdn.gdn_segment_summary_bwd(q, k, v, g, beta, L, dM, dS, valid_len=vl)
    sync()
    ref = sb.segment_summary_bwd(qf, kf, vf, gf, bf, L, np_f64(dM), np_f64(dS), inp.valid_len)
    assert int(torch.count_nonzero(got[0])) == 0, "the summaries do not read q"
    for nm, x, r in zip(NAMES[1:], got[1:], ref[1:]):
        check(x, r, tol, case[0] + " summary " + nm)
    if inp.valid_len is not None:
        for b in range(inp.w.B):
            n = int(inp.valid_len[b])
            for x in got:
                assert torch.all(x[b, n:] == 0)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_composed_segment_backward_equals_the_unsplit_backward(case):
    """apply_bwd, then combine_bwd, then summary_bwd accumulating onto apply's gradients:
    the gradient of the unsplit forward (fp64 oracle and gdn_chunk_bwd), the summaries'
    share nonzero (slow decay keeps the carried state's weight large). On bf16 heads of 128
    the backward calls run the matrix-core backward and the incoming states H_in come out
    of the bf16 matrix-core summaries: the bf16 bound applies; fp32 shapes stay at 1e-4."""
    L = case[8]
    inp = case_inputs(case, 710)
    q, k, v, g, beta, h0, vl = to_dev(inp)
    qf, kf, vf, gf, bf, h0f = inp.f64()
    d_o_t, d_o = output_grad(inp, 711)
    rng = np.random.default_rng(712)
    dhT = (0.1 * rng.standard_normal(h0f.shape)).astype(np.float32)
    dhT_t = torch.from_numpy(dhT).to(dev())
    M, S, _ = gdn.gdn_segment_summary(q, k, v, g, beta, L, valid_len=vl)
    H_in, _, _ = gdn.gdn_summary_combine(M, S, h0)
    *grads, dH_in = gdn.gdn_apply_initial_state_bwd(q, k, v, g, beta, H_in, L, d_o_t, dhT_t, vl)
    apply_dk = grads[1].clone()
    dM, dS, dh0 = gdn.gdn_summary_combine_bwd(M, H_in, dH_in)
    gdn.gdn_segment_summary_bwd(q, k, v, g, beta, L, dM, dS, grads=grads, valid_len=vl)
    unsplit = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o_t, dhT_t, vl)
    sync()
    share = (grads[1] - apply_dk).norm() / grads[1].norm()
    print("%s summaries' share of dk: %.3f" % (case[0], share.item()))
    assert share > 0.05
    ref = backward.gdn_bwd(qf, kf, vf, gf, bf, h0f, d_o, dhT.astype(np.float64), inp.valid_len)
    tol = TOL_BF16 if inp.w.io == "bf16" else TOL_F32
    for nm, x, u, r in zip(NAMES + ("dh0",), list(grads) + [dh0], unsplit, ref):
        check(x, r, tol, case[0] + " composed " + nm + " vs oracle")
        check(x, np_f64(u), tol, case[0] + " composed " + nm + " vs unsplit GPU backward")


def test_composed_segment_backward_stateless_8k():
    """The stateless 8K workload (32 value heads of 128, bf16) in 4 segments of 2048: the
    composed segment backward against the unsplit GPU backward over all gradients (bf16
    bound: the incoming states come from the bf16 summaries)."""
    inp = workload_inputs("stateless_8k")
    q, k, v, g, beta, _, _ = to_dev(inp)
    d_o_t, _ = output_grad(inp, 720)
    L = 2048
    M, S, _ = gdn.gdn_segment_summary(q, k, v, g, beta, L)
    H_in, _, _ = gdn.gdn_summary_combine(M, S, None)
    *grads, dH_in = gdn.gdn_apply_initial_state_bwd(q, k, v, g, beta, H_in, L, d_o_t)
    dM, dS, dh0 = gdn.gdn_summary_combine_bwd(M, H_in, dH_in)
    gdn.gdn_segment_summary_bwd(q, k, v, g, beta, L, dM, dS, grads=grads)
    unsplit = gdn.gdn_chunk_bwd(q, k, v, g, beta, None, d_o_t)
    sync()
    for nm, x, u in zip(NAMES + ("dh0",), list(grads) + [dh0], unsplit):
        check(x, np_f64(u), TOL_BF16, "8k composed " + nm + " vs unsplit")
