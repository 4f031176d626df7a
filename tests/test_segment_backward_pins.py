"""Pins of oracle/segment_backward.py (the backward through summary, combine and apply):

- the combine's reverse recurrence against torch autograd of the combine's forward;
- the summaries' gradients against central finite differences (gradcheck), and the torch
  summaries against the C oracle's;
- the three backward pieces composed (apply, then combine, then summary) against the
  backward of the unsplit forward (oracle.backward), padding and a final-state gradient
  included: splitting the sequence into segments does not change the function, so it
  must not change its gradient;
- a planted mistake (M instead of M^T in the combine's reverse recurrence) fails that pin.
dk != dv throughout, so a transposed state or summary matrix shows."""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward, segment_backward as sb
from helpers import random_problem


def test_combine_bwd_matches_autograd_of_the_combine():
    rng = np.random.default_rng(31)
    B, H, P, dk, dv = 2, 3, 4, 5, 7
    M = 0.5 * rng.standard_normal((B, H, P, dk, dk))
    S = rng.standard_normal((B, H, P, dk, dv))
    h0 = rng.standard_normal((B, H, dk, dv))
    dH_in = rng.standard_normal((B, H, P, dk, dv))
    dhT = rng.standard_normal((B, H, dk, dv))
    tM, tS, th0 = (torch.tensor(x, requires_grad=True) for x in (M, S, h0))
    Hc, H_ins = th0, []
    for p in range(P):
        H_ins.append(Hc)
        Hc = tM[:, :, p] @ Hc + tS[:, :, p]
    loss = (torch.stack(H_ins, 2) * torch.tensor(dH_in)).sum() + (Hc * torch.tensor(dhT)).sum()
    loss.backward()
    H_in = torch.stack(H_ins, 2).detach().numpy()
    dM, dS, dh0 = sb.summary_combine_bwd(M, H_in, dH_in, dhT)
    for got, want in ((dM, tM.grad), (dS, tS.grad), (dh0, th0.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    # and the forward used here is the C oracle's combine
    H_in_c, _, hT_c = oracle.gdn_summary_combine(M, S, h0)
    np.testing.assert_allclose(H_in_c, H_in, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hT_c, Hc.detach().numpy(), rtol=1e-12, atol=1e-12)


def test_summaries_in_torch_match_the_c_oracle(rng):
    q, k, v, g, beta, _ = random_problem(rng, B=2, T=24, H=4, Hqk=2, dk=4, dv=6, h0=False)
    vl = np.array([24, 13], np.int32)
    M, S = sb.segment_summary_torch(*(torch.tensor(x) for x in (q, k, v, g, beta)), 8, vl)
    Mc, Sc = oracle.gdn_segment_summary(q, k, v, g, beta, 8, valid_len=vl)
    np.testing.assert_allclose(M.numpy(), Mc, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S.numpy(), Sc, rtol=1e-12, atol=1e-13)


def test_summary_gradients_match_finite_differences(rng):
    q, k, v, g, beta, _ = random_problem(rng, B=1, T=12, H=2, Hqk=1, dk=3, dv=4, h0=False)
    dM = rng.standard_normal((1, 2, 3, 3, 3))
    dS = rng.standard_normal((1, 2, 3, 3, 4))
    tq = torch.tensor(q)

    def f(k_, v_, g_, b_):
        M, S = sb.segment_summary_torch(tq, k_, v_, g_, b_, 4)
        return (M * torch.tensor(dM)).sum() + (S * torch.tensor(dS)).sum()

    args = tuple(torch.tensor(x, requires_grad=True) for x in (k, v, g, beta))
    assert torch.autograd.gradcheck(f, args, eps=1e-6, atol=1e-7, rtol=1e-5)
    got = sb.segment_summary_bwd(q, k, v, g, beta, 4, dM, dS)
    f(*args).backward()
    for x, a in zip(got[1:], args):
        np.testing.assert_allclose(x, a.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert not np.any(got[0])   # the summaries do not read q


def _composed(q, k, v, g, beta, h0, d_o, dhT, seg_len, vl, combine_bwd=sb.summary_combine_bwd):
    M, S = oracle.gdn_segment_summary(q, k, v, g, beta, seg_len, valid_len=vl)
    H_in, _, _ = oracle.gdn_summary_combine(M, S, h0)
    dq, dk, dv, dg, db, dH_in = sb.apply_initial_state_bwd(q, k, v, g, beta, H_in, seg_len, d_o, dhT, vl)
    dM, dS, dh0 = combine_bwd(M, H_in, dH_in, None)
    sq, sk, sv, sg, sb_ = sb.segment_summary_bwd(q, k, v, g, beta, seg_len, dM, dS, vl)
    return dq + sq, dk + sk, dv + sv, dg + sg, db + sb_, dh0


@pytest.mark.parametrize("padded", [False, True])
def test_segmented_backward_equals_the_unsplit_backward(rng, padded):
    B, T, L = 2, 30, 6
    q, k, v, g, beta, h0 = random_problem(rng, B=B, T=T, H=4, Hqk=2, dk=4, dv=5, gscale=0.1)
    vl = np.array([T, 17], np.int32) if padded else None
    d_o = rng.standard_normal(v.shape)
    dhT = rng.standard_normal(h0.shape)
    want = backward.gdn_bwd(q, k, v, g, beta, h0, d_o, dhT, vl)
    got = _composed(q, k, v, g, beta, h0, d_o, dhT, L, vl)
    for name, x, w in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, want):
        np.testing.assert_allclose(x, w, rtol=1e-9, atol=1e-11, err_msg=name)


def test_a_transposed_summary_matrix_in_the_combine_backward_is_caught(rng):
    B, T, L = 1, 24, 6
    q, k, v, g, beta, h0 = random_problem(rng, B=B, T=T, H=2, Hqk=1, dk=4, dv=5, gscale=0.05)
    d_o = rng.standard_normal(v.shape)
    want = backward.gdn_bwd(q, k, v, g, beta, h0, d_o)

    def wrong(M, H_in, dH_in, dhT=None):   # M where M^T belongs
        return sb.summary_combine_bwd(np.swapaxes(M, -1, -2), H_in, dH_in, dhT)

    got = _composed(q, k, v, g, beta, h0, d_o, None, L, None, combine_bwd=wrong)
    assert not np.allclose(got[5], want[5], rtol=1e-6, atol=1e-9)
