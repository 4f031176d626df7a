"""Pins for the backward oracle: its forward equals the C token oracle, its gradients
equal central finite differences of that forward, and closed forms hold where the
recurrence degenerates (beta = g = 0: o_t = h0^T q_t)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward
from helpers import random_problem, rel_l2


def test_torch_forward_equals_the_c_oracle(rng):
    q, k, v, g, beta, h0 = random_problem(rng, B=2, T=45, H=4, Hqk=2, dk=8, dv=6)
    vl = np.array([45, 30], np.int32)
    o_c, hT_c = oracle.gdn_fwd(q, k, v, g, beta, h0, valid_len=vl)
    T = lambda x: torch.tensor(x)
    o_t, hT_t = backward.gdn_fwd_torch(T(q), T(k), T(v), T(g), T(beta), T(h0), vl)
    assert rel_l2(o_t.numpy(), o_c) < 1e-13 and rel_l2(hT_t.numpy(), hT_c) < 1e-13
    assert np.all(o_t.numpy()[1, 30:] == 0.0)


def test_gradients_match_finite_differences(rng):
    q, k, v, g, beta, h0 = random_problem(rng, B=1, T=6, H=2, Hqk=1, dk=3, dv=2, gscale=0.5)
    vl = np.array([5], np.int32)
    T = lambda x: torch.tensor(x, requires_grad=True)
    args = tuple(map(T, (q, k, v, g, beta, h0)))

    def f(*a):
        o, hT = backward.gdn_fwd_torch(*a, valid_len=vl)
        return o, hT

    assert torch.autograd.gradcheck(f, args, eps=1e-6, atol=1e-8, rtol=1e-6)


def test_gradients_with_output_and_state_cotangents(rng):
    """gdn_bwd returns the gradient of sum(o * d_o) + sum(hT * dhT): one entry checked
    against a central difference of that scalar."""
    q, k, v, g, beta, h0 = random_problem(rng, B=1, T=9, H=2, Hqk=1, dk=4, dv=3, gscale=0.4)
    d_o = rng.standard_normal((1, 9, 2, 3))
    dhT = rng.standard_normal((1, 2, 4, 3))
    grads = backward.gdn_bwd(q, k, v, g, beta, h0, d_o, dhT)

    def loss(**over):
        a = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)
        a.update(over)
        o, hT = oracle.gdn_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"])
        return float(np.sum(o * d_o) + np.sum(hT * dhT))

    eps = 1e-6
    for name, idx, gi in (("k", (0, 3, 0, 1), 1), ("g", (0, 4, 1), 3), ("beta", (0, 7, 0), 4),
                          ("h0", (0, 1, 2, 1), 5), ("q", (0, 8, 0, 3), 0), ("v", (0, 2, 1, 0), 2)):
        base = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)[name]
        up, dn = base.copy(), base.copy()
        up[idx] += eps
        dn[idx] -= eps
        fd = (loss(**{name: up}) - loss(**{name: dn})) / (2 * eps)
        assert abs(fd - grads[gi][idx]) < 1e-6 * max(1.0, abs(fd)), name


def test_closed_form_without_decay_or_update(rng):
    """beta = g = 0: o_t = h0^T q_t, so dq_t = h0 d_o_t (summed over the grouped heads),
    dh0 = sum_t q_t d_o_t^T, dv = dk = 0."""
    q, k, v, g, beta, h0 = random_problem(rng, B=1, T=7, H=4, Hqk=2, dk=5, dv=3)
    g[:] = 0.0
    beta[:] = 0.0
    d_o = rng.standard_normal((1, 7, 4, 3))
    dq, dk, dv, dg, db, dh0 = backward.gdn_bwd(q, k, v, g, beta, h0, d_o)
    rep = 2
    for hq in range(2):
        want = sum(np.einsum("kv,tv->tk", h0[0, h], d_o[0, :, h]) for h in range(hq * rep, hq * rep + rep))
        assert np.max(np.abs(dq[0, :, hq] - want)) < 1e-13
    for h in range(4):
        want = np.einsum("tk,tv->kv", q[0, :, h // rep], d_o[0, :, h])
        assert np.max(np.abs(dh0[0, h] - want)) < 1e-13
    assert np.all(dv == 0) and np.all(dk == 0)
