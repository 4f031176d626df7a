"""fp64 oracle of the Gated DeltaNet backward: the token-by-token forward written in
plain torch operations on the CPU, differentiated by torch's autograd.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke
check and the bench's CPU-baseline leg may use it. It shares no code with the
GPU library.

The gradients follow from the recurrence by the chain rule; the pages (hyper-parallel
issue #320, the test report for PR #1114, section 4) compare dq, dk, dv, dg, dbeta and
dH0 of their kernels against a reference, which is what this provides. The forward
here is the one the C oracle computes (decay, delta error on the decayed state, state
update, output from the updated state; padded tokens skipped with zero output), and a
pin checks that the two agree; finite differences pin the gradients
(tests/test_backward_pins.py).
"""
from __future__ import annotations

import numpy as np
import torch


def gdn_fwd_torch(q, k, v, g, beta, h0=None, valid_len=None):
    """Token-by-token forward on fp64 torch tensors (autograd-friendly).
    q, k [B,T,Hqk,dk]; v [B,T,H,dv]; g, beta [B,T,H]; h0 [B,H,dk,dv] or None.
    Returns (o [B,T,H,dv], hT [B,H,dk,dv])."""
    B, T, Hqk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    rep = H // Hqk
    qh = q.repeat_interleave(rep, dim=2)       # value head h reads query/key head h // rep
    kh = k.repeat_interleave(rep, dim=2)
    S = torch.zeros((B, H, dk, dv), dtype=q.dtype) if h0 is None else h0
    outs = []
    for t in range(T):
        live = torch.ones((B, 1, 1, 1), dtype=q.dtype)
        if valid_len is not None:
            live = torch.tensor([1.0 if t < int(valid_len[b]) else 0.0 for b in range(B)],
                                dtype=q.dtype).view(B, 1, 1, 1)
        kt, vt, qt = kh[:, t], v[:, t], qh[:, t]                     # [B,H,dk], [B,H,dv], [B,H,dk]
        Sd = torch.exp(g[:, t])[:, :, None, None] * S                # decay
        u = beta[:, t][:, :, None] * (vt - torch.einsum("bhkv,bhk->bhv", Sd, kt))   # delta error
        Sn = Sd + kt[:, :, :, None] * u[:, :, None, :]
        S = live * Sn + (1 - live) * S                               # padded tokens keep S
        outs.append(live[:, :, 0] * torch.einsum("bhkv,bhk->bhv", S, qt))
    return torch.stack(outs, dim=1), S


def gdn_bwd(q, k, v, g, beta, h0, d_o, dhT=None, valid_len=None):
    """Gradients (dq, dk, dv, dg, dbeta, dh0) of sum(o * d_o) + sum(hT * dhT), as fp64
    numpy arrays (dh0 is zero-shaped like h0 when h0 is None)."""
    B, H, dk, dv = q.shape[0], v.shape[2], q.shape[3], v.shape[3]
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    tq, tk, tv, tg, tb = map(t, (q, k, v, g, beta))
    th0 = t(h0 if h0 is not None else np.zeros((B, H, dk, dv)))
    o, hT = gdn_fwd_torch(tq, tk, tv, tg, tb, th0, valid_len)
    loss = (o * torch.tensor(np.asarray(d_o, dtype=np.float64))).sum()
    if dhT is not None:
        loss = loss + (hT * torch.tensor(np.asarray(dhT, dtype=np.float64))).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (tq, tk, tv, tg, tb, th0))
