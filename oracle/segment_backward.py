"""fp64 oracle of the backward through the segment calls: the gradients of the
per-segment affine summary (M, S), of the prefix combine and of apply-initial-state.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke check and
the bench's CPU-baseline leg may use it. It shares no code with the GPU library.

The segment calls follow hyper-parallel PR #1035 "linear attention cp" (the p2p and
all_gather modes): each segment p is summarised as H_out = M_p @ H_in + S_p, the
summaries are combined in order into every segment's incoming state H_in_p, and each
segment's token outputs are then computed from H_in_p. The same page's custom autograd
boundary passes the gradient of the state backwards across segments. Reverse mode through
the three calls therefore gives:

  apply:    per segment, the backward of the segment's recurrence started from H_in_p,
            with the output gradient of its tokens and, for the last segment, the gradient
            of the final state: input gradients of the segment and dH_in_p;
  combine:  H_p = M_p H_{p-1} + S_p, H_in_p = H_{p-1}, H_{-1} = h0, hT = H_{P-1}. With G the
            gradient of H_p (G = dhT for p = P - 1):  dS_p = G,  dM_p = G H_in_p^T, and the
            gradient of H_{p-1} is M_p^T G + dH_in_p; dh0 is that of H_{-1};
  summary:  S_p is the segment's recurrence from a zero state and M_p its homogeneous
            transition (zero values, identity start), so their gradients are the backward
            of those two runs with final-state gradients dS_p and dM_p.
The three together are the gradient of the unsplit forward (the pins check this).

The recurrences are written in plain torch fp64 operations (the token loop of
oracle.backward) and differentiated by autograd; the combine's reverse recurrence is
written out from its definition above.
"""
from __future__ import annotations

import numpy as np
import torch

from .backward import gdn_fwd_torch


def _t(x, grad=False):
    return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=grad)


def _seg_valid(valid_len, B, p, L):
    """Valid tokens of segment p of each row (tokens p L .. p L + L - 1 of the row)."""
    if valid_len is None:
        return None
    return np.clip(np.asarray(valid_len, np.int64) - p * L, 0, L)


def summary_combine_bwd(M, H_in, dH_in, dhT=None):
    """Reverse of the prefix combine. M [B,H,P,dk,dk], H_in [B,H,P,dk,dv] (the incoming
    states the combine produced), dH_in [B,H,P,dk,dv] (their gradients), dhT [B,H,dk,dv]
    or None (gradient of the combine's final state). Returns (dM, dS, dh0)."""
    M = np.asarray(M, np.float64)
    H_in = np.asarray(H_in, np.float64)
    dH_in = np.asarray(dH_in, np.float64)
    B, H, P, dk, dv = H_in.shape
    G = np.zeros((B, H, dk, dv)) if dhT is None else np.array(dhT, np.float64)
    dM = np.empty_like(M)
    dS = np.empty_like(H_in)
    for p in range(P - 1, -1, -1):
        dS[:, :, p] = G
        dM[:, :, p] = G @ np.swapaxes(H_in[:, :, p], -1, -2)
        G = np.swapaxes(M[:, :, p], -1, -2) @ G + dH_in[:, :, p]
    return dM, dS, G


def segment_summary_torch(q, k, v, g, beta, seg_len, valid_len=None):
    """Per-segment (M, S) with the token loop of oracle.backward (autograd-friendly torch
    tensors). M [B,H,P,dk,dk], S [B,H,P,dk,dv]."""
    B, T, Hqk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    P = T // seg_len
    eye = torch.eye(dk, dtype=q.dtype).expand(B, H, dk, dk)
    Ms, Ss = [], []
    for p in range(P):
        sl = slice(p * seg_len, (p + 1) * seg_len)
        vl = _seg_valid(valid_len, B, p, seg_len)
        _, S = gdn_fwd_torch(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], None, vl)
        zero_v = torch.zeros((B, seg_len, H, dk), dtype=q.dtype)
        _, Mp = gdn_fwd_torch(q[:, sl], k[:, sl], zero_v, g[:, sl], beta[:, sl], eye, vl)
        Ms.append(Mp)
        Ss.append(S)
    return torch.stack(Ms, dim=2), torch.stack(Ss, dim=2)


def segment_summary_bwd(q, k, v, g, beta, seg_len, dM=None, dS=None, valid_len=None):
    """Gradients (dq, dk, dv, dg, dbeta) of sum(M dM) + sum(S dS) over all segments, as fp64
    numpy arrays (dq is zero: the summaries do not read q)."""
    tq, tk, tv, tg, tb = (_t(x, True) for x in (q, k, v, g, beta))
    M, S = segment_summary_torch(tq, tk, tv, tg, tb, seg_len, valid_len)
    loss = torch.zeros((), dtype=torch.float64)
    if dM is not None:
        loss = loss + (M * _t(dM)).sum()
    if dS is not None:
        loss = loss + (S * _t(dS)).sum()
    loss.backward()
    return tuple(np.zeros(x.shape) if x.grad is None else x.grad.numpy() for x in (tq, tk, tv, tg, tb))


def apply_initial_state_bwd(q, k, v, g, beta, H_in, seg_len, d_o, dhT=None, valid_len=None):
    """Backward of apply-initial-state: every segment p runs from H_in[:, :, p]; d_o is the
    gradient of all token outputs and dhT (or None) that of the last segment's end state.
    Returns (dq, dk, dv, dg, dbeta, dH_in) as fp64 numpy arrays."""
    tq, tk, tv, tg, tb, tH = (_t(x, True) for x in (q, k, v, g, beta, H_in))
    B, T = q.shape[0], q.shape[1]
    P = T // seg_len
    td = _t(d_o)
    loss = torch.zeros((), dtype=torch.float64)
    for p in range(P):
        sl = slice(p * seg_len, (p + 1) * seg_len)
        vl = _seg_valid(valid_len, B, p, seg_len)
        o, hT = gdn_fwd_torch(tq[:, sl], tk[:, sl], tv[:, sl], tg[:, sl], tb[:, sl], tH[:, :, p], vl)
        loss = loss + (o * td[:, sl]).sum()
        if p == P - 1 and dhT is not None:
            loss = loss + (hT * _t(dhT)).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (tq, tk, tv, tg, tb, tH))
