"""Brute-force fp64 Gated DeltaNet by explicit transition-matrix products.

TEST INFRASTRUCTURE (tiny inputs only, T <= 16). It does not run the token
recurrence; it writes the state after token t as a sum of whole-matrix
products,

    A_t      = exp(g_t) (I - beta_t k_t k_t^T)            (dk x dk)
    Phi(t,s) = A_t A_{t-1} ... A_{s+1}                     (identity when s = t)
    S_t      = Phi(t,-1) S_0 + sum_{s<=t} Phi(t,s) beta_s k_s v_s^T
    o_t      = S_t^T q_t

and the segment summary as M = A_{last} ... A_{first}. This is the closed form of
the recurrence S_t = A_t S_{t-1} + beta_t k_t v_t^T (Gated DeltaNet, named in
hyper-parallel PR #1035 "linear attention cp"); the segment summary follows that
page's p2p mode, H_out = M @ H_in + S.
"""
from __future__ import annotations

import numpy as np


def _transitions(k, g, beta):
    T, dk = k.shape
    eye = np.eye(dk)
    return [np.exp(g[t]) * (eye - beta[t] * np.outer(k[t], k[t])) for t in range(T)]


def _phi(A, t, s):
    """A_t A_{t-1} ... A_{s+1}."""
    dk = A[0].shape[0] if A else 0
    out = np.eye(dk)
    for tau in range(s + 1, t + 1):
        out = A[tau] @ out
    return out


def gdn_fwd_head(q, k, v, g, beta, h0=None):
    """One (batch row, head): q,k [T,dk], v [T,dv], g,beta [T]. Returns (o [T,dv], S_T)."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    if T > 16:
        raise ValueError("brute force is for T <= 16")
    S0 = np.zeros((dk, dv)) if h0 is None else np.asarray(h0, np.float64)
    A = _transitions(k, g, beta)
    o = np.zeros((T, dv))
    S_t = S0
    for t in range(T):
        S_t = _phi(A, t, -1) @ S0
        for s in range(t + 1):
            S_t = S_t + _phi(A, t, s) @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = S_t.T @ q[t]
    return o, S_t


def gdn_fwd(q, k, v, g, beta, h0=None):
    """Batched over [B,T,H,...] with the grouped head map h -> h // (H // Hqk)."""
    B, T, Hqk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    rep = H // Hqk
    o = np.zeros((B, T, H, dv))
    hT = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            hq = h // rep
            o[b, :, h], hT[b, h] = gdn_fwd_head(q[b, :, hq], k[b, :, hq], v[b, :, h], g[b, :, h],
                                                beta[b, :, h], None if h0 is None else h0[b, h])
    return o, hT


def segment_m_head(k, g, beta):
    """M = A_{T-1} ... A_0 for one segment of one head."""
    k, g, beta = (np.asarray(x, np.float64) for x in (k, g, beta))
    A = _transitions(k, g, beta)
    return _phi(A, len(A) - 1, -1)
