"""fp64 NumPy model of the chunked (UT / WY) evaluation that the GPU kernels use.

Test aid only -- not the oracle, and not GPU code. It exists so that the chunk
algebra the kernels implement can be checked against the token-by-token oracle
in fp64 before any GPU is involved, and so that a kernel stage can be debugged
on the CPU. For one head and one chunk of C = 64 tokens with incoming state S:

    Gam_i   = g_1 + ... + g_i                     (chunk-local cumulative log-decay)
    A_ij    = beta_i exp(Gam_i - Gam_j) k_i . k_j  for i > j, else 0
    Tinv    = (I + A)^{-1}                         (unit lower triangular)
    That    = Tinv diag(beta)
    X       = V - diag(exp Gam) K S
    U       = That X                               (the delta-rule errors u_i)
    O       = diag(exp Gam) Q S + P U,  P_ij = (q_i . k_j) exp(Gam_i - Gam_j), j <= i
    S_next  = exp(Gam_C) S + (diag(exp(Gam_C - Gam)) K)^T U

The summary matrix M of a segment is the same pass with V = 0 and S = I.
"""
from __future__ import annotations

import numpy as np

C = 64


def _decay_matrix(gam, inclusive):
    """exp(Gam_i - Gam_j) on (i > j) or (i >= j); zero elsewhere, masked before exp."""
    n = gam.shape[0]
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    keep = (i >= j) if inclusive else (i > j)
    diff = np.where(keep, gam[:, None] - gam[None, :], -np.inf)
    return np.exp(diff)


def chunk_prepare(k, q, g, beta):
    """Per-chunk quantities that do not depend on the state."""
    gam = np.cumsum(g)
    kk = k @ k.T
    A = beta[:, None] * _decay_matrix(gam, inclusive=False) * kk
    n = k.shape[0]
    Tinv = np.linalg.solve(np.eye(n) + A, np.eye(n))
    That = Tinv * beta[None, :]
    P = _decay_matrix(gam, inclusive=True) * (q @ k.T)
    return gam, That, P


def chunk_step(S, k, q, v, gam, That, P, want_out=True):
    eg = np.exp(gam)
    X = v - eg[:, None] * (k @ S)
    U = That @ X
    O = eg[:, None] * (q @ S) + P @ U if want_out else None
    egc = np.exp(gam[-1] - gam)
    S_next = np.exp(gam[-1]) * S + (egc[:, None] * k).T @ U
    return O, S_next


def fwd_head(q, k, v, g, beta, S0, nvalid=None):
    """One head: q,k [T,dk], v [T,dv], g,beta [T]. Pads (t >= nvalid) are zeroed."""
    T = k.shape[0]
    nvalid = T if nvalid is None else nvalid
    q, k, v = q.copy(), k.copy(), v.copy()
    g, beta = g.copy(), beta.copy()
    q[nvalid:] = 0
    k[nvalid:] = 0
    v[nvalid:] = 0
    g[nvalid:] = 0
    beta[nvalid:] = 0
    S = S0.copy()
    o = np.zeros_like(v)
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        gam, That, P = chunk_prepare(k[sl], q[sl], g[sl], beta[sl])
        o[sl], S = chunk_step(S, k[sl], q[sl], v[sl], gam, That, P)
    o[nvalid:] = 0
    return o, S


def segment_m_head(k, g, beta):
    dk = k.shape[1]
    S = np.eye(dk)
    zero_v = np.zeros((k.shape[0], dk))
    for c0 in range(0, k.shape[0], C):
        sl = slice(c0, min(c0 + C, k.shape[0]))
        gam, That, P = chunk_prepare(k[sl], k[sl], g[sl], beta[sl])
        _, S = chunk_step(S, k[sl], k[sl], zero_v[sl], gam, That, P, want_out=False)
    return S
