"""fp64 oracle of the Gated DeltaNet layer's input prologue.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke
check and the bench's CPU-baseline leg may use it. It shares no code with the
GPU library.

Before the recurrence, each rank of the pages' context-parallel layer projects
Q, K, V, B and A on its tokens and feeds them to the Gated DeltaNet (PR #1035
"linear attention cp", section "What does this PR do", modes ulysses / p2p);
issue #320's gradient checks name the decay-gate parameters A_log and dt_bias
(test plan, comparison metrics). The pages do not print the formulas; this
follows the published Gated DeltaNet layer (Yang, Kautz and Hatamizadeh, 2025),
as the workload recipe states it:
    q = q_scale * q_raw / |q_raw|,  k = k_raw / |k_raw|   (L2 norm over the head dim,
                                                           per token and head)
    g = -exp(A_log[h]) * softplus(a + dt_bias[h]),  softplus(x) = log(1 + e^x)
    beta = sigmoid(b) = 1 / (1 + e^-b)
Reading: a zero row stays zero (the norm is clamped at 1e-12, as torch's
F.normalize does).

Pins: tests/test_oracle_pins.py (closed forms of softplus and sigmoid, unit rows,
invariance of the forward under positive row scaling, agreement with the input
generator's own derivation of q, k, g and beta).
"""
from __future__ import annotations

import numpy as np

from . import gdn_fwd

NORM_EPS = 1e-12


def l2_normalise(x, eps=NORM_EPS):
    """x / max(|x|, eps) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def softplus(x):
    """log(1 + e^x), written as max(x, 0) + log(1 + e^-|x|) so that large x does not overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):   # e^-x = inf for x < -709 gives the exact limit 0
        return 1.0 / (1.0 + np.exp(-x))


def gdn_prologue(q_raw, k_raw, a, b, A_log, dt_bias, q_scale):
    """(q, k, g, beta) in fp64 from the raw layer inputs.
    q_raw, k_raw [B,T,Hqk,dk]; a, b [B,T,H]; A_log, dt_bias [H]."""
    q = q_scale * l2_normalise(q_raw)
    k = l2_normalise(k_raw)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    g = -np.exp(A_log) * softplus(np.asarray(a, dtype=np.float64) + dt_bias)
    beta = sigmoid(b)
    return q, k, g, beta


def gdn_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, q_scale, h0=None, valid_len=None,
                     want_state=True):
    """The prologue, then the token-by-token forward. Tokens at or past valid_len[b] are
    padding (treated as beta = 0, g = 0 whatever a and b hold)."""
    q, k, g, beta = gdn_prologue(q_raw, k_raw, a, b, A_log, dt_bias, q_scale)
    return gdn_fwd(q, k, v, g, beta, h0, valid_len, want_state)
