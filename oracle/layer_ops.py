"""fp64 oracles of the two streaming layer steps around the Gated DeltaNet core.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke check
and the bench's CPU-baseline leg may use it. It shares no code with the GPU library.

The pages' layer (hyper-parallel PR #1035 "linear attention cp", section "What does
this PR do") runs a depthwise Conv1D on the projected Q/K/V before the Gated DeltaNet
(in p2p mode only the Conv1D's left halo crosses between neighbouring ranks) and
RMSNorm with gating on its output. The pages give neither formula; these are the
published Gated DeltaNet layer's: a causal depthwise convolution with SiLU, and a
root-mean-square norm over the head dim multiplied by a weight and by SiLU of a gate.
Pins: tests/test_layer_ops_pins.py.
"""
from __future__ import annotations

import numpy as np


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def causal_conv1d(x, w, bias=None, x_prev=None, apply_silu=True):
    """y[b,t,c] = act(bias[c] + sum_j w[c,j] x[b, t-K+1+j, c]); tokens before t = 0 come
    from x_prev [B, K-1, C] (zeros if None). x [B,T,C], w [C,K]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, C = x.shape
    K = w.shape[1]
    prev = np.zeros((B, K - 1, C)) if x_prev is None else np.asarray(x_prev, dtype=np.float64)
    xx = np.concatenate([prev, x], axis=1)            # token t of x is row t + K - 1
    y = np.zeros((B, T, C)) if bias is None else np.broadcast_to(np.asarray(bias, np.float64), (B, T, C)).copy()
    for j in range(K):
        y += w[:, j] * xx[:, j:j + T]
    return silu(y) if apply_silu else y


def gated_rmsnorm(o, z, weight, eps):
    """o / sqrt(mean(o^2 over the last axis) + eps) * weight * silu(z)."""
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * np.asarray(weight, np.float64) * silu(z)
