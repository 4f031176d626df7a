"""Seeded synthetic inputs for the Gated DeltaNet forward.

This module draws random tensors and converts dtypes. It holds none of the
recurrence: both the GPU library and the fp64 oracle are fed from here, and
neither imports the other.

Recipe (numpy ``Generator(PCG64(seed))``, draws in float32, in this order):
  1. A_log[H]            = log U[1, 16]                      (per head)
  2. dt[H]               = exp U[ln 1e-3, ln 0.1];  dt_bias = log(expm1(dt))
  3. q_raw, k_raw        ~ N(0, 1)   [B, T, Hqk, dk]
  4. v                   ~ N(0, 1)   [B, T, H, dv]
  5. a, b                ~ N(0, 1)   [B, T, H]
  6. h0 (stateful only)  = 0.1 * N(0, 1)  [B, H, dk, dv]
Derived in float64: q = q_raw / |q_raw| / sqrt(dk), k = k_raw / |k_raw| (per token
and head), g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b). g and beta
are stored as float32; q, k, v in the I/O dtype (bf16 by round-to-nearest-even
from float32). Tokens at or past valid_len[b] get beta = 0 and g = 0.
The raw draws (q_raw, k_raw in the I/O dtype; a, b, and A_log, dt_bias cast to
float32) are kept too, as the inputs of the fused-prologue forward; there, pads
keep their random a and b.

The shapes follow the GDN-core workloads of hyper-parallel issue #320 (test
report for PR #1114): section 4.1 (16 query/key heads copied to 32 value heads,
head dim 128, 8K-32K tokens, with and without an initial state) and section 5.2
(B = 2, T = 8192, valid_length = 7777).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CHUNK = 64


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int
    Hqk: int
    H: int
    dk: int
    dv: int
    io: str                       # "f32" or "bf16"
    h0: Optional[str]             # None, "zeros" or "normal"
    seed: int
    valid_len: Optional[int] = None
    seg_len: Optional[int] = None
    # distribution overrides (slow-decay variant)
    a_log_range: tuple = (1.0, 16.0)
    dt_range: tuple = (1e-3, 0.1)
    b_mean: float = 0.0


WORKLOADS = {
    # tiny fp32 case: B=1, T=128, 4 -> 8 heads, d=16, zero initial state
    "tiny_f32": Workload("tiny_f32", 1, 128, 4, 8, 16, 16, "f32", "zeros", 1),
    # stateless bf16: T=8192, 16 -> 32 heads, d=128, no initial state, output only
    "stateless_8k": Workload("stateless_8k", 1, 8192, 16, 32, 128, 128, "bf16", None, 2),
    # stateful bf16: T=32768, 32 heads (16 query/key heads), d=128, h0 ~ 0.1 N(0,1)
    "stateful_32k": Workload("stateful_32k", 1, 32768, 16, 32, 128, 128, "bf16", "normal", 3),
    # the stateful sequence cut into 8 segments of 4096 (same seed, same inputs)
    "segmented_32k": Workload("segmented_32k", 1, 32768, 16, 32, 128, 128, "bf16", "normal", 3,
                              seg_len=4096),
    # padded batch: B=2, T=8192, valid length 7777 in both rows, no initial state
    "padded_8k": Workload("padded_8k", 2, 8192, 16, 32, 128, 128, "bf16", None, 5,
                          valid_len=7777),
}


def slow_decay(base: Workload, seed: int, seg_len: int = 256) -> Workload:
    """Variant whose incoming state still matters after a segment (beta ~ 0.05)."""
    return dataclasses.replace(base, name=base.name + "_slow", seed=seed, seg_len=seg_len,
                               a_log_range=(1.0, 1.0), dt_range=(1e-5, 1e-4), b_mean=-3.0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (((u >> 16) & 1) + 0x7FFF)
    return (rounded >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    w: Workload
    q: np.ndarray            # [B,T,Hqk,dk]  float32, or uint16 bf16 bits
    k: np.ndarray            # [B,T,Hqk,dk]
    v: np.ndarray            # [B,T,H,dv]
    g: np.ndarray            # [B,T,H] float32
    beta: np.ndarray         # [B,T,H] float32
    h0: Optional[np.ndarray]  # [B,H,dk,dv] float32 or None
    valid_len: Optional[np.ndarray]  # [B] int32 or None
    raw: Optional[dict] = None       # q_raw, k_raw (I/O dtype), a, b [B,T,H], A_log, dt_bias [H] (float32)

    def io_f32(self, name: str) -> np.ndarray:
        x = getattr(self, name)
        return bf16_bits_to_f32(x) if self.w.io == "bf16" else x

    def f64(self):
        """Exact float64 copies of what the GPU sees: (q, k, v, g, beta, h0)."""
        q, k, v = (self.io_f32(n).astype(np.float64) for n in ("q", "k", "v"))
        h0 = None if self.h0 is None else self.h0.astype(np.float64)
        return q, k, v, self.g.astype(np.float64), self.beta.astype(np.float64), h0

    def raw_f64(self):
        """Exact float64 copies of the fused-prologue inputs:
        (q_raw, k_raw, v, a, b, A_log, dt_bias, h0)."""
        r = self.raw
        io = (lambda x: bf16_bits_to_f32(x)) if self.w.io == "bf16" else (lambda x: x)
        h0 = None if self.h0 is None else self.h0.astype(np.float64)
        return (io(r["q_raw"]).astype(np.float64), io(r["k_raw"]).astype(np.float64),
                self.io_f32("v").astype(np.float64), r["a"].astype(np.float64), r["b"].astype(np.float64),
                r["A_log"].astype(np.float64), r["dt_bias"].astype(np.float64), h0)


def _softplus(x):
    return np.logaddexp(0.0, x)


def make_inputs(w: Workload, T: Optional[int] = None, B: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload ``w`` (optionally with T or B overridden)."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lo, hi = w.a_log_range
    a_log = np.log(rng.uniform(lo, hi, size=w.H).astype(np.float32)).astype(np.float64)
    dlo, dhi = w.dt_range
    dt = np.exp(rng.uniform(math.log(dlo), math.log(dhi), size=w.H).astype(np.float32))
    dt_bias = np.log(np.expm1(dt.astype(np.float64)))
    q_raw = rng.standard_normal((B, T, w.Hqk, w.dk), dtype=np.float32)
    k_raw = rng.standard_normal((B, T, w.Hqk, w.dk), dtype=np.float32)
    v = rng.standard_normal((B, T, w.H, w.dv), dtype=np.float32)
    a = rng.standard_normal((B, T, w.H), dtype=np.float32)
    b = rng.standard_normal((B, T, w.H), dtype=np.float32) + np.float32(w.b_mean)
    h0 = None
    if w.h0 == "normal":
        h0 = (0.1 * rng.standard_normal((B, w.H, w.dk, w.dv), dtype=np.float32)).astype(np.float32)
    elif w.h0 == "zeros":
        h0 = np.zeros((B, w.H, w.dk, w.dv), np.float32)

    q64 = q_raw.astype(np.float64)
    q64 /= np.linalg.norm(q64, axis=-1, keepdims=True)
    q64 /= math.sqrt(w.dk)
    k64 = k_raw.astype(np.float64)
    k64 /= np.linalg.norm(k64, axis=-1, keepdims=True)
    g = (-np.exp(a_log) * _softplus(a.astype(np.float64) + dt_bias)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-b.astype(np.float64)))).astype(np.float32)

    valid = None
    if w.valid_len is not None:
        valid = np.full((B,), min(w.valid_len, T), np.int32)
        for r in range(B):
            g[r, valid[r]:] = 0.0
            beta[r, valid[r]:] = 0.0

    q32, k32 = q64.astype(np.float32), k64.astype(np.float32)
    if w.io == "bf16":
        qs, ks, vs = f32_to_bf16_bits(q32), f32_to_bf16_bits(k32), f32_to_bf16_bits(v)
        qr, kr = f32_to_bf16_bits(q_raw), f32_to_bf16_bits(k_raw)
    elif w.io == "f32":
        qs, ks, vs = q32, k32, v
        qr, kr = q_raw, k_raw
    else:
        raise ValueError(w.io)
    raw = {"q_raw": qr, "k_raw": kr, "a": a, "b": b, "A_log": a_log.astype(np.float32),
           "dt_bias": dt_bias.astype(np.float32)}
    return Inputs(w, qs, ks, vs, g, beta, h0, valid, raw)
