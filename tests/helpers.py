"""Shared helpers for the tests (metrics and tiny random problems)."""
import numpy as np


def rel_l2(x, ref):
    """Relative L2 error over all elements, in fp64: |x - ref|_2 / |ref|_2."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)



def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_problem(rng, B=1, T=40, H=4, Hqk=2, dk=8, dv=12, gscale=0.3, h0=True, unit=True):
    """Small fp64 problem with L2-normalised q, k, g < 0 and beta in (0, 1)."""
    q = rng.standard_normal((B, T, Hqk, dk))
    k = rng.standard_normal((B, T, Hqk, dk))
    if unit:
        q = unit_rows(q) / np.sqrt(dk)
        k = unit_rows(k)
    v = rng.standard_normal((B, T, H, dv))
    g = -gscale * rng.random((B, T, H))
    beta = rng.random((B, T, H))
    s0 = 0.1 * rng.standard_normal((B, H, dk, dv)) if h0 else None
    return q, k, v, g, beta, s0


def _worst(num, den, floor):
    """Worst num/den over blocks; a block whose reference norm is below floor times the
    root-mean-square block norm is measured against that floor instead (its error must
    then be small in absolute terms), so that near-zero blocks neither dominate nor hide."""
    num = np.asarray(num, np.float64).ravel()
    den = np.asarray(den, np.float64).ravel()
    if den.size == 0:
        return 0.0, None
    rms = np.sqrt(np.mean(den ** 2))
    eff = np.maximum(den, floor * rms)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(eff > 0, num / eff, np.where(num > 0, np.inf, 0.0))
    i = int(np.argmax(rel))
    return float(rel[i]), i


def worst_token_block(x, ref, chunk=64, floor=0.1):
    """Worst relative L2 over the (b, 64-token chunk, h) blocks of a [B, T, H, D] tensor,
    in fp64. Returns (error, (b, chunk, h)). A tail shorter than 64 tokens is its own block."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    B, T, H, D = ref.shape
    NT = -(-T // chunk)
    pad = NT * chunk - T
    if pad:
        z = np.zeros((B, pad, H, D))
        x = np.concatenate([x, z], axis=1)
        ref = np.concatenate([ref, z], axis=1)
    d = (x - ref).reshape(B, NT, chunk, H, D)
    r = ref.reshape(B, NT, chunk, H, D)
    num = np.sqrt((d ** 2).sum(axis=(2, 4)))
    den = np.sqrt((r ** 2).sum(axis=(2, 4)))
    err, i = _worst(num, den, floor)
    return err, (None if i is None else tuple(int(v) for v in np.unravel_index(i, num.shape)))


def worst_lead_block(x, ref, nlead, floor=0.1):
    """Worst relative L2 over blocks indexed by the first nlead axes (per (b, h) of a state
    [B, H, dk, dv], per (b, h, segment) of a summary [B, H, P, ., .]). Returns (error, index)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    lead = ref.shape[:nlead]
    d = (x - ref).reshape(lead + (-1,))
    r = ref.reshape(lead + (-1,))
    num = np.sqrt((d ** 2).sum(axis=-1))
    den = np.sqrt((r ** 2).sum(axis=-1))
    err, i = _worst(num, den, floor)
    return err, (None if i is None else tuple(int(v) for v in np.unravel_index(i, num.shape)))


def scaled_max_abs(x, ref):
    """max |x - ref| / max |ref| over the whole tensor, in fp64."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.max(np.abs(ref)) if ref.size else 0.0
    e = np.max(np.abs(x - ref)) if ref.size else 0.0
    if m == 0.0:
        return 0.0 if e == 0.0 else float("inf")
    return float(e / m)
