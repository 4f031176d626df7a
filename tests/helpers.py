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
