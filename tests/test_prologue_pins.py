"""Pins for the fp64 oracle of the fused input prologue (q/k L2 norm, q scale,
decay gate g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)).

Each pin ties the oracle to something other than itself: closed forms of
softplus and sigmoid at points where they are known exactly, unit rows, the
invariance of the whole forward under positive scaling of q_raw and k_raw rows,
and the seeded input generator, which derives q, k, g and beta from the same
draws in code of its own. Dropping the exp of A_log, the dt_bias shift, the q
scale, or taking softplus for sigmoid fails one of them.
"""
import math

import numpy as np
import pytest

from oracle import prologue
from helpers import rel_l2
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs


def test_softplus_and_sigmoid_closed_forms():
    assert prologue.softplus(0.0) == math.log(2.0)
    assert prologue.sigmoid(0.0) == 0.5
    # softplus(x) - softplus(-x) = x and sigmoid(x) + sigmoid(-x) = 1
    x = np.linspace(-30.0, 30.0, 121)
    assert np.max(np.abs(prologue.softplus(x) - prologue.softplus(-x) - x)) < 1e-13
    assert np.max(np.abs(prologue.sigmoid(x) + prologue.sigmoid(-x) - 1.0)) < 1e-15
    # no overflow far out: softplus(x) -> x, sigmoid -> 1 / 0
    assert prologue.softplus(800.0) == 800.0 and prologue.softplus(-800.0) == 0.0
    assert prologue.sigmoid(800.0) == 1.0 and prologue.sigmoid(-800.0) == 0.0
    # log(1 + e^x) at x = log(e - 1) is exactly 1
    assert abs(prologue.softplus(math.log(math.e - 1.0)) - 1.0) < 1e-15


def test_gate_closed_forms():
    rng = np.random.default_rng(7)
    H = 5
    A_log = rng.uniform(0.0, 2.8, H)
    dt_bias = rng.uniform(-7.0, -2.0, H)
    # a = -dt_bias: softplus(0) = ln 2, so g = -exp(A_log) ln 2 exactly per head
    a = np.broadcast_to(-dt_bias, (1, 3, H)).copy()
    b = np.zeros((1, 3, H))
    q_raw = rng.standard_normal((1, 3, 1, 4))
    _, _, g, beta = prologue.gdn_prologue(q_raw, q_raw, a, b, A_log, dt_bias, 0.5)
    assert np.max(np.abs(g - (-np.exp(A_log) * math.log(2.0)))) < 1e-15
    assert np.all(beta == 0.5)
    # A_log = 0, a + dt_bias = log(e - 1): g = -1
    a2 = np.full((1, 3, H), math.log(math.e - 1.0)) - dt_bias
    _, _, g2, _ = prologue.gdn_prologue(q_raw, q_raw, a2, b, np.zeros(H), dt_bias, 0.5)
    assert np.max(np.abs(g2 + 1.0)) < 1e-14
    # g < 0 always, and more negative for larger a
    a3 = rng.standard_normal((1, 50, H))
    _, _, g3, beta3 = prologue.gdn_prologue(np.ones((1, 50, 1, 4)), np.ones((1, 50, 1, 4)), a3,
                                            a3, A_log, dt_bias, 1.0)
    assert np.all(g3 < 0)
    order = np.argsort(a3[0, :, 0])
    assert np.all(np.diff(g3[0, order, 0]) <= 0)
    assert np.all((beta3 > 0) & (beta3 < 1))


def test_rows_are_unit_and_zero_rows_stay_zero():
    rng = np.random.default_rng(8)
    q_raw = rng.standard_normal((2, 9, 3, 16)) * rng.uniform(0.01, 100.0, (2, 9, 3, 1))
    k_raw = q_raw[:, ::-1].copy()
    k_raw[0, 4, 1] = 0.0
    z = np.zeros((2, 9, 3))
    q, k, _, _ = prologue.gdn_prologue(q_raw, k_raw, z, z, np.zeros(3), np.zeros(3), 0.25)
    nq = np.linalg.norm(q, axis=-1)
    nk = np.linalg.norm(k, axis=-1)
    assert np.max(np.abs(nq - 0.25)) < 1e-15
    assert np.all(k[0, 4, 1] == 0.0)
    nk[0, 4, 1] = 1.0
    assert np.max(np.abs(nk - 1.0)) < 1e-15
    # direction is kept: q is a positive multiple of q_raw
    cos = np.sum(q * q_raw, axis=-1) / (nq * np.linalg.norm(q_raw, axis=-1))
    assert np.max(np.abs(cos - 1.0)) < 1e-14


def test_forward_is_invariant_under_positive_row_scaling():
    rng = np.random.default_rng(9)
    B, T, Hqk, H, d = 1, 70, 2, 4, 8
    q_raw = rng.standard_normal((B, T, Hqk, d))
    k_raw = rng.standard_normal((B, T, Hqk, d))
    v = rng.standard_normal((B, T, H, d))
    a = rng.standard_normal((B, T, H))
    b = rng.standard_normal((B, T, H))
    A_log = np.log(rng.uniform(1, 16, H))
    dt_bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, H)))
    h0 = 0.1 * rng.standard_normal((B, H, d, d))
    o, hT = prologue.gdn_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, d ** -0.5, h0)
    cq = rng.uniform(0.1, 10.0, (B, T, Hqk, 1))
    ck = rng.uniform(0.1, 10.0, (B, T, Hqk, 1))
    o2, hT2 = prologue.gdn_fwd_prologue(cq * q_raw, ck * k_raw, v, a, b, A_log, dt_bias, d ** -0.5, h0)
    assert rel_l2(o2, o) < 1e-13 and rel_l2(hT2, hT) < 1e-13
    # the q scale scales the output and nothing else
    o3, hT3 = prologue.gdn_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, 3 * d ** -0.5, h0)
    assert rel_l2(o3, 3 * o) < 1e-13 and rel_l2(hT3, hT) < 1e-15


@pytest.mark.parametrize("name", ["stateless_8k", "tiny_f32"])
def test_prologue_matches_the_input_generator(name):
    """The generator derives q, k, g, beta from its raw draws with its own code; the
    prologue oracle on the same draws must agree up to the generator's final roundings
    (float32 for g, beta; the I/O dtype for q, k) and its float32 cast of A_log, dt_bias."""
    w = WORKLOADS[name]
    inp = make_inputs(w, T=min(w.T, 200))
    q_raw, k_raw, v, a, b, A_log, dt_bias, _ = inp.raw_f64()
    q, k, g, beta = prologue.gdn_prologue(q_raw, k_raw, a, b, A_log, dt_bias, w.dk ** -0.5)
    io_tol = 4e-3 if w.io == "bf16" else 1e-6
    if w.io == "bf16":
        # the generator normalises the float32 draws; the prologue sees them rounded to bf16
        io_tol = 8e-3
    assert rel_l2(q, inp.io_f32("q")) < io_tol
    assert rel_l2(k, inp.io_f32("k")) < io_tol
    assert rel_l2(g, inp.g) < 1e-6
    assert rel_l2(beta, inp.beta) < 1e-7
