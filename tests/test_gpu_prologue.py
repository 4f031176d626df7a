"""GPU parity of the forward with the fused input prologue (gdn_chunk_fwd_prologue:
q/k L2 norm, q scale, g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b) inside
the chunk prepare pass) against the fp64 oracle of prologue + forward, at the
stateful 32K workload's full size and on small ragged and padded problems."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import prologue
from gpu_common import TOL_BF16, dev, np_f64, sync, workload_inputs
from helpers import rel_l2
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def raw_to_dev(inp):
    d = dev()
    r = inp.raw
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).view(torch.bfloat16).to(d)
    f = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(d)
    return (bf(r["q_raw"]), bf(r["k_raw"]), bf(inp.v), f(r["a"]), f(r["b"]), f(r["A_log"]),
            f(r["dt_bias"]), f(inp.h0), f(inp.valid_len))


def run(inp, scale_q=1.0, scale_k=1.0):
    q, k, v, a, b, A_log, dt_bias, h0, vl = raw_to_dev(inp)
    if scale_q != 1.0:
        q = (q * scale_q).contiguous()
    if scale_k != 1.0:
        k = (k * scale_k).contiguous()
    o, hT = gdn.gdn_chunk_fwd_prologue(q, k, v, a, b, A_log, dt_bias, inp.w.dk ** -0.5, h0, vl)
    sync()
    return o, hT


def oracle_run(inp):
    q_raw, k_raw, v, a, b, A_log, dt_bias, h0 = inp.raw_f64()
    return prologue.gdn_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, inp.w.dk ** -0.5, h0,
                                     inp.valid_len)


def check(x, ref, tol, what):
    err = rel_l2(x, ref)
    print("%s rel-L2 %.3e (bound %.0e)" % (what, err, tol))
    assert np.all(np.isfinite(x)), what
    assert err <= tol, "%s rel-L2 %.3e > %.0e" % (what, err, tol)


def test_prologue_stateful_32k_matches_oracle():
    inp = workload_inputs("stateful_32k")
    o_ref, hT_ref = oracle_run(inp)
    o, hT = run(inp)
    check(np_f64(o), o_ref, TOL_BF16, "prologue 32k o")
    check(np_f64(hT), hT_ref, TOL_BF16, "prologue 32k hT")


SMALL = [
    # name, B, T, Hqk, H, valid
    ("ragged", 1, 300, 2, 4, None),
    ("padded", 2, 333, 2, 4, 250),
    ("ratio3", 1, 130, 1, 3, None),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_prologue_small_matches_oracle(case):
    name, B, T, Hqk, H, valid = case
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="pro_" + name, B=B, T=T, Hqk=Hqk, H=H,
                            seed=300 + T, valid_len=valid)
    inp = make_inputs(w)
    if valid is not None:
        inp.valid_len[1] = 77   # rows of different lengths
    o_ref, hT_ref = oracle_run(inp)
    o, hT = run(inp)
    of = np_f64(o)
    check(of, o_ref, TOL_BF16, name + " o")
    check(np_f64(hT), hT_ref, TOL_BF16, name + " hT")
    if valid is not None:
        # padded tokens carry random a and b; their output is +0.0 bitwise
        for r in range(B):
            tail = o[r, int(inp.valid_len[r]):].float()
            assert torch.all(tail == 0) and not torch.any(torch.signbit(tail))


def test_prologue_is_invariant_under_row_scaling():
    """Scaling q_raw by 4 and k_raw by 1/2 (exact in bf16) leaves the normalised inputs,
    and so the outputs, unchanged up to rounding: the logs of the row factors enter the
    decay exponents in fp32, and a perturbation of a few fp32 ulps flips the bf16 rounding
    of a few That, P and o elements (one bf16 ulp, 2^-8 relative, each). The bound is that
    bf16 resolution; a missing or misplaced normalisation changes o by O(1)."""
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="pro_scale", T=500, Hqk=2, H=4, seed=321)
    inp = make_inputs(w)
    o, hT = run(inp)
    o2, hT2 = run(inp, scale_q=4.0, scale_k=0.5)
    e_o, e_h = rel_l2(np_f64(o2), np_f64(o)), rel_l2(np_f64(hT2), np_f64(hT))
    print("row scaling: o %.2e, hT %.2e" % (e_o, e_h))
    assert e_o < 2e-3 and e_h < 2e-3


def test_plain_forward_unchanged_by_unit_row_factors():
    """The plain forward runs the same kernels with unit row factors; two runs agree
    bitwise and match the oracle (a regression guard for the shared decay record)."""
    inp = workload_inputs("stateless_8k")
    from gpu_common import oracle_fwd, to_dev
    q, k, v, g, beta, h0, vl = to_dev(inp)
    o1, _ = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, vl, want_state=False)
    o2, _ = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, vl, want_state=False)
    sync()
    assert torch.equal(o1, o2)
    check(np_f64(o1), oracle_fwd("stateless_8k")[0], TOL_BF16, "plain 8k o")
