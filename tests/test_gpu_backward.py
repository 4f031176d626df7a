"""GPU parity of the backward (gdn_chunk_bwd) against the fp64 autograd oracle on the
same seeded inputs: all six gradients, with and without initial state and final-state
gradient, padded rows, grouped heads, bf16 and fp32 inputs, head dims 16 to 128, and
lengths that end inside a chunk.

bf16 inputs with heads of 128 (and narrower heads on rows of at least 256 tokens, padded to
128) run the chunked matrix-core backward (bf16 operands, fp32 accumulation) and are held to
the pages' bf16 bound on gradients (hyper-parallel issue #320, section 4.2); every other
problem runs the fp32 token-level backward, held to the fp32 bound."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import backward
from gpu_common import TOL_BF16, TOL_F32, dev, np_f64, sync, to_dev, workload_inputs
from helpers import rel_l2
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")

CASES = [
    # name, io, d, B, T, Hqk, H, valid, h0, dhT
    ("bf16_d128_ragged", "bf16", 128, 1, 200, 2, 4, None, True, True),
    ("bf16_d64_ratio3", "bf16", 64, 1, 130, 1, 3, None, False, False),
    ("f32_d32_padded", "f32", 32, 2, 150, 2, 4, 97, True, True),
    ("f32_d16_tiny", "f32", 16, 1, 128, 4, 8, None, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, io, d, B, T, Hqk, H, valid, with_h0, with_dhT = case
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="bwd_" + name, B=B, T=T, Hqk=Hqk, H=H, dk=d,
                            dv=d, io=io, seed=500 + T + d, valid_len=valid)
    inp = make_inputs(w)
    rng = np.random.default_rng(T + d)
    d_o = rng.standard_normal((B, T, H, d)).astype(np.float32)
    dhT = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32) if with_dhT else None
    if io == "bf16":   # the GPU sees d_o in bf16; give the oracle exactly those values
        from linear_attention_06_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
        d_o_bits = f32_to_bf16_bits(d_o)
        d_o = bf16_bits_to_f32(d_o_bits)
        d_o_t = torch.from_numpy(d_o_bits.view(np.int16)).view(torch.bfloat16).to(dev())
    else:
        d_o_t = torch.from_numpy(d_o).to(dev())
    q, k, v, g, beta, h0, vl = to_dev(inp)
    if not with_h0:
        h0 = None
    dhT_t = None if dhT is None else torch.from_numpy(dhT).to(dev())
    got = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o_t, dhT_t, vl)
    sync()
    qf, kf, vf, gf, bf, h0f = inp.f64()
    ref = backward.gdn_bwd(qf, kf, vf, gf, bf, h0f if with_h0 else None, d_o.astype(np.float64),
                           None if dhT is None else dhT.astype(np.float64), inp.valid_len)
    tol = TOL_BF16 if (io == "bf16" and (d == 128 or T >= 256)) else TOL_F32
    for nm, x, r in zip(NAMES, got, ref):
        err = rel_l2(np_f64(x), r)
        print("%s %s rel-L2 %.3e" % (name, nm, err))
        assert np.all(np.isfinite(np_f64(x))), nm
        assert err <= tol, "%s %s rel-L2 %.3e > %.0e" % (name, nm, err, tol)
    if valid is not None:
        for r_ in range(B):
            n = int(inp.valid_len[r_])
            for x in got[:5]:
                assert torch.all(x[r_, n:] == 0)


def test_backward_is_deterministic():
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="bwd_det", T=300, Hqk=2, H=4, seed=77)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, vl = to_dev(inp)
    d_o = torch.randn(v.shape, device=dev()).to(torch.bfloat16)
    a = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o)
    b = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o)
    sync()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_sampled_against_oracle():
    """The stateless 8K workload (32 value heads, d = 128) in the launch configuration the
    bench times, with the output gradient nonzero on the first 1024 tokens only and no
    final-state gradient: then the gradients of those tokens depend on them alone and the
    oracle checks query/key head 0 (value heads 0 and 1) on them, while every gradient of the
    later tokens is exactly zero."""
    inp = workload_inputs("stateless_8k")
    q, k, v, g, beta, _, _ = to_dev(inp)
    rng = np.random.default_rng(11)
    L = 1024
    d_o = np.zeros(v.shape, np.float32)
    d_o[:, :L] = rng.standard_normal((1, L) + tuple(v.shape[2:]))
    from linear_attention_06_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    bits = f32_to_bf16_bits(d_o)
    d_o_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    dq, dk, dv, dg, db, dh0 = gdn.gdn_chunk_bwd(q, k, v, g, beta, None, d_o_t)
    sync()
    for x in (dq, dk, dv, dg, db):
        assert torch.all(x[:, L:] == 0)
    qf, kf, vf, gf, bf, _ = inp.f64()
    ref = backward.gdn_bwd(qf[:, :L, :1], kf[:, :L, :1], vf[:, :L, :2], gf[:, :L, :2], bf[:, :L, :2], None,
                           bf16_bits_to_f32(bits)[:, :L, :2].astype(np.float64))
    got = (dq[:, :L, :1], dk[:, :L, :1], dv[:, :L, :2], dg[:, :L, :2], db[:, :L, :2], dh0[:, :2])
    for nm, x, r in zip(NAMES, got, ref):
        err = rel_l2(np_f64(x), r)
        print("8k sampled %s rel-L2 %.3e" % (nm, err))
        assert err <= TOL_BF16, nm


def test_initial_state_gradient_is_the_summary_transpose():
    """With no output gradient, dh0 = M^T dhT where M is the sequence's state-transition
    summary: the backward's reverse recurrence checked against the segment-summary pass
    (split-bf16 matrix cores, an independent GPU path) on a slowly decaying 2048-token
    problem at d = 128, where M is far from zero."""
    from linear_attention_06_amd.inputs import slow_decay
    w = dataclasses.replace(slow_decay(WORKLOADS["stateful_32k"], seed=606, seg_len=2048), T=2048, Hqk=2, H=4)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    M, _, _ = gdn.gdn_segment_summary(q, k, v, g, beta, 2048, want_s=False)
    dhT = torch.randn((1, 4, 128, 128), device=dev())
    zero = torch.zeros_like(v)
    *_, dh0 = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, zero, dhT)
    sync()
    want = torch.matmul(M[:, :, 0].transpose(-1, -2).contiguous(), dhT)
    ratio = (want.norm() / dhT.norm()).item()
    err = rel_l2(np_f64(dh0), np_f64(want))
    print("dh0 vs M^T dhT rel-L2 %.3e (|M^T dhT| / |dhT| = %.3f)" % (err, ratio))
    assert ratio > 0.05
    assert err <= TOL_BF16


def test_backward_full_size_every_token_live():
    """The stateless 8K workload in the bench's launch configuration with an output
    gradient on every token and a final-state gradient, so that the reverse chain over all
    128 chunks carries a nonzero gradient everywhere: query/key head 0 (value heads 0 and
    1) checked against the fp64 oracle over all 8192 tokens, plus the pages' scaled
    max-abs check on each gradient."""
    from helpers import scaled_max_abs
    from gpu_common import TOL_MAXABS
    from linear_attention_06_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    inp = workload_inputs("stateless_8k")
    q, k, v, g, beta, _, _ = to_dev(inp)
    rng = np.random.default_rng(12)
    bits = f32_to_bf16_bits(rng.standard_normal(tuple(v.shape)).astype(np.float32))
    d_o_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    H, d = v.shape[2], v.shape[3]
    dhT = (0.1 * rng.standard_normal((1, H, d, d))).astype(np.float32)
    dq, dk, dv, dg, db, dh0 = gdn.gdn_chunk_bwd(q, k, v, g, beta, None, d_o_t, torch.from_numpy(dhT).to(dev()))
    sync()
    qf, kf, vf, gf, bf, _ = inp.f64()
    ref = backward.gdn_bwd(qf[:, :, :1], kf[:, :, :1], vf[:, :, :2], gf[:, :, :2], bf[:, :, :2], None,
                           bf16_bits_to_f32(bits)[:, :, :2].astype(np.float64), dhT[:, :2].astype(np.float64))
    got = (dq[:, :, :1], dk[:, :, :1], dv[:, :, :2], dg[:, :, :2], db[:, :, :2], dh0[:, :2])
    for nm, x, r in zip(NAMES, got, ref):
        xn = np_f64(x)
        err, late = rel_l2(xn, r), rel_l2(xn[:, -1024:], r[:, -1024:]) if nm != "dh0" else 0.0
        sma = scaled_max_abs(xn, r)
        print("8k live %s rel-L2 %.3e (last 1024 tokens %.3e), scaled max-abs %.3e" % (nm, err, late, sma))
        assert np.all(np.isfinite(xn)), nm
        assert err <= TOL_BF16 and late <= TOL_BF16, nm
        assert sma <= TOL_MAXABS, nm
