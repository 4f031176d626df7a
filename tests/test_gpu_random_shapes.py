"""Seeded sweep of small random problems through the forward, the fused-prologue
forward, the packed variable-length forward and the backward, each against the fp64
oracle: batch, length (ragged tails, one-token and empty rows), head counts and ratio,
head dims, dtype, padding and initial state drawn per case. The draw is fixed, so a
failure names a reproducible case."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import backward, prologue
from gpu_common import TOL_BF16, TOL_F32, dev, np_f64, sync, to_dev
from helpers import rel_l2
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
TOL_BWD_SMALL = 3 * TOL_BF16


def draw(seed):
    r = np.random.default_rng(seed)
    io = "bf16" if r.random() < 0.7 else "f32"
    dk = 128 if (io == "bf16" and r.random() < 0.75) else int(r.choice([16, 32, 64, 128]))
    dv = int(r.choice([16, 32, 64, 128]))
    Hqk = int(r.choice([1, 2, 3]))
    rep = int(r.choice([1, 2, 3]))
    B = int(r.integers(1, 4))
    T = int(r.choice([1, 63, 64, 65, 130, 191, 257]))
    valid = int(r.integers(0, T + 1)) if r.random() < 0.4 else None
    h0 = "normal" if r.random() < 0.6 else None
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="rand%d" % seed, B=B, T=T, Hqk=Hqk, H=Hqk * rep,
                            dk=dk, dv=dv, io=io, h0=h0, seed=1000 + seed, valid_len=valid)
    return w


SEEDS = list(range(100))


def check(x, ref, tol, what):
    err = rel_l2(np_f64(x), ref)
    assert np.all(np.isfinite(np_f64(x))), what
    assert err <= tol, "%s rel-L2 %.3e > %.0e" % (what, err, tol)
    return err


@pytest.mark.parametrize("seed", SEEDS)
def test_random_forward_and_backward(seed):
    w = draw(seed)
    inp = make_inputs(w)
    if inp.valid_len is not None and w.B > 1:
        inp.valid_len[-1] = max(0, inp.valid_len[-1] // 2)   # rows of different lengths
    tol = TOL_BF16 if w.io == "bf16" else TOL_F32
    print("case", seed, w)
    q, k, v, g, beta, h0, vl = to_dev(inp)
    qf, kf, vf, gf, bf, h0f = inp.f64()
    # forward
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, vl)
    sync()
    o_ref, hT_ref = oracle.gdn_fwd(qf, kf, vf, gf, bf, h0f, valid_len=inp.valid_len)
    check(o, o_ref, tol, "o")
    check(hT, hT_ref, tol, "hT")
    # backward: bf16 heads of 128, and narrower bf16 heads on rows of at least 256 tokens
    # (padded to 128), run the chunked matrix-core backward (bf16 operands); everything else
    # the fp32 token-level backward (the fp32 tolerance whatever the input dtype). The pages' bf16 bound on gradients (issue #320 section 4.2) is stated at their
    # sizes (8K-32K tokens); this sweep draws rows of one token, whose dq and dbeta are each a
    # single dot product of bf16-rounded operands (U, dU, X), so that cancellation can
    # multiply the 2^-9 rounding several-fold (2.0e-2 measured on a one-token row). The sweep
    # holds that path to TOL_BWD_SMALL; the full-size and per-path backward tests hold it to 1e-2.
    btol = TOL_BWD_SMALL if (w.io == "bf16" and ((w.dk == 128 and w.dv == 128) or w.T >= 256)) else TOL_F32
    rng = np.random.default_rng(seed)
    d_o = rng.standard_normal(v.shape).astype(np.float32)
    if w.io == "bf16":
        from linear_attention_06_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
        bits = f32_to_bf16_bits(d_o)
        d_o = bf16_bits_to_f32(bits)
        d_o_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    else:
        d_o_t = torch.from_numpy(d_o).to(dev())
    got = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o_t, None, vl)
    sync()
    ref = backward.gdn_bwd(qf, kf, vf, gf, bf, h0f, d_o.astype(np.float64), None, inp.valid_len)
    for nm, x, r_ in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, ref):
        if h0f is None and nm == "dh0":
            continue
        check(x, r_, btol, nm)
    # packed variable-length sequences: each row's valid tokens back to back
    lens = [int(inp.valid_len[b]) if inp.valid_len is not None else w.T for b in range(w.B)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pk = lambda x: torch.cat([x[b:b + 1, :lens[b]] for b in range(w.B)], dim=1).contiguous()
    ov, hTv = gdn.gdn_chunk_fwd_varlen(pk(q), pk(k), pk(v), pk(g), pk(beta),
                                       torch.from_numpy(cu).to(dev()), max(max(lens), 1), h0)
    sync()
    for b in range(w.B):
        assert torch.equal(ov[0, cu[b]:cu[b + 1]], o[b, :lens[b]]), ("varlen row", b)
    assert torch.equal(hTv, hT)


@pytest.mark.parametrize("seed", SEEDS[:32])
def test_random_fused_prologue(seed):
    w = draw(seed)
    w = dataclasses.replace(w, io="bf16", dk=128)   # the prologue runs on the matrix-core path
    inp = make_inputs(w)
    r = inp.raw
    d = dev()
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).view(torch.bfloat16).to(d)
    f = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(d)
    o, hT = gdn.gdn_chunk_fwd_prologue(bf(r["q_raw"]), bf(r["k_raw"]), bf(inp.v), f(r["a"]), f(r["b"]),
                                       f(r["A_log"]), f(r["dt_bias"]), w.dk ** -0.5, f(inp.h0), f(inp.valid_len))
    sync()
    qr, kr, v64, a, b, A_log, dt_bias, h064 = inp.raw_f64()
    o_ref, hT_ref = prologue.gdn_fwd_prologue(qr, kr, v64, a, b, A_log, dt_bias, w.dk ** -0.5, h064,
                                              inp.valid_len)
    check(o, o_ref, TOL_BF16, "prologue o")
    check(hT, hT_ref, TOL_BF16, "prologue hT")


def draw_segments(seed):
    r = np.random.default_rng(5000 + seed)
    io = "bf16" if r.random() < 0.7 else "f32"
    dk = 128 if (io == "bf16" and r.random() < 0.75) else int(r.choice([16, 32, 64, 128]))
    dv = dk if r.random() < 0.6 else int(r.choice([16, 32, 64, 128]))
    Hqk = int(r.choice([1, 2]))
    rep = int(r.choice([1, 2, 3]))
    seg = int(r.choice([64, 128, 192]))
    P = int(r.integers(1, 4))
    B = int(r.integers(1, 3))
    T = seg * P
    valid = int(r.integers(0, T + 1)) if r.random() < 0.4 else None
    h0 = "normal" if r.random() < 0.6 else None
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="rseg%d" % seed, B=B, T=T, Hqk=Hqk, H=Hqk * rep,
                            dk=dk, dv=dv, io=io, h0=h0, seed=2000 + seed, valid_len=valid, seg_len=seg)
    return w


@pytest.mark.parametrize("seed", list(range(32)))
def test_random_segments(seed):
    """Summary (M and S), combine and apply on random shapes against the oracle, and the
    segmented outputs against the unsplit forward."""
    w = draw_segments(seed)
    inp = make_inputs(w)
    print("case", seed, w)
    tol = TOL_BF16 if w.io == "bf16" else TOL_F32
    q, k, v, g, beta, h0, vl = to_dev(inp)
    qf, kf, vf, gf, bf, h0f = inp.f64()
    M, S, ws = gdn.gdn_segment_summary(q, k, v, g, beta, w.seg_len, valid_len=vl)
    H_in, Mp, hT_c = gdn.gdn_summary_combine(M, S, h0, want_prefix=True)
    o, hT = gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, w.seg_len, ws, valid_len=vl)
    sync()
    M_ref, S_ref = oracle.gdn_segment_summary(qf, kf, vf, gf, bf, w.seg_len, valid_len=inp.valid_len)
    # M is a product of decays e^{sum g} over the segment; blocks whose exact value lies below
    # fp32's range (|M| < 1e-30, e.g. a log-decay sum of -150 gives ~1e-65) are zero in the
    # fp32 result. Compare the blocks inside the range; bound the others in absolute terms.
    Mg = np_f64(M).reshape(M.shape[0], M.shape[1], M.shape[2], -1)
    Mr = M_ref.reshape(Mg.shape)
    live = np.linalg.norm(Mr, axis=-1) >= 1e-30
    if live.any():
        err = rel_l2(Mg[live], Mr[live])
        assert err <= tol, "M rel-L2 %.3e > %.0e over %d blocks" % (err, tol, int(live.sum()))
    assert np.all(np.abs(Mg[~live]) <= 1e-30), "M outside the fp32 range is not ~0"
    check(S, S_ref, tol, "S")
    o_ref, hT_ref = oracle.gdn_fwd(qf, kf, vf, gf, bf, h0f, valid_len=inp.valid_len)
    check(o, o_ref, tol, "segmented o")
    check(hT, hT_ref, tol, "segmented hT")
    check(hT_c, hT_ref, tol, "combined hT")


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_layer_steps(seed):
    """Conv1D (random K, halo, bias, SiLU, dtype, C, T, B) and gated RMSNorm (random rows,
    D, dtype, eps) against their oracles."""
    from oracle import layer_ops
    r = np.random.default_rng(7000 + seed)
    io = "bf16" if r.random() < 0.6 else "f32"
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    tol = TOL_BF16 if io == "bf16" else 1e-5
    B, T, C, K = int(r.integers(1, 4)), int(r.choice([1, 3, 63, 64, 65, 200])), 8 * int(r.integers(1, 70)), \
        int(r.choice([2, 3, 4]))
    x = torch.from_numpy(r.standard_normal((B, T, C)).astype(np.float32)).to(dev()).to(tdt)
    w = torch.from_numpy((0.5 * r.standard_normal((C, K))).astype(np.float32)).to(dev())
    bias = torch.from_numpy(r.standard_normal(C).astype(np.float32)).to(dev()) if r.random() < 0.5 else None
    prev = torch.from_numpy(r.standard_normal((B, K - 1, C)).astype(np.float32)).to(dev()).to(tdt) \
        if r.random() < 0.5 else None
    silu = bool(r.random() < 0.7)
    y = gdn.gdn_causal_conv1d(x, w, bias, prev, silu=silu)
    sync()
    ref = layer_ops.causal_conv1d(np_f64(x), np_f64(w), None if bias is None else np_f64(bias),
                                  None if prev is None else np_f64(prev), silu)
    check(y, ref, tol, "conv1d B=%d T=%d C=%d K=%d" % (B, T, C, K))
    rows, D = int(r.integers(1, 3000)), int(r.choice([16, 32, 64, 128]))
    eps = float(r.choice([0.0, 1e-6, 1e-2]))
    o = torch.from_numpy(r.standard_normal((rows, D)).astype(np.float32)).to(dev()).to(tdt)
    z = torch.from_numpy(r.standard_normal((rows, D)).astype(np.float32)).to(dev()).to(tdt)
    wt = torch.from_numpy(r.standard_normal(D).astype(np.float32)).to(dev())
    yn = gdn.gdn_gated_rmsnorm(o, z, wt, eps=eps)
    sync()
    check(yn, layer_ops.gated_rmsnorm(np_f64(o), np_f64(z), np_f64(wt), eps), tol, "norm rows=%d D=%d" % (rows, D))


def test_empty_inputs_of_the_combine_and_backward():
    """No segments: the combine returns the initial state; no tokens: the backward returns
    the final-state gradient as dh0 and empty token gradients."""
    d = 128
    h0 = torch.randn((2, 4, d, d), device=dev())
    M = torch.zeros((2, 4, 0, d, d), device=dev())
    S = torch.zeros((2, 4, 0, d, d), device=dev())
    H_in, _, hT = gdn.gdn_summary_combine(M, S, h0)
    sync()
    assert H_in.numel() == 0 and torch.equal(hT, h0)
    q = torch.zeros((2, 0, 2, d), dtype=torch.bfloat16, device=dev())
    v = torch.zeros((2, 0, 4, d), dtype=torch.bfloat16, device=dev())
    g = torch.zeros((2, 0, 4), device=dev())
    dhT = torch.randn((2, 4, d, d), device=dev())
    dq, dk, dv, dg, db, dh0 = gdn.gdn_chunk_bwd(q, q, v, g, g, h0, v, dhT)
    sync()
    assert dq.numel() == 0 and torch.equal(dh0, dhT)
