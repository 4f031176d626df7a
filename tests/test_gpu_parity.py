"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, at the five workloads' full sizes and at small sizes that
span several chunks and a ragged tail, plus the bit-exact padding, resume and
determinism properties."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (TOL_BF16, TOL_F32, TOL_MAXABS, np_f64, oracle_fwd, sync, to_dev, workload_inputs)
from helpers import rel_l2, scaled_max_abs, worst_lead_block, worst_token_block
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs, slow_decay

pytestmark = pytest.mark.gpu


def run_fwd(inp, h0="given", want_state=True):
    q, k, v, g, beta, h0_t, vl = to_dev(inp)
    if h0 == "none":
        h0_t = None
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0_t, vl, want_state=want_state)
    sync()
    return o, hT


def assert_close(x, ref, tol, what):
    err = rel_l2(x, ref)
    print("%s rel-L2 %.3e (bound %.0e)" % (what, err, tol))
    assert np.all(np.isfinite(x)), what + " has non-finite values"
    assert err <= tol, "%s rel-L2 %.3e > %.0e" % (what, err, tol)


def assert_local(x, ref, tol, what, nlead=None):
    """Localised gates on a full-size tensor: the whole-tensor bound must also hold on every
    (b, 64-token chunk, h) block of a token tensor [B, T, H, D] (nlead None), or on every
    block over the first nlead axes of a state or summary tensor; and the pages' scaled
    max-abs check. One zeroed or garbage block of a 32K output is 1/16384 of the tensor and
    would pass the whole-tensor bound."""
    if nlead is None:
        err, at = worst_token_block(x, ref)
        where = "(b, chunk, h)"
    else:
        err, at = worst_lead_block(x, ref, nlead)
        where = "block"
    sma = scaled_max_abs(x, ref)
    print("%s worst %s rel-L2 %.3e at %s; scaled max-abs %.3e" % (what, where, err, at, sma))
    assert err <= tol, "%s worst %s rel-L2 %.3e at %s > %.0e" % (what, where, err, at, tol)
    assert sma <= TOL_MAXABS, "%s scaled max-abs %.3e > %.0e" % (what, sma, TOL_MAXABS)


# ------------------------------------------------------------------ full workloads
def test_tiny_f32_matches_oracle():
    inp = workload_inputs("tiny_f32")
    o_ref, hT_ref = oracle_fwd("tiny_f32")
    o, hT = run_fwd(inp)
    assert_close(np_f64(o), o_ref, TOL_F32, "tiny o")
    assert_close(np_f64(hT), hT_ref, TOL_F32, "tiny hT")
    # a zero initial state and no initial state give the same bits
    o2, hT2 = run_fwd(inp, h0="none")
    assert torch.equal(o, o2) and torch.equal(hT, hT2)


def test_stateless_8k_matches_oracle():
    inp = workload_inputs("stateless_8k")
    o_ref, _ = oracle_fwd("stateless_8k")
    o, _ = run_fwd(inp, want_state=False)
    on = np_f64(o)
    assert_close(on, o_ref, TOL_BF16, "stateless_8k o")
    assert_local(on, o_ref, TOL_BF16, "stateless_8k o")


@pytest.mark.parametrize("d,io", [(64, "bf16"), (128, "f32")], ids=["bf16_d64", "f32_d128"])
def test_other_paths_full_size_match_oracle(d, io):
    """The stateless 8K workload's shapes off the d = 128 bf16 path (heads of 64 in bf16, run
    by gdn_chunk_fwd on the matrix cores with q and k padded to 128 columns, and fp32 inputs on
    the fp32 matrix-core kernels): the sizes bench.py times for those paths."""
    w = dataclasses.replace(WORKLOADS["stateless_8k"], name="vector_%s_d%d" % (io, d), dk=d, dv=d, io=io)
    inp = make_inputs(w)
    q, k, v, g, beta, _, _ = to_dev(inp)
    assert gdn.gdn_kernel_path(gdn.problem(q, v)) == ("bf16-mfma-padded" if io == "bf16" else "f32-mfma")
    q64, k64, v64, g64, b64, _ = inp.f64()
    o_ref, hT_ref = oracle.gdn_fwd(q64, k64, v64, g64, b64, None)
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, None)
    sync()
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    assert_close(np_f64(o), o_ref, tol, "vector path %s d=%d o" % (io, d))
    assert_close(np_f64(hT), hT_ref, tol, "vector path %s d=%d hT" % (io, d))


def test_bf16_head_dim_128_uses_the_matrix_core_path():
    inp = workload_inputs("stateful_32k")
    q, k, v, g, beta, h0, _ = to_dev(inp)
    assert gdn.gdn_kernel_path(gdn.problem(q, v)) == "bf16-mfma"


def test_stateful_32k_matches_oracle():
    inp = workload_inputs("stateful_32k")
    o_ref, hT_ref = oracle_fwd("stateful_32k")
    o, hT = run_fwd(inp)
    on, hn = np_f64(o), np_f64(hT)
    assert_close(on, o_ref, TOL_BF16, "stateful_32k o")
    assert_close(hn, hT_ref, TOL_BF16, "stateful_32k hT")
    assert_local(on, o_ref, TOL_BF16, "stateful_32k o")
    assert_local(hn, hT_ref, TOL_BF16, "stateful_32k hT", nlead=2)


def test_segmented_32k_matches_oracle_and_unsplit_run():
    w = WORKLOADS["segmented_32k"]
    inp = workload_inputs("stateful_32k")            # the same seeded sequence
    q64, k64, v64, g64, b64, h064 = inp.f64()
    M_ref, S_ref = oracle.gdn_segment_summary(q64, k64, v64, g64, b64, w.seg_len)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    M, S, ws = gdn.gdn_segment_summary(q, k, v, g, beta, w.seg_len)
    H_in, Mp, hT_c = gdn.gdn_summary_combine(M, S, h0, want_prefix=True)
    o, hT = gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, w.seg_len, ws)
    sync()
    assert_close(np_f64(S), S_ref, TOL_BF16, "segment S")
    assert_close(np_f64(M), M_ref, TOL_BF16, "segment M")
    Hin_ref, _, hTc_ref = oracle.gdn_summary_combine(M_ref, S_ref, h064)
    assert_close(np_f64(H_in), Hin_ref, TOL_BF16, "H_in")
    o_ref, hT_ref = oracle_fwd("stateful_32k")
    assert_close(np_f64(o), o_ref, TOL_BF16, "segmented o")
    assert_close(np_f64(hT), hT_ref, TOL_BF16, "segmented hT")
    assert_close(np_f64(hT_c), hT_ref, TOL_BF16, "combined hT")
    assert_local(np_f64(M), M_ref, TOL_BF16, "segment M", nlead=3)
    assert_local(np_f64(S), S_ref, TOL_BF16, "segment S", nlead=3)
    assert_local(np_f64(H_in), Hin_ref, TOL_BF16, "H_in", nlead=3)
    assert_local(np_f64(o), o_ref, TOL_BF16, "segmented o")
    assert_local(np_f64(hT), hT_ref, TOL_BF16, "segmented hT", nlead=2)
    o_full, hT_full = run_fwd(inp)
    assert_close(np_f64(o), np_f64(o_full), TOL_BF16, "segmented vs unsplit o")
    assert_close(np_f64(hT), np_f64(hT_full), TOL_BF16, "segmented vs unsplit hT")


def test_padded_8k_in_segments_matches_oracle():
    """The padded 8K workload (two rows of 7777 valid tokens) through the segment calls in
    4 segments of 2048: the last segment holds the padding, whose transitions are identities."""
    inp = workload_inputs("padded_8k")
    seg = 2048
    q64, k64, v64, g64, b64, _ = inp.f64()
    M_ref, S_ref = oracle.gdn_segment_summary(q64, k64, v64, g64, b64, seg, valid_len=inp.valid_len)
    q, k, v, g, beta, _, vl = to_dev(inp)
    M, S, ws = gdn.gdn_segment_summary(q, k, v, g, beta, seg, valid_len=vl)
    H_in, _, hT_c = gdn.gdn_summary_combine(M, S, None)
    o, hT = gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, seg, ws, valid_len=vl)
    sync()
    assert_close(np_f64(M), M_ref, TOL_BF16, "padded segment M")
    assert_close(np_f64(S), S_ref, TOL_BF16, "padded segment S")
    o_ref, hT_ref = oracle_fwd("padded_8k")
    assert_close(np_f64(o), o_ref, TOL_BF16, "padded segmented o")
    assert_close(np_f64(hT), hT_ref, TOL_BF16, "padded segmented hT")
    assert_close(np_f64(hT_c), hT_ref, TOL_BF16, "padded combined hT")
    tail = o[:, 7777:].float()
    assert torch.all(tail == 0) and not torch.any(torch.signbit(tail))
    # with 6000 valid tokens the last segment (tokens 6144..8191) is pure padding: its
    # transitions are identities, so M = I and S = 0 exactly
    vl2 = torch.full((2,), 6000, dtype=torch.int32, device=v.device)
    M2, S2, _ = gdn.gdn_segment_summary(q, k, v, g, beta, seg, valid_len=vl2)
    sync()
    eye = torch.eye(128, device=M.device).expand_as(M2[:, :, -1])
    assert torch.equal(M2[:, :, -1], eye) and torch.all(S2[:, :, -1] == 0)


def test_padded_8k_matches_oracle_and_is_bit_exact():
    inp = workload_inputs("padded_8k")
    n = int(inp.valid_len[0])
    o_ref, hT_ref = oracle_fwd("padded_8k")
    o, hT = run_fwd(inp)
    on = np_f64(o)
    assert_close(on[:, :n], o_ref[:, :n], TOL_BF16, "padded o (valid tokens)")
    assert_close(np_f64(hT), hT_ref, TOL_BF16, "padded hT")
    assert_local(on[:, :n], o_ref[:, :n], TOL_BF16, "padded o (valid tokens)")
    assert_local(np_f64(hT), hT_ref, TOL_BF16, "padded hT", nlead=2)
    # (i) padded outputs are +0.0, bitwise
    pad_bits = o[:, n:].contiguous().view(torch.int16)
    assert int(torch.count_nonzero(pad_bits)) == 0
    # (ii) valid outputs and final state equal the run on the truncated rows, bitwise
    q, k, v, g, beta, _, _ = to_dev(inp)
    ot, hTt = gdn.gdn_chunk_fwd(q[:, :n].contiguous(), k[:, :n].contiguous(), v[:, :n].contiguous(),
                                g[:, :n].contiguous(), beta[:, :n].contiguous())
    sync()
    assert torch.equal(o[:, :n], ot) and torch.equal(hT, hTt)
    # (iii) each row equals its own B = 1 run, bitwise
    for b in range(2):
        vl = torch.tensor([n], dtype=torch.int32, device=q.device)
        ob, hTb = gdn.gdn_chunk_fwd(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(),
                                    v[b:b + 1].contiguous(), g[b:b + 1].contiguous(),
                                    beta[b:b + 1].contiguous(), None, vl)
        sync()
        assert torch.equal(o[b:b + 1], ob) and torch.equal(hT[b:b + 1], hTb)


# ------------------------------------------------------------------ small shapes
SMALL = [
    # name, io, B, T, Hqk, H, dk, dv
    ("f32_ragged", "f32", 2, 200, 2, 4, 32, 32),
    ("f32_dk_ne_dv", "f32", 1, 130, 1, 2, 16, 32),
    ("f32_d64", "f32", 1, 97, 2, 2, 64, 64),
    ("f32_d128", "f32", 1, 129, 1, 2, 128, 128),
    ("bf16_d128_ragged", "bf16", 2, 1000, 2, 4, 128, 128),
    ("bf16_d64", "bf16", 1, 300, 2, 4, 64, 64),
    ("bf16_one_token", "bf16", 1, 1, 1, 2, 128, 128),
    ("bf16_tail_only", "bf16", 1, 63, 2, 2, 128, 128),
    # matrix-core path with fewer than 8 column tiles per head, value/query-key head
    # ratios 1 and 3 and batch rows that leave the block grid's last XCD slots empty
    ("bf16_dv16_ratio3", "bf16", 1, 260, 1, 3, 128, 16),
    ("bf16_dv32_ratio1_B3", "bf16", 3, 190, 3, 3, 128, 32),
    ("bf16_dv64_B2", "bf16", 2, 700, 2, 4, 128, 64),
]


def small_inputs(name, io, B, T, Hqk, H, dk, dv, seed=100, h0="normal"):
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name=name, B=B, T=T, Hqk=Hqk, H=H, dk=dk,
                            dv=dv, io=io, h0=h0, seed=seed)
    return make_inputs(w)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_match_oracle(case):
    name, io, B, T, Hqk, H, dk, dv = case
    inp = small_inputs(*case)
    q64, k64, v64, g64, b64, h064 = inp.f64()
    o_ref, hT_ref = oracle.gdn_fwd(q64, k64, v64, g64, b64, h064)
    o, hT = run_fwd(inp)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    assert_close(np_f64(o), o_ref, tol, name + " o")
    assert_close(np_f64(hT), hT_ref, tol, name + " hT")


def test_empty_sequence_returns_initial_state():
    inp = small_inputs("empty", "bf16", 2, 0, 2, 4, 128, 128)
    o, hT = run_fwd(inp)
    assert o.numel() == 0
    assert torch.equal(hT.cpu(), torch.from_numpy(inp.h0))
    inp0 = small_inputs("empty0", "bf16", 2, 0, 2, 4, 128, 128, h0=None)
    _, hT0 = run_fwd(inp0)
    assert int(torch.count_nonzero(hT0)) == 0


def test_resume_from_final_state_is_bitwise():
    inp = small_inputs("resume", "bf16", 1, 320, 2, 4, 128, 128)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0)
    T1 = 192
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o1, h1 = gdn.gdn_chunk_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1),
                               sl(beta, 0, T1), h0)
    o2, h2 = gdn.gdn_chunk_fwd(sl(q, T1, 320), sl(k, T1, 320), sl(v, T1, 320), sl(g, T1, 320),
                               sl(beta, T1, 320), h1)
    sync()
    assert torch.equal(torch.cat([o1, o2], dim=1), o) and torch.equal(h2, hT)


def test_runs_are_deterministic():
    inp = small_inputs("determinism", "bf16", 1, 777, 2, 4, 128, 128)
    a = run_fwd(inp)
    b = run_fwd(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_final_state_may_alias_initial_state():
    inp = small_inputs("alias", "bf16", 1, 200, 2, 4, 128, 128)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0.clone())
    buf = h0.clone()
    o2, hT2 = gdn.gdn_chunk_fwd(q, k, v, g, beta, buf, hT=buf)
    sync()
    assert torch.equal(o, o2) and torch.equal(hT, buf)


def test_large_negative_log_decay_resets_without_nan():
    inp = small_inputs("reset", "bf16", 1, 256, 2, 4, 128, 128)
    inp.g[0, 70, :] = -1e4
    inp.g[0, 130:140, 1] = -80.0
    q64, k64, v64, g64, b64, h064 = inp.f64()
    o_ref, hT_ref = oracle.gdn_fwd(q64, k64, v64, g64, b64, h064)
    o, hT = run_fwd(inp)
    assert_close(np_f64(o), o_ref, TOL_BF16, "reset o")
    assert_close(np_f64(hT), hT_ref, TOL_BF16, "reset hT")


def test_slow_decay_segments_exercise_the_combine():
    """Slow decay keeps the incoming state's weight large, so a wrong combine shows."""
    w = slow_decay(WORKLOADS["stateful_32k"], seed=101, seg_len=256)
    inp = make_inputs(w, T=2048)
    q64, k64, v64, g64, b64, h064 = inp.f64()
    M_ref, S_ref = oracle.gdn_segment_summary(q64, k64, v64, g64, b64, w.seg_len)
    Hin_ref, _, _ = oracle.gdn_summary_combine(M_ref, S_ref, h064)
    carried = np.einsum("bhpij,bhpjk->bhpik", M_ref[:, :, 1:], Hin_ref[:, :, 1:])
    ratio = np.linalg.norm(carried) / np.linalg.norm(S_ref[:, :, 1:])
    assert ratio >= 0.1, ratio
    o_ref, hT_ref = oracle.gdn_fwd(q64, k64, v64, g64, b64, h064)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    M, S, ws = gdn.gdn_segment_summary(q, k, v, g, beta, w.seg_len)
    H_in, _, _ = gdn.gdn_summary_combine(M, S, h0)
    o, hT = gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, w.seg_len, ws)
    sync()
    assert_close(np_f64(M), M_ref, TOL_BF16, "slow M")
    assert_close(np_f64(S), S_ref, TOL_BF16, "slow S")
    assert_close(np_f64(o), o_ref, TOL_BF16, "slow o")
    assert_close(np_f64(hT), hT_ref, TOL_BF16, "slow hT")


def test_summary_bf16_narrow_heads_matches_oracle():
    """Segment calls on the matrix-core path with dv = 32 and three value heads per
    query/key head: summaries, prefix products, combine and apply against the oracle."""
    inp = small_inputs("seg_bf16_dv32", "bf16", 1, 512, 1, 3, 128, 32, seed=8)
    q64, k64, v64, g64, b64, h064 = inp.f64()
    M_ref, S_ref = oracle.gdn_segment_summary(q64, k64, v64, g64, b64, 128)
    Hin_ref, Mp_ref, hTc_ref = oracle.gdn_summary_combine(M_ref, S_ref, h064, want_prefix=True)
    o_ref, hT_ref = oracle.gdn_apply_initial_state(q64, k64, v64, g64, b64, Hin_ref, 128)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    M, S, ws = gdn.gdn_segment_summary(q, k, v, g, beta, 128)
    H_in, Mp, hTc = gdn.gdn_summary_combine(M, S, h0, want_prefix=True)
    o, hT = gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, 128, ws)
    sync()
    for x, r, n in ((M, M_ref, "M"), (S, S_ref, "S"), (H_in, Hin_ref, "H_in"), (Mp, Mp_ref, "M_prefix"),
                    (hTc, hTc_ref, "combined hT"), (o, o_ref, "o"), (hT, hT_ref, "hT")):
        assert_close(np_f64(x), r, TOL_BF16, "bf16 dv32 segments " + n)


def test_summary_bf16_both_summaries_in_one_pass():
    """With dk = dv = 128 on the matrix-core path one pass computes M and S together
    (the M and S chains of a column tile share their loaded operands). Both match the
    oracle and, bit for bit, the passes that compute only M or only S; two batch rows,
    five segments and three value heads per query/key head (so the grid's last XCD
    slots stay empty)."""
    inp = small_inputs("seg_bf16_dual", "bf16", 2, 640, 1, 3, 128, 128, seed=9)
    q64, k64, v64, g64, b64, _ = inp.f64()
    M_ref, S_ref = oracle.gdn_segment_summary(q64, k64, v64, g64, b64, 128)
    q, k, v, g, beta, _, _ = to_dev(inp)
    M, S, _ = gdn.gdn_segment_summary(q, k, v, g, beta, 128)
    M1, _, _ = gdn.gdn_segment_summary(q, k, v, g, beta, 128, want_s=False)
    _, S1, _ = gdn.gdn_segment_summary(q, k, v, g, beta, 128, want_m=False)
    sync()
    assert_close(np_f64(M), M_ref, TOL_BF16, "one-pass M")
    assert_close(np_f64(S), S_ref, TOL_BF16, "one-pass S")
    assert torch.equal(M, M1), "M differs from the M-only pass"
    assert torch.equal(S, S1), "S differs from the S-only pass"


def test_summary_f32_small_matches_oracle():
    inp = small_inputs("seg_f32", "f32", 2, 256, 2, 4, 32, 16, seed=7)
    q64, k64, v64, g64, b64, h064 = inp.f64()
    M_ref, S_ref = oracle.gdn_segment_summary(q64, k64, v64, g64, b64, 64)
    Hin_ref, Mp_ref, hTc_ref = oracle.gdn_summary_combine(M_ref, S_ref, h064, want_prefix=True)
    o_ref, hT_ref = oracle.gdn_apply_initial_state(q64, k64, v64, g64, b64, Hin_ref, 64)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    M, S, ws = gdn.gdn_segment_summary(q, k, v, g, beta, 64)
    H_in, Mp, hTc = gdn.gdn_summary_combine(M, S, h0, want_prefix=True)
    o, hT = gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, 64, ws)
    sync()
    for x, r, n in ((M, M_ref, "M"), (S, S_ref, "S"), (H_in, Hin_ref, "H_in"), (Mp, Mp_ref, "M_prefix"),
                    (hTc, hTc_ref, "combined hT"), (o, o_ref, "o"), (hT, hT_ref, "hT")):
        assert_close(np_f64(x), r, TOL_F32, "f32 segments " + n)
