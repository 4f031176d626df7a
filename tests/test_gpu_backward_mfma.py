"""GPU parity of the chunked matrix-core backward (gdn_chunk_bwd on bf16 inputs with heads
of 128: prepare records, forward state pass keeping every chunk's incoming state, reverse
chain, per-chunk gradient pass) against the fp64 autograd oracle on the same seeded inputs,
and against the fp32 token-level backward on the GPU (reached through the one-segment
apply backward, which runs the same gradients token by token).

Every product takes bf16 operands with fp32 accumulation, like the forward; the bound is
the pages' bf16 bound on gradients (hyper-parallel issue #320, section 4.2: relative L2
1e-2), together with their scaled max-abs check (PR #1035 test plan part 1). At full size
every (b, 64-token chunk, head) block of dq, dk and dv is held to 1e-2 as well. The blocks
of dg and dbeta are held to TOL_BLOCK_DG: a token's dg sums decay terms of opposite sign
(the chunk-end term e^{Gam_C} <dS', S> + sum_t W_t against the per-token -W_t, the row and
column sums of dP . P and E . K K^T), so in a chunk where dg is small the bf16 rounding of
the ~20 operands that feed it (none above ~4e-3 alone, in an fp64 emulation of the same
arithmetic) shows at a few times the tensor's relative error; the whole tensors stay under
1e-2."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import backward
from gpu_common import TOL_BF16, TOL_MAXABS, dev, np_f64, sync, to_dev, workload_inputs
from helpers import rel_l2, scaled_max_abs
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs

pytestmark = pytest.mark.gpu
TOL_BLOCK_DG = 5e-2

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def output_grad(shape, seed):
    rng = np.random.default_rng(seed)
    bits = f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev()), bf16_bits_to_f32(bits).astype(np.float64)


CASES = [
    # name, B, T, Hqk, H, valid, h0, dhT
    ("one_chunk", 1, 64, 1, 1, None, True, True),
    ("one_token_token_level", 1, 1, 4, 16, None, True, True),   # under 64 tokens: the fp32 backward
    ("ragged_three_chunks", 1, 150, 2, 4, None, True, True),
    ("padded_rows", 2, 300, 2, 4, 173, False, True),
    ("rep1_no_state", 1, 256, 2, 2, None, False, False),
    ("rep4", 1, 192, 1, 4, None, True, False),
    ("tail_of_one", 1, 129, 2, 4, None, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunked_backward_matches_oracle(case):
    name, B, T, Hqk, H, valid, with_h0, with_dhT = case
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="bwdm_" + name, B=B, T=T, Hqk=Hqk, H=H,
                            seed=800 + T + H, valid_len=valid)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, vl = to_dev(inp)
    assert gdn.gdn_kernel_path(gdn.problem(q, v, vl)) == "bf16-mfma"
    if not with_h0:
        h0 = None
    d_o_t, d_o = output_grad(tuple(v.shape), 801 + T)
    rng = np.random.default_rng(802 + T)
    dhT = (0.1 * rng.standard_normal((B, H, 128, 128))).astype(np.float32) if with_dhT else None
    dhT_t = None if dhT is None else torch.from_numpy(dhT).to(dev())
    got = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o_t, dhT_t, vl)
    sync()
    qf, kf, vf, gf, bf, h0f = inp.f64()
    ref = backward.gdn_bwd(qf, kf, vf, gf, bf, h0f if with_h0 else None, d_o,
                           None if dhT is None else dhT.astype(np.float64), inp.valid_len)
    for nm, x, r in zip(NAMES, got, ref):
        xn = np_f64(x)
        err, sma = rel_l2(xn, r), scaled_max_abs(xn, r)
        print("%s %s rel-L2 %.3e scaled max-abs %.3e" % (name, nm, err, sma))
        assert np.all(np.isfinite(xn)), nm
        assert err <= TOL_BF16, "%s %s rel-L2 %.3e" % (name, nm, err)
        assert sma <= TOL_MAXABS, "%s %s scaled max-abs %.3e" % (name, nm, sma)
    if valid is not None:
        for b in range(B):
            n = int(inp.valid_len[b])
            for x in got[:5]:
                assert torch.all(x[b, n:] == 0)


def test_chunked_backward_is_deterministic():
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="bwdm_det", T=320, Hqk=2, H=4, seed=811)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    d_o, _ = output_grad(tuple(v.shape), 812)
    a = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o)
    b = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o)
    sync()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_chunked_backward_empty_sequence_returns_dhT():
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="bwdm_empty", T=0, Hqk=1, H=2, seed=813)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    dhT = torch.randn((1, 2, 128, 128), device=dev())
    *_, dh0 = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, torch.zeros_like(v), dhT)
    sync()
    assert torch.equal(dh0, dhT)


def token_level(q, k, v, g, beta, h0, d_o, dhT):
    """The fp32 token-level backward of the same problem: the apply backward with one
    segment whose incoming state is h0."""
    B, T, H = v.shape[0], v.shape[1], v.shape[2]
    H_in = (h0 if h0 is not None else torch.zeros((B, H, 128, 128), device=v.device)).unsqueeze(2).contiguous()
    dq, dk, dv, dg, db, dH_in = gdn.gdn_apply_initial_state_bwd(q, k, v, g, beta, H_in, T, d_o, dhT)
    return dq, dk, dv, dg, db, dH_in[:, :, 0]


def test_chunked_backward_matches_token_level_8k_every_head():
    """The stateless 8K workload (32 value heads read by 16 query/key heads) with an output
    gradient on every token and a final-state gradient: all heads and tokens of every
    gradient against the fp32 token-level backward, per tensor and per (query/key or value)
    head and 64-token chunk block, plus the scaled max-abs check."""
    from helpers import worst_token_block
    inp = workload_inputs("stateless_8k")
    q, k, v, g, beta, _, _ = to_dev(inp)
    d_o_t, _ = output_grad(tuple(v.shape), 820)
    dhT = 0.1 * torch.randn((1, v.shape[2], 128, 128), device=dev())
    got = gdn.gdn_chunk_bwd(q, k, v, g, beta, None, d_o_t, dhT)
    ref = token_level(q, k, v, g, beta, None, d_o_t, dhT)
    sync()
    for nm, x, r in zip(NAMES, got, ref):
        xn, rn = np_f64(x), np_f64(r)
        err, sma = rel_l2(xn, rn), scaled_max_abs(xn, rn)
        msg = "8k %s rel-L2 %.3e scaled max-abs %.3e" % (nm, err, sma)
        if nm != "dh0":
            blocks = (xn, rn) if xn.ndim == 4 else (xn[..., None], rn[..., None])
            wb, where = worst_token_block(*blocks)
            msg += " worst block %.3e at %s" % (wb, where)
            assert wb <= (TOL_BLOCK_DG if nm in ("dg", "dbeta") else TOL_BF16), msg
        print(msg)
        assert np.all(np.isfinite(xn)), nm
        assert err <= TOL_BF16 and sma <= TOL_MAXABS, msg


def test_chunked_backward_matches_token_level_stateful_2k():
    """A 2048-token stateful problem with slow decay (the carried state matters across all
    32 chunks) at 32 value heads: every gradient against the fp32 token-level backward."""
    from linear_attention_06_amd.inputs import slow_decay
    w = dataclasses.replace(slow_decay(WORKLOADS["stateful_32k"], seed=830, seg_len=2048), T=2048)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, _ = to_dev(inp)
    d_o_t, _ = output_grad(tuple(v.shape), 831)
    dhT = 0.1 * torch.randn((1, v.shape[2], 128, 128), device=dev())
    got = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o_t, dhT)
    ref = token_level(q, k, v, g, beta, h0, d_o_t, dhT)
    sync()
    for nm, x, r in zip(NAMES, got, ref):
        xn, rn = np_f64(x), np_f64(r)
        err, sma = rel_l2(xn, rn), scaled_max_abs(xn, rn)
        print("2k stateful %s rel-L2 %.3e scaled max-abs %.3e" % (nm, err, sma))
        assert np.all(np.isfinite(xn)), nm
        assert err <= TOL_BF16 and sma <= TOL_MAXABS, nm


SAVED_CASES = [
    # name, B, T, Hqk, H, valid, h0, dhT
    ("ragged_stateful", 1, 150, 2, 4, None, True, True),
    ("padded_rows", 2, 300, 2, 4, 173, False, True),
    ("stateful_2k_rep2", 1, 2048, 16, 32, None, True, True),
    ("empty", 1, 0, 1, 2, None, True, True),
]


@pytest.mark.parametrize("case", SAVED_CASES, ids=[c[0] for c in SAVED_CASES])
def test_saved_forward_and_backward_match_the_plain_calls(case):
    """gdn_chunk_fwd_save gives gdn_chunk_fwd's o and hT bit for bit, and
    gdn_chunk_bwd_saved on its workspace gives gdn_chunk_bwd's gradients bit for bit (the
    same kernels on the same records and states); the backward runs twice on one kept
    forward, as a caller that recomputes a gradient would."""
    name, B, T, Hqk, H, valid, with_h0, with_dhT = case
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="saved_" + name, B=B, T=T, Hqk=Hqk, H=H,
                            seed=840 + T + H, valid_len=valid)
    inp = make_inputs(w)
    q, k, v, g, beta, h0, vl = to_dev(inp)
    if not with_h0:
        h0 = None
    d_o, _ = output_grad(tuple(v.shape), 841 + T)
    dhT = 0.1 * torch.randn((B, H, 128, 128), device=dev()) if with_dhT else None
    o_ref, hT_ref = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, vl)
    ref = gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o, dhT, vl)
    o, hT, ws = gdn.gdn_chunk_fwd_save(q, k, v, g, beta, h0, vl)
    got = gdn.gdn_chunk_bwd_saved(q, k, v, g, beta, d_o, ws, dhT, vl)
    again = gdn.gdn_chunk_bwd_saved(q, k, v, g, beta, d_o, ws, dhT, vl)
    sync()
    assert torch.equal(o, o_ref) and torch.equal(hT, hT_ref)
    for nm, x, y, z in zip(NAMES, got, again, ref):
        assert torch.equal(x, z), "%s %s differs from gdn_chunk_bwd" % (name, nm)
        assert torch.equal(y, z), "%s %s differs on the second backward" % (name, nm)
