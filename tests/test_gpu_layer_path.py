"""The layer's GDN path composed from the library's entry points, against the chained
oracles: causal Conv1D with SiLU over the projected q/k/v channels, the split into q_raw,
k_raw and v, the forward with the fused input prologue, and the gated RMSNorm of its
output; and the forward reading the three parts straight out of the packed conv output
(gdn_chunk_fwd_prologue_qkv), which must give the same bits."""
import numpy as np
import pytest
import torch

from oracle import layer_ops, prologue
from gpu_common import TOL_BF16, dev, np_f64, sync
from helpers import rel_l2
from linear_attention_06_amd import gdn

pytestmark = pytest.mark.gpu


def test_conv_prologue_core_norm_matches_chained_oracles():
    rng = np.random.default_rng(21)
    B, T, Hqk, H, d, K = 1, 333, 2, 4, 128, 4
    C = 2 * Hqk * d + H * d
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev()).to(torch.bfloat16)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    x = bf(rng.standard_normal((B, T, C)))
    w = f32(rng.standard_normal((C, K)) * 0.5)
    a = f32(rng.standard_normal((B, T, H)))
    b = f32(rng.standard_normal((B, T, H)))
    A_log = f32(np.log(rng.uniform(1, 16, H)))
    dt_bias = f32(np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(0.1), H)))))
    z = bf(rng.standard_normal((B, T, H, d)))
    nw = f32(rng.standard_normal(d))
    h0 = f32(0.1 * rng.standard_normal((B, H, d, d)))

    y = gdn.gdn_causal_conv1d(x, w, None, None, silu=True)
    q_raw = y[..., :Hqk * d].reshape(B, T, Hqk, d).contiguous()
    k_raw = y[..., Hqk * d:2 * Hqk * d].reshape(B, T, Hqk, d).contiguous()
    v = y[..., 2 * Hqk * d:].reshape(B, T, H, d).contiguous()
    o, hT = gdn.gdn_chunk_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, d ** -0.5, h0)
    out = gdn.gdn_gated_rmsnorm(o, z, nw, eps=1e-6)
    # the same forward reading q_raw, k_raw and v straight out of the conv output: same bits
    o2, hT2 = gdn.gdn_chunk_fwd_prologue_qkv(y, Hqk, H, d, d, a, b, A_log, dt_bias, d ** -0.5, h0)
    sync()
    assert torch.equal(o2, o) and torch.equal(hT2, hT)

    # oracle chain in fp64 on the exact bf16 / fp32 values the GPU read; the bf16 roundings
    # of the conv output and of o happen on the GPU side only, which the tolerance covers
    y_ref = layer_ops.causal_conv1d(np_f64(x), np_f64(w), None, None, True)
    q_r = y_ref[..., :Hqk * d].reshape(B, T, Hqk, d)
    k_r = y_ref[..., Hqk * d:2 * Hqk * d].reshape(B, T, Hqk, d)
    v_r = y_ref[..., 2 * Hqk * d:].reshape(B, T, H, d)
    o_ref, hT_ref = prologue.gdn_fwd_prologue(q_r, k_r, v_r, np_f64(a), np_f64(b), np_f64(A_log),
                                              np_f64(dt_bias), d ** -0.5, np_f64(h0))
    out_ref = layer_ops.gated_rmsnorm(o_ref, np_f64(z), np_f64(nw), 1e-6)
    for name, got, ref in (("conv", y, y_ref), ("o", o, o_ref), ("hT", hT, hT_ref), ("layer out", out, out_ref)):
        err = rel_l2(np_f64(got), ref)
        print("layer path %s rel-L2 %.3e (bound %.0e)" % (name, err, TOL_BF16))
        assert err <= TOL_BF16, name


def test_packed_qkv_forward_padded_rows():
    """The packed-qkv forward on padded rows of different lengths equals the split-input
    forward bit for bit, and its padded outputs are +0.0."""
    rng = np.random.default_rng(5)
    B, T, Hqk, H, d = 2, 200, 1, 3, 128
    C = 2 * Hqk * d + H * d
    qkv = torch.from_numpy(rng.standard_normal((B, T, C)).astype(np.float32)).to(dev()).to(torch.bfloat16)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    a, b = f32(rng.standard_normal((B, T, H))), f32(rng.standard_normal((B, T, H)))
    A_log, dt_bias = f32(np.zeros(H)), f32(np.full(H, -4.0))
    vl = torch.tensor([200, 131], dtype=torch.int32, device=dev())
    q_raw = qkv[..., :Hqk * d].reshape(B, T, Hqk, d).contiguous()
    k_raw = qkv[..., Hqk * d:2 * Hqk * d].reshape(B, T, Hqk, d).contiguous()
    v = qkv[..., 2 * Hqk * d:].reshape(B, T, H, d).contiguous()
    o, hT = gdn.gdn_chunk_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, None, None, vl)
    o2, hT2 = gdn.gdn_chunk_fwd_prologue_qkv(qkv, Hqk, H, d, d, a, b, A_log, dt_bias, None, None, vl)
    sync()
    assert torch.equal(o2, o) and torch.equal(hT2, hT)
    tail = o2[1, 131:].float()
    assert torch.all(tail == 0) and not torch.any(torch.signbit(tail))


def _layer_inputs(rng, B, T, Hqk, H, d, K, bias=True, halo=True):
    C = 2 * Hqk * d + H * d
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev()).to(torch.bfloat16)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    x = bf(rng.standard_normal((B, T, C)))
    w = f32(rng.standard_normal((C, K)) * 0.5)
    cb = f32(rng.standard_normal(C) * 0.1) if bias else None
    xp = bf(rng.standard_normal((B, K - 1, C))) if halo else None
    a = f32(rng.standard_normal((B, T, H)))
    b = f32(rng.standard_normal((B, T, H)))
    A_log = f32(np.log(rng.uniform(1, 16, H)))
    dt_bias = f32(np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(0.1), H)))))
    h0 = f32(0.1 * rng.standard_normal((B, H, d, d)))
    return x, w, cb, xp, a, b, A_log, dt_bias, h0


FUSED = [
    # name, B, T, Hqk, H, K, bias, halo, valid
    ("k4_bias_halo", 1, 333, 2, 4, 4, True, True, None),
    ("k3_nobias", 2, 200, 1, 3, 3, False, True, None),
    ("k2_nohalo_padded", 2, 257, 2, 4, 2, True, False, [257, 130]),
    ("k4_short", 1, 5, 1, 2, 4, True, True, None),
]


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
def test_conv_fused_into_the_prepare_pass_gives_the_same_bits(case):
    """gdn_chunk_fwd_conv (the Conv1D inside the prepare pass) against the unfused path,
    gdn_causal_conv1d then gdn_chunk_fwd_prologue_qkv: the convolution output y, o and hT
    bit for bit (kernel widths 2-4, with and without bias and halo, padded rows, lengths
    that end inside a chunk)."""
    name, B, T, Hqk, H, K, bias, halo, valid = case
    rng = np.random.default_rng(40 + K + T)
    d = 128
    x, w, cb, xp, a, b, A_log, dt_bias, h0 = _layer_inputs(rng, B, T, Hqk, H, d, K, bias, halo)
    vl = None if valid is None else torch.tensor(valid, dtype=torch.int32, device=dev())
    y_ref = gdn.gdn_causal_conv1d(x, w, cb, xp, silu=True)
    o_ref, hT_ref = gdn.gdn_chunk_fwd_prologue_qkv(y_ref, Hqk, H, d, d, a, b, A_log, dt_bias, None, h0, vl)
    o, hT, y = gdn.gdn_chunk_fwd_conv(x, w, cb, xp, Hqk, H, d, d, a, b, A_log, dt_bias, None, h0, vl)
    sync()
    assert torch.equal(y, y_ref), name + " y"
    assert torch.equal(o, o_ref), name + " o"
    assert torch.equal(hT, hT_ref), name + " hT"


def test_conv_fused_matches_chained_oracles():
    rng = np.random.default_rng(23)
    B, T, Hqk, H, d, K = 1, 300, 2, 4, 128, 4
    x, w, cb, xp, a, b, A_log, dt_bias, h0 = _layer_inputs(rng, B, T, Hqk, H, d, K)
    o, hT, y = gdn.gdn_chunk_fwd_conv(x, w, cb, xp, Hqk, H, d, d, a, b, A_log, dt_bias, None, h0)
    sync()
    y_ref = layer_ops.causal_conv1d(np_f64(x), np_f64(w), np_f64(cb), np_f64(xp), True)
    q_r = y_ref[..., :Hqk * d].reshape(B, T, Hqk, d)
    k_r = y_ref[..., Hqk * d:2 * Hqk * d].reshape(B, T, Hqk, d)
    v_r = y_ref[..., 2 * Hqk * d:].reshape(B, T, H, d)
    o_ref, hT_ref = prologue.gdn_fwd_prologue(q_r, k_r, v_r, np_f64(a), np_f64(b), np_f64(A_log),
                                              np_f64(dt_bias), d ** -0.5, np_f64(h0))
    for nm, got, ref in (("y", y, y_ref), ("o", o, o_ref), ("hT", hT, hT_ref)):
        err = rel_l2(np_f64(got), ref)
        print("fused conv %s rel-L2 %.3e (bound %.0e)" % (nm, err, TOL_BF16))
        assert err <= TOL_BF16, nm


def test_conv_fused_at_the_32k_layer_shapes():
    """The 32K layer's shapes (16 + 16 query/key heads and 32 value heads of 128: C = 8192,
    K = 4, bias, halo) in the launch configuration bench.py times: the same bits as the
    unfused path."""
    rng = np.random.default_rng(24)
    B, T, Hqk, H, d, K = 1, 32768, 16, 32, 128, 4
    x, w, cb, xp, a, b, A_log, dt_bias, h0 = _layer_inputs(rng, B, T, Hqk, H, d, K)
    y_ref = gdn.gdn_causal_conv1d(x, w, cb, xp, silu=True)
    o_ref, hT_ref = gdn.gdn_chunk_fwd_prologue_qkv(y_ref, Hqk, H, d, d, a, b, A_log, dt_bias, None, h0)
    o, hT, y = gdn.gdn_chunk_fwd_conv(x, w, cb, xp, Hqk, H, d, d, a, b, A_log, dt_bias, None, h0)
    sync()
    assert torch.equal(y, y_ref) and torch.equal(o, o_ref) and torch.equal(hT, hT_ref)
