"""GPU parity of the streaming layer steps (causal depthwise Conv1D with a left halo,
gated RMSNorm) against their fp64 oracles, at the 32K layer's channel count (16 + 16
query/key heads and 32 value heads of 128: C = 8192) and at small ragged shapes."""
import numpy as np
import pytest
import torch

from oracle import layer_ops
from gpu_common import TOL_BF16, dev, np_f64, sync
from helpers import rel_l2
from linear_attention_06_amd import gdn

pytestmark = pytest.mark.gpu


def to_io(x, io):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    return t.to(torch.bfloat16) if io == "bf16" else t


def seen(t):
    """The values the GPU reads, in fp64."""
    return np_f64(t)


@pytest.mark.parametrize("io,B,T,C,K,halo,silu", [
    ("bf16", 1, 300, 8192, 4, True, True),
    ("bf16", 2, 65, 64, 4, False, True),
    ("f32", 2, 130, 40, 3, True, False),
    ("f32", 1, 7, 16, 2, True, True),
])
def test_conv1d_matches_oracle(io, B, T, C, K, halo, silu):
    rng = np.random.default_rng(T + C + K)
    x = to_io(rng.standard_normal((B, T, C)), io)
    w = torch.from_numpy(rng.standard_normal((C, K)).astype(np.float32) * 0.5).to(dev())
    bias = torch.from_numpy(rng.standard_normal(C).astype(np.float32) * 0.1).to(dev())
    prev = to_io(rng.standard_normal((B, K - 1, C)), io) if halo else None
    y = gdn.gdn_causal_conv1d(x, w, bias, prev, silu=silu)
    sync()
    ref = layer_ops.causal_conv1d(seen(x), np_f64(w), np_f64(bias), None if prev is None else seen(prev), silu)
    err = rel_l2(np_f64(y), ref)
    tol = TOL_BF16 if io == "bf16" else 1e-6
    print("conv1d %s B=%d T=%d C=%d K=%d rel-L2 %.3e (bound %.0e)" % (io, B, T, C, K, err, tol))
    assert err <= tol


def test_conv1d_halo_splits_a_sequence_bitwise():
    """Conv of the whole sequence equals the conv of two pieces, the second given the
    first's last three tokens as its halo: bit for bit."""
    rng = np.random.default_rng(3)
    B, T, C, K = 2, 200, 256, 4
    x = to_io(rng.standard_normal((B, T, C)), "bf16")
    w = torch.from_numpy(rng.standard_normal((C, K)).astype(np.float32)).to(dev())
    full = gdn.gdn_causal_conv1d(x, w)
    for cut in (3, 64, 101):
        a = gdn.gdn_causal_conv1d(x[:, :cut].contiguous(), w)
        b = gdn.gdn_causal_conv1d(x[:, cut:].contiguous(), w, x_prev=x[:, cut - K + 1:cut].contiguous())
        sync()
        assert torch.equal(torch.cat([a, b], dim=1), full)


@pytest.mark.parametrize("io,rows,D", [("bf16", 4096 * 32, 128), ("bf16", 999, 64), ("f32", 513, 32),
                                        ("f32", 17, 16)])
def test_gated_rmsnorm_matches_oracle(io, rows, D):
    rng = np.random.default_rng(rows + D)
    o = to_io(rng.standard_normal((rows, D)), io)
    z = to_io(rng.standard_normal((rows, D)), io)
    wt = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).to(dev())
    y = gdn.gdn_gated_rmsnorm(o, z, wt, eps=1e-6)
    sync()
    ref = layer_ops.gated_rmsnorm(seen(o), seen(z), np_f64(wt), 1e-6)
    err = rel_l2(np_f64(y), ref)
    tol = TOL_BF16 if io == "bf16" else 1e-5
    print("gated_rmsnorm %s rows=%d D=%d rel-L2 %.3e (bound %.0e)" % (io, rows, D, err, tol))
    assert err <= tol


def test_layer_steps_at_the_timed_sizes_sampled():
    """Both steps at the sizes bench.py times them (Conv1D over [1, 32768, 8192] bf16 with
    K = 4 and SiLU; the gated RMSNorm over 32768 x 32 rows of 128), checked on sampled
    channels and rows: each channel of the conv and each row of the norm is independent,
    so the oracle on a sample is exact for it."""
    gen = torch.Generator(device=dev()).manual_seed(11)
    T, C, K = 32768, 8192, 4
    x = torch.randn((1, T, C), device=dev(), generator=gen).to(torch.bfloat16)
    w = torch.randn((C, K), device=dev(), generator=gen) * 0.5
    bias = torch.randn((C,), device=dev(), generator=gen) * 0.1
    y = gdn.gdn_causal_conv1d(x, w, bias, silu=True)
    sync()
    rng = np.random.default_rng(12)
    # the first and last channel groups, and a random sample of the rest
    chans = np.unique(np.concatenate([np.arange(8), np.arange(C - 8, C), rng.choice(C, 80, replace=False)]))
    ci = torch.from_numpy(chans).to(dev())
    ref = layer_ops.causal_conv1d(seen(x.index_select(2, ci)), np_f64(w[ci]), np_f64(bias[ci]), None, True)
    err = rel_l2(np_f64(y.index_select(2, ci)), ref)
    print("conv1d at 32768 x 8192, %d channels sampled: rel-L2 %.3e (bound %.0e)" % (len(chans), err, TOL_BF16))
    assert err <= TOL_BF16

    rows, D = 32768 * 32, 128
    o = torch.randn((rows, D), device=dev(), generator=gen).to(torch.bfloat16)
    z = torch.randn((rows, D), device=dev(), generator=gen).to(torch.bfloat16)
    wt = torch.randn((D,), device=dev(), generator=gen)
    yn = gdn.gdn_gated_rmsnorm(o, z, wt, eps=1e-6)
    sync()
    ri = torch.from_numpy(np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 4096, replace=False)]))).to(dev())
    ref = layer_ops.gated_rmsnorm(seen(o.index_select(0, ri)), seen(z.index_select(0, ri)), np_f64(wt), 1e-6)
    err = rel_l2(np_f64(yn.index_select(0, ri)), ref)
    print("gated_rmsnorm at %d rows of %d, %d rows sampled: rel-L2 %.3e (bound %.0e)" % (rows, D, len(ri), err, TOL_BF16))
    assert err <= TOL_BF16
