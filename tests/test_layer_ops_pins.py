"""Pins for the conv1d and gated-RMSNorm oracles: special kernels with known outputs
(identity, pure shift), the halo rule that lets a sequence be cut between ranks, and
the closed forms of the norm (unit rows, scale invariance, silu(0) = 0)."""
import numpy as np

from oracle import layer_ops


def test_conv_identity_and_shift_kernels(rng):
    x = rng.standard_normal((2, 11, 16))
    K = 4
    w_id = np.zeros((16, K)); w_id[:, K - 1] = 1.0
    assert np.array_equal(layer_ops.causal_conv1d(x, w_id, apply_silu=False), x)
    w_sh = np.zeros((16, K)); w_sh[:, 0] = 1.0         # y_t = x_{t-3}
    y = layer_ops.causal_conv1d(x, w_sh, apply_silu=False)
    assert np.array_equal(y[:, 3:], x[:, :-3]) and np.all(y[:, :3] == 0)
    prev = rng.standard_normal((2, K - 1, 16))
    y2 = layer_ops.causal_conv1d(x, w_sh, x_prev=prev, apply_silu=False)
    assert np.array_equal(y2[:, :3], prev)
    # bias and SiLU: silu(0) = 0, silu(b) for a zero input
    b = rng.standard_normal(16)
    y3 = layer_ops.causal_conv1d(np.zeros_like(x), w_sh, bias=b)
    assert np.allclose(y3, b / (1 + np.exp(-b)), rtol=1e-15, atol=0)


def test_conv_halo_splits_a_sequence(rng):
    """Conv over the whole sequence == conv over two pieces, the second given the last
    K - 1 tokens of the first as its halo (the p2p exchange)."""
    B, T, C, K = 2, 40, 24, 4
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    full = layer_ops.causal_conv1d(x, w, bias)
    for cut in (1, 3, 17, 39):
        a = layer_ops.causal_conv1d(x[:, :cut], w, bias)
        halo = np.concatenate([np.zeros((B, K - 1, C)), x[:, :cut]], axis=1)[:, -(K - 1):]
        b = layer_ops.causal_conv1d(x[:, cut:], w, bias, x_prev=halo)
        assert np.max(np.abs(np.concatenate([a, b], axis=1) - full)) < 1e-15


def test_conv_matches_numpy_convolve(rng):
    x = rng.standard_normal((1, 30, 8))
    w = rng.standard_normal((8, 3))
    y = layer_ops.causal_conv1d(x, w, apply_silu=False)
    for c in range(8):
        ref = np.convolve(x[0, :, c], w[c, ::-1])[:30]    # causal: output t uses x[t-2..t]
        assert np.max(np.abs(y[0, :, c] - ref)) < 1e-14


def test_norm_closed_forms(rng):
    o = rng.standard_normal((5, 7, 32))
    z = rng.standard_normal((5, 7, 32))
    wt = rng.standard_normal(32)
    y = layer_ops.gated_rmsnorm(o, z, wt, 0.0)
    # rows of o / rms(o) have mean square 1
    u = layer_ops.gated_rmsnorm(o, np.full_like(z, 50.0), np.ones(32), 0.0) / layer_ops.silu(50.0)
    assert np.max(np.abs(np.mean(u * u, axis=-1) - 1.0)) < 1e-13
    # invariant to scaling o when eps = 0; silu(0) = 0 zeroes the output
    assert np.max(np.abs(layer_ops.gated_rmsnorm(3.5 * o, z, wt, 0.0) - y)) < 1e-13
    assert np.all(layer_ops.gated_rmsnorm(o, np.zeros_like(z), wt, 1e-6) == 0)
    # eps: a zero row stays zero
    assert np.all(layer_ops.gated_rmsnorm(np.zeros_like(o), z, wt, 1e-6) == 0)
