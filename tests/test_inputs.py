"""The seeded input generator: determinism, distributions, padding, bf16 rounding."""
import numpy as np
import torch

from linear_attention_06_amd.inputs import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits,
                                            make_inputs, slow_decay)


def test_bf16_rounding_matches_torch(rng):
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -0.0, 65504.0, 1e-30, 3.0e38, 1.00390625, 1.01171875],
                                 np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_same_seed_same_bytes():
    w = WORKLOADS["tiny_f32"]
    a, b = make_inputs(w), make_inputs(w)
    for n in ("q", "k", "v", "g", "beta", "h0"):
        assert np.array_equal(getattr(a, n), getattr(b, n))


def test_tiny_shapes_and_distributions():
    inp = make_inputs(WORKLOADS["tiny_f32"])
    assert inp.q.shape == (1, 128, 4, 16) and inp.v.shape == (1, 128, 8, 16)
    assert inp.q.dtype == np.float32 and inp.g.dtype == np.float32
    assert np.all(inp.h0 == 0)
    assert np.all(inp.g < 0) and np.all((inp.beta > 0) & (inp.beta < 1))
    kn = np.linalg.norm(inp.k.astype(np.float64), axis=-1)
    qn = np.linalg.norm(inp.q.astype(np.float64), axis=-1)
    assert np.allclose(kn, 1.0, atol=1e-6) and np.allclose(qn, 0.25, atol=1e-6)


def test_padded_inputs_zero_gates_past_valid_length():
    inp = make_inputs(WORKLOADS["padded_8k"], T=200)
    assert inp.valid_len.tolist() == [200, 200]            # clamped to T
    inp = make_inputs(WORKLOADS["padded_8k"], T=8192)
    assert inp.valid_len.tolist() == [7777, 7777]
    assert np.all(inp.g[:, 7777:] == 0) and np.all(inp.beta[:, 7777:] == 0)
    assert np.all(inp.g[:, :7777] < 0)
    assert inp.q.dtype == np.uint16                          # bf16 bits


def test_slow_decay_variant():
    w = slow_decay(WORKLOADS["stateless_8k"], seed=101)
    inp = make_inputs(w, T=256)
    assert np.all(inp.g > -1e-2)
    assert 0.02 < float(np.mean(inp.beta)) < 0.15
