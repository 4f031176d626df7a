"""Pins for the oracle's packed variable-length forward. Its only arithmetic is the
token oracle's; what it adds is the slicing of the packed tensors by cu_seqlens and
the per-sequence initial states, which these checks tie to independent arrangements
of the same tokens: the whole tensor as one sequence, equal lengths as a batch of rows,
ragged lengths as padded rows with valid_len, and empty sequences."""
import numpy as np

import oracle
from helpers import random_problem


def test_one_sequence_is_the_plain_forward(rng):
    q, k, v, g, beta, h0 = random_problem(rng, B=1, T=77, H=4, Hqk=2, dk=8, dv=6)
    o, hT = oracle.gdn_fwd(q, k, v, g, beta, h0)
    ov, hTv = oracle.gdn_fwd_varlen(q, k, v, g, beta, [0, 77], h0)
    assert np.array_equal(o, ov) and np.array_equal(hT, hTv)


def test_equal_lengths_are_a_batch_of_rows(rng):
    B, L = 3, 40
    q, k, v, g, beta, h0 = random_problem(rng, B=B, T=L, H=4, Hqk=2, dk=8, dv=6)
    o, hT = oracle.gdn_fwd(q, k, v, g, beta, h0)
    pack = lambda x: x.reshape((1, B * L) + x.shape[2:])
    ov, hTv = oracle.gdn_fwd_varlen(pack(q), pack(k), pack(v), pack(g), pack(beta),
                                    [0, L, 2 * L, 3 * L], h0)
    assert np.array_equal(pack(o), ov) and np.array_equal(hT, hTv)


def test_ragged_lengths_equal_padded_rows(rng):
    lens = [33, 0, 64, 101, 1]
    Tmax = max(lens)
    B = len(lens)
    q, k, v, g, beta, h0 = random_problem(rng, B=B, T=Tmax, H=4, Hqk=2, dk=8, dv=6)
    vl = np.array(lens, np.int32)
    o, hT = oracle.gdn_fwd(q, k, v, g, beta, h0, valid_len=vl)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pk = lambda x: np.concatenate([x[b:b + 1, :lens[b]] for b in range(B)], axis=1)
    ov, hTv = oracle.gdn_fwd_varlen(pk(q), pk(k), pk(v), pk(g), pk(beta), cu, h0)
    assert np.array_equal(hT, hTv)                      # the empty sequence keeps h0
    assert np.array_equal(hTv[1], h0[1])
    for b in range(B):
        assert np.array_equal(o[b, :lens[b]], ov[0, cu[b]:cu[b + 1]])


def test_tokens_outside_every_sequence_are_zero(rng):
    q, k, v, g, beta, h0 = random_problem(rng, B=1, T=50, H=2, Hqk=1, dk=4, dv=4)
    ov, _ = oracle.gdn_fwd_varlen(q, k, v, g, beta, [0, 20, 30], None)
    assert np.all(ov[0, 30:] == 0.0)
    o1, _ = oracle.gdn_fwd(q[:, 20:30], k[:, 20:30], v[:, 20:30], g[:, 20:30], beta[:, 20:30])
    assert np.array_equal(ov[0, 20:30], o1[0])
