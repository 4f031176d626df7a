"""GPU parity of the packed variable-length forward (gdn_chunk_fwd_varlen): against
the oracle's per-sequence forward, bitwise against gdn_chunk_fwd run on each sequence
alone, and at full size against the padded 8K workload packed without its padding."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_common import TOL_BF16, TOL_F32, dev, np_f64, sync, to_dev, workload_inputs
from helpers import rel_l2
from linear_attention_06_amd import gdn
from linear_attention_06_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def check(x, ref, tol, what):
    err = rel_l2(x, ref)
    print("%s rel-L2 %.3e (bound %.0e)" % (what, err, tol))
    assert np.all(np.isfinite(x)), what
    assert err <= tol, "%s rel-L2 %.3e > %.0e" % (what, err, tol)


CASES = [
    # name, io, d, Hqk, H, lengths
    ("bf16_d128", "bf16", 128, 2, 4, [0, 1, 63, 64, 65, 200, 1000, 37]),
    ("bf16_d128_ratio3", "bf16", 128, 1, 3, [130, 0, 64, 513]),
    ("f32_d32", "f32", 32, 2, 4, [5, 0, 64, 130, 71]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_varlen_matches_oracle_and_each_sequence_alone(case):
    name, io, d, Hqk, H, lens = case
    T = sum(lens)
    w = dataclasses.replace(WORKLOADS["stateful_32k"], name="varlen_" + name, T=T, Hqk=Hqk, H=H,
                            dk=d, dv=d, io=io, seed=400 + len(lens), B=1)
    inp = make_inputs(w)
    N = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(5)
    h0 = (0.1 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    q, k, v, g, beta, _, _ = to_dev(inp)
    h0_t = torch.from_numpy(h0).to(dev())
    cu_t = torch.from_numpy(cu).to(dev())
    o, hT = gdn.gdn_chunk_fwd_varlen(q, k, v, g, beta, cu_t, max(lens), h0_t)
    sync()
    qf, kf, vf, gf, bf, _ = inp.f64()
    o_ref, hT_ref = oracle.gdn_fwd_varlen(qf, kf, vf, gf, bf, cu, h0.astype(np.float64))
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    check(np_f64(o), o_ref, tol, name + " o")
    check(np_f64(hT), hT_ref, tol, name + " hT")
    # each sequence equals the plain forward on that sequence alone, bit for bit
    for b in range(N):
        s, e = int(cu[b]), int(cu[b + 1])
        ob, hb = gdn.gdn_chunk_fwd(q[:, s:e].contiguous(), k[:, s:e].contiguous(), v[:, s:e].contiguous(),
                                   g[:, s:e].contiguous(), beta[:, s:e].contiguous(), h0_t[b:b + 1].contiguous())
        sync()
        assert torch.equal(o[:, s:e], ob), (name, b)
        assert torch.equal(hT[b:b + 1], hb), (name, b)


def test_varlen_padded_8k_packed_equals_the_padded_run():
    """The padded 8K workload (two rows, 7777 valid tokens each) packed without its padding:
    the same outputs on the valid tokens and the same final states, bit for bit."""
    inp = workload_inputs("padded_8k")
    q, k, v, g, beta, _, vl = to_dev(inp)
    o_pad, hT_pad = gdn.gdn_chunk_fwd(q, k, v, g, beta, None, vl)
    L = int(inp.valid_len[0])
    pk = lambda x: torch.cat([x[0:1, :L], x[1:2, :L]], dim=1).contiguous()
    cu = torch.tensor([0, L, 2 * L], dtype=torch.int32, device=dev())
    o, hT = gdn.gdn_chunk_fwd_varlen(pk(q), pk(k), pk(v), pk(g), pk(beta), cu, L)
    sync()
    assert torch.equal(o, pk(o_pad))
    assert torch.equal(hT, hT_pad)


@pytest.mark.parametrize("max_seqlen", [0, 1, 64, 100])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 32)])
def test_varlen_all_empty_sequences_return_initial_states(max_seqlen, dtype, d):
    """No tokens at all: every tensor is empty (its data pointer NULL) while max_seqlen may
    still size one or more chunk records; each sequence returns its initial state. (A state
    pass chosen from the NULL value pointer once read the summary-only records here.)"""
    q = torch.zeros((1, 0, 2, d), dtype=dtype, device=dev())
    v = torch.zeros((1, 0, 4, d), dtype=dtype, device=dev())
    g = torch.zeros((1, 0, 4), dtype=torch.float32, device=dev())
    h0 = torch.randn((3, 4, d, d), device=dev())
    cu = torch.zeros(4, dtype=torch.int32, device=dev())
    o, hT = gdn.gdn_chunk_fwd_varlen(q, q, v, g, g, cu, max_seqlen, h0)
    sync()
    assert torch.equal(hT, h0)
    _, hT0 = gdn.gdn_chunk_fwd_varlen(q, q, v, g, g, cu, max_seqlen, None)
    sync()
    assert int(torch.count_nonzero(hT0)) == 0
