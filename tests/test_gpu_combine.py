"""GPU parity of the prefix combine and its backward (gdn_summary_combine,
gdn_summary_combine_bwd) on seeded synthetic summaries, against the oracle's combine and
oracle/segment_backward.py: H_p = M_p H_{p-1} + S_p (hyper-parallel PR #1035, all_gather and
p2p modes). Heads of 128 run the fp32 matrix-core scans; the shapes cover a (b, h) count that
is not a multiple of the eight XCD groups, zero and one segment, a value dim of 64 beside dk =
128, the prefix products M_p ... M_0, and a final-state gradient."""
import numpy as np
import pytest
import torch

import oracle
from oracle import segment_backward as sb
from gpu_common import TOL_F32, dev, np_f64, sync
from helpers import rel_l2
from linear_attention_06_amd import gdn

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, P, dk, dv, with h0, want_prefix, with dhT
    (1, 3, 5, 128, 128, True, True, True),
    (2, 5, 1, 128, 64, False, True, False),
    (1, 2, 0, 128, 128, True, False, True),
    (1, 32, 8, 128, 128, True, False, False),
    (1, 4, 3, 64, 64, True, True, True),     # vector-ALU scans, for comparison
]


def summaries(B, H, P, dk, dv, seed):
    """Contractive transition matrices (as a segment's M is: a product of decayed
    near-projections) and states of unit scale."""
    rng = np.random.default_rng(seed)
    M = (0.9 / np.sqrt(dk)) * rng.standard_normal((B, H, P, dk, dk))
    S = rng.standard_normal((B, H, P, dk, dv))
    h0 = rng.standard_normal((B, H, dk, dv))
    return M.astype(np.float32), S.astype(np.float32), h0.astype(np.float32)


def check(x, ref, what):
    xn = np_f64(x)
    err = rel_l2(xn, ref) if np.linalg.norm(ref) > 0 else float(np.abs(xn).max())
    print("%s rel-L2 %.3e" % (what, err))
    assert np.all(np.isfinite(xn)), what
    assert err <= TOL_F32, "%s rel-L2 %.3e > %.0e" % (what, err, TOL_F32)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_H%d_P%d_dk%d_dv%d" % c[:5])
def test_combine_and_its_backward_match_the_oracle(case):
    B, H, P, dk, dv, with_h0, want_prefix, with_dhT = case
    M, S, h0 = summaries(B, H, P, dk, dv, 900 + P)
    Md, Sd, h0d = (torch.from_numpy(x).to(dev()) for x in (M, S, h0))
    H_in, Mp, hT = gdn.gdn_summary_combine(Md, Sd, h0d if with_h0 else None, want_prefix=want_prefix)
    sync()
    r_hin, r_mp, r_hT = oracle.gdn_summary_combine(M, S, h0 if with_h0 else None, want_prefix=want_prefix)
    if P > 0:
        check(H_in, r_hin, "H_in")
        if want_prefix:
            check(Mp, r_mp, "M prefix")
    check(hT, r_hT, "hT")

    rng = np.random.default_rng(950 + P)
    dH = rng.standard_normal((B, H, P, dk, dv)).astype(np.float32)
    dhT = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if with_dhT else None
    dM, dS, dh0 = gdn.gdn_summary_combine_bwd(Md, H_in, torch.from_numpy(dH).to(dev()),
                                              torch.from_numpy(dhT).to(dev()) if with_dhT else None)
    sync()
    rM, rS, rh0 = sb.summary_combine_bwd(M, np_f64(H_in), dH, dhT)
    if P > 0:
        check(dM, rM, "dM")
        check(dS, rS, "dS")
    check(dh0, rh0, "dh0")
