"""fp64 CPU oracle for the Gated DeltaNet forward and its segment summaries.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this package. The GPU library shares no code with
it: the arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, token by token)
and ``brute.py`` (explicit transition-matrix products for tiny inputs).

The pages that define the method -- hyper-parallel PR #1035 "linear attention
cp" (modes p2p / all_gather: H_out = M @ H_in + S, prefix combine, apply) and
issue #320, the test report for PR #1114 (section 4.1 head copy and stateful /
stateless use, section 5.2 tail padding) -- are cited per function in the C
source.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, special cases and brute force; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_gdn_fwd.argtypes = [i32, i64, i32, i32, i32, i32, _DP, _DP, _DP, _DP, _DP,
                                   _DP, _IP, _DP, _DP]
    lib.oracle_gdn_fwd.restype = None
    lib.oracle_gdn_segment_summary.argtypes = [i32, i64, i32, i32, i32, i32, i64, _DP, _DP,
                                               _DP, _DP, _DP, _IP, _DP, _DP]
    lib.oracle_gdn_segment_summary.restype = None
    lib.oracle_gdn_summary_combine.argtypes = [i32, i32, i32, i32, i32, _DP, _DP, _DP, _DP,
                                               _DP, _DP]
    lib.oracle_gdn_summary_combine.restype = None
    lib.oracle_gdn_apply_initial_state.argtypes = [i32, i64, i32, i32, i32, i32, i64, _DP,
                                                   _DP, _DP, _DP, _DP, _IP, _DP, _DP, _DP]
    lib.oracle_gdn_apply_initial_state.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


def compile_variant(source_text: str, out_path: str) -> str:
    """Compile an edited copy of the oracle source (used by the tests that plant a
    mistake in the oracle to show that the pins catch it)."""
    src_path = out_path + ".c"
    with open(src_path, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                    "-std=c11", "-o", out_path, src_path, "-lm"], check=True)
    return out_path


class Oracle:
    """The oracle's functions bound to one compiled library (default: liboracle.so)."""

    def __init__(self, lib_path=None):
        self._lib = _load() if lib_path is None else _bind(lib_path)

    def gdn_fwd(self, q, k, v, g, beta, h0=None, valid_len=None, want_state=True):
        return gdn_fwd(q, k, v, g, beta, h0, valid_len, want_state, _lib=self._lib)

    def gdn_segment_summary(self, q, k, v, g, beta, seg_len, valid_len=None, want_m=True,
                            want_s=True):
        return gdn_segment_summary(q, k, v, g, beta, seg_len, valid_len, want_m, want_s,
                                   _lib=self._lib)

    def gdn_summary_combine(self, M, S, h0=None, want_prefix=False):
        return gdn_summary_combine(M, S, h0, want_prefix, _lib=self._lib)

    def gdn_apply_initial_state(self, q, k, v, g, beta, H_in, seg_len, valid_len=None):
        return gdn_apply_initial_state(q, k, v, g, beta, H_in, seg_len, valid_len,
                                       _lib=self._lib)


def num_threads() -> int:
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_num_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    if x.dtype == np.int32:
        return x.ctypes.data_as(_IP)
    return x.ctypes.data_as(_DP)


def _vl(valid_len):
    if valid_len is None:
        return None
    return np.ascontiguousarray(valid_len, dtype=np.int32)


def _dims(q, v):
    B, T, Hqk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    if H % Hqk:
        raise ValueError("H must be a multiple of Hqk")
    return B, T, H, Hqk, dk, dv


def gdn_fwd(q, k, v, g, beta, h0=None, valid_len=None, want_state=True, _lib=None):
    """Token-by-token forward. Returns (o [B,T,H,dv], hT [B,H,dk,dv] or None)."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    vl = _vl(valid_len)
    B, T, H, Hqk, dk, dv = _dims(q, v)
    o = np.empty((B, T, H, dv), np.float64)
    hT = np.empty((B, H, dk, dv), np.float64) if want_state else None
    (_lib or _load()).oracle_gdn_fwd(B, T, H, Hqk, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                           _ptr(beta), _ptr(h0), _ptr(vl), _ptr(o), _ptr(hT))
    return o, hT


def gdn_segment_summary(q, k, v, g, beta, seg_len, valid_len=None, want_m=True, want_s=True,
                        _lib=None):
    """Per-segment (M [B,H,P,dk,dk], S [B,H,P,dk,dv]); either may be skipped (None)."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    vl = _vl(valid_len)
    B, T, H, Hqk, dk, dv = _dims(q, v)
    if seg_len <= 0 or T % seg_len:
        raise ValueError("seg_len must divide T")
    P = T // seg_len
    M = np.empty((B, H, P, dk, dk), np.float64) if want_m else None
    S = np.empty((B, H, P, dk, dv), np.float64) if want_s else None
    (_lib or _load()).oracle_gdn_segment_summary(B, T, H, Hqk, dk, dv, seg_len, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(g), _ptr(beta), _ptr(vl), _ptr(M), _ptr(S))
    return M, S


def gdn_summary_combine(M, S, h0=None, want_prefix=False, _lib=None):
    """Prefix combine. Returns (H_in [B,H,P,dk,dv], M_prefix or None, hT [B,H,dk,dv])."""
    M, S, h0 = map(_f64, (M, S, h0))
    B, H, P, dk, dv = S.shape
    H_in = np.empty_like(S)
    Mp = np.empty_like(M) if want_prefix else None
    hT = np.empty((B, H, dk, dv), np.float64)
    (_lib or _load()).oracle_gdn_summary_combine(B, H, P, dk, dv, _ptr(M), _ptr(S), _ptr(h0), _ptr(H_in),
                                       _ptr(Mp), _ptr(hT))
    return H_in, Mp, hT


def gdn_apply_initial_state(q, k, v, g, beta, H_in, seg_len, valid_len=None, _lib=None):
    """Segment outputs from the incoming states. Returns (o, hT of the last segment)."""
    q, k, v, g, beta, H_in = map(_f64, (q, k, v, g, beta, H_in))
    vl = _vl(valid_len)
    B, T, H, Hqk, dk, dv = _dims(q, v)
    if seg_len <= 0 or T % seg_len:
        raise ValueError("seg_len must divide T")
    o = np.empty((B, T, H, dv), np.float64)
    hT = np.empty((B, H, dk, dv), np.float64)
    (_lib or _load()).oracle_gdn_apply_initial_state(B, T, H, Hqk, dk, dv, seg_len, _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(g), _ptr(beta), _ptr(vl), _ptr(H_in),
                                           _ptr(o), _ptr(hT))
    return o, hT


def gdn_fwd_varlen(q, k, v, g, beta, cu_seqlens, h0=None, want_state=True):
    """Packed variable-length forward: sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1
    of the packed inputs (q, k [1,T,Hqk,dk], v [1,T,H,dv], g, beta [1,T,H]); each runs the
    token-by-token forward on its own tokens from h0[b] (zero if h0 is None). The general
    form of the pages' variable-length rows (issue #320, test report for PR #1114, section
    5.2: rows of one batch with different valid lengths). Returns (o [1,T,H,dv] with zeros
    outside every sequence, hT [N,H,dk,dv] or None)."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    H, dk, dv = v.shape[2], q.shape[3], v.shape[3]
    o = np.zeros(v.shape, np.float64)
    hT = np.empty((N, H, dk, dv), np.float64) if want_state else None
    for b in range(N):
        s, e = int(cu[b]), int(cu[b + 1])
        sl = slice(s, e)
        ob, hb = gdn_fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl],
                         None if h0 is None else h0[b:b + 1], want_state=True)
        o[:, sl] = ob
        if want_state:
            hT[b] = hb[0]
    return o, hT
