"""Thin ctypes binding of ``libgdn.so`` (the C ABI in ``include/gdn.h``).

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity, turned into device pointers, and passed with the current HIP
stream. Every step of the computation runs in the HIP kernels; there is no
other implementation behind these functions, and they raise if the library
is missing. Importing this module does not load the library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_EHIP = range(5)
GDN_F32, GDN_BF16 = 0, 1
CHUNK = 64

# The functions include/gdn.h declares.
EXPORTS = ("gdn_status_string", "gdn_last_error", "gdn_kernel_path", "gdn_chunk_fwd_workspace",
           "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_prologue", "gdn_chunk_fwd_prologue_qkv", "gdn_chunk_fwd_conv", "gdn_chunk_fwd_varlen_workspace",
           "gdn_chunk_fwd_varlen", "gdn_chunk_bwd_workspace", "gdn_chunk_bwd", "gdn_chunk_fwd_save_workspace",
           "gdn_chunk_fwd_save", "gdn_chunk_bwd_saved", "gdn_causal_conv1d",
           "gdn_gated_rmsnorm",
           "gdn_segment_workspace", "gdn_segment_summary", "gdn_summary_combine",
           "gdn_apply_initial_state", "gdn_segment_bwd_workspace", "gdn_apply_initial_state_bwd",
           "gdn_summary_combine_bwd", "gdn_segment_summary_bwd")


class GdnProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Hqk", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("valid_len", ctypes.c_void_p)]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, _status_text(status), detail))


_lib = None


def lib():
    """Load libgdn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn.so is not built: run `python -m linear_attention_06_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        pp = ctypes.POINTER(GdnProblem)
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_kernel_path.argtypes = [pp]
        L.gdn_kernel_path.restype = ctypes.c_char_p
        L.gdn_chunk_fwd_workspace.argtypes = [pp, ctypes.POINTER(sz)]
        L.gdn_segment_workspace.argtypes = [pp, i32, ctypes.POINTER(sz)]
        L.gdn_chunk_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_chunk_fwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_chunk_fwd_prologue.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                             vp, sz, vp]
        L.gdn_chunk_fwd_prologue_qkv.argtypes = [pp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.gdn_chunk_fwd_conv.argtypes = [pp, vp, vp, vp, vp, i32, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
                                         sz, vp]
        L.gdn_chunk_fwd_varlen_workspace.argtypes = [pp, i32, ctypes.POINTER(sz)]
        L.gdn_chunk_fwd_varlen.argtypes = [pp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_chunk_bwd_workspace.argtypes = [pp, ctypes.POINTER(sz)]
        L.gdn_chunk_bwd.argtypes = [pp] + [vp] * 15 + [sz, vp]
        L.gdn_chunk_fwd_save_workspace.argtypes = [pp, ctypes.POINTER(sz)]
        L.gdn_chunk_fwd_save.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_chunk_bwd_saved.argtypes = [pp] + [vp] * 14 + [sz, vp]
        L.gdn_causal_conv1d.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp]
        L.gdn_gated_rmsnorm.argtypes = [ctypes.c_int64, i32, i32, vp, vp, vp, ctypes.c_float, vp, vp]
        L.gdn_segment_summary.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_summary_combine.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_apply_initial_state.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_segment_bwd_workspace.argtypes = [pp, i32, ctypes.POINTER(sz)]
        L.gdn_apply_initial_state_bwd.argtypes = [pp, i32] + [vp] * 15 + [sz, vp]
        L.gdn_summary_combine_bwd.argtypes = [i32, i32, i32, i32, i32] + [vp] * 8
        L.gdn_segment_summary_bwd.argtypes = [pp, i32] + [vp] * 12 + [i32, vp, sz, vp]
        for name in ("gdn_chunk_fwd_workspace", "gdn_segment_workspace", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc",
                     "gdn_chunk_fwd_prologue", "gdn_chunk_fwd_prologue_qkv", "gdn_chunk_fwd_conv", "gdn_chunk_fwd_varlen_workspace",
                     "gdn_chunk_fwd_varlen",
                     "gdn_chunk_bwd_workspace", "gdn_chunk_bwd", "gdn_causal_conv1d", "gdn_gated_rmsnorm",
                     "gdn_segment_summary", "gdn_summary_combine", "gdn_apply_initial_state",
                     "gdn_segment_bwd_workspace", "gdn_apply_initial_state_bwd", "gdn_summary_combine_bwd",
                     "gdn_segment_summary_bwd"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_text(status: int) -> str:
    return lib().gdn_status_string(status).decode()


def _check(status: int, where: str):
    if status != GDN_OK:
        raise GdnError(status, where, lib().gdn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def problem(q: torch.Tensor, v: torch.Tensor, valid_len: Optional[torch.Tensor] = None,
            chunk: int = CHUNK) -> GdnProblem:
    """Problem sizes from q [B,T,Hqk,dk] and v [B,T,H,dv]."""
    B, T, Hqk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    io = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}.get(q.dtype, -1)
    vl = None
    if valid_len is not None:
        _dev(valid_len, "valid_len", torch.int32)
        vl = valid_len.data_ptr()
    return GdnProblem(B, T, H, Hqk, dk, dv, chunk, io, vl)


def gdn_kernel_path(p: GdnProblem) -> str:
    """Name of the kernel path the library runs for this problem."""
    r = lib().gdn_kernel_path(ctypes.byref(p))
    if r is None:
        raise GdnError(GDN_EINVAL, "gdn_kernel_path", lib().gdn_last_error().decode())
    return r.decode()


def gdn_chunk_fwd_workspace(p: GdnProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_fwd_workspace(ctypes.byref(p), ctypes.byref(n)), "gdn_chunk_fwd_workspace")
    return n.value


def gdn_segment_workspace(p: GdnProblem, seg_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_segment_workspace(ctypes.byref(p), seg_len, ctypes.byref(n)),
           "gdn_segment_workspace")
    return n.value


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _io_checks(q, k, v, g, beta):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype)
    _dev(g, "g", torch.float32)
    _dev(beta, "beta", torch.float32)


def gdn_chunk_fwd(q, k, v, g, beta, h0=None, valid_len=None, o=None, hT=None, want_state=True,
                  ws=None, stream=None):
    """Chunked forward. Returns (o, hT or None); allocates what is not given."""
    _io_checks(q, k, v, g, beta)
    _dev(h0, "h0", torch.float32)
    p = problem(q, v, valid_len)
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    _dev(o, "o", v.dtype)
    if hT is None and want_state:
        hT = torch.empty((p.B, p.H, p.dk, p.dv), dtype=torch.float32, device=v.device)
    _dev(hT, "hT", torch.float32)
    need = gdn_chunk_fwd_workspace(p)
    if ws is None:
        ws = workspace(need, v.device)
    _check(lib().gdn_chunk_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(h0), _ptr(o), _ptr(hT), _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_chunk_fwd")
    return o, hT


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, h0, o, hT=None, valid_len=None, stream=None):
    """gdn_chunk_fwd without a workspace: the library's static 64 MiB scratch holds the
    chunk records. The caller passes every output (o, and hT or None); nothing is
    allocated here or in the library. Calls that overlap on one GPU race."""
    _io_checks(q, k, v, g, beta)
    _dev(h0, "h0", torch.float32)
    _dev(o, "o", v.dtype)
    _dev(hT, "hT", torch.float32)
    p = problem(q, v, valid_len)
    _check(lib().gdn_chunk_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(h0), _ptr(o), _ptr(hT), _stream(stream)),
           "gdn_chunk_fwd_noalloc")
    return o, hT


def gdn_chunk_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, q_scale=None, h0=None,
                           valid_len=None, o=None, hT=None, want_state=True, ws=None, stream=None):
    """Forward with the input prologue fused in: q_raw, k_raw are normalised per token and
    head (q also scaled by q_scale, default 1/sqrt(dk)), g = -exp(A_log) softplus(a + dt_bias),
    beta = sigmoid(b). Returns (o, hT or None)."""
    for t, n in ((q_raw, "q_raw"), (k_raw, "k_raw"), (v, "v")):
        _dev(t, n, q_raw.dtype)
    for t, n in ((a, "a"), (b, "b"), (A_log, "A_log"), (dt_bias, "dt_bias"), (h0, "h0")):
        _dev(t, n, torch.float32)
    p = problem(q_raw, v, valid_len)
    if q_scale is None:
        q_scale = p.dk ** -0.5
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    _dev(o, "o", v.dtype)
    if hT is None and want_state:
        hT = torch.empty((p.B, p.H, p.dk, p.dv), dtype=torch.float32, device=v.device)
    _dev(hT, "hT", torch.float32)
    need = gdn_chunk_fwd_workspace(p)
    if ws is None:
        ws = workspace(need, v.device)
    _check(lib().gdn_chunk_fwd_prologue(ctypes.byref(p), _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(a), _ptr(b),
                                        _ptr(A_log), _ptr(dt_bias), ctypes.c_float(q_scale), _ptr(h0),
                                        _ptr(o), _ptr(hT), _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_chunk_fwd_prologue")
    return o, hT


def gdn_chunk_fwd_prologue_qkv(qkv, Hqk, H, dk, dv, a, b, A_log, dt_bias, q_scale=None, h0=None,
                               valid_len=None, o=None, hT=None, want_state=True, ws=None, stream=None):
    """The fused-prologue forward reading q_raw, k_raw, v from one packed tensor qkv
    [B, T, 2 Hqk dk + H dv] (bf16) without split copies. Returns (o, hT or None)."""
    _dev(qkv, "qkv", torch.bfloat16)
    for t_, n in ((a, "a"), (b, "b"), (A_log, "A_log"), (dt_bias, "dt_bias"), (h0, "h0")):
        _dev(t_, n, torch.float32)
    B, T, C = qkv.shape
    if C != 2 * Hqk * dk + H * dv:
        raise ValueError("qkv has %d channels, expected 2 Hqk dk + H dv = %d" % (C, 2 * Hqk * dk + H * dv))
    vl = None
    if valid_len is not None:
        _dev(valid_len, "valid_len", torch.int32)
        vl = valid_len.data_ptr()
    p = GdnProblem(B, T, H, Hqk, dk, dv, CHUNK, GDN_BF16, vl)
    if q_scale is None:
        q_scale = dk ** -0.5
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=qkv.device)
    _dev(o, "o", torch.bfloat16)
    if hT is None and want_state:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=qkv.device)
    _dev(hT, "hT", torch.float32)
    need = gdn_chunk_fwd_workspace(p)
    if ws is None:
        ws = workspace(need, qkv.device)
    _check(lib().gdn_chunk_fwd_prologue_qkv(ctypes.byref(p), _ptr(qkv), _ptr(a), _ptr(b), _ptr(A_log),
                                            _ptr(dt_bias), ctypes.c_float(q_scale), _ptr(h0), _ptr(o), _ptr(hT),
                                            _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_chunk_fwd_prologue_qkv")
    return o, hT


def gdn_chunk_fwd_conv(x, conv_w, conv_b, x_prev, Hqk, H, dk, dv, a, b, A_log, dt_bias, q_scale=None, h0=None,
                       valid_len=None, y=None, o=None, hT=None, want_state=True, ws=None, stream=None):
    """The fused-prologue forward with the layer's Conv1D (SiLU) fused into its prepare pass:
    x [B, T, 2 Hqk dk + H dv] bf16 before the convolution, conv_w [C, K] fp32, conv_b [C] or
    None, x_prev [B, K-1, C] or None. Returns (o, hT or None, y), y the convolution's output."""
    _dev(x, "x", torch.bfloat16)
    _dev(x_prev, "x_prev", torch.bfloat16)
    for t_, n in ((conv_w, "conv_w"), (conv_b, "conv_b"), (a, "a"), (b, "b"), (A_log, "A_log"),
                  (dt_bias, "dt_bias"), (h0, "h0")):
        _dev(t_, n, torch.float32)
    B, T, C = x.shape
    if C != 2 * Hqk * dk + H * dv:
        raise ValueError("x has %d channels, expected 2 Hqk dk + H dv = %d" % (C, 2 * Hqk * dk + H * dv))
    vl = None
    if valid_len is not None:
        _dev(valid_len, "valid_len", torch.int32)
        vl = valid_len.data_ptr()
    p = GdnProblem(B, T, H, Hqk, dk, dv, CHUNK, GDN_BF16, vl)
    if q_scale is None:
        q_scale = dk ** -0.5
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", torch.bfloat16)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=x.device)
    _dev(o, "o", torch.bfloat16)
    if hT is None and want_state:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=x.device)
    _dev(hT, "hT", torch.float32)
    if ws is None:
        ws = workspace(gdn_chunk_fwd_workspace(p), x.device)
    _check(lib().gdn_chunk_fwd_conv(ctypes.byref(p), _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(x_prev),
                                    int(conv_w.shape[1]), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                    ctypes.c_float(q_scale), _ptr(h0), _ptr(y), _ptr(o), _ptr(hT), _ptr(ws),
                                    ws.numel(), _stream(stream)), "gdn_chunk_fwd_conv")
    return o, hT, y


def gdn_chunk_fwd_varlen_workspace(p: GdnProblem, max_seqlen: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_fwd_varlen_workspace(ctypes.byref(p), max_seqlen, ctypes.byref(n)),
           "gdn_chunk_fwd_varlen_workspace")
    return n.value


def gdn_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, max_seqlen=None, h0=None, o=None, hT=None,
                         want_state=True, ws=None, stream=None):
    """Packed variable-length forward: q, k [1,T,Hqk,dk], v [1,T,H,dv], g, beta [1,T,H];
    cu_seqlens int32 [N+1] on the device; max_seqlen an int, or None to take it from
    cu_seqlens. Returns (o, hT [N,H,dk,dv] or None). A max_seqlen below the longest
    sequence would cut it (the library leaves the cut tokens unwritten), so it is checked
    against cu_seqlens here (one read of the lengths)."""
    _io_checks(q, k, v, g, beta)
    _dev(h0, "h0", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if q.shape[0] != 1:
        raise ValueError("packed sequences use a batch dimension of 1")
    N = cu_seqlens.numel() - 1
    longest = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if N > 0 else 0
    if max_seqlen is None:
        max_seqlen = longest
    elif int(max_seqlen) < longest:
        raise ValueError("max_seqlen=%d is below the longest sequence (%d tokens)" % (int(max_seqlen), longest))
    p = problem(q, v)
    p.B = N
    if o is None:
        o = torch.zeros(v.shape, dtype=v.dtype, device=v.device)
    _dev(o, "o", v.dtype)
    if hT is None and want_state:
        hT = torch.empty((N, p.H, p.dk, p.dv), dtype=torch.float32, device=v.device)
    _dev(hT, "hT", torch.float32)
    need = gdn_chunk_fwd_varlen_workspace(p, int(max_seqlen))
    if ws is None:
        ws = workspace(need, v.device)
    _check(lib().gdn_chunk_fwd_varlen(ctypes.byref(p), _ptr(cu_seqlens), int(max_seqlen), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), _ptr(ws),
                                      ws.numel(), _stream(stream)),
           "gdn_chunk_fwd_varlen")
    return o, hT


def gdn_chunk_bwd_workspace(p: GdnProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_bwd_workspace(ctypes.byref(p), ctypes.byref(n)), "gdn_chunk_bwd_workspace")
    return n.value


def gdn_chunk_bwd(q, k, v, g, beta, h0, d_o, dhT=None, valid_len=None, want_dh0=True, ws=None, stream=None):
    """Backward of gdn_chunk_fwd. Returns (dq, dk, dv, dg, dbeta, dh0 or None), all fp32."""
    _io_checks(q, k, v, g, beta)
    _dev(d_o, "d_o", v.dtype)
    _dev(h0, "h0", torch.float32)
    _dev(dhT, "dhT", torch.float32)
    p = problem(q, v, valid_len)
    f32 = dict(dtype=torch.float32, device=v.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    dg = torch.empty(g.shape, **f32)
    dbeta = torch.empty(beta.shape, **f32)
    dh0 = torch.empty((p.B, p.H, p.dk, p.dv), **f32) if want_dh0 else None
    need = gdn_chunk_bwd_workspace(p)
    if ws is None:
        ws = workspace(need, v.device)
    _check(lib().gdn_chunk_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                               _ptr(d_o), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
                               _ptr(dh0), _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_chunk_bwd")
    return dq, dk, dv, dg, dbeta, dh0


def gdn_chunk_fwd_save_workspace(p: GdnProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_fwd_save_workspace(ctypes.byref(p), ctypes.byref(n)), "gdn_chunk_fwd_save_workspace")
    return n.value


def gdn_chunk_fwd_save(q, k, v, g, beta, h0=None, valid_len=None, o=None, hT=None, want_state=True,
                       ws=None, stream=None):
    """gdn_chunk_fwd that keeps, in ws, what gdn_chunk_bwd_saved needs. Returns (o, hT or
    None, ws); ws must stay untouched until the backward has run."""
    _io_checks(q, k, v, g, beta)
    _dev(h0, "h0", torch.float32)
    p = problem(q, v, valid_len)
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    _dev(o, "o", v.dtype)
    if hT is None and want_state:
        hT = torch.empty((p.B, p.H, p.dk, p.dv), dtype=torch.float32, device=v.device)
    _dev(hT, "hT", torch.float32)
    need = gdn_chunk_fwd_save_workspace(p)
    if ws is None:
        ws = workspace(need, v.device)
    _check(lib().gdn_chunk_fwd_save(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(h0), _ptr(o), _ptr(hT), _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_chunk_fwd_save")
    return o, hT, ws


def gdn_chunk_bwd_saved(q, k, v, g, beta, d_o, ws, dhT=None, valid_len=None, want_dh0=True, stream=None):
    """Backward from the workspace of gdn_chunk_fwd_save on the same inputs. Returns
    (dq, dk, dv, dg, dbeta, dh0 or None), all fp32."""
    _io_checks(q, k, v, g, beta)
    _dev(d_o, "d_o", v.dtype)
    _dev(dhT, "dhT", torch.float32)
    _dev(ws, "ws", torch.uint8)
    p = problem(q, v, valid_len)
    f32 = dict(dtype=torch.float32, device=v.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    dg = torch.empty(g.shape, **f32)
    dbeta = torch.empty(beta.shape, **f32)
    dh0 = torch.empty((p.B, p.H, p.dk, p.dv), **f32) if want_dh0 else None
    _check(lib().gdn_chunk_bwd_saved(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(d_o), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                     _ptr(dbeta), _ptr(dh0), _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_chunk_bwd_saved")
    return dq, dk, dv, dg, dbeta, dh0


def _io_code(t):
    return {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}.get(t.dtype, -1)


def gdn_causal_conv1d(x, w, bias=None, x_prev=None, silu=True, y=None, stream=None):
    """Causal depthwise Conv1D over tokens: x [B,T,C], w [C,K] fp32, bias [C], x_prev
    [B,K-1,C] (the tokens before the sequence). Returns y [B,T,C] in x's dtype."""
    _dev(x, "x")
    _dev(w, "w", torch.float32)
    _dev(bias, "bias", torch.float32)
    _dev(x_prev, "x_prev", x.dtype)
    B, T, C = x.shape
    K = w.shape[1]
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype)
    _check(lib().gdn_causal_conv1d(B, T, C, K, _io_code(x), _ptr(x), _ptr(w), _ptr(bias), _ptr(x_prev),
                                   1 if silu else 0, _ptr(y), _stream(stream)), "gdn_causal_conv1d")
    return y


def gdn_gated_rmsnorm(o, z, weight, eps=1e-6, y=None, stream=None):
    """Gated RMSNorm over the last dim D of o (rows = all leading dims)."""
    _dev(o, "o")
    _dev(z, "z", o.dtype)
    _dev(weight, "weight", torch.float32)
    D = o.shape[-1]
    if y is None:
        y = torch.empty_like(o)
    _dev(y, "y", o.dtype)
    _check(lib().gdn_gated_rmsnorm(o.numel() // max(D, 1), D, _io_code(o), _ptr(o), _ptr(z), _ptr(weight),
                                   ctypes.c_float(eps), _ptr(y), _stream(stream)), "gdn_gated_rmsnorm")
    return y


def gdn_segment_summary(q, k, v, g, beta, seg_len, M=None, S=None, want_m=True, want_s=True,
                        ws=None, stream=None, valid_len=None):
    """Per-segment (M, S). Returns (M, S, ws); ws is needed by gdn_apply_initial_state."""
    _io_checks(q, k, v, g, beta)
    p = problem(q, v, valid_len)
    P = p.T // seg_len if seg_len > 0 else 0
    dev = v.device
    if M is None and want_m:
        M = torch.empty((p.B, p.H, P, p.dk, p.dk), dtype=torch.float32, device=dev)
    if S is None and want_s:
        S = torch.empty((p.B, p.H, P, p.dk, p.dv), dtype=torch.float32, device=dev)
    _dev(M, "M", torch.float32)
    _dev(S, "S", torch.float32)
    need = gdn_segment_workspace(p, seg_len)
    if ws is None:
        ws = workspace(need, dev)
    _check(lib().gdn_segment_summary(ctypes.byref(p), seg_len, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                     _ptr(beta), _ptr(M), _ptr(S), _ptr(ws), ws.numel(),
                                     _stream(stream)), "gdn_segment_summary")
    return M, S, ws


def gdn_summary_combine(M, S, h0=None, H_in=None, want_prefix=False, M_prefix=None, hT=None,
                        want_state=True, stream=None):
    """Prefix combine. Returns (H_in, M_prefix or None, hT or None)."""
    for t, n in ((M, "M"), (S, "S"), (h0, "h0")):
        _dev(t, n, torch.float32)
    B, H, P, dk, dv = S.shape
    if H_in is None:
        H_in = torch.empty_like(S)
    if M_prefix is None and want_prefix:
        M_prefix = torch.empty_like(M)
    if hT is None and want_state:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=S.device)
    for t, n in ((H_in, "H_in"), (M_prefix, "M_prefix"), (hT, "hT")):
        _dev(t, n, torch.float32)
    _check(lib().gdn_summary_combine(B, H, P, dk, dv, _ptr(M), _ptr(S), _ptr(h0), _ptr(H_in),
                                     _ptr(M_prefix), _ptr(hT), _stream(stream)),
           "gdn_summary_combine")
    return H_in, M_prefix, hT


def gdn_apply_initial_state(q, k, v, g, beta, H_in, seg_len, ws, o=None, hT=None, want_state=True,
                            stream=None, valid_len=None):
    """Segment outputs from their incoming states. Returns (o, hT or None)."""
    _io_checks(q, k, v, g, beta)
    _dev(H_in, "H_in", torch.float32)
    p = problem(q, v, valid_len)
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    if hT is None and want_state:
        hT = torch.empty((p.B, p.H, p.dk, p.dv), dtype=torch.float32, device=v.device)
    _dev(o, "o", v.dtype)
    _dev(hT, "hT", torch.float32)
    _check(lib().gdn_apply_initial_state(ctypes.byref(p), seg_len, _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(g), _ptr(beta), _ptr(H_in), _ptr(o), _ptr(hT),
                                         _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_apply_initial_state")
    return o, hT


def gdn_segment_bwd_workspace(p: GdnProblem, seg_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_segment_bwd_workspace(ctypes.byref(p), seg_len, ctypes.byref(n)), "gdn_segment_bwd_workspace")
    return n.value


def _grads_like(q, k, v, g, beta):
    f32 = dict(dtype=torch.float32, device=v.device)
    return (torch.empty(q.shape, **f32), torch.empty(k.shape, **f32), torch.empty(v.shape, **f32),
            torch.empty(g.shape, **f32), torch.empty(beta.shape, **f32))


def gdn_apply_initial_state_bwd(q, k, v, g, beta, H_in, seg_len, d_o, dhT=None, valid_len=None, want_dH_in=True,
                                ws=None, stream=None):
    """Backward of gdn_apply_initial_state. Returns (dq, dk, dv, dg, dbeta, dH_in or None), fp32."""
    _io_checks(q, k, v, g, beta)
    _dev(H_in, "H_in", torch.float32)
    _dev(d_o, "d_o", v.dtype)
    _dev(dhT, "dhT", torch.float32)
    p = problem(q, v, valid_len)
    dq, dk, dv, dg, db = _grads_like(q, k, v, g, beta)
    dH_in = torch.empty_like(H_in) if want_dH_in else None
    if ws is None:
        ws = workspace(gdn_segment_bwd_workspace(p, seg_len), v.device)
    _check(lib().gdn_apply_initial_state_bwd(ctypes.byref(p), seg_len, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                             _ptr(H_in), _ptr(d_o), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv),
                                             _ptr(dg), _ptr(db), _ptr(dH_in), _ptr(ws), ws.numel(), _stream(stream)),
           "gdn_apply_initial_state_bwd")
    return dq, dk, dv, dg, db, dH_in


def gdn_summary_combine_bwd(M, H_in, dH_in, dhT=None, want_dh0=True, stream=None):
    """Backward of gdn_summary_combine. Returns (dM, dS, dh0 or None)."""
    for t, n in ((M, "M"), (H_in, "H_in"), (dH_in, "dH_in"), (dhT, "dhT")):
        _dev(t, n, torch.float32)
    B, H, P, dk, dv = H_in.shape
    dM = torch.empty_like(M)
    dS = torch.empty_like(H_in)
    dh0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=H_in.device) if want_dh0 else None
    _check(lib().gdn_summary_combine_bwd(B, H, P, dk, dv, _ptr(M), _ptr(H_in), _ptr(dH_in), _ptr(dhT), _ptr(dM),
                                         _ptr(dS), _ptr(dh0), _stream(stream)), "gdn_summary_combine_bwd")
    return dM, dS, dh0


def gdn_segment_summary_bwd(q, k, v, g, beta, seg_len, dM=None, dS=None, grads=None, valid_len=None, ws=None,
                            stream=None):
    """Backward of gdn_segment_summary: the gradients of sum(M dM) + sum(S dS). With grads =
    (dq, dk, dv, dg, dbeta) given, the summaries' share is added to them in place (the
    library accumulates); otherwise new tensors are returned."""
    _io_checks(q, k, v, g, beta)
    _dev(dM, "dM", torch.float32)
    _dev(dS, "dS", torch.float32)
    p = problem(q, v, valid_len)
    accumulate = grads is not None
    if grads is None:
        grads = _grads_like(q, k, v, g, beta)
    for t, n in zip(grads, ("dq", "dk", "dv", "dg", "dbeta")):
        _dev(t, n, torch.float32)
    if ws is None:
        ws = workspace(gdn_segment_bwd_workspace(p, seg_len), v.device)
    _check(lib().gdn_segment_summary_bwd(ctypes.byref(p), seg_len, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(dM), _ptr(dS), *(_ptr(t) for t in grads), 1 if accumulate else 0,
                                         _ptr(ws), ws.numel(), _stream(stream)), "gdn_segment_summary_bwd")
    return grads
