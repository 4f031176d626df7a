"""The C-ABI library without a GPU: it loads, exports what include/gdn.h
declares, sizes workspaces, and rejects bad arguments before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_06_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(gdn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert set(declared_functions()) == set(gdn.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = gdn.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_header_compiles_as_c():
    src = '#include "gdn.h"\nint main(void){ return (int)sizeof(gdn_problem); }\n'
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                          "-x", "c", "-", "-fsyntax-only"], input=src, text=True, capture_output=True)
    assert res.returncode == 0, res.stderr


def P(**kw):
    base = dict(B=1, T=128, H=8, Hqk=4, dk=16, dv=16, chunk=64, io_dtype=gdn.GDN_F32, valid_len=None)
    base.update(kw)
    return gdn.GdnProblem(**base)


def ws_status(p):
    n = ctypes.c_size_t(0)
    return gdn.lib().gdn_chunk_fwd_workspace(ctypes.byref(p), ctypes.byref(n)), n.value


def test_status_strings():
    for s in range(5):
        assert gdn.lib().gdn_status_string(s).decode().startswith("GDN_")


@pytest.mark.parametrize("kw,status", [
    (dict(chunk=32), gdn.GDN_EUNSUPPORTED),
    (dict(dk=48), gdn.GDN_EUNSUPPORTED),
    (dict(dv=256), gdn.GDN_EUNSUPPORTED),
    (dict(io_dtype=7), gdn.GDN_EUNSUPPORTED),
    (dict(H=6, Hqk=4), gdn.GDN_EINVAL),
    (dict(Hqk=0), gdn.GDN_EINVAL),
    (dict(B=-1), gdn.GDN_EINVAL),
    (dict(T=-5), gdn.GDN_EINVAL),
    (dict(dk=0), gdn.GDN_EINVAL),
])
def test_bad_problems_are_rejected(kw, status):
    st, _ = ws_status(P(**kw))
    assert st == status
    assert gdn.lib().gdn_last_error().decode()


def test_workspace_sizes():
    st, n = ws_status(P())
    assert st == gdn.GDN_OK
    nch = 1 * 8 * 2
    assert n >= nch * (2 * 64 * 64 * 2 + 128 * 4)
    st, n0 = ws_status(P(T=0))
    assert st == gdn.GDN_OK and n0 == 0


def call_fwd(p, q=16, k=16, v=16, g=16, b=16, h0=None, o=16, hT=None, ws=None, nbytes=0):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return gdn.lib().gdn_chunk_fwd(ctypes.byref(p) if p is not None else None, vp(q), vp(k), vp(v),
                                   vp(g), vp(b), vp(h0), vp(o), vp(hT), vp(ws), nbytes, None)


def test_fwd_argument_checks_return_before_launch():
    p = P()
    _, need = ws_status(p)
    assert call_fwd(None) == gdn.GDN_EINVAL
    assert call_fwd(p, q=None, ws=256, nbytes=need) == gdn.GDN_EINVAL
    assert call_fwd(p, o=None, ws=256, nbytes=need) == gdn.GDN_EINVAL
    assert call_fwd(p, ws=None, nbytes=0) == gdn.GDN_EWORKSPACE
    assert call_fwd(p, ws=256, nbytes=need - 1) == gdn.GDN_EWORKSPACE
    assert call_fwd(p, ws=258, nbytes=need) == gdn.GDN_EWORKSPACE       # misaligned
    assert call_fwd(P(chunk=128), ws=256, nbytes=need) == gdn.GDN_EUNSUPPORTED
    # token tensors must be 16-byte aligned (moved in 16-byte pieces); without tokens
    # nothing is read
    for name in ("q", "k", "v", "o"):
        assert call_fwd(p, ws=256, nbytes=need, **{name: 24}) == gdn.GDN_EINVAL, name
    assert "16-byte aligned" in gdn.lib().gdn_last_error().decode()
    assert call_fwd(P(B=0), q=24, ws=256, nbytes=need) == gdn.GDN_OK


def call_fwd_prologue(p, q=16, k=16, v=16, a=16, b=16, A_log=16, dt_bias=16, q_scale=0.125, o=16, ws=256,
                      nbytes=1 << 40):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return gdn.lib().gdn_chunk_fwd_prologue(ctypes.byref(p), vp(q), vp(k), vp(v), vp(a), vp(b), vp(A_log),
                                            vp(dt_bias), ctypes.c_float(q_scale), None, vp(o), None, vp(ws),
                                            nbytes, None)


def test_fwd_prologue_argument_checks_return_before_launch():
    bf = P(H=4, Hqk=2, dk=128, dv=128, io_dtype=gdn.GDN_BF16)
    assert call_fwd_prologue(P()) == gdn.GDN_EUNSUPPORTED                 # fp32 path
    assert call_fwd_prologue(P(dk=64, dv=64, io_dtype=gdn.GDN_BF16)) == gdn.GDN_EUNSUPPORTED
    for name in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "o"):
        assert call_fwd_prologue(bf, **{name: None}) == gdn.GDN_EINVAL, name
    assert call_fwd_prologue(bf, q_scale=float("nan")) == gdn.GDN_EINVAL
    assert call_fwd_prologue(bf, q_scale=float("inf")) == gdn.GDN_EINVAL
    assert call_fwd_prologue(bf, ws=None, nbytes=0) == gdn.GDN_EWORKSPACE
    _, need = ws_status(bf)
    assert call_fwd_prologue(bf, nbytes=need - 1) == gdn.GDN_EWORKSPACE
    # the decay record of the matrix-core path is 256 floats per chunk and head
    nch = 1 * 4 * 2
    assert need >= nch * (2 * 6 * 512 * 2 + 256 * 4)


def test_segment_argument_checks():
    L = gdn.lib()
    n = ctypes.c_size_t(0)
    assert L.gdn_segment_workspace(ctypes.byref(P()), 48, ctypes.byref(n)) == gdn.GDN_EINVAL
    assert L.gdn_segment_workspace(ctypes.byref(P(T=192)), 128, ctypes.byref(n)) == gdn.GDN_EINVAL
    assert L.gdn_segment_workspace(ctypes.byref(P()), 0, ctypes.byref(n)) == gdn.GDN_EINVAL
    assert L.gdn_segment_workspace(ctypes.byref(P()), 64, ctypes.byref(n)) == gdn.GDN_OK
    p = P(valid_len=1234)                      # padded rows are allowed in the segment calls
    assert L.gdn_segment_workspace(ctypes.byref(p), 64, ctypes.byref(n)) == gdn.GDN_OK
    vp = ctypes.c_void_p
    st = L.gdn_segment_summary(ctypes.byref(P()), 64, None, vp(16), vp(16), vp(16), vp(16), vp(16), vp(16),
                               vp(256), 1 << 30, None)
    assert st == gdn.GDN_EINVAL
    st = L.gdn_apply_initial_state(ctypes.byref(P()), 64, vp(16), vp(16), vp(16), vp(16), vp(16), None,
                                   vp(16), None, vp(256), 1 << 30, None)
    assert st == gdn.GDN_EINVAL


def test_combine_argument_checks():
    L = gdn.lib()
    vp = ctypes.c_void_p
    assert L.gdn_summary_combine(1, 2, 3, 24, 16, vp(16), vp(16), None, vp(16), None, None, None) == \
        gdn.GDN_EUNSUPPORTED
    assert L.gdn_summary_combine(1, 2, 3, 16, 16, None, vp(16), None, vp(16), None, None, None) == \
        gdn.GDN_EINVAL
    assert L.gdn_summary_combine(-1, 2, 3, 16, 16, vp(16), vp(16), None, vp(16), None, None, None) == \
        gdn.GDN_EINVAL
    # nothing to do: no launch, OK
    assert L.gdn_summary_combine(0, 2, 3, 16, 16, None, None, None, None, None, None, None) == gdn.GDN_OK


def test_importing_the_package_does_not_load_the_library():
    code = ("import linear_attention_06_amd, linear_attention_06_amd.gdn as g, "
            "linear_attention_06_amd.inputs; print(g._lib is None)")
    out = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "True"


def test_kernel_path_selection():
    path = lambda **kw: gdn.gdn_kernel_path(P(**kw))
    assert path(io_dtype=gdn.GDN_BF16, dk=128, dv=128) == "bf16-mfma"
    assert path(io_dtype=gdn.GDN_BF16, dk=128, dv=64) == "bf16-mfma"
    assert path(io_dtype=gdn.GDN_BF16, dk=64, dv=64) == "bf16-mfma-padded"
    assert path(io_dtype=gdn.GDN_F32, dk=64, dv=64) == "f32-mfma-padded"
    assert path(io_dtype=gdn.GDN_F32, dk=16, dv=16) == "f32-mfma-padded"
    assert path(io_dtype=gdn.GDN_F32, dk=128, dv=128) == "f32-mfma"
    assert path(io_dtype=gdn.GDN_F32, dk=128, dv=32) == "f32-mfma"
    with pytest.raises(gdn.GdnError):
        path(chunk=32)


def test_varlen_argument_checks():
    L = gdn.lib()
    n = ctypes.c_size_t(0)
    bf = P(B=3, T=500, H=4, Hqk=2, dk=128, dv=128, io_dtype=gdn.GDN_BF16)
    assert L.gdn_chunk_fwd_varlen_workspace(ctypes.byref(bf), -1, ctypes.byref(n)) == gdn.GDN_EINVAL
    assert L.gdn_chunk_fwd_varlen_workspace(ctypes.byref(bf), 300, ctypes.byref(n)) == gdn.GDN_OK
    # ceil(300 / 64) = 5 chunk records per sequence and head
    assert n.value >= 3 * 4 * 5 * (2 * 6 * 512 * 2 + 256 * 4)
    vp = ctypes.c_void_p
    call = lambda p, cu=1, mx=300, q=1: L.gdn_chunk_fwd_varlen(ctypes.byref(p), vp(cu) if cu else None, mx,
                                                                vp(q) if q else None, vp(16), vp(16), vp(16), vp(16),
                                                                None, vp(16), None, vp(256), 1 << 40, None)
    assert call(bf, cu=None) == gdn.GDN_EINVAL
    assert call(bf, q=None) == gdn.GDN_EINVAL
    assert call(bf, mx=-5) == gdn.GDN_EINVAL
    assert call(P(B=3, T=500, H=4, Hqk=2, dk=128, dv=128, io_dtype=gdn.GDN_BF16, valid_len=1234)) == gdn.GDN_EINVAL


def test_backward_argument_checks():
    L = gdn.lib()
    p = P()
    n = ctypes.c_size_t(0)
    assert L.gdn_chunk_bwd_workspace(ctypes.byref(p), ctypes.byref(n)) == gdn.GDN_OK
    # checkpoints 8 B H ceil(T/64) dk dv and per-tile partials B T H (dv/16) 2 (dk + 1), fp32
    assert n.value >= 4 * (8 * 1 * 8 * 2 * 16 * 16 + 1 * 128 * 8 * 1 * 2 * (16 + 1))
    vp = ctypes.c_void_p
    args = [vp(16)] * 5 + [None, vp(16), None] + [vp(16)] * 5 + [None]
    bad = list(args)
    bad[8] = None                                   # dq
    assert L.gdn_chunk_bwd(ctypes.byref(p), *bad, vp(256), n.value, None) == gdn.GDN_EINVAL
    assert L.gdn_chunk_bwd(ctypes.byref(p), *args, vp(256), n.value - 1, None) == gdn.GDN_EWORKSPACE
    assert L.gdn_chunk_bwd(ctypes.byref(p), *args, vp(258), n.value, None) == gdn.GDN_EWORKSPACE


def test_saved_forward_argument_checks():
    """gdn_chunk_fwd_save / gdn_chunk_bwd_saved: only the chunked matrix-core backward's
    problems, a workspace as large as gdn_chunk_bwd's, and every check before any launch."""
    L = gdn.lib()
    vp = ctypes.c_void_p
    n = ctypes.c_size_t(0)
    assert L.gdn_chunk_fwd_save_workspace(ctypes.byref(P()), ctypes.byref(n)) == gdn.GDN_EUNSUPPORTED
    p = P(B=1, T=300, H=4, Hqk=2, dk=128, dv=128, io_dtype=gdn.GDN_BF16)
    assert L.gdn_chunk_fwd_save_workspace(ctypes.byref(p), ctypes.byref(n)) == gdn.GDN_OK
    nb = ctypes.c_size_t(0)
    assert L.gdn_chunk_bwd_workspace(ctypes.byref(p), ctypes.byref(nb)) == gdn.GDN_OK
    assert n.value == nb.value
    fwd = lambda q=vp(16), o=vp(16), ws=vp(256), nbytes=n.value, pp=p: L.gdn_chunk_fwd_save(
        ctypes.byref(pp), q, vp(16), vp(16), vp(16), vp(16), None, o, None, ws, nbytes, None)
    assert fwd(q=None) == gdn.GDN_EINVAL
    assert fwd(o=None) == gdn.GDN_EINVAL
    assert fwd(nbytes=n.value - 1) == gdn.GDN_EWORKSPACE
    assert fwd(ws=vp(258)) == gdn.GDN_EWORKSPACE
    assert fwd(pp=P()) == gdn.GDN_EUNSUPPORTED
    args = [vp(16)] * 6 + [None] + [vp(16)] * 5 + [None]
    bad = list(args)
    bad[7] = None                                   # dq
    assert L.gdn_chunk_bwd_saved(ctypes.byref(p), *bad, vp(256), n.value, None) == gdn.GDN_EINVAL
    assert L.gdn_chunk_bwd_saved(ctypes.byref(p), *args, vp(256), n.value - 1, None) == gdn.GDN_EWORKSPACE
    assert L.gdn_chunk_bwd_saved(ctypes.byref(P()), *args, vp(256), 1 << 40, None) == gdn.GDN_EUNSUPPORTED
    # heads of 128: the chunked backward (and so the kept forward) on rows of a chunk or more
    for T, ok in ((0, True), (63, False), (64, True)):
        p128 = P(B=1, T=T, H=4, Hqk=2, dk=128, dv=128, io_dtype=gdn.GDN_BF16)
        st = L.gdn_chunk_fwd_save_workspace(ctypes.byref(p128), ctypes.byref(n))
        assert st == (gdn.GDN_OK if ok else gdn.GDN_EUNSUPPORTED), T
    # narrow bf16 heads: kept through the padded problem on rows of 256 tokens or more, with
    # gdn_chunk_bwd's workspace; shorter rows keep the token-level backward and nothing
    for T, ok in ((256, True), (1000, True), (255, False)):
        pn = P(B=2, T=T, H=3, Hqk=1, dk=32, dv=16, io_dtype=gdn.GDN_BF16)
        st = L.gdn_chunk_fwd_save_workspace(ctypes.byref(pn), ctypes.byref(n))
        assert st == (gdn.GDN_OK if ok else gdn.GDN_EUNSUPPORTED), T
        if ok:
            assert L.gdn_chunk_bwd_workspace(ctypes.byref(pn), ctypes.byref(nb)) == gdn.GDN_OK
            assert n.value == nb.value
            assert fwd(pp=pn, nbytes=n.value - 1) == gdn.GDN_EWORKSPACE
            assert L.gdn_chunk_bwd_saved(ctypes.byref(pn), *args, vp(256), n.value - 1, None) == gdn.GDN_EWORKSPACE
        else:
            assert fwd(pp=pn, nbytes=1 << 40) == gdn.GDN_EUNSUPPORTED
            assert L.gdn_chunk_bwd_saved(ctypes.byref(pn), *args, vp(256), 1 << 40, None) == gdn.GDN_EUNSUPPORTED


def test_layer_step_argument_checks():
    L = gdn.lib()
    vp = ctypes.c_void_p
    conv = lambda B=1, T=10, C=16, K=4, io=gdn.GDN_BF16, x=256, w=1, y=512: L.gdn_causal_conv1d(
        B, T, C, K, io, vp(x) if x else None, vp(w) if w else None, None, None, 1, vp(y) if y else None, None)
    assert conv(K=5) == gdn.GDN_EUNSUPPORTED
    assert conv(K=1) == gdn.GDN_EUNSUPPORTED
    assert conv(C=12) == gdn.GDN_EUNSUPPORTED
    assert conv(io=7) == gdn.GDN_EUNSUPPORTED
    assert conv(T=-1) == gdn.GDN_EINVAL
    assert conv(x=None) == gdn.GDN_EINVAL
    assert conv(x=264) == gdn.GDN_EINVAL               # not 16-byte aligned
    assert conv(T=0) == gdn.GDN_OK                      # nothing to do, nothing launched
    norm = lambda rows=10, D=128, io=gdn.GDN_BF16, eps=1e-6, o=256: L.gdn_gated_rmsnorm(
        rows, D, io, vp(o) if o else None, vp(256), vp(16), ctypes.c_float(eps), vp(512), None)
    assert norm(D=48) == gdn.GDN_EUNSUPPORTED
    assert norm(eps=float("nan")) == gdn.GDN_EINVAL
    assert norm(eps=-1.0) == gdn.GDN_EINVAL
    assert norm(o=None) == gdn.GDN_EINVAL
    assert norm(rows=-1) == gdn.GDN_EINVAL
    assert norm(rows=0) == gdn.GDN_OK


def test_noalloc_forward_rejects_oversized_problems_before_any_hip_call():
    """The static scratch of gdn_chunk_fwd_noalloc holds 64 MiB of chunk records; the
    stateful 32K workload needs 208 MiB and is refused before anything touches the GPU."""
    p = P(B=1, T=32768, H=32, Hqk=16, dk=128, dv=128, io_dtype=gdn.GDN_BF16)
    dummy = ctypes.c_void_p(256)
    st = gdn.lib().gdn_chunk_fwd_noalloc(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, None, dummy,
                                         None, None)
    assert st == gdn.GDN_EWORKSPACE
    assert "64" in gdn.lib().gdn_last_error().decode() or "scratch" in gdn.lib().gdn_last_error().decode()
    # a problem of no batch rows is a no-op that needs no device
    assert gdn.lib().gdn_chunk_fwd_noalloc(ctypes.byref(P(B=0)), None, None, None, None, None, None, None,
                                           None, None) == gdn.GDN_OK


def test_padded_narrow_head_workspaces_and_checks():
    """Heads under 128: the forward's workspace holds the dk = 128 problem's records plus q
    and k padded to 128 columns and two 128-row state blocks (bf16 and fp32); the backward pads from 256
    tokens per row on (shorter rows keep the token-level backward's workspace); the checks
    still come before any launch."""
    L = gdn.lib()
    n = ctypes.c_size_t(0)
    B, T, H, Hqk, dk, dv = 2, 300, 4, 2, 64, 32
    p = P(B=B, T=T, H=H, Hqk=Hqk, dk=dk, dv=dv, io_dtype=gdn.GDN_BF16)
    p128 = P(B=B, T=T, H=H, Hqk=Hqk, dk=128, dv=dv, io_dtype=gdn.GDN_BF16)
    st, n_pad = ws_status(p)
    st128, n128 = ws_status(p128)
    assert st == gdn.GDN_OK and st128 == gdn.GDN_OK
    assert n_pad >= n128 + 2 * B * T * Hqk * 128 * 2 + 2 * B * H * 128 * dv * 4
    assert call_fwd(p, ws=256, nbytes=n_pad - 1) == gdn.GDN_EWORKSPACE
    assert call_fwd(p, q=None, ws=256, nbytes=n_pad) == gdn.GDN_EINVAL
    # the segment calls pad too: the dk = 128 problem's segment records, padded q and k,
    # and 128-row staging for M (128 x 128), S / H_in and hT
    nseg, nseg128 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.gdn_segment_workspace(ctypes.byref(p), 64, ctypes.byref(nseg)) == gdn.GDN_EINVAL  # 64 does not divide 300
    ps = P(B=B, T=256, H=H, Hqk=Hqk, dk=dk, dv=dv, io_dtype=gdn.GDN_BF16)
    ps128 = P(B=B, T=256, H=H, Hqk=Hqk, dk=128, dv=dv, io_dtype=gdn.GDN_BF16)
    assert L.gdn_segment_workspace(ctypes.byref(ps), 64, ctypes.byref(nseg)) == gdn.GDN_OK
    assert L.gdn_segment_workspace(ctypes.byref(ps128), 64, ctypes.byref(nseg128)) == gdn.GDN_OK
    blocks = B * H * 4
    assert nseg.value >= nseg128.value + 2 * B * 256 * Hqk * 128 * 2 + blocks * 128 * (128 + dv) * 4
    # the fp32 problem of the same shape pads too, onto the fp32 dk = 128 records
    n_f32 = ws_status(P(B=B, T=T, H=H, Hqk=Hqk, dk=dk, dv=dv))[1]
    n_f32_128 = ws_status(P(B=B, T=T, H=H, Hqk=Hqk, dk=128, dv=dv))[1]
    assert n_f32 >= n_f32_128 + 2 * B * T * Hqk * 128 * 4 + 2 * B * H * 128 * dv * 4
    # backward: padded (T >= 256) needs the dk = dv = 128 problem's workspace and more
    assert L.gdn_chunk_bwd_workspace(ctypes.byref(p), ctypes.byref(n)) == gdn.GDN_OK
    n_bwd = n.value
    full = P(B=B, T=T, H=H, Hqk=Hqk, dk=128, dv=128, io_dtype=gdn.GDN_BF16)
    assert L.gdn_chunk_bwd_workspace(ctypes.byref(full), ctypes.byref(n)) == gdn.GDN_OK
    assert n_bwd > n.value
    short = P(B=B, T=100, H=H, Hqk=Hqk, dk=dk, dv=dv, io_dtype=gdn.GDN_BF16)
    short_f32 = P(B=B, T=100, H=H, Hqk=Hqk, dk=dk, dv=dv)
    assert L.gdn_chunk_bwd_workspace(ctypes.byref(short), ctypes.byref(n)) == gdn.GDN_OK
    n_short = n.value
    assert L.gdn_chunk_bwd_workspace(ctypes.byref(short_f32), ctypes.byref(n)) == gdn.GDN_OK
    assert n_short == n.value
    vp = ctypes.c_void_p
    args = [vp(16)] * 5 + [None, vp(16), None] + [vp(16)] * 5 + [None]
    assert L.gdn_chunk_bwd(ctypes.byref(p), *args, vp(256), n_bwd - 1, None) == gdn.GDN_EWORKSPACE
