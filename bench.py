"""Benchmark of the chunked Gated DeltaNet forward on one MI355X.

One step = one gdn_chunk_fwd call (chunk prepare + sequential state pass with
outputs) over the stateful 32K-token workload: B = 1, T = 32768, 16 query/key
heads read by 32 value heads, dk = dv = 128, bf16 q/k/v/o, fp32 g, beta and
state, h0 ~ 0.1 N(0,1). Inputs are seeded synthetic tensors resident in HBM
before timing starts.

Prints one JSON line with the throughput, the roofline of the dominant kernel
(its average duration measured with HIP events on the stream it runs on) and
the fp64 CPU oracle timed on this host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
    python bench.py --copy-calibration     # plain 1 GiB device copy, for counter scaling
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN fwd tokens/s at H=32,d=128,T=32K bf16; MFMA util % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
WORKLOAD = "stateful_32k"


def algorithmic_bytes(B, T, H, Hqk, dk, dv, io_bytes=2, stateful=True, h0=None, hT=None):
    """Bytes the method must move: q, k (Hqk heads), v, g, beta read once, o written
    once, h0 read and hT written once (each when present; `stateful` sets both)."""
    h0 = stateful if h0 is None else h0
    hT = stateful if hT is None else hT
    qk = 2 * B * T * Hqk * dk * io_bytes
    vo = 2 * B * T * H * dv * io_bytes
    gb = 2 * B * T * H * 4
    st = ((1 if h0 else 0) + (1 if hT else 0)) * B * H * dk * dv * 4
    return qk + vo + gb + st


def flops_per_token_head(C=64, d=128):
    """Triangle-aware chunk-form flops per token and head: A and P (lower
    triangles, 2 x C d), That X and P U (lower triangles, 2 x C d), K S, Q S and
    K^T V'' (3 x 2 d^2), ignoring the O(C^2) solve."""
    return 5 * C * d + 6 * d * d


def dense_flops_per_token_head(C=64, d=128):
    """The same products counted as dense 64-token tiles: A and P 2 x 2 C d, That X and
    P U 2 x 2 C d, K S, Q S and K^T V'' 3 x 2 d^2 (180,224 at C = 64, d = 128)."""
    return 8 * C * d + 6 * d * d


def roofline_of(nbytes, ms):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"algorithmic_bytes": nbytes, "achieved_gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gdn_state_and_prepare_stateful_32k_hbm_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "linear_attention_06_amd", "csrc", "gdn_mfma.hip")


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when that summary was taken on a different version of the kernel source."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("machine-readable:"):
            kv = dict(item.split("=", 1) for item in line.split()[1:])
            if kv.get("kernel") == kernel and kv.get("source_sha256_prefix") == sha:
                return int(kv["traffic_bytes_per_launch"])
    return None


def recorded_step_traffic():
    """HBM bytes of one gdn_chunk_fwd step (prepare + state pass) from the committed
    counter summary, or None when either kernel's figure is for another source version."""
    a, b = recorded_traffic("prepare"), recorded_traffic("state")
    return None if a is None or b is None else a + b


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_one_thread(workloads, make_inputs):
    """The oracle on one value head of the stateless 8K workload (one (row, head) unit, so
    one thread), repeated for about 3 s: tokens/s of the whole 32-head workload per core."""
    import oracle

    w = workloads["stateless_8k"]
    inp = make_inputs(w)
    q, k, v, g, beta, _ = inp.f64()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.gdn_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], g[:, :, :1], beta[:, :, :1], None)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= 3.0:
            break
    return {"value": runs * w.B * w.T / w.H / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d run(s) of 1 of %d heads x %d tokens (stateless 8K), %.1f s" % (runs, w.H, w.T, dt)}


def measured_peaks(dev, stream):
    """Beside the spec peaks: a plain device copy of 1 GiB (HIP events, 10 copies) and a
    dense bf16 GEMM of 8192^3 through torch.matmul (5 products)."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    a_ = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    b_ = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)

    def timed(fn, reps):
        with torch.cuda.stream(stream):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_copy = timed(lambda: dst.copy_(src), 10)
    ms_mm = timed(lambda: torch.matmul(a_, b_), 5)
    return {"copy_gbs": 2 * n / (ms_copy * 1e-3) / 1e9, "copy_bytes_read_and_written": 2 * n,
            "bf16_gemm_tflops": 2 * 8192 ** 3 / (ms_mm * 1e-3) / 1e12, "gemm": "torch.matmul bf16 8192^3",
            "spec_hbm_gbs": HBM_PEAK_GBS, "spec_bf16_tflops": BF16_PEAK_TFLOPS}


def cpu_baseline(inp, budget_s=30.0, min_s=10.0):
    """The fp64 oracle on the host cores: whole heads of the same workload, as
    many as fit the time budget (measured on one head first), repeated until about
    min_s seconds of work have been timed."""
    import oracle

    q, k, v, g, beta, h0 = inp.f64()
    w = inp.w
    rep = w.H // w.Hqk
    t0 = time.perf_counter()
    oracle.gdn_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :rep], g[:, :, :rep], beta[:, :, :rep],
                   None if h0 is None else h0[:, :rep])
    one = time.perf_counter() - t0   # rep heads on up to rep threads
    threads = oracle.num_threads()
    heads = w.H
    est = one * (heads / rep) / max(1, min(threads, heads) / rep)
    if est > budget_s:
        heads = max(rep, int(w.H * budget_s / est) // rep * rep)
    hq = heads // rep
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.gdn_fwd(q[:, :, :hq], k[:, :, :hq], v[:, :, :heads], g[:, :, :heads], beta[:, :, :heads],
                       None if h0 is None else h0[:, :heads])
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or dt * (runs + 1) / runs > budget_s:
            break
    tokens_per_s = runs * w.B * w.T * (heads / w.H) / dt
    used = min(threads, w.B * heads)   # the oracle runs one (row, head) unit per thread
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "%d run(s) of %d of %d heads x %d tokens (B=%d), fp64 token loop, %.1f s"
                      % (runs, heads, w.H, w.T, w.B, dt),
            "cpu_model": cpu_model(), "host_threads": threads}


def segmented_timing(gdn, q, k, v, g, beta, h0, stream, timed):
    """The stateful sequence cut into 8 segments of 4096 tokens: per-segment summary (M, S),
    prefix combine, then the outputs of every segment from its incoming state."""
    seg_len = 4096
    p = gdn.problem(q, v)
    ws = gdn.workspace(gdn.gdn_segment_workspace(p, seg_len), q.device)
    B, T, H = v.shape[0], v.shape[1], v.shape[2]
    P = T // seg_len
    M = torch_empty((B, H, P, p.dk, p.dk), q.device)
    S = torch_empty((B, H, P, p.dk, p.dv), q.device)
    H_in = torch_empty((B, H, P, p.dk, p.dv), q.device)
    hT = torch_empty((B, H, p.dk, p.dv), q.device)
    o = torch_empty_like_v(v)

    def summary():
        gdn.gdn_segment_summary(q, k, v, g, beta, seg_len, M=M, S=S, ws=ws, stream=stream)

    def combine():
        gdn.gdn_summary_combine(M, S, h0, H_in=H_in, hT=hT, stream=stream)

    def apply():
        gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, seg_len, ws, o=o, hT=hT, stream=stream)

    def whole():
        summary()
        combine()
        apply()

    res = {"segments": P, "seg_len": seg_len, "summary_ms": timed(summary, 5),
           "combine_ms": timed(combine, 5), "apply_ms": timed(apply, 5), "step_ms": timed(whole, 5)}
    res["tokens_per_s"] = B * T / (res["step_ms"] * 1e-3)
    # the method's own bytes for the whole sequence (those of the unsplit forward)
    res["roofline"] = roofline_of(algorithmic_bytes(B, T, H, q.shape[2], p.dk, p.dv), res["step_ms"])
    return res


def prologue_timing(gdn, inp, dev, stream, timed):
    """The forward with the input prologue fused in (gdn_chunk_fwd_prologue on the raw
    q/k draws and the gate inputs a, b, A_log, dt_bias of the same workload), beside the
    same prologue as separate torch ops followed by gdn_chunk_fwd (for comparison only)."""
    import torch

    w = inp.w
    r = inp.raw

    def io(x):
        return torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).view(torch.bfloat16).to(dev)

    f = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    q_raw, k_raw, v = io(r["q_raw"]), io(r["k_raw"]), io(inp.v)
    a, b, A_log, dt_bias, h0 = f(r["a"]), f(r["b"]), f(r["A_log"]), f(r["dt_bias"]), f(inp.h0)
    p = gdn.problem(q_raw, v)
    ws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(p), dev)
    o = torch.empty_like(v)
    hT = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    scale = w.dk ** -0.5

    def fused():
        gdn.gdn_chunk_fwd_prologue(q_raw, k_raw, v, a, b, A_log, dt_bias, scale, h0, o=o, hT=hT, ws=ws,
                                   stream=stream)

    def separate():
        with torch.cuda.stream(stream):
            qn = torch.nn.functional.normalize(q_raw.float(), dim=-1).mul_(scale).to(torch.bfloat16)
            kn = torch.nn.functional.normalize(k_raw.float(), dim=-1).to(torch.bfloat16)
            g = -torch.exp(A_log) * torch.nn.functional.softplus(a + dt_bias)
            beta = torch.sigmoid(b)
        gdn.gdn_chunk_fwd(qn, kn, v, g, beta, h0, o=o, hT=hT, ws=ws, stream=stream)

    ms_f, ms_s = timed(fused, 10), timed(separate, 10)
    return {"fused_ms": ms_f, "fused_tokens_per_s": w.B * w.T / (ms_f * 1e-3),
            "torch_prologue_then_core_ms": ms_s}


def backward_timing(gdn, workloads, make_inputs, dev, stream, timed):
    """gdn_chunk_bwd (all six gradients; the chunked matrix-core backward on these bf16
    heads of 128) on the stateless 8K workload with a seeded output gradient, beside the
    forward on the same inputs, the training step with the forward kept, the same gradients
    through the segment calls and the stateful 32K workload; the per-kernel split is in
    profiles/."""
    import torch

    def io(x):
        return torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).view(torch.bfloat16).to(dev)

    def setup(name):
        w = workloads[name]
        inp = make_inputs(w)
        q, k, v = io(inp.q), io(inp.k), io(inp.v)
        g = torch.from_numpy(inp.g).to(dev)
        beta = torch.from_numpy(inp.beta).to(dev)
        h0 = None if inp.h0 is None else torch.from_numpy(inp.h0).to(dev)
        gen = torch.Generator(device=dev).manual_seed(8)
        d_o = torch.randn(v.shape, device=dev, generator=gen).to(torch.bfloat16)
        return w, q, k, v, g, beta, h0, d_o

    w, q, k, v, g, beta, _, d_o = setup("stateless_8k")
    p = gdn.problem(q, v)
    ws = gdn.workspace(gdn.gdn_chunk_bwd_workspace(p), dev)
    fws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(p), dev)

    def step():
        gdn.gdn_chunk_bwd(q, k, v, g, beta, None, d_o, ws=ws, stream=stream)

    def fwd():
        gdn.gdn_chunk_fwd(q, k, v, g, beta, None, ws=fws, stream=stream)

    def train_step():
        # forward keeping its records and states, then the backward from them
        gdn.gdn_chunk_fwd_save(q, k, v, g, beta, None, ws=ws, stream=stream)
        gdn.gdn_chunk_bwd_saved(q, k, v, g, beta, d_o, ws, stream=stream)

    ms = timed(step, 5)
    ms_fwd = timed(fwd, 5)
    ms_train = timed(train_step, 5)
    ms_bwd_saved = timed(lambda: gdn.gdn_chunk_bwd_saved(q, k, v, g, beta, d_o, ws, stream=stream), 5)
    in_bytes = sum(int(x.numel()) * x.element_size() for x in (q, k, v, g, beta, d_o))
    out = {"workload": "stateless_8k", "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
           "forward_ms": ms_fwd, "ratio_to_forward": ms / ms_fwd,
           "workspace_bytes": int(ws.numel()), "input_bytes": in_bytes,
           "path": gdn.gdn_kernel_path(p),
           "kept_forward": {"fwd_save_plus_bwd_saved_ms": ms_train, "bwd_saved_ms": ms_bwd_saved,
                            "bwd_saved_ratio_to_forward": ms_bwd_saved / ms_fwd,
                            "fwd_plus_bwd_ms": ms_fwd + ms}}

    # the same gradients through the segment calls (4 segments of 2048): apply's backward,
    # the combine's, then the summaries' accumulated onto apply's
    L = 2048
    M, S, seg_ws = gdn.gdn_segment_summary(q, k, v, g, beta, L)
    H_in, _, _ = gdn.gdn_summary_combine(M, S, None)
    bws = gdn.workspace(gdn.gdn_segment_bwd_workspace(p, L), dev)

    def seg_step():
        *grads, dH_in = gdn.gdn_apply_initial_state_bwd(q, k, v, g, beta, H_in, L, d_o, ws=bws, stream=stream)
        dM, dS, _ = gdn.gdn_summary_combine_bwd(M, H_in, dH_in, stream=stream)
        gdn.gdn_segment_summary_bwd(q, k, v, g, beta, L, dM, dS, grads=grads, ws=bws, stream=stream)

    ms_seg = timed(seg_step, 2)
    out["segments_4x2048"] = {"ms_per_step": ms_seg, "workspace_bytes": int(bws.numel()),
                              "note": "apply, combine and summary backward composed, each segment a row "
                                      "of the matrix-core backward"}
    del bws, ws, fws

    # the stateful 32K workload (initial state, 32 heads of 128)
    w, q, k, v, g, beta, h0, d_o = setup("stateful_32k")
    p = gdn.problem(q, v)
    ws = gdn.workspace(gdn.gdn_chunk_bwd_workspace(p), dev)
    fws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(p), dev)
    ms = timed(lambda: gdn.gdn_chunk_bwd(q, k, v, g, beta, h0, d_o, ws=ws, stream=stream), 3)
    ms_fwd = timed(lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, ws=fws, stream=stream), 3)
    gdn.gdn_chunk_fwd_save(q, k, v, g, beta, h0, ws=ws, stream=stream)
    ms_saved = timed(lambda: gdn.gdn_chunk_bwd_saved(q, k, v, g, beta, d_o, ws, stream=stream), 3)
    out["stateful_32k"] = {"ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3), "forward_ms": ms_fwd,
                           "ratio_to_forward": ms / ms_fwd, "workspace_bytes": int(ws.numel()),
                           "bwd_saved_ms": ms_saved}
    return out


def layer_ops_timing(gdn, dev, stream, timed):
    """The streaming layer steps at the 32K layer's shapes: causal Conv1D (K = 4, SiLU) over
    the projected q/k/v channels (16 + 16 query/key heads and 32 value heads of 128: C = 8192)
    and the gated RMSNorm over o (32 heads of 128). Achieved GB/s counts each input read and
    each output written once. Then the three composed with the fused-prologue forward."""
    import torch

    gen = torch.Generator(device=dev).manual_seed(9)
    T, C, K, H, D = 32768, 8192, 4, 32, 128
    x = torch.randn((1, T, C), device=dev, generator=gen).to(torch.bfloat16)
    w = torch.randn((C, K), device=dev, generator=gen) * 0.5
    bias = torch.randn((C,), device=dev, generator=gen) * 0.1
    y = torch.empty_like(x)
    o = torch.randn((1, T, H, D), device=dev, generator=gen).to(torch.bfloat16)
    z = torch.randn((1, T, H, D), device=dev, generator=gen).to(torch.bfloat16)
    wt = torch.randn((D,), device=dev, generator=gen)
    yn = torch.empty_like(o)

    def conv():
        gdn.gdn_causal_conv1d(x, w, bias, None, silu=True, y=y, stream=stream)

    def norm():
        gdn.gdn_gated_rmsnorm(o, z, wt, eps=1e-6, y=yn, stream=stream)

    out = {}
    for name, fn, nbytes in (("causal_conv1d_32k", conv, 2 * x.numel() * 2),
                             ("gated_rmsnorm_32k", norm, 3 * o.numel() * 2)):
        ms = timed(fn, 10)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "bytes": nbytes, "achieved_gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}

    # the composed path: Conv1D over q/k/v channels, split, fused-prologue forward from a
    # 0.1 N(0,1) initial state, gated RMSNorm (the split copies are torch plumbing)
    Hqk = 16
    a_g = torch.randn((1, T, H), device=dev, generator=gen)
    b_g = torch.randn((1, T, H), device=dev, generator=gen)
    A_log = torch.log(torch.rand((H,), device=dev, generator=gen) * 15 + 1)
    dt = torch.exp(torch.rand((H,), device=dev, generator=gen) * (np.log(0.1) - np.log(1e-3)) + np.log(1e-3))
    dt_bias = torch.log(torch.expm1(dt))
    h0 = 0.1 * torch.randn((1, H, D, D), device=dev, generator=gen)
    ov = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    p = gdn.problem(torch.empty((1, T, Hqk, D), dtype=torch.bfloat16, device=dev), ov)
    ws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(p), dev)

    def layer():
        gdn.gdn_causal_conv1d(x, w, bias, None, silu=True, y=y, stream=stream)
        with torch.cuda.stream(stream):
            q_raw = y[..., :Hqk * D].reshape(1, T, Hqk, D).contiguous()
            k_raw = y[..., Hqk * D:2 * Hqk * D].reshape(1, T, Hqk, D).contiguous()
            v = y[..., 2 * Hqk * D:].reshape(1, T, H, D).contiguous()
        gdn.gdn_chunk_fwd_prologue(q_raw, k_raw, v, a_g, b_g, A_log, dt_bias, D ** -0.5, h0, o=ov, hT=hT,
                                   ws=ws, stream=stream)
        gdn.gdn_gated_rmsnorm(ov, z, wt, eps=1e-6, y=yn, stream=stream)

    ms = timed(layer, 5)
    out["conv_prologue_core_norm_32k"] = {"ms": ms, "tokens_per_s": T / (ms * 1e-3),
                                          "note": "q/k/v split by torch copies"}

    def layer_packed():   # the forward reads q_raw, k_raw, v straight out of the conv output
        gdn.gdn_causal_conv1d(x, w, bias, None, silu=True, y=y, stream=stream)
        gdn.gdn_chunk_fwd_prologue_qkv(y, Hqk, H, D, D, a_g, b_g, A_log, dt_bias, D ** -0.5, h0, o=ov, hT=hT,
                                       ws=ws, stream=stream)
        gdn.gdn_gated_rmsnorm(ov, z, wt, eps=1e-6, y=yn, stream=stream)

    ms = timed(layer_packed, 5)
    out["conv_prologue_core_norm_32k_packed_qkv"] = {"ms": ms, "tokens_per_s": T / (ms * 1e-3)}

    def core_packed():   # the same without the Conv1D and the norm: the core alone on y
        gdn.gdn_chunk_fwd_prologue_qkv(y, Hqk, H, D, D, a_g, b_g, A_log, dt_bias, D ** -0.5, h0, o=ov, hT=hT,
                                       ws=ws, stream=stream)

    def conv_in_prepare():   # the Conv1D inside the prepare pass (gdn_chunk_fwd_conv)
        gdn.gdn_chunk_fwd_conv(x, w, bias, None, Hqk, H, D, D, a_g, b_g, A_log, dt_bias, D ** -0.5, h0, y=y,
                               o=ov, hT=hT, ws=ws, stream=stream)

    def layer_fused():
        conv_in_prepare()
        gdn.gdn_gated_rmsnorm(ov, z, wt, eps=1e-6, y=yn, stream=stream)

    out["prologue_core_32k_packed_qkv"] = {"ms": timed(core_packed, 5)}
    out["conv_prologue_core_32k_conv_in_prepare"] = {"ms": timed(conv_in_prepare, 5)}
    ms = timed(layer_fused, 5)
    out["conv_prologue_core_norm_32k_conv_in_prepare"] = {"ms": ms, "tokens_per_s": T / (ms * 1e-3)}
    return out


def other_workloads(gdn, workloads, make_inputs, dev, stream, timed):
    """gdn_chunk_fwd step time on the stateless 8K and padded 8K workloads, and the padded
    rows packed as variable-length sequences (gdn_chunk_fwd_varlen)."""
    import torch

    out = {}
    for name in ("stateless_8k", "padded_8k"):
        w = workloads[name]
        inp = make_inputs(w)

        def io(x):
            return torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).view(torch.bfloat16).to(dev)

        q, k, v = io(inp.q), io(inp.k), io(inp.v)
        g = torch.from_numpy(inp.g).to(dev)
        beta = torch.from_numpy(inp.beta).to(dev)
        vl = None if inp.valid_len is None else torch.from_numpy(inp.valid_len).to(dev)
        p = gdn.problem(q, v, vl)
        ws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(p), dev)
        o = torch.empty_like(v)
        hT = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)

        def step():
            gdn.gdn_chunk_fwd(q, k, v, g, beta, None, valid_len=vl, o=o, hT=hT, ws=ws, stream=stream)

        ms = timed(step, 10)
        out[name] = {"B": w.B, "T": w.T, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
                     "roofline": roofline_of(algorithmic_bytes(w.B, w.T, w.H, w.Hqk, w.dk, w.dv, h0=False,
                                                               hT=True), ms)}
        if name == "padded_8k":
            # the same rows packed without their padding, as variable-length sequences
            L = int(inp.valid_len[0])
            pk = lambda x: torch.cat([x[r:r + 1, :L] for r in range(w.B)], dim=1).contiguous()
            qp, kp, vp, gp, bp = pk(q), pk(k), pk(v), pk(g), pk(beta)
            cu = torch.arange(0, (w.B + 1) * L, L, dtype=torch.int32, device=dev)
            pp = gdn.problem(qp, vp)
            pp.B = w.B
            wsp = gdn.workspace(gdn.gdn_chunk_fwd_varlen_workspace(pp, L), dev)
            op = torch.zeros_like(vp)

            def step_varlen():
                gdn.gdn_chunk_fwd_varlen(qp, kp, vp, gp, bp, cu, L, o=op, hT=hT, ws=wsp, stream=stream)

            ms = timed(step_varlen, 10)
            out["packed_varlen_2x7777"] = {"sequences": w.B, "T": w.B * L, "ms_per_step": ms,
                                           "tokens_per_s": w.B * L / (ms * 1e-3)}
    return out


def other_paths_timing(gdn, workloads, make_inputs, dev, stream, timed):
    """gdn_chunk_fwd off the d = 128 bf16 shapes, on the stateless 8K workload's sizes: heads
    of 64 in bf16 (the matrix-core kernels on q and k padded to 128 columns) and fp32 inputs
    with heads of 128 (the fp32 matrix-core kernels); kernel_path names the path."""
    import dataclasses

    import torch

    out = {}
    base = workloads["stateless_8k"]
    for name, d, io in (("stateless_8k_bf16_d64", 64, "bf16"), ("stateless_8k_f32_d128", 128, "f32")):
        w = dataclasses.replace(base, name=name, dk=d, dv=d, io=io)
        inp = make_inputs(w)

        def dev_io(x):
            t = torch.from_numpy(np.ascontiguousarray(x))
            return (t.view(torch.int16).view(torch.bfloat16) if io == "bf16" else t).to(dev)

        q, k, v = dev_io(inp.q), dev_io(inp.k), dev_io(inp.v)
        g = torch.from_numpy(inp.g).to(dev)
        beta = torch.from_numpy(inp.beta).to(dev)
        p = gdn.problem(q, v)
        ws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(p), dev)
        o = torch.empty_like(v)
        hT = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)

        def step():
            gdn.gdn_chunk_fwd(q, k, v, g, beta, None, o=o, hT=hT, ws=ws, stream=stream)

        ms = timed(step, 5)
        out[name] = {"kernel_path": gdn.gdn_kernel_path(p), "T": w.T, "H": w.H, "d": d, "io": io,
                     "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3)}
    return out


def torch_empty(shape, dev):
    import torch

    return torch.empty(shape, dtype=torch.float32, device=dev)


def torch_empty_like_v(v):
    import torch

    return torch.empty_like(v)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the segmented-path and other-workload timings")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    from linear_attention_06_amd import gdn
    from linear_attention_06_amd.inputs import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))
        return

    w = WORKLOADS[WORKLOAD]
    inp = make_inputs(w)

    def io(x):
        return torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).view(torch.bfloat16).to(dev)

    q, k, v = io(inp.q), io(inp.k), io(inp.v)
    g = torch.from_numpy(inp.g).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    h0 = torch.from_numpy(inp.h0).to(dev)
    p = gdn.problem(q, v)
    path = gdn.gdn_kernel_path(p)
    o = torch.empty_like(v)
    hT = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = gdn.workspace(gdn.gdn_chunk_fwd_workspace(p), dev)

    def step():
        gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, o=o, hT=hT, ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # events between the steps give per-step durations without any synchronisation
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    step_stats = {"median": per_step[len(per_step) // 2], "min": per_step[0],
                  "p90": per_step[min(len(per_step) - 1, int(0.9 * len(per_step)))]}

    # Per-kernel durations. The prepare kernel alone: the segment summary with a
    # single segment and no outputs runs only the prepare pass into the workspace.
    # The state pass alone: gdn_apply_initial_state on that workspace.
    H_in = h0.reshape(w.B, w.H, 1, w.dk, w.dv).contiguous()
    seg_ws = gdn.workspace(gdn.gdn_segment_workspace(p, w.T), dev)

    def prep_only():
        gdn.gdn_segment_summary(q, k, v, g, beta, w.T, want_m=False, want_s=False, ws=seg_ws,
                                stream=stream)

    def state_only():
        gdn.gdn_apply_initial_state(q, k, v, g, beta, H_in, w.T, seg_ws, o=o, hT=hT, stream=stream)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    prep_ms = timed(prep_only, args.steps)
    state_ms = timed(state_only, args.steps)
    dominant, dom_ms = ("state", state_ms) if state_ms >= prep_ms else ("prepare", prep_ms)

    tokens = w.B * w.T
    value = tokens / (ms * 1e-3)
    alg_bytes = algorithmic_bytes(w.B, w.T, w.H, w.Hqk, w.dk, w.dv)
    flops = flops_per_token_head(64, w.dk) * tokens * w.H
    achieved_gbs = alg_bytes / (dom_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if path == "bf16-mfma" else "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": w.B, "T": w.T, "H": w.H, "Hqk": w.Hqk, "dk": w.dk,
                   "dv": w.dv, "chunk": 64, "h0": "0.1*N(0,1)", "kernel_path": path},
        "mfma_util_pct": 100.0 * flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        "mfma_util_dense_pct": 100.0 * dense_flops_per_token_head(64, w.dk) * tokens * w.H / (ms * 1e-3)
                               / (BF16_PEAK_TFLOPS * 1e12),
        "step_roofline": dict(roofline_of(alg_bytes, ms), traffic=recorded_step_traffic(),
                              traffic_unit="bytes/step"),
        "algorithmic_gbs_per_step": alg_bytes / (ms * 1e-3) / 1e9,
        "kernels_ms": {"prepare": prep_ms, "state": state_ms},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(dominant), "traffic_unit": "bytes/launch",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "kernel_ms": dom_ms},
        "step_ms_stats": step_stats,
        "workspace_bytes": int(ws.numel()),
        "wall_s_timed_region": wall,
    }
    if not args.no_extra:
        line["segmented_32k"] = segmented_timing(gdn, q, k, v, g, beta, h0, stream, timed)
        line["other_workloads"] = other_workloads(gdn, WORKLOADS, make_inputs, dev, stream, timed)
        line["fused_prologue_32k"] = prologue_timing(gdn, inp, dev, stream, timed)
        line["backward_8k"] = backward_timing(gdn, WORKLOADS, make_inputs, dev, stream, timed)
        line["layer_ops"] = layer_ops_timing(gdn, dev, stream, timed)
        line["other_paths"] = other_paths_timing(gdn, WORKLOADS, make_inputs, dev, stream, timed)
    if not args.no_extra:
        line["measured_peaks"] = measured_peaks(dev, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
        line["cpu_baseline"]["one_thread_stateless_8k"] = cpu_one_thread(WORKLOADS, make_inputs)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
