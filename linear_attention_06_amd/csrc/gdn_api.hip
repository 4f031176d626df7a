// gdn_api.hip -- the C ABI declared in include/gdn.h: argument checks,
// workspace sizing and kernel selection. Every check runs before anything is
// enqueued; no exception leaves this file.
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/gdn.h"
#include "gdn_internal.hpp"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

gdn_status hip_fail(hipError_t e, const char* what) {
    return fail(GDN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Kernel path: bf16 I/O with dk == 128 runs on the bf16 matrix cores; every
// other problem runs on the fp32 vector-ALU kernels.
bool use_mfma(const gdn_problem& p) { return p.io_dtype == GDN_BF16 && p.dk == 128; }

// gdn_chunk_fwd on heads with dk < 128 runs the dk = 128 matrix-core kernels (bf16, or fp32
// for fp32 inputs) on q and k zero-padded to 128 columns (and h0 to 128 rows): the padded
// columns add exact zeros to every q.k and k.k product and to K S, and the state's padded
// rows start at zero and stay zero (their transition is a pure decay), so o and the first
// dk rows of the final state are those of the unpadded problem. Without tokens there is
// nothing to pad (hT = h0 or zero needs no workspace).
bool use_mfma_padded(const gdn_problem& p) { return p.dk < 128 && p.T > 0; }
int64_t io_bytes(const gdn_problem& p) { return p.io_dtype == GDN_BF16 ? 2 : 4; }
gdn_problem padded_problem(const gdn_problem& p) {
    gdn_problem w = p;
    w.dk = 128;
    return w;
}

// Chunk intermediates: one record per (b, h, chunk). The two 64x64 matrices take
// their 6 lower-triangle 16x32 blocks in bf16 on the matrix-core path, and are
// stored whole in fp32 otherwise.
// The segment calls on the matrix-core path also keep the bf16 remainder of
// That (used by the summary-matrix pass).
struct Plan {
    int64_t NT = 0, nch = 0;
    size_t that_off = 0, pmat_off = 0, gates_off = 0, that_lo_off = 0, bytes = 0;
    bool lo = false;
};

// max_len: the longest row in tokens (T, or max_seqlen for packed sequences)
Plan make_plan(const gdn_problem& p, bool segments, int64_t max_len = -1) {
    Plan pl;
    pl.NT = ((max_len < 0 ? static_cast<int64_t>(p.T) : max_len) + gdn::kChunk - 1) / gdn::kChunk;
    pl.nch = static_cast<int64_t>(p.B) * p.H * pl.NT;
    const bool mfma = use_mfma(p);
    const size_t rec = mfma ? static_cast<size_t>(gdn::kTriRecordElems) * 2 : 64 * 64 * sizeof(float);
    const size_t mat = align256(static_cast<size_t>(pl.nch) * rec);
    pl.that_off = 0;
    pl.pmat_off = mat;
    pl.gates_off = 2 * mat;
    const size_t gate = mfma ? gdn::kGateRecordMfma : gdn::kGateRecordF32;
    pl.bytes = 2 * mat + align256(static_cast<size_t>(pl.nch) * gate * sizeof(float));
    pl.lo = mfma && segments;
    if (pl.lo) {
        pl.that_lo_off = pl.bytes;
        pl.bytes += mat;
    }
    return pl;
}

gdn::Workspace carve(const Plan& pl, void* ws) {
    char* base = static_cast<char*>(ws);
    gdn::Workspace w;
    w.that = base + pl.that_off;
    w.pmat = base + pl.pmat_off;
    w.gates = reinterpret_cast<float*>(base + pl.gates_off);
    w.that_lo = pl.lo ? base + pl.that_lo_off : nullptr;
    return w;
}

gdn_status check_problem(const gdn_problem* p) {
    if (!p) return fail(GDN_EINVAL, "problem pointer is NULL");
    if (p->B < 0 || p->T < 0) return fail(GDN_EINVAL, "B=%d and T=%d must be >= 0", p->B, p->T);
    if (p->H <= 0 || p->Hqk <= 0) return fail(GDN_EINVAL, "H=%d and Hqk=%d must be > 0", p->H, p->Hqk);
    if (p->H % p->Hqk) return fail(GDN_EINVAL, "H=%d is not a multiple of Hqk=%d", p->H, p->Hqk);
    if (p->H > 65535) return fail(GDN_EUNSUPPORTED, "H=%d exceeds 65535", p->H);
    if (p->chunk != gdn::kChunk) return fail(GDN_EUNSUPPORTED, "chunk=%d: only 64 is supported", p->chunk);
    if (p->dk <= 0 || p->dv <= 0) return fail(GDN_EINVAL, "dk=%d and dv=%d must be > 0", p->dk, p->dv);
    if (!head_dim_ok(p->dk) || !head_dim_ok(p->dv))
        return fail(GDN_EUNSUPPORTED, "dk=%d, dv=%d: head dims must be 16, 32, 64 or 128", p->dk, p->dv);
    if (p->io_dtype != GDN_F32 && p->io_dtype != GDN_BF16)
        return fail(GDN_EUNSUPPORTED, "io_dtype=%d: only GDN_F32 and GDN_BF16", p->io_dtype);
    if (use_mfma(*p)) {
        // the matrix-core kernels address one batch row of q, k, v, o with 32-bit byte offsets
        const int64_t row_qk = static_cast<int64_t>(p->T + gdn::kChunk) * p->Hqk * p->dk * 2;
        const int64_t row_vo = static_cast<int64_t>(p->T + gdn::kChunk) * p->H * p->dv * 2;
        if (row_qk >= (int64_t(1) << 31) || row_vo >= (int64_t(1) << 31))
            return fail(GDN_EUNSUPPORTED, "one batch row of q/k or v/o exceeds 2 GiB on the bf16 path");
    }
    return GDN_OK;
}

gdn_status check_ws(const Plan& pl, void* ws, size_t ws_bytes) {
    if (pl.bytes == 0) return GDN_OK;
    if (!ws) return fail(GDN_EWORKSPACE, "workspace is NULL, %zu bytes needed", pl.bytes);
    if (ws_bytes < pl.bytes)
        return fail(GDN_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, pl.bytes);
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return fail(GDN_EWORKSPACE, "workspace must be 256-byte aligned");
    return GDN_OK;
}

gdn_status check_segments(const gdn_problem& p, int32_t seg_len, int64_t* P) {
    if (seg_len <= 0 || seg_len % gdn::kChunk)
        return fail(GDN_EINVAL, "seg_len=%d must be a positive multiple of 64", seg_len);
    if (p.T % seg_len) return fail(GDN_EINVAL, "seg_len=%d does not divide T=%d", seg_len, p.T);
    *P = p.T / seg_len;
    if (static_cast<int64_t>(p.B) * *P > 65535)
        return fail(GDN_EUNSUPPORTED, "B * P = %lld exceeds 65535", static_cast<long long>(p.B * *P));
    return GDN_OK;
}

gdn_status run_prep(const gdn_problem& p, const Plan& pl, const void* q, const void* k,
                    const float* g, const float* beta, const gdn::Workspace& w, hipStream_t s,
                    const gdn::Prologue* pro = nullptr, const int32_t* cu_seqlens = nullptr) {
    if (pl.nch == 0) return GDN_OK;
    gdn::PrepArgs a;
    a.B = p.B; a.T = p.T; a.H = p.H; a.Hqk = p.Hqk; a.dk = p.dk; a.NT = static_cast<int>(pl.NT);
    a.q = q; a.k = k; a.g = g; a.beta = beta; a.valid_len = p.valid_len; a.ws = w;
    a.cu_seqlens = cu_seqlens;
    a.qk_stride = static_cast<int64_t>(p.Hqk) * p.dk;
    a.has_prologue = pro ? 1 : 0;
    a.pro = pro ? *pro : gdn::Prologue{nullptr, nullptr, nullptr, nullptr, 1.f};
    a.has_conv = 0;
    a.conv = gdn::PrepConv{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
    hipError_t e = use_mfma(p) ? gdn::launch_prep_mfma(a, s)
                               : gdn::launch_prep_f32path(a, p.io_dtype == GDN_BF16, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "prepare kernel launch");
}

gdn::StateArgs state_args(const gdn_problem& p, const Plan& pl, const void* q, const void* k,
                          const void* v, const gdn::Workspace& w) {
    gdn::StateArgs a;
    a.B = p.B; a.T = p.T; a.H = p.H; a.Hqk = p.Hqk; a.dk = p.dk; a.ncols = p.dv;
    a.NT = static_cast<int>(pl.NT);
    a.P = 1; a.Lc = static_cast<int>(pl.NT);
    a.pass = gdn::kPassOutputs;
    a.q = q; a.k = k; a.v = v; a.valid_len = p.valid_len; a.cu_seqlens = nullptr; a.ws = w;
    a.qk_stride = static_cast<int64_t>(p.Hqk) * p.dk;
    a.v_stride = static_cast<int64_t>(p.H) * p.dv;
    a.init_mode = gdn::kInitZero; a.s_init = nullptr; a.s_init_per_segment = 0;
    a.o = nullptr; a.s_out = nullptr; a.store_mode = gdn::kStoreNone; a.m_out = nullptr;
    return a;
}

gdn_status run_state(const gdn_problem& p, const gdn::StateArgs& a, hipStream_t s) {
    if (p.B == 0 || a.P == 0) return GDN_OK;
    // the summary-M passes read the bf16 remainder of That, which only a segment
    // workspace holds
    if (use_mfma(p) && (a.pass == gdn::kPassM || a.pass == gdn::kPassMS) && !a.ws.that_lo)
        return fail(GDN_EWORKSPACE, "the summary-matrix pass needs a segment workspace");
    hipError_t e = use_mfma(p) ? gdn::launch_state_mfma(a, s)
                               : gdn::launch_state_f32path(a, p.io_dtype == GDN_BF16, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "state kernel launch");
}

// The kernels read and write the token tensors with 16-byte accesses.
bool aligned16(std::initializer_list<const void*> ptrs) {
    for (const void* x : ptrs)
        if (reinterpret_cast<uintptr_t>(x) % 16) return false;
    return true;
}

gdn_status check_fwd_args(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const void* o) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !o))
        return fail(GDN_EINVAL, "q, k, v, g, beta and o must be non-NULL");
    if (tokens && !aligned16({q, k, v, o})) return fail(GDN_EINVAL, "q, k, v and o must be 16-byte aligned");
    return GDN_OK;
}

// The forward on a checked problem with a workspace of at least pl.bytes.
gdn_status run_fwd(const gdn_problem& p, const Plan& pl, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* h0, void* o, float* hT, void* ws,
                   hipStream_t s) {
    if (p.B == 0) return GDN_OK;
    const gdn::Workspace w = carve(pl, ws);
    gdn_status st = run_prep(p, pl, q, k, g, beta, w, s);
    if (st != GDN_OK) return st;
    gdn::StateArgs a = state_args(p, pl, q, k, v, w);
    a.init_mode = h0 ? gdn::kInitLoad : gdn::kInitZero;
    a.s_init = h0;
    a.o = o;
    a.s_out = hT;
    a.store_mode = hT ? gdn::kStoreLastSegment : gdn::kStoreNone;
    return run_state(p, a, s);
}

// Workspace of the padded forward: the dk = 128 problem's chunk records, then q and k
// padded to 128 columns ([B, T, Hqk, 128] bf16), h0 and the final state padded to 128 rows
// ([B, H, 128, dv] fp32).
struct PadPlan {
    Plan rec;
    size_t q_off = 0, k_off = 0, h0_off = 0, hT_off = 0, bytes = 0;
};

// packed: the tokens of B packed sequences lie in one row of T (cu_seqlens)
PadPlan make_pad_plan(const gdn_problem& p, int64_t max_len = -1, bool packed = false) {
    PadPlan pp;
    pp.rec = make_plan(padded_problem(p), false, max_len);
    const size_t tokens = packed ? static_cast<size_t>(p.T) : static_cast<size_t>(p.B) * p.T;
    const size_t qk = align256(tokens * p.Hqk * 128 * io_bytes(p));
    const size_t st = align256(static_cast<size_t>(p.B) * p.H * 128 * p.dv * 4);
    pp.q_off = align256(pp.rec.bytes);
    pp.k_off = pp.q_off + qk;
    pp.h0_off = pp.k_off + qk;
    pp.hT_off = pp.h0_off + st;
    pp.bytes = pp.hT_off + st;
    return pp;
}

gdn_status run_varlen(const gdn_problem& p, const Plan& pl, const int32_t* cu_seqlens, const void* q, const void* k,
                      const void* v, const float* g, const float* beta, const float* h0, void* o, float* hT, void* ws,
                      hipStream_t s);

// The forward of a problem with dk < 128 on padded copies (cu_seqlens: packed sequences,
// through the varlen body).
gdn_status run_fwd_padded(const gdn_problem& p, const PadPlan& pp, const int32_t* cu_seqlens, const void* q,
                          const void* k, const void* v, const float* g, const float* beta, const float* h0,
                          void* o, float* hT, void* ws, hipStream_t s) {
    if (p.B == 0) return GDN_OK;
    char* base = static_cast<char*>(ws);
    const int64_t qk_rows = (cu_seqlens ? static_cast<int64_t>(p.T) : static_cast<int64_t>(p.B) * p.T) * p.Hqk;
    const int64_t blocks = static_cast<int64_t>(p.B) * p.H;
    const int64_t st_in = static_cast<int64_t>(p.dk) * p.dv * 4, st_pad = static_cast<int64_t>(128) * p.dv * 4;
    const int64_t es = io_bytes(p);
    hipError_t e = gdn::launch_copy_rows(q, p.dk * es, base + pp.q_off, 128 * es, qk_rows, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(k, p.dk * es, base + pp.k_off, 128 * es, qk_rows, s);
    if (e == hipSuccess && h0) e = gdn::launch_copy_rows(h0, st_in, base + pp.h0_off, st_pad, blocks, s);
    if (e != hipSuccess) return hip_fail(e, "padding copy launch");
    float* hT_pad = hT ? reinterpret_cast<float*>(base + pp.hT_off) : nullptr;
    const float* h0_pad = h0 ? reinterpret_cast<const float*>(base + pp.h0_off) : nullptr;
    gdn_status st = cu_seqlens ? run_varlen(padded_problem(p), pp.rec, cu_seqlens, base + pp.q_off, base + pp.k_off,
                                            v, g, beta, h0_pad, o, hT_pad, ws, s)
                               : run_fwd(padded_problem(p), pp.rec, base + pp.q_off, base + pp.k_off, v, g, beta,
                                         h0_pad, o, hT_pad, ws, s);
    if (st != GDN_OK || !hT) return st;
    e = gdn::launch_copy_rows(hT_pad, st_pad, hT, st_in, blocks, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "final-state copy launch");
}

// The packed-sequence forward on a checked problem with a workspace of at least pl.bytes.
gdn_status run_varlen(const gdn_problem& p, const Plan& pl, const int32_t* cu_seqlens, const void* q, const void* k,
                      const void* v, const float* g, const float* beta, const float* h0, void* o, float* hT, void* ws,
                      hipStream_t s) {
    if (p.B == 0) return GDN_OK;
    const gdn::Workspace w = carve(pl, ws);
    if (p.T > 0) {
        gdn_status st = run_prep(p, pl, q, k, g, beta, w, s, nullptr, cu_seqlens);
        if (st != GDN_OK) return st;
    }
    gdn::StateArgs a = state_args(p, pl, q, k, v, w);
    a.cu_seqlens = cu_seqlens;
    a.init_mode = h0 ? gdn::kInitLoad : gdn::kInitZero;
    a.s_init = h0;
    a.o = o;
    a.s_out = hT;
    a.store_mode = hT ? gdn::kStoreLastSegment : gdn::kStoreNone;
    return run_state(p, a, s);
}

// Chunk records of gdn_chunk_fwd_noalloc: a static device array, one copy per GPU that
// loads the library, held until the process ends. Nothing in it has to start at zero:
// the prepare pass writes every record the state pass reads. In host code the array's
// name is not its device address; the address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

gdn_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(GDN_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256)
            return fail(GDN_EHIP, "static scratch has no 256-byte aligned device address");
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_EINVAL: return "GDN_EINVAL: invalid argument";
        case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED: unsupported shape, dtype or option";
        case GDN_EWORKSPACE: return "GDN_EWORKSPACE: workspace missing, misaligned or too small";
        case GDN_EHIP: return "GDN_EHIP: HIP runtime error";
    }
    return "unknown gdn_status";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

const char* gdn_kernel_path(const gdn_problem* p) {
    if (check_problem(p) != GDN_OK) return nullptr;
    // (fp32 inputs: the fp32 prepare and state kernels dispatch to their matrix-core
    // versions by dk)
    if (p->io_dtype == GDN_BF16) return p->dk == 128 ? "bf16-mfma" : "bf16-mfma-padded";
    return p->dk == 128 ? "f32-mfma" : "f32-mfma-padded";
}

gdn_status gdn_chunk_fwd_workspace(const gdn_problem* p, size_t* bytes) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_EINVAL, "bytes pointer is NULL");
    if (use_mfma_padded(*p)) {
        const gdn_problem w = padded_problem(*p);
        st = check_problem(&w);
        if (st != GDN_OK) return st;
        *bytes = make_pad_plan(*p).bytes;
        return GDN_OK;
    }
    *bytes = make_plan(*p, false).bytes;
    return GDN_OK;
}

gdn_status gdn_chunk_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* h0, void* o, float* hT,
                         void* ws, size_t ws_bytes, void* stream) {
    try {
        gdn_status st = check_fwd_args(p, q, k, v, g, beta, o);
        if (st != GDN_OK) return st;
        if (use_mfma_padded(*p)) {
            const gdn_problem w = padded_problem(*p);
            st = check_problem(&w);
            if (st != GDN_OK) return st;
            const PadPlan pp = make_pad_plan(*p);
            Plan need;
            need.bytes = pp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            return run_fwd_padded(*p, pp, nullptr, q, k, v, g, beta, h0, o, hT, ws, static_cast<hipStream_t>(stream));
        }
        const Plan pl = make_plan(*p, false);
        st = check_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        return run_fwd(*p, pl, q, k, v, g, beta, h0, o, hT, ws, static_cast<hipStream_t>(stream));
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* h0, void* o, float* hT,
                                 void* stream) {
    try {
        gdn_status st = check_fwd_args(p, q, k, v, g, beta, o);
        if (st != GDN_OK) return st;
        // heads under 128: the padded q, k and state blocks share the array with the records
        const bool padded = use_mfma_padded(*p);
        if (padded) {
            const gdn_problem w = padded_problem(*p);
            st = check_problem(&w);
            if (st != GDN_OK) return st;
        }
        const PadPlan pp = padded ? make_pad_plan(*p) : PadPlan{};
        const Plan pl = padded ? pp.rec : make_plan(*p, false);
        const size_t need = padded ? pp.bytes : pl.bytes;
        if (need > kScratchBytes)
            return fail(GDN_EWORKSPACE,
                        "the problem needs %zu bytes of chunk records; the static scratch holds %zu "
                        "(use gdn_chunk_fwd with a workspace)", need, kScratchBytes);
        if (p->B == 0) return GDN_OK;
        void* ws = nullptr;
        st = scratch_on_current_device(&ws);
        if (st != GDN_OK) return st;
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (padded) return run_fwd_padded(*p, pp, nullptr, q, k, v, g, beta, h0, o, hT, ws, s);
        return run_fwd(*p, pl, q, k, v, g, beta, h0, o, hT, ws, s);
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_chunk_fwd_prologue(const gdn_problem* p, const void* q_raw, const void* k_raw, const void* v,
                                  const float* a, const float* b, const float* A_log, const float* dt_bias,
                                  float q_scale, const float* h0, void* o, float* hT, void* ws,
                                  size_t ws_bytes, void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        if (!use_mfma(*p))
            return fail(GDN_EUNSUPPORTED, "the fused prologue runs on the bf16 matrix-core path only "
                                          "(io_dtype GDN_BF16, dk = 128)");
        if (!(q_scale == q_scale) || q_scale - q_scale != 0.f)
            return fail(GDN_EINVAL, "q_scale must be finite");
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!q_raw || !k_raw || !v || !a || !b || !A_log || !dt_bias || !o))
            return fail(GDN_EINVAL, "q_raw, k_raw, v, a, b, A_log, dt_bias and o must be non-NULL");
        if (tokens && !aligned16({q_raw, k_raw, v, o}))
            return fail(GDN_EINVAL, "q_raw, k_raw, v and o must be 16-byte aligned");
        const Plan pl = make_plan(*p, false);
        st = check_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (p->B == 0) return GDN_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        const gdn::Workspace w = carve(pl, ws);
        const gdn::Prologue pro{a, b, A_log, dt_bias, q_scale};
        st = run_prep(*p, pl, q_raw, k_raw, nullptr, nullptr, w, s, &pro);
        if (st != GDN_OK) return st;
        gdn::StateArgs sa = state_args(*p, pl, q_raw, k_raw, v, w);
        sa.init_mode = h0 ? gdn::kInitLoad : gdn::kInitZero;
        sa.s_init = h0;
        sa.o = o;
        sa.s_out = hT;
        sa.store_mode = hT ? gdn::kStoreLastSegment : gdn::kStoreNone;
        return run_state(*p, sa, s);
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_chunk_fwd_varlen_workspace(const gdn_problem* p, int32_t max_seqlen, size_t* bytes) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    if (max_seqlen < 0) return fail(GDN_EINVAL, "max_seqlen=%d must be >= 0", max_seqlen);
    if (!bytes) return fail(GDN_EINVAL, "bytes pointer is NULL");
    if (use_mfma_padded(*p)) {
        const gdn_problem w = padded_problem(*p);
        st = check_problem(&w);
        if (st != GDN_OK) return st;
        *bytes = make_pad_plan(*p, max_seqlen, true).bytes;
        return GDN_OK;
    }
    *bytes = make_plan(*p, false, max_seqlen).bytes;
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_varlen(const gdn_problem* p, const int32_t* cu_seqlens, int32_t max_seqlen,
                                const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* h0, void* o, float* hT, void* ws,
                                size_t ws_bytes, void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        if (p->valid_len)
            return fail(GDN_EINVAL, "valid_len must be NULL with cu_seqlens (the lengths come from cu_seqlens)");
        if (max_seqlen < 0) return fail(GDN_EINVAL, "max_seqlen=%d must be >= 0", max_seqlen);
        if (p->B > 0 && !cu_seqlens) return fail(GDN_EINVAL, "cu_seqlens must be non-NULL");
        if (p->T > 0 && (!q || !k || !v || !g || !beta || !o))
            return fail(GDN_EINVAL, "q, k, v, g, beta and o must be non-NULL");
        if (p->T > 0 && !aligned16({q, k, v, o})) return fail(GDN_EINVAL, "q, k, v and o must be 16-byte aligned");
        if (use_mfma_padded(*p)) {
            const gdn_problem w = padded_problem(*p);
            st = check_problem(&w);
            if (st != GDN_OK) return st;
            const PadPlan pp = make_pad_plan(*p, max_seqlen, true);
            Plan need;
            need.bytes = pp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            return run_fwd_padded(*p, pp, cu_seqlens, q, k, v, g, beta, h0, o, hT, ws,
                                  static_cast<hipStream_t>(stream));
        }
        const Plan pl = make_plan(*p, false, max_seqlen);
        st = check_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        return run_varlen(*p, pl, cu_seqlens, q, k, v, g, beta, h0, o, hT, ws, static_cast<hipStream_t>(stream));
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

// Backward workspace: the states before every 8th token, then the per-column-tile
// partials of dq, dk and of dg, dbeta.
struct BwdPlan {
    int64_t NT = 0;
    size_t ckpt_off = 0, dqk_off = 0, dgb_off = 0, bytes = 0;
};

// ncols: the widest state the workspace serves (dv, or max(dv, dk) for the segment
// summaries' backward, whose M pass has dk columns); seg_len: segment length (or T).
BwdPlan make_bwd_plan(const gdn_problem& p, int ncols = -1, int64_t seg_len = -1) {
    BwdPlan pl;
    if (ncols < 0) ncols = p.dv;
    const int64_t L = seg_len < 0 ? p.T : seg_len;
    const int64_t P = L > 0 ? p.T / L : 0;
    pl.NT = (L + gdn::kChunk - 1) / gdn::kChunk;   // chunks per row or segment
    const size_t bt = static_cast<size_t>(p.B) * p.T, tiles = static_cast<size_t>(ncols / 16);
    pl.ckpt_off = 0;
    pl.dqk_off = align256(static_cast<size_t>(p.B) * (P > 0 ? P : 1) * p.H * 8 * pl.NT * p.dk * ncols * sizeof(float));
    pl.dgb_off = pl.dqk_off + align256(bt * p.H * tiles * 2 * p.dk * sizeof(float));
    pl.bytes = pl.dgb_off + align256(bt * p.H * tiles * 2 * sizeof(float));
    return pl;
}

gdn::BwdArgs bwd_args(const gdn_problem& p, const BwdPlan& pl, void* ws) {
    char* base = static_cast<char*>(ws);
    gdn::BwdArgs a;
    a.B = p.B; a.T = p.T; a.H = p.H; a.Hqk = p.Hqk; a.dk = p.dk; a.dv = p.dv;
    a.NT = static_cast<int>(pl.NT);
    a.q = a.k = a.v = a.d_o = nullptr;
    a.g = a.beta = a.h0 = a.dhT = nullptr;
    a.valid_len = p.valid_len;
    a.ckpt = reinterpret_cast<float*>(base + pl.ckpt_off);
    a.dqk_part = reinterpret_cast<float*>(base + pl.dqk_off);
    a.dgb_part = reinterpret_cast<float*>(base + pl.dgb_off);
    a.dq_out = a.dk_out = a.dv_out = a.dg_out = a.dbeta_out = a.dh0_out = nullptr;
    a.P = 1; a.L = p.T;
    a.dhT_per_segment = 0; a.h0_identity = 0; a.v_zero = 0; a.do_zero = 0; a.write_dv = 1; a.accumulate = 0;
    return a;
}

gdn_status check_bwd_ws(const BwdPlan& pl, void* ws, size_t ws_bytes) {
    if (pl.bytes == 0) return GDN_OK;
    if (!ws) return fail(GDN_EWORKSPACE, "workspace is NULL, %zu bytes needed", pl.bytes);
    if (ws_bytes < pl.bytes) return fail(GDN_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, pl.bytes);
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(GDN_EWORKSPACE, "workspace must be 256-byte aligned");
    return GDN_OK;
}

// The chunked matrix-core backward (bf16, dk = dv = 128): the prepare pass's records (That,
// P, decay factors; That^T and P^T; Tinv and P row-major), then the state entering every
// chunk and the gradient of the state leaving it (bf16, transposed).
// The gradient pass reads one batch row of the fp32 dv output with 32-bit byte offsets.
// Rows shorter than one chunk keep the fp32 token-level backward: a few tokens' gradients can
// cancel to a small fraction of their terms, where the bf16-rounded operands of the chunked
// backward leave a large relative error (a one-token row: 3.5e-2 on dk), and such rows cost
// little there. Without tokens there is nothing to compute either way.
constexpr int32_t kMfmaBwdMinT = gdn::kChunk;
bool use_bwd_mfma(const gdn_problem& p) {
    return use_mfma(p) && p.dv == 128 && (p.T == 0 || p.T >= kMfmaBwdMinT) &&
           static_cast<int64_t>(p.T + gdn::kChunk) * p.H * p.dv * 4 < (int64_t(1) << 31);
}

struct BwdMfmaPlan {
    Plan fwd;
    size_t thatT_off = 0, pT_off = 0, trm_off = 0, prm_off = 0, states_off = 0, dstates_off = 0, bytes = 0;
};

BwdMfmaPlan make_bwd_mfma_plan(const gdn_problem& p) {
    BwdMfmaPlan pl;
    pl.fwd = make_plan(p, false);
    const size_t nch = static_cast<size_t>(pl.fwd.nch);
    const size_t tri = align256(nch * gdn::kTriRecordElems * 2), rm = align256(nch * 64 * 64 * 2);
    const size_t st = align256(nch * static_cast<size_t>(p.dk) * p.dv * 2);
    pl.thatT_off = pl.fwd.bytes;
    pl.pT_off = pl.thatT_off + tri;
    pl.trm_off = pl.pT_off + tri;
    pl.prm_off = pl.trm_off + rm;
    pl.states_off = pl.prm_off + rm;
    pl.dstates_off = pl.states_off + st;
    pl.bytes = pl.dstates_off + st;
    return pl;
}

gdn::BwdRecords bwd_records(const BwdMfmaPlan& pl, void* ws) {
    char* base = static_cast<char*>(ws);
    gdn::BwdRecords rec;
    rec.thatT = base + pl.thatT_off;
    rec.pT = base + pl.pT_off;
    rec.t_rm = base + pl.trm_off;
    rec.p_rm = base + pl.prm_off;
    return rec;
}

// The prepare pass with the backward's records (and the forward's P record when the
// forward's outputs are wanted too).
gdn_status run_prep_keep(const gdn_problem& p, const BwdMfmaPlan& pl, const void* q, const void* k, const float* g,
                         const float* beta, bool keep_pmat, void* ws, hipStream_t s) {
    if (pl.fwd.nch == 0) return GDN_OK;
    gdn::PrepArgs pa;
    pa.B = p.B; pa.T = p.T; pa.H = p.H; pa.Hqk = p.Hqk; pa.dk = p.dk; pa.NT = static_cast<int>(pl.fwd.NT);
    pa.q = q; pa.k = k; pa.g = g; pa.beta = beta; pa.valid_len = p.valid_len; pa.cu_seqlens = nullptr;
    pa.ws = carve(pl.fwd, ws);
    pa.qk_stride = static_cast<int64_t>(p.Hqk) * p.dk;
    pa.has_prologue = 0;
    pa.pro = gdn::Prologue{nullptr, nullptr, nullptr, nullptr, 1.f};
    pa.has_conv = 0;
    pa.conv = gdn::PrepConv{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
    pa.bwd = bwd_records(pl, ws);
    pa.bwd.keep_pmat = keep_pmat ? 1 : 0;
    hipError_t e = gdn::launch_prep_mfma(pa, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "prepare kernel launch");
}

// The forward state pass keeping the state entering every chunk, from h0 (init_mode) and
// values v (NULL: zero values); with outputs (o non-NULL) it also writes o and hT.
gdn_status run_state_keep(const gdn_problem& p, const BwdMfmaPlan& pl, const void* q, const void* k, const void* v,
                          int init_mode, const float* h0, void* o, float* hT, void* ws, hipStream_t s) {
    if (pl.fwd.nch == 0) return GDN_OK;
    char* base = static_cast<char*>(ws);
    gdn::StateArgs sa = state_args(p, pl.fwd, q, k, v, carve(pl.fwd, ws));
    sa.pass = o ? gdn::kPassOutputs : gdn::kPassS;
    sa.init_mode = init_mode;
    sa.s_init = h0;
    sa.o = o;
    sa.s_out = hT;
    sa.store_mode = hT ? gdn::kStoreLastSegment : gdn::kStoreNone;
    sa.states = base + pl.states_off;
    return run_state(p, sa, s);
}

// The prepare pass with the backward's records and the forward state pass keeping the state
// entering every chunk; with outputs (o non-NULL) the state pass also writes o and hT.
gdn_status run_fwd_keep(const gdn_problem& p, const BwdMfmaPlan& pl, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* h0, void* o, float* hT, void* ws,
                        hipStream_t s) {
    gdn_status st = run_prep_keep(p, pl, q, k, g, beta, o != nullptr, ws, s);
    if (st != GDN_OK) return st;
    return run_state_keep(p, pl, q, k, v, h0 ? gdn::kInitLoad : gdn::kInitZero, h0, o, hT, ws, s);
}

// The reverse chain and the gradient pass on a workspace that holds the records and states.
// v or d_o NULL: zero values / output gradient; dv NULL: not written; accumulate: the
// gradients are added to what dq, dk, dv, dg and dbeta hold.
gdn_status run_bwd_from_saved(const gdn_problem& p, const BwdMfmaPlan& pl, const void* q, const void* k,
                              const void* v, const float* g, const float* beta, const void* d_o, const float* dhT,
                              float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0, void* ws,
                              hipStream_t s, bool accumulate = false) {
    char* base = static_cast<char*>(ws);
    gdn::BwdMfmaArgs a;
    a.B = p.B; a.T = p.T; a.H = p.H; a.Hqk = p.Hqk; a.NT = static_cast<int>(pl.fwd.NT);
    a.q = q; a.k = k; a.v = v; a.d_o = d_o; a.g = g; a.beta = beta; a.dhT = dhT; a.valid_len = p.valid_len;
    a.ws = carve(pl.fwd, ws); a.rec = bwd_records(pl, ws);
    a.states = base + pl.states_off;
    a.dstates = base + pl.dstates_off;
    a.dq_out = dq; a.dk_out = dk; a.dv_out = dv; a.dg_out = dg; a.dbeta_out = dbeta; a.dh0_out = dh0;
    a.accumulate = accumulate ? 1 : 0;
    hipError_t e = gdn::launch_bwd_state_mfma(a, s);
    if (e != hipSuccess) return hip_fail(e, "backward state kernel launch");
    e = gdn::launch_bwd_grad_mfma(a, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "backward gradient kernel launch");
}

gdn_status run_bwd_mfma(const gdn_problem& p, const BwdMfmaPlan& pl, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* h0, const void* d_o, const float* dhT,
                        float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0, void* ws, hipStream_t s) {
    gdn_status st = run_fwd_keep(p, pl, q, k, v, g, beta, h0, nullptr, nullptr, ws, s);
    if (st != GDN_OK) return st;
    return run_bwd_from_saved(p, pl, q, k, v, g, beta, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, ws, s);
}

// The backward of bf16 problems with dk or dv under 128 on the matrix cores: the chunked
// backward of the problem padded to dk = dv = 128 (q, k, v, d_o zero-padded to 128 columns,
// h0 and dhT to 128 x 128 blocks), whose gradients in the padded columns are cut off. The
// padded columns add exact zeros to every product and sum, so the kept gradients are those
// of the unpadded problem, at the bf16 operand precision of that backward. Rows shorter than
// kPadBwdMinT tokens keep the fp32 token-level backward: it costs little there, and a few
// tokens' gradients can cancel to a small fraction of their terms, where the bf16-rounded
// operands of the chunked backward would leave a large relative error (a one-token row:
// 0.27 on dk, whose norm was 4e-4 of dq's).
constexpr int32_t kPadBwdMinT = 256;
gdn_problem padded_bwd_problem(const gdn_problem& p) {
    gdn_problem w = p;
    w.dk = 128;
    w.dv = 128;
    return w;
}
bool use_bwd_mfma_padded(const gdn_problem& p) {
    return p.io_dtype == GDN_BF16 && (p.dk < 128 || p.dv < 128) && p.T >= kPadBwdMinT &&
           use_bwd_mfma(padded_bwd_problem(p));
}

struct BwdPadPlan {
    BwdMfmaPlan bwd;
    size_t q_off = 0, k_off = 0, v_off = 0, do_off = 0, h0_off = 0, dhT_off = 0, dh0_off = 0;
    size_t dq_off = 0, dk_off = 0, dv_off = 0, bytes = 0;
};

BwdPadPlan make_bwd_pad_plan(const gdn_problem& p) {
    BwdPadPlan pp;
    pp.bwd = make_bwd_mfma_plan(padded_bwd_problem(p));
    const size_t tq = static_cast<size_t>(p.B) * p.T * p.Hqk, tv = static_cast<size_t>(p.B) * p.T * p.H;
    const size_t st = align256(static_cast<size_t>(p.B) * p.H * 128 * 128 * 4);
    size_t off = align256(pp.bwd.bytes);
    pp.q_off = off; off += align256(tq * 256);
    pp.k_off = off; off += align256(tq * 256);
    pp.v_off = off; off += align256(tv * 256);
    pp.do_off = off; off += align256(tv * 256);
    pp.h0_off = off; off += st;
    pp.dhT_off = off; off += st;
    pp.dh0_off = off; off += st;
    pp.dq_off = off; off += align256(tq * 512);
    pp.dk_off = off; off += align256(tq * 512);
    pp.dv_off = off; off += align256(tv * 512);
    pp.bytes = off;
    return pp;
}

// The kept forward of a padded problem: q, k, v and h0 padded into the workspace (where the
// backward from it reads them), the dk = dv = 128 forward that keeps its records and states,
// o and the final state cut back. The padded o and final state pass through the slots of the
// padded d_o and dhT, which the forward does not use.
gdn_status run_fwd_save_padded(const gdn_problem& p, const BwdPadPlan& pp, const void* q, const void* k,
                               const void* v, const float* g, const float* beta, const float* h0, void* o, float* hT,
                               void* ws, hipStream_t s) {
    char* base = static_cast<char*>(ws);
    const int64_t tq = static_cast<int64_t>(p.B) * p.T * p.Hqk, tv = static_cast<int64_t>(p.B) * p.T * p.H;
    const int64_t nbh = static_cast<int64_t>(p.B) * p.H, vf = p.dv * 4;
    hipError_t e = gdn::launch_copy_rows(q, p.dk * 2, base + pp.q_off, 256, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(k, p.dk * 2, base + pp.k_off, 256, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(v, p.dv * 2, base + pp.v_off, 256, tv, s);
    if (e == hipSuccess && h0) e = gdn::launch_copy_blocks(h0, p.dk, vf, base + pp.h0_off, 128, 512, nbh, s);
    if (e != hipSuccess) return hip_fail(e, "padding copy launch");
    const gdn_problem w = padded_bwd_problem(p);
    float* hT_p = hT ? reinterpret_cast<float*>(base + pp.dhT_off) : nullptr;
    const float* h0_p = h0 ? reinterpret_cast<const float*>(base + pp.h0_off) : nullptr;
    gdn_status st = run_fwd_keep(w, pp.bwd, base + pp.q_off, base + pp.k_off, base + pp.v_off, g, beta, h0_p,
                                 base + pp.do_off, hT_p, ws, s);
    if (st != GDN_OK) return st;
    e = gdn::launch_copy_rows(base + pp.do_off, 256, o, p.dv * 2, tv, s);
    if (e == hipSuccess && hT) e = gdn::launch_copy_blocks(hT_p, 128, 512, hT, p.dk, vf, nbh, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "output copy launch");
}

// The backward from a padded kept forward: d_o and dhT padded, the backward from the kept
// records and states on the padded q, k, v the forward left in the workspace, the gradients
// cut back.
gdn_status run_bwd_saved_padded(const gdn_problem& p, const BwdPadPlan& pp, const float* g, const float* beta,
                                const void* d_o, const float* dhT, float* dq, float* dk, float* dv, float* dg,
                                float* dbeta, float* dh0, void* ws, hipStream_t s) {
    char* base = static_cast<char*>(ws);
    const int64_t tq = static_cast<int64_t>(p.B) * p.T * p.Hqk, tv = static_cast<int64_t>(p.B) * p.T * p.H;
    const int64_t nbh = static_cast<int64_t>(p.B) * p.H, kf = p.dk * 4, vf = p.dv * 4;
    hipError_t e = gdn::launch_copy_rows(d_o, p.dv * 2, base + pp.do_off, 256, tv, s);
    if (e == hipSuccess && dhT) e = gdn::launch_copy_blocks(dhT, p.dk, vf, base + pp.dhT_off, 128, 512, nbh, s);
    if (e != hipSuccess) return hip_fail(e, "padding copy launch");
    float* dq_p = reinterpret_cast<float*>(base + pp.dq_off);
    float* dk_p = reinterpret_cast<float*>(base + pp.dk_off);
    float* dv_p = reinterpret_cast<float*>(base + pp.dv_off);
    float* dh0_p = dh0 ? reinterpret_cast<float*>(base + pp.dh0_off) : nullptr;
    gdn_status st = run_bwd_from_saved(padded_bwd_problem(p), pp.bwd, base + pp.q_off, base + pp.k_off,
                                       base + pp.v_off, g, beta, base + pp.do_off,
                                       dhT ? reinterpret_cast<const float*>(base + pp.dhT_off) : nullptr, dq_p, dk_p,
                                       dv_p, dg, dbeta, dh0_p, ws, s);
    if (st != GDN_OK) return st;
    e = gdn::launch_copy_rows(dq_p, 512, dq, kf, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(dk_p, 512, dk, kf, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(dv_p, 512, dv, vf, tv, s);
    if (e == hipSuccess && dh0) e = gdn::launch_copy_blocks(dh0_p, 128, 512, dh0, p.dk, vf, nbh, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "gradient copy launch");
}

gdn_status run_bwd_padded(const gdn_problem& p, const BwdPadPlan& pp, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const float* h0, const void* d_o, const float* dhT,
                          float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0, void* ws,
                          hipStream_t s) {
    if (p.B == 0) return GDN_OK;
    char* base = static_cast<char*>(ws);
    const int64_t tq = static_cast<int64_t>(p.B) * p.T * p.Hqk, tv = static_cast<int64_t>(p.B) * p.T * p.H;
    const int64_t nbh = static_cast<int64_t>(p.B) * p.H;
    const int64_t kb = p.dk * 2, vb = p.dv * 2, kf = p.dk * 4, vf = p.dv * 4;
    hipError_t e = gdn::launch_copy_rows(q, kb, base + pp.q_off, 256, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(k, kb, base + pp.k_off, 256, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(v, vb, base + pp.v_off, 256, tv, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(d_o, vb, base + pp.do_off, 256, tv, s);
    if (e == hipSuccess && h0) e = gdn::launch_copy_blocks(h0, p.dk, vf, base + pp.h0_off, 128, 512, nbh, s);
    if (e == hipSuccess && dhT) e = gdn::launch_copy_blocks(dhT, p.dk, vf, base + pp.dhT_off, 128, 512, nbh, s);
    if (e != hipSuccess) return hip_fail(e, "padding copy launch");
    float* dq_p = reinterpret_cast<float*>(base + pp.dq_off);
    float* dk_p = reinterpret_cast<float*>(base + pp.dk_off);
    float* dv_p = reinterpret_cast<float*>(base + pp.dv_off);
    float* dh0_p = dh0 ? reinterpret_cast<float*>(base + pp.dh0_off) : nullptr;
    gdn_status st = run_bwd_mfma(padded_bwd_problem(p), pp.bwd, base + pp.q_off, base + pp.k_off, base + pp.v_off, g,
                                 beta, h0 ? reinterpret_cast<const float*>(base + pp.h0_off) : nullptr,
                                 base + pp.do_off, dhT ? reinterpret_cast<const float*>(base + pp.dhT_off) : nullptr,
                                 dq_p, dk_p, dv_p, dg, dbeta, dh0_p, ws, s);
    if (st != GDN_OK) return st;
    e = gdn::launch_copy_rows(dq_p, 512, dq, kf, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(dk_p, 512, dk, kf, tq, s);
    if (e == hipSuccess) e = gdn::launch_copy_rows(dv_p, 512, dv, vf, tv, s);
    if (e == hipSuccess && dh0) e = gdn::launch_copy_blocks(dh0_p, 128, 512, dh0, p.dk, vf, nbh, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "gradient copy launch");
}

// The backward through the segment calls on the matrix cores: the P segments of each of the
// B rows run as B * P rows of their own (the token-major tensors [B, T, ...] are
// [B * P, L, ...] as they lie), each from its own incoming state; the state blocks move
// between the segment calls' [B, H, P, D, D] and the rows' [B * P, H, D, D] layouts in the
// workspace, behind the chunked backward's own records.
struct SegBwdMfmaPlan {
    gdn_problem rows;
    BwdMfmaPlan bwd;
    size_t h0_off = 0, dhT_off = 0, dh0_off = 0, vl_off = 0, bytes = 0;
};

SegBwdMfmaPlan make_seg_bwd_mfma_plan(const gdn_problem& p, int64_t P, int32_t L) {
    SegBwdMfmaPlan sp;
    sp.rows = p;
    sp.rows.B = static_cast<int32_t>(p.B * P);
    sp.rows.T = L;
    sp.rows.valid_len = nullptr;
    sp.bwd = make_bwd_mfma_plan(sp.rows);
    const size_t blocks = align256(static_cast<size_t>(p.B) * P * p.H * p.dk * p.dv * 4);
    sp.h0_off = align256(sp.bwd.bytes);
    sp.dhT_off = sp.h0_off + blocks;
    sp.dh0_off = sp.dhT_off + blocks;
    sp.vl_off = sp.dh0_off + blocks;
    sp.bytes = sp.vl_off + align256(static_cast<size_t>(p.B) * P * 4);
    return sp;
}

bool use_seg_bwd_mfma(const gdn_problem& p, int64_t P, int32_t L) {
    if (!use_bwd_mfma(p) || P == 0 || p.B * P > 65535) return false;
    gdn_problem rows = p;
    rows.B = static_cast<int32_t>(p.B * P);
    rows.T = L;
    return use_bwd_mfma(rows);
}

// The rows' problem with their valid tokens (from the padded rows' valid_len) in ws.
gdn_problem seg_rows(const SegBwdMfmaPlan& sp, const gdn_problem& p, int64_t P, int32_t L, void* ws, hipStream_t s,
                     hipError_t* e) {
    gdn_problem rows = sp.rows;
    *e = hipSuccess;
    if (p.valid_len) {
        int32_t* vl = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + sp.vl_off);
        *e = gdn::launch_seg_valid_len(p.valid_len, p.B, static_cast<int>(P), L, p.T, vl, s);
        rows.valid_len = vl;
    }
    return rows;
}

hipError_t seg_blocks(const gdn_problem& p, int64_t P, const float* src, float* dst, bool to_rows, bool last_only,
                      hipStream_t s) {
    gdn::SegBlocksArgs a{p.B, p.H, static_cast<int>(P), p.dk, src, dst, to_rows ? 1 : 0, last_only ? 1 : 0};
    return gdn::launch_seg_state_blocks(a, s);
}

gdn_status gdn_chunk_bwd_workspace(const gdn_problem* p, size_t* bytes) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_EINVAL, "bytes pointer is NULL");
    *bytes = use_bwd_mfma(*p) ? make_bwd_mfma_plan(*p).bytes
                              : (use_bwd_mfma_padded(*p) ? make_bwd_pad_plan(*p).bytes : make_bwd_plan(*p).bytes);
    return GDN_OK;
}

gdn_status gdn_chunk_bwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* h0, const void* d_o, const float* dhT, float* dq,
                         float* dk, float* dv, float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes,
                         void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
            return fail(GDN_EINVAL, "q, k, v, g, beta, d_o, dq, dk, dv, dg and dbeta must be non-NULL");
        if (tokens && !aligned16({q, k, v, d_o, dq, dk, dv}))
            return fail(GDN_EINVAL, "q, k, v, d_o, dq, dk and dv must be 16-byte aligned");
        if (use_bwd_mfma(*p)) {
            const BwdMfmaPlan pl = make_bwd_mfma_plan(*p);
            Plan need;
            need.bytes = pl.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            if (p->B == 0) return GDN_OK;
            return run_bwd_mfma(*p, pl, q, k, v, g, beta, h0, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, ws,
                                static_cast<hipStream_t>(stream));
        }
        if (use_bwd_mfma_padded(*p)) {
            const BwdPadPlan pp = make_bwd_pad_plan(*p);
            Plan need;
            need.bytes = pp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            return run_bwd_padded(*p, pp, q, k, v, g, beta, h0, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, ws,
                                  static_cast<hipStream_t>(stream));
        }
        const BwdPlan pl = make_bwd_plan(*p);
        st = check_bwd_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (p->B == 0) return GDN_OK;
        gdn::BwdArgs a = bwd_args(*p, pl, ws);
        a.q = q; a.k = k; a.v = v; a.d_o = d_o; a.g = g; a.beta = beta; a.h0 = h0; a.dhT = dhT;
        a.dq_out = dq; a.dk_out = dk; a.dv_out = dv; a.dg_out = dg; a.dbeta_out = dbeta; a.dh0_out = dh0;
        hipError_t e = gdn::launch_bwd(a, p->io_dtype == GDN_BF16, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? GDN_OK : hip_fail(e, "backward kernel launch");
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_chunk_fwd_save_workspace(const gdn_problem* p, size_t* bytes) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_EINVAL, "bytes pointer is NULL");
    if (use_bwd_mfma_padded(*p)) {
        *bytes = make_bwd_pad_plan(*p).bytes;
        return GDN_OK;
    }
    if (!use_bwd_mfma(*p))
        return fail(GDN_EUNSUPPORTED, "keeping the forward for the backward needs the chunked matrix-core backward's "
                                      "problems (bf16 inputs, dk = dv = 128, or narrower heads on rows of 256 tokens or more)");
    *bytes = make_bwd_mfma_plan(*p).bytes;
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_save(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* h0, void* o, float* hT, void* ws, size_t ws_bytes,
                              void* stream) {
    try {
        gdn_status st = check_fwd_args(p, q, k, v, g, beta, o);
        if (st != GDN_OK) return st;
        if (use_bwd_mfma_padded(*p)) {
            const BwdPadPlan pp = make_bwd_pad_plan(*p);
            Plan need;
            need.bytes = pp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            if (p->B == 0) return GDN_OK;
            return run_fwd_save_padded(*p, pp, q, k, v, g, beta, h0, o, hT, ws, static_cast<hipStream_t>(stream));
        }
        if (!use_bwd_mfma(*p))
            return fail(GDN_EUNSUPPORTED, "keeping the forward for the backward needs the chunked matrix-core backward's "
                                          "problems (bf16 inputs, dk = dv = 128, or narrower heads on rows of 256 tokens or more)");
        const BwdMfmaPlan pl = make_bwd_mfma_plan(*p);
        Plan need;
        need.bytes = pl.bytes;
        st = check_ws(need, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (p->B == 0) return GDN_OK;
        const hipStream_t s = static_cast<hipStream_t>(stream);
        // no chunks: the plain forward (hT = h0, or zero) keeps nothing
        if (pl.fwd.nch == 0) return run_fwd(*p, pl.fwd, q, k, v, g, beta, h0, o, hT, ws, s);
        return run_fwd_keep(*p, pl, q, k, v, g, beta, h0, o, hT, ws, s);
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_chunk_bwd_saved(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const void* d_o, const float* dhT, float* dq, float* dk,
                               float* dv, float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes,
                               void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
            return fail(GDN_EINVAL, "q, k, v, g, beta, d_o, dq, dk, dv, dg and dbeta must be non-NULL");
        if (tokens && !aligned16({q, k, v, d_o, dq, dk, dv}))
            return fail(GDN_EINVAL, "q, k, v, d_o, dq, dk and dv must be 16-byte aligned");
        if (use_bwd_mfma_padded(*p)) {
            const BwdPadPlan pp = make_bwd_pad_plan(*p);
            Plan need;
            need.bytes = pp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            if (p->B == 0) return GDN_OK;
            return run_bwd_saved_padded(*p, pp, g, beta, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, ws,
                                        static_cast<hipStream_t>(stream));
        }
        if (!use_bwd_mfma(*p))
            return fail(GDN_EUNSUPPORTED, "the backward from a kept forward needs the chunked matrix-core backward's "
                                          "problems (bf16 inputs, dk = dv = 128, or narrower heads on rows of 256 tokens or more)");
        const BwdMfmaPlan pl = make_bwd_mfma_plan(*p);
        Plan need;
        need.bytes = pl.bytes;
        st = check_ws(need, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (p->B == 0) return GDN_OK;
        return run_bwd_from_saved(*p, pl, q, k, v, g, beta, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, ws,
                                  static_cast<hipStream_t>(stream));
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_segment_bwd_workspace(const gdn_problem* p, int32_t seg_len, size_t* bytes) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    int64_t P = 0;
    st = check_segments(*p, seg_len, &P);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_EINVAL, "bytes pointer is NULL");
    *bytes = use_seg_bwd_mfma(*p, P, seg_len) ? make_seg_bwd_mfma_plan(*p, P, seg_len).bytes
                                              : make_bwd_plan(*p, p->dv > p->dk ? p->dv : p->dk, seg_len).bytes;
    return GDN_OK;
}

gdn_status gdn_apply_initial_state_bwd(const gdn_problem* p, int32_t seg_len, const void* q, const void* k,
                                       const void* v, const float* g, const float* beta, const float* H_in,
                                       const void* d_o, const float* dhT, float* dq, float* dk, float* dv,
                                       float* dg, float* dbeta, float* dH_in, void* ws, size_t ws_bytes,
                                       void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        int64_t P = 0;
        st = check_segments(*p, seg_len, &P);
        if (st != GDN_OK) return st;
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!q || !k || !v || !g || !beta || !H_in || !d_o || !dq || !dk || !dv || !dg || !dbeta))
            return fail(GDN_EINVAL, "q, k, v, g, beta, H_in, d_o, dq, dk, dv, dg and dbeta must be non-NULL");
        if (tokens && !aligned16({q, k, v, d_o, dq, dk, dv}))
            return fail(GDN_EINVAL, "q, k, v, d_o, dq, dk and dv must be 16-byte aligned");
        if (use_seg_bwd_mfma(*p, P, seg_len)) {
            // every segment as a row of its own, from its incoming state, through the chunked
            // matrix-core backward; the final-state gradient enters the last segment of a row
            const SegBwdMfmaPlan sp = make_seg_bwd_mfma_plan(*p, P, seg_len);
            Plan need;
            need.bytes = sp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            if (!tokens) return GDN_OK;
            hipStream_t s = static_cast<hipStream_t>(stream);
            char* base = static_cast<char*>(ws);
            float* h0r = reinterpret_cast<float*>(base + sp.h0_off);
            float* dhTr = reinterpret_cast<float*>(base + sp.dhT_off);
            float* dh0r = reinterpret_cast<float*>(base + sp.dh0_off);
            hipError_t e;
            const gdn_problem rows = seg_rows(sp, *p, P, seg_len, ws, s, &e);
            if (e == hipSuccess) e = seg_blocks(*p, P, H_in, h0r, true, false, s);
            if (e == hipSuccess) e = seg_blocks(*p, P, dhT, dhTr, true, true, s);
            if (e != hipSuccess) return hip_fail(e, "segment state layout kernel launch");
            st = run_bwd_mfma(rows, sp.bwd, q, k, v, g, beta, h0r, d_o, dhTr, dq, dk, dv, dg, dbeta,
                              dH_in ? dh0r : nullptr, ws, s);
            if (st != GDN_OK || !dH_in) return st;
            e = seg_blocks(*p, P, dh0r, dH_in, false, false, s);
            return e == hipSuccess ? GDN_OK : hip_fail(e, "segment state layout kernel launch");
        }
        const BwdPlan pl = make_bwd_plan(*p, p->dv > p->dk ? p->dv : p->dk, seg_len);
        st = check_bwd_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (!tokens) return GDN_OK;
        gdn::BwdArgs a = bwd_args(*p, pl, ws);
        a.P = static_cast<int>(P); a.L = seg_len;
        a.q = q; a.k = k; a.v = v; a.d_o = d_o; a.g = g; a.beta = beta; a.h0 = H_in; a.dhT = dhT;
        a.dq_out = dq; a.dk_out = dk; a.dv_out = dv; a.dg_out = dg; a.dbeta_out = dbeta; a.dh0_out = dH_in;
        hipError_t e = gdn::launch_bwd(a, p->io_dtype == GDN_BF16, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? GDN_OK : hip_fail(e, "apply backward kernel launch");
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_summary_combine_bwd(int32_t B, int32_t H, int32_t P, int32_t dk, int32_t dv, const float* M,
                                   const float* H_in, const float* dH_in, const float* dhT, float* dM, float* dS,
                                   float* dh0, void* stream) {
    try {
        if (B < 0 || H < 0 || P < 0) return fail(GDN_EINVAL, "B, H and P must be >= 0");
        if (!head_dim_ok(dk) || !head_dim_ok(dv))
            return fail(GDN_EUNSUPPORTED, "dk=%d, dv=%d: head dims must be 16, 32, 64 or 128", dk, dv);
        if (B > 65535 || H > 65535) return fail(GDN_EUNSUPPORTED, "B or H exceeds 65535");
        const bool work = static_cast<int64_t>(B) * H > 0;
        if (work && P > 0 && (!M || !H_in || !dH_in || !dM || !dS))
            return fail(GDN_EINVAL, "M, H_in, dH_in, dM and dS must be non-NULL");
        if (!work) return GDN_OK;
        gdn::ScanBwdArgs a{B, H, P, dk, dv, M, H_in, dH_in, dhT, dM, dS, dh0};
        hipError_t e = gdn::launch_scan_bwd(a, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? GDN_OK : hip_fail(e, "combine backward kernel launch");
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_segment_summary_bwd(const gdn_problem* p, int32_t seg_len, const void* q, const void* k,
                                   const void* v, const float* g, const float* beta, const float* dM,
                                   const float* dS, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                                   int32_t accumulate, void* ws, size_t ws_bytes, void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        int64_t P = 0;
        st = check_segments(*p, seg_len, &P);
        if (st != GDN_OK) return st;
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!q || !k || !v || !g || !beta || !dq || !dk || !dv || !dg || !dbeta))
            return fail(GDN_EINVAL, "q, k, v, g, beta, dq, dk, dv, dg and dbeta must be non-NULL");
        if (tokens && !aligned16({q, k, v, dq, dk, dv}))
            return fail(GDN_EINVAL, "q, k, v, dq, dk and dv must be 16-byte aligned");
        if (use_seg_bwd_mfma(*p, P, seg_len)) {
            // every segment as a row of its own through the chunked matrix-core backward, the
            // chunk records prepared once: S from a zero state with values, M from the
            // identity without values (its value gradient dropped), neither with outputs
            const SegBwdMfmaPlan sp = make_seg_bwd_mfma_plan(*p, P, seg_len);
            Plan need;
            need.bytes = sp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            if (!tokens) return GDN_OK;
            hipStream_t s = static_cast<hipStream_t>(stream);
            float* dhTr = reinterpret_cast<float*>(static_cast<char*>(ws) + sp.dhT_off);
            hipError_t e;
            const gdn_problem rows = seg_rows(sp, *p, P, seg_len, ws, s, &e);
            if (e != hipSuccess) return hip_fail(e, "segment valid-length kernel launch");
            st = run_prep_keep(rows, sp.bwd, q, k, g, beta, false, ws, s);
            if (st != GDN_OK) return st;
            if (dS || !accumulate) {
                e = seg_blocks(*p, P, dS, dhTr, true, false, s);
                if (e != hipSuccess) return hip_fail(e, "segment state layout kernel launch");
                st = run_state_keep(rows, sp.bwd, q, k, v, gdn::kInitZero, nullptr, nullptr, nullptr, ws, s);
                if (st == GDN_OK)
                    st = run_bwd_from_saved(rows, sp.bwd, q, k, v, g, beta, nullptr, dhTr, dq, dk, dv, dg, dbeta, nullptr,
                                            ws, s, accumulate != 0);
                if (st != GDN_OK) return st;
            }
            if (dM) {
                e = seg_blocks(*p, P, dM, dhTr, true, false, s);
                if (e != hipSuccess) return hip_fail(e, "segment state layout kernel launch");
                st = run_state_keep(rows, sp.bwd, q, k, nullptr, gdn::kInitIdentity, nullptr, nullptr, nullptr, ws, s);
                if (st == GDN_OK)
                    st = run_bwd_from_saved(rows, sp.bwd, q, k, nullptr, g, beta, nullptr, dhTr, dq, dk, nullptr, dg, dbeta,
                                            nullptr, ws, s, true);
                if (st != GDN_OK) return st;
            }
            return GDN_OK;
        }
        const BwdPlan pl = make_bwd_plan(*p, p->dv > p->dk ? p->dv : p->dk, seg_len);
        st = check_bwd_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (!tokens) return GDN_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        gdn::BwdArgs a = bwd_args(*p, pl, ws);
        a.P = static_cast<int>(P); a.L = seg_len;
        a.q = q; a.k = k; a.v = v; a.d_o = v; a.g = g; a.beta = beta;
        a.do_zero = 1; a.dhT_per_segment = 1;
        a.dq_out = dq; a.dk_out = dk; a.dv_out = dv; a.dg_out = dg; a.dbeta_out = dbeta;
        // S: the segment's recurrence from a zero state with final-state gradient dS (a NULL
        // dS is a zero gradient; the pass then writes zeros unless accumulating)
        if (dS || !accumulate) {
            a.dhT = dS; a.accumulate = accumulate ? 1 : 0;
            hipError_t e = gdn::launch_bwd(a, p->io_dtype == GDN_BF16, s);
            if (e != hipSuccess) return hip_fail(e, "summary S backward kernel launch");
        }
        // M: the homogeneous recurrence (zero values) from I, final-state gradient dM; M has
        // dk columns and does not depend on v
        if (dM) {
            gdn::BwdArgs m = a;
            m.dv = p->dk; m.v_zero = 1; m.h0_identity = 1; m.write_dv = 0;
            m.dhT = dM;
            m.accumulate = 1;   // onto the S pass's gradients, or the caller's when accumulating
            hipError_t e = gdn::launch_bwd(m, p->io_dtype == GDN_BF16, s);
            if (e != hipSuccess) return hip_fail(e, "summary M backward kernel launch");
        }
        return GDN_OK;
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_causal_conv1d(int32_t B, int32_t T, int32_t C, int32_t K, int32_t io_dtype, const void* x,
                             const float* w, const float* bias, const void* x_prev, int32_t apply_silu, void* y,
                             void* stream) {
    try {
        if (B < 0 || T < 0 || C < 0) return fail(GDN_EINVAL, "B, T and C must be >= 0");
        if (K < 2 || K > 4) return fail(GDN_EUNSUPPORTED, "K=%d: kernel widths 2, 3 and 4 are supported", K);
        if (C % 8) return fail(GDN_EUNSUPPORTED, "C=%d must be a multiple of 8", C);
        if (io_dtype != GDN_F32 && io_dtype != GDN_BF16)
            return fail(GDN_EUNSUPPORTED, "io_dtype=%d: only GDN_F32 and GDN_BF16", io_dtype);
        if (B > 65535) return fail(GDN_EUNSUPPORTED, "B=%d exceeds 65535", B);
        if (T > 65535 * 128) return fail(GDN_EUNSUPPORTED, "T=%d exceeds 65535 runs of 128 tokens", T);
        const int64_t n = static_cast<int64_t>(B) * T * C;
        if (n == 0) return GDN_OK;
        if (!x || !w || !y) return fail(GDN_EINVAL, "x, w and y must be non-NULL");
        const size_t align = io_dtype == GDN_BF16 ? 16 : 32;
        if (reinterpret_cast<uintptr_t>(x) % align || reinterpret_cast<uintptr_t>(y) % align ||
            (x_prev && reinterpret_cast<uintptr_t>(x_prev) % align))
            return fail(GDN_EINVAL, "x, x_prev and y must be %zu-byte aligned", align);
        gdn::ConvArgs a{B, T, C, K, apply_silu ? 1 : 0, x, w, bias, x_prev, y};
        hipError_t e = gdn::launch_causal_conv1d(a, io_dtype == GDN_BF16, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? GDN_OK : hip_fail(e, "conv1d kernel launch");
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t D, int32_t io_dtype, const void* o, const void* z,
                             const float* weight, float eps, void* y, void* stream) {
    try {
        if (rows < 0) return fail(GDN_EINVAL, "rows must be >= 0");
        if (!head_dim_ok(D)) return fail(GDN_EUNSUPPORTED, "D=%d: 16, 32, 64 or 128", D);
        if (io_dtype != GDN_F32 && io_dtype != GDN_BF16)
            return fail(GDN_EUNSUPPORTED, "io_dtype=%d: only GDN_F32 and GDN_BF16", io_dtype);
        if (!(eps >= 0.f) || eps - eps != 0.f) return fail(GDN_EINVAL, "eps must be finite and >= 0");
        if (rows == 0) return GDN_OK;
        if (!o || !z || !weight || !y) return fail(GDN_EINVAL, "o, z, weight and y must be non-NULL");
        const size_t align = io_dtype == GDN_BF16 ? 16 : 32;
        if (reinterpret_cast<uintptr_t>(o) % align || reinterpret_cast<uintptr_t>(z) % align ||
            reinterpret_cast<uintptr_t>(y) % align)
            return fail(GDN_EINVAL, "o, z and y must be %zu-byte aligned", align);
        gdn::NormArgs a{rows, D, eps, o, z, weight, y};
        hipError_t e = gdn::launch_gated_rmsnorm(a, io_dtype == GDN_BF16, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? GDN_OK : hip_fail(e, "gated rmsnorm kernel launch");
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_chunk_fwd_prologue_qkv(const gdn_problem* p, const void* qkv, const float* a, const float* b,
                                      const float* A_log, const float* dt_bias, float q_scale, const float* h0,
                                      void* o, float* hT, void* ws, size_t ws_bytes, void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        if (!use_mfma(*p))
            return fail(GDN_EUNSUPPORTED, "the fused prologue runs on the bf16 matrix-core path only "
                                          "(io_dtype GDN_BF16, dk = 128)");
        if (!(q_scale == q_scale) || q_scale - q_scale != 0.f)
            return fail(GDN_EINVAL, "q_scale must be finite");
        const int64_t C = 2 * static_cast<int64_t>(p->Hqk) * p->dk + static_cast<int64_t>(p->H) * p->dv;
        if ((static_cast<int64_t>(p->T) + gdn::kChunk) * C * 2 >= (int64_t(1) << 31))
            return fail(GDN_EUNSUPPORTED, "one batch row of qkv exceeds 2 GiB on the bf16 path");
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!qkv || !a || !b || !A_log || !dt_bias || !o))
            return fail(GDN_EINVAL, "qkv, a, b, A_log, dt_bias and o must be non-NULL");
        if (reinterpret_cast<uintptr_t>(qkv) % 16) return fail(GDN_EINVAL, "qkv must be 16-byte aligned");
        const Plan pl = make_plan(*p, false);
        st = check_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (p->B == 0) return GDN_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        const gdn::Workspace w = carve(pl, ws);
        const uint16_t* base = static_cast<const uint16_t*>(qkv);
        const void* q = base;
        const void* k = base + static_cast<int64_t>(p->Hqk) * p->dk;
        const void* v = base + 2 * static_cast<int64_t>(p->Hqk) * p->dk;
        const gdn::Prologue pro{a, b, A_log, dt_bias, q_scale};
        if (pl.nch > 0) {
            gdn::PrepArgs pa;
            pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.Hqk = p->Hqk; pa.dk = p->dk;
            pa.NT = static_cast<int>(pl.NT);
            pa.q = q; pa.k = k; pa.g = nullptr; pa.beta = nullptr; pa.valid_len = p->valid_len;
            pa.cu_seqlens = nullptr; pa.qk_stride = C; pa.ws = w; pa.has_prologue = 1; pa.pro = pro;
            pa.has_conv = 0; pa.conv = gdn::PrepConv{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
            const hipError_t e = gdn::launch_prep_mfma(pa, s);
            if (e != hipSuccess) return hip_fail(e, "prepare kernel launch");
        }
        gdn::StateArgs sa = state_args(*p, pl, q, k, v, w);
        sa.qk_stride = C;
        sa.v_stride = C;
        sa.init_mode = h0 ? gdn::kInitLoad : gdn::kInitZero;
        sa.s_init = h0;
        sa.o = o;
        sa.s_out = hT;
        sa.store_mode = hT ? gdn::kStoreLastSegment : gdn::kStoreNone;
        return run_state(*p, sa, s);
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_chunk_fwd_conv(const gdn_problem* p, const void* x, const float* conv_w, const float* conv_b,
                              const void* x_prev, int32_t conv_k, const float* a, const float* b,
                              const float* A_log, const float* dt_bias, float q_scale, const float* h0, void* y,
                              void* o, float* hT, void* ws, size_t ws_bytes, void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        if (!use_mfma(*p) || p->dv != 128)
            return fail(GDN_EUNSUPPORTED, "the fused Conv1D runs on the bf16 matrix-core path with dk = dv = 128 only");
        if (conv_k < 2 || conv_k > 4) return fail(GDN_EUNSUPPORTED, "conv_k=%d: kernel widths 2, 3 and 4", conv_k);
        if (!(q_scale == q_scale) || q_scale - q_scale != 0.f) return fail(GDN_EINVAL, "q_scale must be finite");
        const int64_t C = 2 * static_cast<int64_t>(p->Hqk) * p->dk + static_cast<int64_t>(p->H) * p->dv;
        if ((static_cast<int64_t>(p->T) + gdn::kChunk) * C * 2 >= (int64_t(1) << 31))
            return fail(GDN_EUNSUPPORTED, "one batch row of x exceeds 2 GiB");
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!x || !conv_w || !a || !b || !A_log || !dt_bias || !y || !o))
            return fail(GDN_EINVAL, "x, conv_w, a, b, A_log, dt_bias, y and o must be non-NULL");
        if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 16 ||
            (x_prev && reinterpret_cast<uintptr_t>(x_prev) % 16))
            return fail(GDN_EINVAL, "x, x_prev and y must be 16-byte aligned");
        const Plan pl = make_plan(*p, false);
        st = check_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (p->B == 0) return GDN_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        const gdn::Workspace w = carve(pl, ws);
        const uint16_t* base = static_cast<const uint16_t*>(y);
        const void* q = base;
        const void* k = base + static_cast<int64_t>(p->Hqk) * p->dk;
        const void* v = base + 2 * static_cast<int64_t>(p->Hqk) * p->dk;
        if (pl.nch > 0) {
            gdn::PrepArgs pa;
            pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.Hqk = p->Hqk; pa.dk = p->dk;
            pa.NT = static_cast<int>(pl.NT);
            pa.q = q; pa.k = k; pa.g = nullptr; pa.beta = nullptr; pa.valid_len = p->valid_len;
            pa.cu_seqlens = nullptr; pa.qk_stride = C; pa.ws = w; pa.has_prologue = 1;
            pa.pro = gdn::Prologue{a, b, A_log, dt_bias, q_scale};
            pa.has_conv = 1;
            pa.conv = gdn::PrepConv{static_cast<const uint16_t*>(x), conv_w, conv_b, static_cast<const uint16_t*>(x_prev),
                                    static_cast<uint16_t*>(y), static_cast<int>(C), conv_k};
            const hipError_t e = gdn::launch_prep_mfma(pa, s);
            if (e != hipSuccess) return hip_fail(e, "prepare kernel launch");
        }
        gdn::StateArgs sa = state_args(*p, pl, q, k, v, w);
        sa.qk_stride = C;
        sa.v_stride = C;
        sa.init_mode = h0 ? gdn::kInitLoad : gdn::kInitZero;
        sa.s_init = h0;
        sa.o = o;
        sa.s_out = hT;
        sa.store_mode = hT ? gdn::kStoreLastSegment : gdn::kStoreNone;
        return run_state(*p, sa, s);
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

// The segment calls on heads with dk < 128 run the dk = 128 problem on q and k zero-padded to
// 128 columns, as the padded forward does. A padded segment's transition is block-diagonal
// (the padded state rows only decay and stay apart from the rest), so the first dk rows and
// columns of its M and the first dk rows of its S are the unpadded problem's; H_in enters
// with zero rows below dk, and the final state is cut back. The workspace holds the padded
// problem's segment records (shared by the summary and apply calls, as the plain segment
// workspace is), the padded q and k, and staging for the 128-row M, S / H_in and hT blocks.
struct SegPadPlan {
    Plan rec;
    size_t q_off = 0, k_off = 0, m_off = 0, s_off = 0, h_off = 0, bytes = 0;
};
SegPadPlan make_seg_pad_plan(const gdn_problem& p, int64_t P) {
    SegPadPlan sp;
    sp.rec = make_plan(padded_problem(p), true);
    const size_t qk = align256(static_cast<size_t>(p.B) * p.T * p.Hqk * 128 * io_bytes(p));
    const size_t blocks = static_cast<size_t>(p.B) * p.H * static_cast<size_t>(P);
    sp.q_off = align256(sp.rec.bytes);
    sp.k_off = sp.q_off + qk;
    sp.m_off = sp.k_off + qk;
    sp.s_off = sp.m_off + align256(blocks * 128 * 128 * 4);
    sp.h_off = sp.s_off + align256(blocks * 128 * p.dv * 4);
    sp.bytes = sp.h_off + align256(static_cast<size_t>(p.B) * p.H * 128 * p.dv * 4);
    return sp;
}
// q and k into their padded copies in the workspace
hipError_t pad_qk(const gdn_problem& p, const SegPadPlan& sp, const void* q, const void* k, void* ws,
                  hipStream_t s) {
    char* base = static_cast<char*>(ws);
    const int64_t rows = static_cast<int64_t>(p.B) * p.T * p.Hqk, es = io_bytes(p);
    hipError_t e = gdn::launch_copy_rows(q, p.dk * es, base + sp.q_off, 128 * es, rows, s);
    return e == hipSuccess ? gdn::launch_copy_rows(k, p.dk * es, base + sp.k_off, 128 * es, rows, s) : e;
}

gdn_status gdn_segment_workspace(const gdn_problem* p, int32_t seg_len, size_t* bytes) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    int64_t P = 0;
    st = check_segments(*p, seg_len, &P);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_EINVAL, "bytes pointer is NULL");
    if (use_mfma_padded(*p)) {
        const gdn_problem w = padded_problem(*p);
        st = check_problem(&w);
        if (st != GDN_OK) return st;
        *bytes = make_seg_pad_plan(*p, P).bytes;
        return GDN_OK;
    }
    *bytes = make_plan(*p, true).bytes;
    return GDN_OK;
}

// The segment summaries of a checked problem with a workspace of at least pl.bytes.
gdn_status run_summary(const gdn_problem& pr, const Plan& pl, int64_t P, int32_t seg_len, const void* q,
                       const void* k, const void* v, const float* g, const float* beta, float* M, float* S,
                       void* ws, hipStream_t s) {
    {
        const gdn_problem* p = &pr;
        gdn_status st;
        const gdn::Workspace w = carve(pl, ws);
        st = run_prep(*p, pl, q, k, g, beta, w, s);
        if (st != GDN_OK) return st;
        gdn::StateArgs a = state_args(*p, pl, q, k, v, w);
        a.P = static_cast<int>(P);
        a.Lc = seg_len / gdn::kChunk;
        a.store_mode = gdn::kStoreEverySegment;
        if (S && M && use_mfma(*p) && p->dk == p->dv) {
            // both summaries in one pass: the M and S chains of a column tile share
            // every loaded operand
            a.pass = gdn::kPassMS;
            a.init_mode = gdn::kInitZero;
            a.s_out = S;
            a.m_out = M;
            return run_state(*p, a, s);
        }
        if (S) {
            a.pass = gdn::kPassS;
            a.init_mode = gdn::kInitZero;
            a.s_out = S;
            st = run_state(*p, a, s);
            if (st != GDN_OK) return st;
        }
        if (M) {
            a.pass = gdn::kPassM;
            a.v = nullptr;
            a.ncols = p->dk;
            a.init_mode = gdn::kInitIdentity;
            a.s_out = M;
            st = run_state(*p, a, s);
            if (st != GDN_OK) return st;
        }
        return GDN_OK;
    }
}

gdn_status gdn_segment_summary(const gdn_problem* p, int32_t seg_len, const void* q, const void* k,
                               const void* v, const float* g, const float* beta, float* M, float* S,
                               void* ws, size_t ws_bytes, void* stream) {
    try {
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        int64_t P = 0;
        st = check_segments(*p, seg_len, &P);
        if (st != GDN_OK) return st;
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!q || !k || !g || !beta || (S && !v)))
            return fail(GDN_EINVAL, "q, k, g, beta (and v when S is wanted) must be non-NULL");
        if (tokens && !aligned16({q, k, v})) return fail(GDN_EINVAL, "q, k and v must be 16-byte aligned");
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (use_mfma_padded(*p)) {
            const gdn_problem wp = padded_problem(*p);
            st = check_problem(&wp);
            if (st != GDN_OK) return st;
            const SegPadPlan sp = make_seg_pad_plan(*p, P);
            Plan need;
            need.bytes = sp.bytes;
            st = check_ws(need, ws, ws_bytes);
            if (st != GDN_OK) return st;
            if (!tokens) return GDN_OK;
            hipError_t e = pad_qk(*p, sp, q, k, ws, s);
            if (e != hipSuccess) return hip_fail(e, "padding copy launch");
            char* base = static_cast<char*>(ws);
            float* m_pad = M ? reinterpret_cast<float*>(base + sp.m_off) : nullptr;
            float* s_pad = S ? reinterpret_cast<float*>(base + sp.s_off) : nullptr;
            st = run_summary(wp, sp.rec, P, seg_len, base + sp.q_off, base + sp.k_off, v, g, beta, m_pad, s_pad, ws, s);
            if (st != GDN_OK) return st;
            const int64_t blocks = static_cast<int64_t>(p->B) * p->H * P;
            if (M) e = gdn::launch_copy_blocks(m_pad, 128, 512, M, p->dk, p->dk * 4, blocks, s);
            if (e == hipSuccess && S) e = gdn::launch_copy_blocks(s_pad, 128, p->dv * 4, S, p->dk, p->dv * 4, blocks, s);
            return e == hipSuccess ? GDN_OK : hip_fail(e, "summary copy launch");
        }
        const Plan pl = make_plan(*p, true);
        st = check_ws(pl, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (!tokens) return GDN_OK;
        return run_summary(*p, pl, P, seg_len, q, k, v, g, beta, M, S, ws, s);
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}


gdn_status gdn_summary_combine(int32_t B, int32_t H, int32_t P, int32_t dk, int32_t dv, const float* M,
                               const float* S, const float* h0, float* H_in, float* M_prefix, float* hT,
                               void* stream) {
    try {
        if (B < 0 || H < 0 || P < 0) return fail(GDN_EINVAL, "B, H and P must be >= 0");
        if (!head_dim_ok(dk) || !head_dim_ok(dv))
            return fail(GDN_EUNSUPPORTED, "dk=%d, dv=%d: head dims must be 16, 32, 64 or 128", dk, dv);
        if (B > 65535 || H > 65535) return fail(GDN_EUNSUPPORTED, "B or H exceeds 65535");
        const bool work = static_cast<int64_t>(B) * H > 0;
        if (work && P > 0 && (!M || !S || !H_in))
            return fail(GDN_EINVAL, "M, S and H_in must be non-NULL");
        if (!work) return GDN_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        gdn::ScanArgs a;
        a.B = B; a.H = H; a.P = P; a.dk = dk; a.ncols = dv;
        a.M = M; a.S = S;
        a.init_mode = h0 ? gdn::kInitLoad : gdn::kInitZero;
        a.init = h0;
        a.x_before = H_in; a.x_after = nullptr; a.x_final = hT;
        hipError_t e = gdn::launch_scan(a, s);
        if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
        if (M_prefix && P > 0) {
            a.ncols = dk; a.S = nullptr;
            a.init_mode = gdn::kInitIdentity; a.init = nullptr;
            a.x_before = nullptr; a.x_after = M_prefix; a.x_final = nullptr;
            e = gdn::launch_scan(a, s);
            if (e != hipSuccess) return hip_fail(e, "prefix-product kernel launch");
        }
        return GDN_OK;
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

gdn_status gdn_apply_initial_state(const gdn_problem* p, int32_t seg_len, const void* q, const void* k,
                                   const void* v, const float* g, const float* beta, const float* H_in,
                                   void* o, float* hT, void* ws, size_t ws_bytes, void* stream) {
    try {
        (void)g;
        (void)beta;
        gdn_status st = check_problem(p);
        if (st != GDN_OK) return st;
        int64_t P = 0;
        st = check_segments(*p, seg_len, &P);
        if (st != GDN_OK) return st;
        const bool tokens = static_cast<int64_t>(p->B) * p->T > 0;
        if (tokens && (!q || !k || !v || !H_in || !o))
            return fail(GDN_EINVAL, "q, k, v, H_in and o must be non-NULL");
        if (tokens && !aligned16({q, k, v, o})) return fail(GDN_EINVAL, "q, k, v and o must be 16-byte aligned");
        hipStream_t s = static_cast<hipStream_t>(stream);
        const bool padded = use_mfma_padded(*p);
        const gdn_problem wp = padded ? padded_problem(*p) : *p;
        if (padded) {
            st = check_problem(&wp);
            if (st != GDN_OK) return st;
        }
        const SegPadPlan sp = padded ? make_seg_pad_plan(*p, P) : SegPadPlan{};
        const Plan pl = padded ? sp.rec : make_plan(*p, true);
        Plan need;
        need.bytes = padded ? sp.bytes : pl.bytes;
        st = check_ws(need, ws, ws_bytes);
        if (st != GDN_OK) return st;
        if (!tokens) return GDN_OK;
        char* base = static_cast<char*>(ws);
        const void* qw = q;
        const void* kw = k;
        const float* h_in = H_in;
        float* h_out = hT;
        if (padded) {
            // the padded q, k (again: this call may not follow the summary on the same
            // stream) and H_in with zero rows below dk
            hipError_t e = pad_qk(*p, sp, q, k, ws, s);
            if (e == hipSuccess)
                e = gdn::launch_copy_blocks(H_in, p->dk, p->dv * 4, base + sp.s_off, 128, p->dv * 4,
                                            static_cast<int64_t>(p->B) * p->H * P, s);
            if (e != hipSuccess) return hip_fail(e, "padding copy launch");
            qw = base + sp.q_off;
            kw = base + sp.k_off;
            h_in = reinterpret_cast<const float*>(base + sp.s_off);
            h_out = hT ? reinterpret_cast<float*>(base + sp.h_off) : nullptr;
        }
        const gdn::Workspace w = carve(pl, ws);
        gdn::StateArgs a = state_args(wp, pl, qw, kw, v, w);
        a.P = static_cast<int>(P);
        a.Lc = seg_len / gdn::kChunk;
        a.init_mode = gdn::kInitLoad;
        a.s_init = h_in;
        a.s_init_per_segment = 1;
        a.o = o;
        a.s_out = h_out;
        a.store_mode = h_out ? gdn::kStoreLastSegment : gdn::kStoreNone;
        st = run_state(wp, a, s);
        if (st != GDN_OK || !padded || !hT) return st;
        const hipError_t e = gdn::launch_copy_blocks(h_out, 128, p->dv * 4, hT, p->dk, p->dv * 4,
                                                     static_cast<int64_t>(p->B) * p->H, s);
        return e == hipSuccess ? GDN_OK : hip_fail(e, "final state copy launch");
    } catch (...) {
        return fail(GDN_EHIP, "unexpected exception");
    }
}

}  // extern "C"
