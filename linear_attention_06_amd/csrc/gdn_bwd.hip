// gdn_bwd.hip -- backward of the Gated DeltaNet recurrence for gfx950, fp32 on the
// vector ALUs (any head dim of the forward; q, k, v and the output gradient may be
// fp32 or bf16).
//
// Per batch row b and value head h, with the dk x dv state S and S_{-1} = h0:
//   w_t = S_{t-1}^T k_t,   S_t = e^{g_t} (S_{t-1} - beta_t k_t w_t^T) + beta_t k_t v_t^T,
//   o_t = S_t^T q_t
// (the recurrence of include/gdn.h written with the delta error on the decayed state).
// Given do_t and the gradient dhT of the final state, reverse mode gives, with
// M = dS_t + q_t do_t^T the full gradient of S_t and z = M^T k_t:
//   dq_t = S_t do_t                      dv_t = beta_t z
//   dk_t = beta_t M v_t - e^{g_t} beta_t (M w_t + S_{t-1} z)
//   dbeta_t = z . (v_t - e^{g_t} w_t)    dg_t = e^{g_t} (<M, S_{t-1}> - beta_t z . w_t)
//   dS_{t-1} = e^{g_t} (M - beta_t k_t z^T),   dh0 = dS_{-1}.
// The pages (hyper-parallel issue #320, the test report for PR #1114, section 4)
// check dq, dk, dv, dg, dbeta and dH0 against a reference; this is that gradient.
//
// Three kernels, one block of 16 x TPC threads per (b, h, 16 state columns) for the first
// two: thread TPC c + i holds column c of the tile at rows i + TPC j (j < dk / TPC), so
// that the TPC threads of a column are one DPP row (TPC = 16: four DPP rotations sum a
// column) or two (TPC = 32, used for dk >= 32: then a v_permlane16_swap). With 32 the
// SIMDs run two waves of a block and each thread's share of the token chain halves, which
// measured faster than 16 threads per column; 64 were slower. The sweep's pair sums give
// each thread at most one output, which needs 4 dk <= 16 TPC (true for both choices).
//   bwd_ckpt    the forward state before every 8th token into the workspace (each
//               tile in thread order, so a wave's stores and loads are contiguous);
//   bwd_sweep   chunks in reverse, 8-token pieces in reverse: each piece's states are
//               recomputed into registers from its checkpoint (loaded one piece ahead)
//               and the piece is run backwards; dv and
//               dh0 are complete per tile, dq, dk, dg and dbeta are written as one
//               partial per column tile, their column sums taken through LDS once per
//               pair of tokens (one barrier per pair);
//   bwd_reduce  sums the partials over the column tiles and over the value heads that
//               share a query/key head.
// Tokens at or past valid_len[b] are identities of the recurrence (beta = g = 0) with
// zero output: their gradients are zero.
#include "gdn_internal.hpp"

namespace gdn {
namespace {

__device__ __forceinline__ float ld_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_in(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Sum over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1); every lane gets it.
__device__ __forceinline__ float row_sum16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
    return x;
}

// Sum over the TPC lanes of a column (TPC = 16: one DPP row; TPC = 32: two DPP rows, the
// second step v_permlane16_swap, whose pair of results sums odd and even rows).
template <int TPC>
__device__ __forceinline__ float col_sum(float x) {
    x = row_sum16(x);
    if constexpr (TPC == 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}

// Token range of grid row bz: segment p = bz % P of batch row b = bz / P, tokens p L ..
// p L + L - 1 of the row, valid up to valid_len[b] (P = 1, L = T: the whole row).
template <bool kSeg>
__device__ __forceinline__ RowSpan bwd_span(const BwdArgs& a, int bz) {
    if constexpr (!kSeg) return row_span(nullptr, a.valid_len, bz, a.T, a.NT);
    const int b = bz / a.P, p = bz % a.P;
    int64_t n = a.T;
    if (a.valid_len) {
        n = a.valid_len[b];
        n = n < 0 ? 0 : (n > a.T ? a.T : n);
    }
    const int64_t s = static_cast<int64_t>(p) * a.L;
    n -= s;
    n = n < 0 ? 0 : (n > a.L ? a.L : n);
    return RowSpan{static_cast<int64_t>(b) * a.T + s, n, a.L};
}
// Index of the (row, segment, head) state block in a [B,H,P,dk,dv] array.
template <bool kSeg>
__device__ __forceinline__ int64_t seg_state(const BwdArgs& a, int bz, int h) {
    if constexpr (!kSeg) return static_cast<int64_t>(bz) * a.H + h;
    const int b = bz / a.P, p = bz % a.P;
    return (static_cast<int64_t>(b) * a.H + h) * a.P + p;
}

// Chunk operands in LDS (fp32): K, optionally Q, the tile's columns of V and of the
// output gradient, e^g and beta; padded tokens read as zero (e^g as one).
template <typename IO, int DK, bool kQ>
struct ChunkLds {
    float k[64][DK];
    float q[kQ ? 64 : 1][DK];
    float v[64][16];
    float d[kQ ? 64 : 1][16];
    float eg[64];      // e^{g}
    float beta[64];
};

// A chunk's operands in flight: every thread issues all its loads at once (addresses of
// padded tokens clamped to the row's token 0, which exists whenever the row has a chunk;
// their values are replaced by zero when stored), so one chunk can be fetched while the
// previous one is processed.
template <typename IO, int DK, bool kQ, int NTH>
struct ChunkRegs {
    static constexpr int EK = 64 * DK / NTH, EV = 64 * 16 / NTH;
    static_assert(EK * NTH == 64 * DK && EV * NTH == 64 * 16, "chunk tiles must split evenly");
    float k[EK], q[kQ ? EK : 1], v[EV], d[kQ ? EV : 1], g, beta;
};

template <bool kSeg, typename IO, int DK, bool kQ, int NTH>
__device__ __forceinline__ void fetch_chunk(ChunkRegs<IO, DK, kQ, NTH>& R, const BwdArgs& a, const RowSpan& rs, int h,
                                            int hq, int col0, int n, int tid) {
    using CR = ChunkRegs<IO, DK, kQ, NTH>;
    const IO* k = static_cast<const IO*>(a.k);
    const IO* q = static_cast<const IO*>(a.q);
    const IO* v = static_cast<const IO*>(a.v);
    const IO* d = static_cast<const IO*>(a.d_o);
    const int64_t t0 = static_cast<int64_t>(n) * kChunk;
#pragma unroll
    for (int m = 0; m < CR::EK; ++m) {
        const int e = tid + NTH * m, r = e / DK, x = e % DK;
        const int64_t tok = t0 + r < rs.valid ? t0 + r : 0;
        const int64_t idx = ((rs.start + tok) * a.Hqk + hq) * DK + x;
        R.k[m] = ld_in(k, idx);
        if (kQ) R.q[m] = ld_in(q, idx);
    }
#pragma unroll
    for (int m = 0; m < CR::EV; ++m) {
        const int e = tid + NTH * m, r = e / 16, c = e % 16;
        const int64_t tok = t0 + r < rs.valid ? t0 + r : 0;
        const int64_t idx = ((rs.start + tok) * a.H + h) * a.dv + col0 + c;
        R.v[m] = (kSeg && a.v_zero) ? 0.f : ld_in(v, idx);
        if (kQ) R.d[m] = (kSeg && a.do_zero) ? 0.f : ld_in(d, idx);
    }
    const int64_t tok = t0 + (tid & 63) < rs.valid ? t0 + (tid & 63) : 0;
    const int64_t gi = (rs.start + tok) * a.H + h;
    R.g = a.g[gi];
    R.beta = a.beta[gi];
}

template <typename IO, int DK, bool kQ, int NTH>
__device__ __forceinline__ void store_chunk(ChunkLds<IO, DK, kQ>& L, const ChunkRegs<IO, DK, kQ, NTH>& R,
                                            const RowSpan& rs, int n, int tid) {
    using CR = ChunkRegs<IO, DK, kQ, NTH>;
    const int64_t t0 = static_cast<int64_t>(n) * kChunk;
#pragma unroll
    for (int m = 0; m < CR::EK; ++m) {
        const int e = tid + NTH * m, r = e / DK, x = e % DK;
        const bool ok = t0 + r < rs.valid;
        L.k[r][x] = ok ? R.k[m] : 0.f;
        if (kQ) L.q[r][x] = ok ? R.q[m] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < CR::EV; ++m) {
        const int e = tid + NTH * m, r = e / 16, c = e % 16;
        const bool ok = t0 + r < rs.valid;
        L.v[r][c] = ok ? R.v[m] : 0.f;
        if (kQ) L.d[r][c] = ok ? R.d[m] : 0.f;
    }
    if (tid < 64) {
        const bool ok = t0 + tid < rs.valid;
        L.eg[tid] = ok ? expf(R.g) : 1.f;
        L.beta[tid] = ok ? R.beta : 0.f;
    }
}

// One forward token step on the thread's column slice S[j] = S[i + TPC j][c]; returns w_c.
template <int RJ, int TPC, typename Lds>
__device__ __forceinline__ float fwd_step(float (&S)[RJ], const Lds& L, int u, int i, int c) {
    float w = 0.f;
#pragma unroll
    for (int j = 0; j < RJ; ++j) w += L.k[u][i + TPC * j] * S[j];
    w = col_sum<TPC>(w);
    // e^g (S - beta k w^T) + beta k v^T = e^g S + k (beta (v - e^g w))^T
    const float eg = L.eg[u], ac = L.beta[u] * (L.v[u][c] - eg * w);
#pragma unroll
    for (int j = 0; j < RJ; ++j) S[j] = fmaf(L.k[u][i + TPC * j], ac, eg * S[j]);
    return w;
}

// kSeg: the segment features of BwdArgs (segments, identity start, zero values or output
// gradient, no dv, accumulation) are read; without it the kernels run the plain backward.
template <typename IO, int DK, int TPC, bool kSeg>
__global__ __launch_bounds__(16 * TPC) void bwd_ckpt(BwdArgs a) {
    constexpr int RJ = DK / TPC, NTH = 16 * TPC;
    __shared__ ChunkLds<IO, DK, false> L;
    const int col0 = 16 * blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int hq = h / (a.H / a.Hqk);
    const int tid = threadIdx.x, c = tid / TPC, i = tid % TPC;
    const RowSpan rs = bwd_span<kSeg>(a, b);
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int64_t sb = seg_state<kSeg>(a, b, h);
    float S[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int r = i + TPC * j;
        S[j] = (kSeg && a.h0_identity) ? (r == col0 + c ? 1.f : 0.f) : (a.h0 ? a.h0[(sb * DK + r) * a.dv + col0 + c] : 0.f);
    }
    ChunkRegs<IO, DK, false, NTH> R;
    if (a.NT > 0) fetch_chunk<kSeg>(R, a, rs, h, hq, col0, 0, tid);
    for (int n = 0; n < a.NT; ++n) {
        __syncthreads();
        store_chunk(L, R, rs, n, tid);
        __syncthreads();
        if (n + 1 < a.NT) fetch_chunk<kSeg>(R, a, rs, h, hq, col0, n + 1, tid);
        for (int u = 0; u < 64; ++u) {
            if ((u & 7) == 0) {   // the state before every 8th token, in thread order
                float* ck = a.ckpt + ((bh * 8 * a.NT + 8 * n + (u >> 3)) * (a.dv / 16) + blockIdx.x) * (16 * DK);
#pragma unroll
                for (int j = 0; j < RJ; ++j) ck[j * NTH + tid] = S[j];
            }
            fwd_step<RJ, TPC>(S, L, u, i, c);
        }
    }
}

template <typename IO, int DK, int TPC, bool kSeg>
__global__ __launch_bounds__(16 * TPC) void bwd_sweep(BwdArgs a) {
    constexpr int RJ = DK / TPC, NTH = 16 * TPC;
    __shared__ ChunkLds<IO, DK, true> L;
    // per-column terms of dq and dk, of dg and dbeta, for four tokens in turn: a barrier
    // after every second token, then the block sums that pair's terms; a pair's reads end
    // before the next barrier, which every thread passes before the next pair writes
    __shared__ float red_s[4][2][16][DK];
    __shared__ float red2_s[4][2][16];
    const int tiles = a.dv / 16;
    const int tile = blockIdx.x, col0 = 16 * tile, h = blockIdx.y, b = blockIdx.z;
    const int hq = h / (a.H / a.Hqk);
    const int tid = threadIdx.x, c = tid / TPC, i = tid % TPC;
    const RowSpan rs = bwd_span<kSeg>(a, b);
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int64_t sb = seg_state<kSeg>(a, b, h);
    // the final-state gradient: per segment, or the row's for its last segment only
    const float* dhT = a.dhT;
    int64_t dsb = sb;
    if (kSeg && !a.dhT_per_segment) {
        dsb = static_cast<int64_t>(b / a.P) * a.H + h;
        if (b % a.P != a.P - 1) dhT = nullptr;
    }

    float dS[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j)
        dS[j] = dhT ? dhT[(dsb * DK + i + TPC * j) * a.dv + col0 + c] : 0.f;

    // the checkpoint of 8-token piece m (the state before token 8 m), loaded one piece ahead
    const auto load_ck = [&](int m, float (&x)[RJ]) {
        const float* ck = a.ckpt + ((bh * 8 * a.NT + m) * tiles + tile) * (16 * DK);
#pragma unroll
        for (int j = 0; j < RJ; ++j) x[j] = ck[j * NTH + tid];
    };
    float nxt[RJ];
    if (a.NT > 0) load_ck(8 * a.NT - 1, nxt);

    ChunkRegs<IO, DK, true, NTH> R;
    if (a.NT > 0) fetch_chunk<kSeg>(R, a, rs, h, hq, col0, a.NT - 1, tid);
    // token strides of dv and of the partials; this thread's output of the pair sums:
    // token u + 1 - rp, the dq (rwhich = 0) or dk (1) term of row rr
    static_assert(4 * DK <= NTH, "at most one pair-sum output per thread");
    const int64_t sdv = static_cast<int64_t>(a.H) * a.dv;
    const int64_t sqk = static_cast<int64_t>(a.H) * tiles * 2 * DK;
    const int64_t sgb = static_cast<int64_t>(a.H) * tiles * 2;
    const int rp = tid / (2 * DK), rwhich = (tid / DK) & 1, rr = tid % DK;

    for (int n = a.NT - 1; n >= 0; --n) {
        __syncthreads();
        store_chunk(L, R, rs, n, tid);
        __syncthreads();
        if (n > 0) fetch_chunk<kSeg>(R, a, rs, h, hq, col0, n - 1, tid);
        // the chunk's tokens that take part and that the row writes (0..64), and its
        // output addresses at its first token
        const int64_t ct0 = static_cast<int64_t>(n) * kChunk, r0 = rs.start + ct0;
        const int nvalid = static_cast<int>(rs.valid - ct0 < 0 ? 0 : (rs.valid - ct0 > 64 ? 64 : rs.valid - ct0));
        const int nwrite = static_cast<int>(rs.extent - ct0 < 0 ? 0 : (rs.extent - ct0 > 64 ? 64 : rs.extent - ct0));
        float* const dv_c = a.dv_out + (r0 * a.H + h) * a.dv + col0 + c;
        float* const qk_c = a.dqk_part + ((r0 * a.H + h) * tiles + tile) * 2 * DK + (1 - rp) * sqk + rwhich * DK + rr;
        float* const gb_c = a.dgb_part + ((r0 * a.H + h) * tiles + tile) * 2 + (1 - ((tid >> 5) & 1)) * sgb +
                            ((tid >> 4) & 1);
        for (int s = 7; s >= 0; --s) {
            float* const dv_s = dv_c + 8 * s * sdv;
            float* const qk_s = qk_c + 8 * s * sqk;
            float* const gb_s = gb_c + 8 * s * sgb;
            // the piece's states in registers: St[u] before token 8 s + u, St[u + 1] after it
            float St[9][RJ], w[8];
#pragma unroll
            for (int j = 0; j < RJ; ++j) St[0][j] = nxt[j];
            if (8 * n + s > 0) load_ck(8 * n + s - 1, nxt);
#pragma unroll
            for (int uu = 0; uu < 8; ++uu) {
#pragma unroll
                for (int j = 0; j < RJ; ++j) St[uu + 1][j] = St[uu][j];
                w[uu] = fwd_step<RJ, TPC>(St[uu + 1], L, 8 * s + uu, i, c);
            }
#pragma unroll
            for (int uu = 7; uu >= 0; --uu) {
                const int u = 8 * s + uu;
                const bool valid = u < nvalid;
                const float eg = L.eg[u], bt = L.beta[u], vc = L.v[u][c], doc = L.d[u][c];
                float M[RJ];
                float z = 0.f, ms = 0.f;
#pragma unroll
                for (int j = 0; j < RJ; ++j) {
                    M[j] = dS[j] + L.q[u][i + TPC * j] * doc;
                    z += M[j] * L.k[u][i + TPC * j];
                    ms += M[j] * St[uu][j];
                }
                z = col_sum<TPC>(z);
                ms = col_sum<TPC>(ms);
                // the tail of the last chunk is past the row
                if ((!kSeg || a.write_dv) && i == 0 && u < nwrite) {
                    const float x = valid ? bt * z : 0.f;
                    dv_s[uu * sdv] = (kSeg && a.accumulate) ? dv_s[uu * sdv] + x : x;
                }
                // dk's column terms: M beta (v - e^g w) - e^g beta z S_{t-1}
                const float am = bt * (vc - eg * w[uu]), bz = eg * bt * z;
#pragma unroll
                for (int j = 0; j < RJ; ++j) {
                    const int r = i + TPC * j;
                    red_s[uu & 3][0][c][r] = St[uu + 1][j] * doc;
                    red_s[uu & 3][1][c][r] = fmaf(M[j], am, -bz * St[uu][j]);
                }
                if (i == 0) {
                    red2_s[uu & 3][0][c] = valid ? eg * (ms - bt * z * w[uu]) : 0.f;
                    red2_s[uu & 3][1][c] = valid ? z * (vc - eg * w[uu]) : 0.f;
                }
                if ((uu & 1) == 0) {
                    // the pair of tokens u + 1 (slot p = 0) and u (p = 1)
                    __syncthreads();
                    if (tid < 4 * DK && u + 1 - rp < nwrite) {
                        float acc = 0.f;
#pragma unroll
                        for (int cc = 0; cc < 16; ++cc) acc += red_s[(uu + 1 - rp) & 3][rwhich][cc][rr];
                        qk_s[uu * sqk] = u + 1 - rp < nvalid ? acc : 0.f;
                    }
                    if (tid < 64) {
                        // wave 0: lane 16 (2 p + which) + cc holds column cc's term, and the
                        // 16 lanes of a DPP row sum them
                        const int p = tid / 32, which = (tid / 16) & 1;
                        const float acc = row_sum16(red2_s[(uu + 1 - p) & 3][which][tid & 15]);
                        if ((tid & 15) == 0 && u + 1 - p < nwrite) gb_s[uu * sgb] = acc;
                    }
                }
#pragma unroll
                for (int j = 0; j < RJ; ++j) dS[j] = fmaf(-bz, L.k[u][i + TPC * j], eg * M[j]);
            }
        }
    }
    if (a.dh0_out) {
#pragma unroll
        for (int j = 0; j < RJ; ++j) a.dh0_out[(sb * DK + i + TPC * j) * a.dv + col0 + c] = dS[j];
    }
}

// One block per (t, b): dq, dk per query/key head (sum over column tiles and the
// value heads of the group), dg and dbeta per value head (sum over column tiles).
template <int DK, bool kSeg>
__global__ __launch_bounds__(256) void bwd_reduce(BwdArgs a) {
    const int64_t t = blockIdx.x;
    const int b = blockIdx.y;
    const int tiles = a.dv / 16, rep = a.H / a.Hqk;
    const int64_t row = static_cast<int64_t>(b) * a.T + t;
    // four rows per thread in 16-byte loads, eight tiles' loads in flight at once
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    for (int e = threadIdx.x; e < a.Hqk * (DK / 4); e += 256) {
        const int hq = e / (DK / 4), r = 4 * (e % (DK / 4));
        f32x4 sq = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
        for (int hh = 0; hh < rep; ++hh) {
            const float* part = a.dqk_part + ((row * a.H + hq * rep + hh) * tiles) * 2 * DK + r;
#pragma unroll 8
            for (int tl = 0; tl < tiles; ++tl) {
                sq += *reinterpret_cast<const f32x4*>(part + tl * 2 * DK);
                sk += *reinterpret_cast<const f32x4*>(part + tl * 2 * DK + DK);
            }
        }
        float* dq = a.dq_out + (row * a.Hqk + hq) * DK + r;
        float* dk = a.dk_out + (row * a.Hqk + hq) * DK + r;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            dq[x] = (kSeg && a.accumulate) ? dq[x] + sq[x] : sq[x];
            dk[x] = (kSeg && a.accumulate) ? dk[x] + sk[x] : sk[x];
        }
    }
    for (int hh = threadIdx.x; hh < a.H; hh += 256) {
        const float* part = a.dgb_part + (row * a.H + hh) * tiles * 2;
        float sg = 0.f, sb = 0.f;
        for (int tl = 0; tl < tiles; ++tl) {
            sg += part[2 * tl];
            sb += part[2 * tl + 1];
        }
        a.dg_out[row * a.H + hh] = (kSeg && a.accumulate) ? a.dg_out[row * a.H + hh] + sg : sg;
        a.dbeta_out[row * a.H + hh] = (kSeg && a.accumulate) ? a.dbeta_out[row * a.H + hh] + sb : sb;
    }
}

// Threads per state column: 32 (two DPP rows, 512-thread blocks, two waves per SIMD)
// once dk >= 32, else 16.
constexpr int kTpc(int dk) { return dk >= 32 ? 32 : 16; }

template <typename IO, bool kSeg>
hipError_t bwd_dispatch(const BwdArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.dv / 16), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B * a.P));
    void* args[] = {const_cast<BwdArgs*>(&a)};
    const void *f1 = nullptr, *f2 = nullptr, *f3 = nullptr;
    unsigned nth = 256;
    switch (a.dk) {
#define GDN_BWD_CASE(D)                                                                  \
        case D:                                                                          \
            f1 = reinterpret_cast<const void*>(&bwd_ckpt<IO, D, kTpc(D), kSeg>);         \
            f2 = reinterpret_cast<const void*>(&bwd_sweep<IO, D, kTpc(D), kSeg>);        \
            f3 = reinterpret_cast<const void*>(&bwd_reduce<D, kSeg>);                    \
            nth = 16 * kTpc(D);                                                          \
            break;
        GDN_BWD_CASE(16)
        GDN_BWD_CASE(32)
        GDN_BWD_CASE(64)
        GDN_BWD_CASE(128)
#undef GDN_BWD_CASE
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipLaunchKernel(f1, grid, dim3(nth), args, 0, s);
    if (e != hipSuccess) return e;
    e = hipLaunchKernel(f2, grid, dim3(nth), args, 0, s);
    if (e != hipSuccess || a.T == 0) return e;
    return hipLaunchKernel(f3, dim3(static_cast<unsigned>(a.T), static_cast<unsigned>(a.B)), dim3(256), args, 0, s);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, bool io_bf16, hipStream_t s) {
    const bool seg = a.P != 1 || a.dhT_per_segment || a.h0_identity || a.v_zero || a.do_zero || !a.write_dv ||
                     a.accumulate;
    if (seg) return io_bf16 ? bwd_dispatch<uint16_t, true>(a, s) : bwd_dispatch<float, true>(a, s);
    return io_bf16 ? bwd_dispatch<uint16_t, false>(a, s) : bwd_dispatch<float, false>(a, s);
}

}  // namespace gdn
