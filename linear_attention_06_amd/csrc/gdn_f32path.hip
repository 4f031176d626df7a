// gdn_f32path.hip -- fp32-arithmetic kernels of the chunked Gated DeltaNet
// forward for gfx950. They serve fp32 I/O (where the fp32 tolerance rules out
// bf16 matrix cores) and head dims the matrix-core path does not cover. All
// arithmetic is fp32 on the vector ALUs; q, k, v, o may be fp32 or bf16.
//
// Chunk algebra (chunk of C = 64 tokens, incoming state S, Gam = chunk-local
// cumulative sum of g; see the method statement in include/gdn.h):
//   A_ij  = beta_i exp(Gam_i - Gam_j) k_i.k_j  (i > j),  Tinv = (I + A)^{-1}
//   U     = Tinv diag(beta) (V - diag(exp Gam) K S)        delta-rule errors
//   O     = diag(exp Gam) Q S + P U,   P_ij = (q_i.k_j) exp(Gam_i - Gam_j), j <= i
//   S'    = exp(Gam_C) S + (diag(exp(Gam_C - Gam)) K)^T U
// This is the UT/WY chunk form of the Gated DeltaNet recurrence; the decay
// factors used are all exp of non-positive numbers, so nothing overflows.
#include "gdn_internal.hpp"

namespace gdn {
namespace {

__device__ __forceinline__ float ld_io(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_io(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ void st_io(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st_io(uint16_t* p, int64_t i, float x) {
    p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
}

__device__ __forceinline__ int64_t valid_tokens(const int32_t* vl, int b, int64_t T) {
    if (!vl) return T;
    int64_t n = vl[b];
    return n < 0 ? 0 : (n > T ? T : n);
}

// Two waves per (b, h, chunk): cumulative decay, A, the unit-lower-triangular
// inverse by forward substitution (wave 0), P and the decay factors.
template <typename IO, int DK>
__global__ __launch_bounds__(128) void prep_f32path(PrepArgs a) {
    constexpr int KP = DK + 1;
    constexpr int KT = (64 * KP > 64 * 65) ? 64 * KP : 64 * 65;
    __shared__ float kt_s[KT];          // K rows, later the inverse
    __shared__ float a_s[64 * 65];
    __shared__ float gam_s[64];

    const int64_t ch = blockIdx.x;
    const int n = static_cast<int>(ch % a.NT);
    const int bh = static_cast<int>(ch / a.NT);
    const int h = bh % a.H, b = bh / a.H;
    const int hq = h / (a.H / a.Hqk);
    // two waves: both hold row i = lane of the chunk; wave `half` forms the column pairs
    // j0 = 4 m + 2 half of A and P, and wave 0 alone runs the solve
    const int i = threadIdx.x & 63, half = threadIdx.x >> 6;
    const int64_t t = static_cast<int64_t>(n) * kChunk + i;
    const RowSpan rs = row_span(a.cu_seqlens, a.valid_len, b, a.T, a.NT);
    const bool valid = t < rs.valid;
    const IO* q = static_cast<const IO*>(a.q);
    const IO* k = static_cast<const IO*>(a.k);

    const int64_t gi_idx = (rs.start + t) * a.H + h;
    const float gi = valid ? a.g[gi_idx] : 0.f;
    const float bi = valid ? a.beta[gi_idx] : 0.f;
    float gam = gi;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(gam, off, 64);
        if (i >= off) gam += y;
    }
    if (half == 0) gam_s[i] = gam;
    const int64_t row = ((rs.start + t) * a.Hqk + hq) * DK;
    float qreg[DK];
#pragma unroll
    for (int d = 0; d < DK; ++d) {
        const float kv = valid ? ld_io(k, row + d) : 0.f;
        if (half == 0) kt_s[i * KP + d] = kv;
        qreg[d] = valid ? ld_io(q, row + d) : 0.f;
    }
    __syncthreads();

    float* that = static_cast<float*>(a.ws.that) + ch * 4096;
    float* pm = static_cast<float*>(a.ws.pmat) + ch * 4096;
    // two columns j at a time: the lane's own K row is read once per two products, and its
    // two P values leave in one 8-byte store (wider blocks spill registers at dk = 128)
    for (int j0 = 2 * half; j0 < 64; j0 += 4) {
        float kk[2], qk[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) kk[jj] = qk[jj] = 0.f;
        if (j0 <= i) {
            // fully unrolled, so that qreg stays in registers
#pragma unroll
            for (int d = 0; d < DK; ++d) {
                const float ki = kt_s[i * KP + d];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const float kj = kt_s[(j0 + jj) * KP + d];
                    kk[jj] += ki * kj;
                    qk[jj] += qreg[d] * kj;
                }
            }
        }
        float pv[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = j0 + jj;
            float av = 0.f;
            pv[jj] = 0.f;
            if (j <= i) {
                const float decay = expf(gam - gam_s[j]);
                pv[jj] = decay * qk[jj];
                if (j < i) av = bi * decay * kk[jj];
            }
            a_s[i * 65 + j] = av;
        }
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<f32x2*>(pm + i * 64 + j0) = f32x2{pv[0], pv[1]};
    }
    __syncthreads();
    if (half != 0) return;   // no barrier follows

    // Forward substitution, lane c owns column c of Tinv.
    float* t_s = kt_s;
    const int c = i;
    for (int r = 0; r < 64; ++r) {
        float acc = (r == c) ? 1.f : 0.f;
        for (int j = 0; j < r; ++j) acc -= a_s[r * 65 + j] * t_s[j * 65 + c];
        t_s[r * 65 + c] = acc;
    }
    for (int r = 0; r < 64; ++r) that[r * 64 + c] = t_s[r * 65 + c] * bi;
    const float gam_c = __shfl(gam, 63, 64);
    float* gates = a.ws.gates + ch * 128;
    gates[i] = expf(gam);
    gates[64 + i] = expf(gam_c - gam);
}

// One block of 64 (16 / CPT) threads per (b, h, segment, 16 state columns): the
// sequential pass over the segment's chunks with the state tile in LDS; thread t holds
// token row t / (16 / CPT) and CPT columns from CPT (t % (16 / CPT)).
template <typename IO, int DK, int CPT>
__global__ __launch_bounds__(64 * (16 / CPT)) void state_f32path(StateArgs a) {
    constexpr int KP = DK + 1;
    constexpr int BV = 16;
    constexpr int NTH = 64 * (BV / CPT);   // 64 token rows x BV / CPT groups of CPT columns
    typedef float vecC __attribute__((ext_vector_type(CPT)));
    __shared__ float k_s[64 * KP];
    // the state tile, X and U with rows of 16 floats: every read below is either the same
    // row for the whole wave or consecutive columns, so 16-byte reads are conflict-free
    __shared__ __align__(16) float s_s[DK * BV];
    __shared__ __align__(16) float x_s[64 * BV];
    __shared__ __align__(16) float u_s[64 * BV];
    __shared__ float t_s[64 * 65];     // the chunk's That
    __shared__ float p_s[64 * 65];     // and P (when o is written)
    __shared__ float g_s[128];
    typedef float f32x4 __attribute__((ext_vector_type(4)));

    const int col0 = blockIdx.x * BV;
    const int h = blockIdx.y;
    const int b = blockIdx.z / a.P, seg = blockIdx.z % a.P;
    const int hq = h / (a.H / a.Hqk);
    const int tid = threadIdx.x;
    const RowSpan rs = row_span(a.cu_seqlens, a.valid_len, b, a.T, a.NT);
    const int64_t nvalid = rs.valid;
    const int ncols = a.ncols;
    const IO* q = static_cast<const IO*>(a.q);
    const IO* k = static_cast<const IO*>(a.k);
    const IO* v = static_cast<const IO*>(a.v);
    IO* o = static_cast<IO*>(a.o);
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int64_t tile = static_cast<int64_t>(DK) * ncols;

    for (int e = tid; e < DK * BV; e += NTH) {
        const int i = e / BV, c = e % BV;
        float s0 = 0.f;
        if (a.init_mode == kInitLoad) {
            const int64_t blk = a.s_init_per_segment ? bh * a.P + seg : bh;
            s0 = a.s_init[blk * tile + static_cast<int64_t>(i) * ncols + col0 + c];
        } else if (a.init_mode == kInitIdentity) {
            s0 = (i == col0 + c) ? 1.f : 0.f;
        }
        s_s[i * BV + c] = s0;
    }

    const int r = tid / (BV / CPT);            // token row within the chunk
    const int c4 = (tid % (BV / CPT)) * CPT;   // first of this thread's CPT columns
    const int n0 = seg * a.Lc;
    const int n1 = min(min(n0 + a.Lc, a.NT), static_cast<int>((rs.extent + kChunk - 1) / kChunk));

    // A chunk's operands in flight: K rows, That, P and the decay factors. Every
    // thread issues all its loads at once, one chunk ahead (addresses of padded tokens
    // clamped to the row's first token, which exists whenever the row has a chunk; their
    // values are replaced by zero when stored).
    constexpr int EK = 64 * DK / NTH, ET = 1024 / NTH;
    float kr[EK], gr = 0.f;
    f32x4 tr[ET], pr[ET];
    const auto fetch = [&](int n) {
        const int64_t t0 = static_cast<int64_t>(n) * kChunk;
        const int64_t ch = bh * a.NT + n;
#pragma unroll
        for (int m = 0; m < EK; ++m) {
            const int e = tid + NTH * m, rr = e / DK, d = e % DK;
            const int64_t idx = ((rs.start + (t0 + rr < nvalid ? t0 + rr : 0)) * a.Hqk + hq) * DK + d;
            kr[m] = ld_io(k, idx);
        }
        const f32x4* tg = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.ws.that) + ch * 4096);
        const f32x4* pg = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.ws.pmat) + ch * 4096);
#pragma unroll
        for (int m = 0; m < ET; ++m) {
            tr[m] = tg[tid + NTH * m];
            if (o) pr[m] = pg[tid + NTH * m];
        }
        if (tid < 128) gr = a.ws.gates[ch * 128 + tid];
    };
    if (n0 < n1) fetch(n0);
    for (int n = n0; n < n1; ++n) {
        const int64_t t0 = static_cast<int64_t>(n) * kChunk;
        __syncthreads();
#pragma unroll
        for (int m = 0; m < EK; ++m) {
            const int e = tid + NTH * m, rr = e / DK, d = e % DK;
            k_s[rr * KP + d] = t0 + rr < nvalid ? kr[m] : 0.f;
        }
#pragma unroll
        for (int m = 0; m < ET; ++m) {
            const int e = tid + NTH * m, rr = e / 16, cc = 4 * (e % 16);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                t_s[rr * 65 + cc + x] = tr[m][x];
                if (o) p_s[rr * 65 + cc + x] = pr[m][x];
            }
        }
        if (tid < 128) g_s[tid] = gr;
        __syncthreads();
        if (n + 1 < n1) fetch(n + 1);

        const int64_t tok = t0 + r;
        const bool valid = tok < nvalid;
        // q straight from memory (the row's threads share it), addresses clamped so the
        // unrolled loads issue together; only read when o is written
        const int64_t qrow = ((rs.start + (valid ? tok : 0)) * a.Hqk + hq) * DK;
        float ks[CPT], qs[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) ks[c] = qs[c] = 0.f;
#pragma unroll 8
        for (int i = 0; i < DK; ++i) {
            const float kv = k_s[r * KP + i];
            const float qm = o ? ld_io(q, qrow + i) : 0.f;
            const float qv = valid ? qm : 0.f;
            const vecC sv = *reinterpret_cast<const vecC*>(&s_s[i * BV + c4]);
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                ks[c] += kv * sv[c];
                qs[c] += qv * sv[c];
            }
        }
        const float eg = g_s[r];
        const int64_t vrow = ((rs.start + tok) * a.H + h) * ncols + col0 + c4;
        vecC xv;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float vv = (v && valid) ? ld_io(v, vrow + c) : 0.f;
            xv[c] = vv - eg * ks[c];
        }
        *reinterpret_cast<vecC*>(&x_s[r * BV + c4]) = xv;
        __syncthreads();

        vecC u;
#pragma unroll
        for (int c = 0; c < CPT; ++c) u[c] = 0.f;
        for (int s = 0; s <= r; ++s) {
            const float tv = t_s[r * 65 + s];
            const vecC xs = *reinterpret_cast<const vecC*>(&x_s[s * BV + c4]);
#pragma unroll
            for (int c = 0; c < CPT; ++c) u[c] += tv * xs[c];
        }
        *reinterpret_cast<vecC*>(&u_s[r * BV + c4]) = u;
        __syncthreads();

        if (o && tok < rs.extent) {
            float ov[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) ov[c] = eg * qs[c];
            for (int s = 0; s <= r; ++s) {
                const float pv = p_s[r * 65 + s];
                const vecC us = *reinterpret_cast<const vecC*>(&u_s[s * BV + c4]);
#pragma unroll
                for (int c = 0; c < CPT; ++c) ov[c] += pv * us[c];
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) st_io(o, vrow + c, valid ? ov[c] : 0.f);
        }

        // S <- e^{Gam_C} S + K^T (e^{Gam_C - Gam} U): the thread's elements are rows
        // i0 + RS m of column cs (RS = NTH / BV), so each step reads the column's scaled U
        // value once; with more threads than elements (dk = 16, 512 threads) the rest idle
        constexpr int RS = NTH / BV, ES = (DK + RS - 1) / RS;
        const int cs = tid % BV, i0 = tid / BV;
        if (i0 < DK) {
            const float egC = g_s[63];
            float acc[ES];
#pragma unroll
            for (int m = 0; m < ES; ++m) acc[m] = egC * s_s[(i0 + RS * m) * BV + cs];
            for (int s = 0; s < 64; ++s) {
                const float gu = g_s[64 + s] * u_s[s * BV + cs];
#pragma unroll
                for (int m = 0; m < ES; ++m) acc[m] = fmaf(k_s[s * KP + i0 + RS * m], gu, acc[m]);
            }
#pragma unroll
            for (int m = 0; m < ES; ++m) s_s[(i0 + RS * m) * BV + cs] = acc[m];
        }
    }
    __syncthreads();

    if (a.store_mode == kStoreNone) return;
    if (a.store_mode == kStoreLastSegment && seg != a.P - 1) return;
    const int64_t blk = (a.store_mode == kStoreEverySegment) ? bh * a.P + seg : bh;
    for (int e = tid; e < DK * BV; e += NTH) {
        const int i = e / BV, c = e % BV;
        a.s_out[blk * tile + static_cast<int64_t>(i) * ncols + col0 + c] = s_s[i * BV + c];
    }
}

// X_p = M_p X_{p-1} + S_p over the segments of one (b, h), 16 columns per block.
// Thread t < 2 dk owns row t / 2 and columns 8 (t % 2) .. +7 of the 16: it streams
// row t / 2 of M_p once per step with 16-byte loads against X_{p-1} held in LDS.
// fp32 throughout (the summary products must stay accurate).
template <int DKT>
__global__ __launch_bounds__(256) void affine_scan(ScanArgs a) {
    constexpr int BV = 16;
    constexpr int dk = DKT;
    __shared__ float x_s[DKT * BV];
    const int col0 = blockIdx.x * BV;
    const int h = blockIdx.y, b = blockIdx.z;
    const int ncols = a.ncols;
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int64_t tile = static_cast<int64_t>(dk) * ncols;
    const int tid = threadIdx.x;

    for (int e = tid; e < dk * BV; e += 256) {
        const int i = e / BV, c = e % BV;
        float x0 = 0.f;
        if (a.init_mode == kInitLoad) x0 = a.init[bh * tile + static_cast<int64_t>(i) * ncols + col0 + c];
        else if (a.init_mode == kInitIdentity) x0 = (i == col0 + c) ? 1.f : 0.f;
        x_s[e] = x0;
    }
    __syncthreads();
    const bool active = tid < 2 * dk;
    const int i = tid >> 1, c0 = 8 * (tid & 1);
    const int64_t out0 = static_cast<int64_t>(i) * ncols + col0 + c0;   // this thread's 8 outputs
    for (int p = 0; p < a.P; ++p) {
        const int64_t blk = bh * a.P + p;
        float acc[8];
        if (active) {
            if (a.x_before)
#pragma unroll
                for (int c = 0; c < 8; ++c) a.x_before[blk * tile + out0 + c] = x_s[i * BV + c0 + c];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = a.S ? a.S[blk * tile + out0 + c] : 0.f;
            const float4* mrow = reinterpret_cast<const float4*>(a.M + blk * static_cast<int64_t>(dk) * dk +
                                                                 static_cast<int64_t>(i) * dk);
            float4 mr[dk / 4];   // the whole row in flight at once
#pragma unroll
            for (int l4 = 0; l4 < dk / 4; ++l4) mr[l4] = mrow[l4];
#pragma unroll
            for (int l4 = 0; l4 < dk / 4; ++l4) {
                const float4 m4 = mr[l4];
                const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float* xr = x_s + (4 * l4 + u) * BV + c0;
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[c] += mv[u] * xr[c];
                }
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                x_s[i * BV + c0 + c] = acc[c];
                if (a.x_after) a.x_after[blk * tile + out0 + c] = acc[c];
            }
        }
        __syncthreads();
    }
    if (a.x_final && active) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a.x_final[bh * tile + out0 + c] = x_s[i * BV + c0 + c];
    }
}

// Reverse of the prefix combine, one block per (16 columns, h, b): the gradient G of the
// running state (dk x 16, in LDS) from dhT (or 0); for p = P-1 .. 0 it is stored as dS_p,
// then G <- M_p^T G + dH_in_p; the last G is dh0. Thread (i, half) computes row i of
// M_p^T G for 8 columns, reading column i of M_p.
template <int DKT>
__global__ __launch_bounds__(256) void affine_scan_rev(ScanBwdArgs a) {
    constexpr int BV = 16;
    constexpr int dk = DKT;
    __shared__ float g_s[DKT * BV];
    const int col0 = blockIdx.x * BV;
    const int h = blockIdx.y, b = blockIdx.z;
    const int dv = a.dv;
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int64_t tile = static_cast<int64_t>(dk) * dv;
    const int tid = threadIdx.x;
    for (int e = tid; e < dk * BV; e += 256) {
        const int i = e / BV, c = e % BV;
        g_s[e] = a.dhT ? a.dhT[bh * tile + static_cast<int64_t>(i) * dv + col0 + c] : 0.f;
    }
    __syncthreads();
    const bool active = tid < 2 * dk;
    const int i = tid >> 1, c0 = 8 * (tid & 1);
    const int64_t out0 = static_cast<int64_t>(i) * dv + col0 + c0;
    for (int p = a.P - 1; p >= 0; --p) {
        const int64_t blk = bh * a.P + p;
        float acc[8];
        if (active) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                a.dS[blk * tile + out0 + c] = g_s[i * BV + c0 + c];
                acc[c] = a.dH_in[blk * tile + out0 + c];
            }
            const float* mcol = a.M + blk * static_cast<int64_t>(dk) * dk + i;
            for (int l = 0; l < dk; ++l) {
                const float m = mcol[static_cast<int64_t>(l) * dk];   // M_p[l][i]
                const float* gr = g_s + l * BV + c0;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] += m * gr[c];
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int c = 0; c < 8; ++c) g_s[i * BV + c0 + c] = acc[c];
        }
        __syncthreads();
    }
    if (a.dh0 && active) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a.dh0[bh * tile + out0 + c] = g_s[i * BV + c0 + c];
    }
}

// The two scans above for dk = 128 on v_mfma_f32_16x16x4_f32 (fp32 products, fp32
// accumulation), one block of four waves per (16 columns, h, b); wave w owns rows 32 w ..
// 32 w + 31 of the running state (two 16-row tiles in accumulator layout: lane (c, g) holds
// rows 16 rt + 4 g .. + 3 of column c). The state is exchanged through LDS transposed
// (column c at x_t + c * kScanPitch), so that a lane reads its four rows of a k-tile with one
// 16-byte read. k-step (t, s) of a tile product has lane (., g) supply contraction index
// 16 t + 4 g + s on both sides; over t = 0..7 and s = 0..3 that covers each of the 128 once.
// Each step's M_p fragments are loaded during the previous step's products.
constexpr int kScanPitch = 128 + 4;
typedef float f32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4s mfma_f32_4(float a, float b, f32x4s c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The fragments of M_p (forward) or M_p^T (reverse) of rows 32 w .. + 31 for k-tile t:
// element s of m[rt][t] is M_p[16 (2w + rt) + l16][16 t + 4 g + s] (forward) or
// M_p[16 t + 4 g + s][16 (2w + rt) + l16] (reverse).
template <bool kTrans>
__device__ __forceinline__ void scan_load_m(const float* Mp, int wave, int l16, int g4, f32x4s (&m)[2][8]) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int row = 16 * (2 * wave + rt) + l16;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (!kTrans) {
                m[rt][t] = *reinterpret_cast<const f32x4s*>(Mp + row * 128 + 16 * t + 4 * g4);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) m[rt][t][e] = Mp[(16 * t + 4 * g4 + e) * 128 + row];
            }
        }
    }
}

// acc[rt] += (M_p or M_p^T) X for the wave's two row tiles, X^T in LDS
__device__ __forceinline__ void scan_products(const float* x_t, int l16, int g4, const f32x4s (&m)[2][8],
                                              f32x4s (&acc)[2]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const f32x4s xb = *reinterpret_cast<const f32x4s*>(x_t + l16 * kScanPitch + 16 * t + 4 * g4);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) acc[rt] = mfma_f32_4(m[rt][t][s], xb[s], acc[rt]);
    }
}

// XCD-aware block order of the scans (workgroups go round-robin over the 8 XCDs): the
// 16-column tiles of one (b, h) run on one XCD, so that its L2 reads each M_p from memory
// once for all of them. Returns false for the padding blocks of the last group.
__device__ __forceinline__ bool scan_block(int ntiles, int nbh, int& tile, int& bhi) {
    const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
    tile = slot % ntiles;
    bhi = (slot / ntiles) * 8 + xcd;
    return bhi < nbh;
}

__global__ __launch_bounds__(256) void affine_scan_mfma(ScanArgs a) {
    __shared__ __align__(16) float x_t[16 * kScanPitch];
    const int ncols = a.ncols;
    int ct, bhi;
    if (!scan_block(ncols / 16, a.B * a.H, ct, bhi)) return;
    const int col0 = 16 * ct;
    const int64_t bh = bhi;
    const int64_t tile = static_cast<int64_t>(128) * ncols;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    for (int e = tid; e < 128 * 16; e += 256) {
        const int i = e >> 4, c = e & 15;
        float x0 = 0.f;
        if (a.init_mode == kInitLoad) x0 = a.init[bh * tile + static_cast<int64_t>(i) * ncols + col0 + c];
        else if (a.init_mode == kInitIdentity) x0 = (i == col0 + c) ? 1.f : 0.f;
        x_t[c * kScanPitch + i] = x0;
    }
    f32x4s m[2][8], mn[2][8];
    if (a.P > 0) scan_load_m<false>(a.M + bh * a.P * 128 * 128, wave, l16, g4, m);
    __syncthreads();
    for (int p = 0; p < a.P; ++p) {
        // the next step's fragments are in flight during this step's products
        if (p + 1 < a.P) scan_load_m<false>(a.M + (bh * a.P + p + 1) * 128 * 128, wave, l16, g4, mn);
        const int64_t blk = bh * a.P + p;
        // S_p is added after the products, so that its loads are in flight during them
        f32x4s acc[2], sv[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row0 = 16 * (2 * wave + rt) + 4 * g4;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sv[rt][j] = a.S ? a.S[blk * tile + static_cast<int64_t>(row0 + j) * ncols + col0 + l16] : 0.f;
            if (a.x_before) {
                const f32x4s xo = *reinterpret_cast<const f32x4s*>(x_t + l16 * kScanPitch + row0);
#pragma unroll
                for (int j = 0; j < 4; ++j) a.x_before[blk * tile + static_cast<int64_t>(row0 + j) * ncols + col0 + l16] = xo[j];
            }
            acc[rt] = f32x4s{0.f, 0.f, 0.f, 0.f};
        }
        scan_products(x_t, l16, g4, m, acc);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[rt] += sv[rt];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int t = 0; t < 8; ++t) m[rt][t] = mn[rt][t];
        __syncthreads();   // every read of X_{p-1} is done
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row0 = 16 * (2 * wave + rt) + 4 * g4;
            *reinterpret_cast<f32x4s*>(x_t + l16 * kScanPitch + row0) = acc[rt];
            if (a.x_after)
#pragma unroll
                for (int j = 0; j < 4; ++j) a.x_after[blk * tile + static_cast<int64_t>(row0 + j) * ncols + col0 + l16] = acc[rt][j];
        }
        __syncthreads();
    }
    if (a.x_final)
        for (int e = tid; e < 128 * 16; e += 256) {
            const int i = e >> 4, c = e & 15;
            a.x_final[bh * tile + static_cast<int64_t>(i) * ncols + col0 + c] = x_t[c * kScanPitch + i];
        }
}

__global__ __launch_bounds__(256) void affine_scan_rev_mfma(ScanBwdArgs a) {
    __shared__ __align__(16) float x_t[16 * kScanPitch];
    const int dv = a.dv;
    int ct, bhi;
    if (!scan_block(dv / 16, a.B * a.H, ct, bhi)) return;
    const int col0 = 16 * ct;
    const int64_t bh = bhi;
    const int64_t tile = static_cast<int64_t>(128) * dv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    for (int e = tid; e < 128 * 16; e += 256) {
        const int i = e >> 4, c = e & 15;
        x_t[c * kScanPitch + i] = a.dhT ? a.dhT[bh * tile + static_cast<int64_t>(i) * dv + col0 + c] : 0.f;
    }
    f32x4s m[2][8], mn[2][8];
    if (a.P > 0) scan_load_m<true>(a.M + (bh * a.P + a.P - 1) * 128 * 128, wave, l16, g4, m);
    __syncthreads();
    for (int p = a.P - 1; p >= 0; --p) {
        if (p > 0) scan_load_m<true>(a.M + (bh * a.P + p - 1) * 128 * 128, wave, l16, g4, mn);
        const int64_t blk = bh * a.P + p;
        // dH_in_p is added after the products, so that its loads are in flight during them
        f32x4s acc[2], dv_in[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row0 = 16 * (2 * wave + rt) + 4 * g4;
            const f32x4s go = *reinterpret_cast<const f32x4s*>(x_t + l16 * kScanPitch + row0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t o = blk * tile + static_cast<int64_t>(row0 + j) * dv + col0 + l16;
                dv_in[rt][j] = a.dH_in[o];
                a.dS[o] = go[j];
            }
            acc[rt] = f32x4s{0.f, 0.f, 0.f, 0.f};
        }
        scan_products(x_t, l16, g4, m, acc);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[rt] += dv_in[rt];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int t = 0; t < 8; ++t) m[rt][t] = mn[rt][t];
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            *reinterpret_cast<f32x4s*>(x_t + l16 * kScanPitch + 16 * (2 * wave + rt) + 4 * g4) = acc[rt];
        __syncthreads();
    }
    if (a.dh0)
        for (int e = tid; e < 128 * 16; e += 256) {
            const int i = e >> 4, c = e & 15;
            a.dh0[bh * tile + static_cast<int64_t>(i) * dv + col0 + c] = x_t[c * kScanPitch + i];
        }
}

// dM_p = dS_p H_in_p^T, one block per (16 rows of dM, (b, h, p)): the block's 16 rows of
// dS_p and all of H_in_p in LDS (fp32), thread (r, j0) sums over the dv columns for the
// outputs (r, j0 + 16 u).
__global__ __launch_bounds__(256) void summary_outer(ScanBwdArgs a) {
    __shared__ float sm[(16 + 128) * 129];
    const int dk = a.dk, dv = a.dv, pitch = dv + 1;
    float* ds_s = sm;                 // [16][dv + 1]
    float* hi_s = sm + 16 * pitch;    // [dk][dv + 1]
    const int r0 = 16 * blockIdx.y;
    const int64_t blk = blockIdx.x;   // (b h) P + p
    const float* dS = a.dS + blk * static_cast<int64_t>(dk) * dv;
    const float* Hi = a.H_in + blk * static_cast<int64_t>(dk) * dv;
    const int tid = threadIdx.x;
    for (int e = tid; e < 16 * dv; e += 256) ds_s[(e / dv) * pitch + e % dv] = dS[static_cast<int64_t>(r0) * dv + e];
    for (int e = tid; e < dk * dv; e += 256) hi_s[(e / dv) * pitch + e % dv] = Hi[e];
    __syncthreads();
    const int r = tid >> 4, j0 = tid & 15;
    for (int j = j0; j < dk; j += 16) {
        float acc = 0.f;
        for (int c = 0; c < dv; ++c) acc += ds_s[r * pitch + c] * hi_s[j * pitch + c];
        a.dM[blk * static_cast<int64_t>(dk) * dk + static_cast<int64_t>(r0 + r) * dk + j] = acc;
    }
}

// dM_p = dS_p H_in_p^T for dk = dv = 128 on v_mfma_f32_16x16x4_f32: one block of eight
// waves per (b, h, p); H_in_p is staged in LDS (rows at a pitch of 132 floats) and wave w
// forms the 16 x 128 row tile w of dM_p. k-step (t, s) has lane (., g) supply dv index
// 16 t + 4 g + s of both operands, each read as 16 contiguous bytes of a row of dS_p or
// H_in_p.
__global__ __launch_bounds__(512) void summary_outer_mfma(ScanBwdArgs a) {
    __shared__ __align__(16) float hi_s[128 * kScanPitch];
    const int64_t blk = blockIdx.x;   // (b h) P + p
    const float* dS = a.dS + blk * 128 * 128;
    const float* Hi = a.H_in + blk * 128 * 128;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    f32x4s af[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) af[t] = *reinterpret_cast<const f32x4s*>(dS + (16 * wave + l16) * 128 + 16 * t + 4 * g4);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int e = tid + 512 * u, row = e >> 5, c4 = e & 31;
        *reinterpret_cast<f32x4s*>(hi_s + row * kScanPitch + 4 * c4) = *reinterpret_cast<const f32x4s*>(Hi + row * 128 + 4 * c4);
    }
    __syncthreads();
    for (int jt = 0; jt < 8; ++jt) {
        f32x4s acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4s bf = *reinterpret_cast<const f32x4s*>(hi_s + (16 * jt + l16) * kScanPitch + 16 * t + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_f32_4(af[t][s], bf[s], acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) a.dM[blk * 128 * 128 + (16 * wave + 4 * g4 + j) * 128 + 16 * jt + l16] = acc[j];
    }
}

// The state pass for fp32 inputs with dk = 128 on v_mfma_f32_16x16x4_f32 (fp32 products,
// fp32 accumulation): one block of eight waves per (b, h, segment, 16 state columns), the
// column tiles of one (b, h, segment) on one XCD (the order of the scans above). Computing
// wave w (0-3) keeps rows 32 w .. 32 w + 31 of the state in two accumulator tiles and owns
// token tile w (tokens 16 w .. 16 w + 15) of every chunk:
//   P1  K S and Q S of its tokens over all 128 state rows (the state read back from LDS,
//       transposed), X = V - e^Gam K S;
//   P2  U = That X over the token tiles up to its own (X exchanged through LDS);
//   P3  O = e^Gam Q S + P U (U through LDS), and its state rows
//       S <- e^{Gam_C} S + K^T (e^{Gam_C - Gam} U), the K^T fragments read as single floats
//       from the row-major K tile (conflict-free at a pitch of 132 floats).
// Three barriers per chunk. Waves 4-7 stage every operand in LDS, so that the computing
// waves issue no load (a CU's load path accepts a chunk's ~100 KiB more slowly than the
// products take, and a wave stalls while its loads issue): the next chunk's K and Q are
// loaded while P1 runs; its That, V, P and decay factors after the first barrier; Q is
// written after the first barrier (P1 has read this chunk's), That, V, K and the decay
// factors after the second (P2 has read That), P at the start of the next chunk (P3 has
// read this one's). K and the decay factors have two buffers; padded tokens' K and V are
// zero. Each k-tile's LDS operands are read during the previous one's products, and the
// scheduling barriers pin that order. k-step s of a 16x16x4 product has lane (l16, g4)
// supply contraction index 4 g4 + s of a 16-wide slice, so that one 16-byte LDS read gives
// a lane its operand for four steps.
constexpr int kRawBufferWord3 = 0x00020000;   // raw buffer descriptor word 3 on gfx9-family GPUs

template <bool kOut>
__global__ __launch_bounds__(512) void state_f32mfma(StateArgs a) {
    constexpr int KPf = 132, TP = 68, KQT = 64 * KPf;
    __shared__ __align__(16) float k_s[2 * KQT];
    __shared__ __align__(16) float q_s[kOut ? KQT : 4];
    __shared__ __align__(16) float t_s[64 * TP];           // That, row-major
    __shared__ __align__(16) float p_s[kOut ? 64 * TP : 4];  // P, row-major
    __shared__ __align__(16) float v_t[16 * TP];           // V transposed: V[t][c] at c TP + t
    __shared__ __align__(16) float g_s[2 * 128];           // e^Gam, e^{Gam_C - Gam}
    __shared__ __align__(16) float s_t[16 * KPf];          // the state transposed: S[i][c] at c KPf + i
    __shared__ __align__(16) float x_t[16 * TP];           // X, U and e^{Gam_C - Gam} U transposed
    __shared__ __align__(16) float u_t[16 * TP];
    __shared__ __align__(16) float ug_t[16 * TP];

    const int ncols = a.ncols;
    int ct, bhi;
    if (!scan_block(ncols / 16, a.B * a.P * a.H, ct, bhi)) return;
    const int h = bhi % a.H, bz = bhi / a.H, b = bz / a.P, seg = bz % a.P;
    const int col0 = 16 * ct;
    const int hq = h / (a.H / a.Hqk);
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0-3 compute, 4-7 stage operands
    const bool loader = w >= 4;
    const int ltid = tid & 255;
    const RowSpan rs = row_span(a.cu_seqlens, a.valid_len, b, a.T, a.NT);
    const int64_t nvalid = rs.valid;
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* o = static_cast<float*>(a.o);
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int64_t tile = static_cast<int64_t>(128) * ncols;
    const f32x4s zero = {0.f, 0.f, 0.f, 0.f};
    const int n0 = seg * a.Lc;
    const int n1 = min(min(n0 + a.Lc, a.NT), static_cast<int>((rs.extent + kChunk - 1) / kChunk));

    if (loader) {
        // float4 m of K and Q is row (ltid + 256 m) / 32, columns 4 ((ltid + 256 m) % 32) .. + 3,
        // loaded through a descriptor per chunk that ends at the chunk's last valid row (rows
        // past it read as zero; the whole offset is in the vector offset, which the range
        // check covers). float4 m of That and P is row (ltid + 256 m) / 16, columns
        // 4 ((ltid + 256 m) % 16) .. + 3; of V, token ltid / 4, columns 4 (ltid % 4) .. + 3.
        f32x4s kr[8], qr[8], tr[4], pr[4], vr, gr;
        const int64_t qk_row = static_cast<int64_t>(a.Hqk) * 128;
        const uint32_t kq_voff = static_cast<uint32_t>(((ltid >> 5) * qk_row + 4 * (ltid & 31)) * 4);
        const auto kq_rsrc = [&](const float* base, int64_t t0) {
            const int64_t rows = nvalid - t0 < 0 ? 0 : (nvalid - t0 > 64 ? 64 : nvalid - t0);
            const int64_t bytes = rows > 0 ? ((rows - 1) * qk_row + 128) * 4 : 0;
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base + ((rs.start + t0) * a.Hqk + hq) * 128), 0,
                                                     static_cast<int32_t>(bytes), kRawBufferWord3);
        };
        const auto load_kq = [&](int n) {
            const int64_t t0 = static_cast<int64_t>(n) * kChunk;
            const __amdgpu_buffer_rsrc_t rk = kq_rsrc(k, t0), rq = kq_rsrc(q, t0);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint32_t off = kq_voff + static_cast<uint32_t>(m * 8 * qk_row * 4);
                kr[m] = __builtin_bit_cast(f32x4s, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
                if constexpr (kOut)
                    qr[m] = __builtin_bit_cast(f32x4s, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
            }
        };
        const auto load_rest = [&](int n) {
            const int64_t t0 = static_cast<int64_t>(n) * kChunk;
            const int64_t ch = bh * a.NT + n;
            const float* tg = static_cast<const float*>(a.ws.that) + ch * 4096;
            const float* pg = static_cast<const float*>(a.ws.pmat) + ch * 4096;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                tr[m] = *reinterpret_cast<const f32x4s*>(tg + 4 * (ltid + 256 * m));
                if constexpr (kOut) pr[m] = *reinterpret_cast<const f32x4s*>(pg + 4 * (ltid + 256 * m));
            }
            const int64_t tok = t0 + (ltid >> 2);
            const int64_t tcl = tok < nvalid ? tok : 0;
            vr = v ? *reinterpret_cast<const f32x4s*>(v + ((rs.start + tcl) * a.H + h) * ncols + col0 + 4 * (ltid & 3))
                   : zero;
            if (ltid < 32) gr = *reinterpret_cast<const f32x4s*>(a.ws.gates + ch * 128 + 4 * ltid);
        };
        const auto store_q = [&]() {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int e = ltid + 256 * m;
                if constexpr (kOut) *reinterpret_cast<f32x4s*>(q_s + (e >> 5) * KPf + 4 * (e & 31)) = qr[m];
            }
        };
        // That, V (padded tokens zero) of chunk n, its K and decay factors into buffer buf
        const auto store_tvkg = [&](int n, int buf) {
            const int64_t t0 = static_cast<int64_t>(n) * kChunk;
            float* kb = k_s + buf * KQT;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e = ltid + 256 * m;
                *reinterpret_cast<f32x4s*>(t_s + (e >> 4) * TP + 4 * (e & 15)) = tr[m];
            }
            const int tk = ltid >> 2, c4 = 4 * (ltid & 3);
            const f32x4s vv = t0 + tk < nvalid ? vr : zero;
#pragma unroll
            for (int i = 0; i < 4; ++i) v_t[(c4 + i) * TP + tk] = vv[i];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int e = ltid + 256 * m;
                *reinterpret_cast<f32x4s*>(kb + (e >> 5) * KPf + 4 * (e & 31)) = kr[m];
            }
            if (ltid < 32) *reinterpret_cast<f32x4s*>(g_s + buf * 128 + 4 * ltid) = gr;
        };
        const auto store_p = [&]() {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e = ltid + 256 * m;
                if constexpr (kOut) *reinterpret_cast<f32x4s*>(p_s + (e >> 4) * TP + 4 * (e & 15)) = pr[m];
            }
        };
        if (n0 < n1) {
            load_kq(n0);
            load_rest(n0);
            store_q();
            store_tvkg(n0, n0 & 1);
        }
        __syncthreads();
        // three barriers per chunk, as the computing waves below (the last chunk re-fetches
        // itself where a later one is due; nobody reads what it stores)
        for (int n = n0; n < n1; ++n) {
            const int nf = n + 1 < n1 ? n + 1 : n;
            store_p();                       // this chunk's P (loaded during the previous one)
            load_kq(nf);
            __syncthreads();
            store_q();
            load_rest(nf);
            __syncthreads();
            store_tvkg(nf, (n + 1) & 1);
            __syncthreads();
        }
        return;
    }

    f32x4s st[2];   // state rows 32 w + 16 rt + 4 g4 + j, column col0 + l16
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = 32 * w + 16 * rt + 4 * g4 + j;
            float s0 = 0.f;
            if (a.init_mode == kInitLoad) {
                const int64_t blk = a.s_init_per_segment ? bh * a.P + seg : bh;
                s0 = a.s_init[blk * tile + static_cast<int64_t>(i) * ncols + col0 + l16];
            } else if (a.init_mode == kInitIdentity) {
                s0 = (i == col0 + l16) ? 1.f : 0.f;
            }
            st[rt][j] = s0;
        }
        *reinterpret_cast<f32x4s*>(s_t + l16 * KPf + 32 * w + 16 * rt + 4 * g4) = st[rt];
    }
    __syncthreads();

    for (int n = n0; n < n1; ++n) {
        const int64_t t0 = static_cast<int64_t>(n) * kChunk;
        const float* kb = k_s + (n & 1) * KQT;
        const float* gb_s = g_s + (n & 1) * 128;
        const f32x4s egv = *reinterpret_cast<const f32x4s*>(gb_s + 16 * w + 4 * g4);

        // P1: K S and Q S of token tile w; even and odd k-tiles accumulate in separate chains
        f32x4s ks2[2] = {zero, zero}, qs2[2] = {zero, zero};
        f32x4s sb[2], ka[2], qa[2];
        const auto rd1 = [&](int t, int i) {
            sb[i] = *reinterpret_cast<const f32x4s*>(s_t + l16 * KPf + 16 * t + 4 * g4);
            ka[i] = *reinterpret_cast<const f32x4s*>(kb + (16 * w + l16) * KPf + 16 * t + 4 * g4);
            if constexpr (kOut) qa[i] = *reinterpret_cast<const f32x4s*>(q_s + (16 * w + l16) * KPf + 16 * t + 4 * g4);
        };
        rd1(0, 0);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int i = t & 1;
            if (t + 1 < 8) rd1(t + 1, i ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ks2[i] = mfma_f32_4(ka[i][s], sb[i][s], ks2[i]);
                if constexpr (kOut) qs2[i] = mfma_f32_4(qa[i][s], sb[i][s], qs2[i]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const f32x4s ks = ks2[0] + ks2[1], qs = qs2[0] + qs2[1];
        const f32x4s vc = *reinterpret_cast<const f32x4s*>(v_t + l16 * TP + 16 * w + 4 * g4);
        *reinterpret_cast<f32x4s*>(x_t + l16 * TP + 16 * w + 4 * g4) = vc - egv * ks;
        __syncthreads();

        // P2: U of token tile w (the products stop at w; even and odd token tiles in two chains)
        f32x4s u2[2] = {zero, zero}, xb[4], tc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xb[r] = *reinterpret_cast<const f32x4s*>(x_t + l16 * TP + 16 * r + 4 * g4);
            tc[r] = *reinterpret_cast<const f32x4s*>(t_s + (16 * w + l16) * TP + 16 * r + 4 * g4);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r <= w) {
#pragma unroll
                for (int s = 0; s < 4; ++s) u2[r & 1] = mfma_f32_4(tc[r][s], xb[r][s], u2[r & 1]);
            }
        }
        const f32x4s u = u2[0] + u2[1];
        const f32x4s egcv = *reinterpret_cast<const f32x4s*>(gb_s + 64 + 16 * w + 4 * g4);
        *reinterpret_cast<f32x4s*>(u_t + l16 * TP + 16 * w + 4 * g4) = u;
        *reinterpret_cast<f32x4s*>(ug_t + l16 * TP + 16 * w + 4 * g4) = egcv * u;
        __syncthreads();

        // P3: the output of token tile w
        f32x4s ov = zero;
        if constexpr (kOut) {
            f32x4s ov2[2] = {egv * qs, zero}, ub[4], pc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ub[r] = *reinterpret_cast<const f32x4s*>(u_t + l16 * TP + 16 * r + 4 * g4);
                pc[r] = *reinterpret_cast<const f32x4s*>(p_s + (16 * w + l16) * TP + 16 * r + 4 * g4);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (r <= w) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) ov2[r & 1] = mfma_f32_4(pc[r][s], ub[r][s], ov2[r & 1]);
                }
            }
            ov = ov2[0] + ov2[1];
        }

        // the state rows of the wave; each token tile's K^T values and scaled U are read
        // during the previous tile's products; even and odd token tiles in separate chains
        const float egCn = gb_s[63];
        f32x4s sto[2] = {zero, zero};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) st[rt] *= egCn;
        float kt[2][8];
        f32x4s gb[2];
        const auto rd3 = [&](int r, int i) {
            gb[i] = *reinterpret_cast<const f32x4s*>(ug_t + l16 * TP + 16 * r + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float* kc = kb + (16 * r + 4 * g4 + s) * KPf + 32 * w + l16;
                kt[i][2 * s] = kc[0];
                kt[i][2 * s + 1] = kc[16];
            }
        };
        rd3(0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = r & 1;
            if (r + 1 < 4) rd3(r + 1, i ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    if (i == 0) st[rt] = mfma_f32_4(kt[i][2 * s + rt], gb[i][s], st[rt]);
                    else sto[rt] = mfma_f32_4(kt[i][2 * s + rt], gb[i][s], sto[rt]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            st[rt] += sto[rt];
            *reinterpret_cast<f32x4s*>(s_t + l16 * KPf + 32 * w + 16 * rt + 4 * g4) = st[rt];
        }
        if constexpr (kOut) {
            // unconditional stores through a descriptor that ends at the row's last token
            // (stores past it are dropped)
            const int64_t trow = static_cast<int64_t>(a.H) * ncols;
            const int64_t left = rs.extent - t0;
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                o + (rs.start + t0) * trow, 0, static_cast<int32_t>((left < 64 ? left : 64) * trow * 4),
                kRawBufferWord3);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * w + 4 * g4 + j;
                const float x = t0 + row < nvalid ? ov[j] : 0.f;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), ro,
                                                      static_cast<uint32_t>((row * trow + h * ncols + col0 + l16) * 4), 0, 0);
            }
        }
        __syncthreads();
    }

    if (a.store_mode == kStoreNone) return;
    if (a.store_mode == kStoreLastSegment && seg != a.P - 1) return;
    const int64_t blk = (a.store_mode == kStoreEverySegment) ? bh * a.P + seg : bh;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            a.s_out[blk * tile + static_cast<int64_t>(32 * w + 16 * rt + 4 * g4 + j) * ncols + col0 + l16] = st[rt][j];
}

// The prepare pass for fp32 inputs with dk = 128 on v_mfma_f32_16x16x4_f32: one block of
// four waves per (b, h, chunk), chunk-major with the heads of one chunk back to back on one
// XCD (its L2 serves the q/k rows the value heads of a query/key head share). It writes the
// records of prep_f32path: That = (I + A)^{-1} diag(beta) and P (64 x 64 fp32, row-major,
// zero above the diagonal) and the decay factors.
//   Gram products: the ten lower 16x16 tiles of K K^T and of Q K^T, five per wave, over the
//   128 columns in two halves of 64 (K and Q halves in LDS, 16-byte granules XOR-swizzled by
//   the row so that the fragment reads of 16 consecutive rows are conflict-free; the second
//   half is loaded into registers during the first half's products, and the halves keep the
//   LDS at 45 KiB, three blocks per CU); A = beta_i e^{Gam_i - Gam_j}
//   (K K^T)_ij below the diagonal into LDS, P = e^{Gam_i - Gam_j} (Q K^T)_ij on and below it
//   to memory.
//   Solve: the four diagonal blocks D_b = (I + A_bb)^{-1} by column sweep on one wave (lane =
//   (block, column)); the blocks below them T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj as three
//   per-wave chains of 16x16x16 products (T10 T20 T30 / T21 T31 / T32), each result kept in
//   accumulators and entering the next product as its B operand.
__device__ __forceinline__ int kq_slot(int r, int c4) { return r * 64 + 4 * (c4 ^ (r & 15)); }

__global__ __launch_bounds__(256) void prep_f32mfma(PrepArgs a) {
    constexpr int BP = 20;           // pitch of the 16x16 blocks in LDS (16-byte aligned rows)
    constexpr int BS = 16 * BP;      // floats per block
    __shared__ __align__(16) float kq_s[2 * 64 * 64];    // a half of K and of Q; later the diagonal inverses
    __shared__ __align__(16) float a_s[10 * BS];          // the lower blocks of A, (i, j) at i (i + 1) / 2 + j
    __shared__ float gam_s[64], beta_s[64];
    float* k_s = kq_s;
    float* q_s = kq_s + 64 * 64;
    float* dr_s = kq_s;              // D_b row-major (after the Gram products)
    float* dc_s = kq_s + 4 * BS;     // D_b transposed

    const int64_t L = blockIdx.x;
    const int xcd = static_cast<int>(L & 7);
    const int64_t u = L >> 3;
    const int h = static_cast<int>(u % a.H);
    const int64_t pair = (u / a.H) * 8 + xcd;
    if (pair >= static_cast<int64_t>(a.B) * a.NT) return;
    const int b = static_cast<int>(pair / a.NT), n = static_cast<int>(pair % a.NT);
    const int64_t ch = (static_cast<int64_t>(b) * a.H + h) * a.NT + n;
    const int hq = h / (a.H / a.Hqk);
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(n) * kChunk;
    const RowSpan rs = row_span(a.cu_seqlens, a.valid_len, b, a.T, a.NT);
    const float* kin = static_cast<const float*>(a.k);
    const float* qin = static_cast<const float*>(a.q);
    float* that = static_cast<float*>(a.ws.that) + ch * 4096;
    float* pm = static_cast<float*>(a.ws.pmat) + ch * 4096;
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const f32x4v zero = {0.f, 0.f, 0.f, 0.f};

    // K and Q rows (zero past the valid length) in two halves of 64 columns: float4 m of a
    // half is row (tid + 256 m) / 16, columns 4 ((tid + 256 m) % 16) .. + 3 of the half
    f32x4v kh[4], qh[4];
    const auto load_half = [&](int half) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 256 * m, rr = e >> 4;
            const bool ok = t0 + rr < rs.valid;
            const int64_t idx = ((rs.start + (ok ? t0 + rr : 0)) * a.Hqk + hq) * 128 + 64 * half + 4 * (e & 15);
            kh[m] = *reinterpret_cast<const f32x4v*>(kin + idx);
            qh[m] = *reinterpret_cast<const f32x4v*>(qin + idx);
        }
    };
    const auto store_half = [&]() {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 256 * m, rr = e >> 4, c4 = e & 15;
            const bool ok = t0 + rr < rs.valid;
            *reinterpret_cast<f32x4v*>(k_s + kq_slot(rr, c4)) = ok ? kh[m] : zero;
            *reinterpret_cast<f32x4v*>(q_s + kq_slot(rr, c4)) = ok ? qh[m] : zero;
        }
    };
    load_half(0);
    store_half();
    load_half(1);
    if (w == 0) {
        const bool ok = t0 + lane < rs.valid;
        const int64_t gi = (rs.start + (ok ? t0 + lane : 0)) * a.H + h;
        const float gv = a.g[gi], bv = a.beta[gi];
        float gam = ok ? gv : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gam, off, 64);
            if (lane >= off) gam += y;
        }
        gam_s[lane] = gam;
        beta_s[lane] = ok ? bv : 0.f;
        // decay factors e^{Gam_t} and e^{Gam_C - Gam_t}
        const float gam_c = __shfl(gam, 63, 64);
        a.ws.gates[ch * 128 + lane] = expf(gam);
        a.ws.gates[ch * 128 + 64 + lane] = expf(gam_c - gam);
    }
    // the blocks above the diagonal of That and P are zero
    for (int e = tid; e < 6 * 64; e += 256) {
        // block (i, j), i < j, element quad e % 64: rows 16 i + (e % 64) / 4, columns 16 j + 4 (e % 4)
        const int blk = e >> 6, qd = e & 63;
        const int i = blk < 3 ? 0 : (blk < 5 ? 1 : 2), j = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        const int off = (16 * i + (qd >> 2)) * 64 + 16 * j + 4 * (qd & 3);
        *reinterpret_cast<f32x4v*>(that + off) = zero;
        *reinterpret_cast<f32x4v*>(pm + off) = zero;
    }
    __syncthreads();

    // ---- Gram products: tile item w + 4 v of [K K^T lower tiles, Q K^T lower tiles], each
    // over the two halves of the columns; even and odd k-tiles in separate chains ----
    f32x4v acc2[5][2];
#pragma unroll
    for (int v = 0; v < 5; ++v) acc2[v][0] = acc2[v][1] = zero;
    const auto gram_half = [&]() {
#pragma unroll
        for (int v = 0; v < 5; ++v) {
            const int item = w + 4 * v;
            const int li = item < 10 ? item : item - 10;
            const int bi = li == 0 ? 0 : (li < 3 ? 1 : (li < 6 ? 2 : 3));
            const int bj = li - bi * (bi + 1) / 2;
            const float* left = item < 10 ? k_s : q_s;
            const int ra = 16 * bi + l16, rb = 16 * bj + l16;
            f32x4v fa[2], fb[2];
            fa[0] = *reinterpret_cast<const f32x4v*>(left + kq_slot(ra, g4));
            fb[0] = *reinterpret_cast<const f32x4v*>(k_s + kq_slot(rb, g4));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = t & 1;
                if (t + 1 < 4) {
                    fa[i ^ 1] = *reinterpret_cast<const f32x4v*>(left + kq_slot(ra, 4 * (t + 1) + g4));
                    fb[i ^ 1] = *reinterpret_cast<const f32x4v*>(k_s + kq_slot(rb, 4 * (t + 1) + g4));
                }
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) acc2[v][i] = mfma_f32_4(fa[i][s2], fb[i][s2], acc2[v][i]);
            }
        }
    };
    gram_half();
    __syncthreads();   // every read of the first half is done
    store_half();
    __syncthreads();
    gram_half();
#pragma unroll
    for (int v = 0; v < 5; ++v) {
        const int item = w + 4 * v;
        const int li = item < 10 ? item : item - 10;
        const int bi = li == 0 ? 0 : (li < 3 ? 1 : (li < 6 ? 2 : 3));
        const int bj = li - bi * (bi + 1) / 2;
        const f32x4v acc = acc2[v][0] + acc2[v][1];
        const int jc = 16 * bj + l16;
        const float gj = gam_s[jc];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ii = 16 * bi + 4 * g4 + r;
            const float d = gam_s[ii] - gj;
            const float dec = expf(d < 0.f ? d : 0.f);
            if (item < 10) a_s[li * BS + (4 * g4 + r) * BP + l16] = ii > jc ? beta_s[ii] * dec * acc[r] : 0.f;
            else pm[ii * 64 + jc] = ii >= jc ? dec * acc[r] : 0.f;
        }
    }
    __syncthreads();

    // ---- the diagonal blocks: lane (blk, c) sweeps column c of (I + A_bb)^{-1} ----
    if (w == 0) {
        const int blk = lane >> 4, c = l16;
        const float* ab = a_s + (blk * (blk + 1) / 2 + blk) * BS;
        float tcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = r == c ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc -= ab[r * BP + j] * tcol[j];
            tcol[r] = acc;
        }
        const float bc = beta_s[16 * blk + c];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dr_s[blk * BS + r * BP + c] = tcol[r];
            that[(16 * blk + r) * 64 + 16 * blk + c] = tcol[r] * bc;
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<f32x4v*>(dc_s + blk * BS + c * BP + 4 * r4) =
                f32x4v{tcol[4 * r4], tcol[4 * r4 + 1], tcol[4 * r4 + 2], tcol[4 * r4 + 3]};
    }
    __syncthreads();

    // ---- the blocks below the diagonal ----
    if (w < 3) {
        // A operand: rows l16 of a row-major block, columns 4 g4 .. + 3; B operand from a
        // transposed block: its rows 4 g4 .. + 3 of column l16
        const auto fr = [&](const float* blk) { return *reinterpret_cast<const f32x4v*>(blk + l16 * BP + 4 * g4); };
        const auto mm = [&](const f32x4v& x, const f32x4v& y, f32x4v acc) {
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) acc = mfma_f32_4(x[s2], y[s2], acc);
            return acc;
        };
        const auto ablk = [&](int i, int j) { return a_s + (i * (i + 1) / 2 + j) * BS; };
        const auto put = [&](int i, int j, const f32x4v& tv) {
            const float bc = beta_s[16 * j + l16];
#pragma unroll
            for (int r = 0; r < 4; ++r) that[(16 * i + 4 * g4 + r) * 64 + 16 * j + l16] = tv[r] * bc;
        };
        const int j0 = w;                      // the chain of column block w
        // T_{j0+1, j0} = -D_{j0+1} A_{j0+1, j0} D_{j0}
        f32x4v tprev[3];
        f32x4v y = mm(fr(ablk(j0 + 1, j0)), fr(dc_s + j0 * BS), zero);
        tprev[0] = -mm(fr(dr_s + (j0 + 1) * BS), y, zero);
        put(j0 + 1, j0, tprev[0]);
        // T_{i, j0} = -D_i (A_{i, j0} D_{j0} + sum_{k = j0+1}^{i-1} A_{i, k} T_{k, j0})
#pragma unroll
        for (int i = 2; i < 4; ++i) {
            if (i > j0 + 1) {
                y = mm(fr(ablk(i, j0)), fr(dc_s + j0 * BS), zero);
#pragma unroll
                for (int kk = 1; kk < 3; ++kk)
                    if (j0 + kk < i) y = mm(fr(ablk(i, j0 + kk)), tprev[kk - 1], y);
                tprev[i - j0 - 1] = -mm(fr(dr_s + i * BS), y, zero);
                put(i, j0, tprev[i - j0 - 1]);
            }
        }
    }
}

template <typename IO>
hipError_t prep_dispatch(const PrepArgs& a, hipStream_t s) {
    if constexpr (sizeof(IO) == 4) {
        if (a.dk == 128) {
            // fp32 matrix cores; (b, chunk) groups of 8 x the heads
            const int64_t pairs = static_cast<int64_t>(a.B) * a.NT;
            const dim3 grid(static_cast<unsigned>((pairs + 7) / 8 * 8 * a.H));
            void* args[] = {const_cast<PrepArgs*>(&a)};
            return hipLaunchKernel(reinterpret_cast<const void*>(&prep_f32mfma), grid, dim3(256), args, 0, s);
        }
    }
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.H * a.NT));
    void* args[] = {const_cast<PrepArgs*>(&a)};
    const void* fn = nullptr;
    switch (a.dk) {
        case 16: fn = reinterpret_cast<const void*>(&prep_f32path<IO, 16>); break;
        case 32: fn = reinterpret_cast<const void*>(&prep_f32path<IO, 32>); break;
        case 64: fn = reinterpret_cast<const void*>(&prep_f32path<IO, 64>); break;
        case 128: fn = reinterpret_cast<const void*>(&prep_f32path<IO, 128>); break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, grid, dim3(128), args, 0, s);
}

// Columns per thread of the state pass: 2 (512-thread blocks, two waves per SIMD) against
// 4 and 1: 1.93 / 2.17 / 2.10 ms for bf16 heads of 64 at 8K tokens and 32 heads.
constexpr int kStateCpt = 2;

template <typename IO>
hipError_t state_dispatch(const StateArgs& a, hipStream_t s) {
    void* args[] = {const_cast<StateArgs*>(&a)};
    if constexpr (sizeof(IO) == 4) {
        if (a.dk == 128) {
            // fp32 matrix cores; blocks in the scans' XCD-aware order over (b, segment, h)
            const int64_t groups = (static_cast<int64_t>(a.B) * a.P * a.H + 7) / 8;
            const dim3 grid(static_cast<unsigned>(groups * 8 * (a.ncols / 16)));
            const void* fn = a.o ? reinterpret_cast<const void*>(&state_f32mfma<true>)
                                 : reinterpret_cast<const void*>(&state_f32mfma<false>);
            return hipLaunchKernel(fn, grid, dim3(512), args, 0, s);
        }
    }
    const dim3 grid(static_cast<unsigned>(a.ncols / 16), static_cast<unsigned>(a.H),
                    static_cast<unsigned>(a.B * a.P));
    const void* fn = nullptr;
    switch (a.dk) {
        case 16: fn = reinterpret_cast<const void*>(&state_f32path<IO, 16, kStateCpt>); break;
        case 32: fn = reinterpret_cast<const void*>(&state_f32path<IO, 32, kStateCpt>); break;
        case 64: fn = reinterpret_cast<const void*>(&state_f32path<IO, 64, kStateCpt>); break;
        case 128: fn = reinterpret_cast<const void*>(&state_f32path<IO, 128, kStateCpt>); break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, grid, dim3(64 * (16 / kStateCpt)), args, 0, s);
}

}  // namespace

hipError_t launch_prep_f32path(const PrepArgs& a, bool io_bf16, hipStream_t s) {
    return io_bf16 ? prep_dispatch<uint16_t>(a, s) : prep_dispatch<float>(a, s);
}

hipError_t launch_state_f32path(const StateArgs& a, bool io_bf16, hipStream_t s) {
    return io_bf16 ? state_dispatch<uint16_t>(a, s) : state_dispatch<float>(a, s);
}

// blocks of the XCD-aware scan order: ceil(B H / 8) groups of 8 (b, h) x the column tiles
static dim3 scan_grid_xcd(int B, int H, int ncols) {
    const int64_t groups = (static_cast<int64_t>(B) * H + 7) / 8;
    return dim3(static_cast<unsigned>(groups * 8 * (ncols / 16)));
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.ncols / 16), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    void* args[] = {const_cast<ScanArgs*>(&a)};
    const void* fn = nullptr;
    switch (a.dk) {
        case 16: fn = reinterpret_cast<const void*>(&affine_scan<16>); break;
        case 32: fn = reinterpret_cast<const void*>(&affine_scan<32>); break;
        case 64: fn = reinterpret_cast<const void*>(&affine_scan<64>); break;
        case 128:
            fn = reinterpret_cast<const void*>(&affine_scan_mfma);
            grid = scan_grid_xcd(a.B, a.H, a.ncols);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
}

hipError_t launch_scan_bwd(const ScanBwdArgs& a, hipStream_t s) {
    void* args[] = {const_cast<ScanBwdArgs*>(&a)};
    const void* fn = nullptr;
    dim3 grid(static_cast<unsigned>(a.dv / 16), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    switch (a.dk) {
        case 16: fn = reinterpret_cast<const void*>(&affine_scan_rev<16>); break;
        case 32: fn = reinterpret_cast<const void*>(&affine_scan_rev<32>); break;
        case 64: fn = reinterpret_cast<const void*>(&affine_scan_rev<64>); break;
        case 128:
            fn = reinterpret_cast<const void*>(&affine_scan_rev_mfma);
            grid = scan_grid_xcd(a.B, a.H, a.dv);
            break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
    if (e != hipSuccess || a.P == 0) return e;
    const unsigned nbhp = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.H * a.P);
    if (a.dk == 128 && a.dv == 128)
        return hipLaunchKernel(reinterpret_cast<const void*>(&summary_outer_mfma), dim3(nbhp), dim3(512), args, 0, s);
    return hipLaunchKernel(reinterpret_cast<const void*>(&summary_outer), dim3(nbhp, static_cast<unsigned>(a.dk / 16)),
                           dim3(256), args, 0, s);
}

}  // namespace gdn
