// gdn_mfma.hip -- bf16 matrix-core (MFMA) kernels of the chunked Gated DeltaNet
// forward for gfx950, head dim dk = 128 (the head dim the pages' fused backend
// targets: hyper-parallel issue #320, test report for PR #1114, section 3.1).
//
// Chunk algebra (C = 64 tokens, incoming state S of dk x ncols, Gam the
// chunk-local cumulative log-decay):
//   A_ij = beta_i exp(Gam_i - Gam_j) k_i.k_j (i > j),  Tinv = (I + A)^{-1}
//   That = Tinv diag(beta),  P_ij = (q_i.k_j) exp(Gam_i - Gam_j) (j <= i)
//   X  = V - diag(exp Gam) K S          U = That X            (delta-rule errors)
//   O  = diag(exp Gam) Q S + P U        S' = exp(Gam_C) S + K^T diag(exp(Gam_C - Gam)) U
// The contractions run on bf16 MFMAs with fp32 accumulation; the state stays fp32
// and is rounded to bf16 only as an MFMA operand. The triangular solve stays fp32
// (column sweep on the 16x16 diagonal blocks, v_mfma_f32_16x16x4_f32 for the
// off-diagonal blocks).
//
// MFMA operand layouts used below (lane l):
//   32x32x16 bf16 (prepare pass), q = l / 32, r = l % 32: A row r, k = 8q .. 8q+7;
//     B col r, k = 8q .. 8q+7; C register i holds row 8(i/4) + 4q + (i%4), col r.
//   16x16x32 bf16 (state pass), g = l / 16: A row l%16, k = 8g .. 8g+7; B col l%16,
//     k = 8g .. 8g+7; C register j holds row 4g + j, col l%16.
//   16x16x4 f32: A row l%16, k = l/16;  B col l%16, k = l/16;  C rows 4(l/16)+j, col l%16.
#include "gdn_mfma_common.hpp"

namespace gdn {
namespace {

constexpr int CP = 64 + 8;   // LDS pitch (bf16) of 64-wide rows: 144 B
constexpr bool kEnablePrefetch = true;   // L2 prefetch of chunk operands by the output wave
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}
__device__ __forceinline__ int64_t valid_tokens(const int32_t* vl, int b, int64_t T) {
    if (!vl) return T;
    int64_t n = vl[b];
    return n < 0 ? 0 : (n > T ? T : n);
}
// Workgroup barrier that orders LDS only. __syncthreads() also waits for every
// outstanding global load and store of the wave, which would stall the loads
// issued one chunk ahead at every barrier; the waves here exchange data through
// LDS only.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// Causal depthwise Conv1D of one 8-channel granule over 4 consecutive token rows t0 + r0
// .. + 3 of batch row b, with SiLU and rounding to bf16, the same arithmetic as the
// standalone convolution (acc = bias, then acc += w_j x_{t-K+1+j} for j = 0 .. K - 1):
// out[u] is row r0 + u packed as bf16. The K - 1 rows before the first are read too (from
// x_prev before the sequence). Rows at or past T are not computed (out zero, y untouched);
// y receives the rows below T when write_y.
template <int K>
__device__ __forceinline__ void conv_granule(const PrepConv& cv, int b, int64_t T, int64_t t_first, int chan,
                                             bool write_y, u32x4 (&out)[4]) {
    const uint16_t* x = cv.x + static_cast<int64_t>(b) * T * cv.C + chan;
    float w[8][K], bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int j = 0; j < K; ++j) w[e][j] = cv.w[static_cast<int64_t>(chan + e) * K + j];
        bias[e] = cv.bias ? cv.bias[chan + e] : 0.f;
    }
    // raw rows t_first - K + 1 .. t_first + 3, all loads issued before any is used
    constexpr int NR = K + 3;
    u32x4 raw[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int64_t t = t_first - (K - 1) + j;
        if (t >= 0) {
            raw[j] = *reinterpret_cast<const u32x4*>(x + (t < T ? t : T - 1) * cv.C);
        } else if (cv.x_prev) {
            raw[j] = *reinterpret_cast<const u32x4*>(cv.x_prev + (static_cast<int64_t>(b) * (K - 1) + (K - 1) + t) * cv.C +
                                                     chan);
        } else {
            raw[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = bias[e];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const uint32_t wd = raw[u + j][e >> 1];
                const float xv = __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
                acc += w[e][j] * xv;
            }
            o[e] = acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc));
        }
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pk[e] = static_cast<uint32_t>(bf16_bits(o[2 * e])) | (static_cast<uint32_t>(bf16_bits(o[2 * e + 1])) << 16);
        const int64_t t = t_first + u;
        out[u] = t < T ? pk : u32x4{0u, 0u, 0u, 0u};
        if (write_y && t < T) *reinterpret_cast<u32x4*>(cv.y + (static_cast<int64_t>(b) * T + t) * cv.C + chan) = pk;
    }
}

// ----------------------------------------------------------------------------
// Prepare: one block of 4 waves per (b, h, chunk). kConvK > 0: the Conv1D of width
// kConvK runs in the pass (PrepConv).
// ----------------------------------------------------------------------------
template <int kConvK>
__global__ __launch_bounds__(256, 4) void prep_mfma(PrepArgs a) {
    constexpr int AP = 68;  // fp32 pitch of the 64x64 A and Tinv tiles
    // 35.8 KiB, four blocks per CU: K and Q (bf16, 256-byte rows) fill the first 32 KiB
    // until the products are done; then A lives at the start and Tinv behind it; once
    // the solve is done P (bf16) takes the place of A. Seven 64-float vectors follow:
    // Gam, beta, the prologue's row factors rk = 1/|k_t| and rq = q_scale/|q_t| (1 without
    // a prologue), and the exponents that fold them into the decay masks,
    // Gam_t + ln rk_t, Gam_s - ln rk_s and Gam_t + ln rq_t.
    constexpr int TS_OFF = 64 * AP * 4, GB_OFF = 2 * 64 * AP * 4;
    __shared__ __align__(16) unsigned char smem[GB_OFF + 7 * 256];
    uint16_t* k_s = reinterpret_cast<uint16_t*>(smem);
    uint16_t* q_s = k_s + 64 * DK;
    float* a_s = reinterpret_cast<float*>(smem);              // after the products
    float* t_s = reinterpret_cast<float*>(smem + TS_OFF);     // after the products
    uint16_t* p_s = reinterpret_cast<uint16_t*>(smem);        // after the solve
    float* gam_s = reinterpret_cast<float*>(smem + GB_OFF);
    float* beta_s = gam_s + 64;
    float* rk_s = gam_s + 128;
    float* rq_s = gam_s + 192;
    float* gk_s = gam_s + 256;    // Gam_t + ln rk_t  (row side of A)
    float* gks_s = gam_s + 320;   // Gam_s - ln rk_s  (column side of A and P)
    float* gq_s = gam_s + 384;    // Gam_t + ln rq_t  (row side of P)
    // K / Q element offset of granule g (8 bf16) of row r: XOR-swizzled by the row so
    // that the fragment reads of 16 consecutive rows hit 16 different bank groups
    const auto kq_at = [](int r, int g) { return r * DK + 8 * (g ^ (r & 15)); };

    // Block order: chunk-major, the heads of one (b, chunk) back to back on one XCD
    // (workgroups go round-robin over the 8 XCDs), so that its L2 serves the q/k rows
    // shared by the value heads of a query/key head and the g / beta lines shared by
    // all heads. Chunks run from the last to the first: the state pass that follows
    // starts with the records written last, which the memory-side cache still holds.
    // ch is the (b, h, chunk) record index.
    const int64_t L = blockIdx.x;
    const int xcd = static_cast<int>(L & 7);
    const int64_t u = L >> 3;
    const int h = static_cast<int>(u % a.H);
    const int64_t pair = (u / a.H) * 8 + xcd;
    if (pair >= static_cast<int64_t>(a.B) * a.NT) return;
    const int b = static_cast<int>(pair / a.NT), n = a.NT - 1 - static_cast<int>(pair % a.NT);
    const int64_t ch = (static_cast<int64_t>(b) * a.H + h) * a.NT + n;
    const int hq = h / (a.H / a.Hqk);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 5, lr = lane & 31;
    const int64_t t0 = static_cast<int64_t>(n) * kChunk;
    const RowSpan rs = row_span(a.cu_seqlens, a.valid_len, b, a.T, a.NT);
    const int64_t nvalid = rs.valid;
    // a packed sequence shorter than this chunk's start has nothing here (its state pass
    // stops at its last chunk and never reads this record)
    if (a.cu_seqlens && t0 >= nvalid) return;
    const uint16_t* kin = static_cast<const uint16_t*>(a.k);
    const uint16_t* qin = static_cast<const uint16_t*>(a.q);

    // Loads are unconditional from a clamped, in-bounds token (row 0 of the
    // sequence for padded tokens) and masked afterwards, so that no load waits
    // behind a branch.
    // Wave 0's g and beta loads go out first, then everybody's q/k loads: loads return
    // in issue order, so the decay scan of wave 0 starts while the q/k loads are still
    // in flight (issued after them it would wait for all of them).
    const int64_t tg = t0 + lane;
    const bool gvalid = tg < nvalid;
    // With the prologue, a and b take the place of g and beta.
    float graw = 0.f, braw = 0.f;
    if (wave == 0) {
        const int64_t gi = (rs.start + (gvalid ? tg : 0)) * a.H + h;
        graw = a.has_prologue ? a.pro.a[gi] : a.g[gi];
        braw = a.has_prologue ? a.pro.b[gi] : a.beta[gi];
    }
    // Rows of this thread's four K and Q granules (granule tid % 16): rows tid / 16 + 16 u,
    // or with the Conv1D four consecutive rows 4 (tid / 16) + u, whose window each thread
    // slides over the K - 1 rows before them.
    const auto row_of = [&](int u) { return kConvK > 0 ? 4 * (tid >> 4) + u : (tid >> 4) + 16 * u; };
    u32x4 kv[4], qv[4];
    if constexpr (kConvK > 0) {
        // q, k and v channels of the convolution; the first value head of each query/key
        // group writes the q and k output rows, every value head its own v rows
        const int cb = tid & 15;
        const int64_t tf = t0 + 4 * (tid >> 4);
        const bool qk_owner = h % (a.H / a.Hqk) == 0;
        {
            u32x4 vv[4];   // written to y only
            conv_granule<kConvK>(a.conv, b, a.T, tf, 2 * a.Hqk * DK + h * DK + 8 * cb, true, vv);
        }
        conv_granule<kConvK>(a.conv, b, a.T, tf, hq * DK + 8 * cb, qk_owner, qv);
        conv_granule<kConvK>(a.conv, b, a.T, tf, a.Hqk * DK + hq * DK + 8 * cb, qk_owner, kv);
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = row_of(u), cb = tid & 15;
            const int64_t t = t0 + row;
            const int64_t off =
                (rs.start + (t < nvalid ? t : 0)) * a.qk_stride + hq * DK + 8 * cb;
            kv[u] = *reinterpret_cast<const u32x4*>(kin + off);
            qv[u] = *reinterpret_cast<const u32x4*>(qin + off);
        }
    }
    if (wave == 0) {
        float gv = graw, bv = braw;
        if (a.has_prologue) {
            // g = -exp(A_log) softplus(a + dt_bias), softplus(x) = max(x, 0) + log(1 + exp(-|x|));
            // beta = sigmoid(b)
            const float x = graw + a.pro.dt_bias[h];
            gv = -__expf(a.pro.A_log[h]) * (fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))));
            bv = 1.f / (1.f + __expf(-braw));
        }
        float gam = gvalid ? gv : 0.f;
        const float bt = gvalid ? bv : 0.f;
        // inclusive scan over the 64 lanes with DPP moves: shifts by 1, 2, 4, 8 inside
        // each row of 16 lanes (lanes shifted in from outside the row read 0), then lane
        // 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3
        const auto dpp_add = [](float x, auto ctrl_tag, auto rows_tag) {
            const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl_tag)::value,
                                                      decltype(rows_tag)::value, 0xf, true);
            return x + __int_as_float(y);
        };
        gam = dpp_add(gam, IntTag<0x111>{}, IntTag<0xf>{});   // row_shr:1
        gam = dpp_add(gam, IntTag<0x112>{}, IntTag<0xf>{});   // row_shr:2
        gam = dpp_add(gam, IntTag<0x114>{}, IntTag<0xf>{});   // row_shr:4
        gam = dpp_add(gam, IntTag<0x118>{}, IntTag<0xf>{});   // row_shr:8
        gam = dpp_add(gam, IntTag<0x142>{}, IntTag<0xa>{});   // row_bcast:15
        gam = dpp_add(gam, IntTag<0x143>{}, IntTag<0xc>{});   // row_bcast:31
        gam_s[lane] = gam;
        beta_s[lane] = bt;
    }
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = row_of(u), cb = tid & 15;
            const bool valid = t0 + row < nvalid;
            if (!valid) kv[u] = qv[u] = z;
            *reinterpret_cast<u32x4*>(k_s + kq_at(row, cb)) = kv[u];
            *reinterpret_cast<u32x4*>(q_s + kq_at(row, cb)) = qv[u];
        }
    }
    if (a.has_prologue) {
        // row norms: the 16 lanes of a row (a DPP row of consecutive lanes) each hold 8 of
        // its values
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float k0 = __uint_as_float(kv[u][e] << 16), k1 = __uint_as_float(kv[u][e] & 0xFFFF0000u);
                const float q0 = __uint_as_float(qv[u][e] << 16), q1 = __uint_as_float(qv[u][e] & 0xFFFF0000u);
                sk += k0 * k0 + k1 * k1;
                sq += q0 * q0 + q1 * q1;
            }
            // 1 / max(|x|, 1e-12) as the reciprocal square root of max(|x|^2, 1e-24)
            const float rk = __builtin_amdgcn_rsqf(fmaxf(row_prefix16(sk), 1e-24f));
            const float rq = a.pro.q_scale * __builtin_amdgcn_rsqf(fmaxf(row_prefix16(sq), 1e-24f));
            if ((tid & 15) == 15) {
                const int row = row_of(u);
                rk_s[row] = rk;
                rq_s[row] = rq;
            }
        }
    } else if (tid < 64) {
        rk_s[tid] = 1.f;
        rq_s[tid] = 1.f;
    }
    lds_sync();
    // Waves 0-2 form the Gram tiles, wave 3 the decay record and the mask exponents.
    // (mi, nj): the lower 32x32 tile of K K^T and of Q K^T that wave w < 3 owns.
    const int mi = wave == 0 ? 1 : wave - 1, nj = wave == 0 ? 0 : wave - 1;
    f32x16 acc0 = zero16(), acc1 = zero16();
    if (wave == 3) {
        // the decay record: exp(Gam) rk, exp(Gam_C - Gam) rk, exp(Gam) rq, exp(Gam_C)
        const float gam = gam_s[lane], gam_c = gam_s[63], rk = rk_s[lane], rq = rq_s[lane];
        const float eg = __expf(gam);
        float* gr = a.ws.gates + ch * kGateRecordMfma;
        gr[lane] = eg * rk;
        gr[64 + lane] = __expf(gam_c - gam) * rk;
        gr[128 + lane] = eg * rq;
        gr[192 + lane] = lane == 0 ? __expf(gam_c) : 0.f;
        // the exponents of the decay masks of A and P with the row factors folded in
        // (ln 1 = 0 exactly without a prologue), in base 2 for v_exp_f32
        const float lk = __logf(rk);
        gk_s[lane] = (gam + lk) * kLog2e;
        gks_s[lane] = (gam - lk) * kLog2e;
        gq_s[lane] = (gam + __logf(rq)) * kLog2e;
    } else {
        // K K^T and Q K^T of tile (mi, nj) in one k-loop over the shared K fragments:
        // wave 0 (1,0), wave 1 (0,0), wave 2 (1,1)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const bf16x8 ak = lds_frag(k_s + kq_at(32 * mi + lr, 2 * c + q));
            const bf16x8 aq = lds_frag(q_s + kq_at(32 * mi + lr, 2 * c + q));
            const bf16x8 bv = lds_frag(k_s + kq_at(32 * nj + lr, 2 * c + q));
            acc0 = mfma32(ak, bv, acc0);
            acc1 = mfma32(aq, bv, acc1);
        }
    }
    lds_sync();   // K and Q are dead from here on; A takes their place
    // A (fp32) into LDS. The decay and beta values of the lane's 16 rows are read
    // into registers first: the A stores share the LDS array, and reads placed
    // between them would be issued one at a time.
    auto emit_a = [&](const f32x16& acc, int mi, int nj) {
        const int s = 32 * nj + lr;
        const float gs = gks_s[s];
        f32x4 gt[4], bt[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            gt[i4] = *reinterpret_cast<const f32x4*>(gk_s + 32 * mi + 8 * i4 + 4 * q);
            bt[i4] = *reinterpret_cast<const f32x4*>(beta_s + 32 * mi + 8 * i4 + 4 * q);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 32 * mi + 8 * (i / 4) + 4 * q + (i % 4);
            a_s[t * AP + s] = (t > s) ? bt[i / 4][i % 4] * __builtin_amdgcn_exp2f(gt[i / 4][i % 4] - gs) * acc[i] : 0.f;
        }
    };
    if (wave < 3) emit_a(acc0, mi, nj);
    lds_sync();   // A is complete; P stays in registers until A is dead
    if (wave < 3) {
        // the decay mask of the wave's P tile, while wave 3 inverts the diagonal blocks
        const int s = 32 * nj + lr;
        const float gs = gks_s[s];
        f32x4 gt[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) gt[i4] = *reinterpret_cast<const f32x4*>(gq_s + 32 * mi + 8 * i4 + 4 * q);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 32 * mi + 8 * (i / 4) + 4 * q + (i % 4);
            acc1[i] = (t >= s) ? __builtin_amdgcn_exp2f(gt[i / 4][i % 4] - gs) * acc1[i] : 0.f;
        }
        // zero the strictly upper 16x16 blocks of Tinv, 16 bytes a store
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int e = tid; e < 6 * 64; e += 192) {
            const int blk = e >> 6, w = e & 63;
            const int bi = (blk < 3) ? 0 : (blk < 5 ? 1 : 2);
            const int bj = (blk < 3) ? blk + 1 : (blk < 5 ? blk - 1 : 3);
            *reinterpret_cast<f32x4*>(t_s + (16 * bi + (w >> 2)) * AP + 16 * bj + 4 * (w & 3)) = z;
        }
    } else {
        // diagonal 16x16 blocks: unit lower-triangular inverse by forward substitution,
        // lane (blk, c) of wave 3 owns column c of diagonal block blk.
        // Column sweep: once x[j] is final it is eliminated from every later row, so
        // the dependency chain is 15 steps long instead of one FMA per matrix entry.
        // The block is read in four batches of columns 4q .. 4q+3, one 16-byte read per
        // row below the diagonal (at most 15 reads, so each batch waits once).
        const int c = lane & 15, o = 16 * (lane >> 4);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 v[16];
#pragma unroll
            for (int r = 4 * q + 1; r < 16; ++r) v[r] = *reinterpret_cast<const f32x4*>(a_s + (o + r) * AP + o + 4 * q);
#pragma unroll
            for (int j = 4 * q; j < 4 * q + 4 && j < 15; ++j)
#pragma unroll
                for (int r = j + 1; r < 16; ++r) x[r] -= v[r][j - 4 * q] * x[j];
        }
        // stored after the substitution, so that no store sits between its LDS reads
#pragma unroll
        for (int r = 0; r < 16; ++r) t_s[(o + r) * AP + o + c] = x[r];
    }
    lds_sync();
    // off-diagonal blocks: T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj (T_jj = D_j). Each wave
    // runs one dependency chain with its earlier results kept in registers: wave 0
    // T10, T20, T30; wave 1 T21, T31; wave 2 T32. A 16x16 block product takes four
    // 16x16x4 f32 MFMAs; an operand in LDS is read in any order, and a result held in
    // accumulator layout (lane (j, g) has rows 4g .. 4g+3 of column j) serves as the B
    // operand with k-slot (s, g) standing for row 4g + s.
    const int l16 = lane & 15, g4 = lane >> 4;
    // acc += X_(bi,bk) Y_(bk,bj), both blocks in LDS (X from a_s or t_s, Y from t_s)
    auto mm_ll = [&](const float* x, int bi, int bk, int bj, f32x4 acc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float av = x[(16 * bi + l16) * AP + 16 * bk + 4 * s + g4];
            const float bv = t_s[(16 * bk + 4 * s + g4) * AP + 16 * bj + l16];
            acc = mfma16f32(av, bv, acc);
        }
        return acc;
    };
    // acc += X_(bi,bk) R with X in LDS and R in accumulator layout
    auto mm_lr = [&](const float* x, int bi, int bk, const f32x4& r, f32x4 acc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16f32(x[(16 * bi + l16) * AP + 16 * bk + 4 * g4 + s], r[s], acc);
        return acc;
    };
    // -D_i Y
    auto neg_d = [&](int bi, const f32x4& y) {
        f32x4 r = mm_lr(t_s, bi, bi, y, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = -r[i];
        return r;
    };
    auto put = [&](int bi, int bj, const f32x4& r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t_s[(16 * bi + 4 * g4 + i) * AP + 16 * bj + l16] = r[i];
    };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    if (wave == 0) {
        const f32x4 t10 = neg_d(1, mm_ll(a_s, 1, 0, 0, z4));
        const f32x4 t20 = neg_d(2, mm_lr(a_s, 2, 1, t10, mm_ll(a_s, 2, 0, 0, z4)));
        const f32x4 t30 = neg_d(3, mm_lr(a_s, 3, 2, t20, mm_lr(a_s, 3, 1, t10, mm_ll(a_s, 3, 0, 0, z4))));
        put(1, 0, t10);
        put(2, 0, t20);
        put(3, 0, t30);
    } else if (wave == 1) {
        const f32x4 t21 = neg_d(2, mm_ll(a_s, 2, 1, 1, z4));
        const f32x4 t31 = neg_d(3, mm_lr(a_s, 3, 2, t21, mm_ll(a_s, 3, 1, 1, z4)));
        put(2, 1, t21);
        put(3, 1, t31);
    } else if (wave == 2) {
        put(3, 2, neg_d(3, mm_ll(a_s, 3, 2, 2, z4)));
    }
    lds_sync();
    // P into the space of A
    if (wave < 3) {
        const int s = 32 * nj + lr;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 32 * mi + 8 * (i / 4) + 4 * q + (i % 4);
            p_s[t * CP + s] = bf16_bits(acc1[i]);
        }
    } else {
        // wave 3: the all-zero upper tile of P (rows 0..31, cols 32..63)
        for (int e = lane; e < 32 * 32; e += 64) p_s[(e >> 5) * CP + 32 + (e & 31)] = 0;
    }
    lds_sync();
    // outputs: That = Tinv diag(beta), P and the bf16 remainder of That, in the
    // fragment order of the state pass: lane l of block (r, s) holds row 16r + l % 16
    // at tokens 32s + 4 (l / 16) + (e % 4) + 16 (e / 4), e = 0..7
    for (int p = tid; p < 6 * 64; p += 256) {
        const int blk = p >> 6, l = p & 63;
        const int r = blk < 2 ? blk : 2 + ((blk - 2) >> 1);
        const int s = blk < 2 ? 0 : ((blk - 2) & 1);
        const int i = 16 * r + (l & 15), g = l >> 4;
        u32x4 w, wl, wp;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const int j0 = 32 * s + 4 * g + 2 * (e2 & 1) + 16 * (e2 >> 1), j1 = j0 + 1;
            const float x0 = t_s[i * AP + j0] * beta_s[j0], x1 = t_s[i * AP + j1] * beta_s[j1];
            const uint16_t h0 = bf16_bits(x0), h1 = bf16_bits(x1);
            w[e2] = h0 | (static_cast<uint32_t>(h1) << 16);
            wl[e2] = bf16_bits(x0 - bf16_to_f32(h0)) | (static_cast<uint32_t>(bf16_bits(x1 - bf16_to_f32(h1))) << 16);
            wp[e2] = p_s[i * CP + j0] | (static_cast<uint32_t>(p_s[i * CP + j1]) << 16);
        }
        const int64_t off = ch * kTriRecord + blk * 512 + l * 8;
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.ws.that) + off) = w;
        // the backward alone does not read the forward's P record
        if (!a.bwd.thatT || a.bwd.keep_pmat) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.ws.pmat) + off) = wp;
        if (a.ws.that_lo) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.ws.that_lo) + off) = wl;
    }
    if (a.bwd.thatT) {
        // backward records: That^T (That^T_ij = Tinv_ji beta_i) and P^T on the upper blocks
        // (0,0) (0,1) (1,0) (1,1) (2,1) (3,1) in the same fragment order, then Tinv and P
        // row-major (Tinv and P are exactly zero above their diagonals in LDS)
        for (int p = tid; p < 6 * 64; p += 256) {
            const int blk = p >> 6, l = p & 63;
            const int r = blk < 4 ? blk >> 1 : blk - 2;
            const int s = blk < 4 ? blk & 1 : 1;
            const int i = 16 * r + (l & 15), g = l >> 4;
            const float bi = beta_s[i];
            u32x4 w, wp;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int j0 = 32 * s + 4 * g + 2 * (e2 & 1) + 16 * (e2 >> 1), j1 = j0 + 1;
                w[e2] = pk2(t_s[j0 * AP + i] * bi, t_s[j1 * AP + i] * bi);
                wp[e2] = p_s[j0 * CP + i] | (static_cast<uint32_t>(p_s[j1 * CP + i]) << 16);
            }
            const int64_t off = ch * kTriRecord + blk * 512 + l * 8;
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.bwd.thatT) + off) = w;
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.bwd.pT) + off) = wp;
        }
        for (int p = tid; p < 2 * 512; p += 256) {
            const int row = (p & 511) >> 3, c0 = 8 * (p & 7);
            u32x4 w;
            if (p < 512) {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) w[e2] = pk2(t_s[row * AP + c0 + 2 * e2], t_s[row * AP + c0 + 2 * e2 + 1]);
            } else {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2)
                    w[e2] = p_s[row * CP + c0 + 2 * e2] | (static_cast<uint32_t>(p_s[row * CP + c0 + 2 * e2 + 1]) << 16);
            }
            void* dst = p < 512 ? a.bwd.t_rm : a.bwd.p_rm;
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + ch * 4096 + row * 64 + c0) = w;
        }
    }
}

// ----------------------------------------------------------------------------
// State pass. One block of 8 waves per (b, h, segment, 16 state columns):
//   wave 0, the chain wave, carries the 128 x 16 state slice in registers and runs
//     the sequential part of every chunk:
//       X = V - diag(exp Gam) K S,   U = That X,   S <- exp(Gam_C) S + K^T diag(exp(Gam_C - Gam)) U
//     on v_mfma_f32_16x16x32_bf16. Each product's 16x16 result tiles feed the next
//     product as its B operand straight from the accumulators: the contraction
//     index of a k-step is ordered as the rows the lanes of the result tiles hold
//     (4 rows of one tile and the same 4 rows of the next), and every operand
//     contracted against it is laid out with the same order. The chain wave issues
//     no global memory instruction (issuing one stalls the issuing wave for tens of
//     cycles).
//   wave 1, the output wave (forward only), computes one chunk behind the chain
//     wave O = diag(exp Gam) Q S + P U from the state and U the chain wave leaves in
//     LDS, transposed (O^T = S^T Q^T + U^T P^T) so that each lane ends up holding
//     four consecutive columns of one token, and writes o. When one pass computes
//     both segment summaries, wave 0 runs the chain of the M tile and wave 1 the
//     chain of the S tile instead.
//   the other waves load the chunk operands into registers and write them to LDS
//     an iteration later (K, That and its remainder, V and the decay factors of the
//     next chunk for the chain wave; Q of the current chunk for the output wave,
//     which reads it in the next iteration), with two iterations of loads in flight;
//     two LDS buffers per side. The output wave loads P itself, straight into
//     registers.
// One barrier per chunk.
//
// Layouts. A 1 KiB fragment block holds one 16x32 bf16 MFMA operand, lane l's 16
// bytes at byte 16 l (row l % 16, contraction slots 8 (l / 16) .. +7):
//   K, Q: 4-row blocks, swizzled (see below) so that one 1 KiB load moves 4 whole rows;
//   That, P: blocks (r, s) of the lower triangle, (0,0) (1,0) (2,0) (2,1) (3,0) (3,1),
//     rows = tokens 16r .., slot 8g + e = token 32s + 4g + (e % 4) + 16 (e / 4);
//   V: [64 tokens][16 columns], read with transposing reads into accumulator order.
// State register t (t = 0..7) of lane (c = l % 16, g = l / 16), element j holds
// S[32 (t / 2) + 8g + 4 (t % 2) + j][c], so that the pair of registers 2s, 2s+1 is
// the B fragment of k-step s of K S, and the transposing reads of K give the A
// fragments of K^T for the state update in that same row order.
//
// kSplit (used for the summary matrix M, a product of thousands of near
// projections whose relative error grows with every rounding): the state, X,
// V'' and That enter the MFMAs as bf16 hi + lo pairs (x = hi + lo, lo the bf16 of
// the remainder), the products taken as hi*hi + hi*lo + lo*hi.
// ----------------------------------------------------------------------------

// Loading wave (index among the loading waves) that issues load g of an iteration.
// Waves w and w + 4 of a workgroup run on the same SIMD; the deal gives every SIMD
// the same share of the loads. Mode 1 (outputs: chain and output waves 0 and 1, loading
// waves 2 .. 7): waves 0 and 1 each share their SIMD with one loading wave (indices 2
// and 3), which take two of every eight loads. Mode 2 (two tiles of both summaries: M
// chains on waves 0 and 1, S chains on waves 2 and 3, loading waves 4 .. 7): the loading
// waves beside the S chains (indices 2 and 3) take three of every four loads. Mode 3 (two
// tiles with outputs: chain, output, chain, output on waves 0 .. 3, loading waves 4 .. 7,
// one beside each): round-robin. Mode 4 (one tile with outputs split over two waves: chain,
// output, output on waves 0 .. 2, loading waves 3 .. 7): the two loading waves of the SIMD
// without a compute wave (indices 0 and 4) take five of every eight loads. Mode 0
// (one chain wave, loading waves 1 .. 7): wave 0 shares its SIMD with loading wave 3.
__host__ __device__ constexpr int load_owner(int mode, int g) {
    const int p = g & 7;
    if (mode == 1) return (p == 0 || p == 3) ? 2 : (p == 1 || p == 4) ? 3 : (p == 2) ? 0 : (p == 5) ? 1 : (p == 6) ? 4 : 5;
    if (mode == 2) return (p == 0) ? 0 : (p == 4) ? 1 : (p & 1) ? 2 : 3;
    if (mode == 3) return p & 3;
    if (mode == 4) return (p == 0 || p == 2 || p == 7) ? 0 : (p == 1 || p == 3) ? 4 : p - 3;
    return p == 0 ? 3 : p - 1;
}
__host__ __device__ constexpr int loads_owned(int mode, int n, int me) {
    int c = 0;
    for (int g = 0; g < n; ++g) c += load_owner(mode, g) == me ? 1 : 0;
    return c;
}

template <bool kHasV, bool kSplit, bool kOut, bool kPair = false>
__global__ __launch_bounds__(512) void state_mfma(StateArgs a, int tiles, int qk_groups) {
    constexpr bool outputs = kHasV && kOut;
    // Two column tiles per workgroup with outputs (kPair): waves 0 and 2 run the chains of
    // tiles 0 and 1, waves 1 and 3 their outputs; the four share the loaded operands.
    constexpr bool pair = outputs && kPair;
    // One tile with outputs: the outputs of a chunk's four 16-token tiles are split over
    // waves 1 (tiles 0 and 3) and 2 (tiles 1 and 2), halving each wave's reads of Q.
    constexpr bool split_out = outputs && !kPair;
    // Both summaries in one pass (values, split, no outputs) on two column tiles: waves 0
    // and 1 run the chains of the M tiles (split operands, no values, identity start,
    // written to a.m_out), waves 2 and 3 the chains of the S tiles (values, zero start,
    // written to a.s_out); the four share every loaded operand, each M chain on a SIMD of
    // its own. Requires ncols = dk; `tiles` counts pairs of column tiles.
    constexpr bool dual = kHasV && kSplit && !kOut;
    constexpr bool two_compute = outputs || dual;   // compute waves first, then loading waves
    constexpr int load_mode = dual ? 2 : (pair ? 3 : (split_out ? 4 : (outputs ? 1 : 0)));
    constexpr int vtiles = (dual || pair) ? 2 : 1;   // column tiles per workgroup
    // K-side stage buffer: K, That, That remainder (split), V; Q-side: Q, P.
    // K-side operands of chunk n are written in iteration n - 1 and read in iteration
    // n; Q-side operands in iteration n and read by the output wave, which runs one
    // chunk behind, in iteration n + 1 (two buffers each); the decay factors of a
    // chunk live from their write to the output wave (ring of four).
    constexpr int KB = 64 * DK * 2, TB = kTriRecord * 2, LB = kSplit ? kTriRecord * 2 : 0;
    constexpr int VB = kHasV ? 64 * 16 * 2 * vtiles : 0;
    constexpr int KSB = KB + TB + LB + VB;
    constexpr int QSB = outputs ? KB : 0;
    constexpr int HB = 6 * 1024;   // hand-off: S fragments (4 blocks), U fragments (2 blocks)
    __shared__ __align__(16) unsigned char kst[2 * KSB];
    __shared__ __align__(16) unsigned char qst[outputs ? 2 * QSB : 16];
    __shared__ __align__(16) unsigned char gst[4 * 1024];
    __shared__ __align__(16) unsigned char hst[outputs ? 2 * HB * vtiles : 16];
    __shared__ __align__(16) unsigned char pf_s[outputs ? 256 : 16];   // sink of the L2 prefetches

    // XCD-aware block order (workgroups go round-robin over the 8 XCDs): every column
    // tile of the value heads that read one query/key head of one (b, segment) runs on
    // the same XCD, so that its L2 holds that head's q, k and chunk records once.
    const int L = blockIdx.x;
    const int xcd = L & 7, slot = L >> 3;
    const int tile = slot % tiles;
    const int rep = a.H / a.Hqk;
    const int kk = slot / tiles;
    const int qg = (kk / rep) * 8 + xcd;   // (b, segment, query/key head) group
    if (qg >= qk_groups) return;
    const int bz = qg / a.Hqk, hq = qg % a.Hqk;
    const int h = hq * rep + kk % rep;
    const int b = bz / a.P, seg = bz % a.P;
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    // the workgroup's first column and a compute wave's own tile: in the one-pass summary
    // waves w and w + 2 share tile w % 2, with outputs on two tiles waves 2 t and 2 t + 1
    // work on tile t
    const int sub = dual ? (wave & 1) : (pair ? ((wave >> 1) & 1) : 0);
    const int colp = 16 * vtiles * tile;
    const int col0 = colp + 16 * sub;
    const int ncols = a.ncols;
    const RowSpan rs = row_span(a.cu_seqlens, a.valid_len, b, a.T, a.NT);
    const int64_t nvalid = rs.valid;
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int64_t stile = static_cast<int64_t>(DK) * ncols;
    // a packed sequence stops at its own last chunk
    const int n0 = seg * a.Lc;
    const int n1 = min(min(n0 + a.Lc, a.NT), static_cast<int>((rs.extent + kChunk - 1) / kChunk));

    const int64_t qk_row = a.qk_stride;                          // elements between tokens of q, k
    const int64_t v_row = a.v_stride;                            // ... of v
    const int64_t vo_row = static_cast<int64_t>(a.H) * ncols;   // ... of o
    const uint32_t kstep = static_cast<uint32_t>(kChunk * qk_row * 2);   // bytes per chunk
    const uint32_t vstep = static_cast<uint32_t>(kChunk * v_row * 2);
    const uint32_t ostep = static_cast<uint32_t>(kChunk * vo_row * 2);
    const int first_loader = (dual || pair) ? 4 : (split_out ? 3 : (two_compute ? 2 : 1));
    // K / Q tile layout: quad block j (rows 4j .. 4j+3, 1 KiB) holds granule gk (dk 8gk .. +7)
    // of row 4j + rho at 16-byte slot 16 rho + (gk ^ (4 rho + j % 4)). A 1 KiB load fills one
    // quad block with 16 lanes per row, so that each group of 4 lanes reads one 64-byte piece
    // (lanes of a quad spread over different rows cost the load path 3x as much). The
    // fragment reads are free of bank conflicts: the 16 lanes of a group read rows with 16
    // different (rho, j % 4). A transposing read takes 4 granules of 4 rows per group; the
    // row selects the upper two bits of the slot, so those 16 pieces fill 16 different
    // slots (2-way conflicts remain between the two groups of a half-wave, which read the
    // same 8-byte halves; with the row in the lower bits they were 4-way).
    // Fragment (r, s) of lane (l16, g4): byte 4096 r + frag_lane[s].
    int frag_lane[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        frag_lane[s] = (l16 >> 2) * 1024 + 256 * (l16 & 3) + 16 * ((4 * s + g4) ^ (4 * (l16 & 3) + (l16 >> 2)));

    if (wave >= first_loader) {
        // ---------------- loading waves ----------------
        // q/k/v descriptors over row b end at the last valid token: padded and
        // out-of-range tokens load as zero
        const uint16_t* kin = static_cast<const uint16_t*>(a.k) + rs.start * qk_row;
        const uint16_t* qin = static_cast<const uint16_t*>(a.q) + rs.start * qk_row;
        const uint16_t* vin = static_cast<const uint16_t*>(a.v ? a.v : a.k) + rs.start * v_row;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kin, nvalid * qk_row * 2);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(outputs ? qin : kin, nvalid * qk_row * 2);
        // NULL values (the homogeneous chain's backward) read as zero: no records
        const __amdgpu_buffer_rsrc_t rv = make_rsrc((kHasV && a.v) ? vin : kin, (kHasV && a.v) ? nvalid * v_row * 2 : 0);
        const int64_t rec = static_cast<int64_t>(a.NT) * kTriRecord * 2;   // bytes of one head's records
        const __amdgpu_buffer_rsrc_t rth = make_rsrc(static_cast<const uint16_t*>(a.ws.that) + bh * a.NT * kTriRecord, rec);
        const __amdgpu_buffer_rsrc_t rtl = make_rsrc(
            kSplit ? static_cast<const uint16_t*>(a.ws.that_lo) + bh * a.NT * kTriRecord : static_cast<const uint16_t*>(a.ws.that),
            rec);
        const __amdgpu_buffer_rsrc_t rgt = make_rsrc(a.ws.gates + bh * a.NT * kGateRecordMfma,
                                                     static_cast<int64_t>(a.NT) * kGateRecordMfma * 4);

        // lane l of a quad-block load: slot l = 16 rho + c, row 4j + rho, granule c ^ (4 rho + j % 4)
        uint32_t voff_k[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            voff_k[jj] = static_cast<uint32_t>(((lane >> 4) * qk_row + hq * DK +
                                                8 * ((lane & 15) ^ (4 * (lane >> 4) + jj))) * 2);
        const uint32_t voff_l = static_cast<uint32_t>(16 * lane);
        // V load m: tile m / 2 of the workgroup, tokens 32 (m % 2) + lane / 2
        constexpr int NV = kHasV ? 2 * vtiles : 0;
        uint32_t voff_v[2 * vtiles];
#pragma unroll
        for (int m = 0; m < 2 * vtiles; ++m)
            voff_v[m] = static_cast<uint32_t>(((32 * (m & 1) + (lane >> 1)) * v_row + h * ncols + colp + 16 * (m >> 1) +
                                               8 * (lane & 1)) * 2);
        constexpr int nl = 8 - ((dual || pair) ? 4 : (split_out ? 3 : (two_compute ? 2 : 1)));
        constexpr int NK = 16 + 6 + (kSplit ? 6 : 0) + NV + 1;
        constexpr int NQ = outputs ? 16 : 0;
        constexpr int NI = NK + NQ;   // 1 KiB loads of one full iteration
        static_assert(nl >= 4, "loading waves");

        // Each 1 KiB load (lane l: 16 bytes, written to LDS at 16 l of its block) goes
        // through registers. In iteration n a loading wave writes to LDS what it loaded
        // in iteration n - 2 (the K-side operands of chunk n + 1 and the Q-side operands
        // of chunk n) and then loads the K-side operands of chunk n + 3 and the Q-side
        // operands of chunk n + 2: under the full load of the chip a load takes about
        // one iteration to return, so two iterations of loads are in flight. Each
        // operand spends a single iteration in LDS (two buffers per side).
        // The loads are dealt over the loading waves by load_owner; the loop below is
        // compiled once per wave index and unrolled by two, so that each wave runs its
        // own loads as straight-line code with its registers indexed at compile time.
        auto loader = [&](auto me_tag) {
        constexpr int me = decltype(me_tag)::value;
        constexpr int NS = loads_owned(load_mode, NI, me);
        using Stage = u32x4[NS > 0 ? NS : 1];
        Stage st0, st1;   // loads of even / odd iterations (relative to n0)
        auto load_k = [&](int n, Stage& stage) {   // K-side operands of chunk n
            const uint32_t tr = static_cast<uint32_t>(n) * (kTriRecord * 2);
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                if (load_owner(load_mode, i) != me) continue;
                u32x4& r = stage[loads_owned(load_mode, i, me)];
                if (i < 16) {
                    r = gload16(rk, voff_k[i & 3],
                                static_cast<uint32_t>(4 * i * qk_row * 2) + static_cast<uint32_t>(n) * kstep);
                } else if (i < 22) {
                    r = gload16(rth, voff_l, tr + (i - 16) * 1024);
                } else if (kSplit && i < 28) {
                    r = gload16(rtl, voff_l, tr + (i - 22) * 1024);
                } else if (kHasV && i < NK - 1) {
                    r = gload16(rv, voff_v[i - (NK - 1 - NV)], static_cast<uint32_t>(n) * vstep);
                } else {
                    r = gload16(rgt, voff_l, static_cast<uint32_t>(n) * (kGateRecordMfma * 4u));
                }
            }
        };
        auto store_k = [&](int n, const Stage& stage) {   // into stage buffer n % 2 (decay factors: slot n % 4)
            unsigned char* dst = kst + (n & 1) * KSB + 16 * lane;
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                if (load_owner(load_mode, i) != me) continue;
                unsigned char* p;
                if (i < 16) p = dst + i * 1024;
                else if (i < 22) p = dst + KB + (i - 16) * 1024;
                else if (kSplit && i < 28) p = dst + KB + TB + (i - 22) * 1024;
                else if (kHasV && i < NK - 1) p = dst + KB + TB + LB + (i - (NK - 1 - NV)) * 1024;
                else p = gst + (n % 4) * 1024 + 16 * lane;
                *reinterpret_cast<u32x4*>(p) = stage[loads_owned(load_mode, i, me)];
            }
        };
        auto load_q = [&](int n, Stage& stage) {   // Q of chunk n
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                if (load_owner(load_mode, NK + j) != me) continue;
                stage[loads_owned(load_mode, NK + j, me)] =
                    gload16(rq, voff_k[j & 3], static_cast<uint32_t>(4 * j * qk_row * 2) + static_cast<uint32_t>(n) * kstep);
            }
        };
        auto store_q = [&](int n, const Stage& stage) {   // into buffer n % 2
            unsigned char* dst = qst + (n & 1) * QSB + 16 * lane;
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                if (load_owner(load_mode, NK + j) != me) continue;
                *reinterpret_cast<u32x4*>(dst + j * 1024) = stage[loads_owned(load_mode, NK + j, me)];
            }
        };
        // Iteration n: stores of the loads of iteration n - 2, then the loads of iteration
        // n. The body has no branches, so that the compiler's wait for a store counts
        // only the loads issued before it: loads past the last chunk fetch the last
        // chunk again, and their stores land in buffers nobody reads any more (the
        // K-side buffer of a chunk >= n1 and the Q-side buffer of chunk n1; the chain
        // reads chunk n and the output wave chunk n - 1 in iteration n).
        const int last = n1 > 0 ? n1 - 1 : 0;
        auto step = [&](int n, Stage& stage) {
            chunk_barrier(false);
            // The chain wave reads the chunk's K fragments right after the barrier, between
            // the MFMAs of the pending state update; LDS stores issued at that moment delay
            // those reads on the chain's critical path. With outputs (and in the one-pass
            // summary) the stores wait ~770 cycles, with two tiles of outputs ~1,280, and
            // the operands still land an iteration before their use (stateful 32K forward
            // 0.612 -> 0.575 ms; delays of 384 to 1,024 cycles all help, 768 the most; the
            // segment apply of 8 x 4096 tokens, paired, is best at 1,280; the state pass
            // alone is slower with a delay).
            if constexpr (outputs || dual) __builtin_amdgcn_s_sleep(pair ? 20 : 12);
            store_k(n + 1, stage);
            if constexpr (outputs) store_q(n, stage);
            load_k(min(n + 3, last), stage);
            if constexpr (outputs) load_q(min(n + 2, last), stage);
        };
        // the K-side operands of the first chunk are in LDS before the barrier that opens
        // it; then the loads of iterations n0 - 2 (into st0) and n0 - 1 (into st1)
        load_k(min(n0, last), st0);
        store_k(n0, st0);
        load_k(min(n0 + 1, last), st0);
        if constexpr (outputs) load_q(min(n0, last), st0);
        load_k(min(n0 + 2, last), st1);
        if constexpr (outputs) load_q(min(n0 + 1, last), st1);
        int n = n0;
        for (; n + 1 <= n1; n += 2) {
            step(n, st0);
            step(n + 1, st1);
        }
        if (n <= n1) step(n, st0);
        };
        switch (wave - first_loader) {
            case 0: loader(IntTag<0>{}); break;
            case 1: loader(IntTag<1>{}); break;
            case 2: loader(IntTag<2>{}); break;
            case 3: loader(IntTag<3>{}); break;
            case 4: loader(IntTag<4>{}); break;
            case 5: loader(IntTag<5>{}); break;
            default: if constexpr (nl > 6) loader(IntTag<6>{}); break;
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    if (outputs && (wave == 1 || (pair && wave == 3) || (split_out && wave == 2))) {
        const int half = (split_out && wave == 2) ? 1 : 0;   // which two token tiles (split outputs)
        // ---------------- output wave: chunk n - 1 during chunk n ----------------
        // stores past the row's extent (the tail of a packed sequence's last chunk) are
        // dropped by the descriptor's range
        uint16_t* oout = static_cast<uint16_t*>(a.o) + rs.start * vo_row;
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(oout, rs.extent * vo_row * 2);
        const uint32_t ooff = static_cast<uint32_t>((l16 * vo_row + h * ncols + col0 + 4 * g4) * 2);
        // L2 prefetch, kPrefetch chunks ahead of the chain: the workgroups that read the
        // same lines split them, so that each line is fetched once per XCD (every line
        // costs an L1-to-L2 request slot for a full HBM latency). Lanes 0..31: the 256
        // lines of a chunk's k and q rows, split over the rep x tiles workgroups of the
        // query/key head (16 each when two value heads of 8 tiles share it); 32..47: v
        // rows, 48..59: That and P records, 60..63: decay factors, split over the tiles of
        // the value head. The data lands in a scratch LDS word per lane that nothing reads.
        constexpr int kPrefetch = 4;
        const unsigned char* pf_base;
        int64_t pf_stride;      // bytes per chunk
        int pf_row = -1;        // token row inside the chunk for q/k/v lines, else -1
        bool pf_lane = true;    // this lane has a line to fetch
        {
            const int64_t bT = rs.start;
            // (with two tiles per workgroup each output wave takes the share of one tile)
            const int vt = vtiles * tile + sub, vts = vtiles * tiles;
            const int qk_share = rep * vts, qk_rank = (kk % rep) * vts + vt;
            const int kq_lanes = min(32, (256 + qk_share - 1) / qk_share);
            if (lane < 32) {
                const int lam = kq_lanes * qk_rank + lane;
                pf_lane = lane < kq_lanes && lam < 256;
                const uint16_t* src = static_cast<const uint16_t*>(lam < 128 ? a.k : a.q);
                pf_row = (lam & 127) >> 1;
                pf_base = reinterpret_cast<const unsigned char*>(src + bT * qk_row + hq * DK + 64 * (lam & 1));
                pf_stride = qk_row * 2;
            } else if (lane < 48) {
                const int lam = 16 * vt + lane - 32;
                const int c = (64 * (lam & 1) < ncols) ? 64 * (lam & 1) : 0;
                pf_row = lam >> 1;
                pf_base = reinterpret_cast<const unsigned char*>(static_cast<const uint16_t*>(a.v) + bT * v_row +
                                                                  h * ncols + c);
                pf_stride = v_row * 2;
            } else if (lane < 60) {
                const int lam = (12 * vt + lane - 48) % 96;
                const uint16_t* rec = static_cast<const uint16_t*>(lam < 48 ? a.ws.that : a.ws.pmat);
                pf_base = reinterpret_cast<const unsigned char*>(rec + bh * a.NT * kTriRecord) + 128 * (lam % 48);
                pf_stride = kTriRecord * 2;
            } else {
                // the first 768 bytes of the 1 KiB decay record; even and odd tiles split them
                pf_base = reinterpret_cast<const unsigned char*>(a.ws.gates + bh * a.NT * kGateRecordMfma) +
                          128 * (lane - 60) + 384 * (vt & 1);
                pf_stride = kGateRecordMfma * 4;
            }
        }
        const uint32_t pf_lds = lds_addr(pf_s);
        auto prefetch = [&](int c) {
            const unsigned char* p;
            if (pf_row >= 0) {
                int64_t t = static_cast<int64_t>(c) * kChunk + pf_row;
                if (t > rs.extent - 1) t = rs.extent - 1;
                p = pf_base + t * pf_stride;
            } else {
                p = pf_base + static_cast<int64_t>(c) * pf_stride;
            }
            const uint32_t m0v = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(pf_lds));
            if (pf_lane)
                asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m0v), "v"(p) : "memory", "m0");
        };
        // a row or segment without chunks has no line to prefetch (the clamped token
        // index would fall before the row)
        const bool pf_on = kEnablePrefetch && n1 > n0 && half == 0;   // the tile's share: one wave
        if (pf_on)
            for (int c = n0 + 2; c < n0 + kPrefetch && c < n1; ++c) prefetch(c);
        const int last = n1 > 0 ? n1 - 1 : 0;
        // P goes from global memory straight into registers: its blocks are contiguous
        // 1 KiB records (lane l: 16 bytes at 16 l), loaded two chunks ahead into the
        // register set of the chunk's parity.
        const __amdgpu_buffer_rsrc_t rpm = make_rsrc(static_cast<const uint16_t*>(a.ws.pmat) + bh * a.NT * kTriRecord,
                                                     static_cast<int64_t>(a.NT) * kTriRecord * 2);
        const uint32_t voff_p = static_cast<uint32_t>(16 * lane);
        // with split outputs a wave loads the P blocks of its own token tiles: tiles 0 and 3
        // (blocks 0, 4, 5) or 1 and 2 (blocks 1, 2, 3); its first tile uses pp[0], its
        // second pp[1] and pp[2]
        constexpr int NPB = split_out ? 3 : 6;
        using PSet = bf16x8[NPB];
        PSet p0, p1;
        auto load_p = [&](int c, PSet& pp) {
#pragma unroll
            for (int i = 0; i < NPB; ++i) {
                const int blk = split_out ? (half ? 1 + i : (i == 0 ? 0 : 3 + i)) : i;
                pp[i] = __builtin_bit_cast(bf16x8, gload16(rpm, voff_p, static_cast<uint32_t>(c) * (kTriRecord * 2) +
                                                                            static_cast<uint32_t>(blk * 1024)));
            }
        };
        auto compute = [&](int m, const PSet& pp) {   // outputs of chunk m
            const unsigned char* hb = hst + (2 * sub + (m & 1)) * HB;
            const unsigned char* qs = qst + (m & 1) * QSB;
            const float* gs = reinterpret_cast<const float*>(gst + (m % 4) * 1024);
            bf16x8 sb[4], ub[2];
#pragma unroll
            for (int s = 0; s < 4; ++s) sb[s] = lds_frag_b(hb + s * 1024 + 16 * lane);
#pragma unroll
            for (int s = 0; s < 2; ++s) ub[s] = lds_frag_b(hb + (4 + s) * 1024 + 16 * lane);
#pragma unroll
            for (int ri = 0; ri < (split_out ? 2 : 4); ++ri) {
                const int r = split_out ? (half ? 1 + ri : 3 * ri) : ri;
                f32x4 o0 = zero4(), o1 = zero4();
#pragma unroll
                for (int s = 0; s < 4; s += 2) {
                    o0 = mfma16(sb[s], lds_frag_b(qs + r * 4096 + frag_lane[s]), o0);
                    o1 = mfma16(sb[s + 1], lds_frag_b(qs + r * 4096 + frag_lane[s + 1]), o1);
                }
                const float e = gs[128 + 16 * r + l16];   // exp(Gam) rq
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = e * (o0[j] + o1[j]);
                if constexpr (split_out) {
                    o = mfma16(ub[0], pp[ri == 0 ? 0 : 1], o);
                    if (ri == 1) o = mfma16(ub[1], pp[2], o);
                } else {
                    o = mfma16(ub[0], pp[tri_block(ri, 0)], o);
                    if (ri >= 2) o = mfma16(ub[1], pp[tri_block(ri, 1)], o);
                }
                const int64_t t = static_cast<int64_t>(m) * kChunk + 16 * r + l16;
                const bool ok = t < nvalid;
                const uint32_t w0 = ok ? pk2(o[0], o[1]) : 0u, w1 = ok ? pk2(o[2], o[3]) : 0u;
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, ro,
                                                      ooff + static_cast<uint32_t>(m) * ostep +
                                                          static_cast<uint32_t>(16 * r * vo_row * 2),
                                                      0, 0);
            }
        };
        // iteration n: outputs of chunk n - 1, then the P blocks of chunk n + 1 into the
        // same registers; chunk indices past the end are clamped (a repeated prefetch or
        // load of the last chunk), so that the body has no branches
        auto step = [&](int n, PSet& pp) {
            chunk_barrier(false);
            if (pf_on) prefetch(min(n + kPrefetch, last));
            compute(n - 1, pp);
            load_p(min(n + 1, last), pp);
        };
        load_p(min(n0, last), p0);
        load_p(min(n0 + 1, last), p1);
        chunk_barrier(false);   // iteration n0: no outputs yet
        if (pf_on) prefetch(min(n0 + kPrefetch, last));
        int n = n0 + 1;
        for (; n + 1 <= n1; n += 2) {
            step(n, p0);
            step(n + 1, p1);
        }
        if (n <= n1) step(n, p0);
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    if (wave != 0 && !dual && !(pair && wave == 2)) {   // (with split outputs waves 1 and 2 returned above)
        for (int n = n0; n <= n1; ++n) chunk_barrier(false);
        return;
    }

    // ---------------- chain wave(s) ----------------
    auto chain = [&](auto hv_tag, auto sp_tag, int init_mode, float* s_out) {
    constexpr bool cHasV = decltype(hv_tag)::value != 0;
    constexpr bool cSplit = decltype(sp_tag)::value != 0;
    // Iteration n (between the barriers that open chunks n and n + 1) first applies the
    // state update of chunk n - 1, whose operands (the transposed K fragments and V'')
    // were read and formed in iteration n - 1, while the K fragments of chunk n stream in
    // from LDS; then it runs K S, X and U of chunk n and reads the transposed K fragments
    // of chunk n during the K S steps. Chunk n's K buffer is free once the barrier that
    // opens chunk n + 1 has passed, and every read of it is complete by then.
    f32x4 S[8];
    {
        const int64_t blk = a.s_init_per_segment ? bh * a.P + seg : bh;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 32 * (t >> 1) + 8 * g4 + 4 * (t & 1) + j;
                float s0 = 0.f;
                if (init_mode == kInitLoad) s0 = a.s_init[blk * stile + static_cast<int64_t>(row) * ncols + col0 + l16];
                else if (init_mode == kInitIdentity) s0 = (row == col0 + l16) ? 1.f : 0.f;
                S[t][j] = s0;
            }
    }
    // Transposing reads of K: lane (c, g) of k-step s, half hf reads the 8-byte piece of
    // token 32s + 16hf + 4g + c / 4 at dk 32 (t / 2) + 8 (c % 4) + 4 (t % 2): quad block
    // 8s + 4hf + g, row c / 4 in it, granule 4 (t / 2) + c % 4, byte 8 (t % 2) of the granule.
    int tr_lane[4];
#pragma unroll
    for (int th = 0; th < 4; ++th)
        tr_lane[th] = g4 * 1024 + 256 * (l16 >> 2) + 16 * ((4 * th + (l16 & 3)) ^ (4 * (l16 >> 2) + g4));
    const int v_lane = 2 * (16 * (4 * g4 + (l16 >> 2)) + 4 * (l16 & 3));

    // operands of the pending state update (chunk n - 1): A fragments of K^T for state
    // tile t and token k-step s, and V'' = diag(exp(Gam_C - Gam)) U as B fragments
    u32x2 ktr[8][2][2];
    bf16x8 vb[2], vbl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) vb[s] = vbl[s] = bf16x8{};
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) ktr[t][s][0] = ktr[t][s][1] = u32x2{0u, 0u};

    // state update of the last chunk, applied after the barrier that follows it
    auto state_update = [&]() {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int s = i >> 3, t = i & 7;
            const bf16x8 kt = __builtin_bit_cast(
                bf16x8, u32x4{ktr[t][s][0][0], ktr[t][s][0][1], ktr[t][s][1][0], ktr[t][s][1][1]});
            S[t] = mfma16(kt, vb[s], S[t]);
            if constexpr (cSplit) S[t] = mfma16(kt, vbl[s], S[t]);
        }
    };
    for (int n = n0; n < n1; ++n) {
        chunk_barrier(false);
        const unsigned char* ks = kst + (n & 1) * KSB;
        const unsigned char* ts = ks + KB;
        const unsigned char* tls = ks + KB + TB;
        const unsigned char* vs = ks + KB + TB + LB + 2048 * sub;   // this chain's V tile
        const float* gs = reinterpret_cast<const float*>(gst + (n % 4) * 1024);
        unsigned char* hb = hst + (2 * sub + (n & 1)) * HB;

        // State update of chunk n - 1 (S already holds exp(Gam_C) S): S += K^T V'', state
        // tiles t, token k-steps s (zero operands before the first chunk, which adds
        // exact zeros). Between the MFMAs, the K fragments of chunk n for K S are read in
        // the order K S uses them (k-step major); kf[4 s + r] is token tile r.
        bf16x8 kf[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int s = i >> 3, t = i & 7;
            const bf16x8 kt = __builtin_bit_cast(
                bf16x8, u32x4{ktr[t][s][0][0], ktr[t][s][0][1], ktr[t][s][1][0], ktr[t][s][1][1]});
            S[t] = mfma16(kt, vb[s], S[t]);
            if constexpr (cSplit) S[t] = mfma16(kt, vbl[s], S[t]);
            kf[i] = lds_frag_b(ks + (i & 3) * 4096 + frag_lane[i >> 2]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // the remaining LDS operands of chunk n
        f32x4 eg[4];
        u32x2 vraw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            eg[r] = *reinterpret_cast<const f32x4*>(gs + 16 * r + 4 * g4);
            if constexpr (cHasV) vraw[r] = lds_read_tr(vs + 16 * r * 32 + v_lane);
        }
        bf16x8 th[6], thl[6];
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            th[j] = lds_frag_b(ts + j * 1024 + 16 * lane);
            if constexpr (cSplit) thl[j] = lds_frag_b(tls + j * 1024 + 16 * lane);
        }
        f32x4 egc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) egc[r] = *reinterpret_cast<const f32x4*>(gs + 64 + 16 * r + 4 * g4);
        const float egC = gs[192];   // exp(Gam_C)
        __builtin_amdgcn_sched_barrier(0);

        // the state of chunk n as bf16 B fragments of K S (and for the output wave)
        bf16x8 sb[4], sbl[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if constexpr (cSplit) pack_frag_split(S[2 * s], S[2 * s + 1], sb[s], sbl[s]);
            else sb[s] = pack_frag(S[2 * s], S[2 * s + 1]);
        }
        if constexpr (cHasV && !cSplit) {
            // for the backward: the state entering chunk n as bf16, transposed (lane (c, g)
            // holds column c at rows 32 s + 8 g .. + 7)
            if (a.states) {
                uint16_t* st = static_cast<uint16_t*>(a.states) +
                               ((bh * a.NT + n) * ncols + col0 + l16) * DK + 8 * g4;
#pragma unroll
                for (int s = 0; s < 4; ++s) *reinterpret_cast<bf16x8*>(st + 32 * s) = sb[s];
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        // K S for token tiles r, one accumulator per tile, k-steps s in turn; after each
        // k-step, eight transposing reads of K for the state update go out (into the
        // registers that k-step's fragments leave free).
        f32x4 c0[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int r = 0; r < 4; ++r) c0[r] = mfma16(kf[4 * s + r], sb[s], s == 0 ? zero4() : c0[r]);
            if constexpr (cSplit) {
#pragma unroll
                for (int r = 0; r < 4; ++r) c0[r] = mfma16(kf[4 * s + r], sbl[s], c0[r]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 2 * s + (q >> 1), ks2 = q & 1;
                const int o0 = 8 * ks2 * 1024 + 8 * (t & 1) + tr_lane[t >> 1];
                ktr[t][ks2][0] = lds_read_tr(ks + o0);
                ktr[t][ks2][1] = lds_read_tr(ks + o0 + 4 * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (outputs) {
#pragma unroll
            for (int s = 0; s < 4; ++s) *reinterpret_cast<bf16x8*>(hb + s * 1024 + 16 * lane) = sb[s];
        }

        // X = V - diag(exp Gam) K S for tokens 16r + 4g + j, column l16
        f32x4 x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 v4 = cHasV ? bf16x4_to_f32(vraw[r]) : zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) x[r][j] = v4[j] - eg[r][j] * c0[r][j];
        }
        bf16x8 xb[2], xbl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if constexpr (cSplit) pack_frag_split(x[2 * s], x[2 * s + 1], xb[s], xbl[s]);
            else xb[s] = pack_frag(x[2 * s], x[2 * s + 1]);
        }
        // the scaled old state, off the dependency chain (the fp32 S is next read by the
        // state update that opens the next iteration)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[t][j] *= egC;
        // U = That X (lower triangular: k-steps s <= r / 2)
        f32x4 u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            u[r] = zero4();
#pragma unroll
            for (int s = 0; s <= r / 2; ++s) {
                u[r] = mfma16(th[tri_block(r, s)], xb[s], u[r]);
                if constexpr (cSplit) {
                    u[r] = mfma16(th[tri_block(r, s)], xbl[s], u[r]);
                    u[r] = mfma16(thl[tri_block(r, s)], xb[s], u[r]);
                }
            }
        }
        if constexpr (outputs) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
                *reinterpret_cast<bf16x8*>(hb + (4 + s) * 1024 + 16 * lane) = pack_frag(u[2 * s], u[2 * s + 1]);
        }
        // V'' = diag(exp(Gam_C - Gam)) U, the B operand of the pending state update
        {
            f32x4 w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) w[r][j] = egc[r][j] * u[r][j];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if constexpr (cSplit) pack_frag_split(w[2 * s], w[2 * s + 1], vb[s], vbl[s]);
                else vb[s] = pack_frag(w[2 * s], w[2 * s + 1]);
            }
        }
    }
    chunk_barrier(false);
    state_update();

    if (a.store_mode == kStoreNone) return;
    if (a.store_mode == kStoreLastSegment && seg != a.P - 1) return;
    const int64_t blk = (a.store_mode == kStoreEverySegment) ? bh * a.P + seg : bh;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 32 * (t >> 1) + 8 * g4 + 4 * (t & 1) + j;
            s_out[blk * stile + static_cast<int64_t>(row) * ncols + col0 + l16] = S[t][j];
        }
    };
    if constexpr (dual) {
        if (wave < 2) chain(IntTag<0>{}, IntTag<1>{}, kInitIdentity, a.m_out);
        else chain(IntTag<1>{}, IntTag<0>{}, kInitZero, a.s_out);
    } else {
        chain(IntTag<kHasV ? 1 : 0>{}, IntTag<kSplit ? 1 : 0>{}, a.init_mode, a.s_out);
    }
}

}  // namespace

hipError_t launch_prep_mfma(const PrepArgs& a, hipStream_t s) {
    const int64_t pairs = static_cast<int64_t>(a.B) * a.NT;
    const dim3 grid(static_cast<unsigned>((pairs + 7) / 8 * 8 * a.H));
    void* args[] = {const_cast<PrepArgs*>(&a)};
    const void* fn = reinterpret_cast<const void*>(&prep_mfma<0>);
    if (a.has_conv) {
        switch (a.conv.K) {
            case 2: fn = reinterpret_cast<const void*>(&prep_mfma<2>); break;
            case 3: fn = reinterpret_cast<const void*>(&prep_mfma<3>); break;
            case 4: fn = reinterpret_cast<const void*>(&prep_mfma<4>); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
}

hipError_t launch_state_mfma(const StateArgs& a, hipStream_t s) {
    int qk_groups = a.Hqk * a.B * a.P;
    const int64_t groups = static_cast<int64_t>((qk_groups + 7) / 8) * 8 * (a.H / a.Hqk);
    // Workgroups per value head: one per 16-column tile, or per pair of tiles for M and S
    // in one pass. With outputs, pairs of tiles share their loads when one-tile
    // workgroups would take at least two rounds of the compute units (one workgroup runs
    // per unit): a pair's chunk costs well under two tiles' chunks.
    bool paired = false;
    if (a.pass == kPassOutputs && a.ncols % 32 == 0) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        paired = cus > 0 && groups * (a.ncols / 16) >= 2 * static_cast<int64_t>(cus);
    }
    int tiles = a.ncols / ((a.pass == kPassMS || paired) ? 32 : 16);
    if (a.pass == kPassMS && a.ncols % 32 != 0) return hipErrorInvalidValue;
    const unsigned nblk = static_cast<unsigned>(groups * tiles);
    void* args[] = {const_cast<StateArgs*>(&a), &tiles, &qk_groups};
    // The summary matrix M runs without values and with split operands; M and S together
    // in one pass share the loads. The caller names the pass (an empty tensor's pointer
    // may be NULL, so the pointers do not tell).
    const void* fn = nullptr;
    switch (a.pass) {
        case kPassOutputs:
            fn = paired ? reinterpret_cast<const void*>(&state_mfma<true, false, true, true>)
                        : reinterpret_cast<const void*>(&state_mfma<true, false, true>);
            break;
        case kPassS: fn = reinterpret_cast<const void*>(&state_mfma<true, false, false>); break;
        case kPassM: fn = reinterpret_cast<const void*>(&state_mfma<false, true, false>); break;
        case kPassMS: fn = reinterpret_cast<const void*>(&state_mfma<true, true, false>); break;
        default: return hipErrorInvalidValue;
    }
    // the split-operand passes read the bf16 remainder records of That
    if ((a.pass == kPassM || a.pass == kPassMS) && !a.ws.that_lo) return hipErrorInvalidValue;
    return hipLaunchKernel(fn, dim3(nblk), dim3(512), args, 0, s);
}

}  // namespace gdn
