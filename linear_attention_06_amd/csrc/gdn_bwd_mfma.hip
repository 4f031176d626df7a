// gdn_bwd_mfma.hip -- chunked backward of the Gated DeltaNet recurrence on bf16 matrix
// cores (gfx950), dk = dv = 128, in the chunk form of the forward (gdn_mfma.hip):
//   X = V - diag(e^Gam) K S,   U = That X,   That = Tinv diag(beta),  Tinv = (I + A)^{-1}
//   O = diag(e^Gam) Q S + P U, S' = e^{Gam_C} S + K^T diag(e^{Gam_C - Gam}) U
// (Gam the chunk-local cumulative log-decay, Gam_C its last entry). Reverse mode, with dO
// the output gradient of the chunk and dS' the gradient of the state leaving it:
//   dU = P^T dO + diag(e^{Gam_C - Gam}) K dS',  dX = That^T dU (= dV)
//   dS = e^{Gam_C} dS' + Q^T diag(e^Gam) dO - K^T diag(e^Gam) dX   (the state entering it)
// and, with Zf = diag(e^Gam) dO S^T, Zg = -diag(e^Gam) dX S^T, Zh = diag(e^{Gam_C - Gam}) U dS'^T,
// dP = (dO U^T) masked to j <= i, PD = dP . exp(Gam_i - Gam_j), dThat = dU X^T masked to
// j <= i, dA = -Tinv^T (dThat diag(beta)) Tinv^T masked to j < i, E = dA . beta_i exp(Gam_i - Gam_j):
//   dQ = Zf + PD K,   dK = Zg + Zh + PD^T Q + E K + E^T K
//   dbeta_j = sum_i dThat_ij Tinv_ij + sum_l dA_jl (K K^T)_jl exp(Gam_j - Gam_l)
//   dGam_t = <Zf_t, q_t> + <Zg_t, k_t> - W_t + sum_j (dP . P)_tj - sum_i (dP . P)_it
//            + sum_j (E . K K^T)_tj - sum_i (E . K K^T)_it,   W_t = <Zh_t, k_t>,
//   dGam_C += sum_t W_t + e^{Gam_C} <dS', S>,   dg_s = sum_{t >= s} dGam_t.
// The token recurrence is in hyper-parallel issue #320 (test report for PR #1114, section
// 4.1: the backward takes dO and the final-state gradient and returns the gradients of q,
// k, v, g, beta and the initial state); the chunk form is the published UT/WY form of
// Gated DeltaNet (Yang, Kautz and Hatamizadeh, 2025).
//
// Three passes after the prepare pass: the forward state pass stores the state S_n entering
// every chunk (bf16, transposed); bwd_state_mfma runs the reverse chain above per (b, h,
// 16 columns of dv), writing the gradient dS'_n of the state leaving every chunk;
// bwd_grad_mfma, one block per (b, query/key head, chunk), forms everything else (dv
// included) from S_n and dS'_n, with every product on v_mfma_f32_16x16x32_bf16 and fp32
// accumulation.
#include "gdn_mfma_common.hpp"

namespace gdn {
namespace {

constexpr int KPB = 272;   // LDS row pitch in bytes of 128 bf16 (256 B + 16)
constexpr int SPB = 144;   // LDS row pitch in bytes of 64 bf16 (128 B + 16)

// Block (r, s) of the upper-triangle records (That^T, P^T): (0,0) (0,1) (1,0) (1,1) (2,1) (3,1).
__host__ __device__ constexpr int tri_up(int r, int s) { return r < 2 ? 2 * r + s : r + 2; }

// Fragment of a matrix stored with its contraction index along LDS rows ("k-major": row
// k0 + e holds the 16 output rows or columns at 2-byte steps from c0): two transposing
// reads give lane (i, g) the values at rows k0 + 8 g .. + 7 of column c0 + i, the
// 16x16x32 operand layout. Lane p of a group addresses row k0 + 8 g + 4 hh + p / 4 at
// column c0 + 4 (p % 4).
__device__ __forceinline__ bf16x8 frag_kmajor(const unsigned char* base, int pitch, int k0, int c0, int l16, int g4) {
    const unsigned char* p = base + (k0 + 8 * g4 + (l16 >> 2)) * pitch + (c0 + 4 * (l16 & 3)) * 2;
    const u32x2 a = lds_read_tr(p), b = lds_read_tr(p + 4 * pitch);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}
// Fragment of a matrix stored with its contraction index contiguous ("row-major"): lane
// (i, g) reads row r0 + i at columns k0 + 8 g .. + 7.
__device__ __forceinline__ bf16x8 frag_rowmajor(const unsigned char* base, int pitch, int r0, int k0, int l16, int g4) {
    return lds_frag_b(base + (r0 + l16) * pitch + (k0 + 8 * g4) * 2);
}
// A 16x16 tile of a row-major bf16 matrix in accumulator order: lane (c, g) gets rows
// r0 + 4 g .. + 3 of column c0 + c.
__device__ __forceinline__ f32x4 tile_acc_order(const unsigned char* base, int pitch, int r0, int c0, int l16, int g4) {
    return bf16x4_to_f32(lds_read_tr(base + (r0 + 4 * g4 + (l16 >> 2)) * pitch + (c0 + 4 * (l16 & 3)) * 2));
}
// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then row broadcasts).
__device__ __forceinline__ float wave_scan64(float x) {
    x = row_prefix16(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, true));   // row_bcast:15
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, true));   // row_bcast:31
    return x;
}
// Sum over the 16 lanes of each row of the wave, every lane of the row gets it (DPP row
// rotations by 8, 4, 2, 1: no LDS traffic).
__device__ __forceinline__ float row_sum16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
    return x;
}
// Sum over the four lanes l % 16 == c (lanes c, c + 16, c + 32, c + 48), every one of them
// gets it: v_permlane16_swap pairs rows 0-1 and 2-3, v_permlane32_swap the two halves (the
// sum of a value and its swapped copy is the pair's sum in both lanes).
__device__ __forceinline__ float col_sum4(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// ----------------------------------------------------------------------------
// Reverse chain: one block of 8 waves per (b, h, 16 columns of dv), chunks from last to
// first, one barrier per iteration.
//   wave 0 (chain) carries the 128 x 16 slice of the state gradient in registers (the
//     forward state pass's layout: register t of lane (c, g), element j holds row
//     32 (t / 2) + 8 g + 4 (t % 2) + j of column c) and runs the dependent part of each
//     chunk: K dS', dU, dX = That^T dU and the update of dS (38 MFMAs);
//   wave 1 (helper) computes one chunk ahead the terms that do not depend on the state
//     gradient, P^T dO and Q^T diag(e^Gam) dO, and hands them over in LDS (fp32); one
//     chunk behind it writes the chain's dS' (bf16) to memory, so that the chain wave
//     issues no global memory instruction (dv = dX is formed again in the gradient pass,
//     which recomputes dU anyway);
//   waves 2-7 stage each chunk's operands two iterations ahead through registers: the
//     chain's (K, That^T, decay record) and the helper's (Q, P^T, dO, decay record).
// With c0 = NT - 1, iteration i has the helper on chunk c0 - i, the chain on c0 - i + 1
// and the stores of chunk c0 - i + 2; there are NT + 2 iterations.
// ----------------------------------------------------------------------------
// K and Q tiles in the forward state pass's layout (16 quad blocks of 4 token rows, 1 KiB
// each; granule gk of row 4 j + rho at 16-byte slot 16 rho + (gk ^ (4 rho + j % 4))): its
// fragment reads are free of bank conflicts and its transposing reads 2-way.
constexpr int RK_TT = 64 * 256, RK_G = RK_TT + 6144, RK_SIZE = RK_G + 1024;             // chain side
constexpr int RQ_PT = 64 * 256, RQ_DO = RQ_PT + 6144, RQ_G = RQ_DO + 2048, RQ_SIZE = RQ_G + 1024;   // helper side
constexpr int RA_SIZE = 12 * 1024;   // hand-off ahead: P^T dO (4 x 1 KiB), Q^T e^Gam dO (8 x 1 KiB), fp32
// hand-off behind: dS' as [16 columns][128] bf16 at a pitch of 272 bytes
constexpr int RB_DS = 0, RB_SIZE2 = 16 * 272;
constexpr int kRevLoadsK = 16 + 6 + 1, kRevLoadsQ = 16 + 6 + 2 + 1, kRevLoads = kRevLoadsK + kRevLoadsQ;
constexpr int kRevLoaders = 6;

__host__ __device__ constexpr int rev_loads_owned(int me) {
    int c = 0;
    for (int i = 0; i < kRevLoads; ++i) c += (i % kRevLoaders == me) ? 1 : 0;
    return c;
}

__global__ __launch_bounds__(512) void bwd_state_mfma(BwdMfmaArgs a, int qk_groups) {
    constexpr int tiles = DK / 16;
    __shared__ __align__(16) unsigned char kst[2 * RK_SIZE];
    __shared__ __align__(16) unsigned char qst[2 * RQ_SIZE];
    __shared__ __align__(16) unsigned char ahd[2 * RA_SIZE];
    __shared__ __align__(16) unsigned char bhd[2 * RB_SIZE2];
    __shared__ __align__(16) unsigned char pf_s[256];   // sink of the L2 prefetches

    // XCD-aware order as in the forward state pass: the column tiles of the value heads
    // that share a query/key head run on one XCD
    const int L = blockIdx.x;
    const int xcd = L & 7, slot = L >> 3;
    const int tile = slot % tiles;
    const int rep = a.H / a.Hqk;
    const int kk = slot / tiles;
    const int qg = (kk / rep) * 8 + xcd;
    if (qg >= qk_groups) return;
    const int b = qg / a.Hqk, hq = qg % a.Hqk;
    const int h = hq * rep + kk % rep;
    const int col0 = 16 * tile;
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const RowSpan rs = row_span(nullptr, a.valid_len, b, a.T, a.NT);
    const int64_t nvalid = rs.valid;
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    const int NT = a.NT, c0 = NT - 1, iters = NT + 2;
    const int64_t qk_row = static_cast<int64_t>(a.Hqk) * DK, v_row = static_cast<int64_t>(a.H) * DK;

    // Fragment (token tile r, dk step s) of a K or Q tile: byte 4096 r + frag_lane[s]; the
    // transposing read of state tile t over token step s: 8 KiB s + 8 (t % 2) + tr_lane[t / 2]
    // and 4 KiB further for the second half of the step's tokens.
    int frag_lane[4], tr_lane[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        frag_lane[q] = (l16 >> 2) * 1024 + 256 * (l16 & 3) + 16 * ((4 * q + g4) ^ (4 * (l16 & 3) + (l16 >> 2)));
        tr_lane[q] = g4 * 1024 + 256 * (l16 >> 2) + 16 * ((4 * q + (l16 & 3)) ^ (4 * (l16 >> 2) + g4));
    }

    if (wave >= 2) {
        if (NT == 0) return;
        // ---------------- loading waves ----------------
        const uint16_t* kin = static_cast<const uint16_t*>(a.k) + rs.start * qk_row;
        const uint16_t* qin = static_cast<const uint16_t*>(a.q) + rs.start * qk_row;
        // a NULL output gradient is zero: its descriptor holds no records, so its loads read 0
        const uint16_t* din = static_cast<const uint16_t*>(a.d_o ? a.d_o : a.k) + rs.start * v_row;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kin, nvalid * qk_row * 2);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qin, nvalid * qk_row * 2);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(din, a.d_o ? nvalid * v_row * 2 : 0);
        const int64_t rec = static_cast<int64_t>(NT) * kTriRecord * 2;
        const __amdgpu_buffer_rsrc_t rtt = make_rsrc(static_cast<const uint16_t*>(a.rec.thatT) + bh * NT * kTriRecord, rec);
        const __amdgpu_buffer_rsrc_t rpt = make_rsrc(static_cast<const uint16_t*>(a.rec.pT) + bh * NT * kTriRecord, rec);
        const __amdgpu_buffer_rsrc_t rgt = make_rsrc(a.ws.gates + bh * NT * kGateRecordMfma,
                                                     static_cast<int64_t>(NT) * kGateRecordMfma * 4);
        // lane l of the load of quad block j: row 4 j + l / 16, granule (l % 16) ^ (4 (l / 16) + j % 4)
        uint32_t voff_kq[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            voff_kq[jj] = static_cast<uint32_t>(((lane >> 4) * qk_row + hq * DK + 8 * ((lane & 15) ^ (4 * (lane >> 4) + jj))) * 2);
        const uint32_t voff_l = static_cast<uint32_t>(16 * lane);
        const uint32_t voff_d = static_cast<uint32_t>(((lane >> 1) * v_row + h * DK + col0 + 8 * (lane & 1)) * 2);
        const uint32_t kstep = static_cast<uint32_t>(kChunk * qk_row * 2), dstep = static_cast<uint32_t>(kChunk * v_row * 2);
        // load i of an iteration belongs to loading wave i % 6 (i < 23: the chain side of one
        // chunk, then the helper side of another); each wave's loop is compiled for its own
        // index, so that its stage registers are indexed at compile time
        auto loader = [&](auto me_tag) {
        constexpr int me = decltype(me_tag)::value;
        constexpr int NS = rev_loads_owned(me);
        using Stage = u32x4[NS];
        Stage st0, st1;
        // chain side of chunk ck, helper side of chunk cq (clamped to the first chunk)
        auto load = [&](int ck, int cq, Stage& st) {
            ck = ck < 0 ? 0 : ck;
            cq = cq < 0 ? 0 : cq;
#pragma unroll
            for (int i = me; i < kRevLoads; i += kRevLoaders) {
                u32x4& r = st[i / kRevLoaders];
                if (i < 16) r = gload16(rk, voff_kq[i & 3], static_cast<uint32_t>(4 * i * qk_row * 2) + static_cast<uint32_t>(ck) * kstep);
                else if (i < 22) r = gload16(rtt, voff_l, static_cast<uint32_t>(ck) * (kTriRecord * 2) + (i - 16) * 1024);
                else if (i < 23) r = gload16(rgt, voff_l, static_cast<uint32_t>(ck) * (kGateRecordMfma * 4u));
                else if (i < 39) r = gload16(rq, voff_kq[(i - 23) & 3], static_cast<uint32_t>(4 * (i - 23) * qk_row * 2) + static_cast<uint32_t>(cq) * kstep);
                else if (i < 45) r = gload16(rpt, voff_l, static_cast<uint32_t>(cq) * (kTriRecord * 2) + (i - 39) * 1024);
                else if (i < 47) r = gload16(rd, voff_d, static_cast<uint32_t>(32 * (i - 45) * v_row * 2) + static_cast<uint32_t>(cq) * dstep);
                else r = gload16(rgt, voff_l, static_cast<uint32_t>(cq) * (kGateRecordMfma * 4u));
            }
        };
        // into the buffers of the parities of ck and cq; a side whose chunk is negative (past
        // the first chunk) is not written
        auto store = [&](int ck, int cq, const Stage& st) {
            unsigned char* dk_ = kst + (ck & 1) * RK_SIZE;
            unsigned char* dq_ = qst + (cq & 1) * RQ_SIZE;
#pragma unroll
            for (int i = me; i < kRevLoads; i += kRevLoaders) {
                if ((i < kRevLoadsK ? ck : cq) < 0) continue;
                unsigned char* p;
                if (i < 16) p = dk_ + i * 1024 + 16 * lane;
                else if (i < 22) p = dk_ + RK_TT + (i - 16) * 1024 + 16 * lane;
                else if (i < 23) p = dk_ + RK_G + 16 * lane;
                else if (i < 39) p = dq_ + (i - 23) * 1024 + 16 * lane;
                else if (i < 45) p = dq_ + RQ_PT + (i - 39) * 1024 + 16 * lane;
                else if (i < 47) p = dq_ + RQ_DO + (i - 45) * 1024 + 16 * lane;
                else p = dq_ + RQ_G + 16 * lane;
                *reinterpret_cast<u32x4*>(p) = st[i / kRevLoaders];
            }
        };
        // iteration i stores the chain side of chunk c0 - i and the helper side of chunk
        // c0 - i - 1 (loaded two iterations before) and loads those of c0 - i - 2 and c0 - i - 3
        {
            Stage sq;
            load(c0, c0, sq);
            store(-1, c0, sq);   // the helper side of the first chunk, before the first barrier
        }
        load(c0, c0 - 1, st0);
        load(c0 - 1, c0 - 2, st1);
        for (int i = 0; i < iters; i += 2) {
            chunk_barrier(false);
            store(c0 - i, c0 - i - 1, st0);
            load(c0 - i - 2, c0 - i - 3, st0);
            if (i + 1 < iters) {
                chunk_barrier(false);
                store(c0 - i - 1, c0 - i - 2, st1);
                load(c0 - i - 3, c0 - i - 4, st1);
            }
        }
        };
        switch (wave - 2) {
            case 0: loader(IntTag<0>{}); break;
            case 1: loader(IntTag<1>{}); break;
            case 2: loader(IntTag<2>{}); break;
            case 3: loader(IntTag<3>{}); break;
            case 4: loader(IntTag<4>{}); break;
            default: loader(IntTag<5>{}); break;
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    if (wave == 1) {
        // ---------------- helper wave ----------------
        // L2 prefetch, a few chunks ahead of the loading waves: the workgroups that read the
        // same lines split them, so that each line is fetched from memory once per XCD and the
        // loading waves' requests hit the L2. Lanes 0..15: the 256 lines of a chunk's k and q
        // rows, split over the rep x 8 workgroups of the query/key head; 16..31: the 128 lines
        // of the value head's dO rows, 32..44: its That^T and P^T records (96 lines), 45..47:
        // its decay record, each split over the head's 8 column tiles. The data lands in a
        // scratch LDS word per lane that nothing reads.
        const unsigned char* pf_base = nullptr;
        int64_t pf_stride = 0;   // bytes per chunk
        int pf_row = -1;         // token row inside the chunk for q/k/dO lines, else -1
        bool pf_lane = true;
        {
            const int64_t bT = rs.start;
            const int qk_share = rep * tiles, qk_rank = (kk % rep) * tiles + tile;
            const int kq_lanes = min(16, (256 + qk_share - 1) / qk_share);
            if (lane < 16) {
                const int lam = kq_lanes * qk_rank + lane;
                pf_lane = lane < kq_lanes && lam < 256;
                const uint16_t* src = static_cast<const uint16_t*>(lam < 128 ? a.k : a.q);
                pf_row = (lam & 127) >> 1;
                pf_base = reinterpret_cast<const unsigned char*>(src + bT * qk_row + hq * DK + 64 * (lam & 1));
                pf_stride = qk_row * 2;
            } else if (lane < 32) {
                const int lam = 16 * tile + lane - 16;
                pf_lane = a.d_o != nullptr;
                pf_row = lam >> 1;
                pf_base = reinterpret_cast<const unsigned char*>(static_cast<const uint16_t*>(a.d_o ? a.d_o : a.k) + bT * v_row +
                                                                  h * DK + 64 * (lam & 1));
                pf_stride = v_row * 2;
            } else if (lane < 45) {
                const int lam = 13 * tile + lane - 32;
                pf_lane = lam < 96;
                const uint16_t* rec = static_cast<const uint16_t*>(lam < 48 ? a.rec.thatT : a.rec.pT);
                pf_base = reinterpret_cast<const unsigned char*>(rec + bh * NT * kTriRecord) + 128 * (lam % 48);
                pf_stride = kTriRecord * 2;
            } else if (lane < 48) {
                // the 1 KiB decay record: 8 lines over the 8 tiles' three lanes
                const int lam = 3 * tile + lane - 45;
                pf_lane = lam < 8;
                pf_base = reinterpret_cast<const unsigned char*>(a.ws.gates + bh * NT * kGateRecordMfma) + 128 * (lam & 7);
                pf_stride = kGateRecordMfma * 4;
            } else {
                pf_lane = false;
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
        // a row without chunks has no line to prefetch (the clamped token index would fall
        // before the row)
        const bool pf_on = NT > 0 && rs.extent > 0;
        if (pf_on) {
            prefetch(max(c0 - 2, 0));
            prefetch(max(c0 - 3, 0));
        }
        for (int i = 0; i < iters; ++i) {
            chunk_barrier(false);
            if (pf_on) prefetch(max(c0 - i - 4, 0));
            const int c = c0 - i;
            if (c >= 0) {
                const unsigned char* qs = qst + (c & 1) * RQ_SIZE;
                const float* gs = reinterpret_cast<const float*>(qs + RQ_G);
                // dO in accumulator order (tokens 16 r + 4 g + j, column c) and its fragments
                u32x2 dor[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) dor[r] = lds_read_tr(qs + RQ_DO + (16 * r + 4 * g4 + (l16 >> 2)) * 32 + 8 * (l16 & 3));
                bf16x8 dob[2], qb[2];
                {
                    f32x4 qv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const f32x4 egq = *reinterpret_cast<const f32x4*>(gs + 128 + 16 * r + 4 * g4);
                        const f32x4 dof = bf16x4_to_f32(dor[r]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) qv[r][j] = egq[j] * dof[j];
                    }
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        dob[s] = __builtin_bit_cast(bf16x8, u32x4{dor[2 * s][0], dor[2 * s][1], dor[2 * s + 1][0], dor[2 * s + 1][1]});
                        qb[s] = pack_frag(qv[2 * s], qv[2 * s + 1]);
                    }
                }
                unsigned char* ah = ahd + (c & 1) * RA_SIZE + 16 * lane;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    f32x4 pd = zero4();
#pragma unroll
                    for (int s = (r < 2 ? 0 : 1); s < 2; ++s) pd = mfma16(lds_frag_b(qs + RQ_PT + tri_up(r, s) * 1024 + 16 * lane), dob[s], pd);
                    *reinterpret_cast<f32x4*>(ah + r * 1024) = pd;
                }
                // Q^T diag(e^Gam) dO on the state tiles (the K^T fragments' row order)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int off = 8 * 1024 * s + 8 * (t & 1) + tr_lane[t >> 1];
                        const u32x2 q0 = lds_read_tr(qs + off), q1 = lds_read_tr(qs + off + 4 * 1024);
                        acc = mfma16(__builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]}), qb[s], acc);
                    }
                    *reinterpret_cast<f32x4*>(ah + (4 + t) * 1024) = acc;
                }
            }
            const int cs = c0 - i + 2;   // the chain's outputs of chunk cs
            if (i >= 2 && cs >= 0) {
                const unsigned char* bh_ = bhd + (cs & 1) * RB_SIZE2;
                // dS': store k writes the rows of columns 4 k + l / 16 whole (lane l: granule l % 16)
                uint16_t* st = static_cast<uint16_t*>(a.dstates) + (bh * NT + cs) * DK * DK;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int c = 4 * k + (lane >> 4), gr = lane & 15;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(bh_ + RB_DS + c * 272 + 16 * gr);
                    *reinterpret_cast<u32x4*>(st + (col0 + c) * DK + 8 * gr) = v;
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // ---------------- chain wave ----------------
    // The update of the state gradient by chunk n, dS -= K^T diag(e^Gam) dX, is applied at the
    // start of the next iteration (or after the last chunk), interleaved with the reads of the
    // next chunk's K fragments; its K^T fragments are read between the k-steps of K dS' (as in
    // the forward state pass, so that LDS reads overlap MFMAs instead of sitting between
    // dependent stages). Before the first chunk the pending operands are zero.
    f32x4 dS[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 32 * (t >> 1) + 8 * g4 + 4 * (t & 1) + j;
            dS[t][j] = a.dhT ? a.dhT[bh * DK * DK + row * DK + col0 + l16] : 0.f;
        }
    u32x2 ktr[8][2][2];
    bf16x8 wb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) wb[s] = bf16x8{};
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) ktr[t][s][0] = ktr[t][s][1] = u32x2{0u, 0u};
    auto kt_frag = [&](int t, int s) {
        return __builtin_bit_cast(bf16x8, u32x4{ktr[t][s][0][0], ktr[t][s][0][1], ktr[t][s][1][0], ktr[t][s][1][1]});
    };
    for (int i = 0; i < iters; ++i) {
        chunk_barrier(false);
        const int n = c0 - i + 1;
        if (i < 1 || n < 0) continue;
        const unsigned char* ks = kst + (n & 1) * RK_SIZE;
        const unsigned char* ah = ahd + (n & 1) * RA_SIZE + 16 * lane;
        unsigned char* bh_ = bhd + (n & 1) * RB_SIZE2;
        const float* gs = reinterpret_cast<const float*>(ks + RK_G);
        // pending update of chunk n + 1, with the K fragments of chunk n read in between
        // (kf[4 s + r]: token tile r, dk step s)
        bf16x8 kf[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int s = q >> 3, t = q & 7;
            dS[t] = mfma16(kt_frag(t, s), wb[s], dS[t]);
            kf[q] = lds_frag_b(ks + (q & 3) * 4096 + frag_lane[q >> 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // dS' (the gradient of the state leaving chunk n) as B fragments of K dS', handed to
        // the helper for the gradient pass
        bf16x8 sb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            sb[s] = pack_frag(dS[2 * s], dS[2 * s + 1]);
            *reinterpret_cast<bf16x8*>(bh_ + RB_DS + l16 * 272 + 16 * (4 * s + g4)) = sb[s];
        }
        f32x4 egc[4], eg[4], pd[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            egc[r] = *reinterpret_cast<const f32x4*>(gs + 64 + 16 * r + 4 * g4);
            eg[r] = *reinterpret_cast<const f32x4*>(gs + 16 * r + 4 * g4);
            pd[r] = *reinterpret_cast<const f32x4*>(ah + r * 1024);
        }
        bf16x8 th[6];
#pragma unroll
        for (int q = 0; q < 6; ++q) th[q] = lds_frag_b(ks + RK_TT + q * 1024 + 16 * lane);
        __builtin_amdgcn_sched_barrier(0);
        // K dS' for token tiles r, dk steps s in turn; after each step eight transposing reads
        // of K for the state update go out (into the registers that step frees)
        f32x4 c0r[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int r = 0; r < 4; ++r) c0r[r] = mfma16(kf[4 * s + r], sb[s], s == 0 ? zero4() : c0r[r]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 2 * s + (q >> 1), ts = q & 1;
                const int off = 8 * 1024 * ts + 8 * (t & 1) + tr_lane[t >> 1];
                ktr[t][ts][0] = lds_read_tr(ks + off);
                ktr[t][ts][1] = lds_read_tr(ks + off + 4 * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the scaled state gradient plus the helper's Q^T diag(e^Gam) dO, off the dependency
        // chain (the update that opens the next iteration adds -K^T diag(e^Gam) dX)
        const float egC = gs[192];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 qd = *reinterpret_cast<const f32x4*>(ah + (4 + t) * 1024);
#pragma unroll
            for (int j = 0; j < 4; ++j) dS[t][j] = egC * dS[t][j] + qd[j];
        }
        // dU = P^T dO + e^{Gam_C - Gam} K dS', dX = That^T dU
        f32x4 du[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) du[r][j] = pd[r][j] + egc[r][j] * c0r[r][j];
        bf16x8 dub[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) dub[s] = pack_frag(du[2 * s], du[2 * s + 1]);
        f32x4 dx[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dx[r] = zero4();
#pragma unroll
            for (int s = (r < 2 ? 0 : 1); s < 2; ++s) dx[r] = mfma16(th[tri_up(r, s)], dub[s], dx[r]);
        }
        // -diag(e^Gam) dX as the B operand of the pending update
        {
            f32x4 w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) w[r][j] = -eg[r][j] * dx[r][j];
#pragma unroll
            for (int s = 0; s < 2; ++s) wb[s] = pack_frag(w[2 * s], w[2 * s + 1]);
        }
    }
    // the update of the first chunk
#pragma unroll
    for (int q = 0; q < 16; ++q) dS[q & 7] = mfma16(kt_frag(q & 7, q >> 3), wb[q >> 3], dS[q & 7]);
    if (a.dh0_out) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 32 * (t >> 1) + 8 * g4 + 4 * (t & 1) + j;
                a.dh0_out[bh * DK * DK + row * DK + col0 + l16] = dS[t][j];
            }
    }
}

// ----------------------------------------------------------------------------
// Gradient pass: one block of 8 waves per (b, query/key head, chunk); the value heads that
// read the query/key head run in turn and their dq, dk are summed in registers (wave w
// holds columns 16 w .. + 15 of dq and dk for the 64 tokens). Per value head, in two
// panels of 64 columns of dv:
//   B  (waves 0-3, one 16-column slice each) X = V - e^Gam K S and U = That X; (waves 4-7)
//      dU = P^T dO + e^{Gam_C - Gam} K dS' and dX = That^T dU, written as dv; X, U,
//      e^{Gam_C - Gam} U, dU and -e^Gam dX go to LDS transposed (columns of dv as rows);
//   C  Zf, Zg, Zh (contractions over the panel's columns) into dq, dk and, through their
//      row products with q and k, into dGam; dP and dThat (lower 16x16 tiles) accumulated
//      over both panels;
// then D: PD, dT = dThat diag(beta) (Tinv and P read row-major), Y = dT Tinv^T,
// dA = -Tinv^T Y, K K^T, E; after the last value head dq += PD K, dk += PD^T Q + E K + E^T K
// on PD and E summed over the value heads. Per-token sums
// (dGam, dbeta) go through one LDS row per wave and are added in a fixed order, so the
// result does not depend on timing.
// ----------------------------------------------------------------------------
constexpr int G_K = 0, G_Q = G_K + 64 * KPB, G_ST = G_Q + 64 * KPB, G_DST = G_ST + 64 * KPB,
              G_V = G_DST + 64 * KPB, G_DO = G_V + 64 * SPB, G_DX = G_DO + 64 * SPB, G_XT = G_DX + 64 * SPB,
              G_UET = G_XT + 64 * SPB, G_UT = G_UET + 64 * SPB, G_DUT = G_UT + 64 * SPB, G_VEC = G_DUT + 64 * SPB,
              G_DVP = 68, G_DV = G_VEC + (4 * 64 + 2 * 8 * 64 + 32) * 4, G_SIZE = G_DV + 64 * G_DVP * 4;
// G_DV stages the panel's dv (fp32 [64 tokens][64 columns] at a pitch of 68 floats: the
// writes of a wave's accumulator tiles and the 16-byte row reads are free of bank conflicts)
// Phase D reuses: Tinv (row-major) in G_ST, P in G_DST, PD^T in G_XT, dT^T in G_UT, Y^T in
// G_UET, E^T in G_DUT.

// The 10 lower-triangle 16x16 tiles (ri >= ci) of a 64x64 matrix.
__device__ __forceinline__ void lower_tile(int q, int& ri, int& ci) {
    ri = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;
    ci = q - (ri * (ri + 1)) / 2;
}
__device__ __forceinline__ float wave_sum(float x) { return col_sum4(row_sum16(x)); }
__device__ __forceinline__ u32x2 pack4(const f32x4& v) { return u32x2{pk2(v[0], v[1]), pk2(v[2], v[3])}; }

// Lane index as a value the compiler must re-derive where it is used: the per-lane LDS
// addresses of each phase are then formed in that phase instead of being hoisted out of
// the loops and kept live (LDS offsets above 64 KiB do not fit the instruction's
// immediate field, so every hoisted address would hold a register).
__device__ __forceinline__ int fresh_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

// Zero granule e (0..191) of the six upper 16x16 tiles of a [j][i] (transposed) 64x64 bf16
// matrix at pitch SPB: tiles (row tile jt, column tile it) with it < jt.
__device__ __forceinline__ void zero_upper_tiles_t(unsigned char* base, int e) {
    const int tq = e >> 5, w16 = e & 31;
    const int jt = tq < 1 ? 1 : tq < 3 ? 2 : 3, it = tq - (jt * (jt - 1)) / 2;
    *reinterpret_cast<u32x4*>(base + (16 * jt + (w16 >> 1)) * SPB + 32 * it + 16 * (w16 & 1)) = u32x4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(512) void bwd_grad_mfma(BwdMfmaArgs a) {
    __shared__ __align__(16) unsigned char sm[G_SIZE];
    const int NT = a.NT;
    const int n = static_cast<int>(blockIdx.x % static_cast<unsigned>(NT));
    const int bq = static_cast<int>(blockIdx.x / static_cast<unsigned>(NT));
    const int hq = bq % a.Hqk, b = bq / a.Hqk;
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const RowSpan rs = row_span(nullptr, a.valid_len, b, a.T, NT);
    const int64_t nvalid = rs.valid;
    const int rep = a.H / a.Hqk;
    const int64_t qk_row = static_cast<int64_t>(a.Hqk) * DK, v_row = static_cast<int64_t>(a.H) * DK;
    const int64_t t0 = static_cast<int64_t>(n) * kChunk;
    float* gam_s = reinterpret_cast<float*>(sm + G_VEC);
    float* beta_s = gam_s + 64;
    float* eg_s = gam_s + 128;
    float* egc_s = gam_s + 192;
    float* part_g = gam_s + 256;   // [8 waves][64 tokens]
    float* part_b = gam_s + 768;
    float* misc = gam_s + 1280;    // e^{Gam_C}, per-wave W sums, per-wave <dS', S>
    const int m = wave;            // dq / dk column tile of this wave

    // K and Q of the chunk, zero past the valid tokens
    {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(a.k) + rs.start * qk_row, nvalid * qk_row * 2);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(a.q) + rs.start * qk_row, nvalid * qk_row * 2);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = tid + 512 * u, mat = p >> 10, e = p & 1023, row = e >> 4, gr = e & 15;
            const uint32_t off = static_cast<uint32_t>(((t0 + row) * qk_row + hq * DK + 8 * gr) * 2);
            *reinterpret_cast<u32x4*>(sm + (mat ? G_Q : G_K) + row * KPB + 16 * gr) = gload16(mat ? rq : rk, off, 0);
        }
    }
    f32x4 dq_acc[4], dk_acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dq_acc[r] = dk_acc[r] = zero4();

    // PD and E of the wave's lower 16x16 tiles (tile wave, and wave + 8 for waves 0 and 1),
    // summed over the value heads: dq += PD K and dk += PD^T Q + E K + E^T K are linear in
    // them, so those products run once per block
    f32x4 pd_acc[2], e_acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) pd_acc[i] = e_acc[i] = zero4();

    for (int kk = 0; kk < rep; ++kk) {
        const int h = hq * rep + kk;
        const int64_t bh = static_cast<int64_t>(b) * a.H + h, ch = bh * NT + n;
        // decay vectors of the chunk
        if (wave == 0) {
            const int64_t t = t0 + lane;
            const bool valid = t < nvalid;
            const int64_t gi = (rs.start + (valid ? t : 0)) * a.H + h;
            const float gv = valid ? a.g[gi] : 0.f, bv = valid ? a.beta[gi] : 0.f;
            const float gam = wave_scan64(gv);
            const float gamC = __shfl(gam, 63);
            gam_s[lane] = gam;
            beta_s[lane] = bv;
            eg_s[lane] = __expf(gam);
            egc_s[lane] = __expf(gamC - gam);
            if (lane == 0) misc[0] = __expf(gamC);
        }
        for (int p = tid; p < 1024; p += 512) part_g[p] = 0.f;   // part_g and part_b
        float sdot = 0.f, wsum = 0.f;
        f32x4 acc_pt[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) acc_pt[i] = zero4();
        chunk_barrier(false);

        for (int pn = 0; pn < 2; ++pn) {
            // ---- A: the panel's rows of S^T and dS'^T, and its columns of V and dO ----
            {
                const uint16_t* st = static_cast<const uint16_t*>(a.states) + (ch * DK + 64 * pn) * DK;
                const uint16_t* dst = static_cast<const uint16_t*>(a.dstates) + (ch * DK + 64 * pn) * DK;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int p = tid + 512 * u, row = p >> 4, gr = p & 15;
                    const u32x4 s1 = *reinterpret_cast<const u32x4*>(st + row * DK + 8 * gr);
                    const u32x4 s2 = *reinterpret_cast<const u32x4*>(dst + row * DK + 8 * gr);
                    *reinterpret_cast<u32x4*>(sm + G_ST + row * KPB + 16 * gr) = s1;
                    *reinterpret_cast<u32x4*>(sm + G_DST + row * KPB + 16 * gr) = s2;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sdot += __uint_as_float(s1[e] << 16) * __uint_as_float(s2[e] << 16) +
                                __uint_as_float(s1[e] & 0xFFFF0000u) * __uint_as_float(s2[e] & 0xFFFF0000u);
                }
                // NULL values or output gradient read as zero (descriptors without records)
                const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const uint16_t*>(a.v ? a.v : a.k) + rs.start * v_row,
                                                            a.v ? nvalid * v_row * 2 : 0);
                const __amdgpu_buffer_rsrc_t rd = make_rsrc(static_cast<const uint16_t*>(a.d_o ? a.d_o : a.k) + rs.start * v_row,
                                                            a.d_o ? nvalid * v_row * 2 : 0);
                {
                    const int row = tid >> 3, gr = tid & 7;
                    const uint32_t off = static_cast<uint32_t>(((t0 + row) * v_row + h * DK + 64 * pn + 8 * gr) * 2);
                    *reinterpret_cast<u32x4*>(sm + G_V + row * SPB + 16 * gr) = gload16(rv, off, 0);
                    *reinterpret_cast<u32x4*>(sm + G_DO + row * SPB + 16 * gr) = gload16(rd, off, 0);
                }
            }
            chunk_barrier(false);
            // ---- B ----
            {
                const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
                // That (waves 0-3) or P^T (waves 4-7) fragments of the chunk
                bf16x8 rf[6];
                {
                    const uint16_t* rp = static_cast<const uint16_t*>(wave < 4 ? a.ws.that : a.rec.pT) + ch * kTriRecord;
#pragma unroll
                    for (int j = 0; j < 6; ++j) rf[j] = *reinterpret_cast<const bf16x8*>(rp + j * 512 + lane * 8);
                }
                const int sg = wave & 3;
                f32x4 acc[4];
                const int sel = wave < 4 ? G_ST : G_DST;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[r] = zero4();
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc[r] = mfma16(frag_rowmajor(sm + G_K, KPB, 16 * r, 32 * s, l16, g4),
                                        frag_rowmajor(sm + sel, KPB, 16 * sg, 32 * s, l16, g4), acc[r]);
                }
                unsigned char* colrow = sm + (16 * sg + l16) * SPB + 8 * g4;   // + region + 32 r
                if (wave < 4) {
                    f32x4 x[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const f32x4 vv = tile_acc_order(sm + G_V, SPB, 16 * r, 16 * sg, l16, g4);
                        const f32x4 eg = *reinterpret_cast<const f32x4*>(eg_s + 16 * r + 4 * g4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) x[r][j] = vv[j] - eg[j] * acc[r][j];
                    }
                    bf16x8 xb[2];
#pragma unroll
                    for (int s = 0; s < 2; ++s) xb[s] = pack_frag(x[2 * s], x[2 * s + 1]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        f32x4 u = zero4();
#pragma unroll
                        for (int s = 0; s <= r / 2; ++s) u = mfma16(rf[tri_block(r, s)], xb[s], u);
                        const f32x4 egc = *reinterpret_cast<const f32x4*>(egc_s + 16 * r + 4 * g4);
                        f32x4 ue;
#pragma unroll
                        for (int j = 0; j < 4; ++j) ue[j] = egc[j] * u[j];
                        *reinterpret_cast<u32x2*>(colrow + G_XT + 32 * r) = pack4(x[r]);
                        *reinterpret_cast<u32x2*>(colrow + G_UT + 32 * r) = pack4(u);
                        *reinterpret_cast<u32x2*>(colrow + G_UET + 32 * r) = pack4(ue);
                    }
                } else {
                    u32x2 dor[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dor[r] = lds_read_tr(sm + G_DO + (16 * r + 4 * g4 + (l16 >> 2)) * SPB + (16 * sg + 4 * (l16 & 3)) * 2);
                    bf16x8 dob[2];
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        dob[s] = __builtin_bit_cast(bf16x8, u32x4{dor[2 * s][0], dor[2 * s][1], dor[2 * s + 1][0], dor[2 * s + 1][1]});
                    f32x4 du[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        f32x4 pd = zero4();
#pragma unroll
                        for (int s = (r < 2 ? 0 : 1); s < 2; ++s) pd = mfma16(rf[tri_up(r, s)], dob[s], pd);
                        const f32x4 egc = *reinterpret_cast<const f32x4*>(egc_s + 16 * r + 4 * g4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) du[r][j] = pd[j] + egc[j] * acc[r][j];
                        *reinterpret_cast<u32x2*>(colrow + G_DUT + 32 * r) = pack4(du[r]);
                    }
                    // dX = That^T dU (the value gradient): to LDS as -e^Gam dX, transposed, and
                    // to dv (zero past the valid tokens)
                    {
                        const uint16_t* rp = static_cast<const uint16_t*>(a.rec.thatT) + ch * kTriRecord;
#pragma unroll
                        for (int j = 0; j < 6; ++j) rf[j] = *reinterpret_cast<const bf16x8*>(rp + j * 512 + lane * 8);
                    }
                    bf16x8 dub[2];
#pragma unroll
                    for (int s = 0; s < 2; ++s) dub[s] = pack_frag(du[2 * s], du[2 * s + 1]);
                    float* dvs = reinterpret_cast<float*>(sm + G_DV) + 16 * sg + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        f32x4 dx = zero4();
#pragma unroll
                        for (int s = (r < 2 ? 0 : 1); s < 2; ++s) dx = mfma16(rf[tri_up(r, s)], dub[s], dx);
                        const f32x4 eg = *reinterpret_cast<const f32x4*>(eg_s + 16 * r + 4 * g4);
                        f32x4 dxe;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            dxe[j] = -eg[j] * dx[j];
                            dvs[(16 * r + 4 * g4 + j) * G_DVP] = dx[j];
                        }
                        *reinterpret_cast<u32x2*>(colrow + G_DX + 32 * r) = pack4(dxe);
                    }
                }
            }
            chunk_barrier(false);
            // the panel's dv, whole rows of 64 columns (zero past the valid tokens)
            if (a.dv_out) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int p = tid + 512 * u, row = p >> 4, q4 = p & 15;
                    const int64_t t = t0 + row;
                    if (t < a.T) {
                        f32x4 x = t < nvalid ? *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(sm + G_DV) + row * G_DVP + 4 * q4)
                                             : zero4();
                        f32x4* out = reinterpret_cast<f32x4*>(a.dv_out + (rs.start + t) * v_row + h * DK + 64 * pn + 4 * q4);
                        if (a.accumulate) x += *out;
                        *out = x;
                    }
                }
            }
            // ---- C ----
            {
                const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
                // the B operands (columns 16 m .. of S and dS', contraction over the panel's
                // columns of dv) serve all four token tiles
                bf16x8 stf[2], dstf[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    stf[s] = frag_kmajor(sm + G_ST, KPB, 32 * s, 16 * m, l16, g4);
                    dstf[s] = frag_kmajor(sm + G_DST, KPB, 32 * s, 16 * m, l16, g4);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // transposed products (the S-side fragments as the A operand): lane
                    // (l16, g4) holds token 16 r + l16 at dk columns 16 m + 4 g4 .. + 3, so
                    // that the dGam sum over dk is three adds and a sum over the lane groups
                    f32x4 zf = zero4(), zg = zero4(), zh = zero4();
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        zf = mfma16(stf[s], frag_rowmajor(sm + G_DO, SPB, 16 * r, 32 * s, l16, g4), zf);
                        zg = mfma16(stf[s], frag_kmajor(sm + G_DX, SPB, 32 * s, 16 * r, l16, g4), zg);
                        zh = mfma16(dstf[s], frag_kmajor(sm + G_UET, SPB, 32 * s, 16 * r, l16, g4), zh);
                    }
                    const float eg = eg_s[16 * r + l16];
                    const int qk_off = (16 * r + l16) * KPB + (16 * m + 4 * g4) * 2;
                    const f32x4 qv = bf16x4_to_f32(*reinterpret_cast<const u32x2*>(sm + G_Q + qk_off));
                    const f32x4 kv = bf16x4_to_f32(*reinterpret_cast<const u32x2*>(sm + G_K + qk_off));
                    float gp = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        zf[j] *= eg;
                        wsum += zh[j] * kv[j];
                        gp += zf[j] * qv[j] + (zg[j] - zh[j]) * kv[j];
                        dq_acc[r][j] += zf[j];
                        dk_acc[r][j] += zg[j] + zh[j];
                    }
                    gp = col_sum4(gp);
                    if (g4 == 0) part_g[wave * 64 + 16 * r + l16] += gp;
                    __builtin_amdgcn_sched_barrier(0);   // keeps each tile's operand reads with it
                }
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const int item = wave + 8 * i;
                    if (item >= 20) break;
                    int ri, ci;
                    lower_tile(item % 10, ri, ci);
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        if (item < 10)
                            acc_pt[i] = mfma16(frag_rowmajor(sm + G_DO, SPB, 16 * ri, 32 * s, l16, g4),
                                               frag_kmajor(sm + G_UT, SPB, 32 * s, 16 * ci, l16, g4), acc_pt[i]);
                        else
                            acc_pt[i] = mfma16(frag_kmajor(sm + G_DUT, SPB, 32 * s, 16 * ri, l16, g4),
                                               frag_kmajor(sm + G_XT, SPB, 32 * s, 16 * ci, l16, g4), acc_pt[i]);
                    }
                }
            }
            chunk_barrier(false);
        }

        // ---- D0: Tinv and P row-major; the upper tiles of dT^T are zero ----
        {
            const int row = tid >> 3, gr = tid & 7;
            *reinterpret_cast<u32x4*>(sm + G_ST + row * SPB + 16 * gr) =
                *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.rec.t_rm) + ch * 4096 + row * 64 + 8 * gr);
            *reinterpret_cast<u32x4*>(sm + G_DST + row * SPB + 16 * gr) =
                *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.rec.p_rm) + ch * 4096 + row * 64 + 8 * gr);
            if (tid < 192) zero_upper_tiles_t(sm + G_UT, tid);
        }
        chunk_barrier(false);
        // ---- D1: PD and dT from the dP and dThat tiles ----
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
            const int item = wave + 8 * i;
            if (item >= 20) break;
            int ri, ci;
            lower_tile(item % 10, ri, ci);
            const int J = 16 * ci + l16;
            const float gamJ = gam_s[J], betaJ = beta_s[J];
            f32x4 outv;
            float colacc = 0.f, rmine = 0.f;   // lane l16 < 4 keeps the row sum of row 4 g4 + l16
            const f32x4 mv = tile_acc_order(sm + (item < 10 ? G_DST : G_ST), SPB, 16 * ri, 16 * ci, l16, g4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int I = 16 * ri + 4 * g4 + j;
                const float d = I >= J ? acc_pt[i][j] : 0.f;
                if (item < 10) {
                    const float x = d * mv[j];   // dP . P
                    const float rsum = row_sum16(x);
                    rmine = l16 == j ? rsum : rmine;
                    colacc += x;
                    outv[j] = I >= J ? d * __expf(gam_s[I] - gamJ) : 0.f;
                } else {
                    colacc += d * mv[j];          // dThat . Tinv
                    outv[j] = d * betaJ;
                }
            }
            if (item < 10 && l16 < 4) part_g[wave * 64 + 16 * ri + 4 * g4 + l16] += rmine;
            colacc = col_sum4(colacc);
            if (g4 == 0) {
                if (item < 10) part_g[wave * 64 + J] -= colacc;
                else part_b[wave * 64 + J] += colacc;
            }
            if (item < 10) {
                if (i == 0) pd_acc[0] += outv;
                else pd_acc[1] += outv;
            } else {
                *reinterpret_cast<u32x2*>(sm + G_UT + J * SPB + (16 * ri + 4 * g4) * 2) = pack4(outv);
            }
        }
        chunk_barrier(false);
        // ---- D2: Y = dT Tinv^T (stored as Y^T), and K K^T on the tiles of D3 ----
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
            const int yt = 2 * wave + i, yi = yt >> 2, yj = yt & 3;
            f32x4 y = zero4();
#pragma unroll
            for (int s = 0; s < 2; ++s)
                y = mfma16(frag_kmajor(sm + G_UT, SPB, 32 * s, 16 * yi, l16, g4),
                           frag_rowmajor(sm + G_ST, SPB, 16 * yj, 32 * s, l16, g4), y);
            *reinterpret_cast<u32x2*>(sm + G_UET + (16 * yj + l16) * SPB + (16 * yi + 4 * g4) * 2) = pack4(y);
        }
        f32x4 kkt[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
            kkt[i] = zero4();
            const int q = wave + 8 * i;
            if (q >= 10) break;
            int ri, ci;
            lower_tile(q, ri, ci);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kkt[i] = mfma16(frag_rowmajor(sm + G_K, KPB, 16 * ri, 32 * s, l16, g4),
                                frag_rowmajor(sm + G_K, KPB, 16 * ci, 32 * s, l16, g4), kkt[i]);
        }
        chunk_barrier(false);
        // ---- D3: dA = -Tinv^T Y (strictly lower), E, and their dbeta / dGam terms ----
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
            const int q = wave + 8 * i;
            if (q >= 10) break;
            int ri, ci;
            lower_tile(q, ri, ci);
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 2; ++s)
                acc = mfma16(frag_kmajor(sm + G_ST, SPB, 32 * s, 16 * ri, l16, g4),
                             frag_rowmajor(sm + G_UET, SPB, 16 * ci, 32 * s, l16, g4), acc);
            const int J = 16 * ci + l16;
            const float gamJ = gam_s[J];
            f32x4 ev;
            float colacc = 0.f, bmine = 0.f, gmine = 0.f;   // row sums of row 4 g4 + l16, lanes l16 < 4
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int I = 16 * ri + 4 * g4 + j;
                const bool lower = I > J;
                const float ex = lower ? __expf(gam_s[I] - gamJ) : 0.f;
                const float da = lower ? -acc[j] : 0.f;
                const float dbr = row_sum16(da * kkt[i][j] * ex);
                const float e = da * beta_s[I] * ex;
                const float x = e * kkt[i][j];
                const float rsum = row_sum16(x);
                bmine = l16 == j ? dbr : bmine;
                gmine = l16 == j ? rsum : gmine;
                colacc += x;
                ev[j] = e;
            }
            if (l16 < 4) {
                part_b[wave * 64 + 16 * ri + 4 * g4 + l16] += bmine;
                part_g[wave * 64 + 16 * ri + 4 * g4 + l16] += gmine;
            }
            colacc = col_sum4(colacc);
            if (g4 == 0) part_g[wave * 64 + J] -= colacc;
            if (i == 0) e_acc[0] += ev;
            else e_acc[1] += ev;
        }
        chunk_barrier(false);
        {
            const float ws = wave_sum(wsum), sd = wave_sum(sdot);
            if (lane == 0) {
                misc[1 + wave] = ws;
                misc[9 + wave] = sd;
            }
        }
        chunk_barrier(false);
        // ---- D5: dGam and dbeta per token, dg = reverse cumulative sum of dGam ----
        if (wave == 0) {
            float dgam = 0.f, db = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                dgam += part_g[w * 64 + lane];
                db += part_b[w * 64 + lane];
            }
            if (lane == 63) {
                float ws = 0.f, sd = 0.f;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    ws += misc[1 + w];
                    sd += misc[9 + w];
                }
                dgam += ws + misc[0] * sd;
            }
            const float inc = wave_scan64(dgam);
            const float dg = __shfl(inc, 63) - inc + dgam;
            const int64_t t = t0 + lane;
            if (t < a.T) {
                const bool valid = t < nvalid;
                const int64_t o = (rs.start + t) * a.H + h;
                const float base_g = a.accumulate ? a.dg_out[o] : 0.f, base_b = a.accumulate ? a.dbeta_out[o] : 0.f;
                a.dg_out[o] = base_g + (valid ? dg : 0.f);
                a.dbeta_out[o] = base_b + (valid ? db : 0.f);
            }
        }
        chunk_barrier(false);
    }
    // ---- D4, once per block: PD^T and E^T of all value heads, then dq += PD K,
    // dk += PD^T Q + E K + E^T K ----
    {
        const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
        if (tid < 192) {
            zero_upper_tiles_t(sm + G_XT, tid);
            zero_upper_tiles_t(sm + G_DUT, tid);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = wave + 8 * i;
            if (q >= 10) break;
            int ri, ci;
            lower_tile(q, ri, ci);
            const int off = (16 * ci + l16) * SPB + (16 * ri + 4 * g4) * 2;
            *reinterpret_cast<u32x2*>(sm + G_XT + off) = pack4(pd_acc[i]);
            *reinterpret_cast<u32x2*>(sm + G_DUT + off) = pack4(e_acc[i]);
        }
    }
    chunk_barrier(false);
    {
        const int ln = fresh_lane(lane), l16 = ln & 15, g4 = ln >> 4;
        bf16x8 kt[2], qt[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            kt[s] = frag_kmajor(sm + G_K, KPB, 32 * s, 16 * m, l16, g4);
            qt[s] = frag_kmajor(sm + G_Q, KPB, 32 * s, 16 * m, l16, g4);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // transposed like the accumulators (the K / Q side as the A operand)
                dq_acc[r] = mfma16(kt[s], frag_kmajor(sm + G_XT, SPB, 32 * s, 16 * r, l16, g4), dq_acc[r]);
                dk_acc[r] = mfma16(qt[s], frag_rowmajor(sm + G_XT, SPB, 16 * r, 32 * s, l16, g4), dk_acc[r]);
                dk_acc[r] = mfma16(kt[s], frag_kmajor(sm + G_DUT, SPB, 32 * s, 16 * r, l16, g4), dk_acc[r]);
                dk_acc[r] = mfma16(kt[s], frag_rowmajor(sm + G_DUT, SPB, 16 * r, 32 * s, l16, g4), dk_acc[r]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // dq and dk of the query/key head (zero past the valid tokens): lane (l16, g4) holds
    // token 16 r + l16 at dk columns 16 m + 4 g4 .. + 3
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * r + l16;
        if (t < a.T) {
            const bool valid = t < nvalid;
            const int64_t o = ((rs.start + t) * a.Hqk + hq) * DK + 16 * m + 4 * g4;
            f32x4 xq = valid ? dq_acc[r] : zero4(), xk = valid ? dk_acc[r] : zero4();
            if (a.accumulate) {
                xq += *reinterpret_cast<const f32x4*>(a.dq_out + o);
                xk += *reinterpret_cast<const f32x4*>(a.dk_out + o);
            }
            *reinterpret_cast<f32x4*>(a.dq_out + o) = xq;
            *reinterpret_cast<f32x4*>(a.dk_out + o) = xk;
        }
    }
}

// Segments of B rows as rows of their own. State blocks (D x D fp32, 16 KiB at D = 128)
// move between the segment-major layout [B, H, P, D, D] of the segment calls and the
// row-major layout [B * P, H, D, D] of the backward on segments as rows: dst block
// (b P + p, h) is src block (b, h, p) (to_rows), or the reverse. src NULL gives zero
// blocks. With last_only, src is [B, H, D, D] and lands at p = P - 1, the other blocks zero.
__global__ __launch_bounds__(256) void seg_state_blocks(SegBlocksArgs a) {
    const int64_t n4 = static_cast<int64_t>(a.B) * a.P * a.H * a.D * a.D / 4;
    const int64_t blk4 = static_cast<int64_t>(a.D) * a.D / 4;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t blk = i / blk4, e = i % blk4;
        // blk in the row-major order: (b P + p) H + h
        const int h = static_cast<int>(blk % a.H);
        const int64_t bp = blk / a.H;
        const int p = static_cast<int>(bp % a.P), b = static_cast<int>(bp / a.P);
        const int64_t seg_blk = (static_cast<int64_t>(b) * a.H + h) * a.P + p;
        if (a.to_rows) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (a.src) {
                if (!a.last_only) x = reinterpret_cast<const float4*>(a.src)[seg_blk * blk4 + e];
                else if (p == a.P - 1) x = reinterpret_cast<const float4*>(a.src)[(static_cast<int64_t>(b) * a.H + h) * blk4 + e];
            }
            reinterpret_cast<float4*>(a.dst)[blk * blk4 + e] = x;
        } else {
            reinterpret_cast<float4*>(a.dst)[seg_blk * blk4 + e] = reinterpret_cast<const float4*>(a.src)[blk * blk4 + e];
        }
    }
}

// Valid tokens of every segment as a row: clamp(valid_len[b] - p L, 0, L).
__global__ __launch_bounds__(256) void seg_valid_len(const int32_t* vl, int B, int P, int L, int T, int32_t* out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= B * P) return;
    const int b = i / P, p = i % P;
    int n = vl[b];
    n = n < 0 ? 0 : (n > T ? T : n);
    n -= p * L;
    out[i] = n < 0 ? 0 : (n > L ? L : n);
}

}  // namespace

hipError_t launch_seg_state_blocks(const SegBlocksArgs& a, hipStream_t s) {
    const int64_t n4 = static_cast<int64_t>(a.B) * a.P * a.H * a.D * a.D / 4;
    if (n4 == 0) return hipSuccess;
    const int64_t nblk = (n4 + 255) / 256;
    const unsigned grid = static_cast<unsigned>(nblk < 4096 ? nblk : 4096);
    void* args[] = {const_cast<SegBlocksArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&seg_state_blocks), dim3(grid), dim3(256), args, 0, s);
}

hipError_t launch_seg_valid_len(const int32_t* vl, int B, int P, int L, int T, int32_t* out, hipStream_t s) {
    const int n = B * P;
    if (n == 0) return hipSuccess;
    void* args[] = {const_cast<int32_t**>(&vl), &B, &P, &L, &T, &out};
    return hipLaunchKernel(reinterpret_cast<const void*>(&seg_valid_len), dim3((n + 255) / 256), dim3(256), args, 0, s);
}

hipError_t launch_bwd_state_mfma(const BwdMfmaArgs& a, hipStream_t s) {
    int qk_groups = a.B * a.Hqk;
    const unsigned nblk = static_cast<unsigned>(((qk_groups + 7) / 8) * 8 * (a.H / a.Hqk) * (DK / 16));
    void* args[] = {const_cast<BwdMfmaArgs*>(&a), &qk_groups};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_state_mfma), dim3(nblk), dim3(512), args, 0, s);
}

hipError_t launch_bwd_grad_mfma(const BwdMfmaArgs& a, hipStream_t s) {
    const int64_t nblk = static_cast<int64_t>(a.B) * a.Hqk * a.NT;
    if (nblk == 0) return hipSuccess;
    void* args[] = {const_cast<BwdMfmaArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_grad_mfma), dim3(static_cast<unsigned>(nblk)), dim3(512),
                           args, 0, s);
}

}  // namespace gdn
