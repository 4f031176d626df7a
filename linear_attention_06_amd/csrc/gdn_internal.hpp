// gdn_internal.hpp -- types shared by the host entry points and the kernels of
// the chunked Gated DeltaNet forward (gfx950). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;
// bf16 elements of one That or P record on the matrix-core path (6 blocks of 64 x 8)
constexpr int kTriRecordElems = 6 * 512;
// fp32 words of one decay record: 128 on the fp32 path (exp(Gam), exp(Gam_C - Gam)),
// 256 on the matrix-core path (see prep_mfma)
constexpr int kGateRecordF32 = 128;
constexpr int kGateRecordMfma = 256;

// Token range of batch row b. Without cu_seqlens the rows are T tokens each, one after
// another, and token t of row b is valid when t < valid_len[b] (clamped to [0, T]); the
// row's outputs cover all T tokens (padding written as zero). With cu_seqlens (packed
// variable-length sequences, valid_len unused) row b is sequence b, tokens cu[b] ..
// cu[b+1] - 1 of the packed tensor of T tokens; the ends are clamped into [0, T] and the
// length to at most NT chunks, so that no value of cu_seqlens leads outside the tensors
// or the workspace; a sequence's outputs cover its own tokens only.
struct RowSpan {
    int64_t start;    // first token of the row in the token dimension
    int64_t valid;    // tokens that take part in the recurrence
    int64_t extent;   // tokens whose outputs the row writes
};
__device__ __forceinline__ RowSpan row_span(const int32_t* cu, const int32_t* vl, int b, int64_t T, int NT) {
    if (cu) {
        int64_t s = cu[b], e = cu[b + 1];
        s = s < 0 ? 0 : (s > T ? T : s);
        e = e < s ? s : (e > T ? T : e);
        const int64_t cap = static_cast<int64_t>(NT) * kChunk;
        const int64_t n = e - s > cap ? cap : e - s;
        return RowSpan{s, n, n};
    }
    int64_t n = T;
    if (vl) {
        n = vl[b];
        n = n < 0 ? 0 : (n > T ? T : n);
    }
    return RowSpan{static_cast<int64_t>(b) * T, n, T};
}

// How a state pass starts.
enum InitMode : int { kInitZero = 0, kInitLoad = 1, kInitIdentity = 2 };
// Which state pass to run. Stated by the caller, never inferred from NULL pointers: an
// empty tensor's data pointer may be NULL.
enum StatePass : int {
    kPassOutputs = 0,   // values, token outputs (forward, apply)
    kPassS = 1,         // values, no outputs (summary S)
    kPassM = 2,         // no values, split operands (summary M)
    kPassMS = 3         // M and S of each column tile in one pass
};
// Where a state pass leaves its final state.
enum StoreMode : int { kStoreNone = 0, kStoreEverySegment = 1, kStoreLastSegment = 2 };

// Per-chunk intermediates written by the prepare pass, one record per
// (b, h, chunk), chunk-major within a head:
//   that  [64][64]  Tinv diag(beta), Tinv = (I + A)^{-1},
//                   A_ij = beta_i exp(Gam_i - Gam_j) k_i.k_j (i > j)
//   pmat  [64][64]  P_ij = (q_i.k_j) exp(Gam_i - Gam_j) for j <= i, else 0
//   gates           fp32 decay factors, Gam = chunk-local cumsum of g:
//                   fp32 path [2][64]: exp(Gam_i), exp(Gam_C - Gam_i);
//                   matrix-core path [4][64]: exp(Gam_i) rk_i, exp(Gam_C - Gam_i) rk_i,
//                   exp(Gam_i) rq_i, then exp(Gam_C) and zeros, where rk_i and rq_i are the
//                   row factors of the fused prologue (1/|k_i|, q_scale/|q_i|) or 1
// The element type of that/pmat is fp32 on the fp32 path and bf16 on the
// matrix-core path.
struct Workspace {
    void* that;
    void* pmat;
    float* gates;
    void* that_lo;   // matrix-core path, segment calls only: bf16 remainder That - bf16(That), or NULL
};

// Input prologue of the layer, fused into the prepare pass (matrix-core path):
// q = q_raw q_scale / |q_raw|, k = k_raw / |k_raw| per token and query/key head,
// g = -exp(A_log[h]) softplus(a + dt_bias[h]), beta = sigmoid(b).
struct Prologue {
    const float* a;        // [B,T,H]
    const float* b;        // [B,T,H]
    const float* A_log;    // [H]
    const float* dt_bias;  // [H]
    float q_scale;
};

// The layer's causal depthwise Conv1D fused into the prepare pass (matrix-core path, with
// the prologue): the pass reads the projected channels before the convolution and writes
// its output y, whose q, k and v parts the state pass then reads (token stride C):
//   y[b,t,c] = SiLU(bias[c] + sum_{j<K} w[c,j] x[b, t-K+1+j, c]), tokens before t = 0
//   from x_prev[b, 0..K-2, c] (zero if NULL); channels q (Hqk dk), k (Hqk dk), v (H dv).
struct PrepConv {
    const uint16_t* x;        // [B,T,C] bf16
    const float* w;           // [C,K]
    const float* bias;        // [C] or NULL
    const uint16_t* x_prev;   // [B,K-1,C] bf16 or NULL
    uint16_t* y;              // [B,T,C] bf16
    int C, K;
};

// Records the prepare pass writes in addition for the matrix-core backward (all NULL in
// the forward), bf16, one per (b, h, chunk):
//   thatT, pT  That^T and P^T as the 6 upper-triangle 16x32 blocks (r, s) of the A operand of
//              v_mfma_f32_16x16x32_bf16 (lane l: row 16r + l % 16 at tokens 32s + 4 (l / 16) +
//              (e % 4) + 16 (e / 4), e = 0..7), blocks (0,0) (0,1) (1,0) (1,1) (2,1) (3,1);
//   t_rm, p_rm Tinv = (I + A)^{-1} and P, row-major [64][64].
struct BwdRecords {
    void* thatT = nullptr;
    void* pT = nullptr;
    void* t_rm = nullptr;
    void* p_rm = nullptr;
    int keep_pmat = 0;      // with the backward records, also the forward's P record (for outputs)
};

struct PrepArgs {
    int B, T, H, Hqk, dk, NT;
    const void* q;
    const void* k;
    const float* g;         // unused with a prologue
    const float* beta;      // unused with a prologue
    const int32_t* valid_len;
    const int32_t* cu_seqlens;  // packed sequences (see row_span), or NULL
    int64_t qk_stride;          // elements between consecutive tokens of q and k (Hqk dk if dense)
    Workspace ws;
    int has_prologue;       // 0: q, k, g, beta are used as given
    Prologue pro;
    int has_conv;           // the Conv1D runs in the pass (requires the prologue; q, k unused)
    PrepConv conv;
    BwdRecords bwd;         // matrix-core backward only
};

struct StateArgs {
    int B, T, H, Hqk, dk, ncols, NT;  // ncols = dv, or dk for the M summary
    int P, Lc;                        // segments and chunks per segment (P = 1, Lc = NT: whole sequence)
    int pass;                         // StatePass
    const void* q;
    const void* k;
    const void* v;                    // NULL: values are zero (M summary)
    const int32_t* valid_len;
    const int32_t* cu_seqlens;        // packed sequences (see row_span), or NULL
    int64_t qk_stride, v_stride;      // elements between consecutive tokens of q/k and of v
                                      // (Hqk dk and H ncols when dense; o is always dense)
    Workspace ws;
    int init_mode;
    const float* s_init;              // [B,H,Pin,dk,ncols], Pin = P when loading per segment, else 1
    int s_init_per_segment;
    void* o;                          // NULL: no token output
    float* s_out;
    int store_mode;
    float* m_out;                     // matrix-core path: with v and no o, the M summary
                                      // (ncols = dk) computed in the same pass as S; else NULL
    void* states = nullptr;           // matrix-core path, pass kPassS: bf16 [B,H,NT,ncols,dk], the
                                      // state entering every chunk, transposed; or NULL
};

// Reverse of the prefix combine (gdn_summary_combine_bwd): G = dhT (or 0); for p = P-1
// .. 0: dS_p = G, G <- M_p^T G + dH_in_p; dh0 = G. Then dM_p = dS_p H_in_p^T.
struct ScanBwdArgs {
    int B, H, P, dk, dv;
    const float* M;       // [B,H,P,dk,dk]
    const float* H_in;    // [B,H,P,dk,dv]
    const float* dH_in;   // [B,H,P,dk,dv]
    const float* dhT;     // [B,H,dk,dv] or NULL
    float* dM;            // [B,H,P,dk,dk]
    float* dS;            // [B,H,P,dk,dv]
    float* dh0;           // [B,H,dk,dv] or NULL
};

struct ScanArgs {
    // X_p = M_p X_{p-1} + (S_p or 0), p = 0..P-1; X_{-1} = init
    int B, H, P, dk, ncols;
    const float* M;       // [B,H,P,dk,dk]
    const float* S;       // [B,H,P,dk,ncols] or NULL
    int init_mode;
    const float* init;    // [B,H,dk,ncols] when loading
    float* x_before;      // [B,H,P,dk,ncols]: X_{p-1}, or NULL
    float* x_after;       // [B,H,P,dk,ncols]: X_p, or NULL
    float* x_final;       // [B,H,dk,ncols]: X_{P-1}, or NULL
};

// Backward (fp32 vector-ALU kernels in gdn_bwd.hip).
struct BwdArgs {
    int B, T, H, Hqk, dk, dv, NT;
    const void* q;            // [B,T,Hqk,dk]  io dtype
    const void* k;
    const void* v;            // [B,T,H,dv]    io dtype
    const void* d_o;          // [B,T,H,dv]    io dtype: gradient of o
    const float* g;           // [B,T,H]
    const float* beta;
    const float* h0;          // [B,H,dk,dv] or NULL
    const float* dhT;         // [B,H,dk,dv] gradient of the final state, or NULL
    const int32_t* valid_len;
    float* ckpt;              // workspace [B,H,8 NT,dv/16,16 dk]: state before every 8th token,
                              // each 16-column tile in the order of the threads holding it
    float* dqk_part;          // workspace [B,T,H,dv/16,2,dk]: dq, dk per column tile
    float* dgb_part;          // workspace [B,T,H,dv/16,2]: dg, dbeta per column tile
    float* dq_out;            // [B,T,Hqk,dk]
    float* dk_out;            // [B,T,Hqk,dk]
    float* dv_out;            // [B,T,H,dv]
    float* dg_out;            // [B,T,H]
    float* dbeta_out;         // [B,T,H]
    float* dh0_out;           // [B,H,dk,dv] or NULL
    // Segments: each batch row is P segments of L tokens (P = 1, L = T: the whole row),
    // run as independent sequences (grid rows B P). h0 and dh0 are then [B,H,P,dk,dv]
    // (segment p's incoming state and its gradient); dhT is [B,H,P,dk,dv] when
    // dhT_per_segment, else [B,H,dk,dv] for the last segment only (zero for the others).
    int P, L;
    int dhT_per_segment;
    int h0_identity;          // initial state I (dv == dk) instead of h0
    int v_zero;               // values are zero (v unread)
    int do_zero;              // output gradient is zero (d_o unread)
    int write_dv;             // 0: the value gradient is not wanted (dv_out unread)
    int accumulate;           // add into dq, dk, dv, dg, dbeta instead of writing them
};

// Chunked matrix-core backward (gdn_bwd_mfma.hip; bf16, dk = dv = 128). The prepare pass
// writes the forward records and BwdRecords; the forward state pass (kPassS with states)
// writes the state S_n entering every chunk; bwd_state_mfma runs the reverse chain per
// (b, h, 16 columns), writing dv and the gradient dS_n of the state leaving every chunk;
// bwd_grad_mfma forms dq, dk, dg and dbeta per (b, query/key head, chunk).
struct BwdMfmaArgs {
    int B, T, H, Hqk, NT;
    const void* q;            // [B,T,Hqk,128] bf16
    const void* k;
    const void* v;            // [B,T,H,128] bf16
    const void* d_o;          // [B,T,H,128] bf16
    const float* g;           // [B,T,H]
    const float* beta;
    const float* dhT;         // [B,H,128,128] or NULL
    const int32_t* valid_len;
    Workspace ws;             // that, pmat, gates of the prepare pass
    BwdRecords rec;
    const void* states;       // bf16 [B,H,NT,128 (dv),128 (dk)]: S_n^T
    void* dstates;            // bf16 [B,H,NT,128,128]: the gradient of the state leaving chunk n, transposed
    float* dq_out;            // [B,T,Hqk,128]
    float* dk_out;
    float* dv_out;            // [B,T,H,128]
    float* dg_out;            // [B,T,H]
    float* dbeta_out;
    float* dh0_out;           // [B,H,128,128] or NULL
    // v or d_o NULL: zero values / output gradient; dv_out NULL: dv not written;
    // accumulate: dq, dk, dv, dg, dbeta added to what the buffers hold
    int accumulate = 0;
};

// State blocks between the segment calls' layout [B, H, P, D, D] and segments as rows
// [B * P, H, D, D] (gdn_bwd_mfma.hip).
struct SegBlocksArgs {
    int B, H, P, D;
    const float* src;   // NULL: zero blocks (to_rows)
    float* dst;
    int to_rows;        // 1: segment-major to row-major; 0: back
    int last_only;      // to_rows with src [B, H, D, D] placed at the last segment
};
hipError_t launch_seg_state_blocks(const SegBlocksArgs& a, hipStream_t s);
hipError_t launch_seg_valid_len(const int32_t* vl, int B, int P, int L, int T, int32_t* out, hipStream_t s);

// Layer steps around the core (gdn_layer_ops.hip).
struct ConvArgs {
    int B, T, C, K, silu;
    const void* x;        // [B,T,C] io dtype
    const float* w;       // [C,K]
    const float* bias;    // [C] or NULL
    const void* x_prev;   // [B,K-1,C] io dtype (tokens before the sequence) or NULL
    void* y;              // [B,T,C] io dtype
};
struct NormArgs {
    int64_t rows;
    int D;
    float eps;
    const void* o;        // [rows,D] io dtype
    const void* z;        // [rows,D] io dtype
    const float* weight;  // [D]
    void* y;              // [rows,D] io dtype
};

// Launchers. Each returns the HIP status of its launches.
hipError_t launch_prep_f32path(const PrepArgs& a, bool io_bf16, hipStream_t s);
hipError_t launch_state_f32path(const StateArgs& a, bool io_bf16, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, hipStream_t s);
hipError_t launch_prep_mfma(const PrepArgs& a, hipStream_t s);
hipError_t launch_state_mfma(const StateArgs& a, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, bool io_bf16, hipStream_t s);
hipError_t launch_bwd_state_mfma(const BwdMfmaArgs& a, hipStream_t s);
hipError_t launch_bwd_grad_mfma(const BwdMfmaArgs& a, hipStream_t s);
hipError_t launch_scan_bwd(const ScanBwdArgs& a, hipStream_t s);
hipError_t launch_causal_conv1d(const ConvArgs& a, bool io_bf16, hipStream_t s);
hipError_t launch_gated_rmsnorm(const NormArgs& a, bool io_bf16, hipStream_t s);
// rows of in_row bytes into rows of out_row bytes, zero-padded or cut (multiples of 16)
hipError_t launch_copy_rows(const void* in, int64_t in_row, void* out, int64_t out_row, int64_t rows, hipStream_t s);
// nblk blocks of in_rows x in_row bytes into blocks of out_rows x out_row bytes, zero-padded
// or cut in both directions (row sizes multiples of 16)
hipError_t launch_copy_blocks(const void* in, int64_t in_rows, int64_t in_row, void* out, int64_t out_rows,
                              int64_t out_row, int64_t nblk, hipStream_t s);

}  // namespace gdn
