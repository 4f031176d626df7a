/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunked Gated DeltaNet forward.
 *
 * The method. Per batch row b and value head h, with a dk x dv state S:
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t
 * (Gated DeltaNet linear attention: one small recurrent state per head, named in
 * hyper-parallel PR #1035 "linear attention cp", section "What does this PR do").
 * It is evaluated in chunks of 64 tokens; issue #320 of the same project (the
 * test report for PR #1114, section 3.1) fixes chunk size 64 and head dim 128
 * for the fused backend. This library accepts chunk == 64 and
 * dk, dv in {16, 32, 64, 128}; the bf16 matrix-core path serves dk == 128.
 *
 * The segment calls follow the same PR's p2p and all_gather modes: each
 * segment of a sequence is summarised by the affine map H_out = M @ H_in + S,
 * the summaries are combined in order into each segment's incoming state, and
 * the segment's token outputs are then computed from its prepared chunk
 * intermediates. Here the segments are pieces of one sequence on one GPU.
 *
 * Conventions shared by every call:
 *   - Layouts are row-major and contiguous:
 *       q, k    [B, T, Hqk, dk]   io dtype
 *       v, o    [B, T, H, dv]     io dtype
 *       g, beta [B, T, H]         fp32 (g is the per-token log-decay, beta the
 *                                  delta-rule step)
 *       h0, hT  [B, H, dk, dv]    fp32
 *       M       [B, H, P, dk, dk] fp32;   S, H_in [B, H, P, dk, dv] fp32
 *   - Heads: H % Hqk == 0 and value head h reads query/key head h / (H / Hqk);
 *     this is the grouped copy of 16 query/key heads to 32 value heads that
 *     issue #320, section 4.1 describes, done as an index map instead of a copy.
 *   - Every pointer is device memory owned by the caller (except `p` and `bytes`,
 *     which are host pointers). The library allocates no memory and keeps no
 *     state between calls; calls are reentrant. The token tensors (q, k, v, o, d_o
 *     and the gradients dq, dk, dv) are 16-byte aligned (the kernels move them in
 *     16-byte pieces); a misaligned one is GDN_EINVAL.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *     the call returns after enqueueing. Results are visible after the caller
 *     synchronises that stream.
 *   - Inputs are read-only. Outputs are fully overwritten; the output of a
 *     padded token is written as +0.0. hT may alias h0; no other aliasing.
 *   - Padding (issue #320, section 5.2): token t of row b is valid when
 *     t < valid_len[b] (clamped to [0, T]); invalid tokens are treated as
 *     beta = 0, g = 0 with zero q, k, v, so they give zero output and leave the
 *     state unchanged. T need not be a multiple of 64.
 *   - Errors: arguments are checked before anything is launched; a failed check
 *     returns a status and enqueues nothing. A failed launch returns GDN_EHIP.
 *     Faults inside kernels surface at the caller's stream synchronisation.
 *     No C++ exception crosses this interface. gdn_last_error() gives a
 *     human-readable detail of the last failure on the calling thread.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_EINVAL = 1,        /* bad argument: null required pointer, negative size, H % Hqk != 0 */
    GDN_EUNSUPPORTED = 2,  /* well-formed but not implemented: chunk != 64, head dim, dtype */
    GDN_EWORKSPACE = 3,    /* workspace pointer null or smaller than the sizing call says */
    GDN_EHIP = 4           /* the HIP runtime refused a launch or a query */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct gdn_problem {
    int32_t B, T, H, Hqk, dk, dv;  /* sizes; B, T may be 0 */
    int32_t chunk;                 /* must be 64 */
    int32_t io_dtype;              /* gdn_dtype of q, k, v and o */
    const int32_t* valid_len;      /* device int32[B] or NULL (all T tokens valid) */
} gdn_problem;

/* Text for a status code (static storage). */
const char* gdn_status_string(gdn_status s);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* gdn_last_error(void);

/*
 * Kernel path a problem runs on (static string), or NULL for an invalid problem:
 *   "bf16-mfma"        -- bf16 I/O with dk == 128 (any dv of 16, 32, 64, 128): bf16
 *                         matrix-core contractions with fp32 accumulation and an fp32 state;
 *   "bf16-mfma-padded" -- bf16 I/O with dk < 128: gdn_chunk_fwd, gdn_chunk_fwd_varlen and
 *                         the segment calls run the dk == 128 matrix-core kernels on q and k
 *                         zero-padded to 128 columns (exact: the padded columns add zeros to
 *                         every product), the allocation-free forward included; the segment
 *                         backward calls run such a problem on the fp32 vector-ALU kernels
 *                         (gdn_chunk_bwd pads too, on rows of 256 tokens or more);
 *   "f32-mfma"         -- fp32 I/O with dk == 128: the forward calls' prepare and state
 *                         passes on fp32 matrix cores (v_mfma_f32_16x16x4_f32: fp32 products
 *                         and accumulation); the backward runs the fp32 token-level kernels;
 *   "f32-mfma-padded"  -- fp32 I/O with dk < 128: likewise on the fp32 matrix-core kernels
 *                         (the backward calls run the fp32 token-level kernels).
 */
const char* gdn_kernel_path(const gdn_problem* p);

/*
 * Workspace for gdn_chunk_fwd, in bytes, written to *bytes. The workspace holds
 * the per-chunk intermediates (the triangular-solve factor, the masked intra-chunk
 * q.k block and the chunk decay factors), and for heads with dk < 128 also q and k
 * padded to 128 columns and the initial and final states padded to 128 rows; its
 * contents are undefined on entry.
 */
gdn_status gdn_chunk_fwd_workspace(const gdn_problem* p, size_t* bytes);

/*
 * Full-sequence chunked forward: o (all tokens) and, when hT != NULL, the final
 * state. h0 == NULL starts from the zero state (the stateless use of issue #320,
 * section 4.1); otherwise h0 is the initial state (the stateful use).
 * ws must be 256-byte aligned and at least gdn_chunk_fwd_workspace() bytes.
 */
gdn_status gdn_chunk_fwd(const gdn_problem* p,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* h0,
                         void* o, float* hT,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * and results, without a workspace argument. The chunk records live in a static device
 * array of 64 MiB that every GPU loading the library holds until the process ends; its
 * device address is looked up once per device, on the first call made with that device
 * current. The call allocates nothing and calls no allocating routine. A problem whose
 * records exceed 64 MiB returns GDN_EWORKSPACE before anything is enqueued (the stateless
 * 8K workload, B = 1, T = 8192, H = 32, dk = dv = 128 on the matrix-core path, needs
 * 52 MiB); use gdn_chunk_fwd with a workspace for larger problems. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams, or host
 * threads without ordering) race and give undefined results; calls on one stream are
 * ordered. Nothing in the array has to start at zero (each call writes every record it
 * reads). Heads with dk < 128 run, as in gdn_chunk_fwd, on padded copies of q and k, which
 * share the array with the records (so the limit counts them too).
 */
gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* p,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* h0,
                                 void* o, float* hT, void* stream);

/*
 * Forward with the layer's input prologue fused into the chunk prepare pass
 * (PR #1035, section "What does this PR do": each rank projects Q/K/V/B/A and
 * runs the Gated DeltaNet on them; issue #320's gradient checks name the A_log
 * and dt_bias parameters of the decay gate). Per token t, query/key head and
 * value head h:
 *     q_t  = q_scale * q_raw_t / max(|q_raw_t|, 1e-12)      (L2 norm over dk)
 *     k_t  = k_raw_t / max(|k_raw_t|, 1e-12)
 *     g_t  = -exp(A_log[h]) * softplus(a_t + dt_bias[h]),   softplus(x) = log(1 + e^x)
 *     beta_t = 1 / (1 + exp(-b_t))
 * then the same forward as gdn_chunk_fwd on (q, k, v, g, beta). The norms are taken
 * in fp32 over the bf16 inputs and applied to the fp32 products, so q and k are
 * never rounded after normalisation.
 *   q_raw, k_raw [B, T, Hqk, dk] bf16;  v, o [B, T, H, dv] bf16;
 *   a, b [B, T, H] fp32;  A_log, dt_bias [H] fp32;  q_scale a finite float
 *   (1/sqrt(dk) for the usual attention scale);  h0, hT as in gdn_chunk_fwd.
 * Runs on the bf16 matrix-core path only (io_dtype GDN_BF16, dk == 128); other
 * problems return GDN_EUNSUPPORTED. Padded tokens (valid_len) are treated as
 * beta = 0, g = 0 whatever a and b hold. The workspace is gdn_chunk_fwd_workspace().
 */
gdn_status gdn_chunk_fwd_prologue(const gdn_problem* p,
                                  const void* q_raw, const void* k_raw, const void* v,
                                  const float* a, const float* b,
                                  const float* A_log, const float* dt_bias, float q_scale,
                                  const float* h0, void* o, float* hT,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * The same fused-prologue forward reading q_raw, k_raw and v straight out of one packed
 * tensor, as the Conv1D below produces it from the layer's projection:
 *   qkv [B, T, C] bf16, C = 2 Hqk dk + H dv; token t holds q_raw (Hqk x dk), then k_raw
 *   (Hqk x dk), then v (H x dv).
 * No split copy is made: the kernels read the three parts with the token stride C.
 * qkv must be 16-byte aligned. Everything else as gdn_chunk_fwd_prologue.
 */
gdn_status gdn_chunk_fwd_prologue_qkv(const gdn_problem* p, const void* qkv,
                                      const float* a, const float* b,
                                      const float* A_log, const float* dt_bias, float q_scale,
                                      const float* h0, void* o, float* hT,
                                      void* ws, size_t ws_bytes, void* stream);

/*
 * The same forward with the layer's causal depthwise Conv1D (kernel width conv_k in
 * {2, 3, 4}, SiLU) fused into the chunk prepare pass (PR #1035, section "What does this PR
 * do": the Conv1D runs on the projected Q, K and V before the Gated DeltaNet; its p2p mode
 * exchanges the Conv1D's left halo between ranks):
 *   x [B, T, C] bf16, C = 2 Hqk dk + H dv, the projected channels before the convolution
 *   (per token: q_raw, then k_raw, then v, as in gdn_chunk_fwd_prologue_qkv);
 *   conv_w [C, conv_k] fp32; conv_b [C] fp32 or NULL; x_prev [B, conv_k - 1, C] bf16 or
 *   NULL: the tokens before the sequence (a rank's left halo), zero if NULL;
 *   y [B, T, C] bf16 receives the convolution's output
 *     y[b,t,c] = SiLU(conv_b[c] + sum_{j<conv_k} conv_w[c,j] x[b, t-conv_k+1+j, c])
 *   (the arithmetic of gdn_causal_conv1d, bit for bit), which the state pass reads.
 * Then the fused prologue and the forward of gdn_chunk_fwd_prologue on y's q, k and v
 * parts; the prepare pass takes its q and k from the convolution in registers. Equal, bit
 * for bit, to gdn_causal_conv1d followed by gdn_chunk_fwd_prologue_qkv. bf16 matrix-core
 * path with dk = dv = 128 only; x, x_prev and y 16-byte aligned. y is written for every
 * token t < T (padded tokens included, as the standalone convolution writes them).
 */
gdn_status gdn_chunk_fwd_conv(const gdn_problem* p, const void* x, const float* conv_w,
                              const float* conv_b, const void* x_prev, int32_t conv_k,
                              const float* a, const float* b, const float* A_log,
                              const float* dt_bias, float q_scale, const float* h0,
                              void* y, void* o, float* hT, void* ws, size_t ws_bytes, void* stream);

/*
 * Packed variable-length sequences (the general form of issue #320's variable-length
 * case, section 5.2, where rows of one batch hold different numbers of valid tokens):
 * instead of B rows of T tokens with padding, the B sequences lie back to back in one
 * packed token dimension of p->T tokens,
 *   q, k [1, T, Hqk, dk];  v, o [1, T, H, dv];  g, beta [1, T, H],
 * sequence b at tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1 (cu_seqlens: device
 * int32[B + 1], non-decreasing from 0 to T). Each sequence runs its own recurrence from
 * h0[b] (h0, hT [B, H, dk, dv]; h0 NULL = zero states) and its chunks start at its own
 * first token, so the result for a sequence equals gdn_chunk_fwd on that sequence alone.
 * max_seqlen (host) bounds every sequence's length and sizes the workspace; p->valid_len
 * must be NULL. Only the tokens of the sequences are written. The kernels clamp the
 * cu_seqlens values into [0, T] and each length to max_seqlen rounded up to 64, so that no
 * value reads or writes outside the tensors; a sequence longer than that is cut there, and
 * the outputs of its tokens past the cut are left unwritten (undefined): the caller must
 * pass a max_seqlen of at least the longest sequence (the Python binding checks it).
 * Any head dims and dtypes gdn_chunk_fwd takes.
 */
gdn_status gdn_chunk_fwd_varlen_workspace(const gdn_problem* p, int32_t max_seqlen, size_t* bytes);
gdn_status gdn_chunk_fwd_varlen(const gdn_problem* p, const int32_t* cu_seqlens, int32_t max_seqlen,
                                const void* q, const void* k, const void* v,
                                const float* g, const float* beta, const float* h0,
                                void* o, float* hT,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of gdn_chunk_fwd (the gradients issue #320, section 4 of the test report for
 * PR #1114, checks: dq, dk, dv, dg, dbeta and dH0). Given the forward's inputs, the
 * gradient d_o of o ([B, T, H, dv], io dtype) and, when non-NULL, the gradient dhT of the
 * final state ([B, H, dk, dv] fp32; NULL = zero), writes
 *   dq, dk [B, T, Hqk, dk],  dv [B, T, H, dv],  dg, dbeta [B, T, H]   (all fp32; dq and dk
 *   summed over the value heads that read each query/key head)
 *   dh0 [B, H, dk, dv] fp32 when non-NULL (the gradient of h0; h0 NULL = zero state).
 * Padded tokens (valid_len) get zero gradients. Every head dim and dtype of the forward.
 * bf16 inputs with dk = dv = 128 on rows of 64 tokens or more (T >= 64, or T = 0) run the
 * chunked matrix-core backward (the transposes of the
 * chunk form's products on bf16 MFMAs with fp32 accumulation, relative error a few 1e-3,
 * within the bf16 bound issue #320 section 4.2 states for gradients): workspace per
 * (b, h, 64-token chunk) of 105 KiB (the prepare pass's records, the state entering the chunk
 * and the gradient of the state leaving it, bf16). bf16 inputs with dk or dv under 128 and
 * T >= 256 run the same backward on copies of q, k, v, d_o zero-padded to 128 columns and
 * of h0, dhT padded to 128 x 128 blocks, in the workspace (the padded columns add exact
 * zeros; the gradients are cut back to dk and dv). Every other problem runs the fp32
 * token-level backward on the vector ALUs, with the forward state recomputed from
 * checkpoints every 8 tokens (workspace 8 B H ceil(T/64) dk dv + B T H (dv/16) 2 (dk + 1)
 * fp32). ws must be 256-byte aligned and at least gdn_chunk_bwd_workspace() bytes; results
 * are deterministic (the same bits on every run).
 */
gdn_status gdn_chunk_bwd_workspace(const gdn_problem* p, size_t* bytes);
gdn_status gdn_chunk_bwd(const gdn_problem* p,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* h0,
                         const void* d_o, const float* dhT,
                         float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * The forward and backward of a training step with the forward's intermediates kept: the
 * backward of gdn_chunk_bwd (issue #320, section 4 of the test report for PR #1114) reruns
 * the chunk prepare pass and the forward state pass to rebuild what it needs; here the
 * forward keeps both in the caller's workspace.
 *   gdn_chunk_fwd_save: gdn_chunk_fwd (the same o and hT, bit for bit) that also leaves in ws
 *     the backward's chunk records and the state entering every chunk.
 *   gdn_chunk_bwd_saved: gdn_chunk_bwd (the same gradients, bit for bit) from that ws, for
 *     the same problem and inputs (q, k, v, g, beta unchanged since the forward; h0 is not
 *     needed again: the kept states hold it).
 * Only on the problems gdn_chunk_bwd runs on the chunked matrix-core kernels: bf16 inputs
 * with dk = dv = 128, or bf16 heads with dk or dv under 128 on rows of 256 tokens or more
 * (then q, k, v and h0 are padded to 128 columns / 128 x 128 blocks in ws, the padded problem's
 * forward is kept, o and hT are cut back, and the backward pads d_o and dhT and cuts the
 * gradients back, as gdn_chunk_bwd does); other problems get GDN_EUNSUPPORTED. ws: 256-byte
 * aligned, at least
 * gdn_chunk_fwd_save_workspace() bytes (the size gdn_chunk_bwd_workspace gives for the same
 * problem), owned by the caller between the two calls. Arguments as for gdn_chunk_fwd and
 * gdn_chunk_bwd.
 */
gdn_status gdn_chunk_fwd_save_workspace(const gdn_problem* p, size_t* bytes);
gdn_status gdn_chunk_fwd_save(const gdn_problem* p, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* h0, void* o, float* hT,
                              void* ws, size_t ws_bytes, void* stream);
gdn_status gdn_chunk_bwd_saved(const gdn_problem* p, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const void* d_o, const float* dhT,
                               float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * The layer steps around the core (PR #1035, section "What does this PR do": a
 * depthwise Conv1D on the projected Q/K/V before the Gated DeltaNet, whose left halo is
 * all the p2p mode exchanges between neighbouring ranks; RMSNorm and gating on its
 * output before the output projection). Both are single streaming passes in fp32
 * arithmetic over io-dtype tensors (GDN_F32 or GDN_BF16; pointers 16-byte aligned for
 * bf16, 32-byte for fp32).
 *
 * Causal depthwise Conv1D, channels last:
 *   y[b,t,c] = act(bias[c] + sum_{j<K} w[c,j] x[b, t-K+1+j, c]),  act = SiLU if apply_silu
 * x, y [B, T, C]; w [C, K] fp32; bias [C] fp32 or NULL; x_prev [B, K-1, C] or NULL: the
 * K - 1 tokens before each sequence (a rank's left halo; zeros if NULL). K in {2, 3, 4},
 * C % 8 == 0, B <= 65535, T <= 65535 * 128. y must not alias x.
 */
gdn_status gdn_causal_conv1d(int32_t B, int32_t T, int32_t C, int32_t K, int32_t io_dtype,
                             const void* x, const float* w, const float* bias, const void* x_prev,
                             int32_t apply_silu, void* y, void* stream);

/*
 * Gated RMSNorm over rows of D values (one token and value head of o):
 *   y[r,:] = o[r,:] / sqrt(mean(o[r,:]^2) + eps) * weight * z[r,:] * sigmoid(z[r,:])
 * o, z, y [rows, D]; weight [D] fp32 (shared by all rows); D in {16, 32, 64, 128}.
 * y may alias o.
 */
gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t D, int32_t io_dtype, const void* o, const void* z,
                             const float* weight, float eps, void* y, void* stream);

/*
 * Workspace for the segment calls (gdn_segment_summary, then
 * gdn_apply_initial_state on the same workspace). seg_len must be a positive
 * multiple of 64 that divides T; P = T / seg_len segments. Heads with dk < 128 run the
 * segment calls as the dk = 128 problem on q and k zero-padded to 128 columns (a padded
 * segment's transition is block-diagonal, so M's first dk rows and columns and S's first
 * dk rows are exact; H_in enters with zero rows below dk and hT is cut back); the
 * workspace then also holds the padded q and k and 128-row staging blocks.
 */
gdn_status gdn_segment_workspace(const gdn_problem* p, int32_t seg_len, size_t* bytes);

/*
 * Per-segment affine summary (PR #1035, p2p mode: H_out = M @ H_in + S):
 *   S[b,h,p] = the state reached over segment p from a zero state,
 *   M[b,h,p] = the product of the segment's token transitions
 *              exp(g_t)(I - beta_t k_t k_t^T), later tokens on the left.
 * Either output may be NULL to skip it. Leaves in ws the chunk intermediates that
 * gdn_apply_initial_state reuses. With valid_len, padded tokens are identities (M and S
 * are those of the valid tokens; a segment of padding only has M = I, S = 0).
 */
gdn_status gdn_segment_summary(const gdn_problem* p, int32_t seg_len,
                               const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               float* M, float* S,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Prefix combine of the summaries in segment order (PR #1035, all_gather mode):
 *   H_{-1} = h0 (zero if NULL);  H_in[p] = H_{p-1};  H_p = M_p H_{p-1} + S_p.
 * hT (nullable) receives H_{P-1}. M_prefix (nullable) receives M_p ... M_0.
 * All fp32; H_in and M_prefix use the [B,H,P,...] layouts above.
 */
gdn_status gdn_summary_combine(int32_t B, int32_t H, int32_t P, int32_t dk, int32_t dv,
                               const float* M, const float* S, const float* h0,
                               float* H_in, float* M_prefix, float* hT, void* stream);

/*
 * Token outputs of every segment from its incoming state H_in[b,h,p] (PR #1035,
 * p2p mode: once the initial state arrives, the local outputs come from the
 * prepared chunk intermediates). ws must be the workspace that
 * gdn_segment_summary filled for the same problem, seg_len and inputs. hT
 * (nullable) receives the state at the end of the last segment.
 */
gdn_status gdn_apply_initial_state(const gdn_problem* p, int32_t seg_len,
                                   const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   const float* H_in, void* o, float* hT,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * Backward through the segment calls. PR #1035's p2p mode passes the gradient of the
 * state backwards across its autograd boundary between ranks; here the three forward
 * calls each have a reverse, and composed they give the gradient of the unsplit forward:
 *   1. gdn_apply_initial_state_bwd: each segment's backward from its incoming state, from
 *      the output gradient d_o of its tokens (and, for the last segment, dhT): the inputs'
 *      gradients of that segment and dH_in, the gradient of every incoming state;
 *   2. gdn_summary_combine_bwd: from dH_in (and the combine's own hT gradient) to dM, dS
 *      and dh0;
 *   3. gdn_segment_summary_bwd with accumulate = 1: adds the summaries' share, through
 *      dM and dS, to the inputs' gradients of step 1.
 * All gradients are fp32 with the layouts of their forward tensors (dq, dk [B,T,Hqk,dk];
 * dv [B,T,H,dv]; dg, dbeta [B,T,H]; dH_in, dS [B,H,P,dk,dv]; dM [B,H,P,dk,dk]). Each segment
 * runs as a sequence of its own through gdn_chunk_bwd's kernels: the chunked matrix-core
 * backward for bf16 heads of 128 (gradients within the bf16 bound of issue #320 section
 * 4.2), the fp32 vector-ALU backward otherwise. Padded tokens (valid_len) get zero
 * gradients. seg_len as gdn_segment_summary.
 *
 * Workspace of the two backward calls that take one, in bytes (contents undefined on entry).
 */
gdn_status gdn_segment_bwd_workspace(const gdn_problem* p, int32_t seg_len, size_t* bytes);

/*
 * Backward of gdn_apply_initial_state: segment p runs from H_in[b,h,p]; d_o [B,T,H,dv]
 * (io dtype) is the gradient of all token outputs, dhT [B,H,dk,dv] (nullable: zero) that
 * of the last segment's end state. Writes dq, dk, dv, dg, dbeta and dH_in (nullable).
 */
gdn_status gdn_apply_initial_state_bwd(const gdn_problem* p, int32_t seg_len,
                                       const void* q, const void* k, const void* v,
                                       const float* g, const float* beta, const float* H_in,
                                       const void* d_o, const float* dhT,
                                       float* dq, float* dk, float* dv, float* dg, float* dbeta,
                                       float* dH_in, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of gdn_summary_combine: M and H_in as the combine used and produced them,
 * dH_in the gradient of H_in, dhT (nullable: zero) that of the combine's hT. With G the
 * gradient of H_p (G = dhT for p = P - 1): dS[p] = G, dM[p] = G H_in[p]^T, and the
 * gradient of H_{p-1} is M_p^T G + dH_in[p]; dh0 (nullable) receives that of H_{-1} = h0.
 */
gdn_status gdn_summary_combine_bwd(int32_t B, int32_t H, int32_t P, int32_t dk, int32_t dv,
                                   const float* M, const float* H_in, const float* dH_in,
                                   const float* dhT, float* dM, float* dS, float* dh0, void* stream);

/*
 * Backward of gdn_segment_summary: the gradients of sum(M dM) + sum(S dS) with respect to
 * k, v, g, beta (dq receives zeros: the summaries do not read q). dM or dS NULL is a zero
 * gradient. accumulate = 0 writes dq, dk, dv, dg, dbeta; accumulate = 1 adds to them.
 * S is the segment's recurrence from a zero state and M its homogeneous transition (zero
 * values, identity start); each is run backwards from its final-state gradient.
 */
gdn_status gdn_segment_summary_bwd(const gdn_problem* p, int32_t seg_len,
                                   const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   const float* dM, const float* dS,
                                   float* dq, float* dk, float* dv, float* dg, float* dbeta,
                                   int32_t accumulate, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
