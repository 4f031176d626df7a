/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet (GDN) forward,
 * its per-segment affine state summary, the summary prefix combine and the
 * apply-initial-state step.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this file's library. The GPU library never links or
 * calls it, and it includes no GPU header.
 *
 * What it computes (per batch row b, value head h, one token at a time):
 *
 *   S <- h0[b,h] (or 0)                      S is dk x dv
 *   for t = 0 .. T-1:
 *     if t >= valid_len[b]:  o[b,t,h,:] = 0, S unchanged        (padding)
 *     S  <- exp(g_t) * S                     decay first
 *     u  <- beta_t * (v_t - S^T k_t)         delta-rule error on the decayed state
 *     S  <- S + k_t u^T
 *     o_t <- S^T q_t                         output reads the updated state
 *   hT[b,h] <- S
 *
 * which is S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 * o_t = S_t^T q_t. The value head h reads query/key head h / (H / Hqk).
 *
 * Sources. The pages name the method (Gated DeltaNet linear attention, one
 * small recurrent state per head) in hyper-parallel PR #1035 "linear attention
 * cp", section "What does this PR do"; they do not write the recurrence out,
 * so it is taken in the published Gated DeltaNet form above (decay, then the
 * delta-rule update, then the read-out).
 *   - Segment summary H_out = M @ H_in + S, its packing, the prefix combine and
 *     the use of the combined state as the segment's initial state: same page,
 *     descriptions of the p2p and all_gather modes.
 *   - Grouped head copy (16 query/key heads copied to 32 value heads before
 *     the core): hyper-parallel issue #320 "Linear Attention CP fused-operator
 *     PR #1114 test report", section 4.1.
 *   - Stateless and stateful use (initial state absent or given, final state
 *     returned): same report, section 4.1.
 *   - Tail padding with B=2, T=8192, valid_length=7777 (pad tokens give zero
 *     output and leave the state alone): same report, section 5.2.
 *
 * Layouts (row-major, contiguous): q,k [B,T,Hqk,dk]; v,o [B,T,H,dv];
 * g,beta [B,T,H]; states [B,H,dk,dv]; M [B,H,P,dk,dk]; S,H_in [B,H,P,dk,dv].
 * All arithmetic is double precision in the order written; no reassociation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of valid tokens of row b: valid_len[b] clamped to [0, T], or T. */
static int64_t valid_tokens(const int32_t* valid_len, int b, int64_t T) {
    if (!valid_len) return T;
    int64_t n = valid_len[b];
    if (n < 0) n = 0;
    if (n > T) n = T;
    return n;
}

/*
 * One token of the recurrence on the state S (dk x dv), in place.
 * w is scratch of length dv. Writes o_t (length dv) when out != NULL.
 */
static void token_step(int dk, int dv, double* S, double* w,
                       const double* qt, const double* kt, const double* vt,
                       double gt, double bt, double* out) {
    const double decay = exp(gt);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= decay;
    /* w = S^T k */
    for (int j = 0; j < dv; ++j) w[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double ki = kt[i];
        for (int j = 0; j < dv; ++j) w[j] += S[(int64_t)i * dv + j] * ki;
    }
    /* u = beta (v - S^T k), kept in w */
    for (int j = 0; j < dv; ++j) w[j] = bt * (vt[j] - w[j]);
    /* S += k u^T */
    for (int i = 0; i < dk; ++i) {
        const double ki = kt[i];
        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += ki * w[j];
    }
    if (out) {
        /* o = S^T q */
        for (int j = 0; j < dv; ++j) out[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double qi = qt[i];
            for (int j = 0; j < dv; ++j) out[j] += S[(int64_t)i * dv + j] * qi;
        }
    }
}

/*
 * Runs tokens [t0, t1) of row b, value head h from the state S (in place).
 * Writes o for those tokens when o != NULL (zero for padded tokens).
 */
static void run_tokens(int64_t T, int H, int Hqk, int dk, int dv,
                       const double* q, const double* k, const double* v,
                       const double* g, const double* beta,
                       const int32_t* valid_len, int b, int h,
                       int64_t t0, int64_t t1, double* S, double* w, double* o) {
    const int hq = h / (H / Hqk);
    const int64_t nvalid = valid_tokens(valid_len, b, T);
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t row = (int64_t)b * T + t;
        double* ot = o ? o + (row * H + h) * dv : NULL;
        if (t >= nvalid) {
            if (ot)
                for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            continue;
        }
        token_step(dk, dv, S, w,
                   q + (row * Hqk + hq) * dk, k + (row * Hqk + hq) * dk,
                   v + (row * H + h) * dv, g[row * H + h], beta[row * H + h], ot);
    }
}

/*
 * Full-sequence forward: o [B,T,H,dv] and (when hT != NULL) the final state.
 * h0 == NULL means a zero initial state; valid_len == NULL means all T valid.
 */
void oracle_gdn_fwd(int B, int64_t T, int H, int Hqk, int dk, int dv,
                    const double* q, const double* k, const double* v,
                    const double* g, const double* beta,
                    const double* h0, const int32_t* valid_len,
                    double* o, double* hT) {
    const int units = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int b = u / H, h = u % H;
        const int64_t sz = (int64_t)dk * dv;
        double* S = (double*)malloc(sizeof(double) * (size_t)(sz + dv));
        double* w = S + sz;
        if (h0) memcpy(S, h0 + (int64_t)u * sz, sizeof(double) * (size_t)sz);
        else memset(S, 0, sizeof(double) * (size_t)sz);
        run_tokens(T, H, Hqk, dk, dv, q, k, v, g, beta, valid_len, b, h, 0, T, S, w, o);
        if (hT) memcpy(hT + (int64_t)u * sz, S, sizeof(double) * (size_t)sz);
        free(S);
    }
}

/*
 * Per-segment affine summary. The sequence is cut into P = T / seg_len
 * segments; for segment p of row b, head h:
 *   S_p = the state reached from a zero state over the segment's tokens,
 *   M_p = the product of the segment's token transitions
 *         exp(g_t) (I - beta_t k_t k_t^T), later tokens on the left,
 * so that the state after the segment is M_p H_in + S_p for any incoming H_in.
 * M_p is built one token at a time: M <- exp(g) M, then M <- M - beta k (k^T M).
 * Padded tokens are identity transitions. Either output may be NULL.
 */
void oracle_gdn_segment_summary(int B, int64_t T, int H, int Hqk, int dk, int dv,
                                int64_t seg_len,
                                const double* q, const double* k, const double* v,
                                const double* g, const double* beta,
                                const int32_t* valid_len, double* M, double* S) {
    const int64_t P = T / seg_len;
    const int64_t units = (int64_t)B * H * P;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t p = u % P;
        const int bh = (int)(u / P);
        const int b = bh / H, h = bh % H;
        const int hq = h / (H / Hqk);
        const int64_t nvalid = valid_tokens(valid_len, b, T);
        const int64_t ssz = (int64_t)dk * dv, msz = (int64_t)dk * dk;
        double* Sp = (double*)calloc((size_t)(ssz + dv + msz + dk), sizeof(double));
        double* w = Sp + ssz;
        double* Mp = w + dv;
        double* r = Mp + msz;
        for (int i = 0; i < dk; ++i) Mp[(int64_t)i * dk + i] = 1.0;
        for (int64_t t = p * seg_len; t < (p + 1) * seg_len; ++t) {
            if (t >= nvalid) continue;
            const int64_t row = (int64_t)b * T + t;
            const double* kt = k + (row * Hqk + hq) * dk;
            const double gt = g[row * H + h], bt = beta[row * H + h];
            if (S)
                token_step(dk, dv, Sp, w, NULL, kt, v + (row * H + h) * dv, gt, bt, NULL);
            if (M) {
                const double decay = exp(gt);
                for (int64_t e = 0; e < msz; ++e) Mp[e] *= decay;
                /* r = k^T M */
                for (int j = 0; j < dk; ++j) r[j] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dk; ++j) r[j] += kt[i] * Mp[(int64_t)i * dk + j];
                /* M -= beta k r */
                for (int i = 0; i < dk; ++i) {
                    const double c = bt * kt[i];
                    for (int j = 0; j < dk; ++j) Mp[(int64_t)i * dk + j] -= c * r[j];
                }
            }
        }
        if (S) memcpy(S + u * ssz, Sp, sizeof(double) * (size_t)ssz);
        if (M) memcpy(M + u * msz, Mp, sizeof(double) * (size_t)msz);
        free(Sp);
    }
}

/*
 * Prefix combine of the segment summaries, in segment order:
 *   H_{-1} = h0 (or 0);  H_in[p] = H_{p-1};  H_p = M_p H_{p-1} + S_p;  hT = H_{P-1}.
 * M_prefix[p] = M_p M_{p-1} ... M_0 when M_prefix != NULL. hT may be NULL.
 */
void oracle_gdn_summary_combine(int B, int H, int P, int dk, int dv,
                                const double* M, const double* S, const double* h0,
                                double* H_in, double* M_prefix, double* hT) {
    const int units = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int64_t ssz = (int64_t)dk * dv, msz = (int64_t)dk * dk;
        double* Hc = (double*)malloc(sizeof(double) * (size_t)(2 * ssz + 2 * msz));
        double* Hn = Hc + ssz;
        double* Pc = Hn + ssz;
        double* Pn = Pc + msz;
        if (h0) memcpy(Hc, h0 + (int64_t)u * ssz, sizeof(double) * (size_t)ssz);
        else memset(Hc, 0, sizeof(double) * (size_t)ssz);
        memset(Pc, 0, sizeof(double) * (size_t)msz);
        for (int i = 0; i < dk; ++i) Pc[(int64_t)i * dk + i] = 1.0;
        for (int p = 0; p < P; ++p) {
            const double* Mp = M + ((int64_t)u * P + p) * msz;
            const double* Sp = S + ((int64_t)u * P + p) * ssz;
            memcpy(H_in + ((int64_t)u * P + p) * ssz, Hc, sizeof(double) * (size_t)ssz);
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int l = 0; l < dk; ++l) acc += Mp[(int64_t)i * dk + l] * Hc[(int64_t)l * dv + j];
                    Hn[(int64_t)i * dv + j] = acc + Sp[(int64_t)i * dv + j];
                }
            memcpy(Hc, Hn, sizeof(double) * (size_t)ssz);
            if (M_prefix) {
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dk; ++j) {
                        double acc = 0.0;
                        for (int l = 0; l < dk; ++l) acc += Mp[(int64_t)i * dk + l] * Pc[(int64_t)l * dk + j];
                        Pn[(int64_t)i * dk + j] = acc;
                    }
                memcpy(Pc, Pn, sizeof(double) * (size_t)msz);
                memcpy(M_prefix + ((int64_t)u * P + p) * msz, Pc, sizeof(double) * (size_t)msz);
            }
        }
        if (hT) memcpy(hT + (int64_t)u * ssz, Hc, sizeof(double) * (size_t)ssz);
        free(Hc);
    }
}

/*
 * Apply the incoming states: segment p of row b, head h runs its tokens from
 * H_in[b,h,p] and writes their outputs; hT (nullable) receives the state at the
 * end of the last segment.
 */
void oracle_gdn_apply_initial_state(int B, int64_t T, int H, int Hqk, int dk, int dv,
                                    int64_t seg_len,
                                    const double* q, const double* k, const double* v,
                                    const double* g, const double* beta,
                                    const int32_t* valid_len, const double* H_in,
                                    double* o, double* hT) {
    const int64_t P = T / seg_len;
    const int64_t units = (int64_t)B * H * P;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t p = u % P;
        const int bh = (int)(u / P);
        const int b = bh / H, h = bh % H;
        const int64_t sz = (int64_t)dk * dv;
        double* S = (double*)malloc(sizeof(double) * (size_t)(sz + dv));
        double* w = S + sz;
        memcpy(S, H_in + u * sz, sizeof(double) * (size_t)sz);
        run_tokens(T, H, Hqk, dk, dv, q, k, v, g, beta, valid_len, b, h,
                   p * seg_len, (p + 1) * seg_len, S, w, o);
        if (hT && p == P - 1) memcpy(hT + (int64_t)bh * sz, S, sizeof(double) * (size_t)sz);
        free(S);
    }
}
