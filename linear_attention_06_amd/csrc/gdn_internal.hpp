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

// How a state pass starts.
enum InitMode : int { kInitZero = 0, kInitLoad = 1, kInitIdentity = 2 };
// Where a state pass leaves its final state.
enum StoreMode : int { kStoreNone = 0, kStoreEverySegment = 1, kStoreLastSegment = 2 };

// Per-chunk intermediates written by the prepare pass, one record per
// (b, h, chunk), chunk-major within a head:
//   that  [64][64]  Tinv diag(beta), Tinv = (I + A)^{-1},
//                   A_ij = beta_i exp(Gam_i - Gam_j) k_i.k_j (i > j)
//   pmat  [64][64]  P_ij = (q_i.k_j) exp(Gam_i - Gam_j) for j <= i, else 0
//   gates [2][64]   exp(Gam_i) and exp(Gam_C - Gam_i), Gam = chunk-local cumsum of g
// The element type of that/pmat is fp32 on the fp32 path and bf16 on the
// matrix-core path; gates are always fp32.
struct Workspace {
    void* that;
    void* pmat;
    float* gates;
    void* that_lo;   // matrix-core path, segment calls only: bf16 remainder That - bf16(That), or NULL
};

struct PrepArgs {
    int B, T, H, Hqk, dk, NT;
    const void* q;
    const void* k;
    const float* g;
    const float* beta;
    const int32_t* valid_len;
    Workspace ws;
};

struct StateArgs {
    int B, T, H, Hqk, dk, ncols, NT;  // ncols = dv, or dk for the M summary
    int P, Lc;                        // segments and chunks per segment (P = 1, Lc = NT: whole sequence)
    const void* q;
    const void* k;
    const void* v;                    // NULL: values are zero (M summary)
    const int32_t* valid_len;
    Workspace ws;
    int init_mode;
    const float* s_init;              // [B,H,Pin,dk,ncols], Pin = P when loading per segment, else 1
    int s_init_per_segment;
    void* o;                          // NULL: no token output
    float* s_out;
    int store_mode;
    float* m_out;                     // matrix-core path: with v and no o, the M summary
                                      // (ncols = dk) computed in the same pass as S; else NULL
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

// Launchers. Each returns the HIP status of its launches.
hipError_t launch_prep_f32path(const PrepArgs& a, bool io_bf16, hipStream_t s);
hipError_t launch_state_f32path(const StateArgs& a, bool io_bf16, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, hipStream_t s);
hipError_t launch_prep_mfma(const PrepArgs& a, hipStream_t s);
hipError_t launch_state_mfma(const StateArgs& a, hipStream_t s);

}  // namespace gdn
