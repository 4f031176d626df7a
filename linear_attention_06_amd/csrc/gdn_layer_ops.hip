// gdn_layer_ops.hip -- the two streaming steps around the Gated DeltaNet core in the
// layer the pages describe (hyper-parallel PR #1035 "linear attention cp", section "What
// does this PR do": the depthwise Conv1D runs on the projected Q/K/V before the Gated
// DeltaNet, and RMSNorm and gating run on its output before the output projection; the
// p2p mode exchanges only the left halo of the Conv1D between neighbouring ranks).
//
//   causal_conv1d   y[b,t,c] = act(bias[c] + sum_{j<K} w[c,j] x[b, t-K+1+j, c]), tokens
//                   before t = 0 taken from the halo x_prev[b, 0..K-2, c] (zero if none);
//                   act = SiLU or identity. Channels-last [B, T, C] layout.
//   gated_rmsnorm   y[r,:] = o[r,:] / sqrt(mean(o[r,:]^2) + eps) * weight * silu(z[r,:])
//                   over rows of D values (one token and head).
// Both are single passes over HBM: each input element is read once and each output
// written once, 16 bytes per lane in coalesced rows; all arithmetic is fp32.
#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 8 values per lane: bf16 (16 bytes) or fp32 (32 bytes). fetch() issues the load and
// unpack() widens it where it is used, so a load can stay in flight across iterations.
template <typename IO>
struct Vec8;
template <>
struct Vec8<uint16_t> {
    struct Raw {
        u32x4 u;
    };
    static __device__ __forceinline__ Raw fetch(const uint16_t* p) { return Raw{*reinterpret_cast<const u32x4*>(p)}; }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(r.u[e] << 16);
            x[2 * e + 1] = __uint_as_float(r.u[e] & 0xFFFF0000u);
        }
    }
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[8]) { unpack(fetch(p), x); }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[8]) {
        u32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * e]));
            const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * e + 1]));
            u[e] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(p) = u;
    }
};
template <>
struct Vec8<float> {
    struct Raw {
        u32x4 a, b;
    };
    static __device__ __forceinline__ Raw fetch(const float* p) {
        return Raw{*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 4)};
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = __uint_as_float(r.a[e]);
            x[4 + e] = __uint_as_float(r.b[e]);
        }
    }
    static __device__ __forceinline__ void load(const float* p, float (&x)[8]) { unpack(fetch(p), x); }
    static __device__ __forceinline__ void store(float* p, const float (&x)[8]) {
        *reinterpret_cast<u32x4*>(p) = u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                                             __float_as_uint(x[3])};
        *reinterpret_cast<u32x4*>(p + 4) = u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                                                 __float_as_uint(x[7])};
    }
};

// x sigmoid(x) with the hardware reciprocal (about 1 ulp) in place of a division
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// One thread per (b, group of 8 channels, run of kRun tokens); the K - 1 previous rows
// of its channels stay in registers as the window slides. Runs of 128 tokens: every block
// resident at once, four waves per SIMD, at T = 32768, C = 8192 (64: 0.226 ms, 128: 0.221 ms).
constexpr int kRun = 128;

template <typename IO, int K>
__global__ __launch_bounds__(256) void causal_conv1d(ConvArgs a) {
    const int64_t cg = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // channel group
    if (cg * 8 >= a.C) return;
    const int b = blockIdx.z;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kRun;
    const int c0 = static_cast<int>(cg * 8);
    const IO* x = static_cast<const IO*>(a.x) + static_cast<int64_t>(b) * a.T * a.C + c0;
    IO* y = static_cast<IO*>(a.y) + static_cast<int64_t>(b) * a.T * a.C + c0;
    float w[8][K], bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int j = 0; j < K; ++j) w[e][j] = a.w[static_cast<int64_t>(c0 + e) * K + j];
        bias[e] = a.bias ? a.bias[c0 + e] : 0.f;
    }
    // window: win[j] holds row t - K + 1 + j for the next output row t
    float win[K][8];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        const int64_t tt = t0 - (K - 1) + j;
        if (tt >= 0) {
            Vec8<IO>::load(x + tt * a.C, win[j]);
        } else if (a.x_prev) {
            // halo row K - 1 + tt of x_prev[b] (the tokens just before this sequence)
            Vec8<IO>::load(static_cast<const IO*>(a.x_prev) + (static_cast<int64_t>(b) * (K - 1) + (K - 1) + tt) * a.C + c0,
                           win[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
        }
    }
    const int64_t t1 = t0 + kRun < a.T ? t0 + kRun : a.T;
    // rows t + 1 and t + 2 in flight while row t is computed (t0 < T: the grid covers T)
    typename Vec8<IO>::Raw n1 = Vec8<IO>::fetch(x + t0 * a.C);
    typename Vec8<IO>::Raw n2 = t0 + 1 < t1 ? Vec8<IO>::fetch(x + (t0 + 1) * a.C) : n1;
    // unrolled so that the sliding window renames registers instead of copying them
#pragma unroll 4
    for (int64_t t = t0; t < t1; ++t) {
        const typename Vec8<IO>::Raw cur = n1;
        n1 = n2;
        if (t + 2 < t1) n2 = Vec8<IO>::fetch(x + (t + 2) * a.C);
        Vec8<IO>::unpack(cur, win[K - 1]);
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = bias[e];
#pragma unroll
            for (int j = 0; j < K; ++j) acc += w[e][j] * win[j][e];
            out[e] = a.silu ? silu(acc) : acc;
        }
        Vec8<IO>::store(y + t * a.C, out);
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) win[j][e] = win[j + 1][e];
    }
}

// D / 8 lanes per row (a power of two up to 16, consecutive lanes), 256 / (D / 8) rows
// per block; blocks stride over the rows when there are more than 2^30 blocks' worth.
template <typename IO, int D>
__global__ __launch_bounds__(256) void gated_rmsnorm(NormArgs a) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const int lane_in_row = threadIdx.x % LPR;
    float wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = a.weight[lane_in_row * 8 + e];
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR; r < a.rows;
         r += static_cast<int64_t>(gridDim.x) * RPB) {
        const int64_t off = r * D + lane_in_row * 8;
        float o[8], z[8];
        Vec8<IO>::load(static_cast<const IO*>(a.o) + off, o);
        Vec8<IO>::load(static_cast<const IO*>(a.z) + off, z);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += o[e] * o[e];
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, LPR);
        const float inv = 1.f / sqrtf(ss / D + a.eps);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = o[e] * inv * wv[e] * silu(z[e]);
        Vec8<IO>::store(static_cast<IO*>(a.y) + off, y);
    }
}

template <typename IO>
hipError_t conv_dispatch(const ConvArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((a.C / 8 + 255) / 256), static_cast<unsigned>((a.T + kRun - 1) / kRun),
                    static_cast<unsigned>(a.B));
    void* args[] = {const_cast<ConvArgs*>(&a)};
    const void* fn = nullptr;
    switch (a.K) {
        case 2: fn = reinterpret_cast<const void*>(&causal_conv1d<IO, 2>); break;
        case 3: fn = reinterpret_cast<const void*>(&causal_conv1d<IO, 3>); break;
        case 4: fn = reinterpret_cast<const void*>(&causal_conv1d<IO, 4>); break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
}

template <typename IO>
hipError_t norm_dispatch(const NormArgs& a, hipStream_t s) {
    // one row per lane group: every block is resident briefly and many rows are in flight
    // (a grid-striding loop over fewer blocks streams at 5.3 TB/s against 6.0)
    const int rpb = 256 / (a.D / 8);
    const int64_t need = (a.rows + rpb - 1) / rpb;
    const unsigned blocks = static_cast<unsigned>(need < (int64_t(1) << 30) ? need : (int64_t(1) << 30));
    void* args[] = {const_cast<NormArgs*>(&a)};
    const void* fn = nullptr;
    switch (a.D) {
        case 16: fn = reinterpret_cast<const void*>(&gated_rmsnorm<IO, 16>); break;
        case 32: fn = reinterpret_cast<const void*>(&gated_rmsnorm<IO, 32>); break;
        case 64: fn = reinterpret_cast<const void*>(&gated_rmsnorm<IO, 64>); break;
        case 128: fn = reinterpret_cast<const void*>(&gated_rmsnorm<IO, 128>); break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, s);
}

// nblk blocks of in_rows rows of in_row bytes copied into blocks of out_rows rows of out_row
// bytes (row sizes multiples of 16), 16 bytes a thread: output rows and row parts past the
// input's are zero (padding), input rows and row parts past the output's are dropped
// (cropping).
__global__ __launch_bounds__(256) void copy_blocks(const unsigned char* in, int64_t in_rows, int64_t in_row,
                                                   unsigned char* out, int64_t out_rows, int64_t out_row,
                                                   int64_t nblk) {
    const int64_t per_row = out_row / 16, per_blk = out_rows * per_row;
    const int64_t n = nblk * per_blk;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t blk = i / per_blk, e = i % per_blk, r = e / per_row, c = (e % per_row) * 16;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (r < in_rows && c < in_row) x = *reinterpret_cast<const u32x4*>(in + (blk * in_rows + r) * in_row + c);
        *reinterpret_cast<u32x4*>(out + (blk * out_rows + r) * out_row + c) = x;
    }
}

}  // namespace

hipError_t launch_copy_blocks(const void* in, int64_t in_rows, int64_t in_row, void* out, int64_t out_rows,
                              int64_t out_row, int64_t nblk, hipStream_t s) {
    if (nblk <= 0 || out_rows <= 0 || out_row <= 0) return hipSuccess;
    if (in_row % 16 || out_row % 16) return hipErrorInvalidValue;
    const int64_t n = nblk * out_rows * (out_row / 16);
    const int64_t need = (n + 255) / 256;
    const unsigned blocks = static_cast<unsigned>(need < 65536 ? need : 65536);
    const unsigned char* src = static_cast<const unsigned char*>(in);
    unsigned char* dst = static_cast<unsigned char*>(out);
    void* args[] = {&src, &in_rows, &in_row, &dst, &out_rows, &out_row, &nblk};
    return hipLaunchKernel(reinterpret_cast<const void*>(&copy_blocks), dim3(blocks), dim3(256), args, 0, s);
}

hipError_t launch_copy_rows(const void* in, int64_t in_row, void* out, int64_t out_row, int64_t rows, hipStream_t s) {
    return launch_copy_blocks(in, 1, in_row, out, 1, out_row, rows, s);
}

hipError_t launch_causal_conv1d(const ConvArgs& a, bool io_bf16, hipStream_t s) {
    return io_bf16 ? conv_dispatch<uint16_t>(a, s) : conv_dispatch<float>(a, s);
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, bool io_bf16, hipStream_t s) {
    return io_bf16 ? norm_dispatch<uint16_t>(a, s) : norm_dispatch<float>(a, s);
}

}  // namespace gdn
