// gdn_mfma_common.hpp -- device helpers shared by the bf16 matrix-core kernels
// (forward in gdn_mfma.hip, backward in gdn_bwd_mfma.hip), gfx950 only.
//
// MFMA operand layouts (lane l):
//   32x32x16 bf16, q = l / 32, r = l % 32: A row r, k = 8q .. 8q+7; B col r, k = 8q .. 8q+7;
//     C register i holds row 8(i/4) + 4q + (i%4), col r.
//   16x16x32 bf16, g = l / 16: A row l%16, k = 8g .. 8g+7; B col l%16, k = 8g .. 8g+7;
//     C register j holds row 4g + j, col l%16.
//   16x16x4 f32: A row l%16, k = l/16;  B col l%16, k = l/16;  C rows 4(l/16)+j, col l%16.
#pragma once

#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int DK = 128;
// That and P leave the prepare kernel as the 6 lower-triangle 16x32 blocks (r, s),
// s <= r / 2, of 64 lanes x 8 bf16 each; block (r, s) sits at position tri_block(r, s).
constexpr int kTriRecord = kTriRecordElems;
__host__ __device__ constexpr int tri_block(int r, int s) { return r < 2 ? r : 2 + 2 * (r - 2) + s; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// A compile-time integer as a value (template arguments of generic lambdas).
template <int V>
struct IntTag {
    static constexpr int value = V;
};
// Inclusive prefix sum over each row of 16 lanes with DPP row shifts by 1, 2, 4, 8
// (lanes shifted in from outside the row read 0): lane 15 of a row ends with the row total.
__device__ __forceinline__ float row_prefix16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
    return x;
}
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// Two accumulator tiles (4 rows each per lane) as one bf16 B fragment.
__device__ __forceinline__ bf16x8 pack_frag(const f32x4& a, const f32x4& b) {
    bf16x8 f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f[u] = static_cast<__bf16>(a[u]);
        f[4 + u] = static_cast<__bf16>(b[u]);
    }
    return f;
}
// hi + lo split of the same pair: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void pack_frag_split(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const __bf16 ha = static_cast<__bf16>(a[u]), hb = static_cast<__bf16>(b[u]);
        hi[u] = ha;
        hi[4 + u] = hb;
        lo[u] = static_cast<__bf16>(a[u] - static_cast<float>(ha));
        lo[4 + u] = static_cast<__bf16>(b[u] - static_cast<float>(hb));
    }
}
__device__ __forceinline__ uint32_t pk2(float a, float b) {
    return bf16_bits(a) | (static_cast<uint32_t>(bf16_bits(b)) << 16);
}
__device__ __forceinline__ bf16x8 lds_frag_b(const unsigned char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte pieces addressed by lanes
// i/4, 4 + i/4, 8 + i/4, 12 + i/4 of its group.
__device__ __forceinline__ u32x2 lds_read_tr(const unsigned char* p) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
    lds_bf16x4* lp = (lds_bf16x4*)(const_cast<unsigned char*>(p));   // generic to LDS address space
#pragma clang diagnostic pop
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}
__device__ __forceinline__ f32x4 bf16x4_to_f32(u32x2 v) {
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                 __uint_as_float(v[1] & 0xFFFF0000u)};
}

constexpr int kBufferFlags = 0x00020000;   // raw buffer descriptor word 3 on gfx9-family GPUs

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int32_t n = static_cast<int32_t>(bytes < 0 ? 0 : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufferFlags);
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
#pragma clang diagnostic pop
}
// 16-byte load per lane from byte voff + off of a buffer into registers. The whole
// byte offset goes into the per-lane (VGPR) offset and the scalar offset is 0: the
// range check of a raw buffer covers the VGPR and instruction offsets only, so an
// offset placed in the scalar operand would let rows past the descriptor's end load
// real memory instead of zero.
__device__ __forceinline__ u32x4 gload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + off, 0, 0));
}
// Barrier of the state pass: this wave's LDS accesses complete, then s_barrier
// (optionally after all of its vector-memory accesses). One asm statement with a
// memory clobber, so the compiler keeps LDS accesses on their side of it.
__device__ __forceinline__ void chunk_barrier(bool vm_wait) {
    if (vm_wait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace
}  // namespace gdn
