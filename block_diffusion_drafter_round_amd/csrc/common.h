// Device-side helpers shared by the gfx950 kernels of libdflash.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DFL_WAVE 64

// storage types (same values as the public DFLASH_* constants)
enum { WT_F32 = 0, WT_BF16 = 1, WT_FP8 = 2 };

// ---------------------------------------------------------------------------
// MFMA on gfx950.  Lane layouts (lane l, g = l / 16):
//   16x16x32 bf16: A[row l%16][k 8g..8g+7], B[k 8g..8g+7][col l%16],
//                  C[row 4g+j][col l%16], j = 0..3.
//   16x16x4 f32:   A[row l%16][k g], B[k g][col l%16], C as above.
// Any permutation of the reduction index k is allowed, as long as A and B
// use the same one.  The kernels rely on this to load each lane's operands
// as contiguous 16-byte pieces.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 bit patterns <-> float
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// round-to-nearest-even f32 pair -> packed bf16 bits, a in the low half
// (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t bf16_pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// round-to-nearest-even f32 -> bf16 bits
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return bf16_pack(f, 0.f) & 0xFFFFu; }

// Split 8 floats into bf16 hi + lo parts, hi = rne(x), lo = rne(x - hi).
// hi + lo carries about 16 significant bits, so a bf16 MFMA over (hi, lo)
// keeps the activation side close to f32 precision.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = bf16_pack(x[2 * i], x[2 * i + 1]);
        const float r0 = x[2 * i] - __uint_as_float(h[i] << 16), r1 = x[2 * i + 1] - __uint_as_float(h[i] & 0xFFFF0000u);
        l[i] = bf16_pack(r0, r1);
    }
    u32x4 hv = {h[0], h[1], h[2], h[3]};
    u32x4 lv = {l[0], l[1], l[2], l[3]};
    hi = __builtin_bit_cast(bf16x8, hv);
    lo = __builtin_bit_cast(bf16x8, lv);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float (&x)[8]) {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = bf16_pack(x[2 * i], x[2 * i + 1]);
    u32x4 v = {h[0], h[1], h[2], h[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// 8 fp8 e4m3fn codes (two 32-bit words) -> 8 bf16.  The hardware converts
// to f32 (OCP e4m3fn on gfx950); e4m3 has 4 significant bits, so truncating
// the f32 to bf16 is exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
    auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
    auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
    auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
    u32x4 v;
    v.x = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xFFFF0000u);
    v.y = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xFFFF0000u);
    v.z = (__float_as_uint(c[0]) >> 16) | (__float_as_uint(c[1]) & 0xFFFF0000u);
    v.w = (__float_as_uint(d[0]) >> 16) | (__float_as_uint(d[1]) & 0xFFFF0000u);
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// wave reductions
// ---------------------------------------------------------------------------
// All of these stay in the VALU (no LDS round trip).  Within a 16-lane row
// the DPP row rotations combine lane i with lanes i - n (mod 16); across
// rows the gfx950 lane swaps: swapping a register with itself between
// 16-lane rows (32-lane halves) leaves every lane holding its own value in
// one result and its partner's, lane ^ 16 (lane ^ 32), in the other.
template <int N>
__device__ __forceinline__ float row_ror(float v) {   // lane i gets lane (i - N) mod 16 of its row
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
// lane i gets lane i - 1 of its 16-lane row (the first lane of a row gets 0)
__device__ __forceinline__ float row_shr1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor16_sum(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// over all 64 lanes
__device__ __forceinline__ float wave_sum(float v) {
    v += row_ror<1>(v);
    v += row_ror<2>(v);
    v += row_ror<4>(v);
    v += row_ror<8>(v);
    return xor32_sum(xor16_sum(v));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, row_ror<1>(v));
    v = fmaxf(v, row_ror<2>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<8>(v));
    return xor32_max(xor16_max(v));
}
// over the 16 lanes that share l % 4
__device__ __forceinline__ float stride4_sum(float v) {
    v += row_ror<4>(v);
    v += row_ror<8>(v);
    return xor32_sum(xor16_sum(v));
}
// over the 4 lanes that share l % 16 (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float group4_sum(float v) { return xor32_sum(xor16_sum(v)); }
__device__ __forceinline__ float group4_max(float v) { return xor32_max(xor16_max(v)); }

// streaming (non-temporal) 16-byte load for weights that are read once
__device__ __forceinline__ u32x4 ld_stream16(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ float4 ld_f4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
