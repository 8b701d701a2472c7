// la_device.h -- device-side helpers shared by the liblinattn kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// ---------------------------------------------------------------- numbers --

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN inputs do not occur on the path).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// phi = SiLU(x) = x * sigmoid(x)  (feature map on q, k and v)
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
__device__ __forceinline__ float sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (RNE), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) { return cvt_pk_bf16(a, b); }

// Split two fp32 values into bf16 hi + bf16 lo with hi = RNE(x), lo = RNE(x - hi);
// hi*hi' + hi*lo' + lo*hi' then carries ~16 significant bits of each product.
// x - hi comes from one bf16 dot product per value, (hi0, hi1) . (-1, -0) + x0
// and (hi0, hi1) . (0, -1) + x1: both products are exact in fp32 and x - hi
// is representable, so the result is exact whatever the rounding.  The
// multiplier of x0 is (-1, -0), bits 0x8000bf80, on purpose: the compiler
// encodes (-1, +0) as the inline constant -1.0, which the hardware reads as
// the fp32 bit pattern 0xbf800000, i.e. (+0, -1) -- a wrong split.  No inline
// constant has the pattern 0x8000bf80, so it is emitted as a literal.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const f32x2_t v = {x0, x1};
    const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    const bf16x2_t m0 = {(__bf16)-1.0f, (__bf16)-0.0f};
    const bf16x2_t m1 = {(__bf16)0.0f, (__bf16)-1.0f};
    const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, m0, x0, false);
    const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, m1, x1, false);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = cvt_pk_bf16(l0, l1);
}

// The same split for values that stay live afterwards (the dot product
// accumulates in place, which would cost a copy): x - hi by unpacking hi.
__device__ __forceinline__ void split2_keep(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = cvt_pk_bf16(x0, x1);
    lo = cvt_pk_bf16(x0 - bf16_lo_to_f32(hi), x1 - bf16_hi_to_f32(hi));
}

template <typename T> __device__ __forceinline__ float load_as_f32(const T* p);
template <> __device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) {
    return bf16_to_f32(*p);
}

template <typename T> __device__ __forceinline__ void store_from_f32(T* p, float v);
template <> __device__ __forceinline__ void store_from_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t* p, float v) {
    *p = f32_to_bf16(v);
}

// ------------------------------------------------------------ matrix core --
// v_mfma_f32_16x16x32_bf16, lane l = 16*g + c (g = l/16, c = l%16):
//   A (16 x 32): lane holds row c, k = 8g .. 8g+7
//   B (32 x 16): lane holds column c, k = 8g .. 8g+7
//   C (16 x 16): lane holds column c, rows 4g .. 4g+3
// Any permutation of k applied identically to A and B gives the same product.
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(i16x4_t lo, i16x4_t hi) {
    i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// 8-byte LDS read.
__device__ __forceinline__ i16x4_t lds_read8(const uint16_t* p) { return *(const i16x4_t*)p; }

// Transposing LDS read (ds_read_b64_tr_b16).  For a row-major bf16 tile with
// row stride `stride` elements, returns for this lane's 16-lane group the
// 4 x 16 block at rows [r0, r0+4), columns [c0, c0+16): this lane receives
// column c0 + (lane % 16), rows r0 .. r0+3.  r0 may differ between groups.
__device__ __forceinline__ i16x4_t lds_read_tr4(const uint16_t* tile, int stride, int r0, int c0,
                                                int lane16) {
    const uint16_t* p = tile + (r0 + (lane16 >> 2)) * stride + c0 + 4 * (lane16 & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

}  // namespace la
