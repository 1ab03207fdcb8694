// Device helpers: number formats and MFMA vector types for gfx950.
//
// Everything here works on bit patterns so that every rounding is explicit:
// E4M3 (OCP "e4m3fn": bias 7, largest finite 448, S.1111.111 NaN), BF16,
// FP16, UE8M0 (2^(b-127), b = 255 NaN) and int8.  Exact conversions use the
// gfx950 conversion instructions where those are exact by construction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nq {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) loads of 16 / 8 bytes, for weights read once: a
// plain streaming read of 89 MB / 1 GiB takes 14.6 / 156 us this way against
// 15.4 / 170 us with plain global loads and 16.0 / 176 us with default buffer
// loads.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void ld_nt(uint4& d, const void* p) { d = ld_nt16(p); }
__device__ __forceinline__ void ld_nt(uint2& d, const void* p) { d = ld_nt8(p); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// FP32 -> BF16 bits, round to nearest even (subnormals and overflow follow
// from the carry into the exponent field); NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// E4M3 code -> FP32, exact, from the fields (NaN codes -> quiet NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t sign = (c & 0x80u) << 24;
    const uint32_t em = c & 0x7Fu;
    if (em == 0x7Fu) return __uint_as_float(0x7FC00000u);
    float mag;
    if (em >= 8u) mag = __uint_as_float((em << 20) + (120u << 23));   // (1+m/8) 2^(e-7)
    else mag = (float)em * 0.001953125f;                               // m 2^-9, exact
    return __uint_as_float(__float_as_uint(mag) | sign);
}

// UE8M0 byte -> its FP32 value 2^(b-127), exact (b = 0 is the subnormal 2^-127).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) {
    if (b == 255u) return __uint_as_float(0x7FC00000u);
    if (b == 0u) return __uint_as_float(0x00400000u);
    return __uint_as_float(b << 23);
}

// FP32 -> E4M3 code, round to nearest even, saturating at +-448, sign of zero
// kept, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;                  // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;           // |f| >= 448 (and inf)
    if (a >= 0x3C800000u) {                              // |f| >= 2^-6: normal result
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // keep 3 mantissa bits, RNE
        return sign | (r - (120u << 3));
    }
    const float t = __uint_as_float(a) * 512.0f;          // |f| 2^9 < 8, exact
    return sign | (uint32_t)__builtin_rintf(t);           // 0..8 quanta of 2^-9, RNE
}

// x / s as the IEEE FP32 quotient, computed as RN32((double)x * r) with
// r = RN64(1 / s) (one FP64 division per row or group).  Exact whenever x and
// s together carry at most 32 significant bits (an FP32 numerator over a BF16
// scale, or a BF16 numerator over an FP32 scale): such a quotient is either an
// FP32 value itself or at least 2^-33 (relative) away from every FP32 rounding
// boundary, while the FP64 product lies within 2^-52 of it, so both round to
// the same FP32 value.  The IEEE special cases carry over: x * inf = x / 0,
// 0 * inf = NaN = 0 / 0, x * 0 = x / inf, NaN stays NaN.
__device__ __forceinline__ float div_via_recip64(float x, double r) { return (float)((double)x * r); }

// Four FP32 values -> four E4M3 codes (bytes 0..3), round to nearest even, by
// the hardware convert.  It agrees with f32_to_e4m3_sat for every |v| < 464
// (checked exhaustively on all such FP32 inputs, both signs); callers pass
// only such values.
__device__ __forceinline__ uint32_t f32x4_to_e4m3_hw(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// FP32 -> int8 code: round to nearest even, clamp to [-127, 127], NaN -> 0.
__device__ __forceinline__ int32_t f32_to_i8_sat(float f) {
    float r = __builtin_rintf(f);
    r = (f == f) ? r : 0.0f;
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int32_t)r;
}

// Four E4M3 codes in a dword -> four FP32 values (exact; hardware convert).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> packed BF16 pair times an FP32
// power-of-two scale (exact for results in the BF16 normal range).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, float scale) {
    v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// Two FP32 -> packed BF16 pair, RNE (exact for small integers).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    v2bf r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace nq
