// device_common.hpp -- small gfx950 device helpers shared by the fp8q kernels.
//
// Numeric rule implemented here (one tile, one fp32 scale):
//   s = fl32(amax / 448),  code = E4M3FN(fl32(x / s))  (nearest even, +-448
//   saturation, sign kept); or, for power-of-two scales, s = the smallest
//   power of two >= amax / 448 (at least 2^-127) with the same code rule.
//   The mapping of the tile maximum onto the largest
//   FP8 value is the per-tensor practice that page 1 (why-be.why-be.co.kr,
//   wr_id=65900) describes, applied per small group as in its passage on
//   groups sharing exponent bits; tile shapes follow page 4
//   (sunipension.com, wr_id=314414), passage on Figure 7(a).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Largest finite OCP E4M3FN magnitude.
constexpr float kE4M3Max = 448.0f;

// Scales at or above this bound take the reciprocal path in quotient(); below
// it the reciprocal 1/s could overflow and the exact IEEE division is used.
constexpr float kFastScaleMin = 0x1p-64f;

// ------------------------------------------------------------------ DPP
// DPP16 row rotate: every lane of a 16-lane row reads the lane `n` places to
// the right (with wrap-around) in the same row.
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
    static_assert(N >= 1 && N <= 15, "row_ror amount");
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xf, 0xf, false);
}

// Maximum over the 16 lanes of each DPP row; every lane receives the result.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    v = max(v, row_ror<8>(v));
    v = max(v, row_ror<4>(v));
    v = max(v, row_ror<2>(v));
    v = max(v, row_ror<1>(v));
    return v;
}

// ------------------------------------------------------------------ scalars
__device__ __forceinline__ float bits_f32(uint32_t b) { return __uint_as_float(b); }

// bf16 pair packed in one dword -> two fp32 values (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Magnitude bits of a finite fp32 value; unsigned order of these bits is the
// order of |x|, so amax can be an integer max.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

// Per-tile constants: scale s, its correctly rounded reciprocal r, and the
// choice of quotient path.
struct TileScale {
    float s;
    float r;
    bool fast;
};

__device__ __forceinline__ TileScale make_scale(uint32_t amax_bits) {
    TileScale t;
    t.s = __uint_as_float(amax_bits) / kE4M3Max;  // IEEE division, round to nearest even
    t.fast = t.s >= kFastScaleMin;
    t.r = t.fast ? 1.0f / t.s : 0.0f;
    return t;
}

// Power-of-two scale of a tile: the smallest s = 2^e with 448 * s >= amax,
// e >= -127 (an E8M0 value), s = 0 for amax == 0.  With amax = (1 + f) * 2^E,
// 448 = 1.75 * 2^8 gives e = E - 8 when 1 + f <= 1.75 (mantissa bits <=
// 0x600000) and E - 7 otherwise; subnormal amax needs e < -127 and takes the
// clamp.  r = 2^-e is exact (e <= 120 since amax < 2^128), so the quotient is
// the single rounding of x * r, and x = +-0 keeps its sign.
__device__ __forceinline__ TileScale make_scale_pow2(uint32_t amax_bits) {
    TileScale t;
    const int field = (int)(amax_bits >> 23);
    int e = field - 135 + ((amax_bits & 0x7fffffu) > 0x600000u ? 1 : 0);
    e = field == 0 || e < -127 ? -127 : e;
    const float s_pos = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
    t.s = amax_bits == 0 ? 0.0f : s_pos;
    t.r = __uint_as_float((uint32_t)(127 - e) << 23);
    t.fast = true;
    return t;
}

template <bool POW2>
__device__ __forceinline__ TileScale make_scale_mode(uint32_t amax_bits) {
    if constexpr (POW2)
        return make_scale_pow2(amax_bits);
    else
        return make_scale(amax_bits);
}

// fl32(x / s), bit-exact with IEEE division wherever the result can change
// an E4M3 code (|x/s| >= 2^-12), with the sign of x always kept.
// Fast path: y = x*r, then one correction step with the exact residual
// y*s - x (Markstein's theorem: with r = RN(1/s) and a faithful y, the
// corrected quotient is RN(x/s) when no intermediate underflows; the
// residual is formed as y*s - x so that x = -0 gives -0).
__device__ __forceinline__ float quotient(float x, const TileScale& t) {
    if (t.fast) {
        float y = x * t.r;
        float e = __builtin_fmaf(y, t.s, -x);
        return __builtin_fmaf(-e, t.r, y);
    }
    if (t.s == 0.0f) return __builtin_copysignf(0.0f, x);
    return x / t.s;
}

// Two quotients -> two E4M3 codes written into byte pair WORD (false: bits
// 0..15, true: bits 16..31) of `old`.  The hardware conversion rounds to nearest
// even; the clamp to +-448 gives saturation.
template <bool WORD>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old) {
    a = __builtin_amdgcn_fmed3f(a, kE4M3Max, -kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, kE4M3Max, -kE4M3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, WORD);
}

// As cvt2, without the clamp, for quotients known to lie below 464 in
// magnitude: there the hardware's nearest-even conversion already gives +-448
// for everything from 448 up (the midpoint to the next binade's first value,
// 480, which E4M3FN spends on NaN, is 464).  A tile scale s = fl32(amax/448)
// that is a normal number is within a relative 2^-24 of amax/448, so every
// quotient of its tile is at most 448*(1 + 2^-23); a power-of-two scale has
// 448*s >= amax exactly.
template <bool WORD>
__device__ __forceinline__ uint32_t cvt2_in_range(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, WORD);
}

// Four values -> one dword of four codes (byte i = code of v[i]).
__device__ __forceinline__ uint32_t encode4(float v0, float v1, float v2, float v3,
                                            const TileScale& t) {
    uint32_t w = cvt2<false>(quotient(v0, t), quotient(v1, t), 0u);
    return cvt2<true>(quotient(v2, t), quotient(v3, t), w);
}

// Power-of-two scales: the quotient is x * r with r = 1/s exact.
__device__ __forceinline__ uint32_t encode4_mul(float v0, float v1, float v2, float v3, float r) {
    const uint32_t w = cvt2_in_range<false>(v0 * r, v1 * r, 0u);
    return cvt2_in_range<true>(v2 * r, v3 * r, w);
}

// Exact E4M3FN decode of the four codes of a dword (byte i -> v[i]).
__device__ __forceinline__ void decode4(uint32_t w, float v[4]) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    v[0] = lo[0];
    v[1] = lo[1];
    v[2] = hi[0];
    v[3] = hi[1];
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 with round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

}  // namespace fp8q
