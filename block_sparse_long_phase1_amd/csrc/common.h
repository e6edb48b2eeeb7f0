// Device-side helpers shared by the gfx950 kernels of libstarattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace star {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no score seen yet": exp2(x - kNoMax) underflows to 0 for every
// finite x, and unlike -inf it never produces inf - inf.
constexpr float kNoMax = -1.0e30f;

// bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 p = {(__bf16)lo, (__bf16)hi};  // round-to-nearest-even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight E4M3 codes (bytes in memory order) -> eight bf16 (exact: every E4M3 value is a bf16).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return r;
}

// Combine a value with the one held 32 lanes away (lanes l and l^32).  With the same
// register as both operands, v_permlane32_swap returns {own, partner} in an order that
// depends on the lane's half, so only symmetric combinations of the pair are formed.
__device__ __forceinline__ float half_pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value of lane (l ^ 1), (l ^ 2), mirrored inside each half row (l ^ 7 within 8 lanes) and
// mirrored inside each row (l ^ 15 within 16 lanes): DPP moves, no LDS round trip.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xb1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4e;      // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Max / sum over all 64 lanes, the same bits in every lane: a butterfly inside each 16-lane
// row by DPP, then lanes l, l^16, l^32, l^48 through the permlane swaps.  Each step pairs a
// lane with one whose partial covers a disjoint set of lanes; the operations are commutative,
// so both lanes of a pair form the same value.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return half_pair_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppRowMirror>(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return half_pair_sum(x);
}

// Select bytes of the pair (hi:lo) -- v_perm_b32.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low halves of two words -> (lo16(a) | lo16(b) << 16); high halves likewise.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

}  // namespace star
