// E4M3 context KV cache: per-kv-head scales and quantisation.
//
// "Star Attention: Efficient LLM Inference over Long Sequences" (paper-graph-ui
// summary), section "Related Work", part "Memory Optimization and KV Cache
// Compression": KV-cache quantisation is orthogonal to the method and combines
// with it.  The context hosts' cached K and V are stored here as OCP E4M3 codes
// with one fp32 scale per kv head: code = the E4M3 value nearest to the
// correctly rounded fp32 quotient x / scale (ties to the even mantissa,
// magnitudes from 448 up saturate to 448, NaN stays NaN), and the cached value
// is scale * decode(code).  The decode step reads the codes through the
// hardware's exact E4M3 -> bf16 conversion (decode.hip).
//
// Both kernels stream one kv head per grid row (blockIdx.y) in 16-byte vectors, several
// per thread in flight; they are HBM-bound (2 or 4 bytes read per element, 1 written by
// the quantiser).
#include "common.h"
#include "internal.h"

namespace star {

namespace {
constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte loads in flight per thread and loop step

// E4M3 code of an fp32 value (OCP E4M3: sign, 4 exponent bits with bias 7, 3 mantissa
// bits, subnormals m/8 * 2^-6, S.1111.111 = NaN, largest finite 448).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t s = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return s | 0x7fu;    // NaN
    if (a >= 0x43e00000u) return s | 0x7eu;   // |v| >= 448, infinities included: saturate
    if (a < 0x3c800000u) {                    // |v| < 2^-6: subnormal steps of 2^-9
        // |v| * 512 is exact; rounding it to an integer (half to even) gives the step count,
        // and 8 steps is code 0x08, the smallest normal.
        return s | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    // Normal range: keep 3 of the 23 mantissa bits, rounding half to even (a carry moves
    // into the exponent), then move the exponent bias from 127 to 7.
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    return s | ((r >> 20) - (120u << 3));
}

// Scales whose reciprocal and products stay far from fp32 underflow and overflow:
// [2^-90, 2^90] as bit patterns.  Inside, clamped_quotient() is exact wherever it decides
// the code; outside, the quantiser divides with __fdiv_rn.
constexpr uint32_t kFastScaleLo = 0x12800000u;
constexpr uint32_t kFastScaleHi = 0x6c800000u;

// The quotient ax / s (ax = |x|, s in the range above, r = RN(1/s)) clamped to 448, in the
// form the hardware conversion takes.  ax * r is within two ulps of ax / s; two
// Newton-Raphson corrections with exact remainders (fma) make it faithful and then correctly
// rounded (Markstein's theorem: a faithful quotient plus the remainder times the correctly
// rounded reciprocal, rounded once, is the correctly rounded quotient).  Far outside the
// E4M3 range the corrections may lose accuracy or give NaN (an infinite x, or ax / s past
// the fp32 range), where the code no longer depends on it: below 2^-12 every value rounds
// to zero, and fminf maps anything at or above 448 (and NaN) to 448, the saturated code.
// A NaN x is passed through as NaN.  The GPU tests compare the codes with the oracle's for
// every bf16 value and for fp32 values at and around every E4M3 rounding midpoint, under
// scales on both sides of the range above.
__device__ __forceinline__ float clamped_quotient(uint32_t axb, float s, float r) {
    const float ax = __uint_as_float(axb);
    const float q0 = ax * r;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, ax), r, q0);
    const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, s, ax), r, q1);
    return axb > 0x7f800000u ? ax : __builtin_fminf(q2, 448.0f);
}

// Four E4M3 codes (bytes in element order) of clamped quotients: the hardware conversion
// rounds to nearest even, subnormals included, exactly as the rule above for every value
// in [0, 448] (compared over every fp32 value there), and turns NaN into 0xFF.  The sign bits are then those of x (x / s with s > 0
// has the sign of x, NaN included), so a NaN becomes 0x7F or 0xFF by its own sign.
__device__ __forceinline__ uint32_t e4m3x4(const float (&q)[4], const uint32_t (&xb)[4]) {
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c, true);
    const uint32_t sign = ((xb[0] >> 24) & 0x80u) | ((xb[1] >> 16) & 0x8000u) | ((xb[2] >> 8) & 0x800000u) |
                          (xb[3] & 0x80000000u);
    return ((uint32_t)c & 0x7f7f7f7fu) | sign;
}

__global__ void __launch_bounds__(kThreads) kv_bits_zero_kernel(uint32_t* bits, int n) {
    for (int i = threadIdx.x; i < n; i += kThreads) bits[i] = 0u;
}

// Largest |x| of each kv head, as fp32 bit patterns (for non-negative floats the unsigned
// order of the patterns is the numeric order), folded into bits[g] with an atomic max.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) kv_absmax_kernel(const void* x, int64_t per_head, uint32_t* bits) {
    __shared__ uint32_t red[kThreads / 64];
    const int g = blockIdx.y;
    constexpr int kPer = BF16 ? 8 : 4;   // elements per 16-byte vector
    const int64_t nvec = per_head / kPer;
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(x) +
                                                      (size_t)g * per_head * (BF16 ? 2 : 4));
    uint32_t m = 0u;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += kUnroll * stride) {
        u32x4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            w[u] = i + u * stride < nvec ? __builtin_nontemporal_load(src + i + u * stride) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (BF16) {
                    m = max(m, (w[u][j] << 16) & 0x7fffffffu);
                    m = max(m, w[u][j] & 0x7fff0000u);
                } else {
                    m = max(m, w[u][j] & 0x7fffffffu);
                }
            }
    }
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, sh));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) b = max(b, red[w]);
        __hip_atomic_fetch_max(bits + g, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// bits[g] (the head's max |x|) -> scale[g] = max / 448, in place; 1 for an all-zero head.
__global__ void __launch_bounds__(kThreads) kv_scale_from_bits_kernel(uint32_t* bits, int n) {
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const uint32_t b = bits[i];
        const float s = b == 0u ? 1.0f : __fdiv_rn(__uint_as_float(b), 448.0f);
        reinterpret_cast<float*>(bits)[i] = s;
    }
}

// Eight elements as fp32 bit patterns from one (bf16) or two (fp32) 16-byte vectors.
template <bool BF16>
__device__ __forceinline__ void widen8(const u32x4 (&w)[2], uint32_t (&xb)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (BF16) {
            xb[2 * j] = w[0][j] << 16;
            xb[2 * j + 1] = w[0][j] & 0xffff0000u;
        } else {
            xb[j] = w[0][j];
            xb[4 + j] = w[1][j];
        }
    }
}

// 8 elements per thread step: one (bf16) or two (fp32) 16-byte loads, one 8-byte store;
// kUnroll steps' loads are issued before any is used.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) kv_quantize_kernel(const void* x, int64_t per_head, const float* scale,
                                                               uint8_t* out) {
    constexpr int kVec = BF16 ? 1 : 2;   // 16-byte vectors per 8 elements
    const int g = blockIdx.y;
    const float s = scale[g];
    const int64_t n8 = per_head / 8;
    const char* src = static_cast<const char*>(x) + (size_t)g * per_head * (BF16 ? 2 : 4);
    const u32x4* sv = reinterpret_cast<const u32x4*>(src);
    u32x2* dst = reinterpret_cast<u32x2*>(out + (size_t)g * per_head);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const uint32_t sbits = __float_as_uint(s);
    if (sbits >= kFastScaleLo && sbits <= kFastScaleHi) {   // the same for the whole grid row
        const float r = __fdiv_rn(1.0f, s);
        for (int64_t i = i0; i < n8; i += kUnroll * stride) {
            u32x4 w[kUnroll][2];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int h = 0; h < kVec; ++h)
                    w[u][h] = i + u * stride < n8 ? __builtin_nontemporal_load(sv + kVec * (i + u * stride) + h)
                                                  : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (i + u * stride >= n8) continue;
                uint32_t xb[8];
                widen8<BF16>(w[u], xb);
                u32x2 o;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float q[4];
                    uint32_t xh[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xh[j] = xb[4 * h + j];
                        q[j] = clamped_quotient(xh[j] & 0x7fffffffu, s, r);
                    }
                    o[h] = e4m3x4(q, xh);
                }
                __builtin_nontemporal_store(o, dst + i + u * stride);
            }
        }
        return;
    }
    for (int64_t i = i0; i < n8; i += stride) {
        float v[8];
        if (BF16) {
            const u32x4 w = reinterpret_cast<const u32x4*>(src)[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = bf16_lo(w[j]);
                v[2 * j + 1] = bf16_hi(w[j]);
            }
        } else {
            const u32x4 w0 = reinterpret_cast<const u32x4*>(src)[2 * i];
            const u32x4 w1 = reinterpret_cast<const u32x4*>(src)[2 * i + 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = __uint_as_float(w0[j]);
                v[4 + j] = __uint_as_float(w1[j]);
            }
        }
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = e4m3_code(__fdiv_rn(v[j], s));
        u32x2 o;
        o[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        o[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        dst[i] = o;
    }
}

// Workgroups per kv head: enough for the vectors, at most `total` over all heads (about 4
// (abs-max) or 8 (quantiser) per CU, the best measured).
dim3 stream_grid(int64_t vecs, int hkv, int total) {
    int64_t nb = (vecs + kThreads - 1) / kThreads;
    const int64_t cap = (total + hkv - 1) / hkv;
    if (nb > cap) nb = cap;
    if (nb < 1) nb = 1;
    return dim3((unsigned)nb, (unsigned)hkv);
}
}  // namespace

hipError_t launch_kv_fp8_scales(const void* x, int64_t tokens, int hkv, int d, bool bf16, float* scale,
                                hipStream_t stream) {
    if (hkv < 1 || hkv > 65535 || tokens < 0 || d % 8) return hipErrorInvalidValue;
    const int64_t per_head = tokens * d;
    uint32_t* bits = reinterpret_cast<uint32_t*>(scale);
    hipLaunchKernelGGL(kv_bits_zero_kernel, dim3(1), dim3(kThreads), 0, stream, bits, hkv);
    if (per_head > 0) {
        const dim3 grid = stream_grid(per_head / (bf16 ? 8 : 4), hkv, 1024);
        if (bf16)
            hipLaunchKernelGGL(kv_absmax_kernel<true>, grid, dim3(kThreads), 0, stream, x, per_head, bits);
        else
            hipLaunchKernelGGL(kv_absmax_kernel<false>, grid, dim3(kThreads), 0, stream, x, per_head, bits);
    }
    hipLaunchKernelGGL(kv_scale_from_bits_kernel, dim3(1), dim3(kThreads), 0, stream, bits, hkv);
    return hipGetLastError();
}

hipError_t launch_kv_quantize_fp8(const void* x, int64_t tokens, int hkv, int d, bool bf16, const float* scale,
                                  uint8_t* out, hipStream_t stream) {
    if (hkv < 1 || hkv > 65535 || tokens < 0 || d % 8) return hipErrorInvalidValue;
    const int64_t per_head = tokens * d;
    if (per_head == 0) return hipSuccess;
    const dim3 grid = stream_grid(per_head / 8, hkv, 2048);
    if (bf16)
        hipLaunchKernelGGL(kv_quantize_kernel<true>, grid, dim3(kThreads), 0, stream, x, per_head, scale, out);
    else
        hipLaunchKernelGGL(kv_quantize_kernel<false>, grid, dim3(kThreads), 0, stream, x, per_head, scale, out);
    return hipGetLastError();
}

}  // namespace star
