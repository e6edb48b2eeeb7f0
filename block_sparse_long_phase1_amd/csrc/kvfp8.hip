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
// Both kernels stream one kv head per grid row (blockIdx.y) in 16-byte vectors;
// they are HBM-bound (2 or 4 bytes read per element, 1 written by the quantiser).
#include "common.h"
#include "internal.h"

namespace star {

namespace {
constexpr int kThreads = 256;

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
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
        const u32x4 w = src[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (BF16) {
                m = max(m, (w[j] << 16) & 0x7fffffffu);
                m = max(m, w[j] & 0x7fff0000u);
            } else {
                m = max(m, w[j] & 0x7fffffffu);
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

// 8 elements per thread step: one (bf16) or two (fp32) 16-byte loads, one 8-byte store.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) kv_quantize_kernel(const void* x, int64_t per_head, const float* scale,
                                                               uint8_t* out) {
    const int g = blockIdx.y;
    const float s = scale[g];
    const int64_t n8 = per_head / 8;
    const char* src = static_cast<const char*>(x) + (size_t)g * per_head * (BF16 ? 2 : 4);
    u32x2* dst = reinterpret_cast<u32x2*>(out + (size_t)g * per_head);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
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

dim3 stream_grid(int64_t vecs, int hkv) {
    int64_t nb = (vecs + kThreads - 1) / kThreads;
    const int64_t cap = (2048 + hkv - 1) / hkv;   // about 8 workgroups per CU in all
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
        const dim3 grid = stream_grid(per_head / (bf16 ? 8 : 4), hkv);
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
    const dim3 grid = stream_grid(per_head / 8, hkv);
    if (bf16)
        hipLaunchKernelGGL(kv_quantize_kernel<true>, grid, dim3(kThreads), 0, stream, x, per_head, scale, out);
    else
        hipLaunchKernelGGL(kv_quantize_kernel<false>, grid, dim3(kThreads), 0, stream, x, per_head, scale, out);
    return hipGetLastError();
}

}  // namespace star
