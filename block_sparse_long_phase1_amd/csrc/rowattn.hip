// Plain vector attention, one wave per (q head, row): the path for fp32
// inputs and for shapes the MFMA kernels do not cover.  It computes the same
// quantities as the fast kernels:
//   * Phase 1 rows ("Star Attention: Efficient LLM Inference over Long
//     Sequences", paper-graph-ui summary, section 3.4, Phase 1 Steps 2-4):
//     anchor [0, anchor) for blocks >= 1, then the own block up to the row;
//   * explicit key segments with an optional causal limit (Phase 2 Step 3
//     partials, and a whole decode step over context + query-host cache).
// Keys are taken 64 at a time, one per lane (full-d dot product against q
// held in LDS); the running softmax state is wave-uniform and each lane owns
// up to 4 of the d output columns.
#include "common.h"
#include "internal.h"

namespace star {

namespace {
constexpr int kThreads = 256;
constexpr int kMaxD = 256;

__device__ __forceinline__ float ld_elem(const void* base, int is_bf16, int64_t idx) {
    if (is_bf16) {
        uint32_t w = reinterpret_cast<const uint16_t*>(base)[idx];
        return __uint_as_float(w << 16);
    }
    return reinterpret_cast<const float*>(base)[idx];
}
}  // namespace

__global__ void __launch_bounds__(kThreads)
row_attn_kernel(const RowAttnArgs a, int64_t rows) {
    __shared__ float qs[kThreads / 64][kMaxD];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    if (item >= (int64_t)a.hq * rows) return;   // whole wave leaves; no block barriers below
    const int h = (int)(item / rows);
    const int64_t i = item % rows;
    const int d = a.d;
    const int G = a.hq / a.hkv;
    const int g = h / G;
    const float sl2 = a.scale * kLog2e;

    for (int e = lane; e < d; e += 64) qs[wave][e] = ld_elem(a.q, a.is_bf16, ((int64_t)h * a.q_rows + i) * d + e);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    RowKeySeg seg[3];
    int n_seg;
    int64_t crow = i + a.row_offset;
    if (a.mode == 0) {
        const int64_t p = i;
        const int64_t blk = p / a.block, start = blk * a.block;
        seg[0].k = a.k; seg[0].v = a.v; seg[0].head_stride = a.L * d;
        seg[0].n = blk >= 1 ? a.anchor : 0; seg[0].causal_lim = -1;
        const int64_t off = start * d * (a.is_bf16 ? 2 : 4);
        seg[1].k = reinterpret_cast<const char*>(a.k) + off;
        seg[1].v = reinterpret_cast<const char*>(a.v) + off;
        seg[1].head_stride = a.L * d;
        seg[1].n = p - start + 1; seg[1].causal_lim = -1;
        n_seg = 2;
    } else {
        n_seg = a.n_seg;
        for (int s = 0; s < 3; ++s) seg[s] = a.seg[s];
    }

    float m = kNoMax, l = 0.f;
    float o[kMaxD / 64];
#pragma unroll
    for (int j = 0; j < kMaxD / 64; ++j) o[j] = 0.f;

    for (int s = 0; s < n_seg; ++s) {
        const int64_t hoff = (int64_t)g * seg[s].head_stride;
        for (int64_t t0 = 0; t0 < seg[s].n; t0 += 64) {
            const int64_t t = t0 + lane;
            const bool valid = t < seg[s].n && (seg[s].causal_lim < 0 || t <= seg[s].causal_lim + crow);
            float x = -INFINITY;
            if (valid) {
                float dot = 0.f;
                for (int e = 0; e < d; ++e) dot = fmaf(qs[wave][e], ld_elem(seg[s].k, a.is_bf16, hoff + t * d + e), dot);
                x = dot * sl2;
            }
            const float gmax = wave_max(x);
            if (gmax == -INFINITY) continue;
            const float mnew = fmaxf(m, gmax);
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int j = 0; j < kMaxD / 64; ++j) o[j] *= alpha;
            const float pr = valid ? fast_exp2(x - m) : 0.f;
            l += wave_sum(pr);
            const int64_t cnt = seg[s].n - t0 < 64 ? seg[s].n - t0 : 64;
            for (int jj = 0; jj < cnt; ++jj) {
                const float pj = __shfl(pr, jj);
                if (pj == 0.f) continue;
                const int64_t row = hoff + (t0 + jj) * d;
#pragma unroll
                for (int j = 0; j < kMaxD / 64; ++j) {
                    const int e = lane + 64 * j;
                    if (e < d) o[j] = fmaf(pj, ld_elem(seg[s].v, a.is_bf16, row + e), o[j]);
                }
            }
        }
    }

    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.0f / l;
    const int64_t out_row = (int64_t)h * rows + i;
    if (a.a_out) {
#pragma unroll
        for (int j = 0; j < kMaxD / 64; ++j) {
            const int e = lane + 64 * j;
            if (e < d) a.a_out[out_row * d + e] = o[j] * inv;
        }
        if (lane == 0) {
            a.m_out[out_row] = empty ? -INFINITY : m * kLn2;
            a.l_out[out_row] = empty ? 0.f : l;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kMaxD / 64; ++j) {
            const int e = lane + 64 * j;
            if (e >= d) continue;
            if (a.is_bf16) reinterpret_cast<uint16_t*>(a.o)[out_row * d + e] = to_bf16(o[j] * inv);
            else reinterpret_cast<float*>(a.o)[out_row * d + e] = o[j] * inv;
        }
        if (lane == 0 && a.lse) a.lse[out_row] = empty ? -INFINITY : (m + __builtin_amdgcn_logf(l)) * kLn2;
    }
}

hipError_t launch_row_attn(const RowAttnArgs& a, int64_t rows, hipStream_t stream) {
    if (a.d > kMaxD || a.d < 1) return hipErrorInvalidValue;
    const int64_t items = (int64_t)a.hq * rows;
    if (items <= 0) return hipSuccess;
    const int64_t grid = (items + 3) / 4;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(row_attn_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a, rows);
    return hipGetLastError();
}

__global__ void tail_append_kernel(const char* k_new, const char* v_new, char* k_tail, char* v_tail,
                                   int64_t tail_len, int64_t tail_cap, int64_t row_bytes) {
    const int g = blockIdx.x;
    for (int64_t b = threadIdx.x; b < row_bytes; b += blockDim.x) {
        k_tail[((int64_t)g * tail_cap + tail_len) * row_bytes + b] = k_new[(int64_t)g * row_bytes + b];
        v_tail[((int64_t)g * tail_cap + tail_len) * row_bytes + b] = v_new[(int64_t)g * row_bytes + b];
    }
}

hipError_t launch_tail_append(const void* k_new, const void* v_new, void* k_tail, void* v_tail,
                              int64_t tail_len, int64_t tail_cap, int hkv, int d, int elem_bytes,
                              hipStream_t stream) {
    hipLaunchKernelGGL(tail_append_kernel, dim3(hkv), dim3(256), 0, stream,
                       reinterpret_cast<const char*>(k_new), reinterpret_cast<const char*>(v_new),
                       reinterpret_cast<char*>(k_tail), reinterpret_cast<char*>(v_tail),
                       tail_len, tail_cap, (int64_t)d * elem_bytes);
    return hipGetLastError();
}

}  // namespace star
