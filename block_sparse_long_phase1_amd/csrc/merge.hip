// Log-space aggregation of partial attention results.
//
// "NVIDIA/Star-Attention" README (shadowgraph.io mirror), "Two Phases of Star
// Attention", Phase 2: the query host sums the partitions' exponent sums into
// the global denominator and weights each partition's local output by its
// share.  "Star Attention: Efficient LLM Inference over Long Sequences"
// (paper-graph-ui summary), section 3.4, Phase 2 Step 5, asks for the same
// sum kept in log space.  With partitions carried as (A_p, m_p, l_p),
// s_p = e^{m_p} l_p, M = max m_p and w_p = l_p e^{m_p - M}:
//   O = sum_p w_p A_p / sum_p w_p,   LSE = M + ln sum_p w_p.
// Empty partitions (m = -inf, l = 0) weigh nothing.
//
// One workgroup per output row.  The 256 threads first reduce M and sum w_p
// over the partitions, then split into part-groups x float4 lanes of d so
// that every A_p row is read once with 16-byte loads.
#include "common.h"
#include "internal.h"

namespace star {

namespace {
constexpr int kMergeThreads = 256;

__device__ float block_reduce(float x, bool is_max, float* red) {
    x = is_max ? wave_max(x) : wave_sum(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kMergeThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}
}  // namespace

__global__ void __launch_bounds__(kMergeThreads)
merge_kernel(const float* __restrict__ a, const float* __restrict__ m, const float* __restrict__ l,
             int n_parts, int64_t n_rows, int d, void* __restrict__ o, int out_bf16,
             float* __restrict__ lse_out, float* __restrict__ m_out, float* __restrict__ l_out) {
    __shared__ float red[kMergeThreads / 64];
    __shared__ f32x4 part_acc[kMergeThreads];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;

    float mx = -INFINITY;
    for (int pi = tid; pi < n_parts; pi += kMergeThreads) mx = fmaxf(mx, m[(int64_t)pi * n_rows + row]);
    const float M = block_reduce(mx, true, red);

    float ws = 0.f;
    if (M != -INFINITY)
        for (int pi = tid; pi < n_parts; pi += kMergeThreads) {
            float mp = m[(int64_t)pi * n_rows + row];
            if (mp != -INFINITY) ws += l[(int64_t)pi * n_rows + row] * __expf(mp - M);
        }
    const float W = block_reduce(ws, false, red);
    const float inv = (M == -INFINITY || !(W > 0.f)) ? 0.f : 1.0f / W;

    // d/4 float4 columns; the remaining thread dimension walks the partitions.
    const int d4 = d >> 2;
    const int groups = kMergeThreads / d4;
    const int e4 = tid % d4, pg = tid / d4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (pg < groups && inv != 0.f)
        for (int pi = pg; pi < n_parts; pi += groups) {
            int64_t idx = (int64_t)pi * n_rows + row;
            float mp = m[idx];
            if (mp == -INFINITY) continue;
            float w = l[idx] * __expf(mp - M);
            f32x4 v = *reinterpret_cast<const f32x4*>(a + idx * d + e4 * 4);
            acc += w * v;
        }
    part_acc[tid] = acc;
    __syncthreads();
    if (tid < d4) {
        f32x4 s = part_acc[tid];
        for (int gi = 1; gi < groups; ++gi) s += part_acc[gi * d4 + tid];
        s *= inv;
        if (out_bf16) {
            uint16_t* op = reinterpret_cast<uint16_t*>(o) + row * d + tid * 4;
            u32x2 w;
            w[0] = pack_bf16x2(s[0], s[1]);
            w[1] = pack_bf16x2(s[2], s[3]);
            *reinterpret_cast<u32x2*>(op) = w;
        } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + row * d + tid * 4) = s;
        }
    }
    if (tid == 0) {
        const bool empty = (M == -INFINITY) || !(W > 0.f);
        if (lse_out) lse_out[row] = empty ? -INFINITY : M + __logf(W);
        if (m_out) m_out[row] = empty ? -INFINITY : M;
        if (l_out) l_out[row] = empty ? 0.f : W;
    }
}

hipError_t launch_merge(const float* a, const float* m, const float* l, int n_parts, int64_t n_rows,
                        int d, void* o, bool out_bf16, float* lse_out, float* m_out, float* l_out,
                        hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    if (n_rows > 0x7fffffffLL || d % 4 || d / 4 > kMergeThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)n_rows), dim3(kMergeThreads), 0, stream,
                       a, m, l, n_parts, n_rows, d, o, out_bf16 ? 1 : 0, lse_out, m_out, l_out);
    return hipGetLastError();
}

}  // namespace star
