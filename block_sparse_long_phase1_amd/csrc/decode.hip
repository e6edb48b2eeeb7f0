// Split-KV grouped-query decode for one generated token (bf16, d = 128).
//
// "Star Attention: Efficient LLM Inference over Long Sequences"
// (paper-graph-ui summary), section 3.4, Phase 2: each context host computes
// the new token's local attention over its cached keys (Step 3) and the query
// host does the same over its own growing cache (Steps 3 and 7); the partials
// are merged in log space (Step 5, done by merge.hip).  Per generated token
// the work is linear in the cached length, so this kernel is a stream over the
// K/V cache: every K/V byte is read exactly once per step for all G q heads of
// its kv head.
//
// Grid: (kv head, key chunk).  Chunks never straddle a host partition; the
// query host's partition also holds the new token, read from k_new / v_new,
// and the workgroup that owns it appends k_new / v_new to the tail cache (no
// one reads that slot from memory in the same launch).
//
// Each wave walks 64-key groups of its chunk.  Scores use MFMA
// (v_mfma_f32_16x16x32_bf16, q heads of the group as the 16 rows, keys as the
// 16 columns), fed straight from 16-byte global loads of K.  P.V is plain fp32
// VALU work on 16-byte loads of V (lane = key quarter x 8-wide d slice), which
// keeps every V load coalesced and needs no transpose.  Per-wave online softmax
// state is combined across the 4 waves in LDS, and each workgroup writes one
// normalised partial (A, m, l).
#include "common.h"
#include "internal.h"

namespace star {

namespace {
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kD = 128;
constexpr int kGroup = 64;   // keys per wave iteration

struct DecodeArgs {
    const uint16_t* q_new;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const uint16_t* k_ctx;
    const uint16_t* v_ctx;
    uint16_t* k_tail;
    uint16_t* v_tail;
    int64_t L, tail_len, tail_cap;
    int hq, hkv, G;
    float sl2;
    DecodeChunkPlan plan;
    float* pa;
    float* pm;
    float* pl;
};

__device__ __forceinline__ float xor_max16(float x) {
    x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 2));
    x = fmaxf(x, __shfl_xor(x, 4));
    x = fmaxf(x, __shfl_xor(x, 8));
    return x;
}
__device__ __forceinline__ float xor_sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}
}  // namespace

template <int G>
__global__ void __launch_bounds__(kThreads, 2)
decode_kernel(const DecodeArgs p) {
    // Per-wave P exchange: [64 keys][G] probabilities + G rescale factors + G maxima.
    __shared__ float p_lds[kWaves][kGroup * G];
    __shared__ float alpha_lds[kWaves][G];
    __shared__ float wm[kWaves][G], wl[kWaves][G];
    __shared__ f32x4 wo[kWaves][G][kD / 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.x % p.hkv;
    const int c = blockIdx.x / p.hkv;
    const DecodeChunkPlan& pl = p.plan;

    // ---- chunk -> key range
    const uint16_t* kb;
    const uint16_t* vb;
    int64_t lo, hi, new_key = -1;
    if (c < pl.chunk_prefix[pl.n_shards]) {
        int r = 0;
        while (c >= pl.chunk_prefix[r + 1]) ++r;
        lo = pl.shard_lo[r] + (int64_t)(c - pl.chunk_prefix[r]) * pl.chunk;
        hi = lo + pl.chunk < pl.shard_lo[r + 1] ? lo + pl.chunk : pl.shard_lo[r + 1];
        kb = p.k_ctx + (int64_t)g * p.L * kD;
        vb = p.v_ctx + (int64_t)g * p.L * kD;
    } else {
        int64_t tc = c - pl.chunk_prefix[pl.n_shards];
        lo = tc * pl.chunk;
        int64_t n_tail = p.tail_len + 1;
        hi = lo + pl.chunk < n_tail ? lo + pl.chunk : n_tail;
        kb = p.k_tail + (int64_t)g * p.tail_cap * kD;
        vb = p.v_tail + (int64_t)g * p.tail_cap * kD;
        if (hi == n_tail) {
            new_key = p.tail_len;
            // Append the new token's k / v to the query host's cache (32 lanes x 16 B).
            if (tid < 32) {
                const uint16_t* src = (tid < 16 ? p.k_new : p.v_new) + (int64_t)g * kD + (tid & 15) * 8;
                uint16_t* dst = (tid < 16 ? p.k_tail : p.v_tail) + ((int64_t)g * p.tail_cap + p.tail_len) * kD + (tid & 15) * 8;
                *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
            }
        }
    }
    const uint16_t* knew = p.k_new + (int64_t)g * kD;
    const uint16_t* vnew = p.v_new + (int64_t)g * kD;

    // ---- Q as the MFMA A operand: row m = lane % 16 (q head g*G + m), 8 d per slot group
    const int qm = lane & 15, qk = lane >> 4;
    bf16x8 qa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qm < G) w = *reinterpret_cast<const u32x4*>(p.q_new + (int64_t)(g * G + qm) * kD + s * 32 + qk * 8);
        qa[s] = __builtin_bit_cast(bf16x8, w);
    }

    // Running state.  S-layout lanes (lane/16 = query quad) track m for queries 4*(lane/16)+r;
    // every lane accumulates O for all G queries over its d slice (lane % 16) and key quarter.
    float m_run[4] = {kNoMax, kNoMax, kNoMax, kNoMax};
    float l_part[4] = {0.f, 0.f, 0.f, 0.f};
    float o_acc[G][8];
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) o_acc[q][e] = 0.f;

    const int n_groups = (int)((hi - lo + kGroup - 1) / kGroup);
    for (int gi = wave; gi < n_groups; gi += kWaves) {
        const int64_t k0 = lo + (int64_t)gi * kGroup;
        // K loads in MFMA B layout: sub-tile t, k-step s -> key k0+16t+lane%16, d 32s+8(lane/16)
        u32x4 kr[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            int64_t key = k0 + 16 * t + (lane & 15);
            key = key < hi ? key : hi - 1;
            const uint16_t* src = key == new_key ? knew : kb + key * kD;
#pragma unroll
            for (int s = 0; s < 4; ++s) kr[t][s] = *reinterpret_cast<const u32x4*>(src + s * 32 + qk * 8);
        }
        // V loads: j -> key k0 + 4j + lane/16, d slice 8*(lane%16)
        u32x4 vr[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            int64_t key = k0 + 4 * j + (lane >> 4);
            key = key < hi ? key : hi - 1;
            const uint16_t* src = key == new_key ? vnew : vb + key * kD;
            vr[j] = *reinterpret_cast<const u32x4*>(src + (lane & 15) * 8);
        }

        // S = Q K^T for 4 sub-tiles of 16 keys
        f32x4 sc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, kr[t][s]), sc[t], 0, 0, 0);
        }
        // scale to log2 units and mask keys past the chunk
        float gmax[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) gmax[r] = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool valid = k0 + 16 * t + (lane & 15) < hi;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = valid ? sc[t][r] * p.sl2 : -INFINITY;
                sc[t][r] = x;
                gmax[r] = fmaxf(gmax[r], x);
            }
        }
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mnew = fmaxf(m_run[r], xor_max16(gmax[r]));
            alpha[r] = fast_exp2(m_run[r] - mnew);
            m_run[r] = mnew;
            l_part[r] *= alpha[r];
        }
        // probabilities to LDS: p_lds[key][query]
        const int qq = 4 * (lane >> 4);
        if (qq < G) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f32x4 pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float e = fast_exp2(sc[t][r] - m_run[r]);
                    pv[r] = e;
                    l_part[r] += e;
                }
                if (G >= 4) {
                    *reinterpret_cast<f32x4*>(&p_lds[wave][(16 * t + (lane & 15)) * G + qq]) = pv;
                } else {
#pragma unroll
                    for (int r = 0; r < G; ++r) p_lds[wave][(16 * t + (lane & 15)) * G + r] = pv[r];
                }
            }
            if ((lane & 15) == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (qq + r < G) alpha_lds[wave][qq + r] = alpha[r];
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // rescale O and accumulate P.V
#pragma unroll
        for (int q = 0; q < G; ++q) {
            float al = alpha_lds[wave][q];
#pragma unroll
            for (int e = 0; e < 8; ++e) o_acc[q][e] *= al;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int key = 4 * j + (lane >> 4);
            float vf[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                vf[2 * w] = bf16_lo(vr[j][w]);
                vf[2 * w + 1] = bf16_hi(vr[j][w]);
            }
#pragma unroll
            for (int q = 0; q < G; ++q) {
                float pq = p_lds[wave][key * G + q];
#pragma unroll
                for (int e = 0; e < 8; ++e) o_acc[q][e] = fmaf(pq, vf[e], o_acc[q][e]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- reduce inside the wave: O over the 4 key quarters, l over the 16 key lanes
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o_acc[q][e];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            o_acc[q][e] = x;
        }
    float lw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lw[r] = xor_sum16(l_part[r]);
    if ((lane & 15) == 0) {
        const int qq = 4 * (lane >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (qq + r < G) {
                wm[wave][qq + r] = m_run[r];
                wl[wave][qq + r] = lw[r];
            }
    }
    if (lane < 16) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
            wo[wave][q][2 * lane] = f32x4{o_acc[q][0], o_acc[q][1], o_acc[q][2], o_acc[q][3]};
            wo[wave][q][2 * lane + 1] = f32x4{o_acc[q][4], o_acc[q][5], o_acc[q][6], o_acc[q][7]};
        }
    }
    __syncthreads();

    // ---- combine the 4 waves and write this chunk's partial for each q head
    for (int idx = tid; idx < G * (kD / 4); idx += kThreads) {
        const int q = idx / (kD / 4), e4 = idx % (kD / 4);
        float M = wm[0][q];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[w][q]);
        float W = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            float sc = fast_exp2(wm[w][q] - M);
            W += wl[w][q] * sc;
            o += sc * wo[w][q][e4];
        }
        const float inv = W > 0.f ? 1.0f / W : 0.f;
        const int64_t prow = (int64_t)c * p.hq + g * G + q;
        *reinterpret_cast<f32x4*>(p.pa + prow * kD + e4 * 4) = o * inv;
        if (e4 == 0) {
            p.pm[prow] = W > 0.f ? M * kLn2 : -INFINITY;
            p.pl[prow] = W > 0.f ? W : 0.f;
        }
    }
}

bool decode_bf16_supported(int d, int hq, int hkv) {
    if (d != kD || hkv < 1 || hq % hkv) return false;
    int G = hq / hkv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

int64_t decode_chunk_len(int64_t L, int64_t tail_cap, int32_t hkv) {
    // About 2048 workgroups in total, chunks a multiple of the 4 x 64 keys a pass covers.
    int64_t per_head = L + tail_cap;
    int64_t want = (per_head * hkv + 2047) / 2048;
    int64_t ch = 256;
    while (ch < want && ch < 8192) ch <<= 1;
    return ch;
}

hipError_t launch_decode_bf16(const uint16_t* q_new, const uint16_t* k_new, const uint16_t* v_new,
                              const uint16_t* k_ctx, const uint16_t* v_ctx, int64_t L,
                              uint16_t* k_tail, uint16_t* v_tail, int64_t tail_len, int64_t tail_cap,
                              int hq, int hkv, float scale, const DecodeChunkPlan& plan,
                              float* part_a, float* part_m, float* part_l, hipStream_t stream) {
    DecodeArgs a;
    a.q_new = q_new; a.k_new = k_new; a.v_new = v_new;
    a.k_ctx = k_ctx; a.v_ctx = v_ctx; a.k_tail = k_tail; a.v_tail = v_tail;
    a.L = L; a.tail_len = tail_len; a.tail_cap = tail_cap;
    a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
    a.sl2 = scale * kLog2e;
    a.plan = plan;
    a.pa = part_a; a.pm = part_m; a.pl = part_l;
    const int64_t grid = (int64_t)hkv * plan.n_chunks;
    if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 gd((unsigned)grid), bd(kThreads);
    switch (a.G) {
        case 1: hipLaunchKernelGGL(decode_kernel<1>, gd, bd, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(decode_kernel<2>, gd, bd, 0, stream, a); break;
        case 4: hipLaunchKernelGGL(decode_kernel<4>, gd, bd, 0, stream, a); break;
        case 8: hipLaunchKernelGGL(decode_kernel<8>, gd, bd, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace star
