// Split-KV grouped-query decode for one generated token (bf16, d = 64 or 128).
//
// "Star Attention: Efficient LLM Inference over Long Sequences"
// (paper-graph-ui summary), section 3.4, Phase 2: each context host computes
// the new token's local attention over its cached keys (Step 3), the query
// host does the same over its own growing cache (Steps 3 and 7), and the
// partial results are aggregated in log space (Step 5).  Per generated token
// the work is linear in the cached length, so this kernel is a stream over the
// K/V cache: every K/V byte is read once per step for all G q heads of its kv
// head.
//
// Grid: (kv head, key chunk).  Chunks never straddle a host partition; the
// query host's partition also holds the new token, read from k_new / v_new,
// and the workgroup that owns it appends k_new / v_new to the query host's
// cache (no one reads that slot from memory in the same launch).
//
// Each wave walks 32-key tiles of its chunk with non-temporal loads (the stream is read once
// per step and gains nothing from the last-level cache).  Both products run on
// v_mfma_f32_16x16x32_bf16 with the G <= 16 q heads as the 16-wide column
// block: S^T = K Q^T takes K straight from 16-byte global loads, and
// O^T += V^T P^T takes V^T from a wave-private LDS copy of the V tile (stored
// row-major, read back with the transposing ds_read_b64_tr_b16).  Each wave
// keeps an online softmax; the four waves are combined in LDS into one partial
// (A, m, l) per chunk.  With up to four q heads per kv head, the last workgroup
// of a kv head to finish (an atomic ticket in the workspace) merges that head's
// chunk partials in log space and writes the output, then resets its ticket
// counter to zero.  With more q heads the launcher runs merge_kernel over the
// same partials instead.
//
// The KV8 instantiations read the context hosts' partitions as E4M3 codes with
// one scale per kv head for K and for V (kvfp8.hip).  The codes are widened to
// bf16 in registers with the exact hardware conversion, the K scale is folded
// into the score scale and the V scale into the chunk's partial, so the tiles,
// the softmax and the merge are those of the bf16 path.  The query host's
// partition stays bf16.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace star {

namespace {
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kT = 32;         // keys per tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units

struct DecodeArgs {
    const uint16_t* q_new;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const uint16_t* k_ctx;
    const uint16_t* v_ctx;
    const uint8_t* k8;       // E4M3 context cache (KV8 instantiations), else null
    const uint8_t* v8;
    const float* k_scale;    // [hkv] scales of k8 / v8
    const float* v_scale;
    uint16_t* k_tail;
    uint16_t* v_tail;
    int64_t L, tail_len, tail_cap;
    int hq, hkv, G;
    float sl2;
    DecodeChunkPlan plan;
    float* pa;          // chunk partials: A [n_chunks][hq][d], m and l [n_chunks][hq]
    float* pm;
    float* pl;
    unsigned* tickets;  // [hkv], zero between calls
    uint16_t* o;        // [hq][d]
    float* lse;         // [hq] or null
    int merge_here;     // the last chunk of a kv head merges (else merge_kernel runs next)
};

typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// One tile's operand registers: K (the A operands of S^T) and the V pieces bound for LDS,
// as bf16 or as E4M3 codes (half the bytes).
template <int NK, int NV>
struct TileBf16 {
    u32x4 k[NK];
    u32x4 v[NV];
};
template <int NK, int NV>
struct TileE4m3 {
    u32x4 k[NK];
    u32x4 v[NV];
};

// A load of the K/V stream, marked non-temporal.  Every cached byte is read once per step, so
// caching it in the last-level cache only costs bandwidth: measured on 8b_1m, the bf16 stream
// runs at 7.1 TB/s with these loads against 6.0 TB/s with ordinary ones, and the E4M3 stream
// at 6.9 against 5.8 TB/s.  All of them are 16-byte loads; with 8-byte E4M3 K loads the
// non-temporal form was 12% slower instead.
template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
    return __builtin_nontemporal_load(p);
}

// Four keys of one head-dim column from a row-major LDS tile (see the kernel comment).
__device__ __forceinline__ u32x2v lds_read_tr(const uint16_t* p) {
    lds_bf16x4* lp = (lds_bf16x4*)((__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(p)));
    return __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}
// Max / sum over lanes l, l^16, l^32, l^48 (one q column of the 16x16 layout).  With the
// same register as both operands each swap returns {own, partner} in a lane-dependent order,
// so only symmetric combinations are formed.
__device__ __forceinline__ float quad_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return half_pair_max(x);
}
__device__ __forceinline__ float quad_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return half_pair_sum(x);
}
}  // namespace

#ifdef STAR_DECODE_TIMELINE
// Profiling build only (libstarattn_timeline.so): per-workgroup timestamps of the constant
// 100 MHz clock at fixed points of a launch, read back by star_decode_timeline_read.  Slots:
// 0 start, 1 stream done (waves combined), 2 partial stores complete, 3 ticket drawn,
// 4 merger past its acquire, 5 merge done; 6 holds the ticket.
constexpr int kTimelineGroups = 4096;
__device__ unsigned long long g_decode_timeline[kTimelineGroups][8];
#define STAR_TIMELINE(slot, value)                                                          \
    do {                                                                                    \
        if (threadIdx.x == 0 && blockIdx.x < kTimelineGroups)                               \
            g_decode_timeline[blockIdx.x][slot] = (value);                                  \
    } while (0)
#else
#define STAR_TIMELINE(slot, value) \
    do {                           \
    } while (0)
#endif

template <int G, int D, bool KV8>
__global__ void __launch_bounds__(kThreads, 3)
decode_kernel(const DecodeArgs p) {
    STAR_TIMELINE(0, __builtin_amdgcn_s_memrealtime());
    constexpr int kD = D;                 // head dim, 64 or 128
    constexpr int kVPitch = D + 16;       // bf16 per V row in LDS: 4 consecutive rows hit disjoint banks
    constexpr int kDD = D / 32;           // 32-wide head-dim blocks of the S^T products
    constexpr int kDB = D / 16;           // 16-row blocks of O^T
    constexpr int kRowChunks = D / 8;     // 16-byte chunks per K/V row
    constexpr int kVPieces = kT * kRowChunks / 64;   // 16-byte V pieces per lane per tile
    __shared__ __attribute__((aligned(16))) uint16_t vlds[kWaves][kT * kVPitch];
    __shared__ float wm[kWaves][G], wl[kWaves][G];
    __shared__ float wo[kWaves][G][kD];
    __shared__ unsigned ticket_sh;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, col = lane & 15;   // 16x16 MFMA layout: row group and column
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
        const int64_t tc = c - pl.chunk_prefix[pl.n_shards];
        lo = tc * pl.chunk;
        const int64_t n_tail = p.tail_len + 1;
        hi = lo + pl.chunk < n_tail ? lo + pl.chunk : n_tail;
        kb = p.k_tail + (int64_t)g * p.tail_cap * kD;
        vb = p.v_tail + (int64_t)g * p.tail_cap * kD;
        if (hi == n_tail) {
            new_key = p.tail_len;
            // Append the new token's k / v to the query host's cache (2 x D/8 lanes x 16 B).
            if (tid < 2 * kRowChunks) {
                const bool is_k = tid < kRowChunks;
                const int c16 = tid % kRowChunks;
                const uint16_t* src = (is_k ? p.k_new : p.v_new) + (int64_t)g * kD + c16 * 8;
                uint16_t* dst = (is_k ? p.k_tail : p.v_tail) + ((int64_t)g * p.tail_cap + p.tail_len) * kD + c16 * 8;
                *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
            }
        }
    }
    const uint16_t* knew = p.k_new + (int64_t)g * kD;
    const uint16_t* vnew = p.v_new + (int64_t)g * kD;
    // E4M3 context chunk (uniform over the workgroup)
    const bool f8 = KV8 && c < pl.chunk_prefix[pl.n_shards];
    const uint8_t* kb8 = KV8 ? p.k8 + (int64_t)g * p.L * kD : nullptr;
    const uint8_t* vb8 = KV8 ? p.v8 + (int64_t)g * p.L * kD : nullptr;

    // O^T accumulators: head-dim block db of 16 rows; lane (grp, col) holds rows 16db + 4grp + r.
    f32x4 acc[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref = kNoMax, lsum = 0.f;
    uint16_t* vt = vlds[wave];
    // transposing-read addressing (see the P.V comment below)
    const int trow = 4 * grp + (col >> 2);
    const int tcol = 4 * (col & 3);

    const int n_tiles = (int)((hi - lo + kT - 1) / kT);
    // The tile loop, instantiated for bf16 chunks and (KV8) for E4M3 context chunks.
    auto run_tiles = [&](auto f8_tag) {
    constexpr bool F8 = decltype(f8_tag)::value;
    constexpr int kV8Pieces = kT * kD / 16 / 64;   // 16-byte E4M3 V pieces per lane per tile
    // ---- Q^T as the B operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16): lane (grp, col)
    //      holds q head g*G + col (zero past G) and, for head-dim block dd, the eight head-dim
    //      entries that its K operand holds.  The contraction order over the head dim is free
    //      as long as K and Q agree.  bf16 chunks take block dd, slot 8grp + i as head-dim
    //      32dd + 8grp + i.  E4M3 chunks take it as 64(dd/2) + 16grp + 8(dd%2) + i, so that one
    //      16-byte load of codes per lane covers the blocks 2j and 2j + 1.
    bf16x8 qb[kDD];
#pragma unroll
    for (int dd = 0; dd < kDD; ++dd) {
        const int off = F8 ? 64 * (dd / 2) + 16 * grp + 8 * (dd % 2) : 32 * dd + 8 * grp;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (col < G) w = *reinterpret_cast<const u32x4*>(p.q_new + (int64_t)(g * G + col) * kD + off);
        qb[dd] = __builtin_bit_cast(bf16x8, w);
    }
    // score scale (log2 units), with the K scale of an E4M3 chunk folded in
    const float sl2 = F8 ? p.sl2 * p.k_scale[g] : p.sl2;
    // K operands (16-key block kb, head-dim block dd: key k0 + 16kb + col, the head-dim order
    // above) and V row-major pieces for LDS, for the tile that starts at key k0.  Keys past the
    // chunk are clamped to its last key.  E4M3 chunks load half the bytes (one 16-byte load per
    // lane for two head-dim blocks) and widen them to bf16 when they are used; a wave keeps two
    // of their tiles in flight (kDepth), so that it has as many bytes outstanding as with one
    // bf16 tile.
    using Tile = typename std::conditional<F8, TileE4m3<kDD, kV8Pieces>, TileBf16<2 * kDD, kVPieces>>::type;
    constexpr int kDepth = F8 ? 2 : 1;
    Tile buf[kDepth];
    auto load_tile = [&](Tile& b, int64_t k0) {
        if constexpr (F8) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                int64_t key = k0 + 16 * kb2 + col;
                key = key < hi ? key : hi - 1;
                const uint8_t* src = kb8 + key * kD;
#pragma unroll
                for (int j = 0; j < kDD / 2; ++j)
                    b.k[kb2 * (kDD / 2) + j] = stream_load(reinterpret_cast<const u32x4*>(src + 64 * j + 16 * grp));
            }
#pragma unroll
            for (int i = 0; i < kV8Pieces; ++i) {
                const int cc = lane + 64 * i;
                int64_t vkey = k0 + cc / (kD / 16);
                vkey = vkey < hi ? vkey : hi - 1;
                b.v[i] = stream_load(reinterpret_cast<const u32x4*>(vb8 + vkey * kD + (cc % (kD / 16)) * 16));
            }
        } else {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            int64_t key = k0 + 16 * kb2 + col;
            key = key < hi ? key : hi - 1;
            const uint16_t* src = key == new_key ? knew : kb + key * kD;
#pragma unroll
            for (int dd = 0; dd < kDD; ++dd) b.k[kb2 * kDD + dd] = stream_load(reinterpret_cast<const u32x4*>(src + dd * 32 + grp * 8));
        }
#pragma unroll
        for (int i = 0; i < kVPieces; ++i) {
            const int cc = lane + 64 * i;
            int64_t vkey = k0 + cc / kRowChunks;
            vkey = vkey < hi ? vkey : hi - 1;
            const uint16_t* vsrc = vkey == new_key ? vnew : vb + vkey * kD;
            b.v[i] = stream_load(reinterpret_cast<const u32x4*>(vsrc + (cc % kRowChunks) * 8));
        }
        }
    };
    // One tile of this wave: S^T from b, V from b into LDS, then b takes the load of the
    // tile kDepth steps ahead while the softmax and P.V of this one run.
    auto tile_body = [&](Tile& b, int t) {
        const int64_t k0 = lo + (int64_t)t * kT;
        // S^T = K Q^T: s[kb][r] is key k0 + 16kb + 4grp + r for q column col; and this tile's V
        // into the wave's LDS tile
        f32x4 s[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            s[kb2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dd = 0; dd < kDD; ++dd) {
                u32x4 kop;
                if constexpr (F8)
                    kop = e4m3x8_to_bf16x8(b.k[kb2 * (kDD / 2) + dd / 2][2 * (dd % 2)],
                                           b.k[kb2 * (kDD / 2) + dd / 2][2 * (dd % 2) + 1]);
                else
                    kop = b.k[kb2 * kDD + dd];
                s[kb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop), qb[dd], s[kb2], 0, 0, 0);
            }
        }
        if constexpr (F8) {
#pragma unroll
            for (int i = 0; i < kV8Pieces; ++i) {
                const int cc = lane + 64 * i;
                uint16_t* dst = vt + (cc / (kD / 16)) * kVPitch + (cc % (kD / 16)) * 16;
                *reinterpret_cast<u32x4*>(dst) = e4m3x8_to_bf16x8(b.v[i][0], b.v[i][1]);
                *reinterpret_cast<u32x4*>(dst + 8) = e4m3x8_to_bf16x8(b.v[i][2], b.v[i][3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kVPieces; ++i) {
                const int cc = lane + 64 * i;
                *reinterpret_cast<u32x4*>(vt + (cc / kRowChunks) * kVPitch + (cc % kRowChunks) * 8) = b.v[i];
            }
        }
        // The operand registers are free again: the next tile's loads fly while this
        // tile's softmax and P.V run.
        __builtin_amdgcn_sched_barrier(0);
        if (t + kDepth * kWaves < n_tiles) load_tile(b, k0 + (int64_t)kDepth * kWaves * kT);
        __builtin_amdgcn_sched_barrier(0);
        if (k0 + kT > hi) {
            const int lim = (int)(hi - k0);
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * kb2 + 4 * grp + r >= lim) s[kb2][r] = -INFINITY;
        }
        // online softmax with a lazily moved reference; a column's 32 keys sit in lanes
        // col, col+16, col+32, col+48
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = quad_max(mx) * sl2;
        if (__builtin_amdgcn_ballot_w64(mx > mref + kRescaleThreshold)) {
            const float nref = fmaxf(mref, mx);
            const float alpha = fast_exp2(mref - nref);
            mref = nref;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < kDB; ++db) acc[db] *= alpha;
        }
        bf16x8 pb;
        {
            const float negm = -mref;
            float e[8];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 4; ++r) e[4 * kb2 + r] = fast_exp2(fmaf(s[kb2][r], sl2, negm));
            lsum += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
            u32x4 w;
            w[0] = pack_bf16x2(e[0], e[1]);
            w[1] = pack_bf16x2(e[2], e[3]);
            w[2] = pack_bf16x2(e[4], e[5]);
            w[3] = pack_bf16x2(e[6], e[7]);
            pb = __builtin_bit_cast(bf16x8, w);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // O^T += V^T P^T over the 32 keys.  k-slot i of lane group grp is key 4grp + i (i < 4)
        // or 16 + 4grp + i - 4, the S^T layout above.  In each 16-lane group of a transposing
        // read, source lane s points at key (s/4) of its four-key set and at columns
        // 4*(s%4) .. +3 of the 16-wide head-dim block; result lane i then holds column i of
        // the block for the four keys.  Two reads give the 8 slots.
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const uint16_t* base = vt + trow * kVPitch + db * 16 + tcol;
            const u32x2v a0 = lds_read_tr(base);
            const u32x2v a1 = lds_read_tr(base + 16 * kVPitch);
            const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, acc[db], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
#pragma unroll
    for (int j = 0; j < kDepth; ++j)
        if (wave + j * kWaves < n_tiles) load_tile(buf[j], lo + (int64_t)(wave + j * kWaves) * kT);
    for (int t = wave; t < n_tiles; t += kDepth * kWaves) {
#pragma unroll
        for (int j = 0; j < kDepth; ++j)
            if (t + j * kWaves < n_tiles) tile_body(buf[j], t + j * kWaves);
    }
    };
    if constexpr (KV8) {
        if (f8)
            run_tiles(std::true_type{});
        else
            run_tiles(std::false_type{});
    } else {
        run_tiles(std::false_type{});
    }

    // ---- combine the four waves into this chunk's partial
    const float lw = quad_sum(lsum);
    if (col < G) {
        if (grp == 0) {
            wm[wave][col] = mref;
            wl[wave][col] = lw;
        }
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) wo[wave][col][db * 16 + 4 * grp + r] = acc[db][r];
    }
    __syncthreads();
    STAR_TIMELINE(1, __builtin_amdgcn_s_memrealtime());
    const float vsc = (KV8 && f8) ? p.v_scale[g] : 1.0f;   // V scale of an E4M3 chunk
    for (int idx = tid; idx < G * kD; idx += kThreads) {
        const int q = idx / kD, d = idx % kD;
        float M = wm[0][q];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[w][q]);
        float W = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = fast_exp2(wm[w][q] - M);
            W += wl[w][q] * sc;
            o += sc * wo[w][q][d];
        }
        const int64_t prow = (int64_t)c * p.hq + g * G + q;
        // Device-scope stores: they complete at the level that every XCD reads.
        __hip_atomic_store(p.pa + prow * kD + d, W > 0.f ? (o / W) * vsc : 0.f, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
            __hip_atomic_store(p.pm + prow, W > 0.f ? M * kLn2 : -INFINITY, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p.pl + prow, W > 0.f ? W : 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    if (!p.merge_here) return;
    // ---- the last chunk of this kv head to finish merges all of them.
    // The partial was written with device-scope stores, so once they have completed
    // (vmcnt 0) every workgroup can see it.  A device-scope release fence would add a
    // write-back of this XCD's whole L2 per workgroup, which costs more than the merge.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    STAR_TIMELINE(2, __builtin_amdgcn_s_memrealtime());
    if (tid == 0) ticket_sh = __hip_atomic_fetch_add(&p.tickets[g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    STAR_TIMELINE(3, __builtin_amdgcn_s_memrealtime());
    STAR_TIMELINE(6, ticket_sh);
    if (ticket_sh != (unsigned)(pl.n_chunks - 1)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // no stale cached partials below
    STAR_TIMELINE(4, __builtin_amdgcn_s_memrealtime());
    const int nc = pl.n_chunks;
    // One wave per q head.  The chunks are taken in batches of 64, and every load of a batch is
    // issued at once (one memory round trip): lane i loads the statistics (m, l) of chunk
    // c0 + i, and the column loads are 16 bytes wide, so that one load instruction covers
    // kRows = 256 / D chunk rows (D/4 lanes per row) and a batch needs 64 / kRows of them, within
    // the per-wave limit on loads in flight.  The wave then forms the batch max and weights and
    // folds the weighted columns, rescaling what earlier batches left when the max grows; the
    // kRows lane groups each sum every kRows-th chunk and are added at the end.
    constexpr int kLanesPerRow = D / 4;
    constexpr int kRows = 64 / kLanesPerRow;
    constexpr int kBatch = 64;
    constexpr int kLoads = kBatch / kRows;
    const int sub = lane / kLanesPerRow, c4 = lane % kLanesPerRow;
    for (int q = wave; q < G; q += kWaves) {
        const int h = g * G + q;
        float M = -INFINITY, W = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nc; c0 += kBatch) {
            const int nb = nc - c0 < kBatch ? nc - c0 : kBatch;
            float m = -INFINITY, l = 0.f;
            if (lane < nb) {
                const int64_t row = (int64_t)(c0 + lane) * p.hq + h;
                m = p.pm[row];
                l = p.pl[row];
            }
            // chunk rows are hq * D floats apart; load jb takes row c0 + kRows*jb + sub
            f32x4 a[kLoads];
            const float* rowp = p.pa + ((int64_t)(c0 + sub) * p.hq + h) * kD + 4 * c4;
            const int64_t row_step = (int64_t)kRows * p.hq * kD;
#pragma unroll
            for (int jb = 0; jb < kLoads; ++jb) {
                a[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (kRows * jb + sub < nb) a[jb] = *reinterpret_cast<const f32x4*>(rowp);
                rowp += row_step;
            }
            const float nM = fmaxf(M, wave_max(m));
            const float so = M == -INFINITY ? 0.f : __expf(M - nM);
            const float w = m == -INFINITY ? 0.f : l * __expf(m - nM);   // zero past nb
            W = W * so + wave_sum(w);
            o *= so;
#pragma unroll
            for (int jb = 0; jb < kLoads; ++jb) {
                if (kRows * jb < nb) {
                    // the weight of chunk c0 + kRows*jb + sub
                    float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), kRows * jb));
#pragma unroll
                    for (int r = 1; r < kRows; ++r) {
                        const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), kRows * jb + r));
                        wj = sub == r ? wr : wj;
                    }
                    o += wj * a[jb];
                }
            }
            M = nM;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = kRows == 2 ? half_pair_sum(o[e]) : quad_sum(o[e]);
        const bool empty = M == -INFINITY || !(W > 0.f);
        const float inv = empty ? 0.f : 1.0f / W;
        if (sub == 0) {
            u32x2 ow;
            ow[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
            ow[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
            *reinterpret_cast<u32x2*>(p.o + (int64_t)h * kD + 4 * c4) = ow;
        }
        if (lane == 0 && p.lse) p.lse[h] = empty ? -INFINITY : M + __logf(W);
    }
#ifdef STAR_DECODE_TIMELINE
    __syncthreads();
    STAR_TIMELINE(5, __builtin_amdgcn_s_memrealtime());
#endif
    // ready for the next call on this stream
    if (tid == 0) __hip_atomic_store(&p.tickets[g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

namespace {
template <int D, bool KV8>
hipError_t launch_decode_g(const DecodeArgs& a, dim3 gd, hipStream_t stream) {
    const dim3 bd(kThreads);
    switch (a.G) {
        case 1: hipLaunchKernelGGL((decode_kernel<1, D, KV8>), gd, bd, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<2, D, KV8>), gd, bd, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<4, D, KV8>), gd, bd, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((decode_kernel<8, D, KV8>), gd, bd, 0, stream, a); break;
        case 16: hipLaunchKernelGGL((decode_kernel<16, D, KV8>), gd, bd, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_bf16(const uint16_t* q_new, const uint16_t* k_new, const uint16_t* v_new,
                              const uint16_t* k_ctx, const uint16_t* v_ctx, const uint8_t* k8, const uint8_t* v8,
                              const float* k_scale, const float* v_scale, int64_t L,
                              uint16_t* k_tail, uint16_t* v_tail, int64_t tail_len, int64_t tail_cap,
                              int hq, int hkv, int d, float scale, const DecodeChunkPlan& plan,
                              float* part_a, float* part_m, float* part_l, unsigned* tickets,
                              uint16_t* o, float* lse, hipStream_t stream) {
    DecodeArgs a;
    a.q_new = q_new; a.k_new = k_new; a.v_new = v_new;
    a.k_ctx = k_ctx; a.v_ctx = v_ctx; a.k_tail = k_tail; a.v_tail = v_tail;
    a.k8 = k8; a.v8 = v8; a.k_scale = k_scale; a.v_scale = v_scale;
    a.L = L; a.tail_len = tail_len; a.tail_cap = tail_cap;
    a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
    a.sl2 = scale * kLog2e;
    a.plan = plan;
    a.pa = part_a; a.pm = part_m; a.pl = part_l;
    a.tickets = tickets;
    a.o = o; a.lse = lse;
    const int64_t grid = (int64_t)hkv * plan.n_chunks;
    if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool kv8 = k8 != nullptr;
    if (kv8 && (!v8 || !k_scale || !v_scale)) return hipErrorInvalidValue;
    const dim3 gd((unsigned)grid);
    // Up to four q heads per kv head, the last chunk of each kv head merges in the same launch
    // (one wave per q head).  With more, a wave would merge several q heads one after the
    // other, which measured no faster than merge_kernel over the same partials (one
    // workgroup per q head) in a second launch.
    a.merge_here = a.G <= kWaves;
    hipError_t e = hipErrorInvalidValue;
    if (d == 128) e = kv8 ? launch_decode_g<128, true>(a, gd, stream) : launch_decode_g<128, false>(a, gd, stream);
    if (d == 64) e = kv8 ? launch_decode_g<64, true>(a, gd, stream) : launch_decode_g<64, false>(a, gd, stream);
    if (e != hipSuccess || a.merge_here) return e;
    return launch_merge(part_a, part_m, part_l, plan.n_chunks, hq, d, o, true, lse, nullptr, nullptr, stream);
}

}  // namespace star

#ifdef STAR_DECODE_TIMELINE
// Profiling build only: copy the timestamps of the last decode launch to host (at most
// 4096 workgroups x 8 slots of 8 bytes), or clear them (host == NULL).  Synchronous.
extern "C" STAR_API int star_decode_timeline_read(void* host, size_t bytes) {
    if (bytes > sizeof(star::g_decode_timeline)) return (int)hipErrorInvalidValue;
    if (!host) {
        static unsigned long long zeros[star::kTimelineGroups][8];
        return (int)hipMemcpyToSymbol(HIP_SYMBOL(star::g_decode_timeline), zeros, sizeof(zeros), 0,
                                      hipMemcpyHostToDevice);
    }
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(star::g_decode_timeline), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

