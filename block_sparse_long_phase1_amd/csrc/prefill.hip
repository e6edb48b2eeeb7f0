// Anchored flash-style attention on gfx950 bf16 MFMA.
//
// One kernel body serves two callers:
//   * Phase 1 context encoding ("Star Attention: Efficient LLM Inference over
//     Long Sequences", paper-graph-ui summary, section 3.4, Phase 1 Steps 2-5):
//     a row in block i >= 1 sees the anchor [0, anchor) unmasked and its own
//     block causally; block 0 rows see their block causally.
//   * Phase 2 local attention of query rows over one KV partition (same page,
//     Phase 2 Step 3): no mask for a context shard, a causal offset for the
//     query host's own cache; key splits of one partition are merged later.
//
// Head dim 64 or 128 (template parameter D).
//
// Work unit: one workgroup = 256 queries that share one kv head (G q heads x
// 256/G consecutive rows), so each K/V tile staged in LDS feeds the whole GQA
// group.  8 waves (two per SIMD), 32 queries each; every value stays in VGPRs.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// every lane owns one query column, so the softmax row statistics need no
// cross-lane reduction beyond one exchange between lanes l and l^32.  The
// probabilities P^T come out of the score accumulators already in the
// B-operand layout of the second product O^T += V^T P^T, whose V^T operand is
// read from the row-major V tile with transposing LDS reads.
//
// Tiles of 64 keys are double-buffered in LDS and copied there by direct
// global-to-LDS loads, which take no registers and no LDS store instructions;
// the copy of tile j+1 is in flight while tile j is multiplied.  The two stages
// are separate LDS objects so that reads of one never wait for the copy into
// the other.  Softmax runs in the exp2 domain with a lazily updated reference
// max: the accumulators are only rescaled when a row's max grows by more than
// 2^8, which keeps every probability below 256 and is exact after the final
// normalisation.
#include "common.h"
#include "internal.h"

namespace star {

namespace {

constexpr int kThreads = 512;
constexpr int kBN = 64;          // keys per tile
constexpr int kQPB = 256;        // queries per workgroup
constexpr int kKB = kBN / 32;    // 32-key MFMA blocks per tile
// LDS tile layout for head dim D (rows of 2D bytes).  A tile's 64 key rows sit in 1 KB
// blocks of 1024/(2D) rows: with NB = 64 / (rows per block) blocks, block b holds rows
// b, b + NB, b + 2NB, ...; consecutive rows therefore fall in consecutive blocks.  Blocks
// are padded so that each starts 16 B (K) or 64 B (V) further around the 256-byte bank
// cycle than the previous one: the 16 rows read by a K operand read, and the 4 rows x 4
// chunks of a transposing V read, then touch distinct banks, and every operand address
// is one per-lane base plus a constant.
constexpr int kKBlock = 1024 + 16;            // bytes per K block
constexpr int kVBlock = 1024 + 64;            // bytes per V block
template <int D>
struct Geo {
    static_assert(D == 64 || D == 128, "head dim");
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
    static constexpr int kRowsPerBlock = 1024 / kRowBytes;
    static constexpr int kBlocks = kBN / kRowsPerBlock;
    static constexpr int kKTileBytes = kBlocks * kKBlock;
    static constexpr int kVTileBytes = kBlocks * kVBlock;
    static constexpr int kStageBytes = kKTileBytes + kVTileBytes;
    static constexpr int kST = D / 16;                      // k-steps of S^T = K Q^T
    static constexpr int kDB = D / 32;                      // 32-row blocks of O^T
    // byte offset, inside the V tile, of row r + 8 relative to row r (r % NB < 8)
    static constexpr int kPlus8 = (8 % kBlocks) * kVBlock + (8 / kBlocks) * kRowBytes;
};
constexpr float kRescaleThreshold = 8.0f;     // log2 units
constexpr float kSumBound = 1048576.0f;       // 2^20

typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// Four keys of one head-dim column from a row-major LDS tile (see the P.V comment).
__device__ __forceinline__ u32x2v lds_read_tr(const char* p) {
    lds_bf16x4* lp = (lds_bf16x4*)((__attribute__((address_space(3))) char*)(const_cast<char*>(p)));
    return __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

typedef __attribute__((address_space(3))) void lds_void;

// Copy one K/V tile straight from global memory into an LDS stage (no registers).
// One instruction fills one 1 KB block (lane i writes bytes 16i .. 16i+15 of it):
// row b + NB*(i / chunks per row), 16-byte chunk i % chunks per row.  Waves 0-3 fill
// the K blocks, waves 4-7 the V blocks.  Keys at or past `kmax` are clamped to kmax-1
// (always a valid row); their scores are masked later.  Key offsets from the kv head's
// base fit in 32 bits (checked on the host).  `wave` must be wave-uniform.
template <int D>
__device__ __forceinline__ void dma_tile(char* stage, const uint16_t* __restrict__ kb,
                                         const uint16_t* __restrict__ vb, int key0, int kmax, int wave, int lane) {
    using T = Geo<D>;
    const bool is_k = wave < 4;
    const char* src = reinterpret_cast<const char*>(is_k ? kb : vb);
    char* dst = stage + (is_k ? 0 : T::kKTileBytes);
    const int blk_bytes = is_k ? kKBlock : kVBlock;
    const int w4 = wave & 3;
    constexpr int kPerWave = T::kBlocks / 4;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int b = w4 * kPerWave + i;
        const int row = b + T::kBlocks * (lane / T::kChunks);
        const int key = min(key0 + row, kmax - 1);
        const uint32_t off = (uint32_t)key * T::kRowBytes + (uint32_t)(lane % T::kChunks) * 16u;
        __builtin_amdgcn_global_load_lds((const void*)(src + off), (lds_void*)(dst + b * blk_bytes), 16, 0, 0);
    }
}

// Description of the keys one workgroup visits: segment A (tiles [0, nta)),
// then segment B.  Positions are token indices into the kv head's rows.
struct KeyPlan {
    int64_t a_lo, a_hi;   // segment A: no causal mask, keys >= a_hi masked
    int64_t b_lo, b_hi;   // segment B: keys >= b_hi masked; causal if `causal`
    int nta, ntb;
    bool causal;
    int64_t diag;         // causal: visible iff key <= row + diag  (row = query row index)
    int64_t kmax;         // tokens available in memory for this kv head
};

}  // namespace

// MODE 0 = Phase 1 encode, 1 = Phase 2 partial; D = head dim (64 or 128).
template <int MODE, int D>
__global__ void __launch_bounds__(kThreads, 2)
attn_mfma_kernel(const AttnMfmaArgs p) {
    using T = Geo<D>;
    constexpr int kD = D;
    __shared__ __attribute__((aligned(16))) char smem0[T::kStageBytes];
    __shared__ __attribute__((aligned(16))) char smem1[T::kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;   // which 4-row group of the 32x32 layout this lane holds
    const int col = lane & 31;    // query column inside the wave's 32-query block

    // ---------------------------------------------------------------- work item
    // Work order.  Heads interleave (blockIdx % Hkv) while the whole K/V cache fits the
    // 256 MB last-level cache: with 8 kv heads that pins each head to one XCD and its L2.
    // Larger caches go head by head, so the workgroups running together share one head's
    // anchor tiles in the last-level cache.
    int g;
    int64_t rank;
    if (MODE == 0 && p.head_major) {
        const int64_t per_head = p.tiles_ge1 + p.nt0;
        g = (int)(blockIdx.x / per_head);
        rank = blockIdx.x % per_head;
    } else {
        g = blockIdx.x % p.hkv;
        rank = blockIdx.x / p.hkv;
    }
    int64_t row0, row_end;        // query rows [row0, row_end) valid for this workgroup
    KeyPlan kp;
    int split = 0;
    const uint16_t* kptr = p.k;   // this work item's key partition
    const uint16_t* vptr = p.v;
    int64_t hstride = p.kv_head_stride;
    if (MODE == 0) {
        // Heaviest tiles first: last row tiles of blocks >= 1, then block 0.
        int64_t blk, rt;
        if (rank < p.tiles_ge1) {
            const int64_t hi_levels = (p.nt_full - p.nt_last) * (p.n_blocks - 2);
            if (rank < hi_levels) {
                rt = p.nt_full - 1 - rank / (p.n_blocks - 2);
                blk = 1 + rank % (p.n_blocks - 2);
            } else {
                const int64_t r = rank - hi_levels;
                rt = p.nt_last - 1 - r / (p.n_blocks - 1);
                blk = 1 + r % (p.n_blocks - 1);
            }
        } else {
            blk = 0;
            rt = p.nt0 - 1 - (rank - p.tiles_ge1);
        }
        const int64_t bstart = blk * p.block;
        const int64_t bend = bstart + p.block < p.L ? bstart + p.block : p.L;
        row0 = bstart + rt * p.rows_per_wg;
        row_end = row0 + p.rows_per_wg < bend ? row0 + p.rows_per_wg : bend;
        kp.a_lo = 0;
        kp.a_hi = blk >= 1 ? p.anchor : 0;
        kp.b_lo = bstart;
        kp.b_hi = row_end;  // keys past the last valid row are never visible
        kp.causal = true;
        kp.diag = 0;
        kp.kmax = p.L;
    } else {
        // Split `split` of partition `part` (global split order), row tile rt.
        const PartPlan& pl = p.plan;
        const int64_t rt = rank % p.n_row_tiles;
        split = (int)(rank / p.n_row_tiles);
        int part = 0;
        while (split >= pl.split_prefix[part + 1]) ++part;
        row0 = rt * p.rows_per_wg;
        row_end = row0 + p.rows_per_wg < p.rows ? row0 + p.rows_per_wg : p.rows;
        const int64_t n_kv = pl.n_kv[part];
        const int64_t lo = (int64_t)(split - pl.split_prefix[part]) * pl.split_len;
        int64_t hi = lo + pl.split_len < n_kv ? lo + pl.split_len : n_kv;
        kp.causal = pl.causal[part] >= 0;
        kp.diag = pl.causal[part];
        if (kp.causal) {
            const int64_t lim = kp.diag + row_end;  // keys >= lim are invisible to every row here
            hi = hi < lim ? hi : lim;
        }
        kp.a_lo = kp.a_hi = 0;
        kp.b_lo = lo;
        kp.b_hi = hi > lo ? hi : lo;
        kp.kmax = n_kv;
        kptr = pl.k[part];
        vptr = pl.v[part];
        hstride = pl.head_stride[part];
    }
    kp.nta = (int)((kp.a_hi - kp.a_lo + kBN - 1) / kBN);
    kp.ntb = (int)((kp.b_hi - kp.b_lo + kBN - 1) / kBN);
    const int nt = kp.nta + kp.ntb;

    // ---------------------------------------------------------------- this lane's query
    // Query index qi in [0, 256): head g*G + qi / rows_per_wg, row row0 + qi % rows_per_wg.
    const int qi = wave * 32 + col;
    const int qhead = g * p.G + qi / p.rows_per_wg;
    const int64_t qrow = row0 + qi % p.rows_per_wg;
    const bool qvalid = (qi / p.rows_per_wg) < p.G && qrow < row_end;
    bf16x8 qb[T::kST];
    {
        const uint16_t* qp = p.q + ((int64_t)qhead * p.q_rows + (qvalid ? qrow : 0)) * kD;
#pragma unroll
        for (int st = 0; st < T::kST; ++st) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (qvalid) w = *reinterpret_cast<const u32x4*>(qp + st * 16 + half * 8);
            qb[st] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x16 acc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float mref = kNoMax;   // reference max (log2 units) used in the exponent
    float mtrue = kNoMax;  // largest score seen (log2 units)
    float lsum = 0.f;      // this lane's half of the row sum
    const float sl2 = p.scale_log2;

    const uint16_t* kbase = kptr + (int64_t)g * hstride;
    const uint16_t* vbase = vptr + (int64_t)g * hstride;
    const int kmax = (int)kp.kmax;
    const int a_lo = (int)kp.a_lo, b_lo = (int)kp.b_lo;
    auto tile_key0 = [&](int j) -> int { return j < kp.nta ? a_lo + j * kBN : b_lo + (j - kp.nta) * kBN; };

    f32x16 s[kKB];   // S^T of the current tile, one 32-key block per entry

    // Mask tile j's scores in place where the tile can hold an invisible key.
    auto mask = [&](int j) {
        const int key0 = tile_key0(j);
        const bool in_a = j < kp.nta;
        const int seg_hi = in_a ? (int)kp.a_hi : (int)kp.b_hi;
        bool need = key0 + kBN > seg_hi;
        if (!in_a && kp.causal) need |= (int64_t)key0 + kBN - 1 > row0 + kp.diag;
        if (need) {
            const int lim = min(seg_hi - key0, kBN);
            const int64_t r64 = (in_a || !kp.causal) ? (int64_t)kBN : qrow + kp.diag - key0;
            const int rlim = r64 > kBN ? kBN : (r64 < -1 ? -1 : (int)r64);
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rel = kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                    if (rel >= lim || rel > rlim) s[kb][r] = -INFINITY;
                }
        }
    };

    // transposing-read addressing inside a 16-key step (see the P.V comment below)
    const int trow = 4 * half + ((lane & 15) >> 2);
    const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);

    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    auto step = [&](int j, const char* cur, char* nxt) {
        if (j + 1 < nt) dma_tile<D>(nxt, kbase, vbase, tile_key0(j + 1), kmax, uwave, lane);
        const char* vs = cur + T::kKTileBytes;
        // K operand: row kb*32 + col, chunk 2*st + half: row col is in block col % NB at
        // position col / NB; kb adds 32 rows, i.e. 32/NB positions of 2D bytes (512 B).
        const char* kp = cur + (col % T::kBlocks) * kKBlock + (col / T::kBlocks) * T::kRowBytes + half * 16;
        // V operand rows 16u + trow (+8): block trow (+8), row u inside it.
        const char* vp = vs + trow * kVBlock + tcol * 2;   // trow < 8 <= NB: block trow, position 0

        // ---- S^T = K Q^T, one 32-key block at a time, all eight K operands read first
        auto scores = [&]() {
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) {
                u32x4 ka[T::kST];
#pragma unroll
                for (int st = 0; st < T::kST; ++st)
                    ka[st] = *reinterpret_cast<const u32x4*>(kp + kb * 512 + st * 32);
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
                for (int st = 0; st < T::kST; ++st)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[st]), qb[st], s[kb],
                                                                   0, 0, 0);
            }
        };
        scores();
        mask(j);

        // ---- tile max; move the reference (and rescale) only if it grew past 2^8
        auto rescale_to_max = [&]() {
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = half_pair_max(mx) * sl2;
            mtrue = fmaxf(mtrue, mx);
            if (__builtin_amdgcn_ballot_w64(mx > mref + kRescaleThreshold)) {
                const float nref = fmaxf(mref, mx);
                const float alpha = fast_exp2(mref - nref);
                mref = nref;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < T::kDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            }
        };
        // Phase-2 partials report the true max, so they take the max of every tile; Phase 1
        // takes it on its first tile only (see below).
        if (MODE == 1 || j == 0) rescale_to_max();

        // ---- P^T = exp2(S^T - ref) in place, row sums from the unrounded values
        auto exps = [&]() -> float {
            const float negm = -mref;
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] = fast_exp2(fmaf(s[kb][r], sl2, negm));
                    ls += s[kb][r];
                }
            return ls;
        };
        float ls = exps();
        // Phase 1 keeps the tile when every row's sum of probabilities is at most 2^20: no
        // probability overflowed and the accumulators stay far from the fp32 range, so the
        // reference need not move.  Else (scores far above the reference) the scores are
        // recomputed from the K tile, the reference moves to their max and the probabilities
        // are redone.  This replaces a max over every tile's scores.
        if (MODE == 0 && __builtin_amdgcn_ballot_w64(!(ls <= kSumBound))) {
            scores();
            mask(j);
            rescale_to_max();
            ls = exps();
        }
        lsum += ls;

        // ---- V^T operands by transposing reads of the row-major V tile.  16-key step u:
        //      slot i of lane half h is key 16u + 8*(i/4) + 4h + i%4, the S^T layout.  In a
        //      16-lane group, source lane s points at key (s/4) of a four-key set and at
        //      columns 4*(s%4) .. +3 of the group's 16-wide head-dim slice; result lane i
        //      holds column i of that slice for the four keys.
        u32x4 va[2 * kKB][T::kDB];
#pragma unroll
        for (int u = 0; u < 2 * kKB; ++u)
#pragma unroll
            for (int db = 0; db < T::kDB; ++db) {
                // row 16u + trow: 16 rows are 16/NB positions of 2D bytes (256 B) further on
                const u32x2v a0 = lds_read_tr(vp + u * 256 + db * 64);
                const u32x2v a1 = lds_read_tr(vp + T::kPlus8 + u * 256 + db * 64);
                va[u][db] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }


        // ---- O^T += V^T P^T
#pragma unroll
        for (int u = 0; u < 2 * kKB; ++u) {
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = pack_bf16x2(s[u >> 1][8 * (u & 1) + 2 * i], s[u >> 1][8 * (u & 1) + 2 * i + 1]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int db = 0; db < T::kDB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[u][db]), pb,
                                                                 acc[db], 0, 0, 0);
        }
        // This wave's copies into `nxt` have landed; after the barrier every wave's have,
        // and every wave is done reading `cur`.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (nt > 0) {
        dma_tile<D>(smem0, kbase, vbase, tile_key0(0), kmax, uwave, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int j = 0;
        for (; j + 1 < nt; j += 2) {
            step(j, smem0, smem1);
            step(j + 1, smem1, smem0);
        }
        if (j < nt) step(j, smem0, smem1);
    }

    // ---------------------------------------------------------------- epilogue
    const float l = half_pair_sum(lsum);
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.0f / l;
    if (!qvalid) return;
    const int64_t hr = (int64_t)qhead * p.q_rows + qrow;
    if (MODE == 0) {
        uint16_t* op = p.o + hr * kD;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = db * 32 + gq * 8 + half * 4;
                u32x2 w;
                w[0] = pack_bf16x2(acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv);
                w[1] = pack_bf16x2(acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv);
                *reinterpret_cast<u32x2*>(op + d0) = w;
            }
        if (p.lse && half == 0) p.lse[hr] = (mref + __builtin_amdgcn_logf(l)) * kLn2;
    } else {
        const int64_t out_row = (int64_t)split * p.hq * p.q_rows + hr;
        float* ap = p.a_out + out_row * kD;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = db * 32 + gq * 8 + half * 4;
                const f32x4 w = {acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv,
                                 acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv};
                *reinterpret_cast<f32x4*>(ap + d0) = w;
            }
        if (half == 0) {
            // Report (m, l) against the true max so that m is the largest scaled score.
            p.m_out[out_row] = empty ? -INFINITY : mtrue * kLn2;
            p.l_out[out_row] = empty ? 0.f : l * fast_exp2(mref - mtrue);
        }
    }
}

// ------------------------------------------------------------------------- launchers

bool attn_mfma_supported(int d, int hq, int hkv) {
    if ((d != 64 && d != 128) || hkv < 1 || hq % hkv) return false;
    const int G = hq / hkv;
    return G >= 1 && G <= kQPB && (kQPB % G) == 0;
}

int64_t attn_mfma_max_tokens(int d) { return ((int64_t)1 << 31) / d; }

hipError_t launch_phase1_mfma(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* o, float* lse, int64_t L, int64_t block, int64_t anchor,
                              int hq, int hkv, int d, float scale, hipStream_t stream) {
    AttnMfmaArgs a = {};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.L = L; a.block = block; a.anchor = anchor;
    a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
    a.rows_per_wg = kQPB / a.G;
    a.q_rows = L;
    a.kv_head_stride = L * d;
    a.scale_log2 = scale * kLog2e;
    const int64_t rw = a.rows_per_wg;
    a.n_blocks = (L + block - 1) / block;
    const int64_t len0 = block < L ? block : L;
    const int64_t len_last = L - (a.n_blocks - 1) * block;
    a.nt_full = (block + rw - 1) / rw;
    a.nt_last = (len_last + rw - 1) / rw;
    a.nt0 = (len0 + rw - 1) / rw;
    int64_t tiles_ge1 = 0;
    if (a.n_blocks >= 2) tiles_ge1 = (a.n_blocks - 2) * a.nt_full + a.nt_last;
    a.tiles_ge1 = tiles_ge1;
    const int64_t tiles = tiles_ge1 + a.nt0;
    const int64_t grid = tiles * hkv;
    a.head_major = 2.0 * hkv * (double)L * d * 2 > 256.0 * (1 << 20);
    if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (d == 128) hipLaunchKernelGGL((attn_mfma_kernel<0, 128>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else if (d == 64) hipLaunchKernelGGL((attn_mfma_kernel<0, 64>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

static int partial_splits_wanted(int32_t rows, int32_t hq, int32_t hkv, int* n_row_tiles) {
    const int G = hq / hkv;
    const int rw = kQPB / G;
    const int nrt = (rows + rw - 1) / rw;
    const int64_t base = (int64_t)hkv * nrt;
    *n_row_tiles = nrt;
    // One workgroup of eight waves fills a compute unit; aim for one per CU (256).
    return (int)(base >= 256 ? 1 : 256 / base);
}

int partial_mfma_plan(PartPlan& plan, int32_t rows, int32_t hq, int32_t hkv) {
    int nrt;
    const int want = partial_splits_wanted(rows, hq, hkv, &nrt);
    int64_t total_tiles = 0;
    for (int i = 0; i < plan.n_parts; ++i) total_tiles += (plan.n_kv[i] + kBN - 1) / kBN;
    int64_t tps = (total_tiles + want - 1) / want;
    if (tps < 8) tps = 8;   // enough tiles per split to amortise the partial's write and merge
    plan.split_len = tps * kBN;
    plan.split_prefix[0] = 0;
    for (int i = 0; i < plan.n_parts; ++i) {
        int64_t ns = (plan.n_kv[i] + plan.split_len - 1) / plan.split_len;
        if (ns < 1) ns = 1;   // an empty partition still reports its (empty) partial
        plan.split_prefix[i + 1] = plan.split_prefix[i] + (int32_t)ns;
    }
    return nrt;
}

int64_t partial_mfma_max_splits(int32_t rows, int32_t hq, int32_t hkv, int n_parts) {
    int nrt;
    // ceil(tiles_i / tps) <= tiles_i / tps + 1 and sum(tiles_i) / tps <= want.
    return (int64_t)partial_splits_wanted(rows, hq, hkv, &nrt) + n_parts;
}

hipError_t launch_partial_mfma(const uint16_t* q, int32_t rows, int hq, int hkv, int d, float scale,
                               const PartPlan& plan, int n_row_tiles, float* a_out, float* m_out,
                               float* l_out, hipStream_t stream) {
    AttnMfmaArgs a = {};
    a.q = q;
    a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
    a.rows_per_wg = kQPB / a.G;
    a.q_rows = rows;
    a.rows = rows;
    a.scale_log2 = scale * kLog2e;
    a.a_out = a_out; a.m_out = m_out; a.l_out = l_out;
    a.n_row_tiles = n_row_tiles;
    a.plan = plan;
    const int64_t grid = (int64_t)hkv * n_row_tiles * plan.split_prefix[plan.n_parts];
    if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (d == 128) hipLaunchKernelGGL((attn_mfma_kernel<1, 128>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else if (d == 64) hipLaunchKernelGGL((attn_mfma_kernel<1, 64>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace star
