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
// Tiles of 64 keys go through a ring of four LDS stages, copied there by direct
// global-to-LDS loads, which take no registers and no LDS store instructions;
// the copy of tile j+3 is in flight while tile j is multiplied.  (Partitions of
// E4M3 codes instead load the codes into registers three tiles ahead and write
// them, widened to bf16, into the same stage layout.)  Each tile runs as two
// 32-key halves so that one half's exponentials issue between the other half's
// MFMAs.  Softmax runs in the exp2 domain with a lazily updated reference max:
// Phase-2 partials rescale the accumulators only when a row's max grows by more
// than 2^8; Phase 1 keeps a half-tile when each row's probability sum over it is
// at most 2^20 and otherwise redoes it against a moved reference.  Either way
// the result is exact after the final normalisation.
#include "common.h"
#include "internal.h"

namespace star {

namespace {

constexpr int kThreads = 512;
constexpr int kBN = kAttnKeysPerTile;        // keys per tile (64)
constexpr int kQPB = kAttnQueriesPerGroup;   // queries per workgroup (256)
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

// One 16-byte-per-lane global-to-LDS copy (global_load_lds_dwordx4), issued from asm so that
// the compiler's wait insertion does not track it: with the builtin it cannot tell the LDS
// stages apart and waits for every copy in flight before each barrier.  Copies are waited
// for explicitly (s_waitcnt vmcnt before the barrier that publishes a stage).  LDS reads
// still complete in order among themselves, so the compiler's partial lgkmcnt waits stay
// correct.  The s_nop is the wait state an M0 write needs before a load that writes LDS.
// gbase and lds_addr are wave-uniform; voff is this lane's byte offset.
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 : : "v"(voff), "s"(gbase), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

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
        lds_copy16(src, off, lds_addr_of(dst + b * blk_bytes));
    }
}

// s_waitcnt operand that waits until at most two tile copies (this wave's share of each:
// Geo<D>::kBlocks / 4 loads) are outstanding; expcnt and lgkmcnt at their "no wait" maxima.
template <int D>
constexpr int wait_two_copies() {
    constexpr int n = 2 * (Geo<D>::kBlocks / 4);
    static_assert(n < 64, "vmcnt field");
    return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
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

// MODE 0 = Phase 1 encode, 1 = Phase 2 partial; D = head dim (64 or 128).  F8 (Phase-2
// partials only): partitions [0, plan.n_f8) hold E4M3 codes with per-kv-head scales.
template <int MODE, int D, bool F8 = false>
__global__ void __launch_bounds__(kThreads, 2)
attn_mfma_kernel(const AttnMfmaArgs p) {
    using T = Geo<D>;
    constexpr int kD = D;
    __shared__ __attribute__((aligned(16))) char smem0[T::kStageBytes];
    __shared__ __attribute__((aligned(16))) char smem1[T::kStageBytes];
    __shared__ __attribute__((aligned(16))) char smem2[T::kStageBytes];
    __shared__ __attribute__((aligned(16))) char smem3[T::kStageBytes];

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
    bool f8 = false;              // this work item's partition holds E4M3 codes (uniform)
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
        kptr = static_cast<const uint16_t*>(pl.k[part]);
        vptr = static_cast<const uint16_t*>(pl.v[part]);
        f8 = F8 && part < pl.n_f8;
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
    // score scale (log2 units); an E4M3 partition folds its kv head's K scale in
    const float sl2 = (F8 && f8) ? p.scale_log2 * p.plan.k_scale[g] : p.scale_log2;

    const uint16_t* kbase = kptr + (int64_t)g * hstride;
    const uint16_t* vbase = vptr + (int64_t)g * hstride;
    const int kmax = (int)kp.kmax;

    // E4M3 partitions: each thread loads D/64 16-byte pieces of a tile's codes (K pieces
    // first, then V) three tiles ahead into registers, and widens them exactly to bf16 in the
    // stage layout the tile copies produce, before the barrier that publishes that stage.
    constexpr int kF8PiecesPerTensor = kBN * D / 16;          // 16-byte pieces of codes per K or V tile
    constexpr int kF8Pieces = F8 ? 2 * kF8PiecesPerTensor / kThreads : 1;
    u32x4 f8buf[kF8Pieces];
    // A piece's row and column follow from the thread index.  They are rebuilt at each use from
    // an opaque copy of it, so that the compiler does not keep them live across the tile loop
    // (at d = 128 the loop has no registers to spare: kept, they were spilled and reloaded
    // every tile); unsigned and masked, the rebuild is a few shifts and masks.
    auto f8_piece = [&](int pc, int& row, int& col0, bool& is_v) __attribute__((always_inline)) {
        unsigned ut = threadIdx.x;
        asm volatile("" : "+v"(ut));
        ut &= kThreads - 1;
        const unsigned pi = ut + pc * kThreads;
        is_v = pi >= (unsigned)kF8PiecesPerTensor;
        const unsigned idx = is_v ? pi - kF8PiecesPerTensor : pi;
        row = (int)(idx / (D / 16));
        col0 = (int)(idx % (D / 16)) * 16;
    };
    auto f8_load = [&](int key0) __attribute__((always_inline)) {
        const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(kptr) + (int64_t)g * hstride;
        const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(vptr) + (int64_t)g * hstride;
#pragma unroll
        for (int pc = 0; pc < kF8Pieces; ++pc) {
            int row, col0;
            bool is_v;
            f8_piece(pc, row, col0, is_v);
            const int key = min(key0 + row, kmax - 1);
            f8buf[pc] = *reinterpret_cast<const u32x4*>((is_v ? vb8 : kb8) + (int64_t)key * D + col0);
        }
    };
    auto f8_store = [&](char* stage) __attribute__((always_inline)) {
#pragma unroll
        for (int pc = 0; pc < kF8Pieces; ++pc) {
            int row, col0;
            bool is_v;
            f8_piece(pc, row, col0, is_v);
            char* dst = stage + (is_v ? T::kKTileBytes + (row % T::kBlocks) * kVBlock
                                      : (row % T::kBlocks) * kKBlock) +
                        (row / T::kBlocks) * T::kRowBytes + col0 * 2;
            *reinterpret_cast<u32x4*>(dst) = e4m3x8_to_bf16x8(f8buf[pc][0], f8buf[pc][1]);
            *reinterpret_cast<u32x4*>(dst + 16) = e4m3x8_to_bf16x8(f8buf[pc][2], f8buf[pc][3]);
        }
    };
    const int a_lo = (int)kp.a_lo, b_lo = (int)kp.b_lo;
    auto tile_key0 = [&](int j) -> int { return j < kp.nta ? a_lo + j * kBN : b_lo + (j - kp.nta) * kBN; };

    f32x16 s[kKB];   // S^T of the current tile, one 32-key block per entry

    // transposing-read addressing inside a 16-key step (see the P.V comment below)
    const int trow = 4 * half + ((lane & 15) >> 2);
    const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);

    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    // One 64-key tile as two 32-key halves: half 0's exponentials issue between half 1's
    // score MFMAs, and half 1's between half 0's P.V MFMAs, so that no stretch of the
    // softmax runs without MFMAs of the same wave in flight.
    auto step = [&](int j, const char* cur, char* nxt) {
        // Copy tile j + 3 into the stage read during step j - 1 (every wave is past it).  The
        // last three steps copy the last tile again, into stages nobody reads, so that exactly
        // two copies are in flight behind every wait below.
        if (F8 && f8)
            f8_load(tile_key0(min(j + 3, nt - 1)));
        else
            dma_tile<D>(nxt, kbase, vbase, tile_key0(min(j + 3, nt - 1)), kmax, uwave, lane);
        // Masking: does tile j hold a key that some row may not see (uniform)?
        const int key0 = tile_key0(j);
        const bool in_a = j < kp.nta;
        const int seg_hi = in_a ? (int)kp.a_hi : (int)kp.b_hi;
        bool need = key0 + kBN > seg_hi;
        if (!in_a && kp.causal) need |= (int64_t)key0 + kBN - 1 > row0 + kp.diag;
        const int lim = min(seg_hi - key0, kBN);
        int rlim = kBN;
        if (!in_a && kp.causal) {
            const int64_t r64 = qrow + kp.diag - key0;
            rlim = r64 > kBN ? kBN : (r64 < -1 ? -1 : (int)r64);
        }
        // Phase-2 partials take every tile's max (they report the true max); Phase 1 takes it
        // on its first tile only and otherwise checks the sum bound after the exponentials.
        const bool take_max = MODE == 1 || j == 0;

        const char* vs = cur + T::kKTileBytes;
        // K operand: row kb*32 + col, chunk 2*st + half: row col is in block col % NB at
        // position col / NB; kb adds 32 rows, i.e. 32/NB positions of 2D bytes (512 B).
        const char* kop = cur + (col % T::kBlocks) * kKBlock + (col / T::kBlocks) * T::kRowBytes + half * 16;
        // V operand rows 16u + trow (+8): block trow (+8), row u inside it.
        const char* vp = vs + trow * kVBlock + tcol * 2;   // trow < 8 <= NB: block trow, position 0

        auto read_k = [&](int kb, u32x4 (&ka)[T::kST]) __attribute__((always_inline)) {
#pragma unroll
            for (int st = 0; st < T::kST; ++st) ka[st] = *reinterpret_cast<const u32x4*>(kop + kb * 512 + st * 32);
        };
        // V^T operands of 16-key steps 2kb and 2kb+1 by transposing reads of the row-major V
        // tile.  Step u: slot i of lane half h is key 16u + 8*(i/4) + 4h + i%4, the S^T
        // layout.  In a 16-lane group, source lane s points at key (s/4) of a four-key set
        // and at columns 4*(s%4) .. +3 of the group's 16-wide head-dim slice; result lane i
        // holds column i of that slice for the four keys.
        auto read_v = [&](int kb, u32x4 (&va)[2][T::kDB]) __attribute__((always_inline)) {
#pragma unroll
            for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) {
                    // row 16u + trow: 16 rows are 16/NB positions of 2D bytes (256 B) further on
                    const int u = 2 * kb + uu;
                    const u32x2v a0 = lds_read_tr(vp + u * 256 + db * 64);
                    const u32x2v a1 = lds_read_tr(vp + T::kPlus8 + u * 256 + db * 64);
                    va[uu][db] = u32x4{a0[0], a0[1], a1[0], a1[1]};
                }
        };
        auto score_mfma = [&](int kb, int st, const u32x4 (&ka)[T::kST]) __attribute__((always_inline)) {
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[st]), qb[st], s[kb], 0, 0, 0);
        };
        auto score_blk = [&](int kb) __attribute__((always_inline)) {
            u32x4 ka[T::kST];
            read_k(kb, ka);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int st = 0; st < T::kST; ++st) score_mfma(kb, st, ka);
        };
        auto mask_blk = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rel = kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                if (rel >= lim || rel > rlim) s[kb][r] = -INFINITY;
            }
        };
        // Move the reference (and rescale) if this half's max grew past it by 2^8.
        auto max_blk = [&](int kb) __attribute__((always_inline)) {
            float mx = s[kb][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
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
                // Half 0's probabilities are taken before half 1's max and enter the
                // accumulators only afterwards: they move to the new reference too (once
                // they are in the accumulators this is a harmless write to dead values).
                if (kb == 1) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[0][r] *= alpha;
                }
            }
        };
        auto exp_one = [&](int kb, int r, float negm, float& ls) __attribute__((always_inline)) {
            s[kb][r] = fast_exp2(fmaf(s[kb][r], sl2, negm));
            ls += s[kb][r];
        };
        // Phase 1 keeps a half when every row's sum of its probabilities is at most 2^20: no
        // probability overflowed and the accumulators stay far from the fp32 range, so the
        // reference need not move.  Else (scores far above the reference) the half's scores
        // are recomputed from the K tile, the reference moves to their max and the
        // probabilities are redone.  This replaces a max over every tile's scores.
        auto check = [&](int kb, float ls) __attribute__((always_inline)) -> float {
            if (MODE == 0 && __builtin_amdgcn_ballot_w64(!(ls <= kSumBound))) {
                score_blk(kb);
                if (need) mask_blk(kb);
                max_blk(kb);
                const float negm = -mref;
                ls = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) exp_one(kb, r, negm, ls);
            }
            return ls;
        };
        auto pack = [&](int kb, int uu) __attribute__((always_inline)) -> bf16x8 {
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(s[kb][8 * uu + 2 * i], s[kb][8 * uu + 2 * i + 1]);
            return __builtin_bit_cast(bf16x8, w);
        };
        constexpr int kEPM = 16 / T::kST;         // half-0 exponentials per half-1 score MFMA
        constexpr int kEPV = 16 / (2 * T::kDB);   // half-1 exponentials per half-0 P.V MFMA

        // ---- half 0 scores; half 1's K operands read while they run
        u32x4 ka[T::kST];
        {
            u32x4 k0[T::kST];
            read_k(0, k0);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[0][r] = 0.f;
#pragma unroll
            for (int st = 0; st < T::kST; ++st) score_mfma(0, st, k0);
            read_k(1, ka);
            __builtin_amdgcn_sched_group_barrier(0x100, T::kST, 0);
#pragma unroll
            for (int st = 0; st < T::kST; ++st) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        if (need) mask_blk(0);
        if (take_max) max_blk(0);
        // ---- half 1 scores || half 0 exponentials and V operands
        float ls0 = 0.f;
        u32x4 va[2][T::kDB];
        {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[1][r] = 0.f;
            const float negm = -mref;
#pragma unroll
            for (int st = 0; st < T::kST; ++st) {
                score_mfma(1, st, ka);
#pragma unroll
                for (int e = 0; e < kEPM; ++e) exp_one(0, st * kEPM + e, negm, ls0);
            }
            read_v(0, va);
#pragma unroll
            for (int st = 0; st < T::kST; ++st) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 4 * T::kDB / T::kST, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3 * kEPM, 0);
            }
        }
        lsum += check(0, ls0);
        if (need) mask_blk(1);
        if (take_max) max_blk(1);
        // ---- half 0 P.V || half 1 exponentials and V operands
        float ls1 = 0.f;
        u32x4 vb[2][T::kDB];
        {
            const bf16x8 p0 = pack(0, 0), p1 = pack(0, 1);
            const float negm = -mref;
#pragma unroll
            for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) {
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[uu][db]),
                                                                     uu ? p1 : p0, acc[db], 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < kEPV; ++e) exp_one(1, (uu * T::kDB + db) * kEPV + e, negm, ls1);
                }
            read_v(1, vb);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
            for (int m = 0; m < 2 * T::kDB; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3 * kEPV, 0);
            }
        }
        lsum += check(1, ls1);
        // ---- half 1 P.V
        {
            const bf16x8 p0 = pack(1, 0), p1 = pack(1, 1);
#pragma unroll
            for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                for (int db = 0; db < T::kDB; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vb[uu][db]),
                                                                     uu ? p1 : p0, acc[db], 0, 0, 0);
        }
        if (F8 && f8) f8_store(nxt);   // tile j + 3, into the stage every wave left at the last barrier
        // This wave's copies of tile j + 1 have landed (those of tiles j + 2 and j + 3 may still
        // be in flight); after the barrier every wave's have, and every wave is done reading
        // `cur`.
        __builtin_amdgcn_s_waitcnt(wait_two_copies<D>());
        __syncthreads();
    };

    if (nt > 0) {
        // The query loads have landed: from here on the only loads in flight are tile copies,
        // which the waits count.  Tiles 0-2 go into stages 0-2; tile j lives in stage j % 4.
        __builtin_amdgcn_s_waitcnt(0);
        if (F8 && f8) {
            f8_load(tile_key0(0));
            f8_store(smem0);
            f8_load(tile_key0(min(1, nt - 1)));
            f8_store(smem1);
            f8_load(tile_key0(min(2, nt - 1)));
            f8_store(smem2);
        } else {
            dma_tile<D>(smem0, kbase, vbase, tile_key0(0), kmax, uwave, lane);
            dma_tile<D>(smem1, kbase, vbase, tile_key0(min(1, nt - 1)), kmax, uwave, lane);
            dma_tile<D>(smem2, kbase, vbase, tile_key0(min(2, nt - 1)), kmax, uwave, lane);
        }
        __builtin_amdgcn_s_waitcnt(wait_two_copies<D>());
        __syncthreads();
        int j = 0;
        for (; j + 3 < nt; j += 4) {
            step(j, smem0, smem3);
            step(j + 1, smem1, smem0);
            step(j + 2, smem2, smem1);
            step(j + 3, smem3, smem2);
        }
        if (j < nt) step(j, smem0, smem3);
        if (j + 1 < nt) step(j + 1, smem1, smem0);
        if (j + 2 < nt) step(j + 2, smem2, smem1);
        __builtin_amdgcn_s_waitcnt(0);   // the trailing copies
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
        // an E4M3 partition's values carry its kv head's V scale
        const float inv_a = (F8 && f8) ? inv * p.plan.v_scale[g] : inv;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = db * 32 + gq * 8 + half * 4;
                const f32x4 w = {acc[db][gq * 4 + 0] * inv_a, acc[db][gq * 4 + 1] * inv_a,
                                 acc[db][gq * 4 + 2] * inv_a, acc[db][gq * 4 + 3] * inv_a};
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
    const bool f8 = plan.n_f8 > 0;
    if (f8 && (!plan.k_scale || !plan.v_scale)) return hipErrorInvalidValue;
    if (d == 128) {
        if (f8) hipLaunchKernelGGL((attn_mfma_kernel<1, 128, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((attn_mfma_kernel<1, 128>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    } else if (d == 64) {
        if (f8) hipLaunchKernelGGL((attn_mfma_kernel<1, 64, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((attn_mfma_kernel<1, 64>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace star
