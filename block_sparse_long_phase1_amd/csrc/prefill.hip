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
// Work unit: one workgroup = 4 waves = 256 queries that share one kv head
// (G q heads x 256/G consecutive rows), so each K/V tile staged in LDS feeds
// the whole GQA group.  Each wave owns 64 queries (two 32-query column
// blocks).  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: every lane then owns one query column, so the
// softmax row statistics need no cross-lane reduction beyond one exchange
// between lane l and l^32.  The probabilities P^T come out of the score
// accumulators already in the B-operand layout of the second product
// O^T += V^T P^T; V is transposed once per tile while it is written to LDS.
// K/V tiles of 32 keys are double-buffered in LDS (global loads for tile j+1
// are in flight while tile j is multiplied).  Softmax runs in the exp2
// domain with a lazily updated reference max: the accumulators are only
// rescaled when a row's max grows by more than 2^8, which keeps every
// probability below 256 and is exact after the final normalisation.
#include "common.h"
#include "internal.h"

namespace star {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 32;          // keys per tile
constexpr int kD = 128;          // head dim of this kernel
constexpr int kQPB = 256;        // queries per workgroup
constexpr int kKPitch = kD + 8;  // bf16 per K row in LDS (272 B: conflict-free 16 B reads)
constexpr int kVPitch = kBN + 4; // bf16 per V^T row in LDS (72 B: conflict-free 8 B reads)
constexpr int kKTile = kBN * kKPitch;
constexpr int kVTile = kD * kVPitch;
constexpr int kStage = kKTile + kVTile;       // bf16 elements per pipeline stage
constexpr float kRescaleThreshold = 8.0f;     // log2 units

struct TileSrc {
    u32x4 k[2];   // 2 x 16 B of K rows
    u32x4 v[2];   // 2 consecutive keys x 8 d of V
};

// Issue the global loads of one 32-key tile.  Keys at or past `kmax` are
// clamped to kmax-1 (always a valid row); their scores are masked later.
__device__ __forceinline__ void load_tile(TileSrc& t, const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, int64_t key0,
                                          int64_t kmax, int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int c = tid + kThreads * j;
        int row = c >> 4, col8 = c & 15;
        int64_t key = key0 + row;
        key = key < kmax ? key : kmax - 1;
        t.k[j] = *reinterpret_cast<const u32x4*>(kb + key * kD + col8 * 8);
    }
    int kp2 = tid & 15, oct = tid >> 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int64_t key = key0 + kp2 * 2 + j;
        key = key < kmax ? key : kmax - 1;
        t.v[j] = *reinterpret_cast<const u32x4*>(vb + key * kD + oct * 8);
    }
}

// Write a loaded tile into one LDS stage: K row-major, V transposed (V^T[d][key]).
__device__ __forceinline__ void store_tile(const TileSrc& t, uint16_t* __restrict__ stage, int tid) {
    uint16_t* ks = stage;
    uint16_t* vs = stage + kKTile;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int c = tid + kThreads * j;
        int row = c >> 4, col8 = c & 15;
        *reinterpret_cast<u32x4*>(ks + row * kKPitch + col8 * 8) = t.k[j];
    }
    int kp2 = tid & 15, oct = tid >> 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // word w of each key row holds d = 8*oct + 2w, +1
        int d = oct * 8 + 2 * w;
        *reinterpret_cast<uint32_t*>(vs + d * kVPitch + kp2 * 2) = pack_lo16(t.v[0][w], t.v[1][w]);
        *reinterpret_cast<uint32_t*>(vs + (d + 1) * kVPitch + kp2 * 2) = pack_hi16(t.v[0][w], t.v[1][w]);
    }
}

// Description of the keys one workgroup visits: segment A (tiles [0, nta)),
// then segment B.  Positions are token indices into the kv head's rows.
struct KeyPlan {
    int64_t a_lo, a_hi;   // segment A: no causal mask, keys >= a_hi masked
    int64_t b_lo, b_hi;   // segment B: keys >= b_hi masked; causal if `causal`
    int nta, ntb;
    bool causal;          // key (token index) visible iff key <= row_key_limit(row)
    int64_t diag;         // visible iff key <= row + diag  (row = query row index)
    int64_t kmax;         // tokens available in memory for this kv head
};

}  // namespace

template <int MODE>  // 0 = Phase 1 encode, 1 = Phase 2 partial
__global__ void __launch_bounds__(kThreads, 1)
attn_mfma_kernel(const AttnMfmaArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;   // which 4-row group of the 32x32 layout this lane holds
    const int col = lane & 31;    // query column inside a 32-query block

    // ---------------------------------------------------------------- work item
    const int g = blockIdx.x % p.hkv;
    int64_t rank = blockIdx.x / p.hkv;
    int64_t row0, row_end;        // query rows [row0, row_end) valid for this workgroup
    KeyPlan kp;
    int split = 0;
    if (MODE == 0) {
        // Heaviest tiles first: last row tiles of blocks >= 1, then block 0.
        int64_t blk, rt;
        if (rank < p.tiles_ge1) {
            int64_t hi_levels = (p.nt_full - p.nt_last) * (p.n_blocks - 2);
            if (rank < hi_levels) {
                rt = p.nt_full - 1 - rank / (p.n_blocks - 2);
                blk = 1 + rank % (p.n_blocks - 2);
            } else {
                int64_t r = rank - hi_levels;
                rt = p.nt_last - 1 - r / (p.n_blocks - 1);
                blk = 1 + r % (p.n_blocks - 1);
            }
        } else {
            blk = 0;
            rt = p.nt0 - 1 - (rank - p.tiles_ge1);
        }
        int64_t bstart = blk * p.block;
        int64_t bend = bstart + p.block < p.L ? bstart + p.block : p.L;
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
        int64_t rt = rank % p.n_row_tiles;
        split = (int)(rank / p.n_row_tiles);
        row0 = rt * p.rows_per_wg;
        row_end = row0 + p.rows_per_wg < p.rows ? row0 + p.rows_per_wg : p.rows;
        int64_t lo = (int64_t)split * p.split_len;
        int64_t hi = lo + p.split_len < p.n_kv ? lo + p.split_len : p.n_kv;
        kp.causal = p.causal_offset >= 0;
        kp.diag = p.causal_offset;
        if (kp.causal) {
            int64_t lim = p.causal_offset + row_end;  // keys >= lim are invisible to every row here
            hi = hi < lim ? hi : lim;
        }
        kp.a_lo = kp.a_hi = 0;
        kp.b_lo = lo;
        kp.b_hi = hi > lo ? hi : lo;
        kp.kmax = p.n_kv;
    }
    kp.nta = (int)((kp.a_hi - kp.a_lo + kBN - 1) / kBN);
    kp.ntb = (int)((kp.b_hi - kp.b_lo + kBN - 1) / kBN);
    const int nt = kp.nta + kp.ntb;

    // ---------------------------------------------------------------- this lane's queries
    // Query index qi in [0, 256): head g*G + qi / rows_per_wg, row row0 + qi % rows_per_wg.
    int64_t qrow[2];
    int qhead[2];
    bool qvalid[2];
    bf16x8 qb[2][8];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        int qi = wave * 64 + cb * 32 + col;
        qhead[cb] = g * p.G + qi / p.rows_per_wg;
        qrow[cb] = row0 + qi % p.rows_per_wg;
        qvalid[cb] = (qi / p.rows_per_wg) < p.G && qrow[cb] < row_end;
        const uint16_t* qp = p.q + ((int64_t)qhead[cb] * p.q_rows + (qvalid[cb] ? qrow[cb] : 0)) * kD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (qvalid[cb]) w = *reinterpret_cast<const u32x4*>(qp + s * 16 + half * 8);
            qb[cb][s] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][db][r] = 0.f;
    float mref[2] = {kNoMax, kNoMax};   // reference max (log2 units) used in the exponent
    float mtrue[2] = {kNoMax, kNoMax};  // largest score seen (log2 units)
    float lsum[2] = {0.f, 0.f};         // this lane's half of the row sums
    const float sl2 = p.scale_log2;

    const uint16_t* kbase = p.k + (int64_t)g * p.kv_head_stride;
    const uint16_t* vbase = p.v + (int64_t)g * p.kv_head_stride;

    auto tile_key0 = [&](int j) -> int64_t {
        return j < kp.nta ? kp.a_lo + (int64_t)j * kBN : kp.b_lo + (int64_t)(j - kp.nta) * kBN;
    };

    if (nt > 0) {
        TileSrc src;
        load_tile(src, kbase, vbase, tile_key0(0), kp.kmax, tid);
        store_tile(src, smem, tid);
        __syncthreads();

        for (int j = 0; j < nt; ++j) {
            const uint16_t* ks = smem + (j & 1) * kStage;
            const uint16_t* vs = ks + kKTile;
            const bool more = j + 1 < nt;
            if (more) load_tile(src, kbase, vbase, tile_key0(j + 1), kp.kmax, tid);

            // ---- S^T = K Q^T  (rows: the tile's 32 keys, cols: 2 x 32 queries)
            f32x16 s[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[cb][r] = 0.f;
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                u32x4 a = *reinterpret_cast<const u32x4*>(ks + col * kKPitch + st * 16 + half * 8);
                bf16x8 ab = __builtin_bit_cast(bf16x8, a);
                s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, qb[0][st], s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, qb[1][st], s[1], 0, 0, 0);
            }

            // ---- masks (only on tiles that can hold an invisible key)
            const int64_t key0 = tile_key0(j);
            const bool in_a = j < kp.nta;
            const int64_t seg_hi = in_a ? kp.a_hi : kp.b_hi;
            bool need_mask = key0 + kBN > seg_hi;
            if (!in_a && kp.causal) need_mask |= key0 + kBN - 1 > row0 + kp.diag;
            if (need_mask) {
                // Offsets relative to key0, clamped into int range (a tile spans 64 keys).
                const int64_t lim64 = seg_hi - key0;
                const int lim = lim64 > kBN ? kBN : (int)lim64;
                int rlim[2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    int64_t r64 = (in_a || !kp.causal) ? (int64_t)kBN : qrow[cb] + kp.diag - key0;
                    rlim[cb] = r64 > kBN ? kBN : (r64 < -1 ? -1 : (int)r64);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rel = (r >> 2) * 8 + half * 4 + (r & 3);
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        if (rel >= lim || rel > rlim[cb]) s[cb][r] = -INFINITY;
                }
            }

            // ---- online softmax (exp2 domain, lazy reference max)
            bf16x8 pb[2][2];  // [cb][u]: B operands for the two 16-key steps
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                float mx = s[cb][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[cb][r]);
                mx = half_pair_max(mx);
                const float mxl = mx * sl2;
                mtrue[cb] = fmaxf(mtrue[cb], mxl);
                if (__builtin_amdgcn_ballot_w64(mxl > mref[cb] + kRescaleThreshold)) {
                    float nref = fmaxf(mref[cb], mxl);
                    float alpha = fast_exp2(mref[cb] - nref);
                    mref[cb] = nref;
                    lsum[cb] *= alpha;
#pragma unroll
                    for (int db = 0; db < 4; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[cb][db][r] *= alpha;
                }
                const float negm = -mref[cb];
                float ls = 0.f;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float e[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        e[i] = fast_exp2(fmaf(s[cb][8 * u + i], sl2, negm));
                        ls += e[i];
                    }
                    u32x4 w;
                    w[0] = pack_bf16x2(e[0], e[1]);
                    w[1] = pack_bf16x2(e[2], e[3]);
                    w[2] = pack_bf16x2(e[4], e[5]);
                    w[3] = pack_bf16x2(e[6], e[7]);
                    pb[cb][u] = __builtin_bit_cast(bf16x8, w);
                }
                lsum[cb] += ls;
            }

            // ---- O^T += V^T P^T  (16-key steps; slot i of lane half h is key
            //      16u + 8*(i/4) + 4h + i%4 of the tile, matching the S^T layout)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const uint16_t* vp = vs + (db * 32 + col) * kVPitch + u * 16 + half * 4;
                    u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
                    u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
                    u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                    bf16x8 ab = __builtin_bit_cast(bf16x8, a);
                    acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, pb[0][u], acc[0][db], 0, 0, 0);
                    acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, pb[1][u], acc[1][db], 0, 0, 0);
                }

            if (more) store_tile(src, smem + ((j + 1) & 1) * kStage, tid);
            __syncthreads();
        }
    }

    // ---------------------------------------------------------------- epilogue
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        float l = half_pair_sum(lsum[cb]);
        const bool empty = !(l > 0.f);
        const float inv = empty ? 0.f : 1.0f / l;
        if (!qvalid[cb]) continue;
        const int64_t hr = (int64_t)qhead[cb] * p.q_rows + qrow[cb];
        if (MODE == 0) {
            uint16_t* op = p.o + hr * kD;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    int d0 = db * 32 + gq * 8 + half * 4;
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[cb][db][gq * 4 + 0] * inv, acc[cb][db][gq * 4 + 1] * inv);
                    w[1] = pack_bf16x2(acc[cb][db][gq * 4 + 2] * inv, acc[cb][db][gq * 4 + 3] * inv);
                    *reinterpret_cast<u32x2*>(op + d0) = w;
                }
            if (p.lse && half == 0) p.lse[hr] = (mref[cb] + __builtin_amdgcn_logf(l)) * kLn2;
        } else {
            const int64_t out_row = (int64_t)split * p.hq * p.q_rows + hr;
            float* ap = p.a_out + out_row * kD;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    int d0 = db * 32 + gq * 8 + half * 4;
                    f32x4 w = {acc[cb][db][gq * 4 + 0] * inv, acc[cb][db][gq * 4 + 1] * inv,
                               acc[cb][db][gq * 4 + 2] * inv, acc[cb][db][gq * 4 + 3] * inv};
                    *reinterpret_cast<f32x4*>(ap + d0) = w;
                }
            if (half == 0) {
                // Report (m, l) against the true max so that m is the largest scaled score.
                p.m_out[out_row] = empty ? -INFINITY : mtrue[cb] * kLn2;
                p.l_out[out_row] = empty ? 0.f : l * fast_exp2(mref[cb] - mtrue[cb]);
            }
        }
    }
}

// ------------------------------------------------------------------------- launchers

bool attn_mfma_supported(int d, int hq, int hkv) {
    if (d != kD || hkv < 1 || hq % hkv) return false;
    int G = hq / hkv;
    return G >= 1 && G <= kQPB && (kQPB % G) == 0;
}

hipError_t launch_phase1_mfma(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* o, float* lse, int64_t L, int64_t block, int64_t anchor,
                              int hq, int hkv, float scale, hipStream_t stream) {
    AttnMfmaArgs a = {};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.L = L; a.block = block; a.anchor = anchor;
    a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
    a.rows_per_wg = kQPB / a.G;
    a.q_rows = L;
    a.kv_head_stride = L * kD;
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
    if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_mfma_kernel<0>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

void partial_mfma_plan(int32_t rows, int64_t n_kv, int32_t hq, int32_t hkv,
                       int* n_row_tiles, int* n_splits, int64_t* split_len) {
    const int G = hq / hkv;
    const int rw = kQPB / G;
    int nrt = (rows + rw - 1) / rw;
    int64_t tiles = (n_kv + kBN - 1) / kBN;
    int64_t base = (int64_t)hkv * nrt;
    // Aim for at least two workgroups per compute unit (256 CUs).
    int64_t want = (512 + base - 1) / base;
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    int64_t tiles_per_split = (tiles + want - 1) / want;
    if (tiles_per_split < 1) tiles_per_split = 1;
    int64_t ns = (tiles + tiles_per_split - 1) / tiles_per_split;
    if (ns < 1) ns = 1;
    *n_row_tiles = nrt;
    *n_splits = (int)ns;
    *split_len = tiles_per_split * kBN;
}

hipError_t launch_partial_mfma(const uint16_t* q, int32_t rows, const uint16_t* k, const uint16_t* v,
                               int64_t kv_head_stride, int64_t n_kv, int64_t causal_offset,
                               int hq, int hkv, float scale, float* a_out, float* m_out, float* l_out,
                               int n_splits, int64_t split_len, int n_row_tiles, hipStream_t stream) {
    AttnMfmaArgs a = {};
    a.q = q; a.k = k; a.v = v;
    a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
    a.rows_per_wg = kQPB / a.G;
    a.q_rows = rows;
    a.rows = rows;
    a.kv_head_stride = kv_head_stride;
    a.n_kv = n_kv;
    a.causal_offset = causal_offset;
    a.scale_log2 = scale * kLog2e;
    a.a_out = a_out; a.m_out = m_out; a.l_out = l_out;
    a.n_row_tiles = n_row_tiles;
    a.split_len = split_len;
    const int64_t grid = (int64_t)hkv * n_row_tiles * n_splits;
    if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_mfma_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace star
