// Host-side work planning and argument checks (see host_plan.h).
#include "host_plan.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace star {

namespace {
// The decode kernel's four waves walk 32-key tiles: chunks are a multiple of one pass.
constexpr int64_t kDecodeChunkQuantum = 128;

// Query-row tiles of a partial launch and the key splits wanted per partition set.
int partial_splits_wanted(int32_t rows, int32_t hq, int32_t hkv, int* n_row_tiles) {
    const int G = hq / hkv;
    const int rw = kAttnQueriesPerGroup / G;
    const int nrt = (rows + rw - 1) / rw;
    const int64_t base = (int64_t)hkv * nrt;
    *n_row_tiles = nrt;
    // One workgroup of eight waves fills a compute unit; aim for one per CU (256).
    return (int)(base >= 256 ? 1 : 256 / base);
}

}  // namespace

bool attn_mfma_supported(int d, int hq, int hkv) {
    if ((d != 64 && d != 128) || hkv < 1 || hq % hkv) return false;
    const int G = hq / hkv;
    return G >= 1 && G <= kAttnQueriesPerGroup && (kAttnQueriesPerGroup % G) == 0;
}

int64_t attn_mfma_max_tokens(int d) { return ((int64_t)1 << 31) / d; }

int partial_mfma_plan(PartPlan& plan, int32_t rows, int32_t hq, int32_t hkv) {
    int nrt;
    const int want = partial_splits_wanted(rows, hq, hkv, &nrt);
    int64_t total_tiles = 0;
    for (int i = 0; i < plan.n_parts; ++i) total_tiles += (plan.n_kv[i] + kAttnKeysPerTile - 1) / kAttnKeysPerTile;
    int64_t tps = (total_tiles + want - 1) / want;
    if (tps < 8) tps = 8;   // enough tiles per split to amortise the partial's write and merge
    plan.split_len = tps * kAttnKeysPerTile;
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

bool decode_bf16_supported(int d, int hq, int hkv) {
    if ((d != 64 && d != 128) || hkv < 1 || hq % hkv) return false;
    const int G = hq / hkv;
    return G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
}

int64_t decode_chunk_len(const int64_t* shard_bounds, int n_shards, int32_t hkv) {
    // About one context chunk per compute unit (256 CUs), all in one round: each kv head gets
    // up to 272/hkv - 1 context chunks, spread over its shards by length, plus
    // its query-host chunk(s).  Chunks are a multiple of the 4 x 32 keys one pass covers.
    const int64_t L = shard_bounds[n_shards] - shard_bounds[0];
    int64_t budget = 272 / hkv - 1;
    if (budget < n_shards) budget = n_shards;
    int64_t ch = kDecodeChunkQuantum;
    for (int r = 0; r < n_shards; ++r) {
        const int64_t len = shard_bounds[r + 1] - shard_bounds[r];
        if (len <= 0) continue;
        // the shard's share of the budget, rounded to nearest (rounding down could halve the
        // chunks of many equal shards: 16 shards of 1.94 chunks each would get 1 apiece)
        const int64_t Ld = L > 0 ? L : 1;
        int64_t cr = (2 * budget * len + Ld) / (2 * Ld);
        if (cr < 1) cr = 1;
        const int64_t need = (len + cr - 1) / cr;
        if (need > ch) ch = need;
    }
    return (ch + kDecodeChunkQuantum - 1) / kDecodeChunkQuantum * kDecodeChunkQuantum;
}

int64_t decode_max_chunks(int64_t tail_cap, int n_shards, int32_t hkv) {
    // The plan above gives each shard at most budget*len/L + 1/2 chunks (at least 1), hence
    // at most budget + n_shards context chunks, and the query host at most ceil(tail_cap / 128).
    int64_t budget = 272 / hkv - 1;
    if (budget < n_shards) budget = n_shards;
    return budget + n_shards + (tail_cap + kDecodeChunkQuantum - 1) / kDecodeChunkQuantum;
}


namespace host {

thread_local std::string g_last_error;

star_status_t fail(star_status_t s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

star_status_t ok() {
    g_last_error.clear();
    return STAR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(star_dtype_t dt) { return dt == STAR_BF16 ? 2 : 4; }

star_status_t check_heads(int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt) {
    if (hq < 1 || hkv < 1) return fail(STAR_ERR_INVALID_ARG, "hq (%d) and hkv (%d) must be >= 1", hq, hkv);
    if (hq % hkv) return fail(STAR_ERR_INVALID_ARG, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
    if (d < 1) return fail(STAR_ERR_INVALID_ARG, "d (%d) must be >= 1", d);
    if (dt != STAR_F32 && dt != STAR_BF16) return fail(STAR_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
    if (d > 256 || d % 4)
        return fail(STAR_ERR_UNSUPPORTED, "head dim %d not supported (need d %% 4 == 0 and d <= 256)", d);
    return STAR_OK;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t partials_bytes(int64_t n_parts, int64_t n_rows, int32_t d) {
    return round_up((size_t)n_parts * n_rows * d * 4) + 2 * round_up((size_t)n_parts * n_rows * 4);
}
void partials_ptrs(void* ws, int64_t n_parts, int64_t n_rows, int32_t d, float** a, float** m, float** l) {
    char* base = static_cast<char*>(ws);
    *a = reinterpret_cast<float*>(base);
    *m = reinterpret_cast<float*>(base + round_up((size_t)n_parts * n_rows * d * 4));
    *l = reinterpret_cast<float*>(base + round_up((size_t)n_parts * n_rows * d * 4) +
                                  round_up((size_t)n_parts * n_rows * 4));
}

star_status_t check_decode(const void* q_new, const void* k_new, const void* v_new, int64_t L,
                           const int64_t* shard_bounds, int32_t n_shards, const void* k_tail, const void* v_tail,
                           int64_t tail_len, int64_t tail_cap, int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt,
                           float scale, const void* o, const float* lse) {
    if (!q_new || !k_new || !v_new || !k_tail || !v_tail || !o || !shard_bounds)
        return fail(STAR_ERR_INVALID_ARG, "required pointer is null");
    if (L < 1) return fail(STAR_ERR_INVALID_ARG, "L must be >= 1");
    if (n_shards < 1 || n_shards > 64) return fail(STAR_ERR_INVALID_ARG, "n_shards (%d) must be in [1, 64]", n_shards);
    if (shard_bounds[0] != 0 || shard_bounds[n_shards] != L)
        return fail(STAR_ERR_INVALID_ARG, "shard bounds must start at 0 and end at L");
    for (int r = 0; r < n_shards; ++r)
        if (shard_bounds[r + 1] < shard_bounds[r]) return fail(STAR_ERR_INVALID_ARG, "shard bounds must be non-decreasing");
    if (tail_len < 0 || tail_cap < 1 || tail_len + 1 > tail_cap)
        return fail(STAR_ERR_INVALID_ARG, "need 0 <= tail_len < tail_cap (tail_len %lld, tail_cap %lld)",
                    (long long)tail_len, (long long)tail_cap);
    if (!(std::isfinite(scale) && scale >= 0.f)) return fail(STAR_ERR_INVALID_ARG, "scale must be finite and >= 0");
    star_status_t s = check_heads(hq, hkv, d, dt);
    if (s != STAR_OK) return s;
    if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_tail) || !aligned16(v_tail) ||
        !aligned16(o) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    return STAR_OK;
}

star_status_t check_query(const void* q, int32_t rows, int64_t L, const int64_t* shard_bounds, int32_t n_shards,
                          const void* k_tail, const void* v_tail, int64_t tail_len, int64_t tail_cap, int32_t hq,
                          int32_t hkv, int32_t d, star_dtype_t dt, float scale, const void* o, const float* lse) {
    if (!q || !k_tail || !v_tail || !o || !shard_bounds) return fail(STAR_ERR_INVALID_ARG, "required pointer is null");
    if (L < 1) return fail(STAR_ERR_INVALID_ARG, "L must be >= 1");
    if (rows < 1) return fail(STAR_ERR_INVALID_ARG, "rows (%d) must be >= 1", rows);
    if (n_shards < 1 || n_shards > 64) return fail(STAR_ERR_INVALID_ARG, "n_shards (%d) must be in [1, 64]", n_shards);
    if (shard_bounds[0] != 0 || shard_bounds[n_shards] != L)
        return fail(STAR_ERR_INVALID_ARG, "shard bounds must start at 0 and end at L");
    for (int r = 0; r < n_shards; ++r)
        if (shard_bounds[r + 1] < shard_bounds[r]) return fail(STAR_ERR_INVALID_ARG, "shard bounds must be non-decreasing");
    if (tail_len < rows || tail_len > tail_cap)
        return fail(STAR_ERR_INVALID_ARG, "need rows <= tail_len <= tail_cap (rows %d, tail_len %lld, tail_cap %lld)",
                    rows, (long long)tail_len, (long long)tail_cap);
    if (!(std::isfinite(scale) && scale >= 0.f)) return fail(STAR_ERR_INVALID_ARG, "scale must be finite and >= 0");
    star_status_t s = check_heads(hq, hkv, d, dt);
    if (s != STAR_OK) return s;
    if (!aligned16(q) || !aligned16(k_tail) || !aligned16(v_tail) || !aligned16(o) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    return STAR_OK;
}

star_status_t plan_decode(const int64_t* shard_bounds, int32_t n_shards, int64_t tail_len, int64_t tail_cap,
                          int32_t hq, int32_t hkv, int32_t d, void* workspace, size_t workspace_bytes,
                          DecodeLaunch* dl, unsigned* tickets) {
    DecodeChunkPlan& plan = dl->plan;
    plan = {};
    plan.n_shards = n_shards;
    plan.chunk = decode_chunk_len(shard_bounds, n_shards, hkv);
    int64_t nc = 0;
    for (int r = 0; r < n_shards; ++r) {
        plan.shard_lo[r] = shard_bounds[r];
        plan.chunk_prefix[r] = (int32_t)nc;
        nc += (shard_bounds[r + 1] - shard_bounds[r] + plan.chunk - 1) / plan.chunk;
    }
    plan.shard_lo[n_shards] = shard_bounds[n_shards];
    plan.chunk_prefix[n_shards] = (int32_t)nc;
    nc += (tail_len + 1 + plan.chunk - 1) / plan.chunk;
    plan.chunk_prefix[n_shards + 1] = (int32_t)nc;
    plan.n_chunks = (int32_t)nc;
    const int64_t n_max = decode_max_chunks(tail_cap, n_shards, hkv);
    if (nc > n_max) return fail(STAR_ERR_HIP, "decode chunk plan exceeds its bound");
    const size_t part_bytes = partials_bytes(n_max, hq, d);
    const size_t need = part_bytes + (tickets ? 0 : round_up((size_t)hkv * 4));
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(STAR_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    partials_ptrs(workspace, n_max, hq, d, &dl->a, &dl->m, &dl->l);
    dl->tickets = tickets ? tickets : reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + part_bytes);
    return STAR_OK;
}

star_status_t check_kv_fp8(const void* x, int64_t tokens, int32_t hkv, int32_t d, star_dtype_t dt) {
    if (!x) return fail(STAR_ERR_INVALID_ARG, "x must be non-null");
    if (tokens < 0) return fail(STAR_ERR_INVALID_ARG, "tokens (%lld) must be >= 0", (long long)tokens);
    if (hkv < 1 || hkv > 65535) return fail(STAR_ERR_INVALID_ARG, "hkv (%d) must be in [1, 65535]", hkv);
    if (dt != STAR_F32 && dt != STAR_BF16) return fail(STAR_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
    if (d < 8 || d > 256 || d % 8)
        return fail(STAR_ERR_UNSUPPORTED, "head dim %d not supported (need d %% 8 == 0 and 8 <= d <= 256)", d);
    if (!aligned16(x)) return fail(STAR_ERR_INVALID_ARG, "x must be 16-byte aligned");
    return STAR_OK;
}

const char* last_error() { return g_last_error.c_str(); }

}  // namespace host
}  // namespace star
