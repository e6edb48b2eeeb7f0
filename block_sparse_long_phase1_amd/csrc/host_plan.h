// Host-side work planning and argument checks of libstarattn.
//
// Plain C++ with no device code and no HIP runtime calls, so that these pieces also build
// on their own with a host compiler (a sanitizer build checks them that way).  The kernels
// (prefill.hip, decode.hip) and the C-ABI layer (star_attn.cpp) use them.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "star_attn.h"

namespace star {

// Tile geometry of the MFMA attention kernel that the planners depend on.
constexpr int kAttnKeysPerTile = 64;        // keys per LDS tile
constexpr int kAttnQueriesPerGroup = 256;   // queries per workgroup (G q heads x 256/G rows)

// Key partitions of one Phase-2 partial launch.  Partition i holds keys [0, n_kv[i]) at
// k[i] / v[i], kv heads head_stride[i] elements apart; query row r sees token t iff
// causal[i] < 0 or t <= causal[i] + r.  Partitions are cut into splits of split_len keys;
// partition i owns global splits [split_prefix[i], split_prefix[i + 1]).
constexpr int kMaxParts = 65;
struct PartPlan {
    int n_parts;
    int64_t split_len;
    const void* k[kMaxParts];   // bf16 elements, or E4M3 codes for parts [0, n_f8)
    const void* v[kMaxParts];
    int64_t head_stride[kMaxParts];
    int64_t n_kv[kMaxParts];
    int64_t causal[kMaxParts];
    int32_t split_prefix[kMaxParts + 1];
    int n_f8;                   // parts [0, n_f8) hold E4M3 codes (with per-kv-head scales)
    const float* k_scale;       // [hkv], for E4M3 parts
    const float* v_scale;
};

// Key chunks of one decode launch: the context shards' chunks in order, then the query
// host's.
struct DecodeChunkPlan {
    int n_shards;
    int64_t chunk;                 // keys per chunk
    int64_t shard_lo[65];          // shard token bounds
    int32_t chunk_prefix[66];      // first chunk index of each shard; [n_shards] = first tail chunk
    int32_t n_chunks;              // total chunks including the tail ones
};

// MFMA attention kernel: head dim 64 or 128, G = hq / hkv dividing 256.
bool attn_mfma_supported(int d, int hq, int hkv);
// Largest per-kv-head token count the MFMA kernel addresses with 32-bit offsets.
int64_t attn_mfma_max_tokens(int d);
// Cut the partitions of `plan` (n_parts, n_kv set) into key splits: fills split_len and
// split_prefix and returns the number of query-row tiles.  Splits aim at one workgroup
// per compute unit with at least 8 key tiles each.
int partial_mfma_plan(PartPlan& plan, int32_t rows, int32_t hq, int32_t hkv);
// Upper bound on the splits partial_mfma_plan makes for n_parts partitions.
int64_t partial_mfma_max_splits(int32_t rows, int32_t hq, int32_t hkv, int n_parts);

// Split-KV decode kernel: bf16, d = 64 or 128, G in {1, 2, 4, 8, 16}.
bool decode_bf16_supported(int d, int hq, int hkv);
// Keys per decode chunk for a shard layout, and an upper bound on the chunk count of any
// call with at most tail_cap query-host tokens and n_shards shards.
int64_t decode_chunk_len(const int64_t* shard_bounds, int n_shards, int32_t hkv);
int64_t decode_max_chunks(int64_t tail_cap, int n_shards, int32_t hkv);

namespace host {

// Record a failure for star_last_error() and return its status; ok() clears the record.
star_status_t fail(star_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
star_status_t ok();
const char* last_error();

bool aligned16(const void* p);
int elem_bytes(star_dtype_t dt);
size_t round_up(size_t x);   // to 256 bytes

// Head counts, head dim and dtype every entry point shares.
star_status_t check_heads(int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt);

// Workspace layout of split partials: A [n][rows][d] fp32, then m [n][rows], then l [n][rows].
size_t partials_bytes(int64_t n_parts, int64_t n_rows, int32_t d);
void partials_ptrs(void* ws, int64_t n_parts, int64_t n_rows, int32_t d, float** a, float** m, float** l);

// Checks shared by the decode entry points and by the query-phase entry points (the
// context pointers are checked by each entry point).
star_status_t check_decode(const void* q_new, const void* k_new, const void* v_new, int64_t L,
                           const int64_t* shard_bounds, int32_t n_shards, const void* k_tail, const void* v_tail,
                           int64_t tail_len, int64_t tail_cap, int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt,
                           float scale, const void* o, const float* lse);
star_status_t check_query(const void* q, int32_t rows, int64_t L, const int64_t* shard_bounds, int32_t n_shards,
                          const void* k_tail, const void* v_tail, int64_t tail_len, int64_t tail_cap, int32_t hq,
                          int32_t hkv, int32_t d, star_dtype_t dt, float scale, const void* o, const float* lse);
star_status_t check_kv_fp8(const void* x, int64_t tokens, int32_t hkv, int32_t d, star_dtype_t dt);

// Chunk plan of the decode kernel and its workspace carve-up.
struct DecodeLaunch {
    DecodeChunkPlan plan;
    float *a, *m, *l;
    unsigned* tickets;
};
// Workspace layout: the chunk partials, then hkv 32-bit counters.  With `tickets` given, the
// counters live there instead and the workspace holds the partials only.
star_status_t plan_decode(const int64_t* shard_bounds, int32_t n_shards, int64_t tail_len, int64_t tail_cap,
                          int32_t hq, int32_t hkv, int32_t d, void* workspace, size_t workspace_bytes,
                          DecodeLaunch* dl, unsigned* tickets = nullptr);

}  // namespace host
}  // namespace star
