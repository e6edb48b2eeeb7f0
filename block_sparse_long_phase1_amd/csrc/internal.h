// Internal interfaces between the C-ABI layer (star_attn.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_plan.h"

namespace star {

// Arguments of the bf16 MFMA attention kernel (Phase 1 and Phase-2 partials).
struct AttnMfmaArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int64_t kv_head_stride;   // elements between kv heads
    int64_t q_rows;           // rows per q head in q (and in the outputs)
    int hq, hkv, G, rows_per_wg;
    int head_major;           // Phase 1: work items ordered head by head (else heads interleave)
    float scale_log2;         // scale * log2(e)
    // Phase 1
    int64_t L, block, anchor;
    int64_t n_blocks, nt_full, nt_last, nt0, tiles_ge1;
    uint16_t* o;
    float* lse;
    // Phase-2 partial
    int64_t rows;
    int64_t n_row_tiles;
    float* a_out;     // [splits][hq][rows][d], m and l [splits][hq][rows]
    float* m_out;
    float* l_out;
    PartPlan plan;
};

hipError_t launch_phase1_mfma(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* o, float* lse, int64_t L, int64_t block, int64_t anchor,
                              int hq, int hkv, int d, float scale, hipStream_t stream);

// Partials of every split of `plan` into a_out / m_out / l_out (global split order).
hipError_t launch_partial_mfma(const uint16_t* q, int32_t rows, int hq, int hkv, int d, float scale,
                               const PartPlan& plan, int n_row_tiles, float* a_out, float* m_out,
                               float* l_out, hipStream_t stream);

// Log-space merge of n_parts partials laid out [n_parts][n_rows][d] / [n_parts][n_rows].
// Writes o ([n_rows][d], fp32 or bf16 per out_bf16), and optionally lse, or (m, l).
hipError_t launch_merge(const float* a, const float* m, const float* l, int n_parts, int64_t n_rows,
                        int d, void* o, bool out_bf16, float* lse_out, float* m_out, float* l_out,
                        hipStream_t stream);

// Split-KV decode (bf16, d = 64 or 128): chunk partials for every kv head, the append of the
// new token into the query host's cache, and the log-space merge by the last chunk of
// each kv head (tickets: hkv zero-initialised counters, left at zero).
// k8 / v8 non-null: the context partitions are E4M3 codes with per-kv-head scales
// k_scale / v_scale (k_ctx / v_ctx unused); null: bf16 k_ctx / v_ctx.
hipError_t launch_decode_bf16(const uint16_t* q_new, const uint16_t* k_new, const uint16_t* v_new,
                              const uint16_t* k_ctx, const uint16_t* v_ctx, const uint8_t* k8, const uint8_t* v8,
                              const float* k_scale, const float* v_scale, int64_t L,
                              uint16_t* k_tail, uint16_t* v_tail, int64_t tail_len, int64_t tail_cap,
                              int hq, int hkv, int d, float scale, const DecodeChunkPlan& plan,
                              float* part_a, float* part_m, float* part_l, unsigned* tickets,
                              uint16_t* o, float* lse, hipStream_t stream);

// E4M3 context cache (kvfp8.hip).  Both need d % 8 == 0 and 16-byte aligned x.
// Scales: scale[g] = max |x[g]| / 448 (1 for an all-zero head); three launches.
hipError_t launch_kv_fp8_scales(const void* x, int64_t tokens, int hkv, int d, bool bf16, float* scale,
                                hipStream_t stream);
// out[g] = E4M3 code of x[g] / scale[g] (nearest, ties to even, saturating at 448).
hipError_t launch_kv_quantize_fp8(const void* x, int64_t tokens, int hkv, int d, bool bf16, const float* scale,
                                  uint8_t* out, hipStream_t stream);

// Plain vector path (fp32 or bf16 inputs, any d <= 256 with d % 4 == 0): one wave per row.
struct RowKeySeg {
    const void* k;       // base of token 0 of this segment for kv head 0
    const void* v;
    int64_t head_stride; // elements between kv heads
    int64_t n;           // tokens in the segment
    int64_t causal_lim;  // < 0: all visible; else token t visible to row i iff t <= causal_lim + i
};
struct RowAttnArgs {
    const void* q;
    int64_t q_rows;      // rows per head in q
    int hq, hkv, d;
    int is_bf16;
    float scale;
    int mode;            // 0: phase 1 (segments derived per row); 1: explicit segments
    // mode 0
    const void* k;
    const void* v;
    int64_t L, block, anchor;
    // mode 1
    RowKeySeg seg[3];
    int n_seg;
    // outputs: o (dtype) + lse, or (a, m, l) fp32
    void* o;
    float* lse;
    float* a_out;
    float* m_out;
    float* l_out;
    int64_t row_offset;  // mode 1: row i uses causal row index i + row_offset
};
hipError_t launch_row_attn(const RowAttnArgs& a, int64_t rows, hipStream_t stream);

// Copy n_bytes of k_new / v_new rows into the tail at `tail_len` (vector path append).
hipError_t launch_tail_append(const void* k_new, const void* v_new, void* k_tail, void* v_tail,
                              int64_t tail_len, int64_t tail_cap, int hkv, int d, int elem_bytes,
                              hipStream_t stream);

}  // namespace star
