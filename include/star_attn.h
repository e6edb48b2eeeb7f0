/*
 * star_attn.h -- C ABI of libstarattn.so: the Star Attention two-phase
 * attention hot path on one AMD Instinct MI355X (gfx950).
 *
 * Sources (pages, cited by title and section):
 *   [SUM]    "Star Attention: Efficient LLM Inference over Long Sequences",
 *            paper-graph-ui long-form summary of arXiv 2411.17116, section 3.4
 *            "Detailed, Sentence-Based Technical Breakdown".
 *   [README] "NVIDIA/Star-Attention" (shadowgraph.io mirror of the project
 *            README), section "Two Phases of Star Attention".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  One sequence (see Batches below), head-major, contiguous: queries [Hq, rows, d], keys and
 *   values [Hkv, tokens, d].  Grouped-query attention maps q head h to kv
 *   head h / (Hq / Hkv) (contiguous groups).  Hq must be a multiple of Hkv.
 * Scale.  Scores are scale * <q, k>; pass scale = 1/sqrt(d) for the pages'
 *   attention ([SUM] 3.4 "The Attention Decomposition").  All logs and
 *   log-sum-exps are natural logs of the scaled scores.  scale must be finite
 *   and >= 0 (else STAR_ERR_INVALID_ARG): the kernels take a row's largest
 *   score as scale times its largest dot product.
 * Softmax statistics.  A partial result over a key partition is (A, m, l):
 *   A is normalised over that partition alone, m is the largest scaled score
 *   and l = sum exp(score - m), so the pages' s_h equals e^m * l.  An empty
 *   partition is A = 0, m = -inf, l = 0 and weighs nothing in a merge.
 * Types.  STAR_BF16 inputs are accumulated in fp32.  The MFMA kernels take
 *   d = 64 or 128 (Phase 1, Phase-2 partials and queries, the decode step);
 *   other bf16 shapes and STAR_F32 inputs take a plain vector path
 *   (d <= 256, any multiple of 4).  Partials and LSEs are always fp32.
 * Batches.  B sequences of equal length, laid out [B, H, tokens, d], are one
 *   call with hq = B*Hq and hkv = B*Hkv: q head b*Hq + h then maps to kv head
 *   b*Hkv + h/G, which is that sequence's own kv head.
 * Memory and ownership.  Every pointer not marked "host" is device memory
 *   owned by the caller, 16-byte aligned.  The library never allocates or
 *   frees device memory and keeps no state between calls other than what a
 *   caller-provided workspace holds; entry points that need scratch take such
 *   a workspace, whose size the matching *_workspace_bytes() call returns.
 *   The one exception, star_decode_step_noalloc, keeps its scratch in a fixed
 *   static device array instead (see there).
 * Streams and errors.  Every call only enqueues work on `stream` and returns
 *   without synchronising.  Arguments are checked on the host before anything
 *   is enqueued: a bad argument returns STAR_ERR_INVALID_ARG, a shape the
 *   kernels do not cover returns STAR_ERR_UNSUPPORTED, a short workspace
 *   STAR_ERR_WORKSPACE, and a failed launch STAR_ERR_HIP.  On any error
 *   nothing has been enqueued except, for STAR_ERR_HIP, work launched before
 *   the failing launch.  star_last_error() describes the last failure on the
 *   calling thread.  No C++ exception crosses this interface.  Calls are
 *   thread-safe; calls that write the same buffers must be ordered by the
 *   caller's streams.
 */
#ifndef STAR_ATTN_H
#define STAR_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The entry points below are the library's only exported symbols (it is built with hidden
 * visibility). */
#define STAR_API __attribute__((visibility("default")))

typedef enum {
    STAR_OK = 0,
    STAR_ERR_INVALID_ARG = 1,
    STAR_ERR_UNSUPPORTED = 2,
    STAR_ERR_HIP = 3,
    STAR_ERR_WORKSPACE = 4
} star_status_t;

typedef enum { STAR_F32 = 0, STAR_BF16 = 1 } star_dtype_t;

/* Static name of a status code. */
STAR_API const char *star_status_str(star_status_t status);

/* Human-readable description of the last failure on the calling thread
 * ("" if none).  The string stays valid until the thread's next call. */
STAR_API const char *star_last_error(void);

/* Library version, "major.minor.patch". */
STAR_API const char *star_version(void);

/*
 * Phase 1: anchored blockwise-local context encoding.
 * [SUM] 3.4 Phase 1 Steps 1-5; [README] "Phase 1 - Context Encoding".
 *
 * The context of L tokens is cut into n = ceil(L / block) contiguous blocks
 * (the last may be shorter).  Block 0 is attended causally on its own; every
 * later block i is attended causally after the anchor, i.e. the row of
 * context position p in block i >= 1 sees the anchor tokens [0, anchor) and
 * its own block's tokens [i*block, p].  The anchor keeps its original
 * positions, so with post-rotary inputs its keys are the block-0 keys and are
 * read in place; anchor rows of later blocks are not produced and anchor
 * keys/values are never copied, so k and v, unchanged, are the Phase-2
 * context cache (each token once).
 *
 *   q    [hq, L, d]    queries of the context tokens (dt)
 *   k, v [hkv, L, d]   keys / values of the context tokens (dt)
 *   o    [hq, L, d]    output (dt, round-to-nearest-even)
 *   lse  [hq, L]       fp32 log-sum-exp of each row's scores, or NULL
 *   L >= 1, block >= 1, 0 <= anchor <= block.
 * One kernel launch: bf16 with d = 64 or 128 and hq/hkv a divisor of 256 run
 * the MFMA kernel, which addresses a kv head with 32-bit offsets and so takes
 * at most 2^31 / d tokens (more returns STAR_ERR_UNSUPPORTED); fp32 and other
 * head dims (d % 4 == 0, d <= 256) run the vector kernel.
 */
STAR_API star_status_t star_phase1_encode(const void *q, const void *k, const void *v,
                                          void *o, float *lse,
                                          int64_t L, int64_t block, int64_t anchor,
                                          int32_t hq, int32_t hkv, int32_t d,
                                          star_dtype_t dt, float scale, hipStream_t stream);

/*
 * Phase 2, one partition ("host"): local attention of the query rows over
 * one KV partition and its softmax statistics.
 * [SUM] 3.4 Phase 2 Step 3 (the A_h and s_h equations); [README] "Phase 2".
 *
 *   q [hq, rows, d] (dt); rows >= 1
 *   k, v: partition token t of kv head g is at element offset
 *         g * kv_head_stride + t * d, for 0 <= t < n_kv (n_kv >= 0).  A
 *         context shard [lo, hi) of a [hkv, L, d] cache is k + lo*d with
 *         kv_head_stride = L*d and n_kv = hi - lo.
 *   causal_offset < 0: every row sees every partition token; otherwise row i
 *         sees token t only if t <= causal_offset + i (the query host's own
 *         cache, where query tokens are causal among themselves).
 *   a_out [hq, rows, d], m_out [hq, rows], l_out [hq, rows]: fp32 (A, m, l).
 *   workspace: star_phase2_workspace_bytes(rows, n_kv, hq, hkv, d) bytes
 *         (may be 0, then workspace may be NULL).
 * One or two kernel launches (a key-split pass and its merge).  Shapes and the
 * 2^31 / d token limit of the MFMA kernel as for star_phase1_encode (n_kv
 * counts the tokens).
 */
STAR_API size_t star_phase2_workspace_bytes(int32_t rows, int64_t n_kv, int32_t hq, int32_t hkv, int32_t d);

STAR_API star_status_t star_phase2_partial(const void *q, int32_t rows,
                                           const void *k, const void *v,
                                           int64_t kv_head_stride, int64_t n_kv, int64_t causal_offset,
                                           int32_t hq, int32_t hkv, int32_t d,
                                           star_dtype_t dt, float scale,
                                           float *a_out, float *m_out, float *l_out,
                                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Phase 2 query encoding on the query host, every partition in one call.
 * [SUM] 3.4 Phase 2 Steps 1-5; [README] "Phase 2 - Query Processing and Token
 * Generation".
 *
 * The `rows` query tokens are the last `rows` entries of the query host's cache
 * (their k/v already stored there): query row i sits at cache position
 * c_i = tail_len - rows + i and sees every context token plus cache positions
 * [0, c_i].  The local partial of each context shard and of the query host's
 * cache is computed and all are merged in log space, which gives the exact
 * global attention of the query rows.
 *
 *   q [hq, rows, d] (dt); rows >= 1
 *   k_ctx, v_ctx [hkv, L, d]                context cache (dt), L >= 1
 *   shard_bounds (host) int64[n_shards + 1]: 0 = b_0 <= b_1 <= ... <= b_S = L;
 *                                            1 <= n_shards <= 64
 *   k_tail, v_tail [hkv, tail_cap, d]       query-host cache (dt); entries
 *                                           [0, tail_len) are valid
 *   rows <= tail_len <= tail_cap.
 *   o [hq, rows, d] (dt), lse [hq, rows] fp32 or NULL
 *   workspace: star_phase2_query_workspace_bytes(rows, n_shards, hq, hkv, d)
 *         bytes (may be 0 for shapes without the MFMA path; then workspace may
 *         be NULL).  Scratch only: its contents need no initialisation.
 * bf16 with d = 64 or 128 and hq/hkv a divisor of 256: two kernel launches (the
 * partials of every key split of every partition, then their merge), for at most
 * 2^31 / d tokens in the context and in the query host's cache (more returns
 * STAR_ERR_UNSUPPORTED).  Other shapes: one vector-path launch.
 */
STAR_API size_t star_phase2_query_workspace_bytes(int32_t rows, int32_t n_shards, int32_t hq, int32_t hkv, int32_t d);

STAR_API star_status_t star_phase2_query(const void *q, int32_t rows,
                                         const void *k_ctx, const void *v_ctx, int64_t L,
                                         const int64_t *shard_bounds, int32_t n_shards,
                                         const void *k_tail, const void *v_tail, int64_t tail_len, int64_t tail_cap,
                                         int32_t hq, int32_t hkv, int32_t d,
                                         star_dtype_t dt, float scale,
                                         void *o, float *lse,
                                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Global aggregation of partitions in log space.
 * [README] "Phase 2" (s_global = sum s_h, A_global = sum (s_h/s_global) A_h);
 * [SUM] 3.4 Phase 2 Step 5 (the same sum kept in log space).
 *
 *   a [n_parts, hq, rows, d], m and l [n_parts, hq, rows]: fp32 partials.
 *   o [hq, rows, d] (out_dt), lse_out [hq, rows] fp32 or NULL.
 *   With M = max_p m_p and w_p = l_p e^{m_p - M}:
 *   o = sum w_p A_p / sum w_p and lse = M + log sum w_p.  Rows whose
 *   partitions are all empty get o = 0 and lse = -inf.
 * One kernel launch.
 */
STAR_API star_status_t star_softmax_merge(const float *a, const float *m, const float *l, int32_t n_parts,
                                          int32_t hq, int32_t rows, int32_t d,
                                          void *o, star_dtype_t out_dt, float *lse_out, hipStream_t stream);

/*
 * Phase 2, one generated token on the query host.
 * [SUM] 3.4 Phase 2 Steps 3-5 and 7; [README] "Phase 2".
 *
 * Appends the new token's k/v to the query host's cache (the only cache that
 * grows) and computes its attention over every context token plus the query
 * host's cache including itself, as per-partition partials merged in log
 * space.  The context cache is split into the n_shards host partitions
 * given by shard_bounds; each is further split into key chunks internally.
 *
 *   q_new [hq, d], k_new / v_new [hkv, d]   the new token (dt)
 *   k_ctx, v_ctx [hkv, L, d]                context cache (dt), L >= 1
 *   shard_bounds (host) int64[n_shards + 1]: 0 = b_0 <= b_1 <= ... <= b_S = L;
 *                                            1 <= n_shards <= 64
 *   k_tail, v_tail [hkv, tail_cap, d]       query-host cache (dt); entries
 *                                           [0, tail_len) are valid on entry,
 *                                           entry tail_len is written
 *   o [hq, d] (dt), lse [hq] fp32 or NULL
 *   workspace: star_decode_workspace_bytes(L, tail_cap, n_shards, hq, hkv, d)
 *         bytes.  It must be zero-filled before its first use; every call that
 *         completes leaves it ready for the next (its per-kv-head completion
 *         counters back at zero).  Calls that share a workspace must be
 *         ordered on one stream.
 *   0 <= tail_len < tail_cap.
 * bf16 with d = 64 or 128 and hq/hkv of 1, 2 or 4: one kernel launch (chunk
 * partials, the append, and the merge done by the last chunk of each kv head);
 * hq/hkv of 8 or 16: that launch without the merge, then a merge launch.  Other
 * shapes: an append launch and a vector-path launch.
 */
STAR_API size_t star_decode_workspace_bytes(int64_t L, int64_t tail_cap, int32_t n_shards,
                                            int32_t hq, int32_t hkv, int32_t d);

STAR_API star_status_t star_decode_step(const void *q_new, const void *k_new, const void *v_new,
                                        const void *k_ctx, const void *v_ctx, int64_t L,
                                        const int64_t *shard_bounds, int32_t n_shards,
                                        void *k_tail, void *v_tail, int64_t tail_len, int64_t tail_cap,
                                        int32_t hq, int32_t hkv, int32_t d,
                                        star_dtype_t dt, float scale,
                                        void *o, float *lse,
                                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * star_decode_step without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.
 *
 * Arguments, results and launches as star_decode_step, minus the workspace.
 * The bf16 MFMA path (d = 64 or 128, hq/hkv of 1, 2, 4, 8 or 16) keeps its
 * chunk partials and per-kv-head completion counters in a static device array
 * of STAR_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; the other shapes need no scratch.  A shape
 * whose partials need more than STAR_DECODE_NOALLOC_SCRATCH_BYTES minus
 * 4 * STAR_DECODE_NOALLOC_MAX_HKV bytes (the bound star_decode_workspace_bytes
 * gives, less the counters), or with hkv above STAR_DECODE_NOALLOC_MAX_HKV,
 * returns STAR_ERR_WORKSPACE before anything is enqueued.  This call never
 * allocates or frees memory; its first call on a device looks up that device's
 * copy of the array (no allocation, no stream work).
 * The counters are zero when the library is loaded and every completed call
 * leaves them at zero.  All calls on one GPU share its one array: calls that
 * may overlap on one GPU (on different streams, or from several threads
 * without ordering) race and give wrong results; order them on one stream.
 */
#define STAR_DECODE_NOALLOC_SCRATCH_BYTES (8u << 20)
#define STAR_DECODE_NOALLOC_MAX_HKV 1024

STAR_API star_status_t star_decode_step_noalloc(const void *q_new, const void *k_new, const void *v_new,
                                                const void *k_ctx, const void *v_ctx, int64_t L,
                                                const int64_t *shard_bounds, int32_t n_shards,
                                                void *k_tail, void *v_tail, int64_t tail_len, int64_t tail_cap,
                                                int32_t hq, int32_t hkv, int32_t d,
                                                star_dtype_t dt, float scale,
                                                void *o, float *lse, hipStream_t stream);

/*
 * E4M3 context KV cache.
 * [SUM] "Related Work", part "Memory Optimization and KV Cache Compression":
 * KV-cache quantisation is orthogonal to the method and combines with it.
 * The pages fix no format; here the context hosts' cached K and V may be held
 * as OCP E4M3 codes (1 byte per element: sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, largest finite 448, S.1111.111 = NaN) with one fp32 scale
 * per kv head for K and one for V; the cached value is scale * decode(code).
 * The query host's cache stays in the compute dtype.  A typical order: Phase
 * 1, then star_kv_fp8_scales and star_kv_quantize_fp8 on each context tensor,
 * then the query phase (star_phase2_query, or star_phase2_query_kv8 on the
 * codes) and star_decode_step_kv8 per generated token.
 *
 * star_kv_fp8_scales: scale[g] = max |x[g]| / 448 in fp32 (1 for a head that
 * is all zeros), so each head's largest element maps to +-448.
 *   x [hkv, tokens, d] (dt: STAR_BF16 or STAR_F32), 16-byte aligned;
 *   tokens >= 0; 1 <= hkv <= 65535; d % 8 == 0, 8 <= d <= 256
 *   scale [hkv] fp32 (device), written.  Three kernel launches, no memset.
 *
 * star_kv_quantize_fp8: out[g] = E4M3 code of the correctly rounded fp32
 * quotient x[g] / scale[g]: the nearest E4M3 value, a tie going to the even
 * mantissa; magnitudes from 448 up (infinities too) give +-448, NaN gives the
 * NaN code of its sign.  The sign bit is kept (-0 and negative values that
 * round to zero give 0x80).
 *   x as above; scale [hkv] fp32 (device), positive and finite;
 *   out [hkv, tokens, d] uint8 (device, 16-byte aligned), written.
 *   One kernel launch.  x and out may not overlap.
 */
STAR_API star_status_t star_kv_fp8_scales(const void *x, int64_t tokens, int32_t hkv, int32_t d,
                                          star_dtype_t dt, float *scale, hipStream_t stream);

STAR_API star_status_t star_kv_quantize_fp8(const void *x, int64_t tokens, int32_t hkv, int32_t d,
                                            star_dtype_t dt, const float *scale, void *out,
                                            hipStream_t stream);

/*
 * Phase 2, one partition held as E4M3 codes.
 * [SUM] 3.4 Phase 2 Step 3 over the dequantised partition (see above).
 *
 * Arguments and behaviour as star_phase2_partial, except:
 *   k8, v8: E4M3 codes (uint8, 16-byte aligned) replace k / v, with the same
 *   element offsets (g * kv_head_stride + t * d; kv_head_stride a multiple of
 *   16); k_scale, v_scale [hkv] fp32 (device, 4-byte aligned) are their
 *   scales, so token t of kv head g has key k_scale[g] * decode(k8[...]).
 *   The (A, m, l) outputs are those of the dequantised partition.  dt must be
 *   STAR_BF16 (q), d 64 or 128 and hq/hkv a divisor of 256; other shapes return
 *   STAR_ERR_UNSUPPORTED.  The workspace is star_phase2_workspace_bytes(...)
 *   bytes, with the same rules.
 */
STAR_API star_status_t star_phase2_partial_kv8(const void *q, int32_t rows,
                                               const void *k8, const void *v8,
                                               const float *k_scale, const float *v_scale,
                                               int64_t kv_head_stride, int64_t n_kv, int64_t causal_offset,
                                               int32_t hq, int32_t hkv, int32_t d,
                                               star_dtype_t dt, float scale,
                                               float *a_out, float *m_out, float *l_out,
                                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Phase 2 query encoding over an E4M3 context cache.
 * [SUM] 3.4 Phase 2 Steps 1-5 over the dequantised context (see above).
 *
 * Arguments and behaviour as star_phase2_query, except:
 *   k_ctx8, v_ctx8 [hkv, L, d] uint8 E4M3 codes (16-byte aligned) replace
 *   k_ctx / v_ctx; k_scale, v_scale [hkv] fp32 (device, 4-byte aligned) are
 *   their scales.  dt must be STAR_BF16 (q, the query-host cache and o), d 64
 *   or 128 and hq/hkv a divisor of 256; other shapes return
 *   STAR_ERR_UNSUPPORTED.  The workspace is
 *   star_phase2_query_workspace_bytes(...) bytes, with the same rules.  Two
 *   kernel launches as star_phase2_query's bf16 path; the context tiles are
 *   widened exactly to bf16 on their way into LDS.
 */
STAR_API star_status_t star_phase2_query_kv8(const void *q, int32_t rows,
                                             const void *k_ctx8, const void *v_ctx8,
                                             const float *k_scale, const float *v_scale, int64_t L,
                                             const int64_t *shard_bounds, int32_t n_shards,
                                             const void *k_tail, const void *v_tail,
                                             int64_t tail_len, int64_t tail_cap,
                                             int32_t hq, int32_t hkv, int32_t d,
                                             star_dtype_t dt, float scale,
                                             void *o, float *lse,
                                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Phase 2, one generated token over an E4M3 context cache.
 * [SUM] 3.4 Phase 2 Steps 3-5 and 7 over the dequantised context (see above).
 *
 * Arguments and behaviour as star_decode_step, except:
 *   k_ctx8, v_ctx8 [hkv, L, d] uint8 E4M3 codes (16-byte aligned) replace
 *   k_ctx / v_ctx; k_scale, v_scale [hkv] fp32 (device) are their scales.
 *   dt must be STAR_BF16 (q_new, k_new, v_new, the query-host cache and o),
 *   d 64 or 128 and hq/hkv one of 1, 2, 4, 8, 16; other shapes return
 *   STAR_ERR_UNSUPPORTED.  The workspace is star_decode_workspace_bytes(...)
 *   bytes, with the same rules.  Launches as star_decode_step's bf16 path.
 */
STAR_API star_status_t star_decode_step_kv8(const void *q_new, const void *k_new, const void *v_new,
                                            const void *k_ctx8, const void *v_ctx8,
                                            const float *k_scale, const float *v_scale, int64_t L,
                                            const int64_t *shard_bounds, int32_t n_shards,
                                            void *k_tail, void *v_tail, int64_t tail_len, int64_t tail_cap,
                                            int32_t hq, int32_t hkv, int32_t d,
                                            star_dtype_t dt, float scale,
                                            void *o, float *lse,
                                            void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STAR_ATTN_H */
