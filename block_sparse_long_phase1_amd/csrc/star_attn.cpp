// C ABI of libstarattn.so: argument checking, work planning and dispatch to
// the gfx950 kernels.  Every entry point validates on the host before it
// enqueues anything, never allocates device memory and never synchronises.
#include "star_attn.h"

#include <mutex>

#include "internal.h"

using namespace star::host;

namespace {

star_status_t hip_fail(hipError_t e, const char* where) {
    return fail(STAR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// One partition on the MFMA kernel (E4M3 codes when k_scale is set): its key splits, then
// their merge into (A, m, l) when there are several.
star_status_t partial_mfma(const void* q, int32_t rows, const void* k, const void* v, const float* k_scale,
                           const float* v_scale, int64_t kv_head_stride, int64_t n_kv, int64_t causal_offset,
                           int32_t hq, int32_t hkv, int32_t d, float scale, float* a_out, float* m_out,
                           float* l_out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                           const char* who) {
    if (n_kv > star::attn_mfma_max_tokens(d))
        return fail(STAR_ERR_UNSUPPORTED, "n_kv (%lld) above %lld tokens per partition", (long long)n_kv,
                    (long long)star::attn_mfma_max_tokens(d));
    star::PartPlan plan = {};
    plan.n_parts = 1;
    plan.k[0] = k;
    plan.v[0] = v;
    plan.head_stride[0] = kv_head_stride;
    plan.n_kv[0] = n_kv;
    plan.causal[0] = causal_offset < 0 ? -1 : causal_offset;
    plan.n_f8 = k_scale ? 1 : 0;
    plan.k_scale = k_scale;
    plan.v_scale = v_scale;
    const int nrt = star::partial_mfma_plan(plan, rows, hq, hkv);
    const int32_t ns = plan.split_prefix[1];
    const uint16_t* qb = static_cast<const uint16_t*>(q);
    hipError_t e;
    if (ns == 1) {
        e = star::launch_partial_mfma(qb, rows, hq, hkv, d, scale, plan, nrt, a_out, m_out, l_out, stream);
        if (e != hipSuccess) return hip_fail(e, who);
        return ok();
    }
    const size_t need = partials_bytes(ns, (int64_t)hq * rows, d);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(STAR_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    float *wa, *wm, *wl;
    partials_ptrs(workspace, ns, (int64_t)hq * rows, d, &wa, &wm, &wl);
    e = star::launch_partial_mfma(qb, rows, hq, hkv, d, scale, plan, nrt, wa, wm, wl, stream);
    if (e != hipSuccess) return hip_fail(e, who);
    e = star::launch_merge(wa, wm, wl, ns, (int64_t)hq * rows, d, a_out, false, nullptr, m_out, l_out, stream);
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
}

// The query phase on the MFMA kernel: one partial launch over every context shard and the
// query host's cache (E4M3 context shards when k_scale is set), then the merge.
star_status_t query_mfma(const void* q, int32_t rows, const void* k_ctx, const void* v_ctx, const float* k_scale,
                         const float* v_scale, int64_t L, const int64_t* shard_bounds, int32_t n_shards,
                         const void* k_tail, const void* v_tail, int64_t tail_len, int64_t tail_cap, int32_t hq,
                         int32_t hkv, int32_t d, float scale, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, const char* who) {
    if (L > star::attn_mfma_max_tokens(d) || tail_cap > star::attn_mfma_max_tokens(d))
        return fail(STAR_ERR_UNSUPPORTED, "more than %lld tokens per kv head", (long long)star::attn_mfma_max_tokens(d));
    const bool f8 = k_scale != nullptr;
    const int eb = f8 ? 1 : 2;   // bytes per context element
    star::PartPlan plan = {};
    plan.n_parts = n_shards + 1;
    for (int r = 0; r < n_shards; ++r) {
        plan.k[r] = static_cast<const char*>(k_ctx) + shard_bounds[r] * d * eb;
        plan.v[r] = static_cast<const char*>(v_ctx) + shard_bounds[r] * d * eb;
        plan.head_stride[r] = L * d;
        plan.n_kv[r] = shard_bounds[r + 1] - shard_bounds[r];
        plan.causal[r] = -1;
    }
    plan.k[n_shards] = k_tail;
    plan.v[n_shards] = v_tail;
    plan.head_stride[n_shards] = tail_cap * d;
    plan.n_kv[n_shards] = tail_len;
    plan.causal[n_shards] = tail_len - rows;   // row i sees query-host tokens t <= tail_len - rows + i
    plan.n_f8 = f8 ? n_shards : 0;
    plan.k_scale = k_scale;
    plan.v_scale = v_scale;
    const int nrt = star::partial_mfma_plan(plan, rows, hq, hkv);
    const int32_t ns = plan.split_prefix[plan.n_parts];
    const int64_t n_max = star::partial_mfma_max_splits(rows, hq, hkv, plan.n_parts);
    if (ns > n_max) return fail(STAR_ERR_HIP, "%s: split plan exceeds its bound", who);
    const size_t need = partials_bytes(n_max, (int64_t)hq * rows, d);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(STAR_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    float *wa, *wm, *wl;
    partials_ptrs(workspace, ns, (int64_t)hq * rows, d, &wa, &wm, &wl);
    hipError_t e = star::launch_partial_mfma(static_cast<const uint16_t*>(q), rows, hq, hkv, d, scale, plan, nrt,
                                             wa, wm, wl, stream);
    if (e != hipSuccess) return hip_fail(e, who);
    e = star::launch_merge(wa, wm, wl, ns, (int64_t)hq * rows, d, o, true, lse, nullptr, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
}

// ---- Scratch of star_decode_step_noalloc, for callers that cannot allocate.
// A file-scope device array: every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  Its first kNoAllocTicketBytes hold the per-kv-head
// completion counters, at a fixed place so that no call's partials ever land on them: they
// are zero when the library is loaded and every completed decode call leaves them at zero.
// The rest holds one call's chunk partials, which need no initialisation.
constexpr size_t kNoAllocScratchBytes = STAR_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr size_t kNoAllocTicketBytes = 4 * STAR_DECODE_NOALLOC_MAX_HKV;
static_assert(kNoAllocTicketBytes % 256 == 0, "partials stay 256-byte aligned");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The device address of this device's `scratch`, looked up once per device with that device
// current.  Host code uses this address, never the array's name (a host-side stand-in).
star_status_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "star_decode_step_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(STAR_ERR_UNSUPPORTED, "device ordinal %d above %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "star_decode_step_noalloc: hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(STAR_ERR_HIP, "star_decode_step_noalloc: no device address for the scratch array");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return STAR_OK;
}

}  // namespace

extern "C" {

const char* star_status_str(star_status_t status) {
    switch (status) {
        case STAR_OK: return "STAR_OK";
        case STAR_ERR_INVALID_ARG: return "STAR_ERR_INVALID_ARG";
        case STAR_ERR_UNSUPPORTED: return "STAR_ERR_UNSUPPORTED";
        case STAR_ERR_HIP: return "STAR_ERR_HIP";
        case STAR_ERR_WORKSPACE: return "STAR_ERR_WORKSPACE";
    }
    return "STAR_ERR_UNKNOWN";
}

const char* star_last_error(void) { return star::host::last_error(); }

const char* star_version(void) { return "0.1.0"; }

// ------------------------------------------------------------------------ Phase 1
star_status_t star_phase1_encode(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t L, int64_t block, int64_t anchor, int32_t hq, int32_t hkv,
                                 int32_t d, star_dtype_t dt, float scale, hipStream_t stream) {
    try {
        if (!q || !k || !v || !o) return fail(STAR_ERR_INVALID_ARG, "q, k, v and o must be non-null");
        if (L < 1) return fail(STAR_ERR_INVALID_ARG, "L (%lld) must be >= 1", (long long)L);
        if (block < 1) return fail(STAR_ERR_INVALID_ARG, "block (%lld) must be >= 1", (long long)block);
        if (anchor < 0 || anchor > block)
            return fail(STAR_ERR_INVALID_ARG, "anchor (%lld) must satisfy 0 <= anchor <= block (%lld)",
                        (long long)anchor, (long long)block);
        if (!(std::isfinite(scale) && scale >= 0.f)) return fail(STAR_ERR_INVALID_ARG, "scale must be finite and >= 0");
        star_status_t s = check_heads(hq, hkv, d, dt);
        if (s != STAR_OK) return s;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
            (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
            return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
        hipError_t e;
        if (dt == STAR_BF16 && star::attn_mfma_supported(d, hq, hkv)) {
            if (L > star::attn_mfma_max_tokens(d))
                return fail(STAR_ERR_UNSUPPORTED, "L (%lld) above %lld tokens per kv head", (long long)L,
                            (long long)star::attn_mfma_max_tokens(d));
            e = star::launch_phase1_mfma(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                                         L, block, anchor, hq, hkv, d, scale, stream);
        } else {
            star::RowAttnArgs a = {};
            a.q = q; a.q_rows = L; a.hq = hq; a.hkv = hkv; a.d = d;
            a.is_bf16 = dt == STAR_BF16; a.scale = scale; a.mode = 0;
            a.k = k; a.v = v; a.L = L; a.block = block; a.anchor = anchor;
            a.o = o; a.lse = lse;
            e = star::launch_row_attn(a, L, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "star_phase1_encode launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_phase1_encode: internal error");
    }
}

// ------------------------------------------------------------------------ Phase 2 partial
size_t star_phase2_workspace_bytes(int32_t rows, int64_t n_kv, int32_t hq, int32_t hkv, int32_t d) {
    if (rows < 1 || n_kv < 0 || hq < 1 || hkv < 1 || hq % hkv || d < 1) return 0;
    if (!star::attn_mfma_supported(d, hq, hkv)) return 0;
    star::PartPlan plan = {};
    plan.n_parts = 1;
    plan.n_kv[0] = n_kv;
    star::partial_mfma_plan(plan, rows, hq, hkv);
    const int32_t ns = plan.split_prefix[1];
    return ns > 1 ? partials_bytes(ns, (int64_t)hq * rows, d) : 0;
}

star_status_t star_phase2_partial(const void* q, int32_t rows, const void* k, const void* v,
                                  int64_t kv_head_stride, int64_t n_kv, int64_t causal_offset,
                                  int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt, float scale,
                                  float* a_out, float* m_out, float* l_out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    try {
        if (!q || !a_out || !m_out || !l_out) return fail(STAR_ERR_INVALID_ARG, "q, a_out, m_out, l_out must be non-null");
        if (n_kv > 0 && (!k || !v)) return fail(STAR_ERR_INVALID_ARG, "k and v must be non-null when n_kv > 0");
        if (rows < 1) return fail(STAR_ERR_INVALID_ARG, "rows (%d) must be >= 1", rows);
        if (n_kv < 0) return fail(STAR_ERR_INVALID_ARG, "n_kv must be >= 0");
        if (!(std::isfinite(scale) && scale >= 0.f)) return fail(STAR_ERR_INVALID_ARG, "scale must be finite and >= 0");
        star_status_t s = check_heads(hq, hkv, d, dt);
        if (s != STAR_OK) return s;
        if (hkv > 1 && kv_head_stride < n_kv * d)
            return fail(STAR_ERR_INVALID_ARG, "kv_head_stride (%lld) smaller than n_kv * d", (long long)kv_head_stride);
        if (kv_head_stride < 0) return fail(STAR_ERR_INVALID_ARG, "kv_head_stride must be >= 0");
        if (!aligned16(q) || (k && !aligned16(k)) || (v && !aligned16(v)) || !aligned16(a_out) ||
            (reinterpret_cast<uintptr_t>(m_out) & 3u) || (reinterpret_cast<uintptr_t>(l_out) & 3u) ||
            ((kv_head_stride * elem_bytes(dt)) % 16))
            return fail(STAR_ERR_INVALID_ARG, "pointers and the kv head stride must be 16-byte aligned");
        if (dt == STAR_BF16 && star::attn_mfma_supported(d, hq, hkv))
            return partial_mfma(q, rows, k, v, nullptr, nullptr, kv_head_stride, n_kv, causal_offset, hq, hkv, d,
                                scale, a_out, m_out, l_out, workspace, workspace_bytes, stream, "star_phase2_partial");
        star::RowAttnArgs a = {};
        a.q = q; a.q_rows = rows; a.hq = hq; a.hkv = hkv; a.d = d;
        a.is_bf16 = dt == STAR_BF16; a.scale = scale; a.mode = 1;
        a.n_seg = n_kv > 0 ? 1 : 0;
        a.seg[0].k = k; a.seg[0].v = v; a.seg[0].head_stride = kv_head_stride;
        a.seg[0].n = n_kv; a.seg[0].causal_lim = causal_offset;
        a.a_out = a_out; a.m_out = m_out; a.l_out = l_out;
        const hipError_t e = star::launch_row_attn(a, rows, stream);
        if (e != hipSuccess) return hip_fail(e, "star_phase2_partial launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_phase2_partial: internal error");
    }
}

star_status_t star_phase2_partial_kv8(const void* q, int32_t rows, const void* k8, const void* v8,
                                      const float* k_scale, const float* v_scale, int64_t kv_head_stride,
                                      int64_t n_kv, int64_t causal_offset, int32_t hq, int32_t hkv, int32_t d,
                                      star_dtype_t dt, float scale, float* a_out, float* m_out, float* l_out,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    try {
        if (!q || !a_out || !m_out || !l_out || !k_scale || !v_scale)
            return fail(STAR_ERR_INVALID_ARG, "q, the scales, a_out, m_out, l_out must be non-null");
        if (n_kv > 0 && (!k8 || !v8)) return fail(STAR_ERR_INVALID_ARG, "k8 and v8 must be non-null when n_kv > 0");
        if (rows < 1) return fail(STAR_ERR_INVALID_ARG, "rows (%d) must be >= 1", rows);
        if (n_kv < 0) return fail(STAR_ERR_INVALID_ARG, "n_kv must be >= 0");
        if (!(std::isfinite(scale) && scale >= 0.f)) return fail(STAR_ERR_INVALID_ARG, "scale must be finite and >= 0");
        star_status_t s = check_heads(hq, hkv, d, dt);
        if (s != STAR_OK) return s;
        if (kv_head_stride < 0) return fail(STAR_ERR_INVALID_ARG, "kv_head_stride must be >= 0");
        if (hkv > 1 && kv_head_stride < n_kv * d)
            return fail(STAR_ERR_INVALID_ARG, "kv_head_stride (%lld) smaller than n_kv * d", (long long)kv_head_stride);
        if (!aligned16(q) || (k8 && !aligned16(k8)) || (v8 && !aligned16(v8)) || !aligned16(a_out) ||
            (reinterpret_cast<uintptr_t>(m_out) & 3u) || (reinterpret_cast<uintptr_t>(l_out) & 3u) ||
            (reinterpret_cast<uintptr_t>(k_scale) & 3u) || (reinterpret_cast<uintptr_t>(v_scale) & 3u) ||
            (kv_head_stride % 16))
            return fail(STAR_ERR_INVALID_ARG,
                        "pointers and the kv head stride must be 16-byte aligned (scales, m and l 4-byte)");
        if (dt != STAR_BF16 || !star::attn_mfma_supported(d, hq, hkv))
            return fail(STAR_ERR_UNSUPPORTED, "E4M3 partial needs bf16, d = 64 or 128 and hq/hkv dividing 256");
        return partial_mfma(q, rows, k8, v8, k_scale, v_scale, kv_head_stride, n_kv, causal_offset, hq, hkv, d,
                            scale, a_out, m_out, l_out, workspace, workspace_bytes, stream, "star_phase2_partial_kv8");
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_phase2_partial_kv8: internal error");
    }
}

// ------------------------------------------------------------------------ Phase 2 query
size_t star_phase2_query_workspace_bytes(int32_t rows, int32_t n_shards, int32_t hq, int32_t hkv, int32_t d) {
    if (rows < 1 || n_shards < 1 || n_shards > 64 || hq < 1 || hkv < 1 || hq % hkv || d < 1) return 0;
    if (!star::attn_mfma_supported(d, hq, hkv)) return 0;
    return partials_bytes(star::partial_mfma_max_splits(rows, hq, hkv, n_shards + 1), (int64_t)hq * rows, d);
}

star_status_t star_phase2_query(const void* q, int32_t rows, const void* k_ctx, const void* v_ctx, int64_t L,
                                const int64_t* shard_bounds, int32_t n_shards, const void* k_tail,
                                const void* v_tail, int64_t tail_len, int64_t tail_cap, int32_t hq, int32_t hkv,
                                int32_t d, star_dtype_t dt, float scale, void* o, float* lse, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    try {
        if (!k_ctx || !v_ctx) return fail(STAR_ERR_INVALID_ARG, "required pointer is null");
        if (!aligned16(k_ctx) || !aligned16(v_ctx)) return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
        star_status_t s = check_query(q, rows, L, shard_bounds, n_shards, k_tail, v_tail, tail_len, tail_cap, hq, hkv,
                                      d, dt, scale, o, lse);
        if (s != STAR_OK) return s;
        const int64_t causal = tail_len - rows;   // row i sees query-host tokens t <= causal + i
        if (dt == STAR_BF16 && star::attn_mfma_supported(d, hq, hkv))
            return query_mfma(q, rows, k_ctx, v_ctx, nullptr, nullptr, L, shard_bounds, n_shards, k_tail, v_tail,
                              tail_len, tail_cap, hq, hkv, d, scale, o, lse, workspace, workspace_bytes, stream,
                              "star_phase2_query");
        star::RowAttnArgs a = {};
        a.q = q; a.q_rows = rows; a.hq = hq; a.hkv = hkv; a.d = d;
        a.is_bf16 = dt == STAR_BF16; a.scale = scale; a.mode = 1;
        a.n_seg = 2;
        a.seg[0].k = k_ctx; a.seg[0].v = v_ctx; a.seg[0].head_stride = L * d;
        a.seg[0].n = L; a.seg[0].causal_lim = -1;
        a.seg[1].k = k_tail; a.seg[1].v = v_tail; a.seg[1].head_stride = tail_cap * d;
        a.seg[1].n = tail_len; a.seg[1].causal_lim = causal;
        a.o = o; a.lse = lse;
        const hipError_t e = star::launch_row_attn(a, rows, stream);
        if (e != hipSuccess) return hip_fail(e, "star_phase2_query launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_phase2_query: internal error");
    }
}

star_status_t star_phase2_query_kv8(const void* q, int32_t rows, const void* k_ctx8, const void* v_ctx8,
                                    const float* k_scale, const float* v_scale, int64_t L,
                                    const int64_t* shard_bounds, int32_t n_shards, const void* k_tail,
                                    const void* v_tail, int64_t tail_len, int64_t tail_cap, int32_t hq, int32_t hkv,
                                    int32_t d, star_dtype_t dt, float scale, void* o, float* lse, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    try {
        if (!k_ctx8 || !v_ctx8 || !k_scale || !v_scale) return fail(STAR_ERR_INVALID_ARG, "required pointer is null");
        if (!aligned16(k_ctx8) || !aligned16(v_ctx8) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
            (reinterpret_cast<uintptr_t>(v_scale) & 3u))
            return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned (scales 4-byte)");
        star_status_t s = check_query(q, rows, L, shard_bounds, n_shards, k_tail, v_tail, tail_len, tail_cap, hq, hkv,
                                      d, dt, scale, o, lse);
        if (s != STAR_OK) return s;
        if (dt != STAR_BF16 || !star::attn_mfma_supported(d, hq, hkv))
            return fail(STAR_ERR_UNSUPPORTED, "E4M3 context query needs bf16, d = 64 or 128 and hq/hkv dividing 256");
        return query_mfma(q, rows, k_ctx8, v_ctx8, k_scale, v_scale, L, shard_bounds, n_shards, k_tail, v_tail,
                          tail_len, tail_cap, hq, hkv, d, scale, o, lse, workspace, workspace_bytes, stream,
                          "star_phase2_query_kv8");
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_phase2_query_kv8: internal error");
    }
}

// ------------------------------------------------------------------------ merge
star_status_t star_softmax_merge(const float* a, const float* m, const float* l, int32_t n_parts,
                                 int32_t hq, int32_t rows, int32_t d, void* o, star_dtype_t out_dt,
                                 float* lse_out, hipStream_t stream) {
    try {
        if (!a || !m || !l || !o) return fail(STAR_ERR_INVALID_ARG, "a, m, l and o must be non-null");
        if (n_parts < 1) return fail(STAR_ERR_INVALID_ARG, "n_parts must be >= 1");
        if (hq < 1 || rows < 1) return fail(STAR_ERR_INVALID_ARG, "hq and rows must be >= 1");
        if (out_dt != STAR_F32 && out_dt != STAR_BF16) return fail(STAR_ERR_INVALID_ARG, "unknown dtype");
        if (d < 4 || d % 4 || d > 1024) return fail(STAR_ERR_UNSUPPORTED, "merge needs d %% 4 == 0 and 4 <= d <= 1024");
        if (!aligned16(a) || !aligned16(o) || (reinterpret_cast<uintptr_t>(m) & 3u) ||
            (reinterpret_cast<uintptr_t>(l) & 3u) || (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)))
            return fail(STAR_ERR_INVALID_ARG, "a and o must be 16-byte aligned");
        hipError_t e = star::launch_merge(a, m, l, n_parts, (int64_t)hq * rows, d, o, out_dt == STAR_BF16,
                                          lse_out, nullptr, nullptr, stream);
        if (e != hipSuccess) return hip_fail(e, "star_softmax_merge launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_softmax_merge: internal error");
    }
}

// ------------------------------------------------------------------------ decode
size_t star_decode_workspace_bytes(int64_t L, int64_t tail_cap, int32_t n_shards, int32_t hq,
                                   int32_t hkv, int32_t d) {
    if (L < 1 || tail_cap < 1 || n_shards < 1 || n_shards > 64 || hq < 1 || hkv < 1 || hq % hkv || d < 1)
        return 0;
    return partials_bytes(star::decode_max_chunks(tail_cap, n_shards, hkv), hq, d) + round_up((size_t)hkv * 4);
}

star_status_t star_decode_step(const void* q_new, const void* k_new, const void* v_new,
                               const void* k_ctx, const void* v_ctx, int64_t L,
                               const int64_t* shard_bounds, int32_t n_shards,
                               void* k_tail, void* v_tail, int64_t tail_len, int64_t tail_cap,
                               int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt, float scale,
                               void* o, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    try {
        if (!k_ctx || !v_ctx) return fail(STAR_ERR_INVALID_ARG, "required pointer is null");
        if (!aligned16(k_ctx) || !aligned16(v_ctx)) return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
        star_status_t s = check_decode(q_new, k_new, v_new, L, shard_bounds, n_shards, k_tail, v_tail, tail_len,
                                       tail_cap, hq, hkv, d, dt, scale, o, lse);
        if (s != STAR_OK) return s;
        hipError_t e;
        if (dt == STAR_BF16 && star::decode_bf16_supported(d, hq, hkv)) {
            DecodeLaunch dl;
            s = plan_decode(shard_bounds, n_shards, tail_len, tail_cap, hq, hkv, d, workspace, workspace_bytes, &dl);
            if (s != STAR_OK) return s;
            e = star::launch_decode_bf16(static_cast<const uint16_t*>(q_new), static_cast<const uint16_t*>(k_new),
                                         static_cast<const uint16_t*>(v_new), static_cast<const uint16_t*>(k_ctx),
                                         static_cast<const uint16_t*>(v_ctx), nullptr, nullptr, nullptr, nullptr, L,
                                         static_cast<uint16_t*>(k_tail), static_cast<uint16_t*>(v_tail), tail_len,
                                         tail_cap, hq, hkv, d, scale, dl.plan, dl.a, dl.m, dl.l, dl.tickets,
                                         static_cast<uint16_t*>(o), lse, stream);
            if (e != hipSuccess) return hip_fail(e, "star_decode_step launch");
        } else {
            e = star::launch_tail_append(k_new, v_new, k_tail, v_tail, tail_len, tail_cap, hkv, d, elem_bytes(dt), stream);
            if (e != hipSuccess) return hip_fail(e, "star_decode_step append launch");
            star::RowAttnArgs a = {};
            a.q = q_new; a.q_rows = 1; a.hq = hq; a.hkv = hkv; a.d = d;
            a.is_bf16 = dt == STAR_BF16; a.scale = scale; a.mode = 1;
            a.n_seg = 2;
            a.seg[0].k = k_ctx; a.seg[0].v = v_ctx; a.seg[0].head_stride = L * d;
            a.seg[0].n = L; a.seg[0].causal_lim = -1;
            a.seg[1].k = k_tail; a.seg[1].v = v_tail; a.seg[1].head_stride = tail_cap * d;
            a.seg[1].n = tail_len + 1; a.seg[1].causal_lim = -1;
            a.o = o; a.lse = lse;
            e = star::launch_row_attn(a, 1, stream);
            if (e != hipSuccess) return hip_fail(e, "star_decode_step launch");
        }
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_decode_step: internal error");
    }
}

star_status_t star_decode_step_noalloc(const void* q_new, const void* k_new, const void* v_new,
                                       const void* k_ctx, const void* v_ctx, int64_t L,
                                       const int64_t* shard_bounds, int32_t n_shards,
                                       void* k_tail, void* v_tail, int64_t tail_len, int64_t tail_cap,
                                       int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt, float scale,
                                       void* o, float* lse, hipStream_t stream) {
    try {
        if (!k_ctx || !v_ctx) return fail(STAR_ERR_INVALID_ARG, "required pointer is null");
        if (!aligned16(k_ctx) || !aligned16(v_ctx)) return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
        star_status_t s = check_decode(q_new, k_new, v_new, L, shard_bounds, n_shards, k_tail, v_tail, tail_len,
                                       tail_cap, hq, hkv, d, dt, scale, o, lse);
        if (s != STAR_OK) return s;
        if (!(dt == STAR_BF16 && star::decode_bf16_supported(d, hq, hkv))) {
            // The vector path uses no scratch: the same launches as star_decode_step.
            return star_decode_step(q_new, k_new, v_new, k_ctx, v_ctx, L, shard_bounds, n_shards, k_tail, v_tail,
                                    tail_len, tail_cap, hq, hkv, d, dt, scale, o, lse, nullptr, 0, stream);
        }
        if (hkv > STAR_DECODE_NOALLOC_MAX_HKV)
            return fail(STAR_ERR_WORKSPACE, "star_decode_step_noalloc: hkv (%d) above %d", hkv,
                        STAR_DECODE_NOALLOC_MAX_HKV);
        const size_t need = partials_bytes(star::decode_max_chunks(tail_cap, n_shards, hkv), hq, d);
        if (need > kNoAllocScratchBytes - kNoAllocTicketBytes)
            return fail(STAR_ERR_WORKSPACE,
                        "star_decode_step_noalloc: this shape needs %zu bytes of chunk partials, above the %zu the "
                        "static scratch holds; use star_decode_step with a workspace",
                        need, kNoAllocScratchBytes - kNoAllocTicketBytes);
        void* base = nullptr;
        s = noalloc_scratch(&base);
        if (s != STAR_OK) return s;
        DecodeLaunch dl;
        s = plan_decode(shard_bounds, n_shards, tail_len, tail_cap, hq, hkv, d,
                        static_cast<char*>(base) + kNoAllocTicketBytes, kNoAllocScratchBytes - kNoAllocTicketBytes,
                        &dl, static_cast<unsigned*>(base));
        if (s != STAR_OK) return s;
        const hipError_t e = star::launch_decode_bf16(
            static_cast<const uint16_t*>(q_new), static_cast<const uint16_t*>(k_new),
            static_cast<const uint16_t*>(v_new), static_cast<const uint16_t*>(k_ctx),
            static_cast<const uint16_t*>(v_ctx), nullptr, nullptr, nullptr, nullptr, L,
            static_cast<uint16_t*>(k_tail), static_cast<uint16_t*>(v_tail), tail_len, tail_cap, hq, hkv, d, scale,
            dl.plan, dl.a, dl.m, dl.l, dl.tickets, static_cast<uint16_t*>(o), lse, stream);
        if (e != hipSuccess) return hip_fail(e, "star_decode_step_noalloc launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_decode_step_noalloc: internal error");
    }
}

// ------------------------------------------------------------------------ E4M3 context cache
star_status_t star_kv_fp8_scales(const void* x, int64_t tokens, int32_t hkv, int32_t d, star_dtype_t dt,
                                 float* scale, hipStream_t stream) {
    try {
        star_status_t s = check_kv_fp8(x, tokens, hkv, d, dt);
        if (s != STAR_OK) return s;
        if (!scale || (reinterpret_cast<uintptr_t>(scale) & 3u))
            return fail(STAR_ERR_INVALID_ARG, "scale must be a non-null, 4-byte aligned device pointer");
        hipError_t e = star::launch_kv_fp8_scales(x, tokens, hkv, d, dt == STAR_BF16, scale, stream);
        if (e != hipSuccess) return hip_fail(e, "star_kv_fp8_scales launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_kv_fp8_scales: internal error");
    }
}

star_status_t star_kv_quantize_fp8(const void* x, int64_t tokens, int32_t hkv, int32_t d, star_dtype_t dt,
                                   const float* scale, void* out, hipStream_t stream) {
    try {
        star_status_t s = check_kv_fp8(x, tokens, hkv, d, dt);
        if (s != STAR_OK) return s;
        if (!scale || (reinterpret_cast<uintptr_t>(scale) & 3u))
            return fail(STAR_ERR_INVALID_ARG, "scale must be a non-null, 4-byte aligned device pointer");
        if (!out || !aligned16(out)) return fail(STAR_ERR_INVALID_ARG, "out must be a non-null, 16-byte aligned device pointer");
        hipError_t e = star::launch_kv_quantize_fp8(x, tokens, hkv, d, dt == STAR_BF16, scale,
                                                    static_cast<uint8_t*>(out), stream);
        if (e != hipSuccess) return hip_fail(e, "star_kv_quantize_fp8 launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_kv_quantize_fp8: internal error");
    }
}

star_status_t star_decode_step_kv8(const void* q_new, const void* k_new, const void* v_new,
                                   const void* k_ctx8, const void* v_ctx8, const float* k_scale,
                                   const float* v_scale, int64_t L, const int64_t* shard_bounds, int32_t n_shards,
                                   void* k_tail, void* v_tail, int64_t tail_len, int64_t tail_cap,
                                   int32_t hq, int32_t hkv, int32_t d, star_dtype_t dt, float scale,
                                   void* o, float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    try {
        if (!k_ctx8 || !v_ctx8 || !k_scale || !v_scale) return fail(STAR_ERR_INVALID_ARG, "required pointer is null");
        if (!aligned16(k_ctx8) || !aligned16(v_ctx8) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
            (reinterpret_cast<uintptr_t>(v_scale) & 3u))
            return fail(STAR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned (scales 4-byte)");
        star_status_t s = check_decode(q_new, k_new, v_new, L, shard_bounds, n_shards, k_tail, v_tail, tail_len,
                                       tail_cap, hq, hkv, d, dt, scale, o, lse);
        if (s != STAR_OK) return s;
        if (dt != STAR_BF16 || !star::decode_bf16_supported(d, hq, hkv))
            return fail(STAR_ERR_UNSUPPORTED, "E4M3 context decode needs bf16, d = 64 or 128 and hq/hkv in {1,2,4,8,16}");
        DecodeLaunch dl;
        s = plan_decode(shard_bounds, n_shards, tail_len, tail_cap, hq, hkv, d, workspace, workspace_bytes, &dl);
        if (s != STAR_OK) return s;
        hipError_t e = star::launch_decode_bf16(
            static_cast<const uint16_t*>(q_new), static_cast<const uint16_t*>(k_new),
            static_cast<const uint16_t*>(v_new), nullptr, nullptr, static_cast<const uint8_t*>(k_ctx8),
            static_cast<const uint8_t*>(v_ctx8), k_scale, v_scale, L, static_cast<uint16_t*>(k_tail),
            static_cast<uint16_t*>(v_tail), tail_len, tail_cap, hq, hkv, d, scale, dl.plan, dl.a, dl.m, dl.l,
            dl.tickets, static_cast<uint16_t*>(o), lse, stream);
        if (e != hipSuccess) return hip_fail(e, "star_decode_step_kv8 launch");
        return ok();
    } catch (...) {
        return fail(STAR_ERR_HIP, "star_decode_step_kv8: internal error");
    }
}

}  // extern "C"
