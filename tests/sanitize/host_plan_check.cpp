// Host-side planning and argument checks of libstarattn, built on their own with a host
// compiler and AddressSanitizer / UndefinedBehaviorSanitizer (tests/test_sanitized_host.py).
//
// Exercises the decode chunk plan, the Phase-2 split plan and every shared argument check
// over seeded random shapes of the kind the GPU sweep uses, plus the edges: 64 shards, empty
// shards, an empty query-host cache (tail_len = 0), contexts at the 2^24-token limit, bad
// arguments of every kind.  Each plan is checked against its own invariants: the chunks of
// every shard and of the query host tile their key ranges exactly (mapped the way the decode
// kernel maps a chunk index), counts stay under the bounds the workspace sizes are built
// from, and every pointer carved from a workspace lies inside it.  Exit status 0 and a
// final "ok" line mean every check passed and no sanitizer fired.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "host_plan.h"

using namespace star;

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            std::fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond);   \
            std::exit(1);                                                            \
        }                                                                            \
    } while (0)

namespace {

std::mt19937_64 rng(20241203);
int64_t uni(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }

// Never dereferenced: the checks only look at values and alignment.
const void* fake(uintptr_t a) { return reinterpret_cast<const void*>(a); }
const void* const P = fake(0x100000);

std::vector<int64_t> random_bounds(int64_t L, int S, bool allow_empty) {
    std::vector<int64_t> b(S + 1);
    b[0] = 0;
    b[S] = L;
    std::vector<int64_t> cuts;
    for (int i = 0; i < S - 1; ++i) cuts.push_back(allow_empty ? uni(0, L) : uni(1, L > 1 ? L - 1 : 1));
    std::sort(cuts.begin(), cuts.end());
    for (int i = 0; i < S - 1; ++i) b[i + 1] = cuts[i];
    return b;
}

// The decode chunk plan of one call, checked the way the kernel reads it.
void check_decode_plan(const std::vector<int64_t>& bounds, int64_t tail_len, int64_t tail_cap, int hq, int hkv,
                       int d) {
    const int S = (int)bounds.size() - 1;
    const int64_t L = bounds[S];
    const size_t ws_bytes = host::partials_bytes(decode_max_chunks(tail_cap, S, hkv), hq, d) + host::round_up((size_t)hkv * 4);
    std::vector<unsigned char> buf(ws_bytes + 256);
    void* ws = buf.data() + (256 - (reinterpret_cast<uintptr_t>(buf.data()) & 255)) % 256;
    host::DecodeLaunch dl;
    CHECK(host::plan_decode(bounds.data(), S, tail_len, tail_cap, hq, hkv, d, ws, ws_bytes, &dl) == STAR_OK);
    const DecodeChunkPlan& p = dl.plan;
    CHECK(p.n_shards == S);
    CHECK(p.chunk >= 128 && p.chunk % 128 == 0);
    CHECK(p.n_chunks >= 1 && p.n_chunks <= decode_max_chunks(tail_cap, S, hkv));
    // map every chunk index to its key range as the kernel does, and tile the partitions
    std::vector<int64_t> covered(S + 1, 0);
    for (int c = 0; c < p.n_chunks; ++c) {
        int64_t lo, hi;
        int part;
        if (c < p.chunk_prefix[S]) {
            int r = 0;
            while (c >= p.chunk_prefix[r + 1]) ++r;
            CHECK(r < S);
            lo = p.shard_lo[r] + (int64_t)(c - p.chunk_prefix[r]) * p.chunk;
            hi = lo + p.chunk < p.shard_lo[r + 1] ? lo + p.chunk : p.shard_lo[r + 1];
            CHECK(lo == bounds[r] + covered[r]);
            part = r;
            CHECK(hi <= bounds[r + 1]);
        } else {
            const int64_t tc = c - p.chunk_prefix[S];
            lo = tc * p.chunk;
            hi = lo + p.chunk < tail_len + 1 ? lo + p.chunk : tail_len + 1;
            CHECK(lo == covered[S]);
            part = S;
        }
        CHECK(hi > lo);
        covered[part] += hi - lo;
    }
    for (int r = 0; r < S; ++r) CHECK(covered[r] == bounds[r + 1] - bounds[r]);
    CHECK(covered[S] == tail_len + 1);
    CHECK(p.shard_lo[S] == L);
    // carved pointers inside the workspace
    const char* w0 = static_cast<const char*>(ws);
    const char* w1 = w0 + ws_bytes;
    CHECK(reinterpret_cast<const char*>(dl.a) >= w0);
    CHECK(reinterpret_cast<const char*>(dl.a + (size_t)p.n_chunks * hq * d) <= reinterpret_cast<const char*>(dl.m));
    CHECK(reinterpret_cast<const char*>(dl.m + (size_t)p.n_chunks * hq) <= reinterpret_cast<const char*>(dl.l));
    CHECK(reinterpret_cast<const char*>(dl.l + (size_t)p.n_chunks * hq) <= w1);
    CHECK(reinterpret_cast<const char*>(dl.tickets) >= reinterpret_cast<const char*>(dl.l + (size_t)p.n_chunks * hq));
    CHECK(reinterpret_cast<const char*>(dl.tickets + hkv) <= w1);
    CHECK((reinterpret_cast<uintptr_t>(dl.a) & 255) == 0 && (reinterpret_cast<uintptr_t>(dl.m) & 255) == 0);
    // a workspace one byte short, a misaligned one and none at all are refused
    CHECK(host::plan_decode(bounds.data(), S, tail_len, tail_cap, hq, hkv, d, ws, ws_bytes - 1, &dl) == STAR_ERR_WORKSPACE);
    CHECK(host::plan_decode(bounds.data(), S, tail_len, tail_cap, hq, hkv, d, static_cast<char*>(ws) + 8, ws_bytes, &dl) ==
          STAR_ERR_WORKSPACE);
    CHECK(host::plan_decode(bounds.data(), S, tail_len, tail_cap, hq, hkv, d, nullptr, ws_bytes, &dl) == STAR_ERR_WORKSPACE);
    // counters kept elsewhere: the workspace then holds the partials only
    unsigned tickets[1];
    const size_t part_only = host::partials_bytes(decode_max_chunks(tail_cap, S, hkv), hq, d);
    CHECK(host::plan_decode(bounds.data(), S, tail_len, tail_cap, hq, hkv, d, ws, part_only, &dl, tickets) == STAR_OK);
    CHECK(dl.tickets == tickets);
}

// The Phase-2 split plan over random partitions.
void check_split_plan(int n_parts, int rows, int hq, int hkv, int64_t max_kv) {
    PartPlan plan = {};
    plan.n_parts = n_parts;
    for (int i = 0; i < n_parts; ++i) plan.n_kv[i] = uni(0, 9) == 0 ? 0 : uni(1, max_kv);
    const int nrt = partial_mfma_plan(plan, rows, hq, hkv);
    const int G = hq / hkv;
    CHECK(nrt == (rows + kAttnQueriesPerGroup / G - 1) / (kAttnQueriesPerGroup / G));
    CHECK(plan.split_len >= 8 * kAttnKeysPerTile && plan.split_len % kAttnKeysPerTile == 0);
    CHECK(plan.split_prefix[0] == 0);
    for (int i = 0; i < n_parts; ++i) {
        const int ns = plan.split_prefix[i + 1] - plan.split_prefix[i];
        CHECK(ns >= 1);
        CHECK((int64_t)ns * plan.split_len >= plan.n_kv[i]);
        CHECK(ns == 1 || (int64_t)(ns - 1) * plan.split_len < plan.n_kv[i]);
    }
    CHECK(plan.split_prefix[n_parts] <= partial_mfma_max_splits(rows, hq, hkv, n_parts));
}

void check_arguments() {
    const int64_t b3[] = {0, 50, 100};
    const float* lse = nullptr;
    // decode: good, then every kind of bad argument
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, 0, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_OK);
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, 7, 8, 4, 2, 128, STAR_BF16, 0.0f, P, lse) == STAR_OK);
    CHECK(host::check_decode(nullptr, P, P, 100, b3, 2, P, P, 0, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, 8, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, -1, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 0, P, P, 0, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 65, P, P, 0, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 99, b3, 2, P, P, 0, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, 0, 8, 4, 2, 128, STAR_BF16, -0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, 0, 8, 4, 2, 128, STAR_BF16, NAN, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, 0, 8, 5, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_decode(P, P, P, 100, b3, 2, P, P, 0, 8, 4, 2, 130, STAR_BF16, 0.1f, P, lse) == STAR_ERR_UNSUPPORTED);
    CHECK(host::check_decode(fake(0x100008), P, P, 100, b3, 2, P, P, 0, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) ==
          STAR_ERR_INVALID_ARG);
    const int64_t bad[] = {0, 60, 50};
    CHECK(host::check_decode(P, P, P, 50, bad, 2, P, P, 0, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    // 64 shards, most of them empty
    std::vector<int64_t> b64(65, 0);
    for (int i = 60; i <= 64; ++i) b64[i] = 10 * (i - 59);
    CHECK(host::check_decode(P, P, P, 50, b64.data(), 64, P, P, 0, 1, 4, 2, 64, STAR_BF16, 0.1f, P, lse) == STAR_OK);
    // query phase
    CHECK(host::check_query(P, 8, 100, b3, 2, P, P, 8, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_OK);
    CHECK(host::check_query(P, 0, 100, b3, 2, P, P, 8, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_query(P, 8, 100, b3, 2, P, P, 7, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_query(P, 8, 100, b3, 2, P, P, 9, 8, 4, 2, 128, STAR_BF16, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_query(P, 8, 100, b3, 2, P, P, 8, 8, 4, 2, 128, STAR_BF16, -1.f, P, lse) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_query(P, 8, 100, b3, 2, P, P, 8, 8, 4, 2, 128, (star_dtype_t)7, 0.1f, P, lse) == STAR_ERR_INVALID_ARG);
    // E4M3 cache arguments
    CHECK(host::check_kv_fp8(P, 0, 8, 128, STAR_BF16) == STAR_OK);
    CHECK(host::check_kv_fp8(P, -1, 8, 128, STAR_BF16) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_kv_fp8(P, 10, 70000, 128, STAR_BF16) == STAR_ERR_INVALID_ARG);
    CHECK(host::check_kv_fp8(P, 10, 8, 100, STAR_BF16) == STAR_ERR_UNSUPPORTED);
    CHECK(host::check_kv_fp8(fake(0x100004), 10, 8, 128, STAR_F32) == STAR_ERR_INVALID_ARG);
    // a message longer than the formatting buffer is cut, not overrun
    const std::string huge(4000, 'x');
    CHECK(host::fail(STAR_ERR_HIP, "%s", huge.c_str()) == STAR_ERR_HIP);
    CHECK(std::strlen(host::last_error()) < 512);
    CHECK(host::ok() == STAR_OK && host::last_error()[0] == '\0');
}

}  // namespace

int main() {
    check_arguments();
    int n_decode = 0, n_split = 0;
    // seeded random decode shapes (GQA groups, head dims, shards with empty ones, tails)
    for (int it = 0; it < 3000; ++it) {
        const int hkv = (int)uni(1, 8);
        const int G = 1 << uni(0, 4);
        const int d = uni(0, 1) ? 128 : 64;
        const int64_t L = uni(0, 3) == 0 ? uni(1, 200) : uni(1, (int64_t)1 << uni(10, 24));
        const int S = (int)uni(1, 64);
        const int64_t tail_cap = uni(1, 5000);
        const int64_t tail_len = uni(0, 2) == 0 ? 0 : uni(0, tail_cap - 1);
        check_decode_plan(random_bounds(L, S, true), tail_len, tail_cap, hkv * G, hkv, d);
        ++n_decode;
    }
    // the edges named above, and the workloads' own layouts
    std::vector<int64_t> b64(65);
    for (int i = 0; i <= 64; ++i) b64[i] = i < 63 ? 0 : (i == 63 ? 1 : 2);
    check_decode_plan(b64, 0, 1, 32, 8, 128);
    for (int i = 0; i <= 64; ++i) b64[i] = (int64_t)i * (((int64_t)1 << 24) / 64);
    check_decode_plan(b64, 0, 4096, 16, 1, 128);
    const int64_t w1m[] = {0, 65536, 131072, 196608, 262144, 327680, 393216, 458752, 524288, 589824, 655360,
                           720896, 786432, 851968, 917504, 983040, 1048576};
    check_decode_plan(std::vector<int64_t>(w1m, w1m + 17), 159, 160, 32, 8, 128);
    check_decode_plan(std::vector<int64_t>{0, 8192, 16384, 24576, 32768}, 0, 160, 32, 8, 128);
    check_decode_plan(std::vector<int64_t>{0, 16384, 32768, 49152, 65536, 81920, 98304, 114688, 131072}, 319, 320, 64, 8,
                      128);
    // Phase-2 split plans
    for (int it = 0; it < 3000; ++it) {
        const int hkv = (int)uni(1, 8);
        const int Gs[] = {1, 2, 4, 8, 16, 32, 64, 128, 256};
        const int G = Gs[uni(0, 8)];
        check_split_plan((int)uni(1, kMaxParts), (int)uni(1, 600), hkv * G, hkv, uni(1, (int64_t)1 << uni(6, 24)));
        ++n_split;
    }
    CHECK(attn_mfma_supported(128, 32, 8) && attn_mfma_supported(64, 256, 1) && !attn_mfma_supported(96, 4, 1));
    CHECK(!attn_mfma_supported(128, 3 * 2, 2) && decode_bf16_supported(128, 16, 1) && !decode_bf16_supported(128, 32, 1));
    CHECK(attn_mfma_max_tokens(128) == ((int64_t)1 << 24));
    std::printf("ok: %d decode plans, %d split plans, argument checks\n", n_decode, n_split);
    return 0;
}
