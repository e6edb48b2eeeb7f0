/*
 * A plain C99 consumer of include/star_attn.h, linked against libstarattn.so.
 * It calls only entry points that finish on the host: the status strings, the
 * version, the workspace-size queries and argument checks that fail before any
 * HIP call.  Built and run by tests/test_abi_c_consumer.py; prints one line per
 * check and exits non-zero on the first mismatch.
 */
#include <stdio.h>
#include <string.h>

#include "star_attn.h"

static int failures = 0;

static void expect(int cond, const char *what) {
    printf("%s %s\n", cond ? "ok  " : "FAIL", what);
    if (!cond) failures++;
}

int main(void) {
    /* Never dereferenced: every call below is rejected by its argument checks. */
    void *fake = (void *)(uintptr_t)0x100000;
    const int64_t bounds[3] = {0, 50, 100};
    const int64_t bad_bounds[3] = {0, 60, 50};

    expect(strcmp(star_status_str(STAR_OK), "STAR_OK") == 0, "status string of STAR_OK");
    expect(strcmp(star_status_str(STAR_ERR_WORKSPACE), "STAR_ERR_WORKSPACE") == 0, "status string of STAR_ERR_WORKSPACE");
    expect(star_version() != NULL && strchr(star_version(), '.') != NULL, "version string");

    expect(star_decode_workspace_bytes(32768, 160, 4, 32, 8, 128) > 0, "decode workspace size");
    expect(star_decode_workspace_bytes(0, 160, 4, 32, 8, 128) == 0, "decode workspace size of an empty context");
    expect(star_phase2_query_workspace_bytes(128, 4, 32, 8, 128) > 0, "query workspace size");
    expect(star_phase2_workspace_bytes(128, 8192, 32, 8, 128) > 0, "partial workspace size");

    expect(star_phase1_encode(NULL, fake, fake, fake, NULL, 64, 32, 32, 4, 2, 128, STAR_BF16, 0.1f, 0) ==
               STAR_ERR_INVALID_ARG, "phase 1 rejects a null q");
    expect(strlen(star_last_error()) > 0, "the last error names the reason");
    expect(star_phase1_encode(fake, fake, fake, fake, NULL, 64, 32, 33, 4, 2, 128, STAR_BF16, 0.1f, 0) ==
               STAR_ERR_INVALID_ARG, "phase 1 rejects anchor > block");
    expect(star_phase1_encode(fake, fake, fake, fake, NULL, 64, 32, 32, 4, 2, 130, STAR_BF16, 0.1f, 0) ==
               STAR_ERR_UNSUPPORTED, "phase 1 rejects head dim 130");
    expect(star_decode_step(fake, fake, fake, fake, fake, 100, bad_bounds, 2, fake, fake, 0, 8, 4, 2, 128,
                            STAR_BF16, 0.1f, fake, NULL, fake, (size_t)1 << 30, 0) == STAR_ERR_INVALID_ARG,
           "decode rejects non-monotone shard bounds");
    expect(star_decode_step(fake, fake, fake, fake, fake, 100, bounds, 2, fake, fake, 0, 8, 4, 2, 128,
                            STAR_BF16, 0.1f, fake, NULL, fake, 16, 0) == STAR_ERR_WORKSPACE,
           "decode rejects a short workspace");
    expect(star_decode_step_kv8(fake, fake, fake, fake, fake, fake, fake, 100, bounds, 2, fake, fake, 0, 8, 4, 2, 96,
                                STAR_BF16, 0.1f, fake, NULL, fake, (size_t)1 << 30, 0) == STAR_ERR_UNSUPPORTED,
           "E4M3 decode rejects head dim 96");
    expect(star_phase2_query_kv8(fake, 8, fake, fake, (const float *)fake, (const float *)fake, 100, bounds, 2, fake,
                                 fake, 8, 8, 4, 2, 128, STAR_F32, 0.1f, fake, NULL, fake, (size_t)1 << 30, 0) ==
               STAR_ERR_UNSUPPORTED,
           "E4M3 query rejects fp32");
    expect(star_kv_fp8_scales(fake, 100, 8, 100, STAR_BF16, (float *)fake, 0) == STAR_ERR_UNSUPPORTED,
           "E4M3 scales reject d % 8 != 0");
    expect(star_softmax_merge((const float *)fake, (const float *)fake, (const float *)fake, 0, 4, 1, 128, fake,
                              STAR_BF16, NULL, 0) == STAR_ERR_INVALID_ARG, "merge rejects zero partials");
    return failures ? 1 : 0;
}
