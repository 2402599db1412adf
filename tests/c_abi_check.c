/* Plain C99 consumer of include/pgemm.h: compiled with gcc and linked
 * against libpgemm.so by tests/test_abi.py.  It calls only entry points
 * whose argument checks fail (or that are host-only), so it needs no GPU:
 * every check runs on the host before any HIP call. */
#include <stdio.h>
#include <string.h>

#include "pgemm.h"

#define EXPECT(expr, want)                                                  \
    do {                                                                    \
        long long got_ = (long long)(expr);                                 \
        if (got_ != (long long)(want)) {                                    \
            fprintf(stderr, "%s: got %lld, want %lld\n", #expr, got_,       \
                    (long long)(want));                                     \
            return 1;                                                       \
        }                                                                   \
    } while (0)

int main(void) {
    char* p = (char*)0x10000000;  /* never dereferenced */
    int64_t head = 0;
    int hv = 0, tv = 0;
    EXPECT(pgemm_f16(p, p + 0x1000000, p + 0x2000000, -1, 8, 8, NULL), PGEMM_EINVAL);
    EXPECT(pgemm_f16(p, p + 0x1000000, p + 0x2000000, 8, 12, 8, NULL), PGEMM_EUNSUPPORTED);
    EXPECT(pgemm_f16(NULL, NULL, NULL, 0, 8, 8, NULL), PGEMM_OK);
    EXPECT(pgemm_f16_variant(p, p, p, 8, 8, 8, -1, NULL), PGEMM_EUNSUPPORTED);
    EXPECT(pgemm_f16_num_variants() >= 8, 1);
    EXPECT(pgemm_f16_choose_variant(4096, 4096, 4096) >= 1, 1);
    EXPECT(pgemm_f16_plan(4096, 4096, 4096, 256, &head, &hv, &tv), PGEMM_OK);
    EXPECT(head, 4096);
    EXPECT(pgemm_f16_splitk(p, p, p, 64, 64, 512, 0, NULL, 0, NULL), PGEMM_EUNSUPPORTED);
    EXPECT(pgemm_f16_splitk_noalloc(p, p + 0x10000000, p + 0x20000000, 2048, 2048, 40960, 5, NULL),
           PGEMM_ESCRATCH);
    EXPECT(pgemm_f16_splitk_workspace_bytes(2048, 2048, 32768, 4), 4LL * 2048 * 2048 * 4);
    EXPECT(pgemm_f16_splitk_workspace_bytes(2048, 2048, 32768, 4) <= PGEMM_STATIC_SCRATCH_BYTES, 1);
    EXPECT(pgemm_f16_splitk_default_splits(2048, 2048, 32768), 4);
    EXPECT(pstream_add((const float*)p, NULL, (float*)p, 4, NULL), PGEMM_EINVAL);
    EXPECT(pstream_add_blocked((const float*)p, (const float*)p, (float*)p, 0, 1000, NULL),
           PGEMM_EUNSUPPORTED);
    EXPECT(pstream_add_scalar(NULL, 1.0f, NULL, 0, NULL), PGEMM_OK);
    EXPECT(preduce_sum_f32(NULL, (float*)p, 8, 8, NULL), PGEMM_EINVAL);
    EXPECT(pgemm_test_fill_f32(NULL, 42.0f, 4, NULL), PGEMM_EINVAL);
    EXPECT(pgemm_test_iota_f32((float*)p, -1, NULL), PGEMM_EINVAL);
    EXPECT(strcmp(pgemm_status_string(PGEMM_OK), "ok"), 0);
    EXPECT(pgemm_last_hip_error(), 0);
    EXPECT(pgemm_version() >= 100, 1);
    printf("c abi ok\n");
    return 0;
}
