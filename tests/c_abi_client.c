/* A plain C99 client of the attention library: it includes the public
 * header, links libfa.so and makes only calls that the library answers
 * before any device call (argument checks, sizes, empty problems), so it
 * runs on a machine without a GPU.  Prints "ok" and exits 0 on success. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int failures = 0;

#define CHECK(cond)                                                  \
    do {                                                             \
        if (!(cond)) {                                               \
            printf("failed: %s (line %d)\n", #cond, __LINE__);       \
            ++failures;                                              \
        }                                                            \
    } while (0)

static fa_params_t params(int64_t B, int64_t H, int64_t N, int64_t d) {
    fa_params_t p;
    memset(&p, 0, sizeof p);
    p.B = B;
    p.H = H;
    p.N = N;
    p.d = d;
    p.dtype = FA_BF16;
    p.causal = 1;
    p.scale = 0.125f;
    return p;
}

int main(void) {
    /* never dereferenced: every call below is refused or has nothing to do */
    void *fake = (void *)(uintptr_t)0x10000;
    fa_params_t p;

    CHECK(sizeof(fa_params_t) == 64);
    CHECK(offsetof(fa_params_t, seed) == 48 && offsetof(fa_params_t, Nk) == 60);
    CHECK(fa_status_str(FA_OK) != NULL && fa_status_str(FA_EINVAL) != NULL);

    /* empty problems: FA_OK, no launch, no workspace */
    p = params(0, 2, 16, 64);
    CHECK(fa_fwd(&p, NULL, NULL, NULL, NULL, NULL, NULL) == FA_OK);
    CHECK(fa_bwd_workspace_bytes(&p) == 0);

    /* workspace of a real problem: two fp32 row arrays, 256-byte aligned */
    p = params(2, 3, 100, 128);
    CHECK(fa_bwd_workspace_bytes(&p) == 2 * ((2 * 3 * 100 * 4 + 255) / 256 * 256));

    /* refused before any device call */
    p = params(1, 2, 16, 80);
    CHECK(fa_fwd(&p, fake, fake, fake, fake, fake, NULL) == FA_EUNSUPPORTED);
    CHECK(fa_bwd_workspace_bytes(&p) == (size_t)-1);
    p = params(1, 2, 16, 64);
    p.scale = -1.0f;
    CHECK(fa_fwd(&p, fake, fake, fake, fake, fake, NULL) == FA_EINVAL);
    CHECK(strlen(fa_last_error()) > 0);
    p = params(1, 2, 16, 64);
    CHECK(fa_fwd(&p, NULL, fake, fake, fake, fake, NULL) == FA_EINVAL);
    p = params(1, 2, 16, 64);
    p.dropout_p = 1e-6f;   /* threshold rounds to zero */
    CHECK(fa_fwd(&p, fake, fake, fake, fake, fake, NULL) == FA_EUNSUPPORTED);

    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
