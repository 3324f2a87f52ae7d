// Exercise the argument checks of every C-ABI entry point (include/tsd_attn.h) without a GPU, so that a
// build of the host code with AddressSanitizer and UndefinedBehaviorSanitizer sees each path: invalid
// arguments must return ATTN_EINVAL or ATTN_EUNSUPPORTED with a message, empty shapes ATTN_OK, and calls
// that pass every check reach the (stubbed) launchers and return ATTN_EHIP. Test infrastructure, built
// and run by tests/test_sanitizers.py with sanitize_stubs.cpp in place of the kernels.
#include "tsd_attn.h"

#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int fails = 0;
#define EXPECT(call, want)                                                                                     \
    do {                                                                                                       \
        const attn_status_t got_ = (call);                                                                     \
        if (got_ != (want)) {                                                                                  \
            fprintf(stderr, "line %d: %s -> %d, want %d (%s)\n", __LINE__, #call, (int)got_, (int)(want),      \
                    attn_last_error());                                                                        \
            ++fails;                                                                                           \
        } else if (got_ != ATTN_OK && attn_last_error()[0] == '\0') {                                          \
            fprintf(stderr, "line %d: %s failed without a message\n", __LINE__, #call);                      \
            ++fails;                                                                                           \
        }                                                                                                      \
    } while (0)

static void *fake(int i) { return (void *)(uintptr_t)((1u << 20) + (uintptr_t)i * (1u << 28)); }

int main()
{
    const float s = 0.125f;
    int32_t *vl = (int32_t *)fake(9);
    // attn_fwd / attn_fwd_ex
    EXPECT(attn_fwd(fake(0), fake(1), fake(2), 0, nullptr, s, fake(3), 1, 1, 8, 8, 64, 1, 1, nullptr), ATTN_EHIP);
    EXPECT(attn_fwd(nullptr, fake(1), fake(2), 0, nullptr, s, fake(3), 1, 1, 8, 8, 64, 1, 1, nullptr), ATTN_EINVAL);
    EXPECT(attn_fwd(fake(0), fake(1), fake(2), 9, nullptr, s, fake(3), 1, 1, 8, 8, 64, 1, 1, nullptr), ATTN_EINVAL);
    EXPECT(attn_fwd(fake(0), fake(1), fake(2), 1, nullptr, s, fake(3), 1, 1, 8, 9, 64, 1, 1, nullptr),
           ATTN_EUNSUPPORTED);
    EXPECT(attn_fwd(fake(0), fake(1), fake(2), 0, nullptr, s, fake(3), 1, 1, 0, 8, 64, 1, 1, nullptr), ATTN_OK);
    EXPECT(attn_fwd_ex(fake(0), fake(1), fake(2), 3, vl, s, fake(3), (float *)fake(4), 2, 4, 2, 8, 8, 128, 1, 0,
                       nullptr), ATTN_EHIP);
    EXPECT(attn_fwd_ex(fake(0), fake(1), fake(2), 0, nullptr, s, fake(3), (float *)fake(0), 2, 4, 2, 8, 8, 128, 1,
                       0, nullptr), ATTN_EINVAL);
    EXPECT(attn_fwd_ex(fake(0), fake(1), fake(2), 0, nullptr, s, fake(3), nullptr, 2, 4, 3, 8, 8, 128, 1, 0,
                       nullptr), ATTN_EINVAL);
    EXPECT(attn_fwd(fake(0), fake(1), fake(2), 0, nullptr, s, fake(3), 1, 1, 8, 8, 32, 0, 0, nullptr), ATTN_EHIP);
    EXPECT(attn_fwd(fake(0), fake(1), fake(2), 0, nullptr, s, fake(3), 1, 1, 8, 8, 48, 0, 0, nullptr),
           ATTN_EUNSUPPORTED);
    // attn_weights
    EXPECT(attn_weights(fake(0), fake(1), 0, nullptr, s, (float *)fake(2), 1, 2, 2, 8, 8, 64, 1, nullptr),
           ATTN_EHIP);
    EXPECT(attn_weights(fake(0), fake(1), 0, nullptr, s, (float *)fake(2), 1, 2, 2, 8, 2000, 64, 1, nullptr),
           ATTN_EUNSUPPORTED);
    EXPECT(attn_weights(fake(0), fake(1), 2, nullptr, s, (float *)fake(2), 1, 2, 2, 8, 8, 64, 1, nullptr),
           ATTN_EINVAL);
    EXPECT(attn_weights(fake(0), fake(1), 0, nullptr, s, (float *)fake(2), 1, 2, 2, 0, 8, 64, 1, nullptr), ATTN_OK);
    // attn_bwd / attn_bwd_noalloc
    void *b[10];
    for (int i = 0; i < 10; ++i) b[i] = fake(i);
    const size_t ws = attn_bwd_workspace_bytes(1, 4, 8);
    EXPECT(attn_bwd(b[0], b[1], b[2], b[3], b[4], (float *)b[5], 0, nullptr, s, b[6], b[7], b[8], 1, 4, 2, 8, 8, 64,
                    1, b[9], ws, nullptr), ATTN_EHIP);
    EXPECT(attn_bwd(b[0], b[1], b[2], b[3], b[4], (float *)b[5], 0, nullptr, s, b[6], b[7], b[8], 1, 4, 2, 8, 8, 64,
                    1, b[9], ws - 1, nullptr), ATTN_EINVAL);
    EXPECT(attn_bwd(b[0], b[1], b[2], b[3], b[4], (float *)b[5], 0, nullptr, s, b[0], b[7], b[8], 1, 4, 2, 8, 8, 64,
                    1, b[9], ws, nullptr), ATTN_EINVAL);
    EXPECT(attn_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, s, nullptr, nullptr, nullptr, 0,
                    4, 2, 8, 8, 64, 1, nullptr, 0, nullptr), ATTN_OK);
    EXPECT(attn_bwd_noalloc(b[0], b[1], b[2], b[3], b[4], (float *)b[5], 0, nullptr, s, b[6], b[7], b[8], 1, 32, 32,
                            40000, 8, 64, 1, nullptr), ATTN_EINVAL);
    EXPECT(attn_bwd_noalloc(b[0], b[1], b[2], b[3], b[4], (float *)b[5], 0, nullptr, s, b[6], b[7], b[8], 1, 4, 2, 8,
                            8, 64, 1, nullptr), ATTN_EHIP);
    if (attn_bwd_noalloc_max_scratch_bytes() != ((size_t)8 << 20)) ++fails;
    // mha_fwd
    const size_t mws = mha_workspace_bytes(1, 16, 512, 8, 1);
    EXPECT(mha_fwd(fake(0), fake(1), fake(2), 8, fake(3), 1, 16, 512, 1, fake(4), mws, nullptr), ATTN_EHIP);
    EXPECT(mha_fwd(fake(0), fake(1), fake(2), 7, fake(3), 1, 16, 512, 1, fake(4), mws, nullptr), ATTN_EINVAL);
    EXPECT(mha_fwd(fake(0), fake(1), fake(2), 8, fake(3), 1, 16, 512, 1, fake(4), mws - 2, nullptr), ATTN_EINVAL);
    EXPECT(mha_fwd(fake(0), fake(1), fake(2), 8, fake(3), 0, 16, 512, 1, fake(4), mws, nullptr), ATTN_OK);
    // mha_cross_fwd
    const size_t cws = mha_cross_workspace_bytes(2, 16, 24, 512, 8, 1);
    EXPECT(mha_cross_fwd(fake(0), fake(1), fake(2), fake(3), 8, 2, vl, fake(4), 2, 16, 24, 512, 1, fake(5), cws,
                         nullptr), ATTN_EHIP);
    EXPECT(mha_cross_fwd(fake(0), fake(1), fake(2), fake(3), 8, 1, nullptr, fake(4), 2, 16, 24, 512, 1, fake(5), cws,
                         nullptr), ATTN_EUNSUPPORTED);
    EXPECT(mha_cross_fwd(fake(0), fake(1), fake(2), fake(3), 8, 0, nullptr, fake(4), 2, 16, 24, 512, 1, fake(5),
                         cws - 1, nullptr), ATTN_EINVAL);
    EXPECT(mha_cross_fwd(fake(0), nullptr, fake(2), fake(3), 8, 0, nullptr, fake(4), 2, 16, 0, 512, 1, fake(5), cws,
                         nullptr), ATTN_EHIP);
    for (int st = -1; st < 5; ++st)
        if (!attn_status_string(st) || !strlen(attn_status_string(st))) ++fails;
    if (fails) return 1;
    printf("C-ABI driver: all checks passed\n");
    return 0;
}
