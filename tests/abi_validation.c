/*
 * Host-side validation of every librd entry point, for the sanitizer build
 * (address + undefined-behaviour sanitizers on the library's host code and
 * on this driver).  Only calls that return before anything reaches the
 * device are made: invalid arguments, empty batches, the size queries that
 * reject their arguments, the status strings, the knobs and the debug
 * switch.  Prints "ok" and exits 0 when every status is the documented one.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rd.h"

static int failures = 0;

#define EXPECT(call, want)                                                        \
    do {                                                                          \
        const long long got_ = (long long)(call);                                 \
        if (got_ != (long long)(want)) {                                          \
            fprintf(stderr, "%s:%d: %s -> %lld, want %lld\n", __FILE__, __LINE__, \
                    #call, got_, (long long)(want));                              \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

int main(void) {
    void *f = (void *)(uintptr_t)0x1000; /* never dereferenced on the host */
    int32_t *fi = (int32_t *)f;
    uint32_t *fu = (uint32_t *)f;

    for (int s = 0; s >= RD_E_SCRATCH; --s) {
        const char *msg = rd_status_string(s);
        if (!msg || strncmp(msg, "RD_", 3) != 0) {
            fprintf(stderr, "status string %d: %s\n", s, msg ? msg : "(null)");
            ++failures;
        }
    }
    EXPECT(strcmp(rd_status_string(7), "unknown rd status"), 0);
    EXPECT(rd_version() >= 100, 1);

    /* pack / mask */
    EXPECT(rd_pack_beams(NULL, -1, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL), RD_E_ARG);
    EXPECT(rd_pack_beams(NULL, 0, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL), RD_OK);
    EXPECT(rd_pack_beams(NULL, 2, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL), RD_E_ARG);
    EXPECT(rd_pack_beams(fi, 2, 65, 4, fi, fi, fi, NULL, NULL, NULL), RD_E_UNSUPPORTED);
    EXPECT(rd_pack_beams(fi, 2, 4, 17, fi, fi, fi, NULL, NULL, NULL), RD_E_UNSUPPORTED);
    EXPECT(rd_pack_beams_mask(fi, 2, 4, 4, fi, fi, fi, NULL, NULL, NULL, NULL), RD_E_ARG);
    EXPECT(rd_pack_beams_mask(NULL, 3, 0, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL), RD_OK);
    EXPECT(rd_pack_beams_mask_ragged(fi, NULL, fi, 2, 4, 4, fi, fi, fi, NULL, NULL, fu, NULL), RD_E_ARG);
    EXPECT(rd_tree_mask(NULL, NULL, 2, -3, 4, NULL, NULL), RD_E_ARG);
    EXPECT(rd_tree_mask(fi, fi, 2, 4, 17, fu, NULL), RD_E_UNSUPPORTED);

    /* attention */
    EXPECT(rd_tree_attention(7, f, f, f, f, f, fi, fu, fi, 2, 8, 4, 4, 128, 64, 0.f, f, f, 0, NULL),
           RD_E_UNSUPPORTED);
    EXPECT(rd_tree_attention(1, f, f, f, f, f, fi, fu, fi, 2, 8, 4, 4, 96, 64, 0.f, f, f, 0, NULL),
           RD_E_UNSUPPORTED);
    EXPECT(rd_tree_attention(1, f, f, f, f, f, fi, fu, fi, 2, 8, 6, 4, 128, 64, 0.f, f, f, 0, NULL), RD_E_ARG);
    EXPECT(rd_tree_attention(1, f, f, f, f, f, fi, fu, fi, 2, 8, 4, 4, 128, 64, -1.f, f, f, 0, NULL), RD_E_ARG);
    EXPECT(rd_tree_attention(1, f, f, f, f, f, fi, fu, fi, 0, 8, 4, 4, 128, 64, 0.f, f, f, 0, NULL), RD_OK);
    EXPECT(rd_tree_attention(1, NULL, f, f, f, f, fi, fu, fi, 2, 8, 4, 4, 128, 64, 0.f, f, f, 0, NULL), RD_E_ARG);
    EXPECT(rd_tree_attention(1, f, f, f, f, f, fi, fu, fi, 2, 2048, 4, 4, 128, 64, 0.f, f, f, 0, NULL),
           RD_E_UNSUPPORTED);
    EXPECT(rd_tree_attention_workspace_size(1, 2, 8, 6, 4, 128, 64), 0);
    EXPECT(rd_tree_attention_paged(1, f, f, f, f, f, 8, 32, fi, 4, fi, fu, fi, 2, 8, 4, 4, 128, 0.f, f, f,
                                   1 << 20, NULL),
           RD_E_UNSUPPORTED);
    EXPECT(rd_tree_attention_paged(1, f, f, f, f, f, 8, 0, fi, 4, fi, fu, fi, 2, 8, 4, 4, 128, 0.f, f, f,
                                   1 << 20, NULL),
           RD_E_ARG);
    EXPECT(rd_tree_attention_paged(1, f, f, f, f, f, 8, 64, NULL, 4, fi, fu, fi, 2, 8, 4, 4, 128, 0.f, f, f,
                                   1 << 20, NULL),
           RD_E_ARG);
    EXPECT(rd_tree_attention_paged(1, f, f, f, f, f, 8, 64, fi, 4, fi, fu, fi, 0, 8, 4, 4, 128, 0.f, f, f, 0,
                                   NULL),
           RD_OK);

    /* projection */
    EXPECT(rd_lm_head_argmax(1, f, fi, f, 2, 8, 100, 50, f, fi, f, 1 << 20, NULL), RD_E_UNSUPPORTED);
    EXPECT(rd_lm_head_argmax(5, f, fi, f, 2, 8, 128, 50, f, fi, f, 1 << 20, NULL), RD_E_UNSUPPORTED);
    EXPECT(rd_lm_head_argmax(1, f, fi, f, 0, 8, 128, 50, f, fi, f, 0, NULL), RD_OK);
    EXPECT(rd_lm_head_argmax(1, f, fi, f, 2, 8, 0, 50, f, fi, f, 1 << 20, NULL), RD_E_ARG);
    EXPECT(rd_lm_head_workspace_size(1, -1, 8, 128, 50), 0);
    EXPECT(rd_lm_head_argmax_unpack(1, NULL, NULL, NULL, NULL, 0, 4, 3, 128, 50, NULL, NULL, NULL, 0, NULL), RD_OK);
    EXPECT(rd_lm_head_argmax_unpack(1, f, fi, f, fi, 2, 65, 3, 128, 50, f, fi, f, 1 << 20, NULL), RD_E_UNSUPPORTED);
    EXPECT(rd_lm_head_argmax_unpack(1, f, fi, f, NULL, 2, 4, 3, 128, 50, f, fi, f, 1 << 20, NULL), RD_E_ARG);
    EXPECT(rd_lm_head_argmax_unpack(1, f, fi, f, fi, 2, 4, -3, 128, 50, f, fi, f, 1 << 20, NULL), RD_E_ARG);
    EXPECT(rd_lm_head_argmax_unpack(1, f, fi, f, fi, 2, 4, 3, 128, 50, f, fi, f, 16, NULL), RD_E_WORKSPACE);
    EXPECT(rd_lm_head_argmax_unpack_workspace_size(1, 2, 4, 3, 128, 50) >
               rd_lm_head_workspace_size(1, 2, 12, 128, 50), 1);
    EXPECT(rd_lm_head_argmax_unpack_workspace_size(1, 2, 65, 3, 128, 50), 0);
    EXPECT(rd_lm_head_argmax_noalloc(1, f, fi, f, 2, 8, 100, 50, f, fi, NULL), RD_E_UNSUPPORTED);
    EXPECT(rd_lm_head_argmax_noalloc(1, f, fi, f, 0, 8, 128, 50, f, fi, NULL), RD_OK);
    EXPECT(rd_lm_head_argmax_noalloc(1, NULL, fi, f, 2, 8, 128, 50, f, fi, NULL), RD_E_ARG);
    EXPECT(rd_lm_head_workspace_size(1, 2, 40000, 4096, 32000) > RD_NOALLOC_SCRATCH_BYTES, 1);
    EXPECT(rd_lm_head_argmax_noalloc(1, f, fi, f, 2, 40000, 4096, 32000, f, fi, NULL), RD_E_SCRATCH);

    /* unpack / accept */
    EXPECT(rd_unpack_accept(NULL, NULL, NULL, NULL, NULL, 1, 8, 2, 4, 0, NULL, NULL, NULL, NULL, NULL), RD_OK);
    EXPECT(rd_unpack_accept(fi, fi, fi, f, f, 9, 8, 2, 4, 3, fi, fi, fi, fi, NULL), RD_E_UNSUPPORTED);
    EXPECT(rd_unpack_accept(fi, fi, fi, f, f, 1, -8, 2, 4, 3, fi, fi, fi, fi, NULL), RD_E_ARG);
    EXPECT(rd_unpack_accept_ragged(fi, NULL, fi, fi, fi, f, f, 1, 8, 2, 4, 3, fi, fi, fi, fi, NULL), RD_E_ARG);

    /* stochastic accept */
    EXPECT(rd_stochastic_accept(5, fi, fi, fi, f, (float *)f, (float *)f, (float *)f, 2, 8, 5, 1000, fi, fi, fi,
                                NULL, f, 1 << 20, NULL),
           RD_E_UNSUPPORTED);
    EXPECT(rd_stochastic_accept(1, fi, fi, fi, f, NULL, (float *)f, (float *)f, 2, 8, 5, 1000, fi, fi, fi, NULL,
                                f, 1 << 20, NULL),
           RD_E_ARG);
    EXPECT(rd_stochastic_accept(1, fi, fi, fi, f, (float *)f, (float *)f, (float *)f, 2, 8, 5, 1000, fi, fi, fi,
                                NULL, f, 16, NULL),
           RD_E_WORKSPACE);
    EXPECT(rd_stochastic_accept_workspace_size(2, 8, 5), 2 * 40 * 12);
    EXPECT(rd_stochastic_accept_workspace_size(2, 65, 5), 0);

    /* commit */
    EXPECT(rd_commit_accepted(1, fi, fi, fi, f, f, f, 0, 8, 5, 32, 128, 4096, 1024, f, f, fi, f, NULL), RD_OK);
    EXPECT(rd_commit_accepted(1, fi, fi, fi, f, f, f, 2, 8, 5, 32, 128, 4096, 1024, NULL, f, fi, f, NULL),
           RD_E_ARG);
    EXPECT(rd_commit_accepted(1, fi, fi, fi, f, f, f, 2, 8, 5, 32, 128, 4096, 1024, f, f, fi, NULL, NULL),
           RD_E_ARG);
    EXPECT(rd_commit_accepted(1, fi, fi, fi, f, f, f, 2, 8, 5, 0, 128, 4096, 1024, f, f, fi, f, NULL), RD_E_ARG);
    EXPECT(rd_commit_accepted(3, fi, fi, fi, f, f, f, 2, 8, 5, 32, 128, 4096, 1024, f, f, fi, f, NULL),
           RD_E_UNSUPPORTED);
    EXPECT(rd_commit_accepted(1, fi, fi, fi, f, f, f, 2, 8, 17, 32, 128, 4096, 1024, f, f, fi, f, NULL),
           RD_E_UNSUPPORTED);
    EXPECT(rd_commit_accepted_paged(1, fi, fi, fi, f, f, f, 2, 8, 5, 32, 128, 4096, f, f, 16, 0, fi, 4, fi, f,
                                    NULL),
           RD_E_ARG);
    EXPECT(rd_commit_accepted_paged(1, fi, fi, fi, f, f, f, 2, 8, 5, 32, 128, 4096, f, f, 16, 64, NULL, 4, fi, f,
                                    NULL),
           RD_E_ARG);

    /* knobs and the debug switch */
    EXPECT(rd_set_knob(RD_KNOB_ATTN_SPLITS, 5), 0);
    EXPECT(rd_set_knob(RD_KNOB_ATTN_SPLITS, 0), 5);
    EXPECT(rd_set_knob(RD_KNOB_COUNT, 1), RD_E_ARG);
    EXPECT(rd_set_knob(RD_KNOB_LM_SHAPE, -1), RD_E_ARG);
    const int prev = rd_set_debug(1);
    EXPECT(rd_set_debug(prev), 1);

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
