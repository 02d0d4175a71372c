/*
 * abi_sanitize_driver.c -- the host side of libqsa under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_abi_sanitizers.py). Every entry point
 * is called with arguments the library must reject before any device work
 * (NULL or misaligned pointers, negative, overflowing or unsupported sizes), with zero-size calls that are no-ops, and through the workspace-size
 * helpers; each returned status and message is checked. No call reaches a GPU.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qsa.h"

static int fails = 0;

static void expect(qsa_status got, qsa_status want, const char *what)
{
    const char *msg = qsa_last_error();
    if (got != want || (want != QSA_OK && (msg == NULL || msg[0] == '\0'))) {
        fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, msg ? msg : "(null)");
        ++fails;
    }
}

#define FAKE ((void *)(uintptr_t)0x10000)       /* 256-byte aligned, never dereferenced */
#define AT(off) ((void *)((uintptr_t)0x10000 + (off)))

int main(void)
{
    /* attention: records and fused */
    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 0, 12, 128, 0.1f, FAKE, NULL), QSA_OK,
           "attn T = 0");
    expect(qsa_attn(NULL, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 4, 12, 128, 0.1f, FAKE, NULL), QSA_ERR_ARG,
           "attn NULL q");
    expect(qsa_attn(AT(8), FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 4, 12, 128, 0.1f, FAKE, NULL), QSA_ERR_ARG,
           "attn misaligned q");
    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 65, 10, 4, 12, 128, 0.1f, FAKE, NULL), QSA_ERR_ARG,
           "attn ids_stride % 64");
    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 64, 10, 4, 12, 128, 0.1f, FAKE, NULL), QSA_ERR_ARG,
           "attn n_cells < 0");
    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 4, 12, 64, 0.1f, FAKE, NULL),
           QSA_ERR_UNSUPPORTED, "attn D = 64");
    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 4, 17, 128, 0.1f, FAKE, NULL),
           QSA_ERR_UNSUPPORTED, "attn H = 17");
    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, -1, 4, 12, 128, 0.1f, FAKE, NULL), QSA_ERR_ARG,
           "attn pos0 < 0");
    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 2147483646, 4, 12, 128, 0.1f, FAKE, NULL),
           QSA_ERR_ARG, "attn pos0 + T overflows");
    expect(qsa_attn_merge(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 0, 12, 128, 0.1f, FAKE, NULL), QSA_OK,
           "attn_merge T = 0");
    expect(qsa_attn_merge(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 4, 12, 128, 0.1f, NULL, NULL),
           QSA_ERR_ARG, "attn_merge NULL out");
    expect(qsa_attn_merge(FAKE, FAKE, NULL, FAKE, FAKE, 100, FAKE, 64, 10, 4, 12, 128, 0.1f, FAKE, NULL),
           QSA_ERR_ARG, "attn_merge NULL vq");

    /* merge */
    expect(qsa_merge(FAKE, 3, 0, 12, 128, FAKE, NULL), QSA_OK, "merge T = 0");
    expect(qsa_merge(FAKE, -1, 4, 12, 128, FAKE, NULL), QSA_ERR_ARG, "merge n_chunks < 0");
    expect(qsa_merge(AT(128), 3, 4, 12, 128, FAKE, NULL), QSA_ERR_ARG, "merge misaligned part");
    expect(qsa_merge(FAKE, 3, 4, 12, 96, FAKE, NULL), QSA_ERR_UNSUPPORTED, "merge D = 96");
    expect(qsa_merge(FAKE, 3, 4, 0, 128, FAKE, NULL), QSA_ERR_ARG, "merge H = 0");

    expect(qsa_attn(FAKE, FAKE, FAKE, FAKE, FAKE, 13, FAKE, 64, 10, 4, 12, 128, 0.1f, FAKE, NULL), QSA_ERR_ARG,
           "attn n_cells < pos0 + T");

    /* gated merge and gated fused attention */
    expect(qsa_merge_gated(FAKE, 3, 0, 12, 128, FAKE, FAKE, FAKE, NULL), QSA_OK, "merge_gated T = 0");
    expect(qsa_merge_gated(FAKE, 3, 4, 12, 128, NULL, FAKE, FAKE, NULL), QSA_ERR_ARG, "merge_gated NULL gate");
    expect(qsa_merge_gated(FAKE, 3, 4, 12, 128, AT(8), FAKE, FAKE, NULL), QSA_ERR_ARG,
           "merge_gated misaligned gate");
    expect(qsa_merge_gated(FAKE, 3, 4, 12, 128, FAKE, FAKE, AT(2), NULL), QSA_ERR_ARG,
           "merge_gated misaligned sums");
    expect(qsa_attn_merge_gated(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 0, 12, 128, 0.1f, FAKE, FAKE,
                                NULL, NULL), QSA_OK, "attn_merge_gated T = 0");
    expect(qsa_attn_merge_gated(FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 64, 10, 4, 12, 128, 0.1f, NULL, FAKE,
                                NULL, NULL), QSA_ERR_ARG, "attn_merge_gated NULL gate");
    expect(qsa_attn_merge_gated(FAKE, FAKE, FAKE, FAKE, FAKE, 13, FAKE, 64, 10, 4, 12, 128, 0.1f, FAKE, FAKE,
                                NULL, NULL), QSA_ERR_ARG, "attn_merge_gated n_cells < pos0 + T");

    /* score */
    expect(qsa_score(FAKE, FAKE, 100, 10, 0, 12, 128, 1.0f, -1.0f, FAKE, 100, NULL), QSA_OK, "score T = 0");
    expect(qsa_score(FAKE, FAKE, 100, 10, 4, 12, 128, 1.0f, -1.0f, FAKE, 13, NULL), QSA_ERR_ARG,
           "score row_stride < pos0 + T");
    expect(qsa_score(FAKE, FAKE, 100, 10, 4, 0, 128, 1.0f, -1.0f, FAKE, 100, NULL), QSA_ERR_ARG,
           "score Hs = 0");
    expect(qsa_score(FAKE, FAKE, 100, 10, 4, 17, 128, 1.0f, -1.0f, FAKE, 100, NULL), QSA_ERR_UNSUPPORTED,
           "score Hs = 17");
    expect(qsa_score(AT(4), FAKE, 100, 10, 4, 12, 128, 1.0f, -1.0f, FAKE, 100, NULL), QSA_ERR_ARG,
           "score misaligned q");
    expect(qsa_score_ws_bytes(65) == 65536 ? QSA_OK : QSA_ERR_ARG, QSA_OK, "score workspace bytes");
    expect(qsa_score_ws(FAKE, FAKE, 100, 10, 0, 12, 128, 1.0f, -1.0f, FAKE, 100, NULL, 0, NULL), QSA_OK,
           "score_ws T = 0");
    expect(qsa_score_ws(FAKE, FAKE, 100, 10, 4, 12, 128, 1.0f, -1.0f, FAKE, 100, FAKE, 32767, NULL), QSA_ERR_ARG,
           "score_ws short workspace");
    expect(qsa_score_ws(FAKE, FAKE, 100, 10, 4, 12, 128, 1.0f, -1.0f, FAKE, 100, NULL, 32768, NULL), QSA_ERR_ARG,
           "score_ws NULL workspace");
    expect(qsa_score_ws(FAKE, FAKE, 100, 10, 4, 12, 128, 1.0f, -1.0f, FAKE, 100, AT(8), 32768, NULL), QSA_ERR_ARG,
           "score_ws misaligned workspace");

    /* cache writer */
    expect(qsa_quant_append(FAKE, FAKE, 0, 128, FAKE, FAKE, FAKE, FAKE, 0, 10, NULL), QSA_OK, "quant n_rows = 0");
    expect(qsa_quant_append(FAKE, FAKE, 8, 128, FAKE, FAKE, FAKE, FAKE, 5, 10, NULL), QSA_ERR_ARG,
           "quant past the cache");
    expect(qsa_quant_append(FAKE, FAKE, 8, 100, FAKE, FAKE, FAKE, FAKE, 0, 10, NULL), QSA_ERR_UNSUPPORTED,
           "quant D = 100");
    expect(qsa_quant_append(FAKE, NULL, 8, 128, FAKE, FAKE, FAKE, FAKE, 0, 10, NULL), QSA_ERR_ARG, "quant NULL v");

    /* selection */
    expect(qsa_select(FAKE, 100, 10, 0, 5, FAKE, 64, NULL), QSA_OK, "select T = 0");
    expect(qsa_select(FAKE, 100, 10, 4, 0, FAKE, 64, NULL), QSA_ERR_ARG, "select K = 0");
    expect(qsa_select(FAKE, 200, 100, 4, 100, FAKE, 64, NULL), QSA_ERR_ARG, "select id row too short");
    expect(qsa_select(FAKE, 33554440, 33554430, 4, 100, FAKE, 128, NULL), QSA_ERR_UNSUPPORTED, "select row too long");
    expect(qsa_select(FAKE, 13, 10, 4, 5, FAKE, 64, NULL), QSA_ERR_ARG, "select row_stride < pos0 + T");

    /* workspace helpers */
    size_t o = 1, m = 1, l = 1;
    qsa_part_offsets(1984, 12, 128, 33, &o, &m, &l);
    if (o != 0 || m % 256 != 0 || l % 256 != 0 || l <= m || qsa_part_bytes(1984, 12, 128, 33) <= l) {
        fprintf(stderr, "part layout\n");
        ++fails;
    }
    qsa_part_offsets(3, 5, 128, 7, NULL, &m, NULL);
    if (qsa_part_bytes(-1, 1, 128, 1) != 0) {
        fprintf(stderr, "part bytes of a negative shape\n");
        ++fails;
    }

    if (fails) {
        fprintf(stderr, "%d ABI checks failed\n", fails);
        return 1;
    }
    printf("abi sanitizer driver: ok\n");
    return 0;
}
