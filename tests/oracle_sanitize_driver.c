/*
 * oracle_sanitize_driver.c -- runs every oracle entry point on small inputs
 * that reach its edge cases, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py). A sanitizer
 * report aborts the run; the driver itself checks only return codes and that
 * every written value is finite or an intended sentinel.
 *
 * Cases: poisoned slots (-1, negative, at and past n_cells), an empty chunk, a
 * row with no valid slot, a ragged last chunk, implicit all-causal rows,
 * scores with a clipped dead-key tail, quantisation of zero, huge, subnormal
 * and tied groups, selection with K above and below the row length, gates at
 * 0, +-inf, +-100 and NaN on outputs at the binary16 limits, per-16 sums over
 * infinities and signed zeros, and rejected shapes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double qso_half_to_double(uint16_t h);
uint16_t qso_double_to_half(double x);
int qso_attn_chunks(const uint16_t *q, const int8_t *kq, const int8_t *vq, const uint16_t *ksc, const uint16_t *vsc,
                    int32_t n_cells, const int32_t *ids, int32_t ids_stride, int32_t pos0, int32_t T, int32_t H,
                    int32_t D, double scale, int32_t t_begin, int32_t t_end, double *m, double *l, double *o,
                    double *oabs);
int qso_merge(const double *m, const double *l, const double *o, int32_t C, int32_t T, int32_t H, int32_t D,
              int32_t t_begin, int32_t t_end, double *out64, uint16_t *out16);
int qso_score(const float *q, const float *k, int32_t n_cells, int32_t pos0, int32_t T, int32_t Hs, int32_t D,
              double scale, double dead, double *scores, int64_t row_stride, int32_t t_begin, int32_t t_end);
int qso_quant_rows(const float *x, int32_t n_rows, int32_t D, int8_t *codes, uint16_t *scales);
int qso_select(const float *scores, int64_t row_stride, int32_t pos0, int32_t T, int32_t K, int32_t *ids,
               int32_t ids_stride, int32_t t_begin, int32_t t_end);
int qso_gate(const double *y, const float *gate, int64_t n, double *out64, uint16_t *out16);
int qso_sums16(const uint16_t *x, int64_t n_rows, int32_t D, float *sums);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng_state >> 32);
}
static double next_unit(void) { return (next_u32() + 0.5) / 4294967296.0; }

static int fails = 0;
#define CHECK(cond, what)                                      \
    do {                                                       \
        if (!(cond)) {                                         \
            fprintf(stderr, "driver check failed: %s\n", what); \
            ++fails;                                           \
        }                                                      \
    } while (0)

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    return p;
}

static void attention_cases(void)
{
    const int32_t T = 6, H = 3, D = 128, n_cells = 150, pos0 = 140, C = 3;
    uint16_t *q = xmalloc(sizeof(uint16_t) * T * H * D);
    int8_t *kq = xmalloc((size_t)n_cells * D), *vq = xmalloc((size_t)n_cells * D);
    uint16_t *ksc = xmalloc(sizeof(uint16_t) * n_cells * (D / 32)), *vsc = xmalloc(sizeof(uint16_t) * n_cells * (D / 32));
    for (int i = 0; i < T * H * D; ++i)
        q[i] = qso_double_to_half(2.0 * next_unit() - 1.0);
    for (int i = 0; i < n_cells * D; ++i) {
        kq[i] = (int8_t)((int)(next_u32() % 255u) - 127);
        vq[i] = (int8_t)((int)(next_u32() % 255u) - 127);
    }
    for (int i = 0; i < n_cells * (D / 32); ++i) {
        ksc[i] = qso_double_to_half(1e-3 + 0.019 * next_unit());
        vsc[i] = qso_double_to_half(1e-3 + 0.019 * next_unit());
    }
    int32_t *ids = xmalloc(sizeof(int32_t) * T * 64 * C);
    for (int t = 0; t < T; ++t)
        for (int s = 0; s < 64 * C; ++s) {
            const uint32_t r = next_u32() % 10u;
            ids[t * 64 * C + s] = r == 0 ? -1 : r == 1 ? n_cells : r == 2 ? -7 : r == 3 ? n_cells + 1000
                                                    : (int32_t)(next_u32() % (uint32_t)(pos0 + t + 1));
        }
    for (int s = 64; s < 128; ++s)
        ids[1 * 64 * C + s] = -1;                    /* an empty chunk */
    for (int s = 0; s < 64 * C; ++s)
        ids[2 * 64 * C + s] = -1;                    /* a row with no valid slot */
    for (int s = 128; s < 192; ++s)
        ids[3 * 64 * C + s] = s < 131 ? pos0 + 3 - (s - 128) : -1;   /* a ragged last chunk */

    const size_t nrec = (size_t)T * C * H;
    double *m = xmalloc(sizeof(double) * nrec), *l = xmalloc(sizeof(double) * nrec);
    double *o = xmalloc(sizeof(double) * nrec * D), *oabs = xmalloc(sizeof(double) * nrec * D);
    for (size_t i = 0; i < nrec * D; ++i)
        o[i] = oabs[i] = -12345.0;                   /* sentinel: left as it was for empty chunks */
    CHECK(qso_attn_chunks(q, kq, vq, ksc, vsc, n_cells, ids, 64 * C, pos0, T, H, D, 0.08838834764831845, 0, T, m, l,
                          o, oabs) == 0, "attn_chunks explicit");
    double *out64 = xmalloc(sizeof(double) * T * H * D);
    uint16_t *out16 = xmalloc(sizeof(uint16_t) * T * H * D);
    CHECK(qso_merge(m, l, o, C, T, H, D, 0, T, out64, out16) == 0, "merge explicit");
    for (int i = 0; i < T * H * D; ++i)
        CHECK(isfinite(out64[i]), "finite merged output");

    /* implicit all-causal rows: C = ceil((pos0 + T) / 64) */
    const int32_t Ci = (pos0 + T + 63) / 64;
    const size_t nreci = (size_t)T * Ci * H;
    double *mi = xmalloc(sizeof(double) * nreci), *li = xmalloc(sizeof(double) * nreci);
    double *oi = xmalloc(sizeof(double) * nreci * D), *oai = xmalloc(sizeof(double) * nreci * D);
    CHECK(qso_attn_chunks(q, kq, vq, ksc, vsc, n_cells, NULL, 0, pos0, T, H, D, 0.0625, 0, T, mi, li, oi, oai) == 0,
          "attn_chunks implicit");
    CHECK(qso_merge(mi, li, oi, Ci, T, H, D, 0, T, out64, NULL) == 0, "merge implicit");

    /* rejected shapes */
    CHECK(qso_attn_chunks(q, kq, vq, ksc, vsc, n_cells, ids, 64 * C, pos0, T, H, 100, 0.1, 0, T, m, l, o, oabs) != 0,
          "attn_chunks rejects D % 32 != 0");
    CHECK(qso_merge(m, l, o, -1, T, H, D, 0, T, out64, out16) != 0, "merge rejects C < 0");

    free(q); free(kq); free(vq); free(ksc); free(vsc); free(ids);
    free(m); free(l); free(o); free(oabs); free(out64); free(out16);
    free(mi); free(li); free(oi); free(oai);
}

static void score_cases(void)
{
    const int32_t T = 5, Hs = 2, D = 128, pos0 = 60, n_cells = 70;
    const int64_t row_stride = 66;                   /* clips the dead-key tail of the last rows */
    float *q = xmalloc(sizeof(float) * T * Hs * D), *k = xmalloc(sizeof(float) * n_cells * D);
    for (int i = 0; i < T * Hs * D; ++i)
        q[i] = (float)(2.0 * next_unit() - 1.0);
    for (int i = 0; i < n_cells * D; ++i)
        k[i] = (float)(2.0 * next_unit() - 1.0);
    double *s = xmalloc(sizeof(double) * T * row_stride);
    for (int i = 0; i < T * row_stride; ++i)
        s[i] = 7.0;                                  /* untouched cells keep it */
    CHECK(qso_score(q, k, n_cells, pos0, T, Hs, D, 1.0, -INFINITY, s, row_stride, 0, T) == 0, "score");
    CHECK(qso_score(q, k, n_cells, pos0, T, Hs, D, 1.0, -INFINITY, s, pos0 + T - 1, 0, T) != 0,
          "score rejects a short row");
    free(q); free(k); free(s);
}

static void quant_cases(void)
{
    const int32_t n = 6, D = 128;
    float *x = xmalloc(sizeof(float) * n * D);
    for (int i = 0; i < n * D; ++i)
        x[i] = (float)(4.0 * next_unit() - 2.0);
    for (int d = 0; d < 32; ++d) {
        x[0 * D + d] = 0.0f;                         /* an all-zero group */
        x[1 * D + d] = 1e30f * (d % 2 ? 1.0f : -1.0f);   /* a scale past the fp16 range */
        x[2 * D + d] = 1e-42f * (float)d;            /* subnormal inputs */
        x[3 * D + d] = (float)((d - 15) + 0.5) * 0.25f;  /* ties at half-integers of the step */
    }
    int8_t *codes = xmalloc((size_t)n * D);
    uint16_t *scales = xmalloc(sizeof(uint16_t) * n * (D / 32));
    CHECK(qso_quant_rows(x, n, D, codes, scales) == 0, "quant_rows");
    CHECK(qso_quant_rows(x, n, 100, codes, scales) != 0, "quant_rows rejects D % 32 != 0");
    free(x); free(codes); free(scales);
}

static void select_cases(void)
{
    const int32_t T = 4, pos0 = 300;
    const int64_t row_stride = pos0 + T + 5;
    float *s = xmalloc(sizeof(float) * T * row_stride);
    for (int i = 0; i < T * row_stride; ++i) {
        const uint32_t r = next_u32() % 8u;
        s[i] = r == 0 ? 0.0f : r == 1 ? -0.0f : r == 2 ? 1.25f : (float)(2.0 * next_unit() - 1.0);
    }
    const int32_t Ks[3] = {1, 64, 1000};             /* the last one is above every row's length */
    for (int i = 0; i < 3; ++i) {
        const int32_t K = Ks[i];
        const int32_t take = K < pos0 + T ? K : pos0 + T;
        const int32_t stride = 64 * ((take + 63) / 64);
        int32_t *ids = xmalloc(sizeof(int32_t) * T * stride);
        CHECK(qso_select(s, row_stride, pos0, T, K, ids, stride, 0, T) == 0, "select");
        for (int t = 0; t < T; ++t)
            for (int j = 1; j < stride; ++j)
                if (ids[t * stride + j] >= 0)
                    CHECK(ids[t * stride + j] > ids[t * stride + j - 1], "ascending ids");
        free(ids);
    }
    int32_t small[64];
    CHECK(qso_select(s, row_stride, pos0, T, 100, small, 64, 0, T) != 0, "select rejects a short id row");
    free(s);
}

static void gate_cases(void)
{
    const int n = 12;
    const double y[12] = {1.0, -1.0, 0.0, -0.0, 65504.0, -65504.0, 1e5, 3e-8, 0.25, -0.75, 7.0, 2.0};
    const float g[12] = {0.0f, 0.0f, 1.0f, -1.0f, INFINITY, -INFINITY, 100.0f, -100.0f, NAN, 2.5f, -2.5f, 1e-30f};
    double out64[12];
    uint16_t out16[12];
    CHECK(qso_gate(y, g, n, out64, out16) == 0, "gate");
    CHECK(out64[0] == 0.5 && out64[1] == -0.5, "sigmoid(0) halves");
    CHECK(out64[4] == 65504.0 && out16[4] == 0x7bff, "sigmoid(+inf) keeps the value");
    CHECK(out64[5] == 0.0 && signbit(out64[5]), "sigmoid(-inf) gives a zero of the value's sign");
    CHECK(out64[8] != out64[8], "NaN gate gives NaN");
    CHECK(qso_gate(y, g, n, NULL, NULL) == 0, "gate with no outputs");
    CHECK(qso_gate(y, g, -1, out64, out16) != 0, "gate rejects n < 0");

    uint16_t x[3 * 32];
    for (int i = 0; i < 3 * 32; ++i)
        x[i] = (uint16_t)(next_u32() & 0xffffu);
    for (int i = 0; i < 16; ++i)
        x[i] = (uint16_t)(i & 1 ? 0x8000u : 0x0000u);   /* signed zeros only */
    x[20] = 0x7c00u;                                     /* +inf */
    x[21] = 0xfc00u;                                     /* -inf */
    float sums[3 * 2];
    CHECK(qso_sums16(x, 3, 32, sums) == 0, "sums16");
    CHECK(sums[0] == 0.0f, "sum of signed zeros");
    CHECK(qso_sums16(x, 3, 24, sums) != 0, "sums16 rejects D % 16 != 0");
}

int main(void)
{
    for (uint32_t b = 0; b < 65536u; ++b) {          /* every binary16 value through both conversions */
        const double v = qso_half_to_double((uint16_t)b);
        if (v == v)
            CHECK(qso_double_to_half(v) == (uint16_t)b || (b == 0x8000u && v == 0.0), "binary16 round trip");
    }
    attention_cases();
    score_cases();
    quant_cases();
    select_cases();
    gate_cases();
    if (fails) {
        fprintf(stderr, "%d driver checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
