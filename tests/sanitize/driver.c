/* Sanitizer driver for the CPU oracle and the seeded input generators.
 *
 * Built by tests/test_sanitize.py with gcc -fsanitize=address,undefined
 * (no recovery) together with oracle/oracle.c and synth/synth.c, and run as
 * a plain executable: every oracle entry point and every generator is called
 * on small inputs in exactly sized heap buffers (so that AddressSanitizer
 * sees any access past them), including the edge cases the oracle takes
 * (zero activation blocks, out-of-range expert ids, topk == E, listed-row
 * modes). A few invariants are checked on the way; the exit status is 0 only
 * if every call returned 0 and every check held. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle/oracle.c */
double oracle_half(uint16_t h);
int oracle_dequant(int fmt, const uint8_t *blocks, int64_t nblocks, double *out);
int oracle_matvec(int fmt, const uint8_t *w, const float *x, int64_t n, int64_t k, const int64_t *rows,
                  int64_t nrows, double *y);
int oracle_quantize_act_q8(const float *x, int64_t m, int64_t k, int8_t *xq, float *xs, float *xsum);
int oracle_blocksums_q4k_q8(const uint8_t *w, const int8_t *xq, int64_t n, int64_t k, int64_t *S);
int oracle_matvec_q8act(int fmt, const uint8_t *w, const int8_t *xq, const float *xs, int64_t n, int64_t k,
                        const int64_t *rows, int64_t nrows, double *y);
int oracle_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids, double *w);
int oracle_moe_qmv(int fmt, const uint8_t *bank, const float *x, int64_t x_div, const int32_t *ids,
                   int64_t nslots, int64_t n, int64_t k, int64_t E, double *y);
int oracle_moe_ffn(const uint8_t *gate, const uint8_t *up, const uint8_t *down, const float *x, const int32_t *ids,
                   const float *wts, int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E,
                   double *h_out, double *d_out, double *y);
int oracle_qmm(int fmt, const uint8_t *w, const int8_t *xq, const float *xs, int64_t m, int64_t n, int64_t k,
               const int64_t *mrows, int64_t nm, double *Y);
int oracle_gemv(const float *w, const float *x, int64_t T, int64_t E, int64_t hidden, double *out);
int oracle_moe_qmm(int fmt, const uint8_t *bank, const int8_t *xq, const float *xs, int64_t x_div,
                   const int32_t *ids, int64_t nslots, int64_t n, int64_t k, int64_t E, const int64_t *slots,
                   int64_t nlist, double *Y);
int oracle_moe_ffn_q8x(const uint8_t *gate, const uint8_t *up, const uint8_t *down, const int8_t *xq,
                       const float *xs, const int32_t *ids, const float *wts, int64_t T, int64_t topk,
                       int64_t hidden, int64_t inter, int64_t E, const int64_t *toks, int64_t ntok, double *y);
int oracle_moe_ffn_q8(const uint8_t *gate, const uint8_t *up, const uint8_t *down, const int8_t *xq,
                      const float *xs, const int32_t *ids, const float *wts, int64_t T, int64_t topk,
                      int64_t hidden, int64_t inter, int64_t E, const int64_t *toks, int64_t ntok, double *y,
                      double *h_out, int8_t *hq_out, float *hs_out);
/* synth/synth.c */
void synth_uniform(uint64_t seed, uint64_t start, int64_t n, float *out);
void synth_normal(uint64_t seed, uint64_t start, int64_t n, float *out);
uint16_t synth_f32_to_f16(float f);
int synth_encode_q8_0(const float *w, int64_t rows, int64_t k, uint8_t *out);
int synth_encode_q4k(const float *w, int64_t rows, int64_t k, uint8_t *out);
int synth_encode_q6k(const float *w, int64_t rows, int64_t k, uint8_t *out);
int synth_encode_q4_0(const float *w, int64_t rows, int64_t k, uint8_t *out);
int synth_encode_q5k(const float *w, int64_t rows, int64_t k, uint8_t *out);
int64_t synth_row_bytes(int fmt, int64_t k);
int synth_weights(int fmt, uint64_t seed, int64_t rows, int64_t k, uint8_t *out);
int synth_random_blocks(int fmt, uint64_t seed, int64_t nblocks, int subnormal_every, uint8_t *out);

static int failures = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static void *xalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int all_finite(const double *v, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

static const int BW[5] = {32, 256, 256, 32, 256};
static const int BB[5] = {34, 144, 210, 18, 176};

static uint8_t *weights(int fmt, uint64_t seed, int64_t rows, int64_t k) {
    uint8_t *w = xalloc((size_t)(rows * synth_row_bytes(fmt, k)));
    CHECK(synth_weights(fmt, seed, rows, k, w) == 0);
    return w;
}

int main(void) {
    /* f16 decode over every bit pattern */
    int nonfinite = 0;
    for (uint32_t h = 0; h < 65536; ++h) nonfinite += !isfinite(oracle_half((uint16_t)h));
    CHECK(nonfinite == 2 * 1024); /* +-inf and the NaNs */
    CHECK(synth_f32_to_f16(1.0f) == 0x3C00);

    const int64_t n = 7, k = 512;
    float *x = xalloc(sizeof(float) * k);
    synth_normal(2, 0, k, x);
    float *u = xalloc(sizeof(float) * n * k);
    synth_uniform(1, 0, n * k, u);

    /* every format: encoders, generators, random blocks, dequant, matvec */
    int (*enc[5])(const float *, int64_t, int64_t, uint8_t *) = {synth_encode_q8_0, synth_encode_q4k,
                                                                 synth_encode_q6k, synth_encode_q4_0,
                                                                 synth_encode_q5k};
    for (int f = 0; f < 5; ++f) {
        const int64_t rb = synth_row_bytes(f, k), nb = n * k / BW[f];
        uint8_t *w = xalloc((size_t)(n * rb));
        CHECK(enc[f](u, n, k, w) == 0);
        uint8_t *wr = xalloc((size_t)(nb * BB[f]));
        CHECK(synth_random_blocks(f, 77, nb, 3, wr) == 0);
        double *dq = xalloc(sizeof(double) * n * k);
        CHECK(oracle_dequant(f, wr, nb, dq) == 0);
        CHECK(all_finite(dq, n * k));
        uint8_t *wg = weights(f, 5, n, k);
        double *y = xalloc(sizeof(double) * n);
        CHECK(oracle_matvec(f, wg, x, n, k, NULL, 0, y) == 0);
        CHECK(all_finite(y, n));
        int64_t rows[3] = {6, 0, 3};
        double yr[3];
        CHECK(oracle_matvec(f, wg, x, n, k, rows, 3, yr) == 0);
        CHECK(yr[0] == y[6] && yr[1] == y[0] && yr[2] == y[3]);
        free(w), free(wr), free(dq), free(wg), free(y);
    }

    /* activation quantizer with a zero block, block sums, q8-activation matvec */
    const int64_t m = 3;
    float *xa = xalloc(sizeof(float) * m * k);
    synth_normal(9, 0, m * k, xa);
    memset(xa + k + 32, 0, sizeof(float) * 32);
    int8_t *xq = xalloc((size_t)(m * k));
    float *xs = xalloc(sizeof(float) * m * (k / 32)), *xsum = xalloc(sizeof(float) * m * (k / 32));
    CHECK(oracle_quantize_act_q8(xa, m, k, xq, xs, xsum) == 0);
    CHECK(xs[k / 32 + 1] == 1.0f && xsum[k / 32 + 1] == 0.0f);
    uint8_t *w4 = weights(1, 1, n, k), *w6 = weights(2, 1, n, k);
    int64_t *S = xalloc(sizeof(int64_t) * n * (k / 32));
    CHECK(oracle_blocksums_q4k_q8(w4, xq, n, k, S) == 0);
    double *y8 = xalloc(sizeof(double) * n);
    for (int f = 0; f < 5; ++f) {
        uint8_t *wf = weights(f, 3, n, k);
        CHECK(oracle_matvec_q8act(f, wf, xq, xs, n, k, NULL, 0, y8) == 0);
        CHECK(all_finite(y8, n));
        free(wf);
    }
    double *Y = xalloc(sizeof(double) * m * n);
    CHECK(oracle_qmm(1, w4, xq, xs, m, n, k, NULL, 0, Y) == 0);
    int64_t mr[2] = {2, 0};
    CHECK(oracle_qmm(2, w6, xq, xs, m, n, k, mr, 2, Y) == 0);

    /* router: ties, topk == E, NaN and infinities */
    const int64_t T = 3, E = 8;
    float lg[24];
    synth_normal(3, 0, 24, lg);
    lg[1] = lg[2];        /* a tie */
    lg[8] = NAN;          /* token 1 */
    lg[9] = INFINITY;
    lg[10] = -INFINITY;
    int32_t ids[24];
    double rw[24];
    CHECK(oracle_moe_route(lg, T, E, 2, ids, rw) == 0);
    CHECK(oracle_moe_route(lg, T, E, E, ids, rw) == 0);
    double tot = 0;
    for (int j = 0; j < E; ++j) tot += rw[j];
    CHECK(fabs(tot - 1.0) < 1e-12);

    /* router gate GEMV */
    float *wr = xalloc(sizeof(float) * E * k);
    synth_uniform(30, 0, E * k, wr);
    double *lgo = xalloc(sizeof(double) * T * E);
    float *xt = xalloc(sizeof(float) * T * k);
    synth_normal(31, 0, T * k, xt);
    CHECK(oracle_gemv(wr, xt, T, E, k, lgo) == 0);
    CHECK(all_finite(lgo, T * E));

    /* MoE: gathers, layers, prefill forms, with out-of-range expert ids */
    const int64_t Em = 3, hidden = 256, inter = 256, Tm = 2, topk = 2, ns = Tm * topk;
    uint8_t *gate = weights(1, 10, Em * inter, hidden), *up = weights(1, 11, Em * inter, hidden);
    uint8_t *down = weights(2, 12, Em * hidden, inter);
    float *xm = xalloc(sizeof(float) * Tm * hidden);
    synth_normal(40, 0, Tm * hidden, xm);
    int32_t mids[4] = {2, -1, 0, 3};
    float mw[4] = {0.5f, 0.5f, 0.75f, 0.25f};
    double *ym = xalloc(sizeof(double) * ns * inter);
    CHECK(oracle_moe_qmv(1, gate, xm, topk, mids, ns, inter, hidden, Em, ym) == 0);
    CHECK(ym[1 * inter] == 0.0 && ym[3 * inter] == 0.0);
    double *h = xalloc(sizeof(double) * ns * inter), *d = xalloc(sizeof(double) * ns * hidden);
    double *yl = xalloc(sizeof(double) * Tm * hidden);
    CHECK(oracle_moe_ffn(gate, up, down, xm, mids, mw, Tm, topk, hidden, inter, Em, h, d, yl) == 0);
    CHECK(all_finite(yl, Tm * hidden));
    int8_t *xmq = xalloc((size_t)(Tm * hidden));
    float *xms = xalloc(sizeof(float) * Tm * (hidden / 32)), *xmsum = xalloc(sizeof(float) * Tm * (hidden / 32));
    CHECK(oracle_quantize_act_q8(xm, Tm, hidden, xmq, xms, xmsum) == 0);
    double *Ym = xalloc(sizeof(double) * ns * inter);
    CHECK(oracle_moe_qmm(1, gate, xmq, xms, topk, mids, ns, inter, hidden, Em, NULL, 0, Ym) == 0);
    int64_t sl[2] = {3, 0};
    CHECK(oracle_moe_qmm(1, gate, xmq, xms, topk, mids, ns, inter, hidden, Em, sl, 2, Ym) == 0);
    CHECK(oracle_moe_ffn_q8x(gate, up, down, xmq, xms, mids, mw, Tm, topk, hidden, inter, Em, NULL, 0, yl) == 0);
    int64_t tk[1] = {1};
    CHECK(oracle_moe_ffn_q8x(gate, up, down, xmq, xms, mids, mw, Tm, topk, hidden, inter, Em, tk, 1, yl) == 0);
    int8_t *hq = xalloc((size_t)(ns * inter));
    float *hs = xalloc(sizeof(float) * ns * (inter / 32));
    CHECK(oracle_moe_ffn_q8(gate, up, down, xmq, xms, mids, mw, Tm, topk, hidden, inter, Em, NULL, 0, yl, h, hq,
                            hs) == 0);
    CHECK(all_finite(yl, Tm * hidden));

    free(x), free(u), free(xa), free(xq), free(xs), free(xsum), free(w4), free(w6), free(S), free(y8), free(Y);
    free(wr), free(lgo), free(xt), free(gate), free(up), free(down), free(xm), free(ym), free(h), free(d), free(yl);
    free(xmq), free(xms), free(xmsum), free(Ym), free(hq), free(hs);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitized oracle + synth run clean\n");
    return 0;
}
