/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C. Every floating-point result is formed in
 * f64 from exactly decoded block values, except the activation quantizer,
 * which the method fixes in f32 and which is reproduced here in f32 step by
 * step. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load this library; the GPU path never calls it, and it shares no code,
 * header or table with the GPU path.
 *
 * Source pages (hanzo-ml 0.11.89 `src/vulkan_backend.rs`, hanzo-ml 0.11.71
 * `tests/vulkan_quant_tests.rs`, hanzo-kernel 0.2.40 `src/main.rs`):
 *  - the ground truth of the quant tests is "dequantize the stored blocks,
 *    then an f64 matvec over the dequantized weights" (module doc of
 *    `tests/vulkan_quant_tests.rs`); every matvec below is that.
 *  - block field order: Q8_0 = f16 scale + 32 int8 (`quantize_q8_blocks`);
 *    Q4_K = d, dmin, scales[12], qs[128] (`quantize_q4k_split`);
 *    Q6_K = ql[128], qh[64], scales[16] int8, d (`quantize_q6k`,
 *    `quantize_q6k_split`); Q4_0 = f16 d + 16 code bytes (`matvec_q4_0_gpu`);
 *    Q5_K = d, dmin, scales[12], qh[32], qs[128] (`quantize_q5k`). The bit
 *    packing inside the fields is not printed
 *    on the pages; the public GGML k-quant packing is used (see the decoder
 *    comments).
 *  - q8 activation triple (xq, xs, xsum = dequantized block sum) per 32
 *    values: doc of `quantize_act_q8` in `src/vulkan_backend.rs`.
 *  - router = softmax, top-k, renormalize: doc of `moe_route_vk`.
 *  - expert-gather matvec y[s,r] = sum_k W[ids[s],r,k] x[s,k]: doc of
 *    `moe_matvec_gpu`.
 *  - router gate = plain f32 GEMV logits[t, e] = Wr[e, :] . x[t, :]: the
 *    "gemv" kernel of `src/vulkan_backend.rs` and `check_gemv` of
 *    hanzo-kernel `src/main.rs`.
 *
 * Compile with -ffp-contract=off (no FMA contraction) and without
 * -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_Q8_0 = 0, ORACLE_Q4K = 1, ORACLE_Q6K = 2, ORACLE_Q4_0 = 3, ORACLE_Q5K = 4, ORACLE_NFMT = 5 };

static const int64_t QK[ORACLE_NFMT] = {32, 256, 256, 32, 256};
static const int64_t QB[ORACLE_NFMT] = {34, 144, 210, 18, 176};

/* ---------------------------------------------------------------------- */
/* O1: IEEE binary16 -> f64, exact, subnormals included. The pages stress  */
/* that f16 d/dmin must decode subnormal-exactly (comments in              */
/* `matvec_q4k_gpu_off` on unpackHalf2x16 and the f16lo_to_f32 fix).        */
/* value = (-1)^s * 2^(e-15) * (1 + f/1024) for 0 < e < 31,                */
/*         (-1)^s * 2^-14 * f/1024 for e = 0.                              */
/* ---------------------------------------------------------------------- */
double oracle_half(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    }
    return s ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ---------------------------------------------------------------------- */
/* O2: block decoders                                                      */
/* ---------------------------------------------------------------------- */

/* Q8_0: w_i = d * q_i, q_i int8. */
static void dec_q8_0(const uint8_t *b, double *out) {
    double d = oracle_half(rd16(b));
    for (int i = 0; i < 32; ++i) out[i] = d * (double)(int8_t)b[2 + i];
}

/* Q4_K 6-bit scale / min of sub-block j from the 12 packed bytes:
 * j < 4 : sc = s[j] & 63,            m = s[j+4] & 63
 * j >= 4: sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
 *         m  = (s[j+4] >> 4) | (s[j]   >> 6) << 4 */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Q4_K: eight sub-blocks of 32; w = d*sc_j*q - dmin*m_j (the affine form the
 * pages' MMQ epilogue and "dmin fold" comments imply). Sub-block j takes its
 * codes from qs bytes 32*(j/2) .. +31, low nibble for even j, high for odd. */
static void dec_q4k(const uint8_t *b, double *out) {
    double d = oracle_half(rd16(b));
    double dmin = oracle_half(rd16(b + 2));
    const uint8_t *sc = b + 4;
    const uint8_t *qs = b + 16;
    for (int j = 0; j < 8; ++j) {
        int s, m;
        q4k_scale_min(sc, j, &s, &m);
        for (int l = 0; l < 32; ++l) {
            uint8_t byte = qs[32 * (j / 2) + l];
            int q = (j & 1) ? (byte >> 4) : (byte & 15);
            out[32 * j + l] = d * (double)s * (double)q - dmin * (double)m;
        }
    }
}

/* Q6_K: w_i = d * sc[i/16] * (q_i - 32), sc int8 (sign-extended), q_i 6 bit:
 * h = i/128, p = i%128, g = p/32, l = p%32,
 * low 4 bits from ql[64h + l + 32*(g%2)] (low nibble if g < 2, else high),
 * high 2 bits = (qh[32h + l] >> 2g) & 3. */
static void dec_q6k(const uint8_t *b, double *out) {
    const uint8_t *ql = b, *qh = b + 128;
    const int8_t *sc = (const int8_t *)(b + 192);
    double d = oracle_half(rd16(b + 208));
    for (int i = 0; i < 256; ++i) {
        int h = i / 128, p = i % 128, g = p / 32, l = p % 32;
        uint8_t lb = ql[64 * h + l + 32 * (g % 2)];
        int lo = g < 2 ? (lb & 15) : (lb >> 4);
        int hi = (qh[32 * h + l] >> (2 * g)) & 3;
        int q = lo | (hi << 4);
        out[i] = d * (double)sc[i / 16] * (double)(q - 32);
    }
}

/* Q4_0 (hanzo-ml `src/vulkan_backend.rs`, `matvec_q4_0_gpu`: the native
 * 18-byte block, f16 d then 16 code bytes): w = d * (q - 8), q 4 bit; byte j
 * holds weight j (low nibble) and weight j + 16 (high nibble), the public
 * GGML order. */
static void dec_q4_0(const uint8_t *b, double *out) {
    double d = oracle_half(rd16(b));
    for (int j = 0; j < 16; ++j) {
        out[j] = d * (double)((b[2 + j] & 15) - 8);
        out[j + 16] = d * (double)((b[2 + j] >> 4) - 8);
    }
}

/* Q5_K (hanzo-ml `src/vulkan_backend.rs`, `quantize_q5k`: d, dmin, 12 scale
 * bytes, 32 qh bytes, 128 qs bytes): w = d*sc_j*q - dmin*m_j with a 5-bit q;
 * scales as Q4_K; sub-block j takes its low 4 bits as Q4_K does from qs and
 * its bit 4 from bit j of qh[l] (public GGML packing). */
static void dec_q5k(const uint8_t *b, double *out) {
    double d = oracle_half(rd16(b));
    double dmin = oracle_half(rd16(b + 2));
    const uint8_t *sc = b + 4, *qh = b + 16, *qs = b + 48;
    for (int j = 0; j < 8; ++j) {
        int s, m;
        q4k_scale_min(sc, j, &s, &m);
        for (int l = 0; l < 32; ++l) {
            uint8_t byte = qs[32 * (j / 2) + l];
            int q = ((j & 1) ? (byte >> 4) : (byte & 15)) | (((qh[l] >> j) & 1) << 4);
            out[32 * j + l] = d * (double)s * (double)q - dmin * (double)m;
        }
    }
}

static void dec_block(int fmt, const uint8_t *b, double *out) {
    if (fmt == ORACLE_Q8_0) dec_q8_0(b, out);
    else if (fmt == ORACLE_Q4K) dec_q4k(b, out);
    else if (fmt == ORACLE_Q6K) dec_q6k(b, out);
    else if (fmt == ORACLE_Q4_0) dec_q4_0(b, out);
    else dec_q5k(b, out);
}

int oracle_dequant(int fmt, const uint8_t *blocks, int64_t nblocks, double *out) {
    if (fmt < 0 || fmt >= ORACLE_NFMT) return -1;
    for (int64_t b = 0; b < nblocks; ++b) dec_block(fmt, blocks + b * QB[fmt], out + b * QK[fmt]);
    return 0;
}

/* Dequantize one weight row of k values. */
static void dec_row(int fmt, const uint8_t *row, int64_t k, double *out) {
    for (int64_t b = 0; b < k / QK[fmt]; ++b) dec_block(fmt, row + b * QB[fmt], out + b * QK[fmt]);
}

static int64_t row_bytes(int fmt, int64_t k) { return k / QK[fmt] * QB[fmt]; }

/* ---------------------------------------------------------------------- */
/* O3: y_r = sum_c W_deq[r,c] * x_c in f64, for the listed rows (all rows   */
/* when `rows` is NULL). y has one entry per listed row.                    */
/* ---------------------------------------------------------------------- */
int oracle_matvec(int fmt, const uint8_t *w, const float *x, int64_t n, int64_t k,
                  const int64_t *rows, int64_t nrows, double *y) {
    if (fmt < 0 || fmt >= ORACLE_NFMT || k % QK[fmt]) return -1;
    double *wd = malloc(sizeof(double) * (size_t)k);
    if (!wd) return -2;
    int64_t cnt = rows ? nrows : n;
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t r = rows ? rows[i] : i;
        dec_row(fmt, w + r * row_bytes(fmt, k), k, wd);
        double acc = 0.0;
        for (int64_t c = 0; c < k; ++c) acc += wd[c] * (double)x[c];
        y[i] = acc;
    }
    free(wd);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* O4: activation quantizer, per 32 consecutive values of each row, in f32: */
/*   amax = max |x|; if amax > 0: inv = 127/amax, xs = amax/127             */
/*   else inv = 0, xs = 1 (the weight quantizer's zero-block convention);   */
/*   xq = clamp(round_half_away(x*inv), -127, 127);                         */
/*   xsum = xs * (float)sum(xq)  -- the dequantized block sum.              */
/* ---------------------------------------------------------------------- */
int oracle_quantize_act_q8(const float *x, int64_t m, int64_t k, int8_t *xq, float *xs,
                           float *xsum) {
    if (k % 32) return -1;
    int64_t nb = m * (k / 32);
    for (int64_t b = 0; b < nb; ++b) {
        const float *v = x + b * 32;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(v[i]);
            if (a > amax) amax = a;
        }
        float inv = 0.0f, scale = 1.0f;
        if (amax > 0.0f) {
            inv = 127.0f / amax;
            scale = amax / 127.0f;
        }
        int sum = 0;
        for (int i = 0; i < 32; ++i) {
            float p = v[i] * inv;
            float r = roundf(p);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            int q = (int)r;
            xq[b * 32 + i] = (int8_t)q;
            sum += q;
        }
        xs[b] = scale;
        xsum[b] = scale * (float)sum;
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* O5: integer block sums of the int8-dot path, Q4_K weights x q8 codes:    */
/* S[r, b] = sum_{i<32} q4[r, 32b+i] * xq[32b+i]  (q4 in 0..15).            */
/* The Q4_K sub-block j of superblock s is q8 block b = 8s + j.             */
/* ---------------------------------------------------------------------- */
int oracle_blocksums_q4k_q8(const uint8_t *w, const int8_t *xq, int64_t n, int64_t k, int64_t *S) {
    if (k % 256) return -1;
    int64_t nsb = k / 256;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t s = 0; s < nsb; ++s) {
            const uint8_t *qs = w + (r * nsb + s) * 144 + 16;
            for (int j = 0; j < 8; ++j) {
                int64_t acc = 0;
                for (int l = 0; l < 32; ++l) {
                    uint8_t byte = qs[32 * (j / 2) + l];
                    int q = (j & 1) ? (byte >> 4) : (byte & 15);
                    acc += (int64_t)q * (int64_t)xq[s * 256 + 32 * j + l];
                }
                S[r * (k / 32) + s * 8 + j] = acc;
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* O6: the int8-dot matvec's result by its plain definition:                */
/* y = W_deq . x_deq with x_deq[c] = xs[c/32] * xq[c], in f64.              */
/* ---------------------------------------------------------------------- */
int oracle_matvec_q8act(int fmt, const uint8_t *w, const int8_t *xq, const float *xs, int64_t n,
                        int64_t k, const int64_t *rows, int64_t nrows, double *y) {
    if (fmt < 0 || fmt >= ORACLE_NFMT || k % QK[fmt] || k % 32) return -1;
    double *wd = malloc(sizeof(double) * (size_t)k);
    double *xd = malloc(sizeof(double) * (size_t)k);
    if (!wd || !xd) { free(wd); free(xd); return -2; }
    for (int64_t c = 0; c < k; ++c) xd[c] = (double)xs[c / 32] * (double)xq[c];
    int64_t cnt = rows ? nrows : n;
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t r = rows ? rows[i] : i;
        dec_row(fmt, w + r * row_bytes(fmt, k), k, wd);
        double acc = 0.0;
        for (int64_t c = 0; c < k; ++c) acc += wd[c] * xd[c];
        y[i] = acc;
    }
    free(wd);
    free(xd);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* O7: router. Per token: order the E logits by value, descending, equal     */
/* values by lower expert index (NaN ranks as -inf); the first topk are the  */
/* ids, in that order. Weights: p_j = exp(l_j - l_max), w_j = p_j / sum of   */
/* the top-k p (the softmax denominator cancels in the renormalization).    */
/* If l_max is -inf every p_j is taken as 1.                                */
/* ---------------------------------------------------------------------- */
static const float *g_keys;
static int cmp_logit(const void *a, const void *b) {
    int i = *(const int *)a, j = *(const int *)b;
    float li = g_keys[i], lj = g_keys[j];
    if (li != li) li = -INFINITY;
    if (lj != lj) lj = -INFINITY;
    if (li > lj) return -1;
    if (li < lj) return 1;
    return i < j ? -1 : (i > j ? 1 : 0);
}

int oracle_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids,
                     double *w) {
    if (topk < 1 || topk > E) return -1;
    int *idx = malloc(sizeof(int) * (size_t)E);
    if (!idx) return -2;
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        for (int e = 0; e < E; ++e) idx[e] = e;
        g_keys = l;
        qsort(idx, (size_t)E, sizeof(int), cmp_logit);
        double lmax = l[idx[0]];
        if (lmax != lmax) lmax = -INFINITY;
        double den = 0.0;
        for (int64_t j = 0; j < topk; ++j) {
            double lj = l[idx[j]];
            if (lj != lj) lj = -INFINITY;
            double p = isinf(lmax) && lmax < 0 ? 1.0 : exp(lj - lmax);
            w[t * topk + j] = p;
            den += p;
        }
        for (int64_t j = 0; j < topk; ++j) {
            ids[t * topk + j] = idx[j];
            w[t * topk + j] /= den;
        }
    }
    free(idx);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Expert-gather matvec: y[s, r] = sum_c W[ids[s], r, c] * x[s / x_div, c]  */
/* over a bank [E, n, k] stored expert-major, row-major. Slots whose id is  */
/* outside [0, E) produce zero rows.                                        */
/* ---------------------------------------------------------------------- */
int oracle_moe_qmv(int fmt, const uint8_t *bank, const float *x, int64_t x_div, const int32_t *ids,
                   int64_t nslots, int64_t n, int64_t k, int64_t E, double *y) {
    if (fmt < 0 || fmt >= ORACLE_NFMT || k % QK[fmt] || x_div < 1) return -1;
    double *wd = malloc(sizeof(double) * (size_t)k);
    if (!wd) return -2;
    int64_t rb = row_bytes(fmt, k);
    for (int64_t s = 0; s < nslots; ++s) {
        int32_t e = ids[s];
        const float *xs = x + (s / x_div) * k;
        for (int64_t r = 0; r < n; ++r) {
            if (e < 0 || e >= E) { y[s * n + r] = 0.0; continue; }
            dec_row(fmt, bank + ((int64_t)e * n + r) * rb, k, wd);
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c) acc += wd[c] * (double)xs[c];
            y[s * n + r] = acc;
        }
    }
    free(wd);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* O8: MoE FFN layer over routed slots s = topk*t + j, e = ids[s]:           */
/*   g = W_gate[e] x_t, u = W_up[e] x_t          (Q4_K banks [E, inter, hidden])*/
/*   h = silu(g) * u, silu(z) = z / (1 + exp(-z))                            */
/*   dvec = W_down[e] h                          (Q6_K bank [E, hidden, inter]) */
/*   y_t = sum_j wts[t, j] * dvec_{topk*t + j}                               */
/* All in f64. h [T*topk, inter], dvec [T*topk, hidden] are returned too     */
/* (pass NULL to skip).                                                     */
/* ---------------------------------------------------------------------- */
int oracle_moe_ffn(const uint8_t *gate, const uint8_t *up, const uint8_t *down, const float *x,
                   const int32_t *ids, const float *wts, int64_t T, int64_t topk, int64_t hidden,
                   int64_t inter, int64_t E, double *h_out, double *d_out, double *y) {
    if (hidden % 256 || inter % 256) return -1;
    int64_t ns = T * topk;
    double *h = malloc(sizeof(double) * (size_t)(ns * inter));
    double *dv = malloc(sizeof(double) * (size_t)(ns * hidden));
    double *wd = malloc(sizeof(double) * (size_t)(hidden > inter ? hidden : inter));
    if (!h || !dv || !wd) { free(h); free(dv); free(wd); return -2; }
    int64_t rb_gu = row_bytes(ORACLE_Q4K, hidden), rb_dn = row_bytes(ORACLE_Q6K, inter);
    for (int64_t s = 0; s < ns; ++s) {
        int32_t e = ids[s];
        const float *xt = x + (s / topk) * hidden;
        for (int64_t r = 0; r < inter; ++r) {
            if (e < 0 || e >= E) { h[s * inter + r] = 0.0; continue; }
            double g = 0.0, u = 0.0;
            dec_row(ORACLE_Q4K, gate + ((int64_t)e * inter + r) * rb_gu, hidden, wd);
            for (int64_t c = 0; c < hidden; ++c) g += wd[c] * (double)xt[c];
            dec_row(ORACLE_Q4K, up + ((int64_t)e * inter + r) * rb_gu, hidden, wd);
            for (int64_t c = 0; c < hidden; ++c) u += wd[c] * (double)xt[c];
            h[s * inter + r] = g / (1.0 + exp(-g)) * u;
        }
        for (int64_t r = 0; r < hidden; ++r) {
            if (e < 0 || e >= E) { dv[s * hidden + r] = 0.0; continue; }
            dec_row(ORACLE_Q6K, down + ((int64_t)e * hidden + r) * rb_dn, inter, wd);
            double acc = 0.0;
            for (int64_t c = 0; c < inter; ++c) acc += wd[c] * h[s * inter + c];
            dv[s * hidden + r] = acc;
        }
    }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t r = 0; r < hidden; ++r) {
            double acc = 0.0;
            for (int64_t j = 0; j < topk; ++j)
                acc += (double)wts[t * topk + j] * dv[(t * topk + j) * hidden + r];
            y[t * hidden + r] = acc;
        }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)(ns * inter));
    if (d_out) memcpy(d_out, dv, sizeof(double) * (size_t)(ns * hidden));
    free(h);
    free(dv);
    free(wd);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* a11 prefill: Y[m, n] = sum_c X_deq[m, c] * W_deq[n, c], X_deq = xs*xq,    */
/* for the listed activation rows (all when `mrows` is NULL). Y has one row */
/* of n values per listed activation row.                                   */
/* ---------------------------------------------------------------------- */
int oracle_qmm(int fmt, const uint8_t *w, const int8_t *xq, const float *xs, int64_t m, int64_t n,
               int64_t k, const int64_t *mrows, int64_t nm, double *Y) {
    if (fmt < 0 || fmt >= ORACLE_NFMT || k % QK[fmt] || k % 32) return -1;
    int64_t cnt = mrows ? nm : m;
    double *wd = malloc(sizeof(double) * (size_t)(n * k));
    double *xd = malloc(sizeof(double) * (size_t)k);
    if (!wd || !xd) { free(wd); free(xd); return -2; }
    for (int64_t r = 0; r < n; ++r) dec_row(fmt, w + r * row_bytes(fmt, k), k, wd + r * k);
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t mi = mrows ? mrows[i] : i;
        for (int64_t c = 0; c < k; ++c) xd[c] = (double)xs[mi * (k / 32) + c / 32] * (double)xq[mi * k + c];
        for (int64_t r = 0; r < n; ++r) {
            const double *wr = wd + r * k;
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c) acc += xd[c] * wr[c];
            Y[i * n + r] = acc;
        }
    }
    free(wd);
    free(xd);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Router gate (hanzo-ml `src/vulkan_backend.rs`, the "gemv" entry of the  */
/* kernel table; hanzo-kernel `src/main.rs`, `check_gemv`): the f32 GEMV   */
/* that produces the router logits of a decode step, one output per        */
/* router row, logits[t, e] = sum_c Wr[e, c] * x[t, c], here in f64.        */
/* Wr: f32[E, hidden] row-major; x: f32[T, hidden]; out: f64[T, E].         */
/* ---------------------------------------------------------------------- */
int oracle_gemv(const float *w, const float *x, int64_t T, int64_t E, int64_t hidden, double *out) {
    if (T < 0 || E < 1 || hidden < 1) return -1;
    for (int64_t t = 0; t < T; ++t) {
        const float *xt = x + t * hidden;
        for (int64_t e = 0; e < E; ++e) {
            const float *we = w + e * hidden;
            double acc = 0.0;
            for (int64_t c = 0; c < hidden; ++c) acc += (double)we[c] * (double)xt[c];
            out[t * E + e] = acc;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Expert-indexed prefill GEMM on a q8 activation (hanzo-kernel            */
/* `src/main.rs`, `check_mmq_q4k_id`: the expert-indexed Q4_K MMQ, the MoE  */
/* prefill twin of the gather matvec): for slot s with expert e = ids[s],  */
/*   Y[s, r] = sum_c W_deq[e, r, c] * xs[a, c/32] * xq[a, c],  a = s/x_div, */
/* in f64, for the listed slots (all when `slots` is NULL); a slot whose   */
/* expert is outside [0, E) has a zero row.                                 */
/* ---------------------------------------------------------------------- */
int oracle_moe_qmm(int fmt, const uint8_t *bank, const int8_t *xq, const float *xs, int64_t x_div,
                   const int32_t *ids, int64_t nslots, int64_t n, int64_t k, int64_t E,
                   const int64_t *slots, int64_t nlist, double *Y) {
    if (fmt < 0 || fmt >= ORACLE_NFMT || k % QK[fmt] || k % 32 || x_div < 1) return -1;
    int64_t cnt = slots ? nlist : nslots;
    double *wd = malloc(sizeof(double) * (size_t)k);
    double *xd = malloc(sizeof(double) * (size_t)k);
    if (!wd || !xd) { free(wd); free(xd); return -2; }
    int64_t rb = row_bytes(fmt, k);
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t s = slots ? slots[i] : i;
        int32_t e = ids[s];
        if (e < 0 || e >= E) {
            for (int64_t r = 0; r < n; ++r) Y[i * n + r] = 0.0;
            continue;
        }
        int64_t a = s / x_div;
        for (int64_t c = 0; c < k; ++c) xd[c] = (double)xs[a * (k / 32) + c / 32] * (double)xq[a * k + c];
        for (int64_t r = 0; r < n; ++r) {
            dec_row(fmt, bank + ((int64_t)e * n + r) * rb, k, wd);
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c) acc += wd[c] * xd[c];
            Y[i * n + r] = acc;
        }
    }
    free(wd);
    free(xd);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* MoE layer at prefill on a q8 activation (the prefill twin of             */
/* oracle_moe_ffn: the expert-indexed MMQ takes quantize_act_q8 output,     */
/* hanzo-kernel `src/main.rs` `check_mmq_q4k_id`; `matmul_q6k_gpu_off` runs  */
/* the down projection on one expert of the bank): x_deq[t, c] =            */
/* xs[t, c/32] * xq[t, c] exactly in f64, then per slot s = topk*t + j,     */
/* e = ids[s] in [0, E): g = Wg[e] x_deq[t], u = Wu[e] x_deq[t],            */
/* h = g / (1 + exp(-g)) * u, d = Wd[e] h; y[t] = sum_j wts[t, j] d_s (a    */
/* slot outside [0, E) adds nothing). y rows of the listed tokens (all when */
/* `toks` is NULL), f64.                                                    */
/* ---------------------------------------------------------------------- */
int oracle_moe_ffn_q8x(const uint8_t *gate, const uint8_t *up, const uint8_t *down, const int8_t *xq,
                       const float *xs, const int32_t *ids, const float *wts, int64_t T, int64_t topk,
                       int64_t hidden, int64_t inter, int64_t E, const int64_t *toks, int64_t ntok, double *y) {
    if (hidden % 256 || inter % 256) return -1;
    int64_t cnt = toks ? ntok : T;
    double *xd = malloc(sizeof(double) * (size_t)hidden);
    double *h = malloc(sizeof(double) * (size_t)inter);
    double *wd = malloc(sizeof(double) * (size_t)(hidden > inter ? hidden : inter));
    if (!xd || !h || !wd) { free(xd); free(h); free(wd); return -2; }
    int64_t rb_gu = row_bytes(ORACLE_Q4K, hidden), rb_dn = row_bytes(ORACLE_Q6K, inter);
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t t = toks ? toks[i] : i;
        for (int64_t c = 0; c < hidden; ++c)
            xd[c] = (double)xs[t * (hidden / 32) + c / 32] * (double)xq[t * hidden + c];
        for (int64_t r = 0; r < hidden; ++r) y[i * hidden + r] = 0.0;
        for (int64_t j = 0; j < topk; ++j) {
            int32_t e = ids[t * topk + j];
            if (e < 0 || e >= E) continue;
            for (int64_t r = 0; r < inter; ++r) {
                double g = 0.0, u = 0.0;
                dec_row(ORACLE_Q4K, gate + ((int64_t)e * inter + r) * rb_gu, hidden, wd);
                for (int64_t c = 0; c < hidden; ++c) g += wd[c] * xd[c];
                dec_row(ORACLE_Q4K, up + ((int64_t)e * inter + r) * rb_gu, hidden, wd);
                for (int64_t c = 0; c < hidden; ++c) u += wd[c] * xd[c];
                h[r] = g / (1.0 + exp(-g)) * u;
            }
            double wj = (double)wts[t * topk + j];
            for (int64_t r = 0; r < hidden; ++r) {
                dec_row(ORACLE_Q6K, down + ((int64_t)e * hidden + r) * rb_dn, inter, wd);
                double acc = 0.0;
                for (int64_t c = 0; c < inter; ++c) acc += wd[c] * h[c];
                y[i * hidden + r] += wj * acc;
            }
        }
    }
    free(xd);
    free(h);
    free(wd);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* MoE layer with q8 activations on both projections (the pages' int8-dot  */
/* MoE decode path: hanzo-ml `src/vulkan_backend.rs` quantizes the         */
/* activation once with `quantize_act_q8` and runs the dp4a gate/up and    */
/* down gathers; the down activation h is quantized the same way): per    */
/* token t, x_deq = xs * xq; per slot s = topk*t + j with e = ids[s] in     */
/* [0, E): h = silu(Wg[e] x_deq) * (Wu[e] x_deq) in f64, rounded to f32 and */
/* quantized by oracle_quantize_act_q8 (hq, hs), d = Wd[e] (hs * hq);       */
/* y[t] = sum_j wts[t, j] d. For the listed tokens (all when `toks` is      */
/* NULL): y rows, and when the pointers are non-NULL the f64 h, hq and hs   */
/* of their slots (zero rows for a slot outside [0, E)).                    */
/* ---------------------------------------------------------------------- */
int oracle_moe_ffn_q8(const uint8_t *gate, const uint8_t *up, const uint8_t *down, const int8_t *xq,
                      const float *xs, const int32_t *ids, const float *wts, int64_t T, int64_t topk,
                      int64_t hidden, int64_t inter, int64_t E, const int64_t *toks, int64_t ntok, double *y,
                      double *h_out, int8_t *hq_out, float *hs_out) {
    if (hidden % 256 || inter % 256) return -1;
    int64_t cnt = toks ? ntok : T;
    double *xd = malloc(sizeof(double) * (size_t)hidden);
    double *h = malloc(sizeof(double) * (size_t)inter);
    float *hf = malloc(sizeof(float) * (size_t)inter);
    int8_t *hq = malloc((size_t)inter);
    float *hs = malloc(sizeof(float) * (size_t)(inter / 32));
    float *hsum = malloc(sizeof(float) * (size_t)(inter / 32));
    double *wd = malloc(sizeof(double) * (size_t)(hidden > inter ? hidden : inter));
    if (!xd || !h || !hf || !hq || !hs || !hsum || !wd) {
        free(xd); free(h); free(hf); free(hq); free(hs); free(hsum); free(wd);
        return -2;
    }
    int64_t rb_gu = row_bytes(ORACLE_Q4K, hidden), rb_dn = row_bytes(ORACLE_Q6K, inter);
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t t = toks ? toks[i] : i;
        for (int64_t c = 0; c < hidden; ++c)
            xd[c] = (double)xs[t * (hidden / 32) + c / 32] * (double)xq[t * hidden + c];
        for (int64_t r = 0; r < hidden; ++r) y[i * hidden + r] = 0.0;
        for (int64_t j = 0; j < topk; ++j) {
            int64_t o = i * topk + j;  /* slot row of the outputs */
            int32_t e = ids[t * topk + j];
            if (e < 0 || e >= E) {
                if (h_out) for (int64_t r = 0; r < inter; ++r) h_out[o * inter + r] = 0.0;
                if (hq_out) memset(hq_out + o * inter, 0, (size_t)inter);
                if (hs_out) for (int64_t b = 0; b < inter / 32; ++b) hs_out[o * (inter / 32) + b] = 0.0f;
                continue;
            }
            for (int64_t r = 0; r < inter; ++r) {
                double g = 0.0, u = 0.0;
                dec_row(ORACLE_Q4K, gate + ((int64_t)e * inter + r) * rb_gu, hidden, wd);
                for (int64_t c = 0; c < hidden; ++c) g += wd[c] * xd[c];
                dec_row(ORACLE_Q4K, up + ((int64_t)e * inter + r) * rb_gu, hidden, wd);
                for (int64_t c = 0; c < hidden; ++c) u += wd[c] * xd[c];
                h[r] = g / (1.0 + exp(-g)) * u;
                hf[r] = (float)h[r];
            }
            oracle_quantize_act_q8(hf, 1, inter, hq, hs, hsum);
            if (h_out) memcpy(h_out + o * inter, h, sizeof(double) * (size_t)inter);
            if (hq_out) memcpy(hq_out + o * inter, hq, (size_t)inter);
            if (hs_out) memcpy(hs_out + o * (inter / 32), hs, sizeof(float) * (size_t)(inter / 32));
            double wj = (double)wts[t * topk + j];
            for (int64_t r = 0; r < hidden; ++r) {
                dec_row(ORACLE_Q6K, down + ((int64_t)e * hidden + r) * rb_dn, inter, wd);
                double acc = 0.0;
                for (int64_t c = 0; c < inter; ++c) acc += wd[c] * (double)hs[c / 32] * (double)hq[c];
                y[i * hidden + r] += wj * acc;
            }
        }
    }
    free(xd); free(h); free(hf); free(hq); free(hs); free(hsum); free(wd);
    return 0;
}
