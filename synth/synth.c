/*
 * Seeded synthetic inputs for the block-quantized matvec / MoE path.
 *
 * This file is shared by the CPU oracle's tests and by the GPU path's tests
 * and benchmark. It only makes inputs: counter-based uniforms and normals,
 * and the weight encoders that turn an f32 matrix into raw GGML-layout
 * Q8_0 / Q4_K / Q6_K blocks. It holds none of the arithmetic that the
 * matvec path itself performs (no block decoding, no dot products, no
 * activation quantization, no routing).
 *
 * Sources for what is generated (hanzo-ml pages):
 *  - uniform counter: the `pseudo` helper of `tests/vulkan_quant_tests.rs`
 *    (a splitmix64-style finaliser of a counter, top 24 bits to [-1, 1));
 *    written here from the published splitmix64 finaliser.
 *  - Q8_0 encoder: `VulkanDevice::quantize_q8` in `src/vulkan_backend.rs`
 *    (per 32 weights: amax, inv = 127/amax, q = round(w*inv) clamped to
 *    +-127, scale = amax/127 stored as f16, all-zero block stores 1.0).
 *  - Q4_K / Q6_K / Q5_K / Q4_0 encoders: the pages only name the block
 *    layouts (`quantize_q5k`, `matvec_q4_0_gpu`) or `QTensor::quantize`; the
 *    encoders below are plain min/max quantizers producing valid blocks of
 *    the public GGML k-quant byte layout (parity is on the bytes, so any
 *    valid encoder serves).
 *
 * Build: gcc -O2 -fPIC -shared -fopenmp -ffp-contract=off synth.c -o libsynth.so
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* counters                                                                */
/* ---------------------------------------------------------------------- */

/* splitmix64 finaliser (Steele, Lea, Flood 2014) applied to a counter. */
static inline uint64_t mix64(uint64_t i) {
    uint64_t z = i + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Stream position of element i of stream `seed`: seed * 2^40 + i. */
static inline uint64_t ctr(uint64_t seed, uint64_t i) { return (seed << 40) + i; }

/* uniform in [-1, 1) with 24-bit resolution: top 24 bits / 2^24 * 2 - 1 */
static inline float unif(uint64_t c) {
    uint32_t t = (uint32_t)(mix64(c) >> 40);
    return ((float)t / 16777216.0f) * 2.0f - 1.0f;
}

/* uniform in (0, 1] with 24-bit resolution, as a double */
static inline double unif01(uint64_t c) {
    uint32_t t = (uint32_t)(mix64(c) >> 40);
    return ((double)t + 1.0) / 16777216.0;
}

void synth_uniform(uint64_t seed, uint64_t start, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = unif(ctr(seed, start + (uint64_t)i));
}

/* N(0,1) by Box-Muller in f64 from the counter pair (2i, 2i+1), cast to f32. */
void synth_normal(uint64_t seed, uint64_t start, int64_t n, float *out) {
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t j = start + (uint64_t)i;
        double u1 = unif01(ctr(seed, 2 * j));
        double u2 = unif01(ctr(seed, 2 * j + 1));
        out[i] = (float)(sqrt(-2.0 * log(u1)) * cos(two_pi * u2));
    }
}

/* ---------------------------------------------------------------------- */
/* f32 -> IEEE binary16, round to nearest even (subnormals and overflow).   */
/* ---------------------------------------------------------------------- */
uint16_t synth_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ex = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;
    if (ex == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    int32_t e = (int32_t)ex - 127 + 15;
    if (e >= 31) return (uint16_t)(sign | 0x7C00u);
    if (e <= 0) {
        /* subnormal half: value = man24 * 2^(ex-150); half ulp = 2^-24 */
        if (e < -10) return (uint16_t)sign;
        uint32_t m = man | 0x800000u;           /* 24-bit significand */
        uint32_t shift = (uint32_t)(14 - e);    /* to units of 2^-24 */
        uint32_t q = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q++;
        return (uint16_t)(sign | q);
    }
    uint32_t q = man >> 13;
    uint32_t rem = man & 0x1FFFu;
    uint32_t out = ((uint32_t)e << 10) | q;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) out++; /* may carry into exponent */
    return (uint16_t)(sign | out);
}

/* binary16 -> f32 for the encoders' own use (the encoder must know the
 * value it stored in order to pick codes against it). */
static float h2f(uint16_t h) {
    uint32_t s = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    float v;
    if (e == 0) v = ldexpf((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(m | 1024u), (int)e - 25);
    return s ? -v : v;
}

static inline float rnd(float v) { return roundf(v); } /* half away from zero */
static inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* ---------------------------------------------------------------------- */
/* Q8_0: 34 bytes per 32 weights = f16 d, 32 x int8                        */
/* ---------------------------------------------------------------------- */
static void enc_q8_0(const float *w, uint8_t *b) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) { float a = fabsf(w[i]); if (a > amax) amax = a; }
    float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    float scale = amax > 0.0f ? amax / 127.0f : 1.0f;
    uint16_t hb = synth_f32_to_f16(scale);
    b[0] = (uint8_t)(hb & 0xFF);
    b[1] = (uint8_t)(hb >> 8);
    for (int i = 0; i < 32; ++i) {
        float q = rnd(w[i] * inv);
        if (q > 127.0f) q = 127.0f;
        if (q < -127.0f) q = -127.0f;
        b[2 + i] = (uint8_t)(int8_t)(int)q;
    }
}

int synth_encode_q8_0(const float *w, int64_t rows, int64_t k, uint8_t *out) {
    if (k % 32) return -1;
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) enc_q8_0(w + r * k + b * 32, out + (r * nb + b) * 34);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Q4_K: 144 bytes per 256 weights                                         */
/*   [0,2) d f16, [2,4) dmin f16, [4,16) 12 bytes of 6-bit scales/mins,     */
/*   [16,144) 128 bytes of 4-bit codes.                                     */
/* Sub-block j (32 weights) reads code byte 32*(j/2)+l, low nibble for even */
/* j, high for odd j. Scale/min packing: bytes 0..3 hold sc0..3 in bits     */
/* 0-5, bytes 4..7 hold m0..3 in bits 0-5; bytes 8..11 hold the low nibbles */
/* of sc4..7 (bits 0-3) and m4..7 (bits 4-7); the top two bits of sc4..7   */
/* and m4..7 sit in bits 6-7 of bytes 0..3 and 4..7 respectively.          */
/* ---------------------------------------------------------------------- */
void synth_pack_q4k_scales(const uint8_t sc[8], const uint8_t mn[8], uint8_t out[12]) {
    memset(out, 0, 12);
    for (int j = 0; j < 4; ++j) {
        out[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        out[j + 4] = (uint8_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
        out[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
}

static void enc_q4k(const float *w, uint8_t *b) {
    float scale[8], minv[8];
    float maxscale = 0.0f, maxmin = 0.0f;
    for (int j = 0; j < 8; ++j) {
        float lo = 0.0f, hi = -INFINITY;
        for (int l = 0; l < 32; ++l) {
            float v = w[32 * j + l];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        scale[j] = (hi - lo) / 15.0f;
        minv[j] = -lo;
        if (scale[j] > maxscale) maxscale = scale[j];
        if (minv[j] > maxmin) maxmin = minv[j];
    }
    uint16_t dh = synth_f32_to_f16(maxscale / 63.0f);
    uint16_t mh = synth_f32_to_f16(maxmin / 63.0f);
    float d = h2f(dh), dmin = h2f(mh);
    uint8_t sc[8], mn[8];
    for (int j = 0; j < 8; ++j) {
        sc[j] = (uint8_t)(d > 0.0f ? clampi((int)rnd(scale[j] / d), 0, 63) : 0);
        mn[j] = (uint8_t)(dmin > 0.0f ? clampi((int)rnd(minv[j] / dmin), 0, 63) : 0);
    }
    b[0] = (uint8_t)(dh & 0xFF); b[1] = (uint8_t)(dh >> 8);
    b[2] = (uint8_t)(mh & 0xFF); b[3] = (uint8_t)(mh >> 8);
    synth_pack_q4k_scales(sc, mn, b + 4);
    uint8_t *qs = b + 16;
    memset(qs, 0, 128);
    for (int j = 0; j < 8; ++j) {
        float ds = d * (float)sc[j];
        float dm = dmin * (float)mn[j];
        for (int l = 0; l < 32; ++l) {
            int q = ds > 0.0f ? clampi((int)rnd((w[32 * j + l] + dm) / ds), 0, 15) : 0;
            qs[32 * (j / 2) + l] |= (uint8_t)((j & 1) ? (q << 4) : q);
        }
    }
}

int synth_encode_q4k(const float *w, int64_t rows, int64_t k, uint8_t *out) {
    if (k % 256) return -1;
    int64_t nb = k / 256;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) enc_q4k(w + r * k + b * 256, out + (r * nb + b) * 144);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Q6_K: 210 bytes per 256 weights                                         */
/*   [0,128) ql low nibbles, [128,192) qh 2-bit highs, [192,208) 16 int8    */
/*   sub-scales, [208,210) d f16.                                           */
/* Weight i: h=i/128, p=i%128, g=p/32, l=p%32; low4 = nibble of             */
/* ql[64h+l+32*(g%2)] (low nibble if g<2), high2 = (qh[32h+l] >> 2g) & 3,   */
/* q = low4 | high2<<4 in [0,63], value d*sc[i/16]*(q-32).                  */
/* ---------------------------------------------------------------------- */
void synth_pack_q6k_codes(const uint8_t q[256], uint8_t ql[128], uint8_t qh[64]) {
    memset(ql, 0, 128);
    memset(qh, 0, 64);
    for (int i = 0; i < 256; ++i) {
        int h = i / 128, p = i % 128, g = p / 32, l = p % 32;
        int lo = q[i] & 15, hi = (q[i] >> 4) & 3;
        ql[64 * h + l + 32 * (g % 2)] |= (uint8_t)(g < 2 ? lo : (lo << 4));
        qh[32 * h + l] |= (uint8_t)(hi << (2 * g));
    }
}

static void enc_q6k(const float *w, uint8_t *b) {
    float s[16], smax = 0.0f;
    for (int t = 0; t < 16; ++t) {
        float a = 0.0f;
        for (int l = 0; l < 16; ++l) { float v = fabsf(w[16 * t + l]); if (v > a) a = v; }
        s[t] = a / 31.0f;
        if (s[t] > smax) smax = s[t];
    }
    uint16_t dh = synth_f32_to_f16(smax / 127.0f);
    float d = h2f(dh);
    int8_t sc[16];
    for (int t = 0; t < 16; ++t) sc[t] = (int8_t)(d > 0.0f ? clampi((int)rnd(s[t] / d), -128, 127) : 0);
    uint8_t q[256];
    for (int i = 0; i < 256; ++i) {
        float ds = d * (float)sc[i / 16];
        q[i] = (uint8_t)(ds != 0.0f ? clampi((int)rnd(w[i] / ds) + 32, 0, 63) : 32);
    }
    synth_pack_q6k_codes(q, b, b + 128);
    memcpy(b + 192, sc, 16);
    b[208] = (uint8_t)(dh & 0xFF);
    b[209] = (uint8_t)(dh >> 8);
}

int synth_encode_q6k(const float *w, int64_t rows, int64_t k, uint8_t *out) {
    if (k % 256) return -1;
    int64_t nb = k / 256;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) enc_q6k(w + r * k + b * 256, out + (r * nb + b) * 210);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Q4_0: 18 bytes per 32 weights = f16 d, 16 bytes of 4-bit codes; byte j   */
/* holds weight j (low nibble) and weight j + 16 (high nibble),             */
/* w = d * (q - 8). Encoder: the weight of largest magnitude m (with its    */
/* sign) maps to code 0, d = m / -8; q = clamp(round(w / d) + 8, 0, 15).     */
/* ---------------------------------------------------------------------- */
static void enc_q4_0(const float *w, uint8_t *b) {
    float m = 0.0f;
    for (int i = 0; i < 32; ++i)
        if (fabsf(w[i]) > fabsf(m)) m = w[i];
    uint16_t dh = synth_f32_to_f16(m / -8.0f);
    float d = h2f(dh);
    b[0] = (uint8_t)(dh & 0xFF); b[1] = (uint8_t)(dh >> 8);
    for (int j = 0; j < 16; ++j) {
        int q0 = d != 0.0f ? clampi((int)rnd(w[j] / d) + 8, 0, 15) : 8;
        int q1 = d != 0.0f ? clampi((int)rnd(w[j + 16] / d) + 8, 0, 15) : 8;
        b[2 + j] = (uint8_t)(q0 | (q1 << 4));
    }
}

int synth_encode_q4_0(const float *w, int64_t rows, int64_t k, uint8_t *out) {
    if (k % 32) return -1;
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) enc_q4_0(w + r * k + b * 32, out + (r * nb + b) * 18);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Q5_K: 176 bytes per 256 weights                                         */
/*   [0,2) d f16, [2,4) dmin f16, [4,16) scales as Q4_K, [16,48) qh,        */
/*   [48,176) qs. Sub-block j: low 4 bits of weight 32j+l from              */
/*   qs[32*(j/2)+l] (low nibble for even j, high for odd), bit 4 from bit j */
/*   of qh[l]; w = d*sc_j*q - dmin*m_j, q in [0, 31]. Encoder: the Q4_K     */
/*   min/max quantizer with 31 levels.                                      */
/* ---------------------------------------------------------------------- */
static void enc_q5k(const float *w, uint8_t *b) {
    float scale[8], minv[8];
    float maxscale = 0.0f, maxmin = 0.0f;
    for (int j = 0; j < 8; ++j) {
        float lo = 0.0f, hi = -INFINITY;
        for (int l = 0; l < 32; ++l) {
            float v = w[32 * j + l];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        scale[j] = (hi - lo) / 31.0f;
        minv[j] = -lo;
        if (scale[j] > maxscale) maxscale = scale[j];
        if (minv[j] > maxmin) maxmin = minv[j];
    }
    uint16_t dh = synth_f32_to_f16(maxscale / 63.0f);
    uint16_t mh = synth_f32_to_f16(maxmin / 63.0f);
    float d = h2f(dh), dmin = h2f(mh);
    uint8_t sc[8], mn[8];
    for (int j = 0; j < 8; ++j) {
        sc[j] = (uint8_t)(d > 0.0f ? clampi((int)rnd(scale[j] / d), 0, 63) : 0);
        mn[j] = (uint8_t)(dmin > 0.0f ? clampi((int)rnd(minv[j] / dmin), 0, 63) : 0);
    }
    b[0] = (uint8_t)(dh & 0xFF); b[1] = (uint8_t)(dh >> 8);
    b[2] = (uint8_t)(mh & 0xFF); b[3] = (uint8_t)(mh >> 8);
    synth_pack_q4k_scales(sc, mn, b + 4);
    uint8_t *qh = b + 16, *qs = b + 48;
    memset(qh, 0, 32);
    memset(qs, 0, 128);
    for (int j = 0; j < 8; ++j) {
        float ds = d * (float)sc[j];
        float dm = dmin * (float)mn[j];
        for (int l = 0; l < 32; ++l) {
            int q = ds > 0.0f ? clampi((int)rnd((w[32 * j + l] + dm) / ds), 0, 31) : 0;
            qs[32 * (j / 2) + l] |= (uint8_t)((j & 1) ? ((q & 15) << 4) : (q & 15));
            qh[l] |= (uint8_t)((q >> 4) << j);
        }
    }
}

int synth_encode_q5k(const float *w, int64_t rows, int64_t k, uint8_t *out) {
    if (k % 256) return -1;
    int64_t nb = k / 256;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) enc_q5k(w + r * k + b * 256, out + (r * nb + b) * 176);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Whole weight matrices straight from the seed, row-chunked so that no     */
/* full f32 copy of a large matrix is ever held. Element (r, c) of a        */
/* [rows, k] matrix is uniform counter r*k + c of stream `seed`.            */
/* fmt: 0 = Q8_0, 1 = Q4_K, 2 = Q6_K, 3 = Q4_0, 4 = Q5_K.                   */
/* ---------------------------------------------------------------------- */
static const int64_t BLK_W[5] = {32, 256, 256, 32, 256};
static const int64_t BLK_B[5] = {34, 144, 210, 18, 176};

int64_t synth_row_bytes(int fmt, int64_t k) {
    if (fmt < 0 || fmt > 4 || k % BLK_W[fmt]) return -1;
    return k / BLK_W[fmt] * BLK_B[fmt];
}

int synth_weights(int fmt, uint64_t seed, int64_t rows, int64_t k, uint8_t *out) {
    int64_t rb = synth_row_bytes(fmt, k);
    if (rb < 0) return -1;
#pragma omp parallel
    {
        float wrow[65536];
        float *buf = k <= 65536 ? wrow : 0;
        if (buf) {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < rows; ++r) {
                for (int64_t c = 0; c < k; ++c) buf[c] = unif(ctr(seed, (uint64_t)(r * k + c)));
                uint8_t *o = out + r * rb;
                int64_t nb = k / BLK_W[fmt];
                for (int64_t b = 0; b < nb; ++b) {
                    const float *wb = buf + b * BLK_W[fmt];
                    if (fmt == 0) enc_q8_0(wb, o + b * 34);
                    else if (fmt == 1) enc_q4k(wb, o + b * 144);
                    else if (fmt == 2) enc_q6k(wb, o + b * 210);
                    else if (fmt == 3) enc_q4_0(wb, o + b * 18);
                    else enc_q5k(wb, o + b * 176);
                }
            }
        }
    }
    return k <= 65536 ? 0 : -2;
}

/* Random raw blocks: every byte drawn from the counter stream, then the f16
 * scale fields overwritten with finite values (magnitudes about 2^-10..2^5)
 * so that no NaN/Inf scale is produced. Exercises every code, every 6-bit
 * scale/min and negative Q6_K sub-scales. Every `subnormal_every`-th block
 * (0 = none) gets subnormal f16 scales instead. */
static uint16_t rand_half(uint64_t c, int subnormal) {
    uint64_t z = mix64(c);
    uint16_t sign = (uint16_t)((z >> 63) << 15);
    if (subnormal) return (uint16_t)(sign | (uint16_t)(1 + (z % 1023)));
    /* exponent 5..20 => magnitudes about 2^-10 .. 2^5, mantissa random */
    uint16_t e = (uint16_t)(5 + (z >> 20) % 16);
    uint16_t m = (uint16_t)((z >> 40) & 1023);
    return (uint16_t)(sign | (e << 10) | m);
}

int synth_random_blocks(int fmt, uint64_t seed, int64_t nblocks, int subnormal_every, uint8_t *out) {
    if (fmt < 0 || fmt > 4) return -1;
    int64_t bb = BLK_B[fmt];
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; ++b) {
        uint8_t *o = out + b * bb;
        for (int64_t i = 0; i < bb; ++i) o[i] = (uint8_t)(mix64(ctr(seed, (uint64_t)(b * bb + i))) >> 56);
        int sub = subnormal_every > 0 && (b % subnormal_every) == 0;
        uint64_t c = ctr(seed ^ 0x5A5Aull, (uint64_t)b * 2);
        if (fmt == 0 || fmt == 3) {
            uint16_t h = rand_half(c, sub);
            o[0] = (uint8_t)h; o[1] = (uint8_t)(h >> 8);
        } else if (fmt == 1 || fmt == 4) {
            uint16_t h0 = rand_half(c, sub), h1 = rand_half(c + 1, sub);
            h0 &= 0x7FFF; h1 &= 0x7FFF; /* d and dmin non-negative as an encoder would emit */
            o[0] = (uint8_t)h0; o[1] = (uint8_t)(h0 >> 8);
            o[2] = (uint8_t)h1; o[3] = (uint8_t)(h1 >> 8);
        } else {
            uint16_t h = rand_half(c, sub);
            o[208] = (uint8_t)h; o[209] = (uint8_t)(h >> 8);
        }
    }
    return 0;
}
