// Per-lane block decoders for the raw GGML layouts (gfx950).
//
// A row of a weight matrix is cut into "units" that one lane decodes and
// dots against activation values it keeps in registers:
//   Q8_0: a unit is a pair of consecutive 34-byte blocks (68 bytes, dword
//         aligned when k % 64 == 0), 64 weights.
//   Q4_K: a unit is one 16-byte run of the 128 code bytes of a superblock
//         (chunk c = 0..7), i.e. 16 weights of sub-block 2*(c/2) (low
//         nibbles) and 16 of sub-block 2*(c/2)+1 (high nibbles), plus the
//         superblock's 16-byte header (d, dmin, packed scales).
//   Q6_K: a unit is (half h, quarter lq) of a superblock: for each of the
//         four 32-weight groups g of half h the 8 weights l = 8*lq..8*lq+7,
//         32 weights in all, read from 8 bytes of ql (twice), 8 of qh,
//         the 8 sub-scales of the half and d.
// Weight value conventions (block layouts: hanzo-ml `src/vulkan_backend.rs`,
// `quantize_q8_blocks`, `quantize_q4k_split`, `quantize_q6k_split`; bit
// packing inside fields: public GGML k-quants):
//   Q8_0 w = d*q;  Q4_K w = d*sc_j*q - dmin*m_j;  Q6_K w = d*sc_t*(q-32).
#pragma once

#include "common.hpp"

// 16-byte vector with only dword alignment promised (Q8_0 pairs start at
// 68-byte steps); gfx950 global loads need dword alignment only.
typedef uint32_t v4u_a4 __attribute__((ext_vector_type(4), aligned(4)));

// ---------------------------------------------------------------- Q8_0 ---
struct Q8Pair {
    uint32_t d[17];
};

QMV_DEV void q8_load(Q8Pair &P, const uint8_t *p) {
    const v4u_a4 *v = reinterpret_cast<const v4u_a4 *>(p);
    v4u_a4 a = v[0], b = v[1], c = v[2], e = v[3];
    P.d[0] = a.x; P.d[1] = a.y; P.d[2] = a.z; P.d[3] = a.w;
    P.d[4] = b.x; P.d[5] = b.y; P.d[6] = b.z; P.d[7] = b.w;
    P.d[8] = c.x; P.d[9] = c.y; P.d[10] = c.z; P.d[11] = c.w;
    P.d[12] = e.x; P.d[13] = e.y; P.d[14] = e.z; P.d[15] = e.w;
    P.d[16] = reinterpret_cast<const uint32_t *>(p)[16];
}

// x holds the 64 activation values of the pair.
QMV_DEV float q8_pair_dot(const Q8Pair &P, const float *x) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t qa = funnel(P.d[t + 1], P.d[t], 2);  // codes of block A start at byte 2
        uint32_t qb = P.d[9 + t];                     // codes of block B start at byte 36
        a = fmaf(sbyte_f<0>(qa), x[4 * t + 0], a);
        a = fmaf(sbyte_f<1>(qa), x[4 * t + 1], a);
        a = fmaf(sbyte_f<2>(qa), x[4 * t + 2], a);
        a = fmaf(sbyte_f<3>(qa), x[4 * t + 3], a);
        b = fmaf(sbyte_f<0>(qb), x[32 + 4 * t + 0], b);
        b = fmaf(sbyte_f<1>(qb), x[32 + 4 * t + 1], b);
        b = fmaf(sbyte_f<2>(qb), x[32 + 4 * t + 2], b);
        b = fmaf(sbyte_f<3>(qb), x[32 + 4 * t + 3], b);
    }
    float da = h2f(P.d[0]);
    float db = h2f(P.d[8] >> 16);
    return da * a + db * b;
}

// ---------------------------------------------------------------- Q4_K ---
// Activation registers of one Q4_K unit: the 16 values under the low
// nibbles (sub-block 2p, l = 16hh..16hh+15), the 16 under the high nibbles
// (sub-block 2p+1) and their sums.
struct Q4KX {
    float lo[16], hi[16];
    float slo, shi;
};

// s: superblock index within the row, c: chunk 0..7.
QMV_DEV void q4k_load_x(Q4KX &X, const float *x, int s, int c) {
    const int p = c >> 1, hh = c & 1;
    const float4 *a = reinterpret_cast<const float4 *>(x + 256 * s + 64 * p + 16 * hh);
    const float4 *b = reinterpret_cast<const float4 *>(x + 256 * s + 64 * p + 32 + 16 * hh);
    float sl = 0.0f, sh = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float4 u = a[t], v = b[t];
        X.lo[4 * t] = u.x; X.lo[4 * t + 1] = u.y; X.lo[4 * t + 2] = u.z; X.lo[4 * t + 3] = u.w;
        X.hi[4 * t] = v.x; X.hi[4 * t + 1] = v.y; X.hi[4 * t + 2] = v.z; X.hi[4 * t + 3] = v.w;
        sl += (u.x + u.y) + (u.z + u.w);
        sh += (v.x + v.y) + (v.z + v.w);
    }
    X.slo = sl;
    X.shi = sh;
}

// 6-bit scales and mins of sub-blocks 2p and 2p+1 from the header dwords
// m1 = scales[0..3], m2 = scales[4..7], m3 = scales[8..11]:
//   j < 4 : sc = s[j] & 63,                   m = s[j+4] & 63
//   j >= 4: sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
//           m  = (s[j+4] >> 4) | (s[j]   >> 6) << 4
// Both sub-blocks of the pair use bytes 2*(p%2) and 2*(p%2)+1 of the dwords.
// Returns sc_lo | sc_hi << 8 in *sc2 and m_lo | m_hi << 8 in *mn2.
QMV_DEV void q4k_scales(uint32_t m1, uint32_t m2, uint32_t m3, int p, uint32_t *sc2, uint32_t *mn2) {
    const uint32_t sh = (uint32_t)(p & 1) * 16u;
    const uint32_t A = (m1 >> sh) & 0xFFFFu, B = (m2 >> sh) & 0xFFFFu, C = (m3 >> sh) & 0xFFFFu;
    if (p < 2) {
        *sc2 = A & 0x3F3Fu;
        *mn2 = B & 0x3F3Fu;
    } else {
        *sc2 = (C & 0x0F0Fu) | ((A >> 2) & 0x3030u);
        *mn2 = ((C >> 4) & 0x0F0Fu) | ((B >> 2) & 0x3030u);
    }
}

// Partial dot of one Q4_K unit: q = the 16 code bytes, m = the 16 header bytes.
QMV_DEV float q4k_unit_dot(uint4 q, uint4 m, const Q4KX &X, int p) {
    float alo = 0.0f, ahi = 0.0f;
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t lo = qw[t] & 0x0F0F0F0Fu;
        const uint32_t hi = qw[t] & 0xF0F0F0F0u;  // 16*q per byte, 1/16 folded below
        alo = fmaf(ubyte_f<0>(lo), X.lo[4 * t + 0], alo);
        alo = fmaf(ubyte_f<1>(lo), X.lo[4 * t + 1], alo);
        alo = fmaf(ubyte_f<2>(lo), X.lo[4 * t + 2], alo);
        alo = fmaf(ubyte_f<3>(lo), X.lo[4 * t + 3], alo);
        ahi = fmaf(ubyte_f<0>(hi), X.hi[4 * t + 0], ahi);
        ahi = fmaf(ubyte_f<1>(hi), X.hi[4 * t + 1], ahi);
        ahi = fmaf(ubyte_f<2>(hi), X.hi[4 * t + 2], ahi);
        ahi = fmaf(ubyte_f<3>(hi), X.hi[4 * t + 3], ahi);
    }
    uint32_t sc2, mn2;
    q4k_scales(m.y, m.z, m.w, p, &sc2, &mn2);
    const float d = h2f(m.x), dmin = h2f(m.x >> 16);
    const float dlo = d * ubyte_f<0>(sc2);
    const float dhi = d * ubyte_f<1>(sc2);
    const float mlo = dmin * ubyte_f<0>(mn2);
    const float mhi = dmin * ubyte_f<1>(mn2);
    float r = dlo * alo;
    r = fmaf(dhi, ahi * 0.0625f, r);
    r = fmaf(-mlo, X.slo, r);
    r = fmaf(-mhi, X.shi, r);
    return r;
}

// ---------------------------------------------------------------- Q6_K ---
// Activation registers of one Q6_K unit: for group g = 0..3 the 8 values at
// 128h + 32g + 8lq + t, and their sums.
struct Q6KX {
    float v[4][8];
    float s[4];
};

QMV_DEV void q6k_load_x(Q6KX &X, const float *x, int sb, int u) {
    const int h = u >> 2, lq = u & 3;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float4 *a = reinterpret_cast<const float4 *>(x + 256 * sb + 128 * h + 32 * g + 8 * lq);
        float4 p0 = a[0], p1 = a[1];
        X.v[g][0] = p0.x; X.v[g][1] = p0.y; X.v[g][2] = p0.z; X.v[g][3] = p0.w;
        X.v[g][4] = p1.x; X.v[g][5] = p1.y; X.v[g][6] = p1.z; X.v[g][7] = p1.w;
        X.s[g] = ((p0.x + p0.y) + (p0.z + p0.w)) + ((p1.x + p1.y) + (p1.z + p1.w));
    }
}

// Raw dwords of one Q6_K unit, fetched with dword-aligned loads; the
// superblock itself may start at any even byte (210-byte blocks).
struct Q6KRaw {
    uint32_t a[3], b[3], hq[3], sc[3];
    uint32_t d;
    uint32_t sa;  // byte misalignment of the superblock start (0 or 2)
};

// Load 8 bytes starting at the even address p as 3 aligned dwords; the third
// is read only when p is not dword aligned (otherwise it would step past a
// field that ends at the last byte of the buffer).
QMV_DEV void ld8u(uint32_t out[3], const uint8_t *p) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t *b = reinterpret_cast<const uint32_t *>(a & ~(uintptr_t)3);
    const uint32_t off3 = (a & 3) ? 2u : 1u;
    out[0] = b[0];
    out[1] = b[1];
    out[2] = b[off3];
}

QMV_DEV void q6k_load(Q6KRaw &R, const uint8_t *blk, int u) {
    const int h = u >> 2, lq = u & 3;
    ld8u(R.a, blk + 64 * h + 8 * lq);
    ld8u(R.b, blk + 64 * h + 32 + 8 * lq);
    ld8u(R.hq, blk + 128 + 32 * h + 8 * lq);
    ld8u(R.sc, blk + 192 + 8 * h);
    R.d = ld2(blk + 208);
    R.sa = (uint32_t)((uintptr_t)blk & 3);
}

QMV_DEV float q6k_unit_dot(const Q6KRaw &R, const Q6KX &X, int u) {
    const uint32_t s = R.sa;
    const uint32_t A[2] = {funnel(R.a[1], R.a[0], s), funnel(R.a[2], R.a[1], s)};
    const uint32_t Bq[2] = {funnel(R.b[1], R.b[0], s), funnel(R.b[2], R.b[1], s)};
    const uint32_t H[2] = {funnel(R.hq[1], R.hq[0], s), funnel(R.hq[2], R.hq[1], s)};
    const uint32_t S0 = funnel(R.sc[1], R.sc[0], s), S1 = funnel(R.sc[2], R.sc[1], s);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t q0 = (A[w] & 0x0F0F0F0Fu) | ((H[w] << 4) & 0x30303030u);
        const uint32_t q1 = (Bq[w] & 0x0F0F0F0Fu) | ((H[w] << 2) & 0x30303030u);
        const uint32_t q2 = ((A[w] >> 4) & 0x0F0F0F0Fu) | (H[w] & 0x30303030u);
        const uint32_t q3 = ((Bq[w] >> 4) & 0x0F0F0F0Fu) | ((H[w] >> 2) & 0x30303030u);
        const uint32_t qq[4] = {q0, q1, q2, q3};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            acc[g] = fmaf(ubyte_f<0>(qq[g]), X.v[g][4 * w + 0], acc[g]);
            acc[g] = fmaf(ubyte_f<1>(qq[g]), X.v[g][4 * w + 1], acc[g]);
            acc[g] = fmaf(ubyte_f<2>(qq[g]), X.v[g][4 * w + 2], acc[g]);
            acc[g] = fmaf(ubyte_f<3>(qq[g]), X.v[g][4 * w + 3], acc[g]);
        }
    }
    // sub-scale of group g: sc[8h + 2g + lq/2] = byte 2g + lq/2 of {S1:S0}
    const uint32_t bsel = (uint32_t)((u & 3) >> 1) * 8u;
    const float d = h2f(R.d);
    const float sc0 = (float)(int8_t)((S0 >> bsel) & 0xFFu);
    const float sc1 = (float)(int8_t)((S0 >> (bsel + 16u)) & 0xFFu);
    const float sc2 = (float)(int8_t)((S1 >> bsel) & 0xFFu);
    const float sc3 = (float)(int8_t)((S1 >> (bsel + 16u)) & 0xFFu);
    float r = sc0 * fmaf(-32.0f, X.s[0], acc[0]);
    r = fmaf(sc1, fmaf(-32.0f, X.s[1], acc[1]), r);
    r = fmaf(sc2, fmaf(-32.0f, X.s[2], acc[2]), r);
    r = fmaf(sc3, fmaf(-32.0f, X.s[3], acc[3]), r);
    return d * r;
}
