// Per-lane block decoders for the raw GGML layouts (gfx950).
//
// A weight row is cut into "units" of 64 weights that one lane decodes and
// dots against 64 activation values it holds in registers (four runs of 16
// consecutive values, X[16*g + t]):
//   Q8_0: unit u = blocks 2u, 2u+1 (68 bytes, dword aligned when k % 64 == 0);
//         runs at 64u + 16g.
//   Q4_K: unit u = (superblock s = u/4, pair p = u%4): the 32 code bytes
//         qs[32p .. 32p+32) (low nibbles = sub-block 2p, high = 2p+1) and the
//         16-byte header (d, dmin, packed 6-bit scales/mins); runs at
//         256s + 64p + 16g (runs 0,1 under the low nibbles, 2,3 under the high).
//   Q6_K: unit u = (superblock s = u/4, half h = (u%4)/2, lh = u%2): for the
//         four 32-weight groups g of half h the 16 weights l = 16lh..16lh+15,
//         from 16 bytes of ql (twice), 16 of qh, the sub-scales and d; runs at
//         256s + 128h + 32g + 16lh. Q6_K superblocks are 210 bytes, so these
//         fields sit at any even address: they are read with dword loads at
//         2-byte alignment (gfx950 global loads handle unaligned addresses).
// Weight values (block layouts: hanzo-ml `src/vulkan_backend.rs`,
// `quantize_q8_blocks`, `quantize_q4k_split`, `quantize_q6k_split`; bit
// packing inside fields: public GGML k-quants):
//   Q8_0 w = d*q;  Q4_K w = d*sc_j*q - dmin*m_j;  Q6_K w = d*sc_t*(q-32).
#pragma once

#include "common.hpp"

// 16-byte vector with only dword alignment promised (Q8_0 pairs start at
// 68-byte steps); gfx950 global loads need dword alignment only.
typedef uint32_t v4u_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Two nibble codes (bytes 0..15) of one 16-bit half of a dword -> f32 pair.
// gfx950 v_cvt_pk_f32_fp8 reads the bytes as OCP E4M3; a byte q in 0..15 is
// the E4M3 value q * 2^-9 exactly (subnormal for q < 8), so the pair comes
// back as (q0, q1) * 2^-9 and the 2^9 is folded into the block scale.
QMV_DEV float2 nib2f_lo(uint32_t v) {
    auto r = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false);
    return make_float2(r[0], r[1]);
}
QMV_DEV float2 nib2f_hi(uint32_t v) {
    auto r = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, true);
    return make_float2(r[0], r[1]);
}

// Activation registers of one unit: 64 values and the sums of the 4 runs.
struct UnitX {
    float v[64];
    float s[4];
};

QMV_DEV void load_x_runs(UnitX &X, const float *x, int r0, int r1, int r2, int r3) {
    const int base[4] = {r0, r1, r2, r3};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float4 *a = reinterpret_cast<const float4 *>(x + base[g]);
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float4 q = a[t];
            X.v[16 * g + 4 * t + 0] = q.x;
            X.v[16 * g + 4 * t + 1] = q.y;
            X.v[16 * g + 4 * t + 2] = q.z;
            X.v[16 * g + 4 * t + 3] = q.w;
            acc += (q.x + q.y) + (q.z + q.w);
        }
        X.s[g] = acc;
    }
}

// Activation staging in LDS: unit u's 64 values (in X.v order) sit at float
// offset XSTRIDE*u; the 4-float pad makes the 16-byte reads of 8 consecutive
// lanes (consecutive units) fall in disjoint LDS banks, and the dense
// matvecs keep the unit's four 16-value sums (X.s) in it, computed once per
// workgroup while staging instead of by every lane that reads the unit.
constexpr int XSTRIDE = 68;

QMV_DEV void load_x_lds(UnitX &X, const float *xl, int u) {
    const float4 *a = reinterpret_cast<const float4 *>(xl + XSTRIDE * u);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float4 q = a[4 * g + t];
            X.v[16 * g + 4 * t + 0] = q.x;
            X.v[16 * g + 4 * t + 1] = q.y;
            X.v[16 * g + 4 * t + 2] = q.z;
            X.v[16 * g + 4 * t + 3] = q.w;
            acc += (q.x + q.y) + (q.z + q.w);
        }
        X.s[g] = acc;
    }
}

// Cooperative fill of the staged layout from x[0..k), in two phases so the
// global loads can be issued before the weight loads (a wait for them then
// does not wait for the weights): fetch() loads this thread's float4 granules
// (at most STAGE_MAX of them, k <= 4*256*STAGE_MAX), store() writes them to
// their slots. A granule never straddles two runs.
// Row passes each wave keeps in flight, per format (measured).
#ifndef QMV_RING_Q8
#define QMV_RING_Q8 1
#endif
#ifndef QMV_RING_Q4K
#define QMV_RING_Q4K 1
#endif
#ifndef QMV_RING_Q6K
#define QMV_RING_Q6K 2
#endif
#ifndef QMV_RING_Q4KQ8
#define QMV_RING_Q4KQ8 1
#endif

constexpr int STAGE_MAX = 8;

// Native vector types: HIP's float4/uint4 wrapper structs are copied with
// memcpy, which keeps a private-memory (scratch) copy alive here.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef f32x4 StageRegs[STAGE_MAX];

// Indices past the end are clamped to the last granule (loaded and stored
// again, harmlessly), which keeps both phases branch-free and in registers.
// Granules (16 bytes of x per thread of a 256-thread block) that a row of
// k <= 64*G*UPL activations needs: k/4 float4 over 256 threads.
constexpr int stage_granules(int G, int UPL) {
    return G * UPL / 16 < 1 ? 1 : (G * UPL / 16 > STAGE_MAX ? STAGE_MAX : G * UPL / 16);
}
template <int NS>
QMV_DEV void fetch_x(StageRegs &S, const float *x, int k) {
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
    const int last = k / 4 - 1;
#pragma unroll
    for (int m = 0; m < NS; ++m) S[m] = x4[min((int)threadIdx.x + 256 * m, last)];
}

template <class F, int NS>
QMV_DEV void store_x(float *xl, const StageRegs &S, int k) {
    const int last = k / 4 - 1;
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int i4 = min((int)threadIdx.x + 256 * m, last);
        int j;
        const int u = F::xslot(4 * i4, &j);
        *reinterpret_cast<f32x4 *>(xl + XSTRIDE * u + j) = S[m];
    }
}

// staging with the four 16-value run sums of each unit written into its pad
// (a run is 4 consecutive granules, held by 4 consecutive lanes)
template <class F, int NS>
QMV_DEV void store_x_sums(float *xl, const StageRegs &S, int k) {
    const int last = k / 4 - 1;
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int i4r = (int)threadIdx.x + 256 * m;
        const int i4 = min(i4r, last);
        int j;
        const int u = F::xslot(4 * i4, &j);
        *reinterpret_cast<f32x4 *>(xl + XSTRIDE * u + j) = S[m];
        float v = (S[m].x + S[m].y) + (S[m].z + S[m].w);
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        if ((threadIdx.x & 3) == 0 && i4r <= last) xl[XSTRIDE * u + 64 + (j >> 4)] = v;
    }
}
QMV_DEV void load_x_lds_pre(UnitX &X, const float *xl, int u) {
    const float4 *a = reinterpret_cast<const float4 *>(xl + XSTRIDE * u);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
        const float4 q = a[g];
        X.v[4 * g + 0] = q.x;
        X.v[4 * g + 1] = q.y;
        X.v[4 * g + 2] = q.z;
        X.v[4 * g + 3] = q.w;
    }
    const float4 sm = a[16];
    X.s[0] = sm.x;
    X.s[1] = sm.y;
    X.s[2] = sm.z;
    X.s[3] = sm.w;
}

// f32 activation pack and its per-unit staging (shared by the f32 units).
struct ActF32 {
    const float *x;
};

template <class F>
struct F32Act {
    static constexpr bool Q8 = false;  // activation: f32 rows
    using Act = ActF32;
    using X = UnitX;
    using Stage = StageRegs;
    static constexpr int ACT_STRIDE = XSTRIDE;
    template <int NS>
    static __device__ __forceinline__ void fetch(Stage &S, ActF32 a, int k) { fetch_x<NS>(S, a.x, k); }
    template <int NS>
    static __device__ __forceinline__ void store(float *xl, const Stage &S, int k) { store_x<F, NS>(xl, S, k); }
    static __device__ __forceinline__ void load_lds(UnitX &X, const float *xl, int u) { load_x_lds(X, xl, u); }
    template <int NS>
    static __device__ __forceinline__ void store_s(float *xl, const Stage &S, int k) { store_x_sums<F, NS>(xl, S, k); }
    static __device__ __forceinline__ void load_lds_s(UnitX &X, const float *xl, int u) { load_x_lds_pre(X, xl, u); }
};

// ---------------------------------------------------------------- Q8_0 ---
struct Q8Unit : F32Act<Q8Unit> {
    static constexpr int BW = 32, BB = 34;
    static constexpr int RING = QMV_RING_Q8;  // row passes in flight per wave (measured best)
    static constexpr int MAX_WG_PER_CU = 2;   // resident workgroups per CU at most (measured)
    static constexpr int UNITS_PER_BLOCKS = 2;  // informational
    struct Raw {
        uint32_t d[17];
    };
    static __device__ __forceinline__ int units_per_row(int k) { return k / 64; }
    static __device__ __forceinline__ void load_x(UnitX &X, const float *x, int u) {
        load_x_runs(X, x, 64 * u, 64 * u + 16, 64 * u + 32, 64 * u + 48);
    }
    // activation index i -> (unit, position within the unit's 64 values)
    static __device__ __forceinline__ int xslot(int i, int *j) {
        *j = i & 63;
        return i >> 6;
    }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) {
        const uint8_t *p = row + 68 * u;
        const v4u_a4 *v = reinterpret_cast<const v4u_a4 *>(p);
        const v4u_a4 a = v[0], b = v[1], c = v[2], e = v[3];
        R.d[0] = a.x; R.d[1] = a.y; R.d[2] = a.z; R.d[3] = a.w;
        R.d[4] = b.x; R.d[5] = b.y; R.d[6] = b.z; R.d[7] = b.w;
        R.d[8] = c.x; R.d[9] = c.y; R.d[10] = c.z; R.d[11] = c.w;
        R.d[12] = e.x; R.d[13] = e.y; R.d[14] = e.z; R.d[15] = e.w;
        R.d[16] = reinterpret_cast<const uint32_t *>(p)[16];
    }
    static __device__ __forceinline__ float dot(const Raw &R, const UnitX &X, int) {
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t qa = funnel(R.d[t + 1], R.d[t], 2);  // block A codes start at byte 2
            const uint32_t qb = R.d[9 + t];                     // block B codes start at byte 36
            a = fmaf(sbyte_f<0>(qa), X.v[4 * t + 0], a);
            a = fmaf(sbyte_f<1>(qa), X.v[4 * t + 1], a);
            a = fmaf(sbyte_f<2>(qa), X.v[4 * t + 2], a);
            a = fmaf(sbyte_f<3>(qa), X.v[4 * t + 3], a);
            b = fmaf(sbyte_f<0>(qb), X.v[32 + 4 * t + 0], b);
            b = fmaf(sbyte_f<1>(qb), X.v[32 + 4 * t + 1], b);
            b = fmaf(sbyte_f<2>(qb), X.v[32 + 4 * t + 2], b);
            b = fmaf(sbyte_f<3>(qb), X.v[32 + 4 * t + 3], b);
        }
        return h2f(R.d[0]) * a + h2f(R.d[8] >> 16) * b;
    }
};

// ---------------------------------------------------------------- Q4_K ---
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

#ifndef QMV_WG_Q4K
#define QMV_WG_Q4K 3
#endif
struct Q4KUnit : F32Act<Q4KUnit> {
    static constexpr int BW = 256, BB = 144;
    static constexpr int RING = QMV_RING_Q4K;
    static constexpr int MAX_WG_PER_CU = QMV_WG_Q4K;
    struct Raw {
        uint4 q0, q1, m;
    };
    static __device__ __forceinline__ int units_per_row(int k) { return (k / 256) * 4; }
    static __device__ __forceinline__ void load_x(UnitX &X, const float *x, int u) {
        const int b = 256 * (u >> 2) + 64 * (u & 3);
        load_x_runs(X, x, b, b + 16, b + 32, b + 48);
    }
    // unit (s, p) covers x[256s + 64p, +64) in order
    static __device__ __forceinline__ int xslot(int i, int *j) {
        *j = i & 63;
        return i >> 6;
    }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) {
        const uint8_t *blk = row + (size_t)(u >> 2) * 144;
        const int p = u & 3;
        R.q0 = ld16(blk + 16 + 32 * p);
        R.q1 = ld16(blk + 32 + 32 * p);
        R.m = ld16(blk);
    }
    // Integer-free dot: nibbles -> f32 pairs (x 2^-9) -> fma against x.
    static __device__ __forceinline__ float dot(const Raw &R, const UnitX &X, int u) {
        const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
        float alo = 0.0f, ahi = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t lo = qw[t] & 0x0F0F0F0Fu;
            const uint32_t hi = (qw[t] >> 4) & 0x0F0F0F0Fu;
            const float2 l0 = nib2f_lo(lo), l1 = nib2f_hi(lo);
            const float2 h0 = nib2f_lo(hi), h1 = nib2f_hi(hi);
            alo = fmaf(l0.x, X.v[4 * t + 0], alo);
            alo = fmaf(l0.y, X.v[4 * t + 1], alo);
            alo = fmaf(l1.x, X.v[4 * t + 2], alo);
            alo = fmaf(l1.y, X.v[4 * t + 3], alo);
            ahi = fmaf(h0.x, X.v[32 + 4 * t + 0], ahi);
            ahi = fmaf(h0.y, X.v[32 + 4 * t + 1], ahi);
            ahi = fmaf(h1.x, X.v[32 + 4 * t + 2], ahi);
            ahi = fmaf(h1.y, X.v[32 + 4 * t + 3], ahi);
        }
        uint32_t sc2, mn2;
        q4k_scales(R.m.y, R.m.z, R.m.w, u & 3, &sc2, &mn2);
        const float d = h2f(R.m.x), dmin = h2f(R.m.x >> 16);
        const float d9 = d * 512.0f;  // undo the 2^-9 of the fp8 read
        float r = (d9 * ubyte_f<0>(sc2)) * alo;
        r = fmaf(d9 * ubyte_f<1>(sc2), ahi, r);
        r = fmaf(-(dmin * ubyte_f<0>(mn2)), X.s[0] + X.s[1], r);
        r = fmaf(-(dmin * ubyte_f<1>(mn2)), X.s[2] + X.s[3], r);
        return r;
    }
};

// ---------------------------------------------------------------- Q4_0 ---
// Native 18-byte blocks (f16 d, 16 code bytes; byte j holds weight j in its
// low nibble and weight j + 16 in its high nibble), w = d * (q - 8). A unit
// is two blocks (36 bytes, 4-byte aligned in a row of k % 64 == 0); the
// nibbles go through the exact fp8 path of the Q4_K unit (q * 2^-9) and the
// offset is folded as d * (sum q*x - 8 * sum x) with the run sums of x.
#ifndef QMV_RING_Q40
#define QMV_RING_Q40 1
#endif
#ifndef QMV_WG_Q40
#define QMV_WG_Q40 4  // measured at 14336 x 4096: 8.6 us at 4 per CU, 8.9 at 3, 10.7 at 2
#endif
struct Q40Unit : F32Act<Q40Unit> {
    static constexpr int BW = 32, BB = 18;
    static constexpr int RING = QMV_RING_Q40;
    static constexpr int MAX_WG_PER_CU = QMV_WG_Q40;
    struct Raw {
        uint32_t d[9];
    };
    static __device__ __forceinline__ int units_per_row(int k) { return k / 64; }
    static __device__ __forceinline__ void load_x(UnitX &X, const float *x, int u) {
        load_x_runs(X, x, 64 * u, 64 * u + 16, 64 * u + 32, 64 * u + 48);
    }
    static __device__ __forceinline__ int xslot(int i, int *j) {
        *j = i & 63;
        return i >> 6;
    }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) {
        const uint8_t *p = row + 36 * u;
        const v4u_a4 *v = reinterpret_cast<const v4u_a4 *>(p);
        const v4u_a4 a = v[0], b = v[1];
        R.d[0] = a.x; R.d[1] = a.y; R.d[2] = a.z; R.d[3] = a.w;
        R.d[4] = b.x; R.d[5] = b.y; R.d[6] = b.z; R.d[7] = b.w;
        R.d[8] = reinterpret_cast<const uint32_t *>(p)[8];
    }
    static __device__ __forceinline__ float dot(const Raw &R, const UnitX &X, int) {
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t qa = funnel(R.d[t + 1], R.d[t], 2);  // block A codes: bytes 2..17
            const uint32_t qb = R.d[5 + t];                     // block B codes: bytes 20..35
            const uint32_t al = qa & 0x0F0F0F0Fu, ah = (qa >> 4) & 0x0F0F0F0Fu;
            const uint32_t bl = qb & 0x0F0F0F0Fu, bh = (qb >> 4) & 0x0F0F0F0Fu;
            const float2 al0 = nib2f_lo(al), al1 = nib2f_hi(al), ah0 = nib2f_lo(ah), ah1 = nib2f_hi(ah);
            const float2 bl0 = nib2f_lo(bl), bl1 = nib2f_hi(bl), bh0 = nib2f_lo(bh), bh1 = nib2f_hi(bh);
            a = fmaf(al0.x, X.v[4 * t + 0], a);
            a = fmaf(al0.y, X.v[4 * t + 1], a);
            a = fmaf(al1.x, X.v[4 * t + 2], a);
            a = fmaf(al1.y, X.v[4 * t + 3], a);
            a = fmaf(ah0.x, X.v[16 + 4 * t + 0], a);
            a = fmaf(ah0.y, X.v[16 + 4 * t + 1], a);
            a = fmaf(ah1.x, X.v[16 + 4 * t + 2], a);
            a = fmaf(ah1.y, X.v[16 + 4 * t + 3], a);
            b = fmaf(bl0.x, X.v[32 + 4 * t + 0], b);
            b = fmaf(bl0.y, X.v[32 + 4 * t + 1], b);
            b = fmaf(bl1.x, X.v[32 + 4 * t + 2], b);
            b = fmaf(bl1.y, X.v[32 + 4 * t + 3], b);
            b = fmaf(bh0.x, X.v[48 + 4 * t + 0], b);
            b = fmaf(bh0.y, X.v[48 + 4 * t + 1], b);
            b = fmaf(bh1.x, X.v[48 + 4 * t + 2], b);
            b = fmaf(bh1.y, X.v[48 + 4 * t + 3], b);
        }
        const float da = h2f(R.d[0]), db = h2f(R.d[4] >> 16);
        float r = (da * 512.0f) * a;  // undo the 2^-9 of the fp8 read
        r = fmaf(-8.0f * da, X.s[0] + X.s[1], r);
        r = fmaf(db * 512.0f, b, r);
        r = fmaf(-8.0f * db, X.s[2] + X.s[3], r);
        return r;
    }
};

// ---------------------------------------------------------------- Q5_K ---
// 176-byte superblocks: d, dmin, scales[12] (as Q4_K), qh[32], qs[128]. A
// unit is a quarter superblock (sub-blocks 2p, 2p+1): the 5-bit code of
// weight l of sub-block j is its Q4_K nibble plus bit j of qh[l] as bit 4,
// w = d*sc_j*q - dmin*m_j.
#ifndef QMV_RING_Q5K
#define QMV_RING_Q5K 1
#endif
#ifndef QMV_WG_Q5K
#define QMV_WG_Q5K 3
#endif
struct Q5KUnit : F32Act<Q5KUnit> {
    static constexpr int BW = 256, BB = 176;
    static constexpr int RING = QMV_RING_Q5K;
    static constexpr int MAX_WG_PER_CU = QMV_WG_Q5K;
    struct Raw {
        uint4 q0, q1, h0, h1, m;
    };
    static __device__ __forceinline__ int units_per_row(int k) { return (k / 256) * 4; }
    static __device__ __forceinline__ void load_x(UnitX &X, const float *x, int u) {
        const int b = 256 * (u >> 2) + 64 * (u & 3);
        load_x_runs(X, x, b, b + 16, b + 32, b + 48);
    }
    static __device__ __forceinline__ int xslot(int i, int *j) {
        *j = i & 63;
        return i >> 6;
    }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) {
        const uint8_t *blk = row + (size_t)(u >> 2) * 176;
        const int p = u & 3;
        R.q0 = ld16(blk + 48 + 32 * p);
        R.q1 = ld16(blk + 64 + 32 * p);
        R.h0 = ld16(blk + 16);
        R.h1 = ld16(blk + 32);
        R.m = ld16(blk);
    }
    static __device__ __forceinline__ float dot(const Raw &R, const UnitX &X, int u) {
        const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
        const uint32_t hw[8] = {R.h0.x, R.h0.y, R.h0.z, R.h0.w, R.h1.x, R.h1.y, R.h1.z, R.h1.w};
        const int jl = 2 * (u & 3);  // sub-blocks jl (low nibbles) and jl + 1 (high)
        float alo = 0.0f, ahi = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t lo = (qw[t] & 0x0F0F0F0Fu) | (((hw[t] >> jl) & 0x01010101u) << 4);
            const uint32_t hi = ((qw[t] >> 4) & 0x0F0F0F0Fu) | (((hw[t] >> (jl + 1)) & 0x01010101u) << 4);
            alo = fmaf(ubyte_f<0>(lo), X.v[4 * t + 0], alo);
            alo = fmaf(ubyte_f<1>(lo), X.v[4 * t + 1], alo);
            alo = fmaf(ubyte_f<2>(lo), X.v[4 * t + 2], alo);
            alo = fmaf(ubyte_f<3>(lo), X.v[4 * t + 3], alo);
            ahi = fmaf(ubyte_f<0>(hi), X.v[32 + 4 * t + 0], ahi);
            ahi = fmaf(ubyte_f<1>(hi), X.v[32 + 4 * t + 1], ahi);
            ahi = fmaf(ubyte_f<2>(hi), X.v[32 + 4 * t + 2], ahi);
            ahi = fmaf(ubyte_f<3>(hi), X.v[32 + 4 * t + 3], ahi);
        }
        uint32_t sc2, mn2;
        q4k_scales(R.m.y, R.m.z, R.m.w, u & 3, &sc2, &mn2);
        const float d = h2f(R.m.x), dmin = h2f(R.m.x >> 16);
        float r = (d * ubyte_f<0>(sc2)) * alo;
        r = fmaf(d * ubyte_f<1>(sc2), ahi, r);
        r = fmaf(-(dmin * ubyte_f<0>(mn2)), X.s[0] + X.s[1], r);
        r = fmaf(-(dmin * ubyte_f<1>(mn2)), X.s[2] + X.s[3], r);
        return r;
    }
};

// ---------------------------------------------------------------- Q6_K ---
// 16 / 8 bytes at an even address, one global load each (see file comment).
QMV_DEV uint4 ld16u(const uint8_t *p) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    return *q;
}
QMV_DEV uint2 ld8u(const uint8_t *p) {
    const uint2 *q = reinterpret_cast<const uint2 *>(p);
    return *q;
}

struct Q6KUnit : F32Act<Q6KUnit> {
    static constexpr int BW = 256, BB = 210;
    static constexpr int RING = QMV_RING_Q6K;
    static constexpr int MAX_WG_PER_CU = 2;
    struct Raw {
        uint4 a, b, h;
        uint2 sc;
        uint32_t d;
    };
    static __device__ __forceinline__ int units_per_row(int k) { return (k / 256) * 4; }
    static __device__ __forceinline__ void load_x(UnitX &X, const float *x, int u) {
        const int b = 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1);
        load_x_runs(X, x, b, b + 32, b + 64, b + 96);
    }
    // x index i = 256s + 128h + 32g + 16lh + t -> unit 4s + 2h + lh, slot 16g + t
    static __device__ __forceinline__ int xslot(int i, int *j) {
        const int s = i >> 8, h = (i >> 7) & 1, g = (i >> 5) & 3, lh = (i >> 4) & 1, t = i & 15;
        *j = 16 * g + t;
        return 4 * s + 2 * h + lh;
    }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) {
        const uint8_t *blk = row + (size_t)(u >> 2) * 210;
        const int h = (u >> 1) & 1, lh = u & 1;
        R.a = ld16u(blk + 64 * h + 16 * lh);
        R.b = ld16u(blk + 64 * h + 32 + 16 * lh);
        R.h = ld16u(blk + 128 + 32 * h + 16 * lh);
        R.sc = ld8u(blk + 192 + 8 * h);
        R.d = ld2(blk + 208);
    }
    static __device__ __forceinline__ float dot(const Raw &R, const UnitX &X, int u) {
        const uint32_t A[4] = {R.a.x, R.a.y, R.a.z, R.a.w};
        const uint32_t B[4] = {R.b.x, R.b.y, R.b.z, R.b.w};
        const uint32_t H[4] = {R.h.x, R.h.y, R.h.z, R.h.w};
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t q0 = (A[t] & 0x0F0F0F0Fu) | ((H[t] << 4) & 0x30303030u);
            const uint32_t q1 = (B[t] & 0x0F0F0F0Fu) | ((H[t] << 2) & 0x30303030u);
            const uint32_t q2 = ((A[t] >> 4) & 0x0F0F0F0Fu) | (H[t] & 0x30303030u);
            const uint32_t q3 = ((B[t] >> 4) & 0x0F0F0F0Fu) | ((H[t] >> 2) & 0x30303030u);
            const uint32_t qq[4] = {q0, q1, q2, q3};
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                acc[g] = fmaf(ubyte_f<0>(qq[g]), X.v[16 * g + 4 * t + 0], acc[g]);
                acc[g] = fmaf(ubyte_f<1>(qq[g]), X.v[16 * g + 4 * t + 1], acc[g]);
                acc[g] = fmaf(ubyte_f<2>(qq[g]), X.v[16 * g + 4 * t + 2], acc[g]);
                acc[g] = fmaf(ubyte_f<3>(qq[g]), X.v[16 * g + 4 * t + 3], acc[g]);
            }
        }
        // sub-scale of group g: sc[8h + 2g + lh] = byte 2g + lh of the 8 bytes
        const int lh = u & 1;
        const uint32_t s0 = R.sc.x >> (8 * lh), s1 = R.sc.y >> (8 * lh);
        const float c0 = sbyte_f<0>(s0), c1 = sbyte_f<2>(s0), c2 = sbyte_f<0>(s1), c3 = sbyte_f<2>(s1);
        float r = c0 * fmaf(-32.0f, X.s[0], acc[0]);
        r = fmaf(c1, fmaf(-32.0f, X.s[1], acc[1]), r);
        r = fmaf(c2, fmaf(-32.0f, X.s[2], acc[2]), r);
        r = fmaf(c3, fmaf(-32.0f, X.s[3], acc[3]), r);
        return h2f(R.d) * r;
    }
};

// ------------------------------------------------------ Q4_K x q8 (dot4) ---
// Same 64-weight unit as Q4KUnit: unit u = (s, p) covers sub-blocks 2p and
// 2p+1 of superblock s, which are exactly q8 activation blocks 2u and 2u+1.
// Its activation form is the 64 int8 codes xq[64u .. 64u+64) as 16 dwords
// plus xs and xsum of blocks 2u, 2u+1; staged in LDS at 20 dwords per unit
// (8 consecutive units' 16-byte reads land in disjoint banks).
struct ActQ8 {
    const int8_t *xq;
    const float *xs;
    const float *xsum;
};

struct UnitQ8 {
    int32_t q[16];
    float xs[2], xsum[2];
};

// Exact integer sums of one unit: S_lo over sub-block 2p (low nibbles),
// S_hi over sub-block 2p+1 (high nibbles), 4 code x 4 activation bytes per
// v_dot4 (codes 0..15 are non-negative int8).
QMV_DEV void q4k_q8_sums(const Q4KUnit::Raw &R, const int32_t *xq16, int32_t *slo, int32_t *shi) {
    const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
    int32_t a = 0, b = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        a = __builtin_amdgcn_sdot4((int)(qw[t] & 0x0F0F0F0Fu), xq16[t], a, false);
        b = __builtin_amdgcn_sdot4((int)((qw[t] >> 4) & 0x0F0F0F0Fu), xq16[8 + t], b, false);
    }
    *slo = a;
    *shi = b;
}

// q8 activation quantizer, one lane's four values of a 32-value block held
// by eight consecutive lanes (lane groups aligned to 8; every lane of the
// wave must call it). Every f32 step is one IEEE operation with
// round-to-nearest (correctly rounded division, the product x*inv rounded to
// f32 before the half-away rounding), so codes and scales equal any IEEE
// implementation's. Returns the four codes packed in a dword; *scale and
// *xsum are the block's xs and xs * sum(xq).
// Reductions over aligned groups of 8 lanes with DPP (no LDS crossbar):
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], then row_half_mirror, which
// pairs each lane with one of the other quad; every lane gets the result.
// fmaxf ignores NaN in any order, so the maximum does not depend on it.
template <int CTRL>
QMV_DEV float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
QMV_DEV int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
QMV_DEV float group8_max(float a) {
    a = fmaxf(a, dpp_f<0xB1>(a));
    a = fmaxf(a, dpp_f<0x4E>(a));
    return fmaxf(a, dpp_f<0x141>(a));
}
QMV_DEV int group8_sum(int s) {
    s += dpp_i<0xB1>(s);
    s += dpp_i<0x4E>(s);
    return s + dpp_i<0x141>(s);
}

QMV_DEV uint32_t quantize_q8_lanes(float4 v, float *scale, float *xsum) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = group8_max(a);
    float inv = 0.0f, sc = 1.0f;
    if (a > 0.0f) {
        inv = __fdiv_rn(127.0f, a);
        sc = __fdiv_rn(a, 127.0f);
    }
    const float vv[4] = {v.x, v.y, v.z, v.w};
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float prod = __fmul_rn(vv[i], inv);
        asm volatile("" : "+v"(prod));  // materialize the rounded f32 product
        float r = roundf(prod);         // half away from zero
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q[i] = (int)r;
    }
    const int s = group8_sum((q[0] + q[1]) + (q[2] + q[3]));
    *scale = sc;
    *xsum = __fmul_rn(sc, (float)s);
    return (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) | ((uint32_t)(q[2] & 0xFF) << 16) |
           ((uint32_t)(q[3] & 0xFF) << 24);
}

struct Q4KQ8Unit {
    static constexpr bool Q8 = true;  // activation: q8 rows (xq, xs, xsum)
    static constexpr int BW = 256, BB = 144;
    static constexpr int RING = QMV_RING_Q4KQ8;
    // 7.15 us at 14336 x 4096 with 4 workgroups per CU, 7.25 with 3, 7.31 with
    // 5, 8.93 with 2; deeper rings were slower at every count
    static constexpr int MAX_WG_PER_CU = 4;
    static constexpr int ACT_STRIDE = 20;
    using Act = ActQ8;
    using X = UnitQ8;
    using Raw = Q4KUnit::Raw;
    static __device__ __forceinline__ int units_per_row(int k) { return (k / 256) * 4; }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) { Q4KUnit::load(R, row, u); }
    // per thread: up to 4 dwords of xq (k <= 4096 per pass of 256 threads,
    // 2 passes for k <= 8192) and up to 1 block's xs/xsum
    typedef u32x4 Stage[3];  // 2 x 16 bytes of xq, then {xs, xsum, -, -}
    // (branch-free: indices past the end are clamped and re-stored)
    template <int NS>  // (the q8 stage is always 2 granules of xq + scales)
    static __device__ __forceinline__ void fetch(Stage &S, ActQ8 a, int k) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(a.xq);
        const int lastq = k / 16 - 1, lastb = k / 32 - 1;
#pragma unroll
        for (int m = 0; m < 2; ++m) S[m] = q[min((int)threadIdx.x + 256 * m, lastq)];
        const int b = min((int)threadIdx.x, lastb);
        S[2].x = __float_as_uint(a.xs[b]);
        S[2].y = __float_as_uint(a.xsum[b]);
    }
    template <int NS>
    static __device__ __forceinline__ void store(float *xl, const Stage &S, int k) {
        uint32_t *l = reinterpret_cast<uint32_t *>(xl);
        const int lastq = k / 16 - 1, lastb = k / 32 - 1;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = min((int)threadIdx.x + 256 * m, lastq);  // dwords 4i..4i+3 of unit i/4
            *reinterpret_cast<u32x4 *>(l + ACT_STRIDE * (i >> 2) + 4 * (i & 3)) = S[m];
        }
        const int b = min((int)threadIdx.x, lastb);
        xl[ACT_STRIDE * (b >> 1) + 16 + (b & 1)] = __uint_as_float(S[2].x);
        xl[ACT_STRIDE * (b >> 1) + 18 + (b & 1)] = __uint_as_float(S[2].y);
    }
    static __device__ __forceinline__ void load_lds(UnitQ8 &X, const float *xl, int u) {
        const int4 *p = reinterpret_cast<const int4 *>(xl + ACT_STRIDE * u);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int4 v = p[t];
            X.q[4 * t] = v.x; X.q[4 * t + 1] = v.y; X.q[4 * t + 2] = v.z; X.q[4 * t + 3] = v.w;
        }
        const float4 f = reinterpret_cast<const float4 *>(xl + ACT_STRIDE * u)[4];
        X.xs[0] = f.x; X.xs[1] = f.y; X.xsum[0] = f.z; X.xsum[1] = f.w;
    }
    // y contribution: d*sc_j*xs_b*S_b - dmin*m_j*xsum_b for the unit's two blocks
    static __device__ __forceinline__ float dot(const Raw &R, const UnitQ8 &X, int u) {
        int32_t slo, shi;
        q4k_q8_sums(R, X.q, &slo, &shi);
        uint32_t sc2, mn2;
        q4k_scales(R.m.y, R.m.z, R.m.w, u & 3, &sc2, &mn2);
        const float d = h2f(R.m.x), dmin = h2f(R.m.x >> 16);
        float r = (d * ubyte_f<0>(sc2)) * (X.xs[0] * (float)slo);
        r = fmaf(d * ubyte_f<1>(sc2), X.xs[1] * (float)shi, r);
        r = fmaf(-(dmin * ubyte_f<0>(mn2)), X.xsum[0], r);
        r = fmaf(-(dmin * ubyte_f<1>(mn2)), X.xsum[1], r);
        return r;
    }
};

// ------------------------------------------------------ Q6_K x q8 (dot4) ---
// A Q6_K unit (64 weights of one superblock, Q6KUnit) against a q8
// activation. Its values are four runs of 16: run g covers values
// 128h + 32g + 16lh + [0, 16) of the superblock, half of q8 block
// 8s + 4h + g. Each run's integer dot S_g = sum (q - 32) * xq is one v_dot4
// chain (exact): the 6-bit codes q (0..63) are non-negative signed bytes as
// they stand, and the chain starts from -32 * sum(xq) of the run, taken once
// when the activation registers are filled. The unit adds
// d * sc_g * xs_g * S_g for its four runs (sc_g: the run's int8 sub-scale).
struct UnitQ8x4 {
    int32_t q[16];  // dwords 4g..4g+3: xq of run g
    float xs[4];    // xs of run g's q8 block
    int32_t m32[4]; // -32 * (sum of the 16 xq of run g)
};

struct Q6KQ8Unit {
    static constexpr bool Q8 = true;
    static constexpr int BW = 256, BB = 210;
    static constexpr int RING = QMV_RING_Q6K;
    static constexpr int MAX_WG_PER_CU = 2;
    static constexpr int ACT_STRIDE = 20;  // 16 dwords of xq + 4 scales per unit
    using Act = ActQ8;                     // (xsum is not read)
    using X = UnitQ8x4;
    using Raw = Q6KUnit::Raw;
    static __device__ __forceinline__ int units_per_row(int k) { return (k / 256) * 4; }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) { Q6KUnit::load(R, row, u); }
    // 16-value granule i of a row (xq bytes 16i..16i+15) -> its unit and run
    static __device__ __forceinline__ int granule_unit(int i, int *g) {
        *g = (i >> 1) & 3;
        return 4 * (i >> 4) + 2 * ((i >> 3) & 1) + (i & 1);
    }
    // q8 block b -> the first of the two units (lh = 0, 1) that read it, and its run
    static __device__ __forceinline__ int block_unit(int b, int *g) {
        *g = b & 3;
        return 4 * (b >> 3) + 2 * ((b >> 2) & 1);
    }
    typedef u32x4 Stage[3];  // granules tid and tid + 256, then {xs, -, -, -}
    template <int NS>
    static __device__ __forceinline__ void fetch(Stage &S, ActQ8 a, int k) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(a.xq);
        const int lastq = k / 16 - 1, lastb = k / 32 - 1;
#pragma unroll
        for (int m = 0; m < 2; ++m) S[m] = q[min((int)threadIdx.x + 256 * m, lastq)];
        S[2].x = __float_as_uint(a.xs[min((int)threadIdx.x, lastb)]);
    }
    template <int NS>
    static __device__ __forceinline__ void store(float *xl, const Stage &S, int k) {
        uint32_t *l = reinterpret_cast<uint32_t *>(xl);
        const int lastq = k / 16 - 1, lastb = k / 32 - 1;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = min((int)threadIdx.x + 256 * m, lastq);
            int g;
            const int u = granule_unit(i, &g);
            *reinterpret_cast<u32x4 *>(l + ACT_STRIDE * u + 4 * g) = S[m];
        }
        int g;
        const int u = block_unit(min((int)threadIdx.x, lastb), &g);
        xl[ACT_STRIDE * u + 16 + g] = __uint_as_float(S[2].x);
        xl[ACT_STRIDE * (u + 1) + 16 + g] = __uint_as_float(S[2].x);
    }
    static __device__ __forceinline__ void load_lds(UnitQ8x4 &X, const float *xl, int u) {
        const int4 *p = reinterpret_cast<const int4 *>(xl + ACT_STRIDE * u);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int4 v = p[t];
            X.q[4 * t] = v.x; X.q[4 * t + 1] = v.y; X.q[4 * t + 2] = v.z; X.q[4 * t + 3] = v.w;
        }
        const float4 f = reinterpret_cast<const float4 *>(xl + ACT_STRIDE * u)[4];
        X.xs[0] = f.x; X.xs[1] = f.y; X.xs[2] = f.z; X.xs[3] = f.w;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int sum = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) sum = __builtin_amdgcn_sdot4(X.q[4 * g + t], 0x01010101, sum, false);
            X.m32[g] = -32 * sum;
        }
    }
    static __device__ __forceinline__ float dot(const Raw &R, const UnitQ8x4 &X, int u) {
        const uint32_t A[4] = {R.a.x, R.a.y, R.a.z, R.a.w};
        const uint32_t B[4] = {R.b.x, R.b.y, R.b.z, R.b.w};
        const uint32_t H[4] = {R.h.x, R.h.y, R.h.z, R.h.w};
        int S[4] = {X.m32[0], X.m32[1], X.m32[2], X.m32[3]};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t q0 = (A[t] & 0x0F0F0F0Fu) | ((H[t] << 4) & 0x30303030u);
            const uint32_t q1 = (B[t] & 0x0F0F0F0Fu) | ((H[t] << 2) & 0x30303030u);
            const uint32_t q2 = ((A[t] >> 4) & 0x0F0F0F0Fu) | (H[t] & 0x30303030u);
            const uint32_t q3 = ((B[t] >> 4) & 0x0F0F0F0Fu) | ((H[t] >> 2) & 0x30303030u);
            S[0] = __builtin_amdgcn_sdot4((int)q0, X.q[t], S[0], false);
            S[1] = __builtin_amdgcn_sdot4((int)q1, X.q[4 + t], S[1], false);
            S[2] = __builtin_amdgcn_sdot4((int)q2, X.q[8 + t], S[2], false);
            S[3] = __builtin_amdgcn_sdot4((int)q3, X.q[12 + t], S[3], false);
        }
        // sub-scale of run g: byte 2g + lh of the 8 scale bytes of half h
        const int lh = u & 1;
        const uint32_t s0 = R.sc.x >> (8 * lh), s1 = R.sc.y >> (8 * lh);
        const float c0 = sbyte_f<0>(s0), c1 = sbyte_f<2>(s0), c2 = sbyte_f<0>(s1), c3 = sbyte_f<2>(s1);
        float r = c0 * (X.xs[0] * (float)S[0]);
        r = fmaf(c1, X.xs[1] * (float)S[1], r);
        r = fmaf(c2, X.xs[2] * (float)S[2], r);
        r = fmaf(c3, X.xs[3] * (float)S[3], r);
        return h2f(R.d) * r;
    }
};

// The Q6_K int8-dot unit on an f32 activation that is quantized while it is
// staged (the steps of quantize_act_q8 per 32 values, so the codes and scales
// are the same bits): the MoE down pass stages its h rows this way instead of
// reading a separately quantized copy (see k_moe_down).
struct Q6KQ8XUnit {
    static constexpr bool Q8 = false;  // takes f32 rows
    static constexpr bool QX = true;   // quantized in the staging
    static constexpr int BW = 256, BB = 210;
    static constexpr int RING = QMV_RING_Q6K;
    static constexpr int MAX_WG_PER_CU = 2;
    static constexpr int ACT_STRIDE = Q6KQ8Unit::ACT_STRIDE;
    using Act = ActF32;
    using X = UnitQ8x4;
    using Raw = Q6KUnit::Raw;
    static __device__ __forceinline__ int units_per_row(int k) { return (k / 256) * 4; }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) { Q6KUnit::load(R, row, u); }
    static __device__ __forceinline__ int granule_unit(int i, int *g) { return Q6KQ8Unit::granule_unit(i, g); }
    static __device__ __forceinline__ int block_unit(int b, int *g) { return Q6KQ8Unit::block_unit(b, g); }
    // f32 values 4c4..4c4+3 of a row, quantized with the 8 lanes that hold
    // the rest of their 32-value block (call with all 8 lanes active), into
    // the Q6KQ8Unit layout of the row staged at xl
    static __device__ __forceinline__ void store_quantized(float *xl, f32x4 v, int c4, bool valid) {
        float sc, xsum;
        const uint32_t packed = quantize_q8_lanes(make_float4(v.x, v.y, v.z, v.w), &sc, &xsum);
        if (valid) {
            int g;
            const int u = granule_unit(c4 >> 2, &g);
            reinterpret_cast<uint32_t *>(xl)[ACT_STRIDE * u + 4 * g + (c4 & 3)] = packed;
            if ((c4 & 7) == 0) {
                int gb;
                const int ub = block_unit(c4 >> 3, &gb);
                xl[ACT_STRIDE * ub + 16 + gb] = sc;
                xl[ACT_STRIDE * (ub + 1) + 16 + gb] = sc;
            }
        }
    }
    static __device__ __forceinline__ void load_lds(UnitQ8x4 &X, const float *xl, int u) { Q6KQ8Unit::load_lds(X, xl, u); }
    static __device__ __forceinline__ float dot(const Raw &R, const UnitQ8x4 &X, int u) { return Q6KQ8Unit::dot(R, X, u); }
};

// ---------------------------------------- Q4_K x q8, quantizing in-kernel ---
// The Q4KQ8Unit decode with the activation given in f32: every workgroup
// quantizes x itself while staging it (the same IEEE steps as
// quantize_act_q8, so the codes and scales are the same bits) straight into
// the q8 unit layout in LDS. One launch instead of quantizer + matvec.
struct Q4KQ8XUnit {
    static constexpr bool Q8 = false;  // takes f32 rows
    static constexpr int BW = 256, BB = 144;
    static constexpr int RING = QMV_RING_Q4KQ8;
    static constexpr int MAX_WG_PER_CU = 3;
    static constexpr int ACT_STRIDE = Q4KQ8Unit::ACT_STRIDE;
    using Act = ActF32;
    using X = UnitQ8;
    using Raw = Q4KUnit::Raw;
    using Stage = StageRegs;
    static __device__ __forceinline__ int units_per_row(int k) { return (k / 256) * 4; }
    static __device__ __forceinline__ void load(Raw &R, const uint8_t *row, int u) { Q4KUnit::load(R, row, u); }
    template <int NS>
    static __device__ __forceinline__ void fetch(Stage &S, ActF32 a, int k) { fetch_x<NS>(S, a.x, k); }
    // float4 i of x (values 4i..4i+3) -> codes at dword i % 16 of unit i / 16;
    // the block b = i / 8 scale and dequantized sum at slots 16 + b % 2 and
    // 18 + b % 2 of unit b / 2 (the Q4KQ8Unit layout)
    template <int NS>
    static __device__ __forceinline__ void store(float *xl, const Stage &S, int k) {
        uint32_t *l = reinterpret_cast<uint32_t *>(xl);
        const int n4 = k / 4;
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int i = (int)threadIdx.x + 256 * m;  // lanes past n4 form whole groups of 8
            float sc, xsum;
            const f32x4 v = S[m];
            const uint32_t packed = quantize_q8_lanes(make_float4(v.x, v.y, v.z, v.w), &sc, &xsum);
            if (i < n4) {
                l[ACT_STRIDE * (i >> 4) + (i & 15)] = packed;
                if ((i & 7) == 0) {
                    const int b = i >> 3;
                    xl[ACT_STRIDE * (b >> 1) + 16 + (b & 1)] = sc;
                    xl[ACT_STRIDE * (b >> 1) + 18 + (b & 1)] = xsum;
                }
            }
        }
    }
    static __device__ __forceinline__ void load_lds(UnitQ8 &X, const float *xl, int u) { Q4KQ8Unit::load_lds(X, xl, u); }
    static __device__ __forceinline__ float dot(const Raw &R, const UnitQ8 &X, int u) { return Q4KQ8Unit::dot(R, X, u); }
};

// ------------------------------- Q4_K matvec with the q8 activation beside ---
// The f32 Q4_K matvec (Q4KUnit, same arithmetic and output bits) whose first
// workgroup also writes quantize_act_q8(x) (one row: codes xq, scale xs and
// dequantized sum xsum per 32-value block, the same IEEE steps and bits) from
// the activation registers it stages anyway, so that an int8-dot matvec of
// the same x needs no quantizer launch of its own.
struct ActF32Q {
    const float *x;
    int8_t *xq;
    float *xs, *xsum;
};
struct Q4KQOutUnit : Q4KUnit {
    using Act = ActF32Q;
    template <int NS>
    static __device__ __forceinline__ void fetch(Stage &S, ActF32Q a, int k) { fetch_x<NS>(S, a.x, k); }
    // every lane quantizes its staged float4s (8 lanes per 32-value block,
    // lanes past the end in whole groups of 8 with clamped values) and
    // writes what lies inside x
    template <int NS>
    static __device__ __forceinline__ void side(const Stage &S, ActF32Q a, int k) {
        const int n4 = k / 4;
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int i = (int)threadIdx.x + 256 * m;
            float sc, xsum;
            const f32x4 v = S[m];
            const uint32_t packed = quantize_q8_lanes(make_float4(v.x, v.y, v.z, v.w), &sc, &xsum);
            if (i < n4) {
                reinterpret_cast<uint32_t *>(a.xq)[i] = packed;
                if ((i & 7) == 0) {
                    a.xs[i >> 3] = sc;
                    a.xsum[i >> 3] = xsum;
                }
            }
        }
    }
};
