// q8 activation path on gfx950: the activation quantizer and the Q4_K matvec
// that dots raw 4-bit codes against int8 activation codes with v_dot4.
//
// hanzo-ml `src/vulkan_backend.rs`: `quantize_act_q8` returns (xq int8,
// xs f32 scale, xsum f32 "dequant block sum") per 32 activation values;
// `matvec_q4k_gpu_off` quantizes x once and runs the int8-dot Q4_K decode;
// the MMQ comments give the affine epilogue xs*(D*dot - M*xsum) ("dmin fold").
#include "blocks.hpp"

namespace {

// ------------------------------------------------------------ quantizer ---
// Eight lanes per 32-value block, four values each. Every f32 step is one
// IEEE operation with round-to-nearest (no contraction, correctly rounded
// division), so the codes and scales equal any IEEE implementation's. In
// particular the product x*inv is rounded to f32 before it is rounded to an
// integer: were it fused into the fraction test of the half-away rounding, a
// product that rounds to k+0.5 but lies just below it would go the other way.
__global__ __launch_bounds__(256) void k_quantize_act_q8(const float *__restrict__ x,
                                                         int8_t *__restrict__ xq,
                                                         float *__restrict__ xs,
                                                         float *__restrict__ xsum, int64_t nblocks) {
#pragma clang fp contract(off)
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b = tid >> 3;
    const int sub = (int)(tid & 7);
    const bool valid = b < nblocks;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *reinterpret_cast<const float4 *>(x + b * 32 + sub * 4);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    float inv = 0.0f, scale = 1.0f;
    if (a > 0.0f) {
        inv = __fdiv_rn(127.0f, a);
        scale = __fdiv_rn(a, 127.0f);
    }
    const float vv[4] = {v.x, v.y, v.z, v.w};
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float prod = vv[i] * inv;
        asm volatile("" : "+v"(prod));  // materialize the rounded f32 product
        float r = roundf(prod);         // half away from zero
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q[i] = (int)r;
    }
    int s = (q[0] + q[1]) + (q[2] + q[3]);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (valid) {
        const uint32_t packed = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) |
                                ((uint32_t)(q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
        *reinterpret_cast<uint32_t *>(xq + b * 32 + sub * 4) = packed;
        if (sub == 0) {
            xs[b] = scale;
            xsum[b] = __fmul_rn(scale, (float)s);
        }
    }
}

// ------------------------------------------------- Q4_K x q8 dot4 matvec ---
// Unit = one 16-byte code chunk c of a superblock (as in the f32 path): 16
// weights of sub-block 2p (low nibbles) and 16 of 2p+1 (high nibbles),
// p = c/2, positions 16*(c%2)..+15 within each sub-block. Sub-block j of
// superblock s is q8 block 8s + j, so each lane holds 4+4 dwords of xq and
// the scales of the two q8 blocks. The two lanes c and c^1 split a q8 block;
// the min term of the block is added by the lane with c even.
struct Q8X {
    int32_t lo[4], hi[4];
    float xs_lo, xs_hi;
    float xsum_lo, xsum_hi;  // zero on the c-odd lane: the block's min term is added once
};

QMV_DEV void q8x_load(Q8X &X, const int8_t *xq, const float *xs, const float *xsum, int s, int c) {
    const int p = c >> 1, hh = c & 1;
    const int4 a = *reinterpret_cast<const int4 *>(xq + 256 * s + 64 * p + 16 * hh);
    const int4 b = *reinterpret_cast<const int4 *>(xq + 256 * s + 64 * p + 32 + 16 * hh);
    X.lo[0] = a.x; X.lo[1] = a.y; X.lo[2] = a.z; X.lo[3] = a.w;
    X.hi[0] = b.x; X.hi[1] = b.y; X.hi[2] = b.z; X.hi[3] = b.w;
    X.xs_lo = xs[8 * s + 2 * p];
    X.xs_hi = xs[8 * s + 2 * p + 1];
    X.xsum_lo = hh == 0 ? xsum[8 * s + 2 * p] : 0.0f;
    X.xsum_hi = hh == 0 ? xsum[8 * s + 2 * p + 1] : 0.0f;
}

// Integer partial sums of the unit: 16 codes x 16 xq per sub-block.
QMV_DEV void q4k_q8_sums(uint4 q, const Q8X &X, int32_t *slo, int32_t *shi) {
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    int32_t a = 0, b = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        a = __builtin_amdgcn_sdot4((int)(qw[t] & 0x0F0F0F0Fu), X.lo[t], a, false);
        b = __builtin_amdgcn_sdot4((int)((qw[t] >> 4) & 0x0F0F0F0Fu), X.hi[t], b, false);
    }
    *slo = a;
    *shi = b;
}

QMV_DEV float q4k_q8_unit_dot(uint4 q, uint4 m, const Q8X &X, int p) {
    int32_t slo, shi;
    q4k_q8_sums(q, X, &slo, &shi);
    uint32_t sc2, mn2;
    q4k_scales(m.y, m.z, m.w, p, &sc2, &mn2);
    const float d = h2f(m.x), dmin = h2f(m.x >> 16);
    float r = (d * ubyte_f<0>(sc2)) * (X.xs_lo * (float)slo);
    r = fmaf(d * ubyte_f<1>(sc2), X.xs_hi * (float)shi, r);
    r = fmaf(-(dmin * ubyte_f<0>(mn2)), X.xsum_lo, r);
    r = fmaf(-(dmin * ubyte_f<1>(mn2)), X.xsum_hi, r);
    return r;
}

constexpr int WAVES_PER_BLOCK = 4;

template <int G, int UPL, int RB>
__global__ __launch_bounds__(256) void k_qmv_q4k_q8(const uint8_t *__restrict__ w,
                                                    const int8_t *__restrict__ xq,
                                                    const float *__restrict__ xs,
                                                    const float *__restrict__ xsum,
                                                    float *__restrict__ y, int n, int passes,
                                                    int per_wave, int U, int row_bytes) {
    constexpr int RPP = 64 / G;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int grow = lane / G;
    const int wave = blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
    const int p0 = wave * per_wave;
    if (p0 >= passes) return;
    const int p1 = min(passes, p0 + per_wave);
    const int c = gl & 7, pr = c >> 1;
    Q8X X[UPL];
    bool uv[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = gl + G * i;
        uv[i] = u < U;
        if (uv[i]) q8x_load(X[i], xq, xs, xsum, u >> 3, c);
    }
    for (int pass = p0; pass < p1; pass += RB) {
        uint4 qd[RB][UPL], md[RB][UPL];
        bool rv[RB];
        int rr[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            rr[b] = (pass + b) * RPP + grow;
            rv[b] = (pass + b) < p1 && rr[b] < n;
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv[b] && uv[i]) {
                    const uint8_t *blk = w + (size_t)rr[b] * row_bytes + (size_t)((gl + G * i) >> 3) * 144;
                    qd[b][i] = ld16(blk + 16 + 16 * c);
                    md[b][i] = ld16(blk);
                }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv[b] && uv[i]) acc += q4k_q8_unit_dot(qd[b][i], md[b][i], X[i], pr);
            acc = group_sum<G>(acc);
            if (gl == 0 && rv[b]) y[rr[b]] = acc;
        }
    }
}

// One wave per row; lanes over units. Writes the exact int32 block sums
// with the same dot4 sequence as the matvec (the two half-block partial sums
// of lanes c and c^1 added together).
__global__ __launch_bounds__(256) void k_blocksums_q4k_q8(const uint8_t *__restrict__ w,
                                                          const int8_t *__restrict__ xq,
                                                          int32_t *__restrict__ sums, int n,
                                                          int U, int row_bytes) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
    if (r >= n) return;
    const int c = lane & 7, p = c >> 1, hh = c & 1;
    const int nb32 = U;  // 8 units per superblock == 8 q8 blocks per superblock
    // U is a multiple of 8, so a lane and its partner lane^1 are valid together.
    for (int u0 = 0; u0 < U; u0 += 64) {
        const int u = u0 + lane;
        const bool valid = u < U;
        int32_t slo = 0, shi = 0;
        if (valid) {
            const int s = u >> 3;
            Q8X X;
            const int4 a = *reinterpret_cast<const int4 *>(xq + 256 * s + 64 * p + 16 * hh);
            const int4 b = *reinterpret_cast<const int4 *>(xq + 256 * s + 64 * p + 32 + 16 * hh);
            X.lo[0] = a.x; X.lo[1] = a.y; X.lo[2] = a.z; X.lo[3] = a.w;
            X.hi[0] = b.x; X.hi[1] = b.y; X.hi[2] = b.z; X.hi[3] = b.w;
            const uint4 q = ld16(w + (size_t)r * row_bytes + (size_t)s * 144 + 16 + 16 * c);
            q4k_q8_sums(q, X, &slo, &shi);
        }
        slo += __shfl_xor(slo, 1);
        shi += __shfl_xor(shi, 1);
        if (valid && hh == 0) {
            const int s = u >> 3;
            sums[(size_t)r * nb32 + 8 * s + 2 * p] = slo;
            sums[(size_t)r * nb32 + 8 * s + 2 * p + 1] = shi;
        }
    }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" int quantize_act_q8(const float *x, int8_t *xq, float *xs, float *xsum, int64_t m,
                               int64_t k, qmv_stream_t stream) {
    if (!x || !xq || !xs || !xsum || m < 1 || k < 32 || k % 32) return QMV_EINVAL;
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(xs, 4) || !aligned(xsum, 4)) return QMV_EALIGN;
    const int64_t nb = m * (k / 32);
    const int64_t threads = nb * 8;
    if (div_up(threads, 256) > 0x7FFFFFFF) return QMV_EUNSUPPORTED;
    hipLaunchKernelGGL(k_quantize_act_q8, dim3((unsigned)div_up(threads, 256)), dim3(256), 0,
                       (hipStream_t)stream, x, xq, xs, xsum, nb);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

extern "C" int qmv_q4k_q8(const void *w, const int8_t *xq, const float *xs, const float *xsum,
                          float *y, int64_t n, int64_t k, qmv_stream_t stream) {
    if (!w || !xq || !xs || !xsum || !y || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (n > (1 << 30) || k > 8 * 256 * 64) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(y, 4))
        return QMV_EALIGN;
    const int U = (int)(k / 256) * 8;
    const int row_bytes = (int)(k / 256) * 144;
    const int G = next_pow2_le64(U);
    const int upl = (U + G - 1) / G;
    const int rpp = 64 / G;
    const int passes = (int)div_up(n, rpp);
    const int per_wave = (int)div_up(passes, 4096);
    const int waves = (int)div_up(passes, per_wave);
    const dim3 grid((unsigned)div_up(waves, WAVES_PER_BLOCK));
    hipStream_t s = (hipStream_t)stream;
#define Q8L(GG, UU) hipLaunchKernelGGL((k_qmv_q4k_q8<GG, UU, 2>), grid, dim3(256), 0, s, \
        static_cast<const uint8_t *>(w), xq, xs, xsum, y, (int)n, passes, per_wave, U, row_bytes)
    switch (G) {
        case 8: Q8L(8, 1); break;
        case 16: Q8L(16, 1); break;
        case 32: Q8L(32, 1); break;
        default:
            if (upl == 1) Q8L(64, 1);
            else if (upl == 2) Q8L(64, 2);
            else if (upl <= 4) Q8L(64, 4);
            else if (upl <= 8) Q8L(64, 8);
            else return QMV_EUNSUPPORTED;
    }
#undef Q8L
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

extern "C" int qmv_debug_blocksums_q4k_q8(const void *w, const int8_t *xq, int32_t *sums, int64_t n,
                                          int64_t k, qmv_stream_t stream) {
    if (!w || !xq || !sums || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (n > (1 << 30) || k > (1 << 24)) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(sums, 4)) return QMV_EALIGN;
    const int U = (int)(k / 256) * 8;
    hipLaunchKernelGGL(k_blocksums_q4k_q8, dim3((unsigned)div_up(n, WAVES_PER_BLOCK)), dim3(256), 0,
                       (hipStream_t)stream, static_cast<const uint8_t *>(w), xq, sums, (int)n, U,
                       (int)((k / 256) * 144));
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}
