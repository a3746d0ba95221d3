// q8 activation path on gfx950: the activation quantizer and the Q4_K matvec
// that dots raw 4-bit codes against int8 activation codes with v_dot4.
//
// hanzo-ml `src/vulkan_backend.rs`: `quantize_act_q8` returns (xq int8,
// xs f32 scale, xsum f32 "dequant block sum") per 32 activation values;
// `matvec_q4k_gpu_off` quantizes x once and runs the int8-dot Q4_K decode;
// the MMQ comments give the affine epilogue xs*(D*dot - M*xsum) ("dmin fold").
#include "dense.hpp"

namespace {

// ------------------------------------------------------------ quantizer ---
// Eight lanes per 32-value block, four values each (quantize_q8_lanes in
// blocks.hpp: every f32 step one IEEE operation; in particular the product
// x*inv is rounded to f32 before it is rounded to an integer -- were it fused
// into the fraction test of the half-away rounding, a product that rounds to
// k+0.5 but lies just below it would go the other way).
__global__ __launch_bounds__(256) void k_quantize_act_q8(const float *__restrict__ x,
                                                         int8_t *__restrict__ xq,
                                                         float *__restrict__ xs,
                                                         float *__restrict__ xsum, int64_t nblocks) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b = tid >> 3;
    const int sub = (int)(tid & 7);
    const bool valid = b < nblocks;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *reinterpret_cast<const float4 *>(x + b * 32 + sub * 4);
    float scale, sum;
    const uint32_t packed = quantize_q8_lanes(v, &scale, &sum);
    if (valid) {
        *reinterpret_cast<uint32_t *>(xq + b * 32 + sub * 4) = packed;
        if (sub == 0) {
            xs[b] = scale;
            xsum[b] = sum;
        }
    }
}

// ------------------------------------------------- Q4_K x q8 dot4 matvec ---
// The matvec runs on the row-streaming skeleton (dense.hpp) with the
// Q4KQ8Unit policy (blocks.hpp). The debug export below recomputes the same
// per-unit integer sums (q4k_q8_sums) and writes them out instead of
// scaling them.
constexpr int WAVES_PER_BLOCK = 4;

// One wave per row, lanes over units: sums[r, 2u] = S_lo, sums[r, 2u+1] = S_hi.
__global__ __launch_bounds__(256) void k_blocksums_q4k_q8(const uint8_t *__restrict__ w,
                                                          const int8_t *__restrict__ xq,
                                                          int32_t *__restrict__ sums, int n,
                                                          int U, int row_bytes) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
    if (r >= n) return;
    for (int u = lane; u < U; u += 64) {
        Q4KUnit::Raw R;
        Q4KUnit::load(R, w + (size_t)r * row_bytes, u);
        int32_t q[16];
        const int4 *p = reinterpret_cast<const int4 *>(xq + 64 * u);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int4 v = p[t];
            q[4 * t] = v.x; q[4 * t + 1] = v.y; q[4 * t + 2] = v.z; q[4 * t + 3] = v.w;
        }
        int32_t slo, shi;
        q4k_q8_sums(R, q, &slo, &shi);
        sums[(size_t)r * (2 * U) + 2 * u] = slo;
        sums[(size_t)r * (2 * U) + 2 * u + 1] = shi;
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
    if (n > (1 << 30) || k > 8192) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(y, 4))
        return QMV_EALIGN;
    qmv_dense::launch_tiled<Q4KQ8Unit>(static_cast<const uint8_t *>(w), ActQ8{xq, xs, xsum}, y, n, k,
                                       (hipStream_t)stream);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

extern "C" int qmv_debug_blocksums_q4k_q8(const void *w, const int8_t *xq, int32_t *sums, int64_t n,
                                          int64_t k, qmv_stream_t stream) {
    if (!w || !xq || !sums || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (n > (1 << 30) || k > (1 << 24)) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(sums, 4)) return QMV_EALIGN;
    const int U = (int)(k / 256) * 4;
    hipLaunchKernelGGL(k_blocksums_q4k_q8, dim3((unsigned)div_up(n, WAVES_PER_BLOCK)), dim3(256), 0,
                       (hipStream_t)stream, static_cast<const uint8_t *>(w), xq, sums, (int)n, U,
                       (int)((k / 256) * 144));
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

extern "C" int qmv_q4k_q8x(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream) {
    if (!w || !x || !y || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (n > (1 << 30) || k > 8192) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QMV_EALIGN;
    qmv_dense::launch_tiled<Q4KQ8XUnit>(static_cast<const uint8_t *>(w), ActF32{x}, y, n, k, (hipStream_t)stream);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}
