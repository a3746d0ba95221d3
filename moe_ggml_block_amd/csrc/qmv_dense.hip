// Dense decode matvecs y = W_deq x over raw Q8_0 / Q4_K / Q6_K / Q4_0 / Q5_K
// rows (gfx950).
//
// Defined by hanzo-ml `src/vulkan_backend.rs`: `matvec_q8_0_gpu`,
// `matvec_q4k_gpu_off` and `matvec_q6k_gpu_off` (y[nout] = Wq * x[k], blocks
// read verbatim from a resident buffer, no requantization). The streaming
// skeleton and its launch shape are in dense.hpp; f32 activations use the
// UnitX register form staged through LDS (blocks.hpp).
#include <type_traits>

#include "dense.hpp"

namespace {

using qmv_dense::WAVES_PER_BLOCK;

// ------------------------------------------------------- generic fallback
// One wave per row, lanes over blocks, byte loads: any k that is a block
// multiple and any alignment of rows (used when the unit tiling above does
// not apply: Q8_0 with k % 64 == 32, or rows longer than 2*64 units).
__device__ float block_dot_generic(int fmt, const uint8_t *b, const float *x) {
    float acc = 0.0f;
    if (fmt == 0) {
        float d = h2f(b[0] | (b[1] << 8));
        for (int i = 0; i < 32; ++i) acc = fmaf((float)(int8_t)b[2 + i], x[i], acc);
        return d * acc;
    }
    if (fmt == 1) {
        float d = h2f(b[0] | (b[1] << 8)), dmin = h2f(b[2] | (b[3] << 8));
        const uint8_t *s = b + 4, *qs = b + 16;
        for (int j = 0; j < 8; ++j) {
            int sc, m;
            if (j < 4) {
                sc = s[j] & 63;
                m = s[j + 4] & 63;
            } else {
                sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
                m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
            }
            float a = 0.0f, xs = 0.0f;
            for (int l = 0; l < 32; ++l) {
                uint8_t v = qs[32 * (j >> 1) + l];
                int q = (j & 1) ? (v >> 4) : (v & 15);
                a = fmaf((float)q, x[32 * j + l], a);
                xs += x[32 * j + l];
            }
            acc += d * (float)sc * a - dmin * (float)m * xs;
        }
        return acc;
    }
    if (fmt == 3) {
        float d = h2f(b[0] | (b[1] << 8));
        for (int j = 0; j < 16; ++j) {
            acc = fmaf((float)((b[2 + j] & 15) - 8), x[j], acc);
            acc = fmaf((float)((b[2 + j] >> 4) - 8), x[j + 16], acc);
        }
        return d * acc;
    }
    if (fmt == 4) {
        float d = h2f(b[0] | (b[1] << 8)), dmin = h2f(b[2] | (b[3] << 8));
        const uint8_t *s = b + 4, *qh = b + 16, *qs = b + 48;
        for (int j = 0; j < 8; ++j) {
            int sc, m;
            if (j < 4) {
                sc = s[j] & 63;
                m = s[j + 4] & 63;
            } else {
                sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
                m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
            }
            float a = 0.0f, xs = 0.0f;
            for (int l = 0; l < 32; ++l) {
                uint8_t v = qs[32 * (j >> 1) + l];
                int q = ((j & 1) ? (v >> 4) : (v & 15)) | (((qh[l] >> j) & 1) << 4);
                a = fmaf((float)q, x[32 * j + l], a);
                xs += x[32 * j + l];
            }
            acc += d * (float)sc * a - dmin * (float)m * xs;
        }
        return acc;
    }
    const uint8_t *ql = b, *qh = b + 128;
    const int8_t *sc = reinterpret_cast<const int8_t *>(b + 192);
    float d = h2f(b[208] | (b[209] << 8));
    for (int t = 0; t < 16; ++t) {
        float a = 0.0f;
        for (int l16 = 0; l16 < 16; ++l16) {
            int i = 16 * t + l16;
            int h = i >> 7, p = i & 127, g = p >> 5, l = p & 31;
            uint8_t lb = ql[64 * h + l + 32 * (g & 1)];
            int lo = g < 2 ? (lb & 15) : (lb >> 4);
            int hi = (qh[32 * h + l] >> (2 * g)) & 3;
            a = fmaf((float)((lo | (hi << 4)) - 32), x[i], a);
        }
        acc += (float)sc[t] * a;
    }
    return d * acc;
}

__global__ __launch_bounds__(256) void k_qmv_generic(int fmt, const uint8_t *__restrict__ w,
                                                     const float *__restrict__ x,
                                                     float *__restrict__ y, int64_t n, int64_t k,
                                                     int64_t row_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
    if (r >= n) return;
    const int bw = (fmt == 0 || fmt == 3) ? 32 : 256;
    const int bb = fmt == 0 ? 34 : fmt == 1 ? 144 : fmt == 2 ? 210 : fmt == 3 ? 18 : 176;
    const int64_t nb = k / bw;
    float acc = 0.0f;
    for (int64_t b = lane; b < nb; b += 64) acc += block_dot_generic(fmt, w + r * row_bytes + b * bb, x + b * bw);
    acc = group_sum<64>(acc);
    if (lane == 0) y[r] = acc;
}

// Q8_0 at up to 16 rows per CU: one workgroup per CU with two passes in
// flight per wave keeps the rows in flight of two workgroups with one pass
// each, with half the waves filling their activation registers (measured at
// 4096 x 4096: 5.35 against 5.55 us; at 14336 x 4096 the two-workgroup form
// is faster, 12.49 against 12.82 us).
struct Q8UnitFew : Q8Unit {
    static constexpr int RING = 2;
    static constexpr int MAX_WG_PER_CU = 1;
};

// ------------------------------------------------------------- dispatch
template <class F>
int launch_dense(const uint8_t *w, const float *x, float *y, int64_t n, int64_t k, hipStream_t s) {
    const int64_t row_bytes = k / F::BW * F::BB;
    const bool tiled = (k % 64 == 0) && k <= 8192;  // units of 64 weights, x fits LDS
    const int fmt = F::BB == 34 ? 0 : F::BB == 144 ? 1 : F::BB == 210 ? 2 : F::BB == 18 ? 3 : 4;
    if (!tiled) {
        const dim3 grid((unsigned)((n + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK));
        hipLaunchKernelGGL(k_qmv_generic, grid, dim3(256), 0, s, fmt, w, x, y, n, k, row_bytes);
        QMV_LAUNCH_CHECK();
        return QMV_OK;
    }
    if constexpr (std::is_same<F, Q8Unit>::value) {
        if (n <= 16 * (int64_t)qmv_dense::compute_units()) {
            qmv_dense::launch_tiled<Q8UnitFew>(w, ActF32{x}, y, n, k, s);
            QMV_LAUNCH_CHECK();
            return QMV_OK;
        }
    }
    qmv_dense::launch_tiled<F>(w, ActF32{x}, y, n, k, s);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

template <class F>
int dense_entry(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream) {
    if (!w || !x || !y || n < 1 || k < F::BW || k % F::BW) return QMV_EINVAL;
    if (n > (int64_t)1 << 30 || k > (int64_t)1 << 24) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QMV_EALIGN;
    return launch_dense<F>(static_cast<const uint8_t *>(w), x, y, n, k, (hipStream_t)stream);
}

}  // namespace

extern "C" int qmv_q8_0(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<Q8Unit>(w, x, y, n, k, s);
}
extern "C" int qmv_q4k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<Q4KUnit>(w, x, y, n, k, s);
}
extern "C" int qmv_q6k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<Q6KUnit>(w, x, y, n, k, s);
}
extern "C" int qmv_q4_0(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<Q40Unit>(w, x, y, n, k, s);
}
extern "C" int qmv_q5k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<Q5KUnit>(w, x, y, n, k, s);
}

// Q4_K matvec of an f32 activation that also writes that activation's q8
// form (one row of quantize_act_q8) from the first workgroup's staged
// registers; past the tiled range the two run as separate launches.
extern "C" int qmv_q4k_qx(const void *w, const float *x, float *y, int8_t *xq, float *xs, float *xsum,
                          int64_t n, int64_t k, qmv_stream_t stream) {
    if (!w || !x || !y || !xq || !xs || !xsum || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (n > (int64_t)1 << 30 || k > (int64_t)1 << 24) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(xq, 4) || !aligned(xs, 4) ||
        !aligned(xsum, 4))
        return QMV_EALIGN;
    const hipStream_t s = (hipStream_t)stream;
    if (k > 8192) {
        const int rc = launch_dense<Q4KUnit>(static_cast<const uint8_t *>(w), x, y, n, k, s);
        return rc != QMV_OK ? rc : quantize_act_q8(x, xq, xs, xsum, 1, k, stream);
    }
    qmv_dense::launch_tiled<Q4KQOutUnit>(static_cast<const uint8_t *>(w), ActF32Q{x, xq, xs, xsum}, y, n, k, s);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}
