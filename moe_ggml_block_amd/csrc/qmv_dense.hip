// Dense decode matvecs y = W_deq x over raw Q8_0 / Q4_K / Q6_K rows (gfx950).
//
// Defined by hanzo-ml `src/vulkan_backend.rs`: `matvec_q8_0_gpu`,
// `matvec_q4k_gpu_off` and `matvec_q6k_gpu_off` (y[nout] = Wq * x[k], blocks
// read verbatim from a resident buffer, no requantization).
//
// Work mapping: a row is cut into U units (see blocks.hpp). An aligned group
// of G lanes (G = next power of two >= U, at most 64) owns one row; lane i of
// the group decodes units i, i+G, i+2G, ... (UPL of them). The activation
// values under a lane's units never change from row to row, so each lane
// loads them into registers once and the wave then streams rows: 64/G rows
// per pass, RB passes' loads issued before any of their math. Partial sums
// are reduced across the G lanes with cross-lane shuffles.
#include "blocks.hpp"

namespace {

constexpr int WAVES_PER_BLOCK = 4;

struct RowSched {
    int n;             // rows
    int passes;        // ceil(n / rows_per_pass)
    int per_wave;      // passes per wave
};

// --------------------------------------------------------------------- Q4_K
template <int G, int UPL, int RB>
__global__ __launch_bounds__(256) void k_qmv_q4k(const uint8_t *__restrict__ w,
                                                 const float *__restrict__ x,
                                                 float *__restrict__ y, RowSched rs, int U,
                                                 int row_bytes) {
    constexpr int RPP = 64 / G;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int grow = lane / G;
    const int wave = blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
    const int p0 = wave * rs.per_wave;
    if (p0 >= rs.passes) return;
    const int p1 = min(rs.passes, p0 + rs.per_wave);
    const int c = gl & 7, pr = c >> 1;

    Q4KX X[UPL];
    bool uv[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = gl + G * i;
        uv[i] = u < U;
        if (uv[i]) q4k_load_x(X[i], x, u >> 3, c);
    }

    for (int pass = p0; pass < p1; pass += RB) {
        uint4 qd[RB][UPL], md[RB][UPL];
        bool rv[RB];
        int rr[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            rr[b] = (pass + b) * RPP + grow;
            rv[b] = (pass + b) < p1 && rr[b] < rs.n;
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                if (rv[b] && uv[i]) {
                    const uint8_t *blk = w + (size_t)rr[b] * row_bytes + (size_t)((gl + G * i) >> 3) * 144;
                    qd[b][i] = ld16(blk + 16 + 16 * c);
                    md[b][i] = ld16(blk);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv[b] && uv[i]) acc += q4k_unit_dot(qd[b][i], md[b][i], X[i], pr);
            acc = group_sum<G>(acc);
            if (gl == 0 && rv[b]) y[rr[b]] = acc;
        }
    }
}

// --------------------------------------------------------------------- Q6_K
template <int G, int UPL, int RB>
__global__ __launch_bounds__(256) void k_qmv_q6k(const uint8_t *__restrict__ w,
                                                 const float *__restrict__ x,
                                                 float *__restrict__ y, RowSched rs, int U,
                                                 int row_bytes) {
    constexpr int RPP = 64 / G;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int grow = lane / G;
    const int wave = blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
    const int p0 = wave * rs.per_wave;
    if (p0 >= rs.passes) return;
    const int p1 = min(rs.passes, p0 + rs.per_wave);
    const int u8 = gl & 7;

    Q6KX X[UPL];
    bool uv[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = gl + G * i;
        uv[i] = u < U;
        if (uv[i]) q6k_load_x(X[i], x, u >> 3, u8);
    }

    for (int pass = p0; pass < p1; pass += RB) {
        Q6KRaw R[RB][UPL];
        bool rv[RB];
        int rr[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            rr[b] = (pass + b) * RPP + grow;
            rv[b] = (pass + b) < p1 && rr[b] < rs.n;
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv[b] && uv[i])
                    q6k_load(R[b][i], w + (size_t)rr[b] * row_bytes + (size_t)((gl + G * i) >> 3) * 210, u8);
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv[b] && uv[i]) acc += q6k_unit_dot(R[b][i], X[i], u8);
            acc = group_sum<G>(acc);
            if (gl == 0 && rv[b]) y[rr[b]] = acc;
        }
    }
}

// --------------------------------------------------------------------- Q8_0
template <int G, int UPL, int RB>
__global__ __launch_bounds__(256) void k_qmv_q8_0(const uint8_t *__restrict__ w,
                                                  const float *__restrict__ x,
                                                  float *__restrict__ y, RowSched rs, int U,
                                                  int row_bytes) {
    constexpr int RPP = 64 / G;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int grow = lane / G;
    const int wave = blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
    const int p0 = wave * rs.per_wave;
    if (p0 >= rs.passes) return;
    const int p1 = min(rs.passes, p0 + rs.per_wave);

    float X[UPL][64];
    bool uv[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = gl + G * i;
        uv[i] = u < U;
        if (uv[i]) {
            const float4 *a = reinterpret_cast<const float4 *>(x + 64 * u);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float4 v = a[t];
                X[i][4 * t] = v.x; X[i][4 * t + 1] = v.y; X[i][4 * t + 2] = v.z; X[i][4 * t + 3] = v.w;
            }
        }
    }

    for (int pass = p0; pass < p1; pass += RB) {
        Q8Pair P[RB][UPL];
        bool rv[RB];
        int rr[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            rr[b] = (pass + b) * RPP + grow;
            rv[b] = (pass + b) < p1 && rr[b] < rs.n;
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv[b] && uv[i]) q8_load(P[b][i], w + (size_t)rr[b] * row_bytes + (size_t)(gl + G * i) * 68);
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv[b] && uv[i]) acc += q8_pair_dot(P[b][i], X[i]);
            acc = group_sum<G>(acc);
            if (gl == 0 && rv[b]) y[rr[b]] = acc;
        }
    }
}

// ------------------------------------------------------- generic fallback
// One wave per row, lanes over blocks, byte loads: any k that is a block
// multiple and any alignment of rows (used when the unit tiling above does
// not apply, e.g. Q8_0 with k % 64 == 32 or very long rows).
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
    const int bw = fmt == 0 ? 32 : 256, bb = fmt == 0 ? 34 : (fmt == 1 ? 144 : 210);
    const int64_t nb = k / bw;
    float acc = 0.0f;
    for (int64_t b = lane; b < nb; b += 64) acc += block_dot_generic(fmt, w + r * row_bytes + b * bb, x + b * bw);
    acc = group_sum<64>(acc);
    if (lane == 0) y[r] = acc;
}

// ------------------------------------------------------------- dispatch
RowSched make_sched(int64_t n, int G, int64_t target_waves) {
    RowSched rs;
    rs.n = (int)n;
    const int rpp = 64 / G;
    rs.passes = (int)((n + rpp - 1) / rpp);
    int per = (int)((rs.passes + target_waves - 1) / target_waves);
    rs.per_wave = per < 1 ? 1 : per;
    return rs;
}

// Waves to aim for: enough rows in flight to cover HBM latency on 256 CUs,
// few enough that each wave amortizes its activation loads over many rows.
constexpr int64_t TARGET_WAVES = 4096;

#define QMV_DISPATCH(KERNEL, G, UPL, ...)                                                     \
    do {                                                                                    \
        RowSched rs = make_sched(n, G, TARGET_WAVES);                                       \
        const int64_t waves = (rs.passes + rs.per_wave - 1) / rs.per_wave;                  \
        const dim3 grid((unsigned)((waves + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK));      \
        hipLaunchKernelGGL((KERNEL<G, UPL, 2>), grid, dim3(256), 0, stream, __VA_ARGS__, rs, \
                           (int)U, (int)row_bytes);                                         \
    } while (0)

template <int F>
int launch_dense(const uint8_t *w, const float *x, float *y, int64_t n, int64_t k, hipStream_t stream) {
    // units per row and their tiling
    const int64_t bw = F == 0 ? 32 : 256, bb = F == 0 ? 34 : (F == 1 ? 144 : 210);
    const int64_t row_bytes = k / bw * bb;
    int64_t U;
    bool tiled;
    if (F == 0) {
        U = k / 64;
        tiled = (k % 64 == 0) && U >= 1;
    } else {
        U = (k / 256) * 8;
        tiled = true;
    }
    const int G = next_pow2_le64(U);
    const int64_t upl = (U + G - 1) / G;
    if (!tiled || upl > (F == 0 ? 2 : 4)) {
        const dim3 grid((unsigned)((n + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK));
        hipLaunchKernelGGL(k_qmv_generic, grid, dim3(256), 0, stream, F, w, x, y, n, k, row_bytes);
        QMV_LAUNCH_CHECK();
        return QMV_OK;
    }
#define QMV_CASES(KERNEL)                                                     \
    switch (G) {                                                              \
        case 1: QMV_DISPATCH(KERNEL, 1, 1, w, x, y); break;                   \
        case 2: QMV_DISPATCH(KERNEL, 2, 1, w, x, y); break;                   \
        case 4: QMV_DISPATCH(KERNEL, 4, 1, w, x, y); break;                   \
        case 8: QMV_DISPATCH(KERNEL, 8, 1, w, x, y); break;                   \
        case 16: QMV_DISPATCH(KERNEL, 16, 1, w, x, y); break;                 \
        case 32: QMV_DISPATCH(KERNEL, 32, 1, w, x, y); break;                 \
        default:                                                              \
            if (upl == 1) QMV_DISPATCH(KERNEL, 64, 1, w, x, y);               \
            else if (upl == 2) QMV_DISPATCH(KERNEL, 64, 2, w, x, y);          \
            else if (F != 0 && upl == 3) QMV_DISPATCH(KERNEL, 64, 3, w, x, y);\
            else if (F != 0) QMV_DISPATCH(KERNEL, 64, 4, w, x, y);            \
    }
    if (F == 0) {
        QMV_CASES(k_qmv_q8_0)
    } else if (F == 1) {
        QMV_CASES(k_qmv_q4k)
    } else {
        QMV_CASES(k_qmv_q6k)
    }
#undef QMV_CASES
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

template <int F>
int dense_entry(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream) {
    const int64_t bw = F == 0 ? 32 : 256;
    if (!w || !x || !y || n < 1 || k < bw || k % bw) return QMV_EINVAL;
    if (n > (int64_t)1 << 30 || k > (int64_t)1 << 24) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QMV_EALIGN;
    return launch_dense<F>(static_cast<const uint8_t *>(w), x, y, n, k, (hipStream_t)stream);
}

}  // namespace

extern "C" int qmv_q8_0(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<0>(w, x, y, n, k, s);
}
extern "C" int qmv_q4k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<1>(w, x, y, n, k, s);
}
extern "C" int qmv_q6k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t s) {
    return dense_entry<2>(w, x, y, n, k, s);
}
