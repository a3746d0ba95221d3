// Dense decode matvecs y = W_deq x over raw Q8_0 / Q4_K / Q6_K rows (gfx950).
//
// Defined by hanzo-ml `src/vulkan_backend.rs`: `matvec_q8_0_gpu`,
// `matvec_q4k_gpu_off` and `matvec_q6k_gpu_off` (y[nout] = Wq * x[k], blocks
// read verbatim from a resident buffer, no requantization).
//
// Work mapping. A row is cut into U units of 64 weights (blocks.hpp). An
// aligned group of G lanes (G = next power of two >= U, at most 64) owns one
// row; lane i of the group decodes units i and i+G (UPL <= 2). The
// activation values under a lane's units are the same for every row, so each
// lane loads its 64*UPL values into registers once (from L1/L2: x is small
// and shared by every wave) and the wave then streams rows, 64/G per pass.
// Each wave owns a contiguous range of passes and keeps a ring of NB passes
// in flight: the weight loads of pass i+NB are issued as soon as pass i has
// been decoded, so HBM latency is covered by NB passes of decode work (and
// by the other waves of the SIMD). All loads are unconditional -- row and
// unit indices past the end are clamped to valid ones and their results
// discarded -- so the compiler can wait for exactly the oldest pass
// (s_waitcnt vmcnt(N)) instead of draining the ring. Partial sums are
// reduced across the G lanes with DPP.
//
// Launch shape: the grid is sized from the occupancy of the kernel so that
// every wave is resident at once (one round, no tail), each wave taking an
// equal share of the passes.
#include "blocks.hpp"

namespace {

#ifndef QMV_NB
#define QMV_NB 4
#endif
#ifndef QMV_ROUNDS_X4
#define QMV_ROUNDS_X4 4
#endif
constexpr int WAVES_PER_BLOCK = 4;
constexpr int NB = QMV_NB;  // passes in flight per wave
// waves launched = resident waves * ROUNDS_X4 / 4
constexpr int ROUNDS_X4 = QMV_ROUNDS_X4;

template <class F, int G, int UPL>
__global__ __launch_bounds__(256) void k_dense(const uint8_t *__restrict__ w,
                                               const float *__restrict__ x,
                                               float *__restrict__ y, int n, int k,
                                               int row_bytes, int per_wave) {
    extern __shared__ float xlds[];
    constexpr int RPP = 64 / G;
    using Raw = typename F::Raw;
    const int tid = threadIdx.x, lane = tid & 63;
    const int gl = lane & (G - 1), grow = lane / G;
    const int U = F::units_per_row(k);
    const int passes = (n + RPP - 1) / RPP;
    const int wave = blockIdx.x * WAVES_PER_BLOCK + (tid >> 6);
    const int p0 = wave * per_wave;
    const int p1 = min(passes, p0 + per_wave);
    const bool idle = p0 >= p1;  // still takes part in the x staging barrier
    bool uv[UPL];
    int uu[UPL];  // unit actually read (clamped into the row)
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        uv[i] = gl + G * i < U;
        uu[i] = uv[i] ? gl + G * i : U - 1;
    }
    Raw R[NB][UPL];
    auto load_pass = [&](Raw (&B)[UPL], int pass) {
        const int r = max(min(pass * RPP + grow, n - 1), 0);
        const uint8_t *row = w + (size_t)r * row_bytes;
#pragma unroll
        for (int i = 0; i < UPL; ++i) F::load(B[i], row, uu[i]);
    };
    // The ring only works if the passes' loads are issued oldest-first: a
    // scheduling barrier after each pass keeps the compiler from reordering
    // them (the first buffer consumed must be the first one requested).
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        load_pass(R[j], min(p0 + j, p1 - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    // activations: coalesced loads into the padded LDS layout, then each
    // lane reads its units' values (conflict-free) into registers
    stage_x<F>(xlds, x, k);
    __syncthreads();
    UnitX X[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) load_x_lds(X[i], xlds, uu[i]);
    if (idle) return;

    for (int pass = p0; pass < p1; pass += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int ps = pass + j;
            const int r = ps * RPP + grow;
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const float d = F::dot(R[j][i], X[i], uu[i]);
                acc += uv[i] ? d : 0.0f;
            }
            __builtin_amdgcn_sched_barrier(0);
            load_pass(R[j], min(ps + NB, p1 - 1));
            __builtin_amdgcn_sched_barrier(0);
            acc = group_sum_last<G>(acc);
            if (gl == G - 1 && ps < p1 && r < n) y[r] = acc;
        }
    }
}

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
struct DevInfo {
    int device = -1;
    int cus = 256;
};

int compute_units() {
    static thread_local DevInfo info;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (info.device != dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        info.device = dev;
        info.cus = cus;
    }
    return info.cus;
}

// Resident waves of a kernel on the whole device (one full round).
template <class K>
int64_t resident_waves(K kernel, size_t lds) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess || per_cu < 1)
        per_cu = 2;
    return (int64_t)per_cu * compute_units() * WAVES_PER_BLOCK * ROUNDS_X4 / 4;
}

template <class F, int G, int UPL>
void launch(const uint8_t *w, const float *x, float *y, int64_t n, int64_t k, int64_t row_bytes,
            hipStream_t s) {
    const int64_t rpp = 64 / G;
    const int64_t passes = (n + rpp - 1) / rpp;
    const size_t lds = (size_t)(k / 64) * XSTRIDE * 4;
    // occupancy depends on (device, LDS bytes) only: remember the last answer
    static thread_local int c_dev = -1;
    static thread_local size_t c_lds = 0;
    static thread_local int64_t c_target = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != c_dev || lds != c_lds) {
        c_target = resident_waves(k_dense<F, G, UPL>, lds);
        c_dev = dev;
        c_lds = lds;
    }
    const int64_t target = c_target;
    int64_t per = (passes + target - 1) / target;
    if (per < 1) per = 1;
    const int64_t waves = (passes + per - 1) / per;
    const dim3 grid((unsigned)((waves + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK));
    hipLaunchKernelGGL((k_dense<F, G, UPL>), grid, dim3(256), lds, s, w, x, y, (int)n, (int)k, (int)row_bytes,
                       (int)per);
}

template <class F>
int launch_dense(const uint8_t *w, const float *x, float *y, int64_t n, int64_t k, hipStream_t s) {
    const int64_t row_bytes = k / F::BW * F::BB;
    const bool tiled = (k % 64 == 0) && k <= 8192;  // units of 64 weights, x fits LDS
    const int64_t U = k / 64;
    const int fmt = F::BB == 34 ? 0 : (F::BB == 144 ? 1 : 2);
    if (!tiled) {
        const dim3 grid((unsigned)((n + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK));
        hipLaunchKernelGGL(k_qmv_generic, grid, dim3(256), 0, s, fmt, w, x, y, n, k, row_bytes);
        QMV_LAUNCH_CHECK();
        return QMV_OK;
    }
    const int G = next_pow2_le64(U);
    switch (G) {
        case 1: launch<F, 1, 1>(w, x, y, n, k, row_bytes, s); break;
        case 2: launch<F, 2, 1>(w, x, y, n, k, row_bytes, s); break;
        case 4: launch<F, 4, 1>(w, x, y, n, k, row_bytes, s); break;
        case 8: launch<F, 8, 1>(w, x, y, n, k, row_bytes, s); break;
        case 16: launch<F, 16, 1>(w, x, y, n, k, row_bytes, s); break;
        case 32: launch<F, 32, 1>(w, x, y, n, k, row_bytes, s); break;
        default:
            if (U <= 64) launch<F, 64, 1>(w, x, y, n, k, row_bytes, s);
            else launch<F, 64, 2>(w, x, y, n, k, row_bytes, s);
    }
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
