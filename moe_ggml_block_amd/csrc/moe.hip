// Indexed-MoE decode path on gfx950: fused router, expert-gather matvecs
// over resident Q4_K / Q6_K banks, fused SiLU(gate)*up, and the weighted
// combine.
//
// hanzo-ml `src/vulkan_backend.rs`:
//  - `moe_route_vk`: softmax + top-k + renormalize in one kernel, one
//    workgroup per token, ids and weights stay on the device;
//  - `moe_matvec_gpu`: y[s, r] = sum_k W[ids[s], r, k] * x[s, k] over a
//    resident [E, n, k] bank, output in slot order, ids never read back;
//  - `silu_mul` and the engine's `broadcast_mul(scores).sum` combine.
//
// Expert grouping: workgroup (row block rb, group g) serves the g-th distinct
// expert present in ids (ascending expert id) and every slot routed to it, in
// slot order, so an expert's rows are streamed from HBM once per call however
// many slots chose it. The grouping is recomputed by each workgroup from ids
// (a bitmap of present experts in LDS and a ballot compaction of the slots);
// the grid has min(E, nslots) groups and workgroups past the number of
// distinct experts exit at once.
#include "blocks.hpp"

namespace {

constexpr int MAX_E = 4096;
constexpr int MAX_SLOTS = 4096;
constexpr int WAVES = 4;

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- router ---
// One wave per token, VPL logits per lane (lane l holds experts l + 64 v).
// topk rounds of a wave-wide argmax on (value desc, index asc); NaN and
// padding rank as -inf, padding and taken entries carry index INT_MAX so a
// real -inf entry always beats them.
template <int VPL>
__global__ __launch_bounds__(256) void k_moe_route(const float *__restrict__ logits,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wts, int T, int E, int topk) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (t >= T) return;
    float v[VPL];
    int ix[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            float l = logits[(size_t)t * E + e];
            v[i] = (l != l) ? -INFINITY : l;
            ix[i] = e;
        } else {
            v[i] = -INFINITY;
            ix[i] = 0x7FFFFFFF;
        }
    }
    float my_v = -INFINITY;
    int my_i = 0x7FFFFFFF;
    for (int j = 0; j < topk; ++j) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (v[i] > bv || (v[i] == bv && ix[i] < bi)) {
                bv = v[i];
                bi = ix[i];
            }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        // remove the winner from its owner's registers
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (ix[i] == bi) {
                v[i] = -INFINITY;
                ix[i] = 0x7FFFFFFF;
            }
        if (lane == j) {
            my_v = bv;
            my_i = bi;
        }
    }
    const float lmax = __shfl(my_v, 0);
    float p = 0.0f;
    if (lane < topk) p = (lmax == -INFINITY) ? 1.0f : expf(my_v - lmax);
    float den = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    if (lane < topk) {
        ids[(size_t)t * topk + lane] = my_i;
        wts[(size_t)t * topk + lane] = p / den;
    }
}

// --------------------------------------------------------- grouping ---
struct Group {
    int expert;  // -1: no such group
    int count;   // slots routed to it
};

// Whole workgroup: find the g-th distinct valid expert of ids[0..nslots) and
// write its slots (ascending) to slot_list. Every thread gets the result.
__device__ Group find_group(const int32_t *__restrict__ ids, int nslots, int E, int g,
                            uint32_t *bitmap, int *slot_list, int *shared) {
    const int tid = threadIdx.x;
    const int words = (E + 31) >> 5;
    for (int i = tid; i < words; i += blockDim.x) bitmap[i] = 0u;
    __syncthreads();
    for (int s = tid; s < nslots; s += blockDim.x) {
        const int e = ids[s];
        if (e >= 0 && e < E) atomicOr(&bitmap[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    if (tid < 64) {
        // wave 0: locate the word holding the g-th set bit by a running popcount
        int base = 0, found = -1;
        for (int w0 = 0; w0 < words && found < 0; w0 += 64) {
            const int wi = w0 + tid;
            const uint32_t bits = wi < words ? bitmap[wi] : 0u;
            int c = __popc(bits);
            // inclusive scan of c across the wave
            int incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(incl, off);
                if (tid >= off) incl += o;
            }
            const int excl = incl - c;
            const bool hit = (g >= base + excl) && (g < base + incl);
            const unsigned long long m = __ballot(hit);
            if (m) {
                const int src = __ffsll((long long)m) - 1;
                if (tid == src) {
                    uint32_t b = bits;
                    int need = g - base - excl;
                    while (need-- > 0) b &= b - 1;
                    shared[0] = wi * 32 + (__ffs((int)b) - 1);
                }
                found = 1;
            }
            base += __shfl(incl, 63);
        }
        if (found < 0 && tid == 0) shared[0] = -1;
    }
    __syncthreads();
    Group G;
    G.expert = shared[0];
    G.count = 0;
    if (G.expert < 0) return G;
    if (tid < 64) {
        int cnt = 0;
        for (int s0 = 0; s0 < nslots; s0 += 64) {
            const int s = s0 + tid;
            const bool f = s < nslots && ids[s] == G.expert;
            const unsigned long long m = __ballot(f);
            if (f) slot_list[cnt + __popcll(m & ((1ull << tid) - 1ull))] = s;
            cnt += __popcll(m);
        }
        if (tid == 0) shared[1] = cnt;
    }
    __syncthreads();
    G.count = shared[1];
    return G;
}

// Zero the output rows [r0, r1) of slots whose id is out of range.
__device__ void zero_invalid(const int32_t *__restrict__ ids, int nslots, int E, float *y, int n,
                             int r0, int r1) {
    for (int s = 0; s < nslots; ++s) {
        const int e = ids[s];
        if (e < 0 || e >= E)
            for (int r = r0 + (int)threadIdx.x; r < r1; r += blockDim.x) y[(size_t)s * n + r] = 0.0f;
    }
}

// ------------------------------------------------------ gather matvec ---
// Rows of the expert are split over row blocks of `rblk` rows; inside a block
// the four waves take passes of 64/G rows in turn. For each chunk of SB slots
// the lanes load those slots' activation values into registers, then stream
// the rows. DUAL: two banks (gate, up) against the same activation, output
// silu(gate.x) * (up.x); otherwise one bank, plain output.
template <class F, int G, int UPL, int SB, bool DUAL>
__global__ __launch_bounds__(256) void k_moe(const uint8_t *__restrict__ bank,
                                             const uint8_t *__restrict__ bank2,
                                             const float *__restrict__ x, int x_div,
                                             const int32_t *__restrict__ ids,
                                             float *__restrict__ y, int nslots, int n, int k,
                                             int E, int rblk) {
    __shared__ uint32_t bitmap[MAX_E / 32];
    __shared__ int slot_list[MAX_SLOTS];
    __shared__ int shared[2];
    constexpr int RPP = 64 / G;
    using Raw = typename F::Raw;
    const int r0 = blockIdx.x * rblk;
    const int r1 = min(n, r0 + rblk);
    if (blockIdx.y == 0) zero_invalid(ids, nslots, E, y, n, r0, r1);
    const Group grp = find_group(ids, nslots, E, blockIdx.y, bitmap, slot_list, shared);
    if (grp.expert < 0) return;
    const int U = F::units_per_row(k);
    const size_t row_bytes = (size_t)(k / F::BW) * F::BB;
    const uint8_t *wb = bank + (size_t)grp.expert * n * row_bytes;
    const uint8_t *wb2 = DUAL ? bank2 + (size_t)grp.expert * n * row_bytes : nullptr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gl = lane & (G - 1), grow = lane / G;
    bool uv[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) uv[i] = gl + G * i < U;

    for (int sc0 = 0; sc0 < grp.count; sc0 += SB) {
        const int ns = min(SB, grp.count - sc0);
        UnitX X[SB][UPL];
        int sl[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) sl[j] = j < ns ? slot_list[sc0 + j] : -1;
#pragma unroll
        for (int i = 0; i < UPL; ++i)
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (uv[i] && j < ns) F::load_x(X[j][i], x + (size_t)(sl[j] / x_div) * k, gl + G * i);
        for (int rb = r0 + wave * RPP; rb < r1; rb += WAVES * RPP) {
            const int r = rb + grow;
            const bool rv = r < r1;
            Raw R[UPL], R2[UPL];
#pragma unroll
            for (int i = 0; i < UPL; ++i)
                if (rv && uv[i]) {
                    F::load(R[i], wb + (size_t)r * row_bytes, gl + G * i);
                    if (DUAL) F::load(R2[i], wb2 + (size_t)r * row_bytes, gl + G * i);
                }
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                if (j >= ns) break;
                float a = 0.0f, b = 0.0f;
#pragma unroll
                for (int i = 0; i < UPL; ++i)
                    if (rv && uv[i]) {
                        a += F::dot(R[i], X[j][i], gl + G * i);
                        if (DUAL) b += F::dot(R2[i], X[j][i], gl + G * i);
                    }
                a = group_sum_last<G>(a);
                if (DUAL) b = group_sum_last<G>(b);
                if (gl == G - 1 && rv) y[(size_t)sl[j] * n + r] = DUAL ? silu(a) * b : a;
            }
        }
    }
}

// ------------------------------------------------------------ combine ---
// y[t, r] = sum_j wts[t, j] * d[topk*t + j, r], j ascending.
__global__ __launch_bounds__(256) void k_moe_combine(const float *__restrict__ d,
                                                     const float *__restrict__ wts,
                                                     float *__restrict__ y, int T, int topk,
                                                     int hidden) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * hidden) return;
    const int t = (int)(i / hidden), r = (int)(i % hidden);
    float acc = 0.0f;
    for (int j = 0; j < topk; ++j)
        acc = fmaf(wts[(size_t)t * topk + j], d[((size_t)t * topk + j) * hidden + r], acc);
    y[i] = acc;
}

// --------------------------------------------------------------- launch ---
// Rows per workgroup: keep >= ~2048 workgroups-worth of waves when few
// experts are active, while each wave still streams several rows.
int pick_rblk(int64_t n, int G, int64_t groups) {
    const int rpp = 64 / G;
    int rblk = WAVES * rpp * 4;  // 4 passes per wave
    while (rblk > WAVES * rpp && div_up(n, rblk) * groups < 1024) rblk /= 2;
    return rblk;
}

template <class F, bool DUAL>
int launch_moe(const uint8_t *bank, const uint8_t *bank2, const float *x, int64_t x_div,
               const int32_t *ids, float *y, int64_t nslots, int64_t n, int64_t k, int64_t E, hipStream_t s) {
    const int64_t U = k / 64;
    const int G = next_pow2_le64(U);
    const int64_t groups = E < nslots ? E : nslots;
    const int rblk = pick_rblk(n, G, groups);
    const dim3 grid((unsigned)div_up(n, rblk), (unsigned)groups);
#define MQ(GG, UU, SB)                                                                                 \
    hipLaunchKernelGGL((k_moe<F, GG, UU, SB, DUAL>), grid, dim3(256), 0, s, bank, bank2, x, (int)x_div, ids, y, \
                       (int)nslots, (int)n, (int)k, (int)E, rblk)
    switch (G) {
        case 1: MQ(1, 1, 2); break;
        case 2: MQ(2, 1, 2); break;
        case 4: MQ(4, 1, 2); break;
        case 8: MQ(8, 1, 2); break;
        case 16: MQ(16, 1, 2); break;
        case 32: MQ(32, 1, 2); break;
        default:
            if (U <= 64) MQ(64, 1, 2);
            else if (U <= 128) MQ(64, 2, 1);
            else return QMV_EUNSUPPORTED;
    }
#undef MQ
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

int launch_moe_q4k(const uint8_t *bank, const uint8_t *bank2, const float *x, int64_t x_div,
                   const int32_t *ids, float *y, int64_t nslots, int64_t n, int64_t k, int64_t E,
                   hipStream_t s) {
    if (bank2) return launch_moe<Q4KUnit, true>(bank, bank2, x, x_div, ids, y, nslots, n, k, E, s);
    return launch_moe<Q4KUnit, false>(bank, nullptr, x, x_div, ids, y, nslots, n, k, E, s);
}

int launch_moe_q6k(const uint8_t *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                   int64_t nslots, int64_t n, int64_t k, int64_t E, hipStream_t s) {
    return launch_moe<Q6KUnit, false>(bank, nullptr, x, x_div, ids, y, nslots, n, k, E, s);
}

int check_moe_args(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                   int64_t nslots, int64_t n, int64_t k, int64_t E) {
    if (!bank || !x || !ids || !y || x_div < 1 || nslots < 1 || n < 1 || E < 1 || k < 256 || k % 256)
        return QMV_EINVAL;
    if (E > MAX_E || nslots > MAX_SLOTS || k > 8192 || n > (1 << 24) ||
        (int64_t)E * n * (k / 256) * 210 > ((int64_t)1 << 40))
        return QMV_EUNSUPPORTED;
    if (!aligned(bank, 16) || !aligned(x, 16) || !aligned(ids, 4) || !aligned(y, 4)) return QMV_EALIGN;
    return QMV_OK;
}

}  // namespace

extern "C" int moe_route(const float *logits, int32_t *ids, float *wts, int64_t T, int64_t E,
                         int64_t topk, qmv_stream_t stream) {
    if (!logits || !ids || !wts || T < 1 || E < 1 || topk < 1 || topk > E || topk > 64) return QMV_EINVAL;
    if (E > MAX_E || T > (1 << 28)) return QMV_EUNSUPPORTED;
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(wts, 4)) return QMV_EALIGN;
    const dim3 grid((unsigned)div_up(T, WAVES));
    hipStream_t s = (hipStream_t)stream;
    const int vpl = (int)div_up(E, 64);
#define RT(V) hipLaunchKernelGGL((k_moe_route<V>), grid, dim3(256), 0, s, logits, ids, wts, (int)T, (int)E, (int)topk)
    if (vpl <= 1) RT(1);
    else if (vpl <= 2) RT(2);
    else if (vpl <= 4) RT(4);
    else if (vpl <= 8) RT(8);
    else if (vpl <= 16) RT(16);
    else if (vpl <= 32) RT(32);
    else RT(64);
#undef RT
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

extern "C" int moe_qmv_q4k(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                           int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream) {
    const int rc = check_moe_args(bank, x, x_div, ids, y, nslots, n, k, E);
    if (rc) return rc;
    return launch_moe_q4k(static_cast<const uint8_t *>(bank), nullptr, x, x_div, ids, y, nslots, n, k, E,
                          (hipStream_t)stream);
}

extern "C" int moe_qmv_q6k(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                           int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream) {
    const int rc = check_moe_args(bank, x, x_div, ids, y, nslots, n, k, E);
    if (rc) return rc;
    return launch_moe_q6k(static_cast<const uint8_t *>(bank), x, x_div, ids, y, nslots, n, k, E,
                          (hipStream_t)stream);
}

extern "C" int64_t moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t hidden, int64_t inter) {
    if (T < 1 || topk < 1 || hidden < 1 || inter < 1) return -1;
    const int64_t ns = T * topk;
    const int64_t h = div_up(ns * inter * 4, 256) * 256;
    const int64_t d = div_up(ns * hidden * 4, 256) * 256;
    return h + d;
}

extern "C" int moe_ffn_q4k_q6k(const void *gate, const void *up, const void *down, const float *x,
                               const int32_t *ids, const float *wts, float *y, void *ws, int64_t ws_bytes,
                               int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E,
                               qmv_stream_t stream) {
    if (!gate || !up || !down || !x || !ids || !wts || !y || !ws) return QMV_EINVAL;
    if (T < 1 || topk < 1 || hidden < 256 || inter < 256 || hidden % 256 || inter % 256) return QMV_EINVAL;
    const int64_t need = moe_ffn_workspace_bytes(T, topk, hidden, inter);
    if (ws_bytes < need) return QMV_EINVAL;
    const int64_t ns = T * topk;
    int rc = check_moe_args(gate, x, topk, ids, y, ns, inter, hidden, E);
    if (rc) return rc;
    rc = check_moe_args(down, x, 1, ids, y, ns, hidden, inter, E);
    if (rc) return rc;
    if (!aligned(up, 16) || !aligned(wts, 4) || !aligned(ws, 16)) return QMV_EALIGN;
    float *h = static_cast<float *>(ws);
    float *d = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + div_up(ns * inter * 4, 256) * 256);
    hipStream_t s = (hipStream_t)stream;
    rc = launch_moe_q4k(static_cast<const uint8_t *>(gate), static_cast<const uint8_t *>(up), x, topk, ids, h,
                        ns, inter, hidden, E, s);
    if (rc) return rc;
    rc = launch_moe_q6k(static_cast<const uint8_t *>(down), h, 1, ids, d, ns, hidden, inter, E, s);
    if (rc) return rc;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)div_up(T * hidden, 256)), dim3(256), 0, s, d, wts, y,
                       (int)T, (int)topk, (int)hidden);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}
