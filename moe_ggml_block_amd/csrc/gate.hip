// Router gate on gfx950: the f32 logits GEMV of a decode step, followed by
// the router (softmax + top-k + renormalize) on those logits.
//
// hanzo-ml `src/vulkan_backend.rs`, kernel table ("gemv"): at one token the
// MoE router gate is an f32 GEMV, logits[e] = Wr[e, :] . x, computed with one
// workgroup per output row and a workgroup reduction instead of the tiled
// GEMM. hanzo-kernel `src/main.rs` (`check_gemv`) sizes it at 128 router rows
// of 4096 f32 (2 MB per layer) and checks it against a CPU dot product.
//
// Work mapping here: a workgroup of four waves owns four consecutive router
// rows, one per wave, and a chunk of tokens. A wave keeps its row in
// registers (lane l holds float4 l, l + 64, l + 128, ... of the row), the
// chunk's activation rows are staged once per workgroup in LDS (coalesced
// 16-byte loads, read back as consecutive float4s per lane, which is
// conflict-free), and for each token every lane forms its partial dot with an
// fma chain, the wave sums the partials with DPP, and the last lane writes the
// logit. Per lane the partial dot is a sum of NV four-term float4 products
// (product, three fmas), so a logit carries at most NV + 9 roundings (4 per
// float4 product, NV - 1 additions, 6 reduction levels). A row is read from HBM once per token chunk; the chunk is as many
// activation rows as fit 64 KB of LDS (every token of a decode step at
// hidden <= 2048 for T <= 8).
//
// Logits go to the caller's buffer; the router kernels then run on them in
// stream order, so ids and weights never leave the device.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int GATE_WAVES = 4;
constexpr int GATE_LDS = 65536;     // staged activation bytes per workgroup
constexpr int GATE_SPT = GATE_LDS / 16 / 256;  // staged float4s per thread, at most
constexpr int GATE_MAX_HIDDEN = 8192;
constexpr int GATE_MAX_E = 4096;    // the router's limit
constexpr int GATE_MAX_YCHUNKS = 1024;

// NV = float4s per lane (hidden/4 rounded up to a multiple of 64, / 64);
// TU = tokens per inner iteration and JC = float4s per lane read per batch
// (at most 32 reads and 192 registers of row plus activations per lane).
template <int NV, int TU = (NV <= 4 ? 8 : NV == 8 ? 4 : NV == 16 ? 2 : 1), int JC = (NV >= 16 ? 16 : NV)>
__global__ __launch_bounds__(256) void k_gate(const float *__restrict__ w, const float *__restrict__ x,
                                              float *__restrict__ logits, int T, int E, int hidden, int tc,
                                              int nchunks) {
    constexpr int RS = 64 * NV;  // LDS row stride in float4s: the row zero-padded to whole slices
    extern __shared__ f4 xs4[];
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * GATE_WAVES + (threadIdx.x >> 6);
    const int er = e < E ? e : E - 1;  // spare waves read a valid row, write nothing
    const int h4 = hidden >> 2;
    const f4 *wrow = reinterpret_cast<const f4 *>(w + (size_t)er * hidden);
    f4 wr[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int v = lane + 64 * j;
        // past the row: 0 (a masked load into a zeroed register, so nothing
        // waits for the loads here); those lanes meet the 0 pad of x
        wr[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        if (v < h4) wr[j] = wrow[v];
    }
    auto chunk = [&](const int c) {
        const int t0 = c * tc;
        const int nt = min(tc, T - t0);
        const int np4 = nt * RS;
        const f4 *xg = reinterpret_cast<const f4 *>(x + (size_t)t0 * hidden);
        // every load of the chunk in flight before the first LDS store (one
        // memory latency per chunk); the pad past each row is written as 0
        f4 v[GATE_SPT];
#pragma unroll
        for (int u = 0; u < GATE_SPT; ++u) {
            const int i = threadIdx.x + 256 * u;
            const int col = i % RS;
            v[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};
            if (i < np4 && col < h4) v[u] = xg[(i / RS) * h4 + col];
        }
#pragma unroll
        for (int u = 0; u < GATE_SPT; ++u) {
            const int i = threadIdx.x + 256 * u;
            if (i < np4) xs4[i] = v[u];
        }
        __syncthreads();
        // TU tokens per iteration (a token index past the chunk repeats the
        // last one and is not stored); each batch of TU x JC reads is issued
        // before its arithmetic, in the same order of additions throughout.
        for (int t = 0; t < nt; t += TU) {
            float acc[TU];
#pragma unroll
            for (int q = 0; q < TU; ++q) acc[q] = 0.0f;
#pragma unroll
            for (int j0 = 0; j0 < NV; j0 += JC) {
                f4 xv[TU][JC];
#pragma unroll
                for (int q = 0; q < TU; ++q) {
                    const f4 *xt = xs4 + min(t + q, nt - 1) * RS + lane + 64 * j0;
#pragma unroll
                    for (int j = 0; j < JC; ++j) xv[q][j] = xt[64 * j];
                }
                // keep the reads ahead of the arithmetic (the scheduler would
                // otherwise keep two in flight to save registers)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < TU; ++q) {
#pragma unroll
                    for (int j = 0; j < JC; ++j) {
                        const f4 wj = wr[j0 + j];
                        float pj = wj.x * xv[q][j].x;
                        pj = fmaf(wj.y, xv[q][j].y, pj);
                        pj = fmaf(wj.z, xv[q][j].z, pj);
                        pj = fmaf(wj.w, xv[q][j].w, pj);
                        acc[q] += pj;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 0; q < TU; ++q) acc[q] = group_sum_last<64>(acc[q]);
#pragma unroll
            for (int q = 0; q < TU; ++q)
                if (lane == 63 && e < E && t + q < nt) logits[(size_t)(t0 + t + q) * E + e] = acc[q];
        }
    };
    // The first chunk is peeled out of the loop so that its activation loads
    // issue right behind the row loads (a loop header makes the compiler wait
    // for every outstanding load first); later chunks wait for the readers of
    // the previous one before overwriting the LDS.
    chunk(blockIdx.y);
    for (int c = blockIdx.y + gridDim.y; c < nchunks; c += gridDim.y) {
        __syncthreads();
        chunk(c);
    }
}

template <int NV>
void launch_gate(const float *w, const float *x, float *logits, int64_t T, int64_t E, int64_t hidden,
                 hipStream_t s) {
    const int64_t row_lds = (int64_t)NV * 64 * 16;  // padded LDS bytes per token
    const int64_t tc = std::min<int64_t>(T, GATE_LDS / row_lds);
    const int64_t nchunks = (T + tc - 1) / tc;
    const dim3 grid((unsigned)((E + GATE_WAVES - 1) / GATE_WAVES),
                    (unsigned)std::min<int64_t>(nchunks, GATE_MAX_YCHUNKS));
    hipLaunchKernelGGL((k_gate<NV>), grid, dim3(256), (size_t)(tc * row_lds), s, w, x, logits, (int)T,
                       (int)E, (int)hidden, (int)tc, (int)nchunks);
}

// logits = x Wr^T (all checks done by the caller)
int launch_logits(const float *wr, const float *x, float *logits, int64_t T, int64_t E, int64_t hidden, hipStream_t s) {
    const int64_t nv64 = (hidden / 4 + 63) / 64;  // float4s per lane
    if (nv64 <= 1) launch_gate<1>(wr, x, logits, T, E, hidden, s);
    else if (nv64 <= 2) launch_gate<2>(wr, x, logits, T, E, hidden, s);
    else if (nv64 <= 4) launch_gate<4>(wr, x, logits, T, E, hidden, s);
    else if (nv64 <= 8) launch_gate<8>(wr, x, logits, T, E, hidden, s);
    else if (nv64 <= 16) launch_gate<16>(wr, x, logits, T, E, hidden, s);
    else launch_gate<32>(wr, x, logits, T, E, hidden, s);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

int check_gate(const float *wr, const float *x, const float *logits, const int32_t *ids, const float *wts, int64_t T,
               int64_t E, int64_t hidden, int64_t topk) {
    if (!wr || !x || !logits || !ids || !wts || T < 1 || E < 1 || hidden < 4 || hidden % 4 || topk < 1 ||
        topk > E || topk > 64)
        return QMV_EINVAL;
    if (E > GATE_MAX_E || hidden > GATE_MAX_HIDDEN || T > (1 << 24)) return QMV_EUNSUPPORTED;
    if (!aligned(wr, 16) || !aligned(x, 16) || !aligned(logits, 4) || !aligned(ids, 4) || !aligned(wts, 4))
        return QMV_EALIGN;
    return QMV_OK;
}

}  // namespace

extern "C" int moe_gate_route(const float *wr, const float *x, float *logits, int32_t *ids, float *wts,
                              int64_t T, int64_t E, int64_t hidden, int64_t topk, qmv_stream_t stream) {
    int rc = check_gate(wr, x, logits, ids, wts, T, E, hidden, topk);
    if (rc) return rc;
    rc = launch_logits(wr, x, logits, T, E, hidden, (hipStream_t)stream);
    if (rc) return rc;
    return moe_route(logits, ids, wts, T, E, topk, stream);
}

// The MoE block from the hidden state: router gate GEMV, then the layer with
// the router fused into its gate/up gather (moe_ffn_routed_q4k_q6k).
extern "C" int moe_block_q4k_q6k(const float *wr, const void *gate, const void *up, const void *down, const float *x,
                                 float *logits, int32_t *ids, float *wts, float *y, void *ws, int64_t ws_bytes,
                                 int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E,
                                 qmv_stream_t stream) {
    int rc = check_gate(wr, x, logits, ids, wts, T, E, hidden, topk);
    if (rc) return rc;
    // the layer's own checks before anything is launched
    rc = qmv_internal::check_decode_layer(gate, up, down, x, ids, wts, y, ws, ws_bytes, T, topk, hidden, inter, E);
    if (rc) return rc;
    rc = launch_logits(wr, x, logits, T, E, hidden, (hipStream_t)stream);
    if (rc) return rc;
    return moe_ffn_routed_q4k_q6k(gate, up, down, x, logits, ids, wts, y, ws, ws_bytes, T, topk, hidden, inter, E,
                                  stream);
}
