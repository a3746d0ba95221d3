// Row-streaming matvec skeleton shared by the decode kernels (gfx950).
//
// y[r] = sum over the row's 64-weight units of F::dot(unit, activation).
// F (blocks.hpp) supplies the raw weight unit (Raw, load, dot), the
// activation pack passed to the kernel (Act), its per-unit register form (X)
// and its staging through registers into LDS (Stage, fetch, store,
// load_lds, ACT_STRIDE).
//
// Work mapping. A row is cut into U units of 64 weights (blocks.hpp). An
// aligned group of G lanes (G = next power of two >= U, at most 64) owns one
// row; lane i of the group decodes units i and i+G (UPL <= 2). The
// activation values under a lane's units are the same for every row: the
// block loads the activation once with coalesced 16-byte loads into a padded
// LDS layout (conflict-free reads; for f32 activations each unit's four
// 16-value sums go into its pad), and each lane then keeps its units'
// values in registers while the wave streams rows, 64/G per pass.
//
// Pass q of a wave is global pass q*nwaves + wave, so at any moment the grid
// reads one contiguous window of rows. Each wave keeps a ring of F::RING
// passes in flight: the weight loads of pass i+RING are issued as soon as
// pass i has been decoded, so HBM latency is covered by RING passes of decode
// work (and by the other waves of the SIMD). The activation loads are issued
// before the first ring loads and consumed after them, so their wait does not
// drain the ring. All loads are unconditional -- row and unit indices past
// the end are clamped to valid ones and their results discarded -- so the
// compiler waits for exactly the oldest pass (s_waitcnt vmcnt(N)) instead of
// draining the ring. Partial sums are reduced across the G lanes with DPP.
//
// Launch shape: the grid is sized from the occupancy of the kernel (capped
// at F::MAX_WG_PER_CU workgroups per CU) so that every wave is resident at
// once (one round, no tail).
#pragma once

#include <type_traits>

#include "blocks.hpp"

namespace qmv_dense {

constexpr int WAVES_PER_BLOCK = 4;

// Units whose first workgroup also writes a side output from the staged
// activation registers (F::side).
template <class F, class = void>
struct has_side : std::false_type {};
template <class F>
struct has_side<F, std::void_t<decltype(&F::template side<1>)>> : std::true_type {};

template <class F, int G, int UPL>
__global__ __launch_bounds__(256) void k_dense(const uint8_t *__restrict__ w,
                                               typename F::Act act,
                                               float *__restrict__ y, int n, int k,
                                               int row_bytes) {
    constexpr int NB = F::RING;  // passes in flight per wave
    extern __shared__ float4 xlds4[];
    float *xlds = reinterpret_cast<float *>(xlds4);
    constexpr int RPP = 64 / G;
    using Raw = typename F::Raw;
    const int tid = threadIdx.x, lane = tid & 63;
    const int gl = lane & (G - 1), grow = lane / G;
    const int U = F::units_per_row(k);
    const int passes = (n + RPP - 1) / RPP;
    // Pass q of this wave is global pass q*nwaves + wave: at any moment the
    // waves of the grid read one contiguous window of rows (DRAM-friendly),
    // not one far-apart stream each.
    const int wave = blockIdx.x * WAVES_PER_BLOCK + (tid >> 6);
    const int nwaves = gridDim.x * WAVES_PER_BLOCK;
    // passes of this wave (0 for the spare waves of the last workgroup); the
    // loop below runs at least once so that no branch separates the ring
    // loads from the barrier (the compiler would sink them past it), and the
    // spare waves discard their clamped pass.
    const int p0 = 0;
    const int pr = (passes - wave + nwaves - 1) / nwaves;  // wave < nwaves
    const int p1 = max(pr, 1);
    bool uv[UPL];
    int uu[UPL];  // unit actually read (clamped into the row)
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        uv[i] = gl + G * i < U;
        uu[i] = uv[i] ? gl + G * i : U - 1;
    }
    // activations first (their wait must not drain the weight ring)
    typename F::Stage S;
    F::template fetch<stage_granules(G, UPL)>(S, act, k);
    Raw R[NB][UPL];
    auto load_pass = [&](Raw (&B)[UPL], int pass) {
        const int r = max(min((pass * nwaves + wave) * RPP + grow, n - 1), 0);
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
    typename F::X X[UPL];
    if constexpr (has_side<F>::value) {
        if (blockIdx.x == 0) F::template side<stage_granules(G, UPL)>(S, act, k);  // uniform
    }
    if constexpr (!F::Q8 && std::is_same<typename F::X, UnitX>::value) {
        F::template store_s<stage_granules(G, UPL)>(xlds, S, k);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < UPL; ++i) F::load_lds_s(X[i], xlds, uu[i]);
    } else {
        F::template store<stage_granules(G, UPL)>(xlds, S, k);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < UPL; ++i) F::load_lds(X[i], xlds, uu[i]);
    }

    int pass = p0;
    do {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int ps = pass + j;
            const int r = (ps * nwaves + wave) * RPP + grow;
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
            if (gl == G - 1 && ps < pr && r < n) y[r] = acc;
        }
        pass += NB;
    } while (pass < p1);
}

struct DevInfo {
    int device = -1;
    int cus = 256;
};

inline int compute_units() {
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

// Resident waves of a kernel on the device (one round), with at most
// max_per_cu workgroups per CU: with more (and more rows in flight) the
// cold-weight streams got slower (F::MAX_WG_PER_CU, measured per format at
// its decode shape).
template <class K>
int64_t resident_waves(K kernel, size_t lds, int max_per_cu) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess || per_cu < 1)
        per_cu = 2;
    if (per_cu > max_per_cu) per_cu = max_per_cu;
    return (int64_t)per_cu * compute_units() * WAVES_PER_BLOCK;
}

template <class F, int G, int UPL>
void launch(const uint8_t *w, typename F::Act act, float *y, int64_t n, int64_t k, int64_t row_bytes,
            hipStream_t s) {
    const int64_t rpp = 64 / G;
    const int64_t passes = (n + rpp - 1) / rpp;
    const size_t lds = (size_t)(k / 64) * F::ACT_STRIDE * 4;
    // occupancy depends on (device, LDS bytes) only: remember the last answer
    static thread_local int c_dev = -1;
    static thread_local size_t c_lds = 0;
    static thread_local int64_t c_target = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != c_dev || lds != c_lds) {
        c_target = resident_waves(k_dense<F, G, UPL>, lds, F::MAX_WG_PER_CU);
        c_dev = dev;
        c_lds = lds;
    }
    const int64_t target = c_target;
    const int64_t waves = passes < target ? passes : target;
    const dim3 grid((unsigned)((waves + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK));
    hipLaunchKernelGGL((k_dense<F, G, UPL>), grid, dim3(256), lds, s, w, act, y, (int)n, (int)k, (int)row_bytes);
}


// Dispatch on the lane-group size G (units per row rounded up to a power of
// two, at most 64) and units per lane (1 or 2). k % 64 == 0, k <= 8192.
template <class F>
void launch_tiled(const uint8_t *w, typename F::Act act, float *y, int64_t n, int64_t k, hipStream_t s) {
    const int64_t row_bytes = k / F::BW * F::BB;
    const int64_t U = k / 64;
    const int G = next_pow2_le64(U);
    switch (G) {
        case 1: launch<F, 1, 1>(w, act, y, n, k, row_bytes, s); break;
        case 2: launch<F, 2, 1>(w, act, y, n, k, row_bytes, s); break;
        case 4: launch<F, 4, 1>(w, act, y, n, k, row_bytes, s); break;
        case 8: launch<F, 8, 1>(w, act, y, n, k, row_bytes, s); break;
        case 16: launch<F, 16, 1>(w, act, y, n, k, row_bytes, s); break;
        case 32: launch<F, 32, 1>(w, act, y, n, k, row_bytes, s); break;
        default:
            if (U <= 64) launch<F, 64, 1>(w, act, y, n, k, row_bytes, s);
            else launch<F, 64, 2>(w, act, y, n, k, row_bytes, s);
    }
}

}  // namespace qmv_dense
