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
// Expert grouping: a work item (expert g, row block rb) covers the rows of
// the block of the g-th distinct expert present in ids (ascending expert id)
// for every slot routed to it, in slot order, so an expert's rows come from
// HBM once per call however many slots chose it (a second slot re-reads the
// block's rows from L2). Each workgroup copies ids into LDS once and derives
// the grouping there (a bitmap of present experts, their ordered list, and a
// ballot compaction of the slots of an item's expert); the workgroups then
// loop over the items, whose number is known only on the device.
//
// The activation row of a slot is staged through registers into a padded
// LDS layout (the dense kernels' layout), the weight loads of the block's
// first passes are issued before that staging, and each lane then keeps its
// unit's 64 activation values in registers while it streams rows.
//
// In the layer, gate and up are one gather over interleaved rows (gate row
// i, then up row i) so that one wave holds both dots of a row and writes
// h = silu(g) * u directly; the down pass is organised by token: workgroup
// (row block, token) streams the rows of the block for each routed expert
// and sums them with the routing weights itself, so no workgroup waits for
// another and no separate combine kernel runs.
#include <climits>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "blocks.hpp"
#include "internal.hpp"

namespace {

constexpr int MAX_E = 4096;
constexpr int MAX_SLOTS = 2048;
// a token's slots held by the down pass (its ids and weights live in LDS
// arrays of this size)
constexpr int MAX_LAYER_TOPK = 64;
constexpr int WAVES = 4;
constexpr int SMALL_E = 256;  // router: one workgroup per token up to this E
constexpr int ROUTE_FUSED_E = 256;  // routing fused into the gather up to this E
// and up to this many tokens: every workgroup routes every token, which
// beat a separate router launch at 1 and 4 tokens and lost at 16 (measured)
#ifndef QMV_ROUTE_FUSED_T
#define QMV_ROUTE_FUSED_T 8
#endif
constexpr int ROUTE_FUSED_T = QMV_ROUTE_FUSED_T;
// q8 decode layer: up to this many tokens the gathers quantize the rows they
// stage instead of separate quantizer launches (measured with the direct
// gathers: sixteen / twenty-four / thirty-two tokens 74.7 / 98.4 / 125.9 ->
// 72.3 / 95.2 / 123.4 us; at thirty-three the launches win, 164.2 against
// 173.0)
#ifndef QMV_Q8_STAGED_T
#define QMV_Q8_STAGED_T 32
#endif
constexpr int Q8_STAGED_T = QMV_Q8_STAGED_T;
// Row passes in flight per wave in the grouped gathers (k_moe): their row
// blocks are short (a few passes per wave), so every pass of a block is
// requested up front. The direct gathers choose theirs per launch.
constexpr int MOE_RING = 2;

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- router ---
// Sort key of (logit, expert): larger key = earlier in the top-k order.
// NaN ranks as -inf, -0 as +0, and equal logits put the lower expert first.
QMV_DEV uint64_t route_key(float v, int e) {
    v = (v != v) ? -INFINITY : v + 0.0f;
    const uint32_t b = __float_as_uint(v);
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e;
}

// E <= 256, one workgroup per token. An expert's rank is the number of keys
// above its own. With EP = next power of two >= E, the key list is cut into
// P = min(256/EP, EP) partitions of L = EP/P keys; thread (part, e) counts
// partition `part` for expert e, so each thread does at most EP*EP/256
// compares (64 at E = 128).
__global__ __launch_bounds__(256) void k_route_small(const float *__restrict__ logits,
                                                     int32_t *__restrict__ ids,
                                                     float *__restrict__ wts, int E, int EP,
                                                     int topk) {
    __shared__ uint64_t keys[SMALL_E];
    __shared__ int part_cnt[256];
    __shared__ float sel_v[64];
    __shared__ int sel_e[64];
    __shared__ float sel_p[64];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float *lg = logits + (size_t)t * E;
    float v = -INFINITY;
    if (tid < EP) {
        uint64_t key = 0;  // padding ranks below every real key
        if (tid < E) {
            v = lg[tid];
            key = route_key(v, tid);
        }
        keys[tid] = key;
    }
    __syncthreads();
    const int P = (256 / EP < EP) ? 256 / EP : EP, L = EP / P;
    const int e = tid % EP, part = tid / EP;
    int c = 0;
    if (part < P) {
        const uint64_t mine = keys[e];
        // 8 independent LDS reads in flight per step (L is a power of two)
        if (L >= 8) {
            for (int i = part * L; i < (part + 1) * L; i += 8) {
#pragma unroll
                for (int q = 0; q < 8; ++q) c += keys[i + q] > mine ? 1 : 0;
            }
        } else {
            for (int i = part * L; i < (part + 1) * L; ++i) c += keys[i] > mine ? 1 : 0;
        }
    }
    part_cnt[tid] = c;
    __syncthreads();
    if (tid < E) {
        int rank = 0;
        for (int p = 0; p < P; ++p) rank += part_cnt[p * EP + tid];
        if (rank < topk) {
            sel_v[rank] = (v != v) ? -INFINITY : v;
            sel_e[rank] = tid;
        }
    }
    __syncthreads();
    if (tid < topk) {
        const float lmax = sel_v[0];
        sel_p[tid] = (lmax == -INFINITY) ? 1.0f : expf(sel_v[tid] - lmax);
    }
    __syncthreads();
    if (tid < topk) {
        float den = 0.0f;
        for (int j = 0; j < topk; ++j) den += sel_p[j];
        ids[(size_t)t * topk + tid] = sel_e[tid];
        wts[(size_t)t * topk + tid] = sel_p[tid] / den;
    }
}

// Wave-wide maximum of an unsigned value through DPP row operations (the
// reduction pattern of group_sum_last: the result lands in lane 63, then a
// readlane makes it wave-uniform). 0 is the identity. Whole wave only.
template <int CTRL, int ROW_MASK>
QMV_DEV uint32_t dpp_max_u32(uint32_t v) {
    const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
    return v > t ? v : t;
}
QMV_DEV uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_u32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_u32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_u32<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_max_u32<0x140, 0xF>(v);  // row_mirror
    v = dpp_max_u32<0x142, 0xA>(v);  // row_bcast15 into rows 1, 3
    v = dpp_max_u32<0x143, 0xC>(v);  // row_bcast31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One token routed by one wave (E <= 64 * VPL): lane l holds the order keys
// (route_key's upper half: logit order, NaN as -inf, -0 as +0) of experts
// l + 64 v. Each of the topk rounds takes the wave maximum of the keys, then
// the lowest expert holding it (a maximum of the complemented index), and
// removes that key; lane j keeps the j-th pick. Lane j < topk returns the
// j-th expert and its renormalized weight. Call with the whole wave.
template <int VPL>
QMV_DEV void route_token_wave(const float *__restrict__ lg, int E, int topk, int lane, int *out_e, float *out_w) {
    uint32_t ord[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        ord[i] = e < E ? (uint32_t)(route_key(lg[e], e) >> 32) : 0u;  // padding below every key
    }
    uint32_t my_e = 0, my_ord = 0;
    for (int j = 0; j < topk; ++j) {
        uint32_t mo = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) mo = ord[i] > mo ? ord[i] : mo;
        const uint32_t M = wave_max_u32(mo);
        uint32_t c = 0;  // ~(lowest expert of this lane with key M)
#pragma unroll
        for (int i = VPL - 1; i >= 0; --i)
            if (ord[i] == M) c = ~(uint32_t)(lane + 64 * i);
        const uint32_t W = ~wave_max_u32(c);
        if ((int)(W & 63) == lane) {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if ((int)(W >> 6) == i) ord[i] = 0;
        }
        if (lane == j) {
            my_e = W;
            my_ord = M;
        }
    }
    // back from the order key to the logit
    const uint32_t bits = (my_ord & 0x80000000u) ? (my_ord & 0x7FFFFFFFu) : ~my_ord;
    const float my_v = __uint_as_float(bits);
    const float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    float p = 0.0f;
    if (lane < topk) p = (lmax == -INFINITY) ? 1.0f : expf(my_v - lmax);
    const float den = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum_last<64>(p)), 63));
    *out_e = (int)my_e;
    *out_w = p / den;
}

// Any E <= 4096: one wave per token.
template <int VPL>
__global__ __launch_bounds__(256) void k_route_wave(const float *__restrict__ logits,
                                                    int32_t *__restrict__ ids,
                                                    float *__restrict__ wts, int T, int E, int topk) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (t >= T) return;
    int e;
    float w;
    route_token_wave<VPL>(logits + (size_t)t * E, E, topk, lane, &e, &w);
    if (lane < topk) {
        ids[(size_t)t * topk + lane] = e;
        wts[(size_t)t * topk + lane] = w;
    }
}

// ------------------------------------------------------ gather matvec ---
struct MoeArgs {
    const uint8_t *bank;   // [E, n, k]; PAIR: the gate bank [E, n/2, k]
    const uint8_t *bank2;  // PAIR: the up bank [E, n/2, k]
    const float *x;        // f32 activation rows (units with F::Q8 false)
    const int8_t *xq;      // q8 activation rows (F::Q8): xq [rows, k], xs / xsum [rows, k/32]
    const float *xs, *xsum;
    int x_div;
    const int32_t *ids;
    float *y;  // [nslots, n]; PAIR: [nslots, n/2]
    int nslots, n, k, E;
    // fused routing (ids == nullptr; the direct gathers only): logits
    // [nslots / topk, E] are routed here (E <= ROUTE_FUSED_E); the item of a
    // slot's first row block writes its ids_out / wts_out
    const float *logits;
    int topk;
    int32_t *ids_out;
    float *wts_out;
};

// Dynamic LDS of k_moe: activation staging, ids (int16, -1 = out of
// range), slot list, present experts (uint16), per-expert slot counts and
// item offsets (int32).
size_t moe_lds_bytes(int k, int act_stride, int nslots, int E, int nsp) {
    const int64_t p = E < nslots ? E : nslots;  // present experts at most
    return (size_t)nsp * (k / 64) * act_stride * 4 + (size_t)div_up(nslots, 2) * 4 * 2 +
           (size_t)div_up(p, 2) * 4 + (size_t)(2 * p + 1) * 4;
}

// Slots of one item staged at once by k_moe (each in its own LDS region,
// one region of (k/64)*ACT_STRIDE floats per slot). int8 dots (q8
// activations, given or quantized in the staging): as many of 4, 2, 1 as
// fit 36 KB at the largest k of the lane mapping (G lanes of UPL units).
// f32 dots: one -- their gathers are bound by the vector
// ALU at many slots per expert (one FMA per weight and slot), and splitting
// the waves among slots halved the rows each workgroup kept in flight
// (128 experts, top-8, 16 tokens: 89.5 -> 94.8 us, while the q8 layer went
// 85.7 -> 82.9 us).
template <class F, int G, int UPL>
constexpr int moe_nsp() {
    constexpr int region = G * UPL * F::ACT_STRIDE * 4;
    constexpr bool f32_dots = std::is_same<typename F::X, UnitX>::value;
    return f32_dots ? 1 : (4 * region <= 36864 ? 4 : (2 * region <= 36864 ? 2 : 1));
}

// Units whose f32 activation rows are quantized while staged (F::QX).
template <class F, class = void>
struct moe_stage_qx : std::false_type {};
template <class F>
struct moe_stage_qx<F, std::void_t<decltype(F::QX)>> : std::bool_constant<F::QX> {};

// Persistent over work items: an item is a block of rows of one present
// expert, for every slot routed to that expert (in slot order):
// y[s, r] = W[e, r, :] . x[s / x_div]. An expert chosen by c slots gets
// row blocks about 1/c as tall as a single-slot expert's, so every item
// costs about the same. The slots of an item are taken NSP at a time (up to
// 4, see moe_nsp): each has its activation row staged in its own LDS region
// and its own share of the workgroup's four waves (4, 2 or 1 waves per
// slot), and all of them walk the block's rows in the same order at the
// same time, so a row read from HBM for one slot is still in the CU's
// caches when the others read it (one slot after another, a block's rows
// have left the L2 before the next slot comes back to them). The items
// (known only on the device) are dealt to the workgroups in turn.
// PAIR: virtual row 2i is gate row i and 2i+1 is up row i; a pass holds
// whole pairs (64/G even), and the lane group of the up row writes
// y[s, i] = silu(gate . x) * (up . x).
// The activation row `row` in the unit's form.
template <class F>
QMV_DEV typename F::Act moe_act(const MoeArgs &a, int row) {
    if constexpr (F::Q8) {
        const size_t kb = (size_t)(a.k / 32) * row;
        return ActQ8{a.xq + (size_t)row * a.k, a.xs + kb, a.xsum ? a.xsum + kb : nullptr};
    } else {
        return ActF32{a.x + (size_t)row * a.k};
    }
}

template <class F, int G, int UPL, bool PAIR>
__global__ __launch_bounds__(256) void k_moe(MoeArgs a) {
    constexpr int NSP = moe_nsp<F, G, UPL>();
    static_assert(WAVES == 4, "slot groups split four waves");
    extern __shared__ float4 dyn4[];
    float *xlds = reinterpret_cast<float *>(dyn4);
    const int xreg = (a.k / 64) * F::ACT_STRIDE;  // floats per staged slot
    const int ns2 = (a.nslots + 1) / 2 * 2;
    const int pmax = a.E < a.nslots ? a.E : a.nslots;
    int16_t *s_ids = reinterpret_cast<int16_t *>(xlds + NSP * xreg);
    uint16_t *slot_list = reinterpret_cast<uint16_t *>(s_ids + ns2);
    uint16_t *experts = slot_list + ns2;
    int *cnt = reinterpret_cast<int *>(experts + (pmax + 1) / 2 * 2);
    int *item0 = cnt + pmax;  // pmax + 1 entries
    __shared__ uint32_t bitmap[MAX_E / 32];
    __shared__ int wprefix[MAX_E / 32];  // present experts in lower words
    __shared__ int sh[4];                // present, invalid, slot count, items
    constexpr int NB = MOE_RING;
    constexpr int RPP = 64 / G;
    constexpr int STEP = WAVES * RPP;  // one pass per wave
    static_assert(!PAIR || RPP % 2 == 0, "pairs need an even number of rows per pass");
    using Raw = typename F::Raw;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ids -> LDS, bitmap of the present experts, count of invalid slots
    const int words = (a.E + 31) >> 5;
    for (int i = tid; i < words; i += 256) bitmap[i] = 0u;
    for (int i = tid; i < pmax; i += 256) cnt[i] = 0;
    if (tid == 0) sh[1] = 0;
    __syncthreads();
    for (int s = tid; s < a.nslots; s += 256) {
        const int e = a.ids[s];
        const bool ok = e >= 0 && e < a.E;
        s_ids[s] = (int16_t)(ok ? e : -1);
        if (ok) atomicOr(&bitmap[e >> 5], 1u << (e & 31));
        else atomicAdd(&sh[1], 1);
    }
    __syncthreads();
    if (wave == 0) {
        // present experts in ascending order (running popcount over words)
        int base = 0;
        for (int w0 = 0; w0 < words; w0 += 64) {
            const int wi = w0 + lane;
            uint32_t bits = wi < words ? bitmap[wi] : 0u;
            const int c = __popc(bits);
            int incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            int pos = base + incl - c;
            if (wi < words) wprefix[wi] = pos;
            while (bits) {
                experts[pos++] = (uint16_t)(wi * 32 + __ffs((int)bits) - 1);
                bits &= bits - 1;
            }
            base += __shfl(incl, 63);
        }
        if (lane == 0) sh[0] = base;
    }
    __syncthreads();
    const int present = sh[0], ninvalid = sh[1];
    // slots per present expert (its rank: present experts below it)
    for (int s = tid; s < a.nslots; s += 256) {
        const int e = s_ids[s];
        if (e >= 0) atomicAdd(&cnt[wprefix[e >> 5] + __popc(bitmap[e >> 5] & ((1u << (e & 31)) - 1u))], 1);
    }
    __syncthreads();
    // rows per item of a single-slot expert, so that the items about match
    // the workgroups: n * valid slots / grid, in whole passes
    const int nvalid = a.nslots - ninvalid;
    int base_rows = (int)(((int64_t)a.n * (nvalid > 0 ? nvalid : 1) + gridDim.x - 1) / gridDim.x);
    base_rows = (base_rows + STEP - 1) / STEP * STEP;
    auto rows_of = [&](int c) {  // rows per item of an expert with c slots
        int r = (base_rows + c - 1) / c;
        r = (r + STEP - 1) / STEP * STEP;
        return r < a.n ? r : (a.n + STEP - 1) / STEP * STEP;
    };
    if (wave == 0) {
        // item offsets: item0[g] = items of the experts below g
        int base = 0;
        for (int g0 = 0; g0 < present; g0 += 64) {
            const int g = g0 + lane;
            const int c = g < present ? (a.n + rows_of(cnt[g]) - 1) / rows_of(cnt[g]) : 0;
            int incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            if (g < present) item0[g] = base + incl - c;
            base += __shfl(incl, 63);
        }
        if (lane == 0) {
            item0[present] = base;
            sh[3] = base;
        }
    }
    __syncthreads();
    const int nitems = sh[3];
    if (!PAIR && ninvalid > 0) {
        // slots with an out-of-range id get zero rows (row ranges dealt out)
        const int chunk = (a.n + gridDim.x - 1) / gridDim.x;
        const int r0 = blockIdx.x * chunk, len = min(a.n, r0 + chunk) - r0;
        for (int i = tid; i < a.nslots * len; i += 256) {
            const int s = i / len, r = r0 + i % len;
            if (s_ids[s] < 0) a.y[(size_t)s * a.n + r] = 0.0f;
        }
    }

    const int U = F::units_per_row(a.k);
    const size_t row_bytes = (size_t)(a.k / F::BW) * F::BB;
    const int nrows_bank = PAIR ? a.n / 2 : a.n;  // rows per expert in a bank
    const int ny = PAIR ? a.n / 2 : a.n;          // output row length
    const int gl = lane & (G - 1), grow = lane / G;
    bool uv[UPL];
    int uu[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        uv[i] = gl + G * i < U;
        uu[i] = uv[i] ? gl + G * i : U - 1;
    }

    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        // the expert of the item: last g with item0[g] <= it
        int lo = 0, hi = present - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (item0[mid] <= it) lo = mid;
            else hi = mid - 1;
        }
        const int g = lo;
        const int expert = experts[g];
        const int rblk = rows_of(cnt[g]);
        const int r0 = (it - item0[g]) * rblk, len = min(a.n, r0 + rblk) - r0;
        __syncthreads();  // the previous item's slot list is no longer read
        if (wave == 0) {
            int c = 0;
            for (int s0 = 0; s0 < a.nslots; s0 += 64) {
                const int s = s0 + lane;
                const bool f = s < a.nslots && s_ids[s] == expert;
                const unsigned long long m = __ballot(f);
                if (f) slot_list[c + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)s;
                c += __popcll(m);
            }
            if (lane == 0) sh[2] = c;
        }
        __syncthreads();
        const int count = sh[2];
        const uint8_t *wb = a.bank + (size_t)expert * nrows_bank * row_bytes;
        const uint8_t *wb2 = PAIR ? a.bank2 + (size_t)expert * nrows_bank * row_bytes : wb;
        // passes of RPP rows inside the block
        const int bpasses = (len + RPP - 1) / RPP;

        for (int c0 = 0; c0 < count; c0 += NSP) {
            // this group of up to NSP slots: wps waves per slot; this wave
            // takes slot c0 + si, block passes q*wps + wo. Spare waves (a
            // group of 3 leaves one) run one clamped pass and store nothing.
            const int ns = min(NSP, count - c0);
            const int wsh = ns == 1 ? 2 : (ns == 2 ? 1 : 0);  // log2 of waves per slot
            const int wps = 1 << wsh;
            const int si = wave >> wsh, wo = wave & (wps - 1);
            const bool active = si < ns;
            const int slot = slot_list[c0 + (active ? si : 0)];
            const int pr = active ? (bpasses - wo + wps - 1) / wps : 0;
            const int p1 = pr > 1 ? pr : 1;
            auto load_pass = [&](Raw (&B)[UPL], int pass) {
                const int v = r0 + min((pass * wps + wo) * RPP + grow, len - 1);
                const uint8_t *row = PAIR ? ((v & 1) ? wb2 : wb) + (size_t)(v >> 1) * row_bytes
                                          : wb + (size_t)v * row_bytes;
#pragma unroll
                for (int i = 0; i < UPL; ++i) F::load(B[i], row, uu[i]);
            };
            // the group's activation rows, slot c0 + j into region j, loaded
            // before the weight ring and stored after it (one slot alone:
            // one row; a group: every region filled, with clamped slots, so
            // that the loads issue unconditionally)
            Raw R[NB][UPL];
            auto ring = [&]() {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    load_pass(R[j], min(j, p1 - 1));
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (NSP == 1 || ns == 1) {
                typename F::Stage S;
                F::template fetch<stage_granules(G, UPL)>(S, moe_act<F>(a, slot / a.x_div), a.k);
                ring();
                __syncthreads();  // the previous group's LDS reads are done
                F::template store<stage_granules(G, UPL)>(xlds, S, a.k);
            } else {
                typename F::Stage S[NSP];
#pragma unroll
                for (int j = 0; j < NSP; ++j) {
                    const int sj = slot_list[c0 + min(j, ns - 1)];
                    F::template fetch<stage_granules(G, UPL)>(S[j], moe_act<F>(a, sj / a.x_div), a.k);
                }
                ring();
                __syncthreads();  // the previous group's LDS reads are done
#pragma unroll
                for (int j = 0; j < NSP; ++j)
                    F::template store<stage_granules(G, UPL)>(xlds + j * xreg, S[j], a.k);
            }
            __syncthreads();
            typename F::X X[UPL];
#pragma unroll
            for (int i = 0; i < UPL; ++i) F::load_lds(X[i], xlds + (active ? si : 0) * xreg, uu[i]);
            float *yrow = a.y + (size_t)slot * ny;
            int pass = 0;
            do {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int ps = pass + j;
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
                    const int rr = (ps * wps + wo) * RPP + grow;
                    if (PAIR) {
                        const float gate = __shfl(acc, lane - G);  // the pair's gate row
                        if ((grow & 1) && gl == G - 1 && ps < pr && rr < len)
                            yrow[(r0 + rr) >> 1] = silu(gate) * acc;
                    } else if (gl == G - 1 && ps < pr && rr < len) {
                        yrow[r0 + rr] = acc;
                    }
                }
                pass += NB;
            } while (pass < p1);
        }
    }
}

// Small batches (up to direct_slots<F>() slots): an item is one slot and a
// block of rblk rows, with no grouping by expert. A workgroup reads its
// slot's expert (or routes the slot's token itself, each wave on its own:
// ids == nullptr) and issues its weight loads at once; the item of a slot's
// first block publishes the routed id and weight. An expert chosen by c
// slots is read c times (from the caches where the reads meet). At a few
// slots that costs less than the grouping's serial steps: ids, present
// experts, counts, item offsets and the slot list, each behind a barrier,
// all before the first weight load (about half of a workgroup's time at
// one token, 128 experts, top-8).
template <class F, int G, int UPL, bool PAIR, int NB>
__global__ __launch_bounds__(256) void k_moe_direct(MoeArgs a, int rblk) {
    extern __shared__ float4 dyn4[];
    float *xlds = reinterpret_cast<float *>(dyn4);
    constexpr int RPP = 64 / G;
    static_assert(!PAIR || RPP % 2 == 0, "pairs need an even number of rows per pass");
    using Raw = typename F::Raw;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int U = F::units_per_row(a.k);
    const size_t row_bytes = (size_t)(a.k / F::BW) * F::BB;
    const int nrows_bank = PAIR ? a.n / 2 : a.n;  // rows per expert in a bank
    const int ny = PAIR ? a.n / 2 : a.n;          // output row length
    const int gl = lane & (G - 1), grow = lane / G;
    bool uv[UPL];
    int uu[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        uv[i] = gl + G * i < U;
        uu[i] = uv[i] ? gl + G * i : U - 1;
    }
    const int nblk = (a.n + rblk - 1) / rblk;
    for (int it = blockIdx.x; it < a.nslots * nblk; it += gridDim.x) {
        const int slot = it / nblk, rb = it - slot * nblk;
        const int r0 = rb * rblk, len = min(a.n, r0 + rblk) - r0;
        int expert;
        if (a.logits) {
            const int t = slot / a.topk, j = slot - t * a.topk;
            int e;
            float w;
            route_token_wave<ROUTE_FUSED_E / 64>(a.logits + (size_t)t * a.E, a.E, a.topk, lane, &e, &w);
            expert = __builtin_amdgcn_readlane(e, j);
            if (rb == 0 && wave == 0 && lane == j) {
                a.ids_out[slot] = e;
                a.wts_out[slot] = w;
            }
        } else {
            expert = __builtin_amdgcn_readfirstlane(a.ids[slot]);
        }
        if (expert < 0 || expert >= a.E) {
            // an out-of-range id: zero rows (the pair form leaves h unwritten,
            // the down pass skips the slot)
            if (!PAIR)
                for (int r = tid; r < len; r += 256) a.y[(size_t)slot * ny + r0 + r] = 0.0f;
            continue;
        }
        const uint8_t *wb = a.bank + (size_t)expert * nrows_bank * row_bytes;
        const uint8_t *wb2 = PAIR ? a.bank2 + (size_t)expert * nrows_bank * row_bytes : wb;
        // this wave takes block passes q*WAVES + wave (spare waves run one
        // clamped pass and store nothing)
        const int bpasses = (len + RPP - 1) / RPP;
        const int pr = (bpasses - wave + WAVES - 1) / WAVES;
        const int p1 = pr > 1 ? pr : 1;
        auto load_pass = [&](Raw (&B)[UPL], int pass) {
            const int v = r0 + min((pass * WAVES + wave) * RPP + grow, len - 1);
            const uint8_t *row = PAIR ? ((v & 1) ? wb2 : wb) + (size_t)(v >> 1) * row_bytes
                                      : wb + (size_t)v * row_bytes;
#pragma unroll
            for (int i = 0; i < UPL; ++i) F::load(B[i], row, uu[i]);
        };
        // the activation row first (its wait must not drain the weight ring)
        typename F::Stage S;
        F::template fetch<stage_granules(G, UPL)>(S, moe_act<F>(a, slot / a.x_div), a.k);
        Raw R[NB][UPL];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            load_pass(R[j], min(j, p1 - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();  // the previous item's LDS reads are done
        F::template store<stage_granules(G, UPL)>(xlds, S, a.k);
        __syncthreads();
        typename F::X X[UPL];
#pragma unroll
        for (int i = 0; i < UPL; ++i) F::load_lds(X[i], xlds, uu[i]);
        float *yrow = a.y + (size_t)slot * ny;
        int pass = 0;
        do {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int ps = pass + j;
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
                const int rr = (ps * WAVES + wave) * RPP + grow;
                if (PAIR) {
                    const float gate = __shfl(acc, lane - G);  // the pair's gate row
                    if ((grow & 1) && gl == G - 1 && ps < pr && rr < len) yrow[(r0 + rr) >> 1] = silu(gate) * acc;
                } else if (gl == G - 1 && ps < pr && rr < len) {
                    yrow[r0 + rr] = acc;
                }
            }
            pass += NB;
        } while (pass < p1);
    }
}

// ------------------------------------------- down pass + weighted combine ---
// Workgroup (row block rb, token t):
//   y[t, r] = sum_j wts[t, j] * W_down[ids[t, j], r, :] . h[topk*t + j, :]
// for r in the block. The h rows of a chunk of the token's slots are staged
// into LDS; the (slot, pass) items of the chunk are dealt to the four waves
// in turn, each wave adds wts*dot into its own LDS row accumulator, and the
// four accumulators are summed in wave order at the end (the result does
// not depend on timing). Slots whose id is out of range contribute nothing.
struct DownArgs {
    const uint8_t *bank;  // Q6_K [E, n, k]
    const float *h;       // [T*topk, k] (units with F::Q8 false)
    const int8_t *hq;     // F::Q8: q8 h rows [T*topk, k], scales hs [T*topk, k/32]
    const float *hs;
    const int32_t *ids;
    const float *wts;
    float *y;  // [T, n]
    int n, k, E, topk, rblk, chunk;
};

template <class F, int G, int NB>
__global__ __launch_bounds__(256) void k_moe_down(DownArgs a) {
    extern __shared__ float4 dyn4[];
    float *hlds = reinterpret_cast<float *>(dyn4);  // chunk x (k/64) units
    float *acc_lds = hlds + (size_t)a.chunk * (a.k / 64) * F::ACT_STRIDE;  // [WAVES][rblk]
    constexpr int RPP = 64 / G;
    using Raw = typename F::Raw;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.y;
    const int r0 = blockIdx.x * a.rblk, r1 = min(a.n, r0 + a.rblk), len = r1 - r0;
    const int U = F::units_per_row(a.k);
    const int ust = (a.k / 64) * F::ACT_STRIDE;  // LDS floats per staged slot
    const size_t row_bytes = (size_t)(a.k / F::BW) * F::BB;
    const int gl = lane & (G - 1), grow = lane / G;
    const bool uv = gl < U;
    const int uu = uv ? gl : U - 1;
    const int bpasses = (len + RPP - 1) / RPP;
    // the token's experts (out of range -> -1) and weights
    __shared__ int s_e[MAX_LAYER_TOPK];
    __shared__ float s_w[MAX_LAYER_TOPK];
    // the ids and weights are requested first, then the f32 h rows of the
    // first chunk (they do not depend on the ids), so the two reads overlap
    // and the ids' wait does not include the h rows' (loads complete in
    // order); h is stored to LDS once the chunk's weight loads are in flight
    // (every load unconditional, at clamped in-range indices: a branch
    // around either would make the compiler wait for all of them at once)
    const int e_in = a.ids[(size_t)t * a.topk + min(tid, a.topk - 1)];
    const float w_in = a.wts[(size_t)t * a.topk + min(tid, a.topk - 1)];
    constexpr int HPRE = 6;  // float4 per thread held: the layer's chunk, 8 slots x 768 values
    const int k4 = a.k / 4;
    const int nch0 = min(a.chunk, a.topk);
    const bool hpre = !F::Q8 && nch0 * k4 <= HPRE * 256;
    f32x4 hv0[HPRE];
    if constexpr (!F::Q8) {
#pragma unroll
        for (int r = 0; r < HPRE; ++r) {
            const int i = tid + 256 * r;
            const int ic = min(i, nch0 * k4 - 1);
            const int j = ic / k4, c4 = ic - j * k4;
            hv0[r] = *reinterpret_cast<const f32x4 *>(a.h + ((size_t)t * a.topk + j) * a.k + 4 * c4);
        }
    }
    for (int i = tid; i < WAVES * a.rblk; i += 256) acc_lds[i] = 0.0f;
    if (tid < a.topk) {
        s_e[tid] = (e_in >= 0 && e_in < a.E) ? e_in : -1;
        s_w[tid] = w_in;
    }
    __syncthreads();

    // one chunk of the token's slots; the first is peeled off the loop, so
    // that its weight loads do not wait on registers the loop reloads
    auto chunk_pass = [&](int j0) {
        const int nch = min(a.chunk, a.topk - j0);
        const int nitems = nch * bpasses;
        // this wave's items: a contiguous run q = qbeg, qbeg + 1, ... (slot
        // j0 + q / bpasses, pass q % bpasses), so that consecutive items
        // mostly share a slot and its activation registers are filled once
        // per slot instead of once per item
        const int ipw = (nitems + WAVES - 1) / WAVES, qbeg = wave * ipw;
        const int pr = max(0, min(nitems - qbeg, ipw));
        const int p1 = pr > 1 ? pr : 1;
        auto load_item = [&](Raw &B, int qi) {
            const int q = min(qbeg + qi, nitems - 1);
            const int j = q / bpasses;
            const int rr = (q - j * bpasses) * RPP + grow;
            const int e = max(s_e[j0 + j], 0);
            const int r = r0 + min(rr, len - 1);
            F::load(B, a.bank + ((size_t)e * a.n + r) * row_bytes, uu);
        };
        Raw R[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            load_item(R[j], min(j, p1 - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();  // the previous chunk's LDS reads are done
        if constexpr (F::Q8) {
            // q8 rows: 16-value granules to their unit's run, each block's
            // scale to the two units that read it
            const int k16 = a.k / 16, k32 = a.k / 32;
            for (int i = tid; i < nch * k16; i += 256) {
                const int j = i / k16, gi = i - j * k16;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(a.hq + ((size_t)t * a.topk + j0 + j) * a.k + 16 * gi);
                int g;
                const int u = F::granule_unit(gi, &g);
                *reinterpret_cast<u32x4 *>(hlds + j * ust + F::ACT_STRIDE * u + 4 * g) = v;
            }
            for (int i = tid; i < nch * k32; i += 256) {
                const int j = i / k32, b = i - j * k32;
                const float sc = a.hs[((size_t)t * a.topk + j0 + j) * k32 + b];
                int g;
                const int u = F::block_unit(b, &g);
                hlds[j * ust + F::ACT_STRIDE * u + 16 + g] = sc;
                hlds[j * ust + F::ACT_STRIDE * (u + 1) + 16 + g] = sc;
            }
        } else if constexpr (moe_stage_qx<F>::value) {
            // f32 h rows quantized while staged (8 consecutive lanes hold one
            // 32-value block; nch * k4 is a multiple of 8, so every group of
            // 8 is wholly inside or wholly past the end, and the lanes past
            // it quantize clamped values and store nothing)
            const int n4 = nch * k4;
            if (j0 == 0 && hpre) {
#pragma unroll
                for (int r = 0; r < HPRE; ++r) {
                    if (256 * r < n4) {
                        const int i = tid + 256 * r, ic = min(i, n4 - 1);
                        const int j = ic / k4, c4 = ic - j * k4;
                        F::store_quantized(hlds + j * ust, hv0[r], c4, i < n4);
                    }
                }
            } else {
                for (int i0 = 0; i0 < n4; i0 += 256) {
                    const int i = i0 + tid, ic = min(i, n4 - 1);
                    const int j = ic / k4, c4 = ic - j * k4;
                    const f32x4 hv = *reinterpret_cast<const f32x4 *>(a.h + ((size_t)t * a.topk + j0 + j) * a.k + 4 * c4);
                    F::store_quantized(hlds + j * ust, hv, c4, i < n4);
                }
            }
        } else if (j0 == 0 && hpre) {
#pragma unroll
            for (int r = 0; r < HPRE; ++r) {
                const int i = tid + 256 * r;
                if (i < nch * k4) {
                    const int j = i / k4, c4 = i - j * k4;
                    int jj;
                    const int u = F::xslot(4 * c4, &jj);
                    *reinterpret_cast<f32x4 *>(hlds + j * ust + F::ACT_STRIDE * u + jj) = hv0[r];
                }
            }
        } else {
            for (int i = tid; i < nch * k4; i += 256) {
                const int j = i / k4, c4 = i - j * k4;
                const f32x4 hv = *reinterpret_cast<const f32x4 *>(a.h + ((size_t)t * a.topk + j0 + j) * a.k + 4 * c4);
                int jj;
                const int u = F::xslot(4 * c4, &jj);
                *reinterpret_cast<f32x4 *>(hlds + j * ust + F::ACT_STRIDE * u + jj) = hv;
            }
        }
        __syncthreads();
        int cur = -1;
        typename F::X X;
        int qi = 0;
        do {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int qs = qi + b;
                const int q = min(qbeg + qs, nitems - 1);
                const int j = q / bpasses;
                const int rr = (q - j * bpasses) * RPP + grow;
                if (j != cur) {  // wave-uniform
                    F::load_lds(X, hlds + j * ust, uu);
                    cur = j;
                }
                float d = F::dot(R[b], X, uu);
                d = uv ? d : 0.0f;
                __builtin_amdgcn_sched_barrier(0);
                load_item(R[b], min(qs + NB, p1 - 1));
                __builtin_amdgcn_sched_barrier(0);
                d = group_sum_last<G>(d);
                if (gl == G - 1 && qs < pr && rr < len && s_e[j0 + j] >= 0)
                    acc_lds[wave * a.rblk + rr] += s_w[j0 + j] * d;
            }
            qi += NB;
        } while (qi < p1);
    };
    chunk_pass(0);
    for (int j0 = a.chunk; j0 < a.topk; j0 += a.chunk) chunk_pass(j0);
    __syncthreads();
    for (int r = tid; r < len; r += 256) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += acc_lds[w * a.rblk + r];
        a.y[(size_t)t * a.n + r0 + r] = v;
    }
}

// --------------------------------------------------------------- launch ---
// Resident workgroups of a kernel on the device (one round).
template <class K>
int64_t resident_wgs(K kernel, size_t lds) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess || per_cu < 1)
        per_cu = 2;
    return (int64_t)per_cu * cus;
}

// Expected number of distinct experts among nslots ids spread over E.
double expected_present(int64_t nslots, int64_t E) {
    const double p = (double)E * (1.0 - std::pow(1.0 - 1.0 / (double)E, (double)nslots));
    return p < 1.0 ? 1.0 : p;
}

// Slots up to which the gathers take the direct form (k_moe_direct), by
// the dots' kind (128 experts, top-8, gate/up [768, 2048], down
// [2048, 768]): the f32 layer at 8 / 16 / 32 / 33 / 48 / 64 tokens takes
// 52.4 / 88.0 / 156.9 / 202.3 / 215.7 / 328.4 us with the grouping and
// 48.5 / 82.8 / 149.6 / 178.3 / 193.2 / 300.9 direct; the q8 layer at 33 /
// 48 tokens 164.5 / 212.7 grouped, 146.0 / 168.2 direct, but at 64 tokens
// (512 slots) 222.4 grouped against 230.1 direct.
#ifndef QMV_DIRECT_SLOTS_F32
#define QMV_DIRECT_SLOTS_F32 512
#endif
#ifndef QMV_DIRECT_SLOTS_Q8
#define QMV_DIRECT_SLOTS_Q8 384
#endif
template <class F>
constexpr int64_t direct_slots() {
    return std::is_same<typename F::X, UnitX>::value ? QMV_DIRECT_SLOTS_F32 : QMV_DIRECT_SLOTS_Q8;
}

// Row passes in flight per wave of the direct gathers (measured, 128
// experts, top-8, gate/up [768, 2048]): the f32 dots want a deeper ring at
// many slots (layer at 16 tokens 83.3 us with two passes, 79.4 with three;
// at 8 tokens 48.4 against 48.7, at one 17.3 against 18.0 with two), the
// int8 dots a shallower one (q8 layer at 4 / 8 / 16 tokens 30.6 / 47.2 /
// 76.8 us with two, 29.0 / 46.2 / 75.3 with one; 17.3 against 17.6 us at
// one token with two).
template <class F>
int direct_ring(int64_t nslots) {
    if constexpr (!std::is_same<typename F::X, UnitX>::value) return nslots >= 32 ? 1 : 2;  // int8 dots
    return nslots >= 96 ? 3 : 2;
}

template <class F, int G, int UPL, bool PAIR, int NB>
int launch_direct_nb(MoeArgs a, hipStream_t s) {
    const size_t lds = (size_t)(a.k / 64) * F::ACT_STRIDE * 4;
    static thread_local int64_t cache[2] = {-1, -1};  // lds, resident workgroups
    if (cache[0] != (int64_t)lds) {
        cache[1] = resident_wgs(k_moe_direct<F, G, UPL, PAIR, NB>, lds);
        cache[0] = (int64_t)lds;
    }
    // blocks of whole passes (one per wave and more), about one item per
    // resident workgroup
    const int64_t step = WAVES * (64 / G);
    int64_t rblk = div_up(div_up((int64_t)a.n * a.nslots, cache[1]), step) * step;
    if (rblk > a.n) rblk = div_up(a.n, step) * step;
    const int64_t items = a.nslots * div_up(a.n, rblk);
    const int64_t grid = items < cache[1] ? items : cache[1];
    hipLaunchKernelGGL((k_moe_direct<F, G, UPL, PAIR, NB>), dim3((unsigned)grid), dim3(256), lds, s, a, (int)rblk);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

template <class F, int G, int UPL, bool PAIR>
int launch_direct_t(MoeArgs a, hipStream_t s) {
    switch (direct_ring<F>(a.nslots)) {
        case 1: return launch_direct_nb<F, G, UPL, PAIR, 1>(a, s);
        case 3: return launch_direct_nb<F, G, UPL, PAIR, 3>(a, s);
        default: return launch_direct_nb<F, G, UPL, PAIR, 2>(a, s);
    }
}

template <class F, int G, int UPL, bool PAIR>
int launch_moe_t(MoeArgs a, hipStream_t s) {
    // the fused routing (logits instead of ids) runs in the direct form only
    if (a.nslots <= direct_slots<F>() || a.logits) return launch_direct_t<F, G, UPL, PAIR>(a, s);
    const size_t lds = moe_lds_bytes(a.k, F::ACT_STRIDE, a.nslots, a.E, moe_nsp<F, G, UPL>());
    static thread_local int64_t cache[2] = {-1, -1};  // lds, resident workgroups
    if (cache[0] != (int64_t)lds) {
        cache[1] = resident_wgs(k_moe<F, G, UPL, PAIR>, lds);
        cache[0] = (int64_t)lds;
    }
    // one round of resident workgroups, but no more than the items of the
    // expected number of present experts at one pass per wave could fill
    const int64_t step = WAVES * (64 / G);
    const double pe = expected_present(a.nslots, a.E);
    int64_t grid = cache[1];
    const int64_t most = (int64_t)(pe * (double)div_up(a.n, step)) + 1;
    if (grid > most) grid = most;
    hipLaunchKernelGGL((k_moe<F, G, UPL, PAIR>), dim3((unsigned)grid), dim3(256), lds, s, a);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

template <class F>
int launch_moe(MoeArgs a, hipStream_t s) {
    const int64_t U = a.k / 64;
    switch (next_pow2_le64(U)) {
        case 1: return launch_moe_t<F, 1, 1, false>(a, s);
        case 2: return launch_moe_t<F, 2, 1, false>(a, s);
        case 4: return launch_moe_t<F, 4, 1, false>(a, s);
        case 8: return launch_moe_t<F, 8, 1, false>(a, s);
        case 16: return launch_moe_t<F, 16, 1, false>(a, s);
        case 32: return launch_moe_t<F, 32, 1, false>(a, s);
        default:
            if (U <= 64) return launch_moe_t<F, 64, 1, false>(a, s);
            if (U <= 128) return launch_moe_t<F, 64, 2, false>(a, s);
            return QMV_EUNSUPPORTED;
    }
}

// gate/up of the layer: pairs need 64/G even, so G <= 32 (two units per
// lane above k = 2048)
template <class F>
int launch_gate_up(MoeArgs a, hipStream_t s) {
    const int64_t U = a.k / 64;
    switch (next_pow2_le64(U)) {
        case 1: return launch_moe_t<F, 1, 1, true>(a, s);
        case 2: return launch_moe_t<F, 2, 1, true>(a, s);
        case 4: return launch_moe_t<F, 4, 1, true>(a, s);
        case 8: return launch_moe_t<F, 8, 1, true>(a, s);
        case 16: return launch_moe_t<F, 16, 1, true>(a, s);
        case 32: return launch_moe_t<F, 32, 1, true>(a, s);
        default:
            if (U <= 64) return launch_moe_t<F, 32, 2, true>(a, s);
            return QMV_EUNSUPPORTED;
    }
}

// Row passes per slot of a down-pass workgroup at least (its rows are
// rblk = passes * RPP). A workgroup that quantizes its h rows while staging
// them (moe_stage_qx) repeats that work for every row block of its token, so
// it takes more rows: q8 layer at one token 18.28 -> 17.40 us with two
// passes (19.19 with four), at four tokens 33.04 -> 30.59 us with four.
template <class F>
int down_min_passes(int64_t T) {
    if constexpr (moe_stage_qx<F>::value) return T >= 4 ? 4 : 2;
    return 1;
}

// Slots staged at once by the down pass: as many as fit 48 KB of LDS, <= 8.
template <class F>
int down_chunk(int64_t k, int64_t topk) {
    const int64_t per = (k / 64) * F::ACT_STRIDE * 4;
    int64_t c = 49152 / per;
    if (c > 8) c = 8;
    if (c < 1) c = 1;
    return (int)(c < topk ? c : topk);
}

template <class F, int G, int NB>
int launch_down_nb(DownArgs a, int64_t T, hipStream_t s) {
    constexpr int RPP = 64 / G;
    const size_t lds0 = (size_t)a.chunk * (a.k / 64) * F::ACT_STRIDE * 4;
    static thread_local int64_t cache[2] = {-1, -1};
    if (cache[0] != (int64_t)lds0) {
        cache[1] = resident_wgs(k_moe_down<F, G, NB>, lds0 + WAVES * 64 * 4);
        cache[0] = (int64_t)lds0;
    }
    // rows per workgroup: within one round of resident workgroups, and
    // enough (slot, pass) items to keep the four waves busy
    // (at most 1024 rows: the row accumulators take WAVES*rblk floats of LDS)
    int rblk = RPP;
    while (rblk < a.n && rblk < 1024 &&
           (div_up(a.n, rblk) * T > cache[1] || (int64_t)a.topk * (rblk / RPP) < WAVES ||
            rblk / RPP < down_min_passes<F>(T)))
        rblk *= 2;
    a.rblk = rblk;
    const size_t lds = lds0 + (size_t)WAVES * a.rblk * 4;
    const dim3 grid((unsigned)div_up(a.n, a.rblk), (unsigned)T);
    hipLaunchKernelGGL((k_moe_down<F, G, NB>), grid, dim3(256), lds, s, a);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

// Row passes in flight per wave of the down pass: the unit's own depth, but
// one for the f32 dots at a single token (layer 17.34 -> 17.07 us; with one
// pass at 4 and 16 tokens 30.9 -> 32.2 and 79.2 -> 83.7 us, and the int8
// down at one token 17.4 -> 18.1 us).
template <class F, int G>
int launch_down_g(DownArgs a, int64_t T, hipStream_t s) {
    if constexpr (std::is_same<typename F::X, UnitX>::value && F::RING == 2) {
        if (T == 1) return launch_down_nb<F, G, 1>(a, T, s);
    }
    return launch_down_nb<F, G, F::RING>(a, T, s);
}

template <class F>
int launch_down(DownArgs a, int64_t T, hipStream_t s) {
    switch (next_pow2_le64(a.k / 64)) {
        case 4: return launch_down_g<F, 4>(a, T, s);
        case 8: return launch_down_g<F, 8>(a, T, s);
        case 16: return launch_down_g<F, 16>(a, T, s);
        case 32: return launch_down_g<F, 32>(a, T, s);
        case 64: return launch_down_g<F, 64>(a, T, s);
        default: return QMV_EUNSUPPORTED;  // k / 64 <= 64 (inter <= 4096) on this path
    }
}

MoeArgs gather_args(const void *bank, const void *bank2, const float *x, int64_t x_div, const int32_t *ids,
                    float *y, int64_t nslots, int64_t n, int64_t k, int64_t E) {
    MoeArgs a{};
    a.bank = static_cast<const uint8_t *>(bank);
    a.bank2 = static_cast<const uint8_t *>(bank2);
    a.x = x;
    a.x_div = (int)x_div;
    a.ids = ids;
    a.y = y;
    a.nslots = (int)nslots;
    a.n = (int)n;
    a.k = (int)k;
    a.E = (int)E;
    return a;
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

// Every check of the f32 decode layer (moe_ffn_q4k_q6k and the routed
// forms), so that an entry point that launches several kernels can run all
// of them before the first launch.
int qmv_internal::check_decode_layer(const void *gate, const void *up, const void *down, const float *x,
                                     const int32_t *ids, const float *wts, const float *y, const void *ws,
                                     int64_t ws_bytes, int64_t T, int64_t topk, int64_t hidden, int64_t inter,
                                     int64_t E) {
    if (!gate || !up || !down || !x || !ids || !wts || !y || !ws) return QMV_EINVAL;
    if (T < 1 || topk < 1 || hidden < 256 || inter < 256 || hidden % 256 || inter % 256) return QMV_EINVAL;
    if (ws_bytes < moe_ffn_workspace_bytes(T, topk, hidden, inter)) return QMV_EINVAL;
    const int64_t ns = T * topk;
    float *yw = const_cast<float *>(y);
    int rc = check_moe_args(gate, x, topk, ids, yw, ns, 2 * inter, hidden, E);
    if (rc) return rc;
    rc = check_moe_args(down, x, 1, ids, yw, ns, hidden, inter, E);
    if (rc) return rc;
    if (topk > MAX_LAYER_TOPK || hidden > 4096 || inter > 4096 || T > 65535) return QMV_EUNSUPPORTED;
    if (!aligned(up, 16) || !aligned(wts, 4) || !aligned(ws, 16)) return QMV_EALIGN;
    return QMV_OK;
}

int qmv_internal::moe_layer_q8x_f32h(const void *gate, const void *up, const void *down, const int8_t *xq,
                                     const float *xs, const float *xsum, const int32_t *ids, const float *wts,
                                     float *y, float *h, int64_t T, int64_t topk, int64_t hidden, int64_t inter,
                                     int64_t E, hipStream_t s) {
    const int64_t ns = T * topk;
    if (topk > MAX_LAYER_TOPK || ns > MAX_SLOTS || E > MAX_E || hidden > 4096 || inter > 4096 || T > 65535)
        return QMV_EUNSUPPORTED;
    if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(down, 16)) return QMV_EALIGN;
    MoeArgs gu = gather_args(gate, up, nullptr, topk, ids, h, ns, 2 * inter, hidden, E);
    gu.xq = xq;
    gu.xs = xs;
    gu.xsum = xsum;
    int rc = launch_gate_up<Q4KQ8Unit>(gu, s);
    if (rc) return rc;
    DownArgs dn{};
    dn.bank = static_cast<const uint8_t *>(down);
    dn.h = h;
    dn.ids = ids;
    dn.wts = wts;
    dn.y = y;
    dn.n = (int)hidden;
    dn.k = (int)inter;
    dn.E = (int)E;
    dn.topk = (int)topk;
    dn.chunk = down_chunk<Q6KUnit>(inter, topk);
    return launch_down<Q6KUnit>(dn, T, s);
}

extern "C" int moe_route(const float *logits, int32_t *ids, float *wts, int64_t T, int64_t E,
                         int64_t topk, qmv_stream_t stream) {
    if (!logits || !ids || !wts || T < 1 || E < 1 || topk < 1 || topk > E || topk > 64) return QMV_EINVAL;
    if (E > MAX_E || T > (1 << 28)) return QMV_EUNSUPPORTED;
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(wts, 4)) return QMV_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (E <= SMALL_E) {
        int ep = 1;
        while (ep < E) ep <<= 1;
        hipLaunchKernelGGL(k_route_small, dim3((unsigned)T), dim3(256), 0, s, logits, ids, wts, (int)E, ep,
                           (int)topk);
        QMV_LAUNCH_CHECK();
        return QMV_OK;
    }
    const dim3 grid((unsigned)div_up(T, WAVES));
    const int vpl = (int)div_up(E, 64);
#define RT(V) hipLaunchKernelGGL((k_route_wave<V>), grid, dim3(256), 0, s, logits, ids, wts, (int)T, (int)E, (int)topk)
    if (vpl <= 8) RT(8);
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
    return launch_moe<Q4KUnit>(gather_args(bank, nullptr, x, x_div, ids, y, nslots, n, k, E), (hipStream_t)stream);
}

extern "C" int moe_qmv_q6k(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                           int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream) {
    const int rc = check_moe_args(bank, x, x_div, ids, y, nslots, n, k, E);
    if (rc) return rc;
    return launch_moe<Q6KUnit>(gather_args(bank, nullptr, x, x_div, ids, y, nslots, n, k, E), (hipStream_t)stream);
}

// workspace: h f32[T*topk, inter]
extern "C" int moe_qmv_q8_0(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                            int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream) {
    const int rc = check_moe_args(bank, x, x_div, ids, y, nslots, n, k, E);
    if (rc) return rc;
    return launch_moe<Q8Unit>(gather_args(bank, nullptr, x, x_div, ids, y, nslots, n, k, E), (hipStream_t)stream);
}

extern "C" int64_t moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t hidden, int64_t inter) {
    if (T < 1 || topk < 1 || hidden < 1 || inter < 1) return -1;
    return div_up(T * topk * inter * 4, 256) * 256;
}

static int launch_decode_layer(const void *gate, const void *up, const void *down, const float *x,
                               const int32_t *ids, const float *wts, float *y, float *h, int64_t T, int64_t topk,
                               int64_t hidden, int64_t inter, int64_t E, hipStream_t s);

extern "C" int moe_ffn_q4k_q6k(const void *gate, const void *up, const void *down, const float *x,
                               const int32_t *ids, const float *wts, float *y, void *ws, int64_t ws_bytes,
                               int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E,
                               qmv_stream_t stream) {
    const int rc = qmv_internal::check_decode_layer(gate, up, down, x, ids, wts, y, ws, ws_bytes, T, topk, hidden,
                                                    inter, E);
    if (rc) return rc;
    return launch_decode_layer(gate, up, down, x, ids, wts, y, static_cast<float *>(ws), T, topk, hidden, inter, E,
                               (hipStream_t)stream);
}

// The decode layer's two launches (all checks done by the caller); h holds
// T*topk*inter floats of scratch.
static int launch_decode_layer(const void *gate, const void *up, const void *down, const float *x,
                               const int32_t *ids, const float *wts, float *y, float *h, int64_t T, int64_t topk,
                               int64_t hidden, int64_t inter, int64_t E, hipStream_t s) {
    const int64_t ns = T * topk;
    // h = silu(gate x) * (up x): one gather over interleaved gate/up rows
    int rc = launch_gate_up<Q4KUnit>(gather_args(gate, up, x, topk, ids, h, ns, 2 * inter, hidden, E), s);
    if (rc) return rc;
    DownArgs dn{};
    dn.bank = static_cast<const uint8_t *>(down);
    dn.h = h;
    dn.ids = ids;
    dn.wts = wts;
    dn.y = y;
    dn.n = (int)hidden;
    dn.k = (int)inter;
    dn.E = (int)E;
    dn.topk = (int)topk;
    dn.chunk = down_chunk<Q6KUnit>(inter, topk);
    return launch_down<Q6KUnit>(dn, T, s);
}

// ------------------------------------------------ allocation-free layer ---
// The decode layer for callers that cannot allocate device memory (graph
// capture, tight serving loops): h lives in `scratch`, a library array of
// QMV_NOALLOC_SCRATCH_BYTES that each GPU holds from the first call on it
// until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and only that address is used. Every call on a GPU shares
// its array, so calls that overlap on one GPU race; nothing in it needs to
// start at zero (the gate/up pass writes every h row the down pass reads).
static __device__ __align__(256) float scratch[QMV_NOALLOC_SCRATCH_BYTES / 4];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[NOALLOC_MAX_DEVICES];

// Device address of `scratch` on the current device (looked up on first use).
int scratch_address(float **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        (void)hipGetLastError();
        return QMV_ELAUNCH;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return QMV_ELAUNCH;
        }
        g_scratch_addr[dev] = p;
    }
    *out = static_cast<float *>(g_scratch_addr[dev]);
    return QMV_OK;
}
}  // namespace

extern "C" int moe_ffn_q4k_q6k_noalloc(const void *gate, const void *up, const void *down, const float *x,
                                       const int32_t *ids, const float *wts, float *y, int64_t T, int64_t topk,
                                       int64_t hidden, int64_t inter, int64_t E, qmv_stream_t stream) {
    // every check of moe_ffn_q4k_q6k except the workspace's (the placeholder
    // is never dereferenced), then the scratch limit
    const void *no_ws = reinterpret_cast<const void *>((uintptr_t)256);
    int rc = qmv_internal::check_decode_layer(gate, up, down, x, ids, wts, y, no_ws, INT64_MAX, T, topk, hidden,
                                              inter, E);
    if (rc) return rc;
    if (moe_ffn_workspace_bytes(T, topk, hidden, inter) > (int64_t)QMV_NOALLOC_SCRATCH_BYTES)
        return QMV_EUNSUPPORTED;
    float *h = nullptr;
    rc = scratch_address(&h);
    if (rc) return rc;
    return launch_decode_layer(gate, up, down, x, ids, wts, y, h, T, topk, hidden, inter, E, (hipStream_t)stream);
}

// The layer with the router fused into the gate/up gather: every workgroup
// of the gather routes the logits itself (softmax + top-k + renormalize,
// the moe_route semantics, one wave per token) before it groups the slots by
// expert, and workgroup 0 writes ids and wts for the down pass and the
// caller. Above ROUTE_FUSED_E experts or ROUTE_FUSED_T tokens the router
// runs as its own kernel first.
extern "C" int moe_ffn_routed_q4k_q6k(const void *gate, const void *up, const void *down, const float *x,
                                      const float *logits, int32_t *ids, float *wts, float *y, void *ws,
                                      int64_t ws_bytes, int64_t T, int64_t topk, int64_t hidden, int64_t inter,
                                      int64_t E, qmv_stream_t stream) {
    if (!logits || topk > E || topk > 64) return QMV_EINVAL;
    if (!aligned(logits, 4)) return QMV_EALIGN;
    int rc = qmv_internal::check_decode_layer(gate, up, down, x, ids, wts, y, ws, ws_bytes, T, topk, hidden,
                                              inter, E);
    if (rc) return rc;
    if (E > ROUTE_FUSED_E || T > ROUTE_FUSED_T) {
        rc = moe_route(logits, ids, wts, T, E, topk, stream);
        if (rc) return rc;
        return moe_ffn_q4k_q6k(gate, up, down, x, ids, wts, y, ws, ws_bytes, T, topk, hidden, inter, E, stream);
    }
    const int64_t ns = T * topk;
    float *h = static_cast<float *>(ws);
    hipStream_t s = (hipStream_t)stream;
    MoeArgs gu = gather_args(gate, up, x, topk, nullptr, h, ns, 2 * inter, hidden, E);
    gu.logits = logits;
    gu.topk = (int)topk;
    gu.ids_out = ids;
    gu.wts_out = wts;
    rc = launch_gate_up<Q4KUnit>(gu, s);
    if (rc) return rc;
    DownArgs dn{};
    dn.bank = static_cast<const uint8_t *>(down);
    dn.h = h;
    dn.ids = ids;
    dn.wts = wts;
    dn.y = y;
    dn.n = (int)hidden;
    dn.k = (int)inter;
    dn.E = (int)E;
    dn.topk = (int)topk;
    dn.chunk = down_chunk<Q6KUnit>(inter, topk);
    return launch_down<Q6KUnit>(dn, T, s);
}

// ------------------------------------------------- q8-activation variants ---
// The gathers and the layer with int8 dot products: activations quantized
// to q8 once (quantize_act_q8), Q4_K codes against xq through v_dot4
// (Q4KQ8Unit), Q6_K codes as signed q - 32 bytes against xq (Q6KQ8Unit).
extern "C" int moe_qmv_q4k_q8(const void *bank, const int8_t *xq, const float *xs, const float *xsum, int64_t x_div,
                              const int32_t *ids, float *y, int64_t nslots, int64_t n, int64_t k, int64_t E,
                              qmv_stream_t stream) {
    if (!xs || !xsum) return QMV_EINVAL;
    const int rc = check_moe_args(bank, reinterpret_cast<const float *>(xq), x_div, ids, y, nslots, n, k, E);
    if (rc) return rc;
    if (!aligned(xs, 4) || !aligned(xsum, 4)) return QMV_EALIGN;
    MoeArgs a = gather_args(bank, nullptr, nullptr, x_div, ids, y, nslots, n, k, E);
    a.xq = xq;
    a.xs = xs;
    a.xsum = xsum;
    return launch_moe<Q4KQ8Unit>(a, (hipStream_t)stream);
}

extern "C" int moe_qmv_q6k_q8(const void *bank, const int8_t *xq, const float *xs, int64_t x_div, const int32_t *ids,
                              float *y, int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream) {
    if (!xs) return QMV_EINVAL;
    const int rc = check_moe_args(bank, reinterpret_cast<const float *>(xq), x_div, ids, y, nslots, n, k, E);
    if (rc) return rc;
    if (!aligned(xs, 4)) return QMV_EALIGN;
    MoeArgs a = gather_args(bank, nullptr, nullptr, x_div, ids, y, nslots, n, k, E);
    a.xq = xq;
    a.xs = xs;
    return launch_moe<Q6KQ8Unit>(a, (hipStream_t)stream);
}

namespace {
struct Q8LayerWs {
    int8_t *xq, *hq;
    float *xs, *xsum, *h, *hs, *hsum;
    int64_t bytes;
};

Q8LayerWs q8_layer_ws(uint8_t *base, int64_t T, int64_t topk, int64_t hidden, int64_t inter) {
    const int64_t S = T * topk;
    Q8LayerWs w{};
    int64_t o = 0;
    auto take = [&](int64_t nbytes) {
        uint8_t *p = base ? base + o : nullptr;
        o += div_up(nbytes, 256) * 256;
        return p;
    };
    w.xq = reinterpret_cast<int8_t *>(take(T * hidden));
    w.xs = reinterpret_cast<float *>(take(4 * T * (hidden / 32)));
    w.xsum = reinterpret_cast<float *>(take(4 * T * (hidden / 32)));
    w.h = reinterpret_cast<float *>(take(4 * S * inter));
    w.hq = reinterpret_cast<int8_t *>(take(S * inter));
    w.hs = reinterpret_cast<float *>(take(4 * S * (inter / 32)));
    w.hsum = reinterpret_cast<float *>(take(4 * S * (inter / 32)));
    w.bytes = o;
    return w;
}
}  // namespace

extern "C" int64_t moe_ffn_q8_workspace_bytes(int64_t T, int64_t topk, int64_t hidden, int64_t inter) {
    if (T < 1 || topk < 1 || hidden < 1 || inter < 1) return -1;
    return q8_layer_ws(nullptr, T, topk, hidden, inter).bytes;
}

extern "C" int moe_ffn_q4k_q6k_q8(const void *gate, const void *up, const void *down, const float *x,
                                  const int32_t *ids, const float *wts, float *y, void *ws, int64_t ws_bytes,
                                  int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E,
                                  qmv_stream_t stream) {
    if (!gate || !up || !down || !x || !ids || !wts || !y || !ws) return QMV_EINVAL;
    if (T < 1 || topk < 1 || hidden < 256 || inter < 256 || hidden % 256 || inter % 256) return QMV_EINVAL;
    if (ws_bytes < moe_ffn_q8_workspace_bytes(T, topk, hidden, inter)) return QMV_EINVAL;
    const int64_t ns = T * topk;
    int rc = check_moe_args(gate, x, topk, ids, y, ns, 2 * inter, hidden, E);
    if (rc) return rc;
    rc = check_moe_args(down, x, 1, ids, y, ns, hidden, inter, E);
    if (rc) return rc;
    if (topk > MAX_LAYER_TOPK || hidden > 4096 || inter > 4096 || T > 65535) return QMV_EUNSUPPORTED;
    if (!aligned(up, 16) || !aligned(wts, 4) || !aligned(ws, 256)) return QMV_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    const Q8LayerWs w = q8_layer_ws(static_cast<uint8_t *>(ws), T, topk, hidden, inter);
    DownArgs dn{};
    dn.bank = static_cast<const uint8_t *>(down);
    dn.ids = ids;
    dn.wts = wts;
    dn.y = y;
    dn.n = (int)hidden;
    dn.k = (int)inter;
    dn.E = (int)E;
    dn.topk = (int)topk;
    if (T <= Q8_STAGED_T) {
        // h = silu(gate x) * (up x) on int8 dots, x quantized as each
        // workgroup stages it; down on int8 dots + combine, h quantized as it
        // is staged (the steps of quantize_act_q8: the same codes as the two
        // quantizer launches below, which at a few tokens cost more than the
        // repeated quantization: 23.2 -> 21.3 us at one token)
        rc = launch_gate_up<Q4KQ8XUnit>(gather_args(gate, up, x, topk, ids, w.h, ns, 2 * inter, hidden, E), s);
        if (rc) return rc;
        dn.h = w.h;
        dn.chunk = down_chunk<Q6KQ8XUnit>(inter, topk);
        return launch_down<Q6KQ8XUnit>(dn, T, s);
    }
    // x -> q8 once; h = silu(gate x) * (up x) on int8 dots; h -> q8; down on
    // int8 dots + combine
    rc = quantize_act_q8(x, w.xq, w.xs, w.xsum, T, hidden, stream);
    if (rc) return rc;
    MoeArgs gu = gather_args(gate, up, nullptr, topk, ids, w.h, ns, 2 * inter, hidden, E);
    gu.xq = w.xq;
    gu.xs = w.xs;
    gu.xsum = w.xsum;
    rc = launch_gate_up<Q4KQ8Unit>(gu, s);
    if (rc) return rc;
    rc = quantize_act_q8(w.h, w.hq, w.hs, w.hsum, ns, inter, stream);
    if (rc) return rc;
    dn.hq = w.hq;
    dn.hs = w.hs;
    dn.chunk = down_chunk<Q6KQ8Unit>(inter, topk);
    return launch_down<Q6KQ8Unit>(dn, T, s);
}

