// Q4_K x q8-activation prefill GEMM on gfx950 matrix cores.
//
// hanzo-ml `src/vulkan_backend.rs`, `mmq_q4k_rt_gpu` / `mmq_q4k_gpu`: affine
// Q4_K weights decoded in-kernel, activation quantized to (xq, xs, xsum),
// epilogue xs*(D*dot - M*xsum) per 32-value block; `mul_mm_q4k_tiled_dp4a`:
// BM rows of the output per workgroup so cold weights are re-read m/BM times.
//
//   Y[i, r] = sum_s d[r,s] * sum_{b in s} xs[i,b] * T[i,r,b]
//           - sum_b xsum[i,b] * dmin[r,s(b)] * m[r,b]
//   T[i,r,b] = sum_{l<32} xq[i,32b+l] * (sc[r,b] * q[r,32b+l])   (an integer)
//
// T is formed on the f16 matrix cores (v_mfma_f32_16x16x32_f16), and it is
// exact there: xq (|xq| <= 127) and sc*q (<= 63*15) are integers that f16
// holds exactly, every product fits the f32 accumulator, and a sum of 32 of
// them stays below 2^24. So one MFMA per 16x16 tile and q8 block gives the
// block's integer dot with the weight's sub-block scale already folded in,
// and the VALU only adds xs*T into a per-superblock accumulator (one FMA per
// output and block) and d times that accumulator once per superblock. The
// min term is a rank-8 f32 product per superblock on v_mfma_f32_16x16x4_f32,
// accumulated straight into the output tile.
//
// Workgroup: 512 threads (8 waves), output tile BM x BN, each wave MT x NT
// 16x16 tiles. K advances by phases of KP through double-buffered LDS: after
// a phase's matrix instructions are issued, the waves convert the next
// phase's codes into the other buffer, so conversion and matrix work
// overlap; the raw codes are loaded into registers two phases before they
// are converted (two register sets), and the per-superblock scales are
// double-buffered by superblock parity.
//  - activation codes: int8 -> f16 through the 1024 + b half bit pattern
//    (v_perm_b32 + v_pk_add_f16, exact);
//  - weight codes: nibbles -> f16 the same way, then times sc with one
//    v_pk_fma_f16 ((1024 + q) * sc - 1024 * sc is exact after the fused
//    rounding because q * sc is);
//  - LDS rows are padded by 8 halves (a 4-bank shift per row) so that the
//    16-byte fragment reads of eight consecutive rows hit distinct banks;
//    the staging writes go eight lanes to eight consecutive 16-byte units
//    of a row (activations) or to one unit of eight rows (weights, xs), so
//    they are conflict-free too.
#include <algorithm>
#include <type_traits>

#include "blocks.hpp"
#include "internal.hpp"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));


// bytes (0, 1) / (2, 3) of w as the low bytes of two halves 0x64bb
QMV_DEV uint32_t half_bytes_lo(uint32_t w) { return __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u); }
QMV_DEV uint32_t half_bytes_hi(uint32_t w) { return __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u); }
QMV_DEV h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
QMV_DEV uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Four int8 codes (one dword) -> four f16 values, exact:
// byte b ^ 0x80 = b + 128 -> half 1024 + 128 + b -> minus 1152.
QMV_DEV uint2 i8x4_to_f16(uint32_t a) {
    const h2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    a ^= 0x80808080u;
    return make_uint2(as_u32(as_h2(half_bytes_lo(a)) + off), as_u32(as_h2(half_bytes_hi(a)) + off));
}

// Four 4-bit codes (one per byte) -> four f16 values sc * q, exact.
QMV_DEV uint2 q4x4_to_f16(uint32_t c, h2 sc, h2 nsc) {
    return make_uint2(as_u32(__builtin_elementwise_fma(as_h2(half_bytes_lo(c)), sc, nsc)),
                      as_u32(__builtin_elementwise_fma(as_h2(half_bytes_hi(c)), sc, nsc)));
}

QMV_DEV h2 splat(float v) { return h2{(_Float16)v, (_Float16)v}; }

struct QmmArgs {
    const uint8_t *w;     // dense weight [n, k/256] blocks, or the expert bank [E, n, k/256]
    const int8_t *xq;     // q8 activation rows
    const float *xs, *xsum;
    float *Y;
    int m, n, k;          // dense: m activation rows; expert-indexed: m slots
    const int32_t *ids;   // expert-indexed only: expert of each slot
    int E, x_div;         // expert-indexed only: slot s reads activation row s / x_div
    // tile table (expert-indexed, built once per layer by k_group_tiles):
    // tile i is expert tile_e[i] on slots tile_slots[BM*i .. BM*i + BM) (-1: none)
    const int *ntiles, *tile_e, *tile_slots;
    const uint8_t *w2;    // PAIR: the up bank (w is the gate bank); Y is then h [nslots, n]
};

constexpr int QMM_ID_CHUNK = 4096;  // slot ids staged in LDS at a time (grouping)
constexpr int QMM_MOE_MAX_E = 1024;

// Expert-indexed tiles. The tile of workgroup row block blockIdx.y is row
// block r0 / BM of the esel-th expert's slots (experts in ascending order,
// each expert's slots in ascending slot order). Every workgroup derives it
// from ids itself: per-expert counts (LDS atomics over ids staged in chunks),
// a wave prefix of the per-expert tile counts, then a ballot compaction of
// its expert's slots into s_slot (-1 past the expert's count). Returns esel,
// or -1 for a workgroup past the last tile: the grid has more row blocks
// than tiles (each present expert adds less than one tile to nslots / BM),
// and those spare workgroups write the zero rows (columns [n0, n0 + ncols)) of
// slots whose expert is outside [0, E), spare j taking slots
// [j*chunk, (j+1)*chunk). s_ids (QMM_ID_CHUNK ints) and s_cnt (E ints) are
// LDS scratch that the caller reuses afterwards; the function ends with a
// barrier. Call from every thread of the workgroup.
template <int BM, int BN, int NTHREADS>
QMV_DEV int qmm_group(const int32_t *__restrict__ ids, int m, int E, int *s_ids, int *s_cnt, int *s_slot,
                      float *__restrict__ Y, int n, int n0, int ncols = BN) {
    constexpr int IPT = QMM_ID_CHUNK / NTHREADS;  // ids per thread per chunk
    constexpr int NW = NTHREADS / 64;
    __shared__ int s_wsum[NW];
    __shared__ int s_sel[3];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto stage_ids = [&](int c0) {  // ids[c0, c0 + QMM_ID_CHUNK) -> s_ids (-1 past the end)
        int v[IPT];
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int sl = c0 + tid + NTHREADS * i;
            v[i] = sl < m ? ids[sl] : -1;
        }
#pragma unroll
        for (int i = 0; i < IPT; ++i) s_ids[tid + NTHREADS * i] = v[i];
    };
    for (int e = tid; e < E; e += NTHREADS) s_cnt[e] = 0;
    for (int i = tid; i < BM; i += NTHREADS) s_slot[i] = -1;
    for (int c0 = 0; c0 < m; c0 += QMM_ID_CHUNK) {
        __syncthreads();  // counts zeroed / previous chunk counted
        stage_ids(c0);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int e = s_ids[tid + NTHREADS * i];
            if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
        }
    }
    __syncthreads();
    if (wave == 0) {
        // lane l owns experts [l*EPL, l*EPL + EPL): tile counts, then an
        // inclusive prefix over the lanes
        constexpr int EPL = QMM_MOE_MAX_E / 64;
        int tl = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            if (e < E) tl += (s_cnt[e] + BM - 1) / BM;
        }
        int inc = tl;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(inc, d);
            if (lane >= d) inc += v;
        }
        const int tile = blockIdx.y;
        int t = inc - tl;
        if (tile >= t && tile < inc) {
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                const int nt = e < E ? (s_cnt[e] + BM - 1) / BM : 0;
                if (tile < t + nt) {
                    s_sel[0] = e;
                    s_sel[1] = (tile - t) * BM;
                    break;
                }
                t += nt;
            }
        }
        if (lane == 63) {
            if (tile >= inc) s_sel[0] = -1;
            s_sel[2] = inc;  // tiles in all
        }
    }
    __syncthreads();
    const int esel = s_sel[0];
    if (esel < 0) {
        const int ntot = s_sel[2], nspare = (int)gridDim.y - ntot, j = (int)blockIdx.y - ntot;
        const int chunk = (m + nspare - 1) / nspare;
        const int s0 = j * chunk, s1 = min(m, s0 + chunk);
        for (int sl = s0 + tid; sl < s1; sl += NTHREADS) {
            const int e = ids[sl];
            if (e < 0 || e >= E)
                for (int c = n0; c < min(n0 + ncols, n); ++c) Y[(size_t)sl * n + c] = 0.0f;
        }
        return -1;
    }
    const int r0 = s_sel[1];
    // ascending compaction: per chunk, wave w takes ids [w*CW, (w+1)*CW) in
    // order; a rank is the running count plus the earlier waves' counts plus
    // the ballot prefix
    constexpr int CW = QMM_ID_CHUNK / NW;
    int run = 0;
    for (int c0 = 0; c0 < m; c0 += QMM_ID_CHUNK) {
        __syncthreads();  // previous chunk's readers done
        stage_ids(c0);
        __syncthreads();
        int cw = 0;
        for (int b = 0; b < CW; b += 64) cw += __popcll(__ballot(s_ids[wave * CW + b + lane] == esel));
        if (lane == 0) s_wsum[wave] = cw;
        __syncthreads();
        int base = run;
        for (int v = 0; v < NW; ++v) {
            if (v < wave) base += s_wsum[v];
            run += s_wsum[v];
        }
        for (int b = 0; b < CW; b += 64) {
            const bool hit = s_ids[wave * CW + b + lane] == esel;
            const uint64_t bal = __ballot(hit);
            const int rank = base + __popcll(bal & ((1ull << lane) - 1ull));
            if (hit && rank >= r0 && rank < r0 + BM) s_slot[rank - r0] = c0 + wave * CW + b + lane;
            base += __popcll(bal);
        }
    }
    __syncthreads();
    return esel;
}

// Expert-indexed tile of this workgroup from the tile table: returns the
// expert (s_slot filled, then a barrier) or -1 past the table's last tile.
template <int BM, int NTHREADS>
QMV_DEV int table_tile(const int *__restrict__ ntiles, const int *__restrict__ tile_e,
                       const int *__restrict__ tile_slots, int *s_slot) {
    if ((int)blockIdx.y >= *ntiles) return -1;
    for (int i = threadIdx.x; i < BM; i += NTHREADS) s_slot[i] = tile_slots[(size_t)blockIdx.y * BM + i];
    __syncthreads();
    return tile_e[blockIdx.y];
}

// MOE: expert-indexed rows (TABLE: from the tile table, else grouped here).
// PAIR (expert-indexed, NT == 2): the tile's columns interleave gate and up
// rows by 16 -- wave column block w holds gate rows and then up rows
// [BN/2 * blockIdx.x + 16 w, +16) -- so one lane holds both dots of an
// output and writes h = silu(gate) * up.
template <int BM, int BN, int KP, int MT, int NT, int NTHREADS, bool MOE = false, bool TABLE = false,
          bool PAIR = false>
__global__ __launch_bounds__(NTHREADS) void k_qmm_q4k(const QmmArgs a) {
    static_assert(!PAIR || (MOE && NT == 2), "paired gate/up tiles");
    const uint8_t *__restrict__ w = a.w;
    const int8_t *__restrict__ xq = a.xq;
    const float *__restrict__ xs = a.xs;
    const float *__restrict__ xsum = a.xsum;
    float *__restrict__ Y = a.Y;
    const int m = a.m, n = a.n, k = a.k;
    constexpr int WM = 16 * MT, WN = 16 * NT;
    constexpr int WGM = BM / WM, WGN = BN / WN;
    static_assert(WGM * WGN == NTHREADS / 64, "the waves tile the workgroup");
    constexpr int ST = KP + 8;                     // halves per LDS row (4-bank shift per row)
    constexpr int NBP = KP / 32;                   // q8 blocks per phase
    constexpr int PPS = 256 / KP;                  // phases per superblock
    static_assert(KP <= 128, "an even number of phases (the loop takes them in pairs)");
    constexpr int AC = BM * KP / (8 * NTHREADS);   // 8-byte activation chunks per thread
    constexpr int ACR = KP / 8;                    // activation chunks per row
    constexpr int BCH = BN * KP / 16;              // 8-code-byte weight chunks per phase
    constexpr int BCT = BCH > NTHREADS ? BCH / NTHREADS : 1;  // weight chunks per thread
    constexpr int XC = (BM * NBP + NTHREADS - 1) / NTHREADS;  // xs values per thread
    static_assert(AC * 8 * NTHREADS == BM * KP, "activation staging");
    static_assert((BCH <= NTHREADS || BCH == BCT * NTHREADS) && NTHREADS % BN == 0, "weight staging");
    static_assert(XC * NTHREADS == BM * NBP || (XC == 1 && BM * NBP < NTHREADS), "xs staging");
    static_assert(ACR >= 8, "eight lanes of a row per activation write");

    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * ST];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * ST];
    __shared__ __attribute__((aligned(16))) float sxs[2][NBP][BM];
    __shared__ __attribute__((aligned(16))) float sxsum[2][8][BM];  // by superblock parity
    __shared__ float sd[2][BN], sdmn[2][8][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WGM, wn = wave / WGM;
    const int li = lane & 15, lq = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int kb = k / 32;
    const size_t row_bytes = (size_t)(k / 256) * 144;

    // Expert-indexed mode: this workgroup's tile
    __shared__ int s_slot[MOE ? BM : 1];
    int esel = 0;  // expert of this workgroup's tile
    if constexpr (MOE) {
        if constexpr (TABLE) {
            esel = table_tile<BM, NTHREADS>(a.ntiles, a.tile_e, a.tile_slots, s_slot);
        } else {
            static_assert(sizeof(Bs[0]) >= QMM_ID_CHUNK * 4 && sizeof(As[0]) >= QMM_MOE_MAX_E * 4,
                          "grouping scratch");
            esel = qmm_group<BM, BN, NTHREADS>(a.ids, m, a.E, reinterpret_cast<int *>(&Bs[0][0]),
                                               reinterpret_cast<int *>(&As[0][0]), s_slot, Y, n, n0);
        }
        if (esel < 0) return;  // uniform over the workgroup
    }
    // activation row of each staging role (-1: no row, zeros are staged)
    auto act_row = [&](int row) -> int {
        if constexpr (MOE) {
            const int sl = s_slot[row];
            return sl >= 0 ? sl / a.x_div : -1;
        } else {
            return m0 + row < m ? m0 + row : -1;
        }
    };

    // weight staging role (rows fastest, so that eight lanes write eight
    // rows at one offset): row brow, code bytes [8*bc, +8) of the phase's
    // slice of the row's 128 code bytes
    const bool bact = tid < BCH;
    const int brow = tid % BN, bc0 = tid / BN;  // chunk i has bc = bc0 + i*NTHREADS/BN
    // weight row of the staging role: row n0 + brow, or for PAIR the gate /
    // up row of the interleaved column brow
    int wr_row = n0 + brow;
    const uint8_t *wsrc = w;
    if constexpr (PAIR) {
        wr_row = (BN / 2) * blockIdx.x + 16 * (brow / 32) + brow % 16;
        if ((brow / 16) & 1) wsrc = a.w2;
    }
    const bool bvalid = bact && wr_row < n;
    const uint8_t *wrow = wsrc + ((size_t)esel * n + (bvalid ? wr_row : 0)) * row_bytes;
    // activation rows of this thread's activation chunks and xs entries
    int arow[AC], xrow[XC];
#pragma unroll
    for (int i = 0; i < AC; ++i) arow[i] = act_row((tid + NTHREADS * i) / ACR);
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int idx = tid + NTHREADS * i;
        xrow[i] = idx < BM * NBP ? act_row(idx % BM) : -1;
    }

    // two register sets of raw codes: phase p is loaded into set p % 2 two
    // phases before it is converted
    uint2 ra[2][AC];
    uint2 rb[2][BCT];
    uint4 rh[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    float rxs[2][XC], rxsum[2][XC];
    uint32_t scp0 = 0, scp1 = 0;  // sc0..3, sc4..7 of the current superblock

    auto prefetch = [&](int ph, int q) {  // q == ph % 2, a constant
        const int k0 = ph * KP, s = k0 / 256, half = ph % PPS;
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c8 = (tid + NTHREADS * i) % ACR;
            const int gm = arow[i];
            ra[q][i] = gm >= 0 ? *reinterpret_cast<const uint2 *>(xq + (size_t)gm * k + k0 + 8 * c8)
                              : make_uint2(0u, 0u);
        }
        if (bvalid) {
            const uint8_t *blk = wrow + (size_t)s * 144;
#pragma unroll
            for (int i = 0; i < BCT; ++i)
                rb[q][i] = *reinterpret_cast<const uint2 *>(blk + 16 + half * (KP / 2) + 8 * (bc0 + i * (NTHREADS / BN)));
            if (half == 0) rh[q] = ld16(blk);
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int bl = (tid + NTHREADS * i) / BM;
            const int gm = xrow[i];
            const bool ok = gm >= 0;
            rxs[q][i] = ok ? xs[(size_t)gm * kb + k0 / 32 + bl] : 0.f;
            rxsum[q][i] = ok ? xsum[(size_t)gm * kb + k0 / 32 + bl] : 0.f;
        }
    };

    auto convert_store = [&](int ph, int buf, int q) {  // q == ph % 2
        const int half = ph % PPS, j0 = half * NBP;  // first sub-block of the phase
        const int sp = (ph / PPS) & 1;               // superblock parity
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int ch = tid + NTHREADS * i, row = ch / ACR, c8 = ch % ACR;
            const uint2 h0 = i8x4_to_f16(ra[q][i].x), h1 = i8x4_to_f16(ra[q][i].y);
            *reinterpret_cast<uint4 *>(&As[buf][row * ST + 8 * c8]) = make_uint4(h0.x, h0.y, h1.x, h1.y);
        }
        if (bact) {
            if (half == 0) {
                // the superblock's scales: sc bytes kept packed, d and dmin*m to LDS
                uint32_t s01, m01, s23, m23, s45, m45, s67, m67;
                const uint4 hd = rh[q];
                q4k_scales(hd.y, hd.z, hd.w, 0, &s01, &m01);
                q4k_scales(hd.y, hd.z, hd.w, 1, &s23, &m23);
                q4k_scales(hd.y, hd.z, hd.w, 2, &s45, &m45);
                q4k_scales(hd.y, hd.z, hd.w, 3, &s67, &m67);
                scp0 = s01 | (s23 << 16);
                scp1 = s45 | (s67 << 16);
                if (bc0 == 0) {
                    const uint32_t mp0 = m01 | (m23 << 16), mp1 = m45 | (m67 << 16);
                    const float dm = h2f(hd.x >> 16);
                    sd[sp][brow] = h2f(hd.x);
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        sdmn[sp][jj][brow] = dm * (float)(((jj < 4 ? mp0 : mp1) >> (8 * (jj & 3))) & 0xFFu);
                }
            }
#pragma unroll
            for (int i = 0; i < BCT; ++i) {
                // code bytes [8bc, +8) of the slice: sub-blocks 2p (low nibbles)
                // and 2p+1 (high) at positions l0..l0+7, p = (half*KP/2 + 8bc)/32
                const int bc = bc0 + i * (NTHREADS / BN);
                const int o0 = half * (KP / 2) + 8 * bc;
                const int p = o0 / 32, l0 = o0 % 32;
                const float sclo = (float)(((2 * p < 4 ? scp0 : scp1) >> (8 * ((2 * p) & 3))) & 0xFFu);
                const float schi = (float)(((2 * p + 1 < 4 ? scp0 : scp1) >> (8 * ((2 * p + 1) & 3))) & 0xFFu);
                const h2 slo = splat(sclo), nslo = splat(-1024.0f * sclo);
                const h2 shi = splat(schi), nshi = splat(-1024.0f * schi);
                const uint2 cw = rb[q][i];
                const uint2 lo0 = q4x4_to_f16(cw.x & 0x0F0F0F0Fu, slo, nslo);
                const uint2 lo1 = q4x4_to_f16(cw.y & 0x0F0F0F0Fu, slo, nslo);
                const uint2 hi0 = q4x4_to_f16((cw.x >> 4) & 0x0F0F0F0Fu, shi, nshi);
                const uint2 hi1 = q4x4_to_f16((cw.y >> 4) & 0x0F0F0F0Fu, shi, nshi);
                *reinterpret_cast<uint4 *>(&Bs[buf][brow * ST + 32 * (2 * p - j0) + l0]) =
                    make_uint4(lo0.x, lo0.y, lo1.x, lo1.y);
                *reinterpret_cast<uint4 *>(&Bs[buf][brow * ST + 32 * (2 * p + 1 - j0) + l0]) =
                    make_uint4(hi0.x, hi0.y, hi1.x, hi1.y);
            }
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int idx = tid + NTHREADS * i, row = idx % BM, bl = idx / BM;
            if (idx < BM * NBP) {
                sxs[buf][bl][row] = rxs[q][i];
                sxsum[sp][j0 + bl][row] = rxsum[q][i];
            }
        }
    };

    v4f acc[MT][NT], out[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
            out[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
        }

    const int nph = k / KP;  // even (k is a multiple of 256)
    prefetch(0, 0);
    convert_store(0, 0, 0);
    prefetch(1, 1);
    if (nph > 2) prefetch(2, 0);
    __syncthreads();
    for (int ph0 = 0; ph0 < nph; ph0 += 2) {
#pragma unroll
        for (int Q = 0; Q < 2; ++Q) {
            const int ph = ph0 + Q;
            const int buf = Q, half = ph % PPS, sp = (ph / PPS) & 1;
            // three-stage pipeline over the phase's blocks: the fragments of
            // block bl + 2 are being read from LDS and the MFMAs of block
            // bl + 1 are in flight while block bl's results are scaled and
            // summed
            h8 fa[NBP][MT], fb[NBP][NT];
            v4f fx[NBP][MT], T[NBP][MT][NT];
            auto load_frag = [&](int bl) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    fa[bl][t] = *reinterpret_cast<const h8 *>(&As[buf][(wm * WM + 16 * t + li) * ST + 32 * bl + 8 * lq]);
                    fx[bl][t] = *reinterpret_cast<const v4f *>(&sxs[buf][bl][wm * WM + 16 * t + 4 * lq]);
                }
#pragma unroll
                for (int u = 0; u < NT; ++u)
                    fb[bl][u] = *reinterpret_cast<const h8 *>(&Bs[buf][(wn * WN + 16 * u + li) * ST + 32 * bl + 8 * lq]);
            };
            auto mma = [&](int bl) {
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int u = 0; u < NT; ++u)
                        T[bl][t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[bl][t], fb[bl][u],
                                                                             (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            };
            load_frag(0);
            if (NBP > 1) load_frag(1);
            mma(0);
#pragma unroll
            for (int bl = 0; bl < NBP; ++bl) {
                if (bl + 2 < NBP) load_frag(bl + 2);
                if (bl + 1 < NBP) mma(bl + 1);
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int u = 0; u < NT; ++u) acc[t][u] = fx[bl][t] * T[bl][t][u] + acc[t][u];
            }
            if (half == PPS - 1) {
                // superblock done: out += d * acc, then the min term on MFMA
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const float dcol = sd[sp][wn * WN + 16 * u + li];
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        out[t][u] = dcol * acc[t][u] + out[t][u];
                        acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int bb = 4 * h + lq;
                    float am[MT], bmn[NT];
#pragma unroll
                    for (int t = 0; t < MT; ++t) am[t] = -sxsum[sp][bb][wm * WM + 16 * t + li];
#pragma unroll
                    for (int u = 0; u < NT; ++u) bmn[u] = sdmn[sp][bb][wn * WN + 16 * u + li];
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int u = 0; u < NT; ++u)
                            out[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[t], bmn[u], out[t][u], 0, 0, 0);
                }
            }
            // the next phase goes into the other buffer (and the other
            // superblock parity) while this one's matrix work drains; its
            // register set is then refilled three phases ahead
            if (ph + 1 < nph) {
                convert_store(ph + 1, buf ^ 1, Q ^ 1);
                if (ph + 3 < nph) prefetch(ph + 3, Q ^ 1);
            }
            __syncthreads();
        }
    }

    if constexpr (PAIR) {
        // out[t][0] = gate, out[t][1] = up for the same slot and h column
        const int col = (BN / 2) * blockIdx.x + 16 * wn + li;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = s_slot[wm * WM + 16 * t + 4 * lq + r];
                if (row >= 0 && col < n) Y[(size_t)row * n + col] = silu(out[t][0][r]) * out[t][1][r];
            }
        return;
    }
    // lane holds rows 4*lq + r, column li of each 16x16 tile
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const int col = n0 + wn * WN + 16 * u + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = wm * WM + 16 * t + 4 * lq + r;
                int row;
                if constexpr (MOE) row = s_slot[tr];
                else row = m0 + tr < m ? m0 + tr : -1;
                if (row >= 0 && col < n) Y[(size_t)row * n + col] = out[t][u][r];
            }
        }
}

// ------------------------------------------------- Q4_K prefill, weight-side
// Same contraction as k_qmm_q4k with the matrix roles swapped: the weights
// are the A operand (16 rows x 32 values per fragment) and the activations
// the B operand, so a lane of a 16x16 result holds four weight rows
// (4*lq + r) of one activation row (li), and that row's xs for a block is a
// single scalar per lane. The weight fragments never pass through LDS: a
// lane loads, per 32-value block, the 8 code bytes its fragment needs (the
// low nibbles of bytes 8*lq..8*lq+7 of a 32-byte pair are values 8*lq.. of
// the even sub-block, the high nibbles those of the odd one) and turns them
// into f16 sc*q in registers. Only the activations are staged, once per
// workgroup and superblock, as f16 in LDS (double-buffered, one barrier per
// superblock).
//
// Eight waves: NG groups of 32 weight rows x MG groups of 64 activation rows
// x KS parts of each superblock's eight blocks (KS = 2: blocks 0-3 and 4-7,
// summed through LDS at the end). Tile: BN = 32*NG weight rows x
// BM = 64*MG activation rows. Per superblock a wave forms, for each of its
// blocks, the 2x4 fragment products T (one v_mfma_f32_16x16x32_f16 each),
// adds xs*T into acc, then out += d*acc and the min term of its blocks
// (-dmin*m x xsum, one v_mfma_f32_16x16x4_f32 per four blocks).
//
// MODE 1 (the MoE prefill gate/up GEMM on the tile table of
// k_group_tiles): workgroup row block blockIdx.y is table tile blockIdx.y
// (its expert and 64 slots, -1 past the expert's count; spare tiles exit),
// activation row of slot s is s / x_div, and the wave's two 16-row fragments
// are gate row i (t = 0) and up row i (t = 1) of the same h column, so a lane
// holds both dots of its outputs and writes h = silu(gate) * up.
// MODE 2 (moe_qmm_q4k): the same expert-indexed rows with the tile derived
// in the kernel from ids (qmm_group), dense column layout, y[slot] rows.
template <int NG, int MG, int KS, int MODE = 0, int NU = 4>
__global__ __launch_bounds__(512) void k_qmm2_q4k(const QmmArgs a, int vec_store) {
    constexpr bool PAIRT = MODE == 1, GROUPED = MODE == 2, MOEM = MODE != 0;
    static_assert(NG * MG * KS == 8 && (KS == 1 || KS == 2), "eight waves");
    constexpr int BN = 32 * NG, BM = 16 * NU * MG;  // NU 16-row activation fragments per group
    constexpr int ST = 256 + 8;          // halves per LDS activation row (4-bank shift per row)
    constexpr int NBW = 8 / KS;          // blocks of a superblock per wave
    constexpr int NPW = NBW / 2;         // code-byte pairs per wave
    constexpr int AC = BM * 32 / 512;    // 8-byte activation chunks per thread and superblock
    constexpr int XV = (BM * 8 + 511) / 512;  // xs (and xsum) values per thread and superblock
    static_assert(AC >= 1 && AC * 512 == BM * 32 && (NU == 3 || NU == 4), "staging");
    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * ST];
    constexpr int XST = 12;              // floats per xs row: 16-byte reads of 16 rows conflict-free
    __shared__ __attribute__((aligned(16))) float sxs[2][BM * XST];
    __shared__ __attribute__((aligned(16))) float sxsum[2][BM * XST];

    const uint8_t *__restrict__ w = a.w;
    const int8_t *__restrict__ xq = a.xq;
    const float *__restrict__ xs = a.xs;
    const float *__restrict__ xsum = a.xsum;
    const int m = a.m, n = a.n, k = a.k;
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index in a scalar register: every role test below is uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = wave % KS, g = (wave / KS) % NG, mg = wave / (KS * NG);
    const int li = lane & 15, lq = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nsb = k / 256, kb = k / 32;
    const size_t row_bytes = (size_t)nsb * 144;
    static_assert(!MOEM || (MG == 1 && KS == 2), "expert-indexed tiles: one group of slots, split blocks");

    // weight banks of the two fragments (gate and up for PAIRT) and the
    // tile's slots
    __shared__ int s_slot[MOEM ? BM : 1];
    const uint8_t *wb[2] = {w, w};
    if constexpr (PAIRT) {
        const int esel = __builtin_amdgcn_readfirstlane(table_tile<BM, 512>(a.ntiles, a.tile_e, a.tile_slots, s_slot));
        if (esel < 0) return;  // uniform: past the last tile
        wb[0] = a.w + (size_t)esel * n * row_bytes;
        wb[1] = a.w2 + (size_t)esel * n * row_bytes;
    } else if constexpr (GROUPED) {
        // the activation buffers serve as the grouping's LDS scratch
        static_assert(sizeof(As[0]) >= QMM_ID_CHUNK * 4 && sizeof(As[1]) >= QMM_MOE_MAX_E * 4, "grouping scratch");
        const int esel = __builtin_amdgcn_readfirstlane(qmm_group<BM, BN, 512>(
            a.ids, m, a.E, reinterpret_cast<int *>(&As[0][0]), reinterpret_cast<int *>(&As[1][0]), s_slot, a.Y, n, n0));
        if (esel < 0) return;  // uniform: a spare workgroup (it wrote its zero rows)
        wb[0] = wb[1] = a.w + (size_t)esel * n * row_bytes;
    }
    // PAIRT: h columns [hb, hb + BN/2) of the workgroup, 16 per wave group
    const int hb = blockIdx.x * (BN / 2);
    // activation row of staging row `row` (always a valid row to read)
    auto act_row = [&](int row) -> int {
        if constexpr (MOEM) {
            const int sl = s_slot[row];
            return sl >= 0 ? sl / a.x_div : 0;
        } else {
            return min(m0 + row, m - 1);
        }
    };

    // Load addresses are a uniform base (the superblock's offset folded in,
    // scalar registers) plus a per-lane 32-bit offset fixed for the whole
    // loop (the host routes shapes whose offsets could pass 2^32 elsewhere).
    // This lane's two weight rows are clamped for the loads (stores are
    // masked); its code bytes of pair NPW*h + pp sit at 16 + 32*pair + 8*lq.
    uint32_t woff[2], qoff[2][NPW];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int wr = PAIRT ? hb + 16 * g + li : n0 + 32 * g + 16 * t + li;
        woff[t] = (uint32_t)((size_t)min(wr, n - 1) * row_bytes);
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) qoff[t][pp] = woff[t] + 16 + 32 * (NPW * h + pp) + 8 * lq;
    }

    // Raw superblock codes of this lane (header and NPW 8-byte pieces per
    // row) and the activation chunks it stages, in registers between the
    // load and their use (one superblock of work to land for the weights,
    // two for the activations).
    struct WSet {
        uint4 hdr[2];
        uint2 qc[2][NPW];
    };
    auto load_w = [&](int s, WSet &W) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t *wsb = wb[t] + (size_t)s * 144;
            W.hdr[t] = ld16(wsb + woff[t]);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) W.qc[t][pp] = *reinterpret_cast<const uint2 *>(wsb + qoff[t][pp]);
        }
    };
    // Activation staging: chunk c = tid + 512*i is row c/32, bytes 8*(c%32)
    // (8-byte pieces, so that consecutive lanes write consecutive 16-byte f16
    // units: conflict-free). The loads read clamped rows unconditionally;
    // rows past m are zeroed when stored, so nothing consumes a loaded value
    // before the store (a select right after the loads would make the
    // compiler wait for them there).
    struct ASet {
        uint2 q[AC];
        float xs[XV], xsum[XV];
    };
    uint32_t aoff[AC], xoff[XV];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int c = tid + 512 * i;
        aoff[i] = (uint32_t)((size_t)act_row(c >> 5) * k + 8 * (c & 31));
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        const int c = min(tid + 512 * i, BM * 8 - 1);  // threads past the tile's xs read its last one
        xoff[i] = (uint32_t)((size_t)act_row(c >> 3) * kb + (c & 7));
    }
    auto load_act = [&](int s, ASet &A) {
        const int8_t *xqs = xq + (size_t)s * 256;
        const float *xss = xs + (size_t)s * 8, *xms = xsum + (size_t)s * 8;
#pragma unroll
        for (int i = 0; i < AC; ++i) A.q[i] = *reinterpret_cast<const uint2 *>(xqs + aoff[i]);
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            A.xs[i] = xss[xoff[i]];
            A.xsum[i] = xms[xoff[i]];
        }
    };
    auto store_act = [&](int buf, const ASet &A) {
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c = tid + 512 * i, row = c >> 5, c8 = c & 31;
            const uint2 v = MOEM || m0 + row < m ? A.q[i] : make_uint2(0u, 0u);
            const uint2 h0 = i8x4_to_f16(v.x), h1 = i8x4_to_f16(v.y);
            *reinterpret_cast<uint4 *>(&As[buf][row * ST + 8 * c8]) = make_uint4(h0.x, h0.y, h1.x, h1.y);
        }
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int c = tid + 512 * i, row = c >> 3, j = c & 7;
            if (BM * 8 % 512 != 0 && c >= BM * 8) continue;
            const bool ok = MOEM || m0 + row < m;
            sxs[buf][row * XST + j] = ok ? A.xs[i] : 0.f;
            sxsum[buf][row * XST + j] = ok ? A.xsum[i] : 0.f;
        }
    };

    v4f acc[2][NU], out[2][NU];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
            out[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
        }

    // One register set each: the next superblock's weights are requested as
    // soon as the current ones are copied out of the set, and the activations
    // of superblock s + 2 as soon as those of s + 1 are stored to LDS (two
    // sets, two superblocks ahead, took more registers and measured slower).
    WSet wset;
    ASet aset;
    // Every load and store below is unconditional: superblock indices past
    // the end are clamped to the last one (its data is loaded again and
    // never used). A branch around them would make the compiler's wait
    // counts assume the shorter path and wait for every load in flight.
    load_w(0, wset);
    load_act(0, aset);
    store_act(0, aset);
    load_act(min(1, nsb - 1), aset);
    __syncthreads();

    // one superblock: P = s % 2 names its register set and LDS buffer
    auto superblock = [&](int s, auto Pc) {
        constexpr int P = decltype(Pc)::value;
        // this superblock's scales: sc of the wave's blocks as f16 splats,
        // -dmin*m of the min-term operand, d of the lane's output rows
        uint32_t scpk[2][NPW];
        float amn[2][KS == 1 ? 2 : 1], dout[2][4];
        uint2 q[2][NPW];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint4 hd = wset.hdr[t];
            const float dmin = h2f(hd.x >> 16);
            uint32_t sc2[NPW], mn2[NPW];
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) q4k_scales(hd.y, hd.z, hd.w, NPW * h + pp, &sc2[pp], &mn2[pp]);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) scpk[t][pp] = sc2[pp];
            // min-term operand: block 4*i + lq of the wave's blocks (lanes
            // lq = 2, 3 take the second pair; bit arithmetic rather than an
            // indexed array, which the compiler would place in LDS)
#pragma unroll
            for (int i = 0; i < (KS == 1 ? 2 : 1); ++i) {
                const uint32_t lo = mn2[2 * i], hi = mn2[2 * i + 1];
                const uint32_t pr = lo ^ ((lo ^ hi) & (0u - (uint32_t)(lq >> 1)));
                amn[t][i] = -dmin * (float)((pr >> (8 * (lq & 1))) & 0xFFu);
            }
            const float down = h2f(hd.x);
#pragma unroll
            for (int r = 0; r < 4; ++r) dout[t][r] = __shfl(down, 4 * lq + r);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) q[t][pp] = wset.qc[t][pp];
        }
        // the next superblock's weights go into the registers just read
        load_w(min(s + 1, nsb - 1), wset);
        // xs of the lane's activation rows for the wave's blocks
        float xv[NU][NBW];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const float *p = &sxs[P][(16 * NU * mg + 16 * u + li) * XST + NBW * h];
#pragma unroll
            for (int c = 0; c < NBW / 4; ++c) {
                const v4f v = *reinterpret_cast<const v4f *>(p + 4 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[u][4 * c + e] = v[e];
            }
        }
        auto mma = [&](int bl, v4f (&R)[2][NU]) {
            const int jb = NBW * h + bl;  // block within the superblock
            h8 bf[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u)
                bf[u] = *reinterpret_cast<const h8 *>(&As[P][(16 * NU * mg + 16 * u + li) * ST + 32 * jb + 8 * lq]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // the block's sc as an f16 pair (exact: the half 1024 + sc,
                // minus 1024); the high nibbles stay in place (16*q), which
                // the scale pair absorbs: (1024 + 16q)*(sc/16) - 64*sc = q*sc
                const uint32_t sb = __builtin_amdgcn_perm(0x64646464u, scpk[t][bl / 2], (bl & 1) ? 0x04010401u : 0x04000400u);
                const h2 sch = as_h2(sb) + splat(-1024.0f);
                const h2 mul = (bl & 1) ? sch * splat(0.0625f) : sch;
                const h2 add = sch * splat((bl & 1) ? -64.0f : -1024.0f);
                const uint2 cw = q[t][bl / 2];
                const uint32_t msk = (bl & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
                const uint2 v0 = q4x4_to_f16(cw.x & msk, mul, add);
                const uint2 v1 = q4x4_to_f16(cw.y & msk, mul, add);
                const h8 af = __builtin_bit_cast(h8, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
                for (int u = 0; u < NU; ++u)
                    R[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[u], (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
        };
#pragma unroll
        for (int bl = 0; bl < NBW; ++bl) {
            v4f T[2][NU];
            mma(bl, T);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < NU; ++u) acc[t][u] = bl == 0 ? xv[u][bl] * T[t][u] : xv[u][bl] * T[t][u] + acc[t][u];
        }

        // superblock done: out += d*acc, then the min term of the wave's blocks
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < NU; ++u) {
#pragma unroll
                for (int r = 0; r < 4; ++r) out[t][u][r] = dout[t][r] * acc[t][u][r] + out[t][u][r];
            }
#pragma unroll
        for (int i = 0; i < (KS == 1 ? 2 : 1); ++i) {
            float xb[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) xb[u] = sxsum[P][(16 * NU * mg + 16 * u + li) * XST + NBW * h + 4 * i + lq];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < NU; ++u)
                    out[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(amn[t][i], xb[u], out[t][u], 0, 0, 0);
        }
        // superblock s + 1's activations (loaded a superblock ago) into the
        // other buffer, which every wave finished reading before the last
        // barrier (after the last superblock this stores unused data), then
        // superblock s + 2's into the registers just stored
        store_act(P ^ 1, aset);
        load_act(min(s + 2, nsb - 1), aset);
        __syncthreads();
    };
    for (int s = 0; s < nsb; s += 2) {
        superblock(s, std::integral_constant<int, 0>{});
        if (s + 1 < nsb) superblock(s + 1, std::integral_constant<int, 1>{});
    }
    if constexpr (KS == 2) {
        // the second half of each superblock's blocks adds in through LDS
        // (the activation buffers are free after the loop's last barrier)
        float *red = reinterpret_cast<float *>(&As[0][0]);
        const int pair = g + NG * mg;
        if (h == 1) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[((pair * 2 + t) * 4 * NU + 4 * u + r) * 64 + lane] = out[t][u][r];
        }
        __syncthreads();
        if (h == 1) return;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[t][u][r] += red[((pair * 2 + t) * 4 * NU + 4 * u + r) * 64 + lane];
    }
    float *__restrict__ Y = a.Y;
    if constexpr (PAIRT) {
        // out[0] = gate, out[1] = up of h columns hb + 16g + 4lq + r
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int slot = s_slot[16 * u + li];
            if (slot < 0) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = hb + 16 * g + 4 * lq + r;
                if (col < n) Y[(size_t)slot * n + col] = silu(out[0][u][r]) * out[1][u][r];
            }
        }
        return;
    }
    // lane holds weight rows 4*lq + r of each 16x16 result, activation row li
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        int row;
        if constexpr (GROUPED) row = s_slot[16 * u + li];
        else row = m0 + 16 * NU * mg + 16 * u + li < m ? m0 + 16 * NU * mg + 16 * u + li : -1;
        if (row < 0) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = n0 + 32 * g + 16 * t + 4 * lq;
            float *dst = Y + (size_t)row * n + col;
            if (vec_store && col + 3 < n) {
                *reinterpret_cast<v4f *>(dst) = out[t][u];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (col + r < n) dst[r] = out[t][u][r];
            }
        }
    }
}

// ------------------------------------- Q4_K prefill on the int8 matrix cores
// The bm = 64 weight-side tile of k_qmm2_q4k<4, 1, 2> (128 weight rows x 64
// activation rows, eight waves, each superblock's eight blocks split 4 + 4
// over two waves) with the integer dot of each block on
// v_mfma_i32_16x16x32_i8 instead of the f16 instruction: the weight codes q
// (0..15, the nibbles masked in place) and the activation codes xq enter as
// int8, K = 32 is one q8 block, and T = sum q*xq is exact in int32. The
// activations are staged as raw int8 (no conversion). What the int8 operands
// cannot carry is the weight's 6-bit sub-block scale (sc*q reaches 945), so
// the epilogue takes, per output and block, the conversion of T and a fused
// multiply-add with sc*xs, plus one product sc*xs per output and block:
// three vector instructions where the f16 form (sc folded into its
// operand) needs one. Kept as the int8 form of the tile, to compare with.
template <int NG>
__global__ __launch_bounds__(512) void k_qmm_i8_q4k(const QmmArgs a, int vec_store) {
    constexpr int KS = 2;
    static_assert(NG * KS == 8, "eight waves");
    constexpr int BN = 32 * NG, BM = 64;
    constexpr int ST = 256 + 16;         // bytes per LDS activation row: 8-byte reads of 32 lanes conflict-free
    constexpr int NBW = 8 / KS;          // blocks of a superblock per wave
    constexpr int NPW = NBW / 2;         // code-byte pairs per wave
    constexpr int AC = BM * 32 / 512;    // 8-byte activation chunks per thread and superblock
    constexpr int XV = BM * 8 / 512;     // xs (and xsum) values per thread and superblock
    static_assert(AC >= 1 && XV >= 1, "staging");
    typedef int v4i __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * ST];
    constexpr int XST = 12;
    __shared__ __attribute__((aligned(16))) float sxs[2][BM * XST];
    __shared__ __attribute__((aligned(16))) float sxsum[2][BM * XST];

    const uint8_t *__restrict__ w = a.w;
    const int8_t *__restrict__ xq = a.xq;
    const float *__restrict__ xs = a.xs;
    const float *__restrict__ xsum = a.xsum;
    const int m = a.m, n = a.n, k = a.k;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = wave % KS, g = wave / KS;
    const int li = lane & 15, lq = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nsb = k / 256, kb = k / 32;
    const size_t row_bytes = (size_t)nsb * 144;

    // uniform base plus a per-lane 32-bit offset (the host routes shapes
    // whose offsets could pass 2^32 elsewhere); rows past n are clamped for
    // the loads and masked at the store
    uint32_t woff[2], qoff[2][NPW];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int wr = n0 + 32 * g + 16 * t + li;
        woff[t] = (uint32_t)((size_t)min(wr, n - 1) * row_bytes);
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) qoff[t][pp] = woff[t] + 16 + 32 * (NPW * h + pp) + 8 * lq;
    }
    struct WSet {
        uint4 hdr[2];
        uint2 qc[2][NPW];
    };
    auto load_w = [&](int s, WSet &W) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t *wsb = w + (size_t)s * 144;
            W.hdr[t] = ld16(wsb + woff[t]);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) W.qc[t][pp] = *reinterpret_cast<const uint2 *>(wsb + qoff[t][pp]);
        }
    };
    struct ASet {
        uint2 q[AC];
        float xs[XV], xsum[XV];
    };
    uint32_t aoff[AC], xoff[XV];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int c = tid + 512 * i;
        aoff[i] = (uint32_t)((size_t)min(m0 + (c >> 5), m - 1) * k + 8 * (c & 31));
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        const int c = tid + 512 * i;
        xoff[i] = (uint32_t)((size_t)min(m0 + (c >> 3), m - 1) * kb + (c & 7));
    }
    auto load_act = [&](int s, ASet &A) {
        const int8_t *xqs = xq + (size_t)s * 256;
        const float *xss = xs + (size_t)s * 8, *xms = xsum + (size_t)s * 8;
#pragma unroll
        for (int i = 0; i < AC; ++i) A.q[i] = *reinterpret_cast<const uint2 *>(xqs + aoff[i]);
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            A.xs[i] = xss[xoff[i]];
            A.xsum[i] = xms[xoff[i]];
        }
    };
    auto store_act = [&](int buf, const ASet &A) {
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c = tid + 512 * i, row = c >> 5, c8 = c & 31;
            const uint2 v = m0 + row < m ? A.q[i] : make_uint2(0u, 0u);
            *reinterpret_cast<uint2 *>(&As[buf][row * ST + 8 * c8]) = v;
        }
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int c = tid + 512 * i, row = c >> 3, j = c & 7;
            const bool ok = m0 + row < m;
            sxs[buf][row * XST + j] = ok ? A.xs[i] : 0.f;
            sxsum[buf][row * XST + j] = ok ? A.xsum[i] : 0.f;
        }
    };

    v4f acc[2][4], out[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
            out[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
        }
    // one register set each, as in k_qmm2_q4k: the next superblock's
    // weights, and the activations of superblock s + 2 once those of s + 1
    // are in LDS
    WSet wset;
    ASet aset;
    load_w(0, wset);
    load_act(0, aset);
    store_act(0, aset);
    load_act(min(1, nsb - 1), aset);
    __syncthreads();

    auto superblock = [&](int s, auto Pc) {
        constexpr int P = decltype(Pc)::value;
        // per weight row of the lane's fragment (row li): the four blocks'
        // sc as bytes; the lane's outputs are rows 4*lq + r, whose sc and d
        // come from the lanes holding those rows
        float amn[2], dout[2][4];
        uint32_t scr[2][4];
        uint2 q[2][NPW];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint4 hd = wset.hdr[t];
            const float dmin = h2f(hd.x >> 16);
            uint32_t sc2[NPW], mn2[NPW];
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) q4k_scales(hd.y, hd.z, hd.w, NPW * h + pp, &sc2[pp], &mn2[pp]);
            const uint32_t sc4 = sc2[0] | (sc2[1] << 16);  // blocks 0..3 of the wave
#pragma unroll
            for (int r = 0; r < 4; ++r) scr[t][r] = __shfl(sc4, 4 * lq + r);
            {
                const uint32_t lo = mn2[0], hi = mn2[1];
                const uint32_t pr = lo ^ ((lo ^ hi) & (0u - (uint32_t)(lq >> 1)));
                amn[t] = -dmin * (float)((pr >> (8 * (lq & 1))) & 0xFFu);
            }
            const float down = h2f(hd.x);
#pragma unroll
            for (int r = 0; r < 4; ++r) dout[t][r] = __shfl(down, 4 * lq + r);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) q[t][pp] = wset.qc[t][pp];
        }
        load_w(min(s + 1, nsb - 1), wset);
        float xv[4][NBW];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float *p = &sxs[P][(16 * u + li) * XST + NBW * h];
            const v4f v = *reinterpret_cast<const v4f *>(p);
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[u][e] = v[e];
        }
#pragma unroll
        for (int bl = 0; bl < NBW; ++bl) {
            const int jb = NBW * h + bl;
            long bf[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                bf[u] = *reinterpret_cast<const long *>(&As[P][(16 * u + li) * ST + 32 * jb + 8 * lq]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint2 cw = q[t][bl / 2];
                const uint32_t c0 = (bl & 1) ? (cw.x >> 4) & 0x0F0F0F0Fu : cw.x & 0x0F0F0F0Fu;
                const uint32_t c1 = (bl & 1) ? (cw.y >> 4) & 0x0F0F0F0Fu : cw.y & 0x0F0F0F0Fu;
                const long af = (long)(((uint64_t)c1 << 32) | c0);
                float scf[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) scf[r] = (float)((scr[t][r] >> (8 * bl)) & 0xFFu);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const v4i T = __builtin_amdgcn_mfma_i32_16x16x32_i8(af, bf[u], (v4i){0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float f = scf[r] * xv[u][bl];
                        acc[t][u][r] = bl == 0 ? f * (float)T[r] : fmaf(f, (float)T[r], acc[t][u][r]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[t][u][r] = dout[t][r] * acc[t][u][r] + out[t][u][r];
        {
            float xb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) xb[u] = sxsum[P][(16 * u + li) * XST + NBW * h + lq];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    out[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(amn[t], xb[u], out[t][u], 0, 0, 0);
        }
        store_act(P ^ 1, aset);
        load_act(min(s + 2, nsb - 1), aset);
        __syncthreads();
    };
    for (int s = 0; s < nsb; s += 2) {
        superblock(s, std::integral_constant<int, 0>{});
        if (s + 1 < nsb) superblock(s + 1, std::integral_constant<int, 1>{});
    }
    // the second half of each superblock's blocks adds in through LDS (the
    // staging buffers are free after the loop's last barrier)
    float *red = reinterpret_cast<float *>(&As[0][0]);
    static_assert(sizeof(As) >= 4 * 32 * 64 * 4, "reduction scratch");
    if (h == 1) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[((g * 32) + 16 * t + 4 * u + r) * 64 + lane] = out[t][u][r];
    }
    __syncthreads();
    if (h == 1) return;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[t][u][r] += red[((g * 32) + 16 * t + 4 * u + r) * 64 + lane];
    float *__restrict__ Y = a.Y;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = m0 + 16 * u + li;
        if (row >= m) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = n0 + 32 * g + 16 * t + 4 * lq;
            float *dst = Y + (size_t)row * n + col;
            if (vec_store && col + 3 < n) {
                *reinterpret_cast<v4f *>(dst) = out[t][u];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (col + r < n) dst[r] = out[t][u][r];
            }
        }
    }
}

// ------------------------------------ Q4_K prefill on a split f16 activation
// Y = W_deq x_deq with x_deq = xs * xq (the q8 activation, dequantized):
// a pre-pass writes each row of x_deq, scaled by a power of two rs that puts
// the row's largest magnitude (xs*127 of its largest block) in [2^14, 2^15),
// as two f16 halves: hi = f16(v), lo = f16(v - hi), v = rs * xs * xq. Their
// sum keeps 22 bits of v (the f32 product itself is within 2^-24), so
//   Y[i, r] = (1/rs_i) * sum_s d[r,s] * sum_{c in s} (sc*q)[r, c] * (hi + lo)[i, c]
//             - sum_b xsum[i,b] * dmin[r,s(b)] * m[r,b]
// needs no per-block epilogue: the matrix cores accumulate a whole
// superblock (two MFMAs per block, hi then lo), and the vector ALU only adds
// d times that sum once per superblock. The min term takes rs*xsum (exact)
// so that it lands in the same scaled units, and the epilogue multiplies by
// 1/rs (exact).
//
// Pre-pass: one 256-thread workgroup per activation row.
QMV_DEV float group_max_wave(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__global__ __launch_bounds__(256) void k_act_split(const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                   _Float16 *__restrict__ hi, _Float16 *__restrict__ lo,
                                                   float *__restrict__ rs, float *__restrict__ rinv, int k) {
    const int row = blockIdx.x, tid = threadIdx.x, kb = k / 32;
    const float *xr = xs + (size_t)row * kb;
    float am = 0.f;
    for (int b = tid; b < kb; b += 256) am = fmaxf(am, xr[b]);
    __shared__ float red[4];
    am = group_max_wave(am);
    if ((tid & 63) == 0) red[tid >> 6] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) * 127.0f;
    // am in [2^e, 2^(e+1)): scale 2^(14 - e), kept normal both ways
    const int e = am > 0.f ? ((int)((__float_as_uint(am) >> 23) & 0xFF) - 127) : 0;
    const int ee = max(min(14 - e, 126), -126);
    const float sc = __uint_as_float((uint32_t)(ee + 127) << 23);
    if (tid == 0) {
        rs[row] = sc;
        rinv[row] = __uint_as_float((uint32_t)(127 - ee) << 23);
    }
    const int8_t *qr = xq + (size_t)row * k;
    for (int c = 8 * tid; c < k; c += 8 * 256) {
        const uint2 q = *reinterpret_cast<const uint2 *>(qr + c);
        const float f = xr[c / 32] * sc;  // exact scaling of xs
        _Float16 h[8], l[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int qv = (int)(int8_t)(((j < 4 ? q.x : q.y) >> (8 * (j & 3))) & 0xFFu);
            const float v = f * (float)qv;
            h[j] = (_Float16)v;
            l[j] = (_Float16)(v - (float)h[j]);
        }
        *reinterpret_cast<h8 *>(hi + (size_t)row * k + c) = h8{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]};
        *reinterpret_cast<h8 *>(lo + (size_t)row * k + c) = h8{l[0], l[1], l[2], l[3], l[4], l[5], l[6], l[7]};
    }
}

// The GEMM: the weight-side tile of k_qmm2_q4k (four groups of 32 weight
// rows, 64 activation rows, the blocks of each superblock split 4 + 4 over
// two waves), with hi and lo staged in LDS as they are (one superblock
// ahead in registers) and each block's fragment products accumulated on the
// matrix cores.
__global__ __launch_bounds__(512) void k_qmm4_q4k(const QmmArgs a, const _Float16 *__restrict__ xhi,
                                                  const _Float16 *__restrict__ xlo, const float *__restrict__ rs,
                                                  const float *__restrict__ rinv, int vec_store) {
    constexpr int BN = 128, BM = 64, NPW = 2;
    constexpr int ST = 256 + 8;  // halves per LDS row (4-bank shift per row)
    constexpr int XST = 12;
    constexpr int AC = BM * 32 / 512;  // 16-byte (8-half) chunks of hi (and of lo) per thread
    __shared__ __attribute__((aligned(16))) _Float16 Ah[2][BM * ST];
    __shared__ __attribute__((aligned(16))) _Float16 Al[2][BM * ST];
    __shared__ __attribute__((aligned(16))) float sxsum[2][BM * XST];

    const uint8_t *__restrict__ w = a.w;
    const float *__restrict__ xsum = a.xsum;
    const int m = a.m, n = a.n, k = a.k;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = wave & 1, g = wave >> 1;
    const int li = lane & 15, lq = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nsb = k / 256, kb = k / 32;
    const size_t row_bytes = (size_t)nsb * 144;

    uint32_t woff[2], qoff[2][NPW];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        woff[t] = (uint32_t)((size_t)min(n0 + 32 * g + 16 * t + li, n - 1) * row_bytes);
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) qoff[t][pp] = woff[t] + 16 + 32 * (NPW * h + pp) + 8 * lq;
    }
    struct WSet {
        uint4 hdr[2];
        uint2 qc[2][NPW];
    };
    auto load_w = [&](int s, WSet &W) {
        const uint8_t *wsb = w + (size_t)s * 144;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            W.hdr[t] = ld16(wsb + woff[t]);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) W.qc[t][pp] = *reinterpret_cast<const uint2 *>(wsb + qoff[t][pp]);
        }
    };
    // staging: chunk c = tid + 512*i is row c/32, halves 8*(c%32) of the
    // superblock (consecutive lanes write consecutive 16-byte units)
    uint32_t aoff[AC];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int c = tid + 512 * i;
        aoff[i] = (uint32_t)((size_t)min(m0 + (c >> 5), m - 1) * k + 8 * (c & 31));
    }
    const int xrow = tid >> 3, xj = tid & 7;
    const int xgm = min(m0 + xrow, m - 1);
    const uint32_t xoff = (uint32_t)((size_t)xgm * kb + xj);
    const float xrs = rs[xgm];
    // native vectors (a HIP uint4 copy is a struct memcpy that the compiler
    // left in scratch memory)
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    struct ASet {
        u4 h[AC], l[AC];
        float xsum;
    };
    auto load_act = [&](int s, ASet &A) {
        const _Float16 *hs = xhi + (size_t)s * 256, *ls = xlo + (size_t)s * 256;
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            A.h[i] = *reinterpret_cast<const u4 *>(hs + aoff[i]);
            A.l[i] = *reinterpret_cast<const u4 *>(ls + aoff[i]);
        }
        A.xsum = xsum[(size_t)s * 8 + xoff];
    };
    // Rows past m hold row m - 1's (finite) data: an activation row only
    // feeds its own output row, which is not stored, so nothing is zeroed
    // (a select on the loaded values let the compiler sink those loads to
    // the store and wait for them there).
    auto store_act = [&](int buf, const ASet &A) {
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c = tid + 512 * i, row = c >> 5, c8 = c & 31;
            *reinterpret_cast<u4 *>(&Ah[buf][row * ST + 8 * c8]) = A.h[i];
            *reinterpret_cast<u4 *>(&Al[buf][row * ST + 8 * c8]) = A.l[i];
        }
        sxsum[buf][xrow * XST + xj] = A.xsum * xrs;
    };

    v4f out[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) out[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};

    // unconditional loads, indices past the end clamped (exact wait counts)
    // (one register set of weights: the next superblock's are requested
    // as soon as the current ones are copied out of it)
    WSet wset;
    {
        ASet a0;
        load_w(0, wset);
        load_act(0, a0);
        store_act(0, a0);
    }
    __syncthreads();

    auto superblock = [&](int s, auto Pc) {
        constexpr int P = decltype(Pc)::value;
        uint32_t scpk[2][NPW];
        float amn[2], dout[2][4];
        uint2 q[2][NPW];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint4 hd = wset.hdr[t];
            const float dmin = h2f(hd.x >> 16);
            uint32_t mn2[NPW];
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) q4k_scales(hd.y, hd.z, hd.w, NPW * h + pp, &scpk[t][pp], &mn2[pp]);
            const uint32_t pr = mn2[0] ^ ((mn2[0] ^ mn2[1]) & (0u - (uint32_t)(lq >> 1)));
            amn[t] = -dmin * (float)((pr >> (8 * (lq & 1))) & 0xFFu);
            const float down = h2f(hd.x);
#pragma unroll
            for (int r = 0; r < 4; ++r) dout[t][r] = __shfl(down, 4 * lq + r);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) q[t][pp] = wset.qc[t][pp];
        }
        // the activations (stored at the end of this superblock) are
        // requested before the weights (used by the next superblock), so
        // that their wait leaves the weight loads in flight
        ASet aset;  // lives within this superblock only (kept in registers)
        load_act(min(s + 1, nsb - 1), aset);
        load_w(min(s + 1, nsb - 1), wset);
        v4f acc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
            const int jb = 4 * h + bl;
            h8 bh[4], bo[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                bh[u] = *reinterpret_cast<const h8 *>(&Ah[P][(16 * u + li) * ST + 32 * jb + 8 * lq]);
                bo[u] = *reinterpret_cast<const h8 *>(&Al[P][(16 * u + li) * ST + 32 * jb + 8 * lq]);
            }
            h8 af[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // sc*q in f16 (exact), the high nibbles in place as in k_qmm2_q4k
                const uint32_t sb = __builtin_amdgcn_perm(0x64646464u, scpk[t][bl / 2], (bl & 1) ? 0x04010401u : 0x04000400u);
                const h2 sch = as_h2(sb) + splat(-1024.0f);
                const h2 mul = (bl & 1) ? sch * splat(0.0625f) : sch;
                const h2 add = sch * splat((bl & 1) ? -64.0f : -1024.0f);
                const uint2 cw = q[t][bl / 2];
                const uint32_t msk = (bl & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
                const uint2 v0 = q4x4_to_f16(cw.x & msk, mul, add);
                const uint2 v1 = q4x4_to_f16(cw.y & msk, mul, add);
                af[t] = __builtin_bit_cast(h8, make_uint4(v0.x, v0.y, v1.x, v1.y));
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t], bh[u], acc[t][u], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t], bo[u], acc[t][u], 0, 0, 0);
        }
        // out += d*acc, then the min term of the wave's blocks (rs*xsum)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[t][u][r] = dout[t][r] * acc[t][u][r] + out[t][u][r];
        float xb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xb[u] = sxsum[P][(16 * u + li) * XST + 4 * h + lq];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u) out[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(amn[t], xb[u], out[t][u], 0, 0, 0);
        // superblock s + 1 into the other buffer (every wave finished
        // reading it before the last barrier; after the last superblock this
        // stores unused data)
        store_act(P ^ 1, aset);
        __syncthreads();
    };
    for (int s = 0; s < nsb; s += 2) {
        superblock(s, std::integral_constant<int, 0>{});
        if (s + 1 < nsb) superblock(s + 1, std::integral_constant<int, 1>{});
    }

    // the second half of each superblock's blocks adds in through LDS
    float *red = reinterpret_cast<float *>(&Ah[0][0]);
    if (h == 1) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[((g * 32) + 16 * t + 4 * u + r) * 64 + lane] = out[t][u][r];
    }
    __syncthreads();
    if (h == 1) return;
    float *__restrict__ Y = a.Y;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = m0 + 16 * u + li;
        if (row >= m) continue;
        const float ri = rinv[row];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            v4f o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = (out[t][u][r] + red[((g * 32) + 16 * t + 4 * u + r) * 64 + lane]) * ri;
            const int col = n0 + 32 * g + 16 * t + 4 * lq;
            float *dst = Y + (size_t)row * n + col;
            if (vec_store && col + 3 < n) {
                *reinterpret_cast<v4f *>(dst) = o;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (col + r < n) dst[r] = o[r];
            }
        }
    }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile configurations (BM, BN, KP, MT, NT, threads) for the two bm settings
// (measured on the 512 x 4096 x 4096 shape).
#ifndef QMM_CFG128
#define QMM_CFG128 128, 64, 128, 2, 2, 512
#define QMM_CFG128_BM 128
#define QMM_CFG128_BN 64
#define QMM_CFG128_NT 512
#endif
#ifndef QMM_CFG256
#define QMM_CFG256 256, 32, 64, 2, 2, 512
#define QMM_CFG256_BM 256
#define QMM_CFG256_BN 32
#define QMM_CFG256_NT 512
#endif
// weight-side kernel at bm = 64: four groups of 32 weight rows, one group of
// 64 activation rows, each superblock's blocks split over two waves, one
// superblock of loads in flight (one register set: 47.3 -> 44.7 us at
// 512 x 4096 x 4096, against two sets two superblocks ahead). The 128-row
// form (2, 2, 2) serves bm = 128: it spilled registers with two sets, and
// with one it fits 256 VGPRs (63.2 us on k_qmm_q4k -> 49.7 us).
#ifndef QMM2_BM64_NG
#define QMM2_BM64_NG 4
#define QMM2_BM64_MG 1
#define QMM2_BM64_KS 2
#endif
// expert-indexed tiles: 64 rows (slots), 128 columns, eight waves; the
// prefill layer also takes 32-row tiles at few slots per expert
#define QMM_MOE32 32, 128, 64, 2, 2, 256
#define QMM_MOE64 64, 128, 64, 2, 2, 512
#define QMM_MOE64_BM 64
#define QMM_MOE64_BN 128
#define QMM_MOE64_NT 512
constexpr int64_t QMM_MOE_MAX_SLOTS = 1 << 20;

}  // namespace

extern "C" int qmm_q4k(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y,
                       int64_t m, int64_t n, int64_t k, int bm, qmv_stream_t stream) {
    if (!w || !xq || !xs || !xsum || !y || m < 1 || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (bm != 64 && bm != 128 && bm != 256) return QMV_EINVAL;
    if (m > (1 << 24) || n > (1 << 24) || k > (1 << 20) || (int64_t)m * k > ((int64_t)1 << 34)) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(y, 4))
        return QMV_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    QmmArgs a{static_cast<const uint8_t *>(w), xq, xs, xsum, y, (int)m, (int)n, (int)k, nullptr, 1, 1};
    const int vec = aligned(y, 16) && n % 4 == 0;
    // the bm = 64 kernel addresses with 32-bit per-lane offsets
    const bool off32 = n * (k / 256) * 144 < ((int64_t)1 << 32) && m * k < ((int64_t)1 << 32);
    if (bm == 64 && !off32) bm = 128;
    if (bm == 64) {
        const dim3 grid((unsigned)div_up(n, 32 * QMM2_BM64_NG), (unsigned)div_up(m, 64 * QMM2_BM64_MG));
        hipLaunchKernelGGL((k_qmm2_q4k<QMM2_BM64_NG, QMM2_BM64_MG, QMM2_BM64_KS>), grid, dim3(512), 0, s, a, vec);
    } else if (bm == 128 && off32) {
        // the weight-side tile with 128 activation rows (two groups of 64),
        // one register set of loads in flight: 256 VGPRs, no spills
        const dim3 grid((unsigned)div_up(n, 64), (unsigned)div_up(m, 128));
        hipLaunchKernelGGL((k_qmm2_q4k<2, 2, 2>), grid, dim3(512), 0, s, a, vec);
    } else if (bm == 128) {
        const dim3 grid((unsigned)div_up(n, QMM_CFG128_BN), (unsigned)div_up(m, QMM_CFG128_BM));
        hipLaunchKernelGGL((k_qmm_q4k<QMM_CFG128>), grid, dim3(QMM_CFG128_NT), 0, s, a);
    } else {
        const dim3 grid((unsigned)div_up(n, QMM_CFG256_BN), (unsigned)div_up(m, QMM_CFG256_BM));
        hipLaunchKernelGGL((k_qmm_q4k<QMM_CFG256>), grid, dim3(QMM_CFG256_NT), 0, s, a);
    }
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

// The same product on the int8 matrix instructions (k_qmm_i8_q4k): a
// comparison form of the bm = 64 tile.
extern "C" int qmm_q4k_i8(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y,
                          int64_t m, int64_t n, int64_t k, qmv_stream_t stream) {
    if (!w || !xq || !xs || !xsum || !y || m < 1 || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (m > (1 << 24) || n > (1 << 24) || k > (1 << 20) || n * (k / 256) * 144 >= ((int64_t)1 << 32) ||
        m * k >= ((int64_t)1 << 32))
        return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(y, 4))
        return QMV_EALIGN;
    QmmArgs a{static_cast<const uint8_t *>(w), xq, xs, xsum, y, (int)m, (int)n, (int)k, nullptr, 1, 1};
    const int vec = aligned(y, 16) && n % 4 == 0;
    const dim3 grid((unsigned)div_up(n, 128), (unsigned)div_up(m, 64));
    hipLaunchKernelGGL((k_qmm_i8_q4k<4>), grid, dim3(512), 0, (hipStream_t)stream, a, vec);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

// workspace of qmm_q4k_split: hi and lo halves of the scaled activation,
// then the row scales and their inverses (each part 256-byte aligned)
static int64_t split_ws_parts(int64_t m, int64_t k, int64_t *o_lo, int64_t *o_rs, int64_t *o_ri) {
    auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
    const int64_t half = up(m * k * 2);
    *o_lo = half;
    *o_rs = 2 * half;
    *o_ri = 2 * half + up(m * 4);
    return 2 * half + 2 * up(m * 4);
}

extern "C" int64_t qmm_q4k_split_workspace_bytes(int64_t m, int64_t k) {
    if (m < 1 || k < 256 || k % 256) return -1;
    int64_t a, b, c;
    return split_ws_parts(m, k, &a, &b, &c);
}

extern "C" int qmm_q4k_split(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y,
                             void *ws, int64_t ws_bytes, int64_t m, int64_t n, int64_t k, qmv_stream_t stream) {
    if (!w || !xq || !xs || !xsum || !y || !ws || m < 1 || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (m > (1 << 24) || n > (1 << 24) || k > (1 << 20) || n * (k / 256) * 144 >= ((int64_t)1 << 32) ||
        m * k * 2 >= ((int64_t)1 << 32))
        return QMV_EUNSUPPORTED;
    int64_t olo, ors, ori;
    if (ws_bytes < split_ws_parts(m, k, &olo, &ors, &ori)) return QMV_EINVAL;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(y, 4) ||
        !aligned(ws, 256))
        return QMV_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = static_cast<uint8_t *>(ws);
    _Float16 *hi = reinterpret_cast<_Float16 *>(base), *lo = reinterpret_cast<_Float16 *>(base + olo);
    float *rs = reinterpret_cast<float *>(base + ors), *ri = reinterpret_cast<float *>(base + ori);
    hipLaunchKernelGGL(k_act_split, dim3((unsigned)m), dim3(256), 0, s, xq, xs, hi, lo, rs, ri, (int)k);
    QMV_LAUNCH_CHECK();
    QmmArgs a{static_cast<const uint8_t *>(w), xq, xs, xsum, y, (int)m, (int)n, (int)k, nullptr, 1, 1};
    const int vec = aligned(y, 16) && n % 4 == 0;
    hipLaunchKernelGGL(k_qmm4_q4k, dim3((unsigned)div_up(n, 128), (unsigned)div_up(m, 64)), dim3(512), 0, s, a, hi,
                       lo, rs, ri, vec);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

namespace {
// The resident-activation Q4_K GEMM of the MoE prefill (k_qmm4r, below).
#ifndef QMV_Q4R
#define QMV_Q4R 1               // 0: the tile GEMMs
#endif
constexpr int Q4R_MAX_NSB = 8;  // k <= 2048
template <bool PAIR, bool GROUPED>
void launch_q4r(const QmmArgs &a, const int *nseg, const int *seg_off, int bmt, hipStream_t s);
}  // namespace

extern "C" int moe_qmm_q4k(const void *bank, const int8_t *xq, const float *xs, const float *xsum, int64_t x_div,
                           const int32_t *ids, float *y, int64_t nslots, int64_t n, int64_t k, int64_t E,
                           qmv_stream_t stream) {
    if (!bank || !xq || !xs || !xsum || !ids || !y || x_div < 1 || nslots < 1 || n < 1 || E < 1 || k < 256 ||
        k % 256)
        return QMV_EINVAL;
    if (E > QMM_MOE_MAX_E || nslots > QMM_MOE_MAX_SLOTS || n > (1 << 24) || k > (1 << 20) ||
        E * n * (k / 256) * 144 > ((int64_t)1 << 40))
        return QMV_EUNSUPPORTED;
    if (!aligned(bank, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(ids, 4) ||
        !aligned(y, 4))
        return QMV_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    QmmArgs a{static_cast<const uint8_t *>(bank), xq, xs, xsum, y, (int)nslots, (int)n, (int)k, ids, (int)E,
              (int)x_div};
    // 64-row tiles (eight waves; faster than 32-row four-wave tiles even at
    // 32 slots per expert, measured); the grid covers the largest possible
    // tile count (every expert adds at most one partial tile) and the spare
    // workgroups exit after the grouping
    const dim3 grid((unsigned)div_up(n, QMM_MOE64_BN), (unsigned)(div_up(nslots, QMM_MOE64_BM) + std::min(E, nslots)));
    // the weight-side tile (128 weight rows x 64 slots, the same grid) while
    // its 32-bit lane offsets hold: one expert's rows and the activation rows
    // below 2^32 bytes
    const int vec = aligned(y, 16) && n % 4 == 0;
    if (QMV_Q4R && k <= 256 * Q4R_MAX_NSB)
        // 32-slot segments grouped in the kernel, the activation resident in LDS
        launch_q4r<false, true>(a, nullptr, nullptr, 32, s);
    else if (n * (k / 256) * 144 < ((int64_t)1 << 32) && div_up(nslots, x_div) * k < ((int64_t)1 << 32))
        hipLaunchKernelGGL((k_qmm2_q4k<4, 1, 2, 2>), grid, dim3(512), 0, s, a, vec);
    else
        hipLaunchKernelGGL((k_qmm_q4k<QMM_MOE64, true>), grid, dim3(QMM_MOE64_NT), 0, s, a);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

namespace {

// ===================================================================== Q6_K
// Q6_K prefill GEMM (hanzo-ml `src/vulkan_backend.rs`, `matmul_q6k_gpu`:
// weights stay quantized and each decoded value is reused over a tile of
// rows; `mul_mm_q6k_tiled_dp4a` on a q8 activation):
//   Y[i, r] = sum_s d[r,s] * sum_{b in s} fx[i,b] * (sc[r,2b'] T[i,r,2b'] + sc[r,2b'+1] T[i,r,2b'+1])
//   T[i,r,t] = sum_{l<16} a[i,16t+l] * (q[r,16t+l] - 32)
// with one q8 block b = two 16-value sub-blocks t. q - 32 (|.| <= 32) is
// exact in f16, but sc*(q - 32) (up to 4064) is not, so the sub-scale stays
// out of the matrix product: each sub-block is one v_mfma_f32_16x16x16_f16
// and the epilogue forms sc_a*T_a + sc_b*T_b per block.
//  - q8 activation (ACT_Q8): a = xq, fx = xs. T is an integer below 2^16 and
//    sc*T + sc*T an integer below 2^24, so the block sum is exact before the
//    one FMA with xs, as in the Q4_K kernel.
//  - f32 activation (ACT_F32): each 32-value block of a row is scaled by a
//    power of two fx^-1 that puts its largest magnitude in [2^14, 2^15)
//    (exact), split into a high f16 and the f16 of the remainder, and both
//    halves go through the matrix cores (two MFMAs per sub-block); fx then
//    undoes the scaling in the epilogue. The split keeps 22 bits of each
//    value, so the product is as accurate as f32 arithmetic.
// Code staging per row and phase of 64 values (a quarter superblock): the
// phase's 64 ql bytes and 32 qh bytes give q = nibble | 2 bits << 4, turned
// into the halves 1024 + q and then q - 32 exactly.
enum { ACT_Q8 = 0, ACT_F32 = 1 };

typedef _Float16 h4 __attribute__((ext_vector_type(4)));

struct Qmm6Args {
    const uint8_t *w;    // dense weight [n, k/256] blocks of 210 bytes, or the bank [E, n, k/256]
    const int8_t *xq;    // ACT_Q8: q8 activation rows
    const float *xs;     // ACT_Q8: per-32 scales
    const float *x;      // ACT_F32: f32 activation rows
    float *Y;
    int m, n, k;
    const int32_t *ids;  // expert-indexed only
    int E, x_div;
    const int *ntiles, *tile_e, *tile_slots;  // tile table (see QmmArgs)
};

// four 6-bit codes (one per byte) -> four f16 values q - 32, exact
QMV_DEV uint2 q6x4_to_f16(uint32_t c) {
    const h2 off = {(_Float16)-1056.0f, (_Float16)-1056.0f};
    return make_uint2(as_u32(as_h2(half_bytes_lo(c)) + off), as_u32(as_h2(half_bytes_hi(c)) + off));
}

template <int BM, int BN, int MT, int NT, int NTHREADS, int ACT, bool MOE, bool TABLE = false, int KP = 64>
__global__ __launch_bounds__(NTHREADS) void k_qmm_q6k(const Qmm6Args a) {
    // KP values per phase: a quarter (64) or half (128) superblock
    static_assert(KP == 64 || KP == 128, "phase length");
    constexpr int PPS = 256 / KP;                // phases per superblock
    constexpr int WM = 16 * MT, WN = 16 * NT;
    constexpr int WGM = BM / WM, WGN = BN / WN;
    static_assert(WGM * WGN == NTHREADS / 64, "the waves tile the workgroup");
    constexpr int ST = KP + 8;                   // halves per LDS row
    constexpr int NBP = KP / 32;                 // q8 blocks per phase
    constexpr int NH = ACT == ACT_F32 ? 2 : 1;   // activation halves (high, low)
    // activation staging: q8 -> 8-byte chunks (8 codes); f32 -> 16-byte chunks (4 values)
    constexpr int AW = ACT == ACT_F32 ? 4 : 8;   // values per chunk
    constexpr int ACR = KP / AW;                 // chunks per row
    constexpr int AC = BM * ACR / NTHREADS;      // chunks per thread
    static_assert(AC >= 1 && AC * NTHREADS == BM * ACR, "activation staging");
    constexpr int BCH = BN * (KP / 8);           // 8-code weight chunks per phase
    constexpr int BCT = BCH / NTHREADS;          // per thread
    static_assert(BCT >= 1 && BCT * NTHREADS == BCH && NTHREADS % BN == 0, "weight staging");
    constexpr int XC = (BM * NBP + NTHREADS - 1) / NTHREADS;  // xs values per thread (ACT_Q8)

    __shared__ __attribute__((aligned(16))) _Float16 As[NH][2][BM * ST];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * ST];
    __shared__ __attribute__((aligned(16))) float sfx[2][NBP][BM];
    __shared__ float ssc[2][16][BN], sd[2][BN];  // by superblock parity

    const float *__restrict__ xsrc = a.x;
    float *__restrict__ Y = a.Y;
    const int m = a.m, n = a.n, k = a.k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WGM, wn = wave / WGM;
    const int li = lane & 15, lq = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int kb = k / 32;
    const size_t row_bytes = (size_t)(k / 256) * 210;

    __shared__ int s_slot[MOE ? BM : 1];
    int esel = 0;
    if constexpr (MOE) {
        if constexpr (TABLE) {
            esel = table_tile<BM, NTHREADS>(a.ntiles, a.tile_e, a.tile_slots, s_slot);
        } else {
            static_assert(sizeof(Bs[0]) >= QMM_ID_CHUNK * 4 && sizeof(As[0][0]) >= QMM_MOE_MAX_E * 4,
                          "grouping scratch");
            esel = qmm_group<BM, BN, NTHREADS>(a.ids, m, a.E, reinterpret_cast<int *>(&Bs[0][0]),
                                               reinterpret_cast<int *>(&As[0][0][0]), s_slot, Y, n, n0);
        }
        if (esel < 0) return;
    }
    auto act_row = [&](int row) -> int {
        if constexpr (MOE) {
            const int sl = s_slot[row];
            return sl >= 0 ? sl / a.x_div : -1;
        } else {
            return m0 + row < m ? m0 + row : -1;
        }
    };

    // weight staging role: row brow, chunks bc = bc0 + i*NTHREADS/BN (8 codes each)
    const int brow = tid % BN, bc0 = tid / BN;
    const bool bvalid = n0 + brow < n;
    const uint8_t *wrow = a.w + ((size_t)esel * n + (bvalid ? n0 + brow : 0)) * row_bytes;
    int arow[AC], xrow[XC];
#pragma unroll
    for (int i = 0; i < AC; ++i) arow[i] = act_row((tid + NTHREADS * i) / ACR);
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int idx = tid + NTHREADS * i;
        xrow[i] = idx < BM * NBP ? act_row(idx % BM) : -1;
    }

    using AReg = typename std::conditional<ACT == ACT_F32, float4, uint2>::type;
    AReg ra[2][AC];
    uint2 rql[2][BCT], rqh[2][BCT];
    uint4 rsc[2];
    uint32_t rd[2] = {0u, 0u};
    float rxs[2][XC];

    auto prefetch = [&](int ph, int q) {
        const int k0 = ph * KP, s = k0 / 256, pi = ph % PPS;
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c = (tid + NTHREADS * i) % ACR, gm = arow[i];
            if constexpr (ACT == ACT_F32)
                ra[q][i] = gm >= 0 ? *reinterpret_cast<const float4 *>(xsrc + (size_t)gm * k + k0 + 4 * c)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            else
                ra[q][i] = gm >= 0 ? *reinterpret_cast<const uint2 *>(a.xq + (size_t)gm * k + k0 + 8 * c)
                                   : make_uint2(0u, 0u);
        }
        if (bvalid) {
            const uint8_t *blk = wrow + (size_t)s * 210;
#pragma unroll
            for (int i = 0; i < BCT; ++i) {
                // values e0..e0+7 of the superblock: half h, 32-run g, position l0
                const int e0 = KP * pi + 8 * (bc0 + i * (NTHREADS / BN));
                const int h = e0 >> 7, g = (e0 >> 5) & 3, l0 = e0 & 31;
                rql[q][i] = *reinterpret_cast<const uint2 *>(blk + 64 * h + 32 * (g & 1) + l0);
                rqh[q][i] = *reinterpret_cast<const uint2 *>(blk + 128 + 32 * h + l0);
            }
            if (pi == 0 && bc0 == 0) {
                rsc[q] = *reinterpret_cast<const uint4 *>(blk + 192);
                rd[q] = ld2(blk + 208);
            }
        }
        if constexpr (ACT == ACT_Q8) {
#pragma unroll
            for (int i = 0; i < XC; ++i) {
                const int bl = (tid + NTHREADS * i) / BM, gm = xrow[i];
                rxs[q][i] = gm >= 0 ? a.xs[(size_t)gm * kb + k0 / 32 + bl] : 0.f;
            }
        }
    };

    auto convert_store = [&](int ph, int buf, int q) {
        const int pi = ph % PPS, sp = (ph / PPS) & 1;
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int ch = tid + NTHREADS * i, row = ch / ACR, c = ch % ACR;
            if constexpr (ACT == ACT_F32) {
                // power-of-two block scale from the block's largest magnitude
                // (8 consecutive lanes hold one 32-value block)
                const float4 v = ra[q][i];
                float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
                am = fmaxf(am, __shfl_xor(am, 1));
                am = fmaxf(am, __shfl_xor(am, 2));
                am = fmaxf(am, __shfl_xor(am, 4));
                // e = exponent of am (am in [2^e, 2^(e+1))); scale 2^(14 - e)
                const int e = am > 0.f ? ((int)((__float_as_uint(am) >> 23) & 0xFF) - 127) : 0;
                const int ee = max(min(14 - e, 126), -126);  // 2^ee and 2^-ee are normal
                const float sc = __uint_as_float((uint32_t)(ee + 127) << 23);
                const float inv = __uint_as_float((uint32_t)(127 - ee) << 23);
                const float y0 = v.x * sc, y1 = v.y * sc, y2 = v.z * sc, y3 = v.w * sc;
                const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1, h2v = (_Float16)y2, h3 = (_Float16)y3;
                const h4 hi = {h0, h1, h2v, h3};
                const h4 lo = {(_Float16)(y0 - (float)h0), (_Float16)(y1 - (float)h1), (_Float16)(y2 - (float)h2v),
                               (_Float16)(y3 - (float)h3)};
                *reinterpret_cast<h4 *>(&As[0][buf][row * ST + 4 * c]) = hi;
                *reinterpret_cast<h4 *>(&As[NH - 1][buf][row * ST + 4 * c]) = lo;
                if ((c & 7) == 0) sfx[buf][c >> 3][row] = inv;
            } else {
                const uint2 h0 = i8x4_to_f16(ra[q][i].x), h1 = i8x4_to_f16(ra[q][i].y);
                *reinterpret_cast<uint4 *>(&As[0][buf][row * ST + 8 * c]) = make_uint4(h0.x, h0.y, h1.x, h1.y);
            }
        }
        if (pi == 0 && bc0 == 0) {
            const uint4 s4 = rsc[q];
            const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int t = 0; t < 16; ++t)
                ssc[sp][t][brow] = (float)(int8_t)((sw[t >> 2] >> (8 * (t & 3))) & 0xFFu);
            sd[sp][brow] = h2f(rd[q]);
        }
#pragma unroll
        for (int i = 0; i < BCT; ++i) {
            const int el = 8 * (bc0 + i * (NTHREADS / BN));  // position in the phase
            const int g = ((KP * pi + el) >> 5) & 3;
            const int nsh = 4 * (g >> 1), sh = 2 * g;  // nibble of ql, bit pair of qh for run g
            const uint2 ql = rql[q][i], qh = rqh[q][i];
            const uint32_t c0 = ((ql.x >> nsh) & 0x0F0F0F0Fu) | (((qh.x >> sh) & 0x03030303u) << 4);
            const uint32_t c1 = ((ql.y >> nsh) & 0x0F0F0F0Fu) | (((qh.y >> sh) & 0x03030303u) << 4);
            const uint2 f0 = q6x4_to_f16(c0), f1 = q6x4_to_f16(c1);
            *reinterpret_cast<uint4 *>(&Bs[buf][brow * ST + el]) = make_uint4(f0.x, f0.y, f1.x, f1.y);
        }
        if constexpr (ACT == ACT_Q8) {
#pragma unroll
            for (int i = 0; i < XC; ++i) {
                const int idx = tid + NTHREADS * i, row = idx % BM, bl = idx / BM;
                if (idx < BM * NBP) sfx[buf][bl][row] = rxs[q][i];
            }
        }
    };

    v4f acc[MT][NT], out[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
            out[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
        }

    const int nph = k / KP;  // even
    prefetch(0, 0);
    convert_store(0, 0, 0);
    prefetch(1, 1);
    if (nph > 2) prefetch(2, 0);
    __syncthreads();
    for (int ph0 = 0; ph0 < nph; ph0 += 2) {
#pragma unroll
        for (int Q = 0; Q < 2; ++Q) {
            const int ph = ph0 + Q, buf = Q, pi = ph % PPS, sp = (ph / PPS) & 1;
#pragma unroll
            for (int bl = 0; bl < NBP; ++bl) {
                v4f T[2][MT][NT];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const int col = 32 * bl + 16 * sb + 4 * lq;
                    h4 fa[NH][MT], fb[NT];
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int hl = 0; hl < NH; ++hl)
                            fa[hl][t] = *reinterpret_cast<const h4 *>(&As[hl][buf][(wm * WM + 16 * t + li) * ST + col]);
#pragma unroll
                    for (int u = 0; u < NT; ++u)
                        fb[u] = *reinterpret_cast<const h4 *>(&Bs[buf][(wn * WN + 16 * u + li) * ST + col]);
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int u = 0; u < NT; ++u) {
                            v4f r = __builtin_amdgcn_mfma_f32_16x16x16f16(fa[0][t], fb[u], (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                            if constexpr (NH == 2) r = __builtin_amdgcn_mfma_f32_16x16x16f16(fa[1][t], fb[u], r, 0, 0, 0);
                            T[sb][t][u] = r;
                        }
                }
                const int sub = (KP * pi) / 16 + 2 * bl;  // first sub-block of this q8 block in the superblock
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const int c = wn * WN + 16 * u + li;
                    const float sa = ssc[sp][sub][c], sbv = ssc[sp][sub + 1][c];
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const v4f fx = *reinterpret_cast<const v4f *>(&sfx[buf][bl][wm * WM + 16 * t + 4 * lq]);
                        const v4f S = sa * T[0][t][u] + sbv * T[1][t][u];
                        acc[t][u] = fx * S + acc[t][u];
                    }
                }
            }
            if (pi == PPS - 1) {
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const float dcol = sd[sp][wn * WN + 16 * u + li];
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        out[t][u] = dcol * acc[t][u] + out[t][u];
                        acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
            if (ph + 1 < nph) {
                convert_store(ph + 1, buf ^ 1, Q ^ 1);
                if (ph + 3 < nph) prefetch(ph + 3, Q ^ 1);
            }
            __syncthreads();
        }
    }

#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const int col = n0 + wn * WN + 16 * u + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = wm * WM + 16 * t + 4 * lq + r;
                int row;
                if constexpr (MOE) row = s_slot[tr];
                else row = m0 + tr < m ? m0 + tr : -1;
                if (row >= 0 && col < n) Y[(size_t)row * n + col] = out[t][u][r];
            }
        }
}

// Q6_K tile configurations (BM, BN, MT, NT, threads), measured at the MoE
// prefill down shape (4,096 slots, [2048, 768] experts): eight-wave tiles
// were 1.4x faster than four-wave 32 x 128 tiles, and 128-value phases
// slower than 64-value ones.
#define QMM6_DENSE 64, 128, 2, 2, 512
#define QMM6_MOE 64, 128, 2, 2, 512    // expert-indexed, q8 activation
#define QMM6_MOE_BM 64
#define QMM6_MOE_BN 128
#define QMM6_MOE_NT 512
#ifndef QMM6_MOEF                       // expert-indexed, f32 activation
#define QMM6_MOEF 64, 128, 2, 2, 512
#define QMM6_MOEF_BM 64
#define QMM6_MOEF_BN 128
#define QMM6_MOEF_NT 512
#define QMM6_MOEF_KP 64
#endif
#define QMM6_PF64 64, 128, 2, 2, 512   // the prefill layer's down projection, 64-slot tiles
#define QMM6_PF32 32, 256, 2, 2, 512   // and 32-slot tiles

// ------------------------- Q6_K expert GEMM on a resident f32 activation
// The MoE down projection at prefill has tens of slots per expert and a
// short k (the expert's inner size): the tile GEMM above then spends most of
// its time waiting on loads between its per-phase barriers. This form keeps
// a workgroup's activation rows in LDS for the whole product and lets every
// wave stream its own weight rows:
//  - a workgroup takes up to 32 slots of one expert and rw weight rows. It
//    stages the slots' rows once as two f16 halves per value under a per-row
//    power of two: v = 2^e x with the row's largest magnitude in
//    [2^14, 2^15), hi = f16(v), lo = f16(v - hi) (22 bits of each value; a
//    value far below the row's largest keeps an absolute error under 2^-25
//    of the scaled units, 2^-39 of that largest). Four values take 16 bytes,
//    [hi x4 | lo x4]; rows are 4k + 16 bytes apart, so that the 16-byte
//    fragment reads of sixteen consecutive rows hit distinct banks.
//  - each wave owns groups of 32 weight rows (two 16-row fragments) and
//    walks each group superblock by superblock, with a ring of register sets
//    holding the raw codes of the next steps in flight. There is no barrier
//    after the staging.
//  - per 16-value sub-block a lane decodes the four codes at its fragment
//    position (q - 32, exact in f16) and the matrix cores form
//    T = A_hi B + A_lo B on two v_mfma_f32_16x16x16_f16. The activation rows
//    are the A operand and the weight rows the B operand, so a lane's four
//    results share its weight row, and the VALU adds d*sc*T of that row.
// Loads read clamped rows unconditionally and stores are masked, so that the
// compiler waits for exactly the oldest step of the ring.
#ifndef QMV_Q6R
#define QMV_Q6R 1               // 0: the tile GEMM for every k
#endif
constexpr int Q6R_SLOTS = 32;   // activation rows per workgroup
constexpr int Q6R_SEG_SHIFT = 25;  // a table segment: slot count (<= 32) << 25 | offset in tile_slots
constexpr int Q6R_MAX_NSB = 4;  // k <= 1024: 32 staged rows of 4k + 16 bytes

// Codes of four consecutive positions l..l+3 in the four 32-value runs of a
// 128-value half: ql0 = ql bytes l..l+3 (runs 0 and 2), ql1 = ql bytes
// 32+l.. (runs 1 and 3), qh = qh bytes l..l+3 (two bits per run). Each
// result holds four 6-bit codes, one per byte.
QMV_DEV void q6_run_codes(uint32_t ql0, uint32_t ql1, uint32_t qh, uint32_t (&c)[4]) {
    c[0] = (ql0 & 0x0F0F0F0Fu) | ((qh << 4) & 0x30303030u);
    c[1] = (ql1 & 0x0F0F0F0Fu) | ((qh << 2) & 0x30303030u);
    c[2] = ((ql0 >> 4) & 0x0F0F0F0Fu) | (qh & 0x30303030u);
    c[3] = ((ql1 >> 4) & 0x0F0F0F0Fu) | ((qh >> 2) & 0x30303030u);
}

// 4x4 transpose of dwords across the four 16-lane rows of a wave: row p's
// dword c becomes row c's dword p (v_permlane32_swap exchanges the upper
// rows of its first operand with the lower rows of its second,
// v_permlane16_swap the odd rows of its first with the even rows of its
// second).
QMV_DEV uint4 rows_transpose(uint4 v) {
    const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return make_uint4(c[0], c[1], d[0], d[1]);
}

// Raw codes of one step (a superblock of the wave's FPW 16-row fragments).
// Lane row lq loads the 16 bytes of its home (hh, lh) = (lq >> 1, lq & 1):
// ql bytes 64hh + 16lh.. (runs 0 and 2), ql bytes 64hh + 32 + 16lh.. (runs 1
// and 3) and qh bytes 32hh + 16lh..; after rows_transpose, dword 2hh + lh of
// each holds positions 16lh + 4lq.. of half hh, the lane's fragment
// positions. sc and d are the row's scales.
template <int FPW>
struct Q6rRaw {
    uint4 ql0[FPW], ql1[FPW], qh[FPW], sc[FPW];
    uint32_t d[FPW];
};

// Steps in flight per wave: one (with the segment-aligned unit runs, MoE
// prefill layer at 64 / 128 / 512 tokens 146.8 / 149.2 / 236.6 us with two,
// 143.7 / 146.5 / 223.5 with one).
#ifndef Q6R_RING
#define Q6R_RING 1
#endif
#ifndef Q6R_FPW
#define Q6R_FPW 1               // 16-row weight fragments per wave (1: 16 waves, 2: 8 waves)
#endif

// Work: the product splits into units of one 32-slot segment (the slots of
// one expert, packed) by 256 weight rows. One workgroup per CU (the staged
// rows fill most of its LDS), each taking an equal run of consecutive units,
// so a workgroup stages once per segment its run touches (one or two) and
// every CU gets the same amount of work. GROUPED: the segments are the
// expert's slots in ascending slot order, 32 at a time, derived in every
// workgroup from ids (per-expert counts, then a ballot compaction of the
// segment's slots); the workgroups also share the zeroing of the rows of
// slots whose expert is outside [0, E). Otherwise the segments come from the
// layer's tile table (nseg, seg_off).
// FPW weight fragments per wave, 16 / FPW waves: 256 weight rows per unit.
// Q8A: the activation rows are q8 (xq, xs per 32 values); staging forms
// each value as xq * xs in f32 and then splits it like an f32 row.
// Units [u, u1) of this workgroup in the resident-activation GEMMs (nseg
// segments of nu units each). A workgroup whose run crosses a segment
// boundary stages twice and ramps its weight loads up twice, so when the
// segments are at most the workgroups (grid / nseg >= 2, or 1 with the
// segments filling three quarters of the grid or more) every segment is
// cut into grid / nseg equal runs and each workgroup takes at most one
// (128 experts, gate projection, 127 segments of 48 units: 52.3 us with
// contiguous shares, 41.1 us at 128 segments, where the shares align);
// otherwise every workgroup takes an equal contiguous share of all units.
__device__ __forceinline__ void resident_unit_range(int nseg, int nu, int64_t *u, int64_t *u1) {
    const int grid = (int)gridDim.x, b = (int)blockIdx.x;
    const int kper = nseg > 0 ? grid / nseg : 0;
    if (kper >= 2 || (kper == 1 && 4 * nseg >= 3 * grid)) {
        if (b < nseg * kper) {
            const int seg = b / kper, part = b - seg * kper;
            *u = (int64_t)seg * nu + (int64_t)nu * part / kper;
            *u1 = (int64_t)seg * nu + (int64_t)nu * (part + 1) / kper;
        } else {
            *u = *u1 = 0;  // no run left for this workgroup
        }
        return;
    }
    const int64_t total = (int64_t)nseg * nu;
    *u = total * b / grid;
    *u1 = total * (b + 1) / grid;
}

template <int NSB, bool GROUPED, int FPW, int SL, bool Q8A = false>
__global__ __launch_bounds__(1024 / FPW) void k_qmm6r(const Qmm6Args a, const int *__restrict__ nseg_p,
                                                       const int *__restrict__ seg_off, int bmt) {
    static_assert(NSB >= 1 && NSB <= Q6R_MAX_NSB, "k <= 1024");
    static_assert(FPW == 1 || FPW == 2, "fragments per wave");
    constexpr int NW = 16 / FPW, NT = 64 * NW;           // waves, threads
    constexpr int PITCH = 1024 * NSB + 16;                // bytes per staged row
    constexpr int D = Q6R_RING;                           // steps in flight per wave
    static_assert(SL == 32 || SL == 48, "slots per segment");
    constexpr int LPR = SL == 32 ? NT / 32 : NT / 64;     // staging lanes per row (a power of two)
    constexpr int CPL = 64 * NSB / LPR;                   // staged float4 per lane
    __shared__ __attribute__((aligned(16))) uint8_t act[SL * PITCH];
    __shared__ int s_slot[SL];
    __shared__ float s_inv[SL];
    __shared__ int s_misc[4], s_wsum[NW];
    __shared__ int s_cnt[GROUPED ? QMM_MOE_MAX_E : 1], s_sb[GROUPED ? QMM_MOE_MAX_E : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lq = lane >> 4;
    const int n = a.n, m = a.m, E = a.E;
    const int ngr = (n + 16 * FPW - 1) / (16 * FPW);  // row groups (one wave's fragments) of a segment
    const int32_t *__restrict__ ids = a.ids;
    float *__restrict__ Y = a.Y;
    int nseg;
    if constexpr (GROUPED) {
        for (int e = tid; e < E; e += NT) s_cnt[e] = 0;
        __syncthreads();
        for (int sl = tid; sl < m; sl += NT) {
            const int e = ids[sl];
            if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
        }
        __syncthreads();
        if (wave == 0) {
            // exclusive prefix of the per-expert segment counts, lane l
            // holding experts [l*EPL, l*EPL + EPL)
            constexpr int EPL = QMM_MOE_MAX_E / 64;
            int tl = 0;
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                if (e < E) tl += (s_cnt[e] + SL - 1) / SL;
            }
            int inc = tl;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(inc, d);
                if (lane >= d) inc += v;
            }
            int run = inc - tl;
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                if (e < E) {
                    s_sb[e] = run;
                    run += (s_cnt[e] + SL - 1) / SL;
                }
            }
            if (lane == 63) s_misc[0] = inc;
        }
        __syncthreads();
        nseg = s_misc[0];
        // rows of slots whose expert is outside [0, E) are zero: this
        // workgroup's share of the slots, a wave per slot
        const int z0 = (int)((int64_t)m * blockIdx.x / gridDim.x), z1 = (int)((int64_t)m * (blockIdx.x + 1) / gridDim.x);
        for (int sl = z0 + wave; sl < z1; sl += NW) {
            const int e = ids[sl];
            if (e < 0 || e >= E)
                for (int c = lane; c < n; c += 64) Y[(size_t)sl * n + c] = 0.0f;
        }
    } else {
        nseg = *nseg_p;
    }

    const size_t row_bytes = (size_t)NSB * 210;
    const int oq = 64 * (lq >> 1) + 16 * (lq & 1), oh = 128 + 32 * (lq >> 1) + 16 * (lq & 1);
    // A unit is ug row groups of a segment: NW (one group per wave, 256
    // rows) when there are six such units per workgroup or more, else single
    // groups (as in k_qmm4r).
    const int ug = (int64_t)nseg * ((ngr + NW - 1) / NW) >= 6 * (int64_t)gridDim.x ? NW : 1;
    const int nu = (ngr + ug - 1) / ug;  // units per segment
    int64_t u, u1;
    resident_unit_range(nseg, nu, &u, &u1);
    while (u < u1) {
        // row groups g0 .. g1 - 1 of segment seg; wave w takes g0 + w,
        // g0 + w + NW, ...
        const int seg = (int)(u / nu), c0 = (int)(u - (int64_t)seg * nu);
        const int c1 = (int)min((int64_t)nu, c0 + (u1 - u));
        u += c1 - c0;
        const int g0 = c0 * ug, g1 = min(ngr, c1 * ug);
        const int nrg = g1 - g0 > wave ? (g1 - g0 - wave + NW - 1) / NW : 0;  // this wave's groups
        __syncthreads();  // the last segment's readers of act, s_slot, s_inv are done
        int esel;
        if constexpr (GROUPED) {
            for (int e = tid; e < E; e += NT) {
                const int b = s_sb[e], ns = (s_cnt[e] + SL - 1) / SL;
                if (seg >= b && seg < b + ns) {
                    s_misc[1] = e;
                    s_misc[2] = SL * (seg - b);
                }
            }
            if (tid < SL) s_slot[tid] = -1;
            __syncthreads();
            esel = s_misc[1];
            const int rank0 = s_misc[2];
            // ascending compaction: per chunk, wave w takes ids [w*CW, (w+1)*CW)
            // in order; a rank is the running count plus the earlier waves'
            // counts plus the ballot prefix
            constexpr int CW = QMM_ID_CHUNK / NW;
            int run = 0;
            for (int q0 = 0; q0 < m && run < rank0 + SL; q0 += QMM_ID_CHUNK) {
                int cw = 0;
                for (int b = 0; b < CW; b += 64) {
                    const int sl = q0 + wave * CW + b + lane;
                    cw += __popcll(__ballot(sl < m && ids[sl] == esel));
                }
                if (lane == 0) s_wsum[wave] = cw;
                __syncthreads();
                int base = run;
                for (int v = 0; v < NW; ++v) {
                    if (v < wave) base += s_wsum[v];
                    run += s_wsum[v];
                }
                for (int b = 0; b < CW; b += 64) {
                    const int sl = q0 + wave * CW + b + lane;
                    const bool hit = sl < m && ids[sl] == esel;
                    const uint64_t bal = __ballot(hit);
                    const int rank = base + __popcll(bal & ((1ull << lane) - 1ull));
                    if (hit && rank >= rank0 && rank < rank0 + SL) s_slot[rank - rank0] = sl;
                    base += __popcll(bal);
                }
                __syncthreads();  // s_wsum is rewritten by the next chunk
            }
        } else {
            // only the segment's own entries (c << 25 | offset, k_group_tiles)
            const int so = seg_off[seg], off = so & ((1 << Q6R_SEG_SHIFT) - 1), scnt = so >> Q6R_SEG_SHIFT;
            if (tid < SL) s_slot[tid] = tid < scnt ? a.tile_slots[off + tid] : -1;
            esel = a.tile_e[off / bmt];
            __syncthreads();
        }
        esel = __builtin_amdgcn_readfirstlane(esel);

        // staging: lanes of row tid / LPR, float4 chunks l + LPR*i; the row's
        // largest magnitude over those lanes, the power of two, then
        // [hi x4 | lo x4] per chunk (rows of slots past the segment are 0)
        if (tid < SL * LPR) {  // whole waves (SL * LPR is a multiple of 64)
            const int srow = tid / LPR, l = tid % LPR;
            const int sslot = s_slot[srow];
            const size_t xrow = (size_t)(sslot >= 0 ? sslot / a.x_div : 0);
            // f32 rows: float4 chunks; q8 rows (Q8A): the chunk's four codes
            // and their block's scale, the values xq * xs formed when written
            float4 xv[Q8A ? 1 : CPL];
            uint32_t q4v[Q8A ? CPL : 1];
            float bsv[Q8A ? CPL : 1];
            float am = 0.f;
            if constexpr (Q8A) {
                const int8_t *qr = a.xq + xrow * (256 * NSB);
                const float *sr = a.xs + xrow * (8 * NSB);
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = 4 * (l + LPR * i);
                    q4v[i] = *reinterpret_cast<const uint32_t *>(qr + c);
                    bsv[i] = sr[c >> 5];
                }
                // |xq * xs| is largest where |xq| is (the rounding is monotonic)
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int q0 = abs((int)(int8_t)(q4v[i] & 0xFFu)), q1 = abs((int)(int8_t)((q4v[i] >> 8) & 0xFFu));
                    const int q2 = abs((int)(int8_t)((q4v[i] >> 16) & 0xFFu)), q3 = abs((int)(int8_t)(q4v[i] >> 24));
                    am = fmaxf(am, (float)max(max(q0, q1), max(q2, q3)) * fabsf(bsv[i]));
                }
            } else {
                const float *xr = a.x + xrow * (256 * NSB);
#pragma unroll
                for (int i = 0; i < CPL; ++i) xv[i] = *reinterpret_cast<const float4 *>(xr + 4 * (l + LPR * i));
#pragma unroll
                for (int i = 0; i < CPL; ++i)
                    am = fmaxf(am, fmaxf(fmaxf(fabsf(xv[i].x), fabsf(xv[i].y)), fmaxf(fabsf(xv[i].z), fabsf(xv[i].w))));
            }
            auto chunk = [&](int i) -> float4 {
                if constexpr (Q8A) {
                    const uint32_t q = q4v[i];
                    const float bs = bsv[i];
                    return make_float4((float)(int8_t)(q & 0xFFu) * bs, (float)(int8_t)((q >> 8) & 0xFFu) * bs,
                                       (float)(int8_t)((q >> 16) & 0xFFu) * bs, (float)(int8_t)(q >> 24) * bs);
                } else {
                    return xv[i];
                }
            };
#pragma unroll
            for (int d = 1; d < LPR; d <<= 1) am = fmaxf(am, __shfl_xor(am, d));
            const int e = am > 0.f ? ((int)((__float_as_uint(am) >> 23) & 0xFF) - 127) : 0;
            const int ee = max(min(14 - e, 126), -126);  // 2^ee and 2^-ee are normal
            const float sc = sslot >= 0 ? __uint_as_float((uint32_t)(ee + 127) << 23) : 0.f;
            const float inv = __uint_as_float((uint32_t)(127 - ee) << 23);
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const float4 v = chunk(i);
                const float y0 = v.x * sc, y1 = v.y * sc, y2 = v.z * sc, y3 = v.w * sc;
                const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1, h2v = (_Float16)y2, h3 = (_Float16)y3;
                const h4 hi = {h0, h1, h2v, h3};
                const h4 lo = {(_Float16)(y0 - (float)h0), (_Float16)(y1 - (float)h1), (_Float16)(y2 - (float)h2v),
                               (_Float16)(y3 - (float)h3)};
                const uint2 hb = __builtin_bit_cast(uint2, hi), lb = __builtin_bit_cast(uint2, lo);
                *reinterpret_cast<uint4 *>(act + srow * PITCH + 16 * (l + LPR * i)) = make_uint4(hb.x, hb.y, lb.x, lb.y);
            }
            if (l == 0) s_inv[srow] = inv;
        }
        __syncthreads();

        if (nrg == 0) continue;  // wave-uniform; no barrier follows before the next segment's
        // the weight ring: step j of this wave is superblock j % NSB of its
        // rows in group g0 + wave + NW * (j / NSB)
        const uint8_t *__restrict__ wb = a.w + (size_t)esel * n * row_bytes;
        auto load_step = [&](Q6rRaw<FPW> &R, int j) {
            const int i = j / NSB, s = j - i * NSB;
#pragma unroll
            for (int f = 0; f < FPW; ++f) {
                const int row = min(16 * FPW * (g0 + wave + NW * i) + 16 * f + li, n - 1);
                const uint8_t *p = wb + (size_t)row * row_bytes + 210 * s;
                R.ql0[f] = ld16(p + oq);
                R.ql1[f] = ld16(p + oq + 32);
                R.qh[f] = ld16(p + oh);
                R.sc[f] = ld16(p + 192);
                R.d[f] = ld2(p + 208);
            }
        };
        const int J = nrg * NSB;  // steps of this wave
        Q6rRaw<FPW> R[D];
#pragma unroll
        for (int q = 0; q < D; ++q) {
            load_step(R[q], min(q, J - 1));
            __builtin_amdgcn_sched_barrier(0);
        }

        // the wave's steps with NF 16-slot fragments (uniform per segment)
        auto run = [&](auto NFc) {
            constexpr int NF = decltype(NFc)::value;
            v4f out[FPW][NF];
            auto compute = [&](const Q6rRaw<FPW> &Rs, int s) {
                const uint8_t *abase = act + li * PITCH + 16 * lq + 1024 * s;
                float dd[FPW];
                uint32_t q0[FPW][4], q1[FPW][4], qh[FPW][4];
#pragma unroll
                for (int f = 0; f < FPW; ++f) {
                    dd[f] = h2f(Rs.d[f]);
                    const uint4 a0 = rows_transpose(Rs.ql0[f]), a1 = rows_transpose(Rs.ql1[f]),
                                ah = rows_transpose(Rs.qh[f]);
                    q0[f][0] = a0.x; q0[f][1] = a0.y; q0[f][2] = a0.z; q0[f][3] = a0.w;
                    q1[f][0] = a1.x; q1[f][1] = a1.y; q1[f][2] = a1.z; q1[f][3] = a1.w;
                    qh[f][0] = ah.x; qh[f][1] = ah.y; qh[f][2] = ah.z; qh[f][3] = ah.w;
                }
                // Sub-blocks in the order m = 4 (2 hh + lh) + g (one decode per
                // (hh, lh) group). The fragments of sub-block m + 1 are read
                // from LDS while m is on the matrix cores, and the products of
                // m are added while those of m + 1 are (Tp, cp: the pending ones).
                auto sub_of = [](int mm) { return 8 * ((mm >> 3) & 1) + 2 * (mm & 3) + ((mm >> 2) & 1); };
                auto read_a = [&](uint4(&A)[NF], int mm) {
#pragma unroll
                    for (int t = 0; t < NF; ++t)
                        A[t] = *reinterpret_cast<const uint4 *>(abase + 16 * t * PITCH + 64 * sub_of(mm));
                };
                v4f Tp[FPW][NF];
                float cp[FPW];
                uint4 An[NF];
                read_a(An, 0);
                uint2 B[FPW][4];
#pragma unroll
                for (int mm = 0; mm < 16; ++mm) {
                    const int hh = mm >> 3, lh = (mm >> 2) & 1, g = mm & 3, sub = sub_of(mm);
                    if (g == 0) {
#pragma unroll
                        for (int f = 0; f < FPW; ++f) {
                            uint32_t c[4];
                            q6_run_codes(q0[f][2 * hh + lh], q1[f][2 * hh + lh], qh[f][2 * hh + lh], c);
#pragma unroll
                            for (int gg = 0; gg < 4; ++gg) B[f][gg] = q6x4_to_f16(c[gg]);
                        }
                    }
                    uint4 A[NF];
#pragma unroll
                    for (int t = 0; t < NF; ++t) A[t] = An[t];
                    if (mm + 1 < 16) read_a(An, mm + 1);
                    v4f Tn[FPW][NF];
                    float cn[FPW];
#pragma unroll
                    for (int f = 0; f < FPW; ++f) {
                        const uint4 s4 = Rs.sc[f];
                        const uint32_t sw =
                            (sub >> 2) == 0 ? s4.x : (sub >> 2) == 1 ? s4.y : (sub >> 2) == 2 ? s4.z : s4.w;
                        cn[f] = dd[f] * (float)(int8_t)((sw >> (8 * (sub & 3))) & 0xFFu);
                        const h4 bw = __builtin_bit_cast(h4, B[f][g]);
#pragma unroll
                        for (int t = 0; t < NF; ++t) {
                            v4f T = __builtin_amdgcn_mfma_f32_16x16x16f16(
                                __builtin_bit_cast(h4, make_uint2(A[t].x, A[t].y)), bw, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                            Tn[f][t] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                                __builtin_bit_cast(h4, make_uint2(A[t].z, A[t].w)), bw, T, 0, 0, 0);
                        }
                    }
                    if (mm > 0) {
#pragma unroll
                        for (int f = 0; f < FPW; ++f)
#pragma unroll
                            for (int t = 0; t < NF; ++t) out[f][t] = cp[f] * Tp[f][t] + out[f][t];
                    }
                    // the additions stay here: left to itself the compiler
                    // issues every product of the step first and keeps them in
                    // scratch memory
#pragma unroll
                    for (int f = 0; f < FPW; ++f)
#pragma unroll
                        for (int t = 0; t < NF; ++t) asm volatile("" : "+v"(out[f][t]));
#pragma unroll
                    for (int f = 0; f < FPW; ++f) {
                        cp[f] = cn[f];
#pragma unroll
                        for (int t = 0; t < NF; ++t) Tp[f][t] = Tn[f][t];
                    }
                }
#pragma unroll
                for (int f = 0; f < FPW; ++f)
#pragma unroll
                    for (int t = 0; t < NF; ++t) out[f][t] = cp[f] * Tp[f][t] + out[f][t];
            };
            for (int j0 = 0; j0 < J; j0 += D) {
#pragma unroll
                for (int q = 0; q < D; ++q) {
                    const int j = j0 + q, i = j / NSB, s = j - i * NSB;
                    if (s == 0) {
#pragma unroll
                        for (int f = 0; f < FPW; ++f)
#pragma unroll
                            for (int t = 0; t < NF; ++t) out[f][t] = (v4f){0.f, 0.f, 0.f, 0.f};
                    }
                    compute(R[q], s);
                    __builtin_amdgcn_sched_barrier(0);
                    load_step(R[q], min(j + D, J - 1));
                    __builtin_amdgcn_sched_barrier(0);
                    if (s == NSB - 1 && i < nrg) {
                        // lane: slots 16t + 4lq + r of weight row `row`
#pragma unroll
                        for (int f = 0; f < FPW; ++f) {
                            const int row = 16 * FPW * (g0 + wave + NW * i) + 16 * f + li;
                            if (row >= n) continue;
#pragma unroll
                            for (int t = 0; t < NF; ++t)
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int ts = 16 * t + 4 * lq + r, slot = s_slot[ts];
                                    if (slot >= 0) Y[(size_t)slot * n + row] = out[f][t][r] * s_inv[ts];
                                }
                        }
                    }
                }
            }
        };
        if constexpr (SL == 48) {
            if (s_slot[32] >= 0) run(std::integral_constant<int, 3>{});
            else if (s_slot[16] >= 0) run(std::integral_constant<int, 2>{});
            else run(std::integral_constant<int, 1>{});
        } else {
            if (s_slot[16] >= 0) run(std::integral_constant<int, 2>{});
            else run(std::integral_constant<int, 1>{});
        }
    }
}

// Slots per k_qmm6r segment: 48 (three 16-slot fragments on one weight
// decode) where the experts average more than 16 slots and 48 staged rows fit
// LDS (k <= 768), else 32.
int q6r_segment_slots(int64_t nslots, int64_t E, int64_t k) { return k <= 768 && nslots > 16 * E ? 48 : 32; }

// k_qmm6r, one workgroup per CU (k <= 1024): GROUPED derives its segments of
// sl slots from ids, otherwise they come from the tile table (nseg, seg_off,
// listed for sl-slot segments).
template <bool GROUPED, bool Q8A = false>
void launch_q6r(const Qmm6Args &a, const int *nseg, const int *seg_off, int bmt, int sl, hipStream_t s) {
    static thread_local int c_dev = -1, c_cus = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != c_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
        c_dev = dev;
        c_cus = cus;
    }
    const dim3 grid((unsigned)c_cus), block(1024 / Q6R_FPW);
    if (sl == 48 && a.k <= 768) {
        switch (a.k / 256) {
            case 1: hipLaunchKernelGGL((k_qmm6r<1, GROUPED, Q6R_FPW, 48, Q8A>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
            case 2: hipLaunchKernelGGL((k_qmm6r<2, GROUPED, Q6R_FPW, 48, Q8A>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
            default: hipLaunchKernelGGL((k_qmm6r<3, GROUPED, Q6R_FPW, 48, Q8A>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        }
        return;
    }
    switch (a.k / 256) {
        case 1: hipLaunchKernelGGL((k_qmm6r<1, GROUPED, Q6R_FPW, 32, Q8A>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 2: hipLaunchKernelGGL((k_qmm6r<2, GROUPED, Q6R_FPW, 32, Q8A>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 3: hipLaunchKernelGGL((k_qmm6r<3, GROUPED, Q6R_FPW, 32, Q8A>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        default: hipLaunchKernelGGL((k_qmm6r<4, GROUPED, Q6R_FPW, 32, Q8A>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
    }
}

// ============================================ Q4_K GEMM, resident activations
// The expert-grouped Q4_K x q8 products of the MoE prefill (the layer's
// paired gate/up projection, and moe_qmm_q4k) with the work split of
// k_qmm6r: a workgroup of 16 waves stages the q8 rows of up to 32 slots of
// one expert once (codes as exact f16, rows 2k + 16 bytes apart so that the
// 16-byte fragment reads of sixteen consecutive rows hit distinct banks; xs
// and xsum per block, rows 4 floats longer than a row's blocks), and each
// wave then streams its own 16 weight rows superblock by superblock, with a
// ring of raw-code register sets in flight and no barrier. The matrix roles
// are those of k_qmm2_q4k: the weight rows are the A operand (per 32-value
// block a lane decodes the 8 codes at its fragment position as f16 sc*q,
// exact), the slots the B operand. One v_mfma_f32_16x16x32_f16 per 16-slot
// fragment and block gives the block's integer dot T, the VALU adds xs*T
// into a per-superblock accumulator, and d times that accumulator plus the
// min term (v_mfma_f32_16x16x4_f32 over four blocks) go into the output tile
// once per superblock.
// PAIR (the layer's gate/up): rows 0-7 of a wave's fragment are gate rows
// c..c+7 and rows 8-15 the up rows of the same h columns, so lane l < 32 and
// lane l + 32 hold the gate and up dots of the same outputs. They exchange
// them with v_permlane32_swap, and each lane stores h = silu(gate) * up for
// one of the two slot fragments.
#ifndef Q4R_RING
#define Q4R_RING 1
#endif
constexpr int Q4R_SLOTS = 32;   // slots staged per workgroup (one table segment)

// Raw codes of one step (a superblock of the wave's 16 rows): the lane's
// row header (d, dmin, 12 scale bytes) and code bytes 8lq.. of each of the
// four 32-byte pairs (values 8lq.. of the pair's two sub-blocks).
struct Q4rRaw {
    uint4 hdr;
    uint2 qc[4];
};

// Work: units of one segment (up to 32 slots of one expert) by NW fragments
// of CW output columns; each workgroup takes an equal run of consecutive
// units and stages once per segment of its run (one or two). GROUPED: the
// segments come from ids (per-expert counts, a ballot compaction; the
// workgroups also zero the rows of slots whose expert is outside [0, E)),
// otherwise from the layer's tile table (nseg, seg_off).
template <int NSB, bool PAIR, bool GROUPED>
__global__ __launch_bounds__(1024) void k_qmm4r(const QmmArgs a, const int *__restrict__ nseg_p,
                                                const int *__restrict__ seg_off, int bmt) {
    static_assert(NSB >= 1 && NSB <= Q4R_MAX_NSB, "k <= 2048");
    constexpr int NW = 16, NT = 64 * NW;
    constexpr int KV = 256 * NSB, KB = 8 * NSB;  // values and q8 blocks per row
    constexpr int PITCH = 2 * KV + 16;            // bytes per staged row
    constexpr int XP = KB + 4;                    // floats per staged xs / xsum row
    constexpr int D = Q4R_RING;                   // steps in flight per wave
    constexpr int CW = PAIR ? 8 : 16;             // output columns of a wave's fragment
    constexpr int LPR = NT / Q4R_SLOTS;           // staging lanes per row
    __shared__ __attribute__((aligned(16))) uint8_t act[Q4R_SLOTS * PITCH];
    __shared__ __attribute__((aligned(16))) float sxs[Q4R_SLOTS * XP];
    __shared__ __attribute__((aligned(16))) float sxm[Q4R_SLOTS * XP];
    __shared__ int s_slot[Q4R_SLOTS];
    __shared__ int s_misc[4], s_wsum[NW];
    __shared__ int s_cnt[GROUPED ? QMM_MOE_MAX_E : 1], s_sb[GROUPED ? QMM_MOE_MAX_E : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lq = lane >> 4;
    const int n = a.n, m = a.m, E = a.E;
    const int ncg = (n + CW - 1) / CW;  // column groups (one wave fragment each) of a segment
    const int32_t *__restrict__ ids = a.ids;
    float *__restrict__ Y = a.Y;
    int nseg;
    if constexpr (GROUPED) {
        for (int e = tid; e < E; e += NT) s_cnt[e] = 0;
        __syncthreads();
        for (int sl = tid; sl < m; sl += NT) {
            const int e = ids[sl];
            if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
        }
        __syncthreads();
        if (wave == 0) {
            // exclusive prefix of the per-expert segment counts, lane l
            // holding experts [l*EPL, l*EPL + EPL)
            constexpr int EPL = QMM_MOE_MAX_E / 64;
            int tl = 0;
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                if (e < E) tl += (s_cnt[e] + Q4R_SLOTS - 1) / Q4R_SLOTS;
            }
            int inc = tl;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(inc, d);
                if (lane >= d) inc += v;
            }
            int run = inc - tl;
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                if (e < E) {
                    s_sb[e] = run;
                    run += (s_cnt[e] + Q4R_SLOTS - 1) / Q4R_SLOTS;
                }
            }
            if (lane == 63) s_misc[0] = inc;
        }
        __syncthreads();
        nseg = s_misc[0];
        // rows of slots whose expert is outside [0, E) are zero: this
        // workgroup's share of the slots, a wave per slot
        const int z0 = (int)((int64_t)m * blockIdx.x / gridDim.x), z1 = (int)((int64_t)m * (blockIdx.x + 1) / gridDim.x);
        for (int sl = z0 + wave; sl < z1; sl += NW) {
            const int e = ids[sl];
            if (e < 0 || e >= E)
                for (int c = lane; c < n; c += 64) Y[(size_t)sl * n + c] = 0.0f;
        }
    } else {
        nseg = *nseg_p;
    }

    const size_t row_bytes = (size_t)NSB * 144;
    // A unit is ug column groups of a segment: NW (one group per wave) when
    // there are six such units per workgroup or more (the waves of a
    // workgroup then take equal shares of each segment), else single groups
    // (the workgroups' shares stay within a group of each other).
    const int ug = (int64_t)nseg * ((ncg + NW - 1) / NW) >= 6 * (int64_t)gridDim.x ? NW : 1;
    const int nu = (ncg + ug - 1) / ug;  // units per segment
    int64_t u, u1;
    resident_unit_range(nseg, nu, &u, &u1);
    while (u < u1) {
        // column groups g0 .. g1 - 1 of segment seg; wave w takes g0 + w,
        // g0 + w + NW, ...
        const int seg = (int)(u / nu), c0 = (int)(u - (int64_t)seg * nu);
        const int c1 = (int)min((int64_t)nu, c0 + (u1 - u));
        u += c1 - c0;
        const int g0 = c0 * ug, g1 = min(ncg, c1 * ug);
        const int nrg = g1 - g0 > wave ? (g1 - g0 - wave + NW - 1) / NW : 0;  // this wave's groups
        __syncthreads();  // the last segment's readers of act, sxs, sxm, s_slot are done
        int esel;
        if constexpr (GROUPED) {
            for (int e = tid; e < E; e += NT) {
                const int b = s_sb[e], ns = (s_cnt[e] + Q4R_SLOTS - 1) / Q4R_SLOTS;
                if (seg >= b && seg < b + ns) {
                    s_misc[1] = e;
                    s_misc[2] = Q4R_SLOTS * (seg - b);
                }
            }
            if (tid < Q4R_SLOTS) s_slot[tid] = -1;
            __syncthreads();
            esel = s_misc[1];
            const int rank0 = s_misc[2];
            // ascending compaction: per chunk, wave w takes ids [w*CWI, (w+1)*CWI)
            // in order; a rank is the running count plus the earlier waves'
            // counts plus the ballot prefix
            constexpr int CWI = QMM_ID_CHUNK / NW;
            int run = 0;
            for (int q0 = 0; q0 < m && run < rank0 + Q4R_SLOTS; q0 += QMM_ID_CHUNK) {
                int cw = 0;
                for (int b = 0; b < CWI; b += 64) {
                    const int sl = q0 + wave * CWI + b + lane;
                    cw += __popcll(__ballot(sl < m && ids[sl] == esel));
                }
                if (lane == 0) s_wsum[wave] = cw;
                __syncthreads();
                int base = run;
                for (int v = 0; v < NW; ++v) {
                    if (v < wave) base += s_wsum[v];
                    run += s_wsum[v];
                }
                for (int b = 0; b < CWI; b += 64) {
                    const int sl = q0 + wave * CWI + b + lane;
                    const bool hit = sl < m && ids[sl] == esel;
                    const uint64_t bal = __ballot(hit);
                    const int rank = base + __popcll(bal & ((1ull << lane) - 1ull));
                    if (hit && rank >= rank0 && rank < rank0 + Q4R_SLOTS) s_slot[rank - rank0] = sl;
                    base += __popcll(bal);
                }
                __syncthreads();  // s_wsum is rewritten by the next chunk
            }
        } else {
            // only the segment's own entries (count << 25 | offset, k_group_tiles)
            const int so = seg_off[seg], off = so & ((1 << Q6R_SEG_SHIFT) - 1), scnt = so >> Q6R_SEG_SHIFT;
            if (tid < Q4R_SLOTS) s_slot[tid] = tid < scnt ? a.tile_slots[off + tid] : -1;
            esel = a.tile_e[off / bmt];
            __syncthreads();
        }
        esel = __builtin_amdgcn_readfirstlane(esel);

        // staging: lanes of row tid / LPR take its 8-code chunks l + LPR*i
        // (16 f16 bytes each) and its blocks l, l + LPR, ... (rows of slots
        // past the segment are zero)
        {
            const int srow = tid / LPR, l = tid % LPR;
            const int sslot = s_slot[srow];
            const size_t xrow = (size_t)(sslot >= 0 ? sslot / a.x_div : 0);
            const int8_t *xr = a.xq + xrow * KV;
            uint2 v[NSB];
#pragma unroll
            for (int i = 0; i < NSB; ++i) v[i] = *reinterpret_cast<const uint2 *>(xr + 8 * (l + LPR * i));
            for (int b = l; b < KB; b += LPR) {
                const float s0 = a.xs[xrow * KB + b], s1 = a.xsum[xrow * KB + b];
                sxs[srow * XP + b] = sslot >= 0 ? s0 : 0.f;
                sxm[srow * XP + b] = sslot >= 0 ? s1 : 0.f;
            }
#pragma unroll
            for (int i = 0; i < NSB; ++i) {
                const uint2 w = sslot >= 0 ? v[i] : make_uint2(0u, 0u);
                const uint2 h0 = i8x4_to_f16(w.x), h1 = i8x4_to_f16(w.y);
                *reinterpret_cast<uint4 *>(act + srow * PITCH + 16 * (l + LPR * i)) = make_uint4(h0.x, h0.y, h1.x, h1.y);
            }
        }
        __syncthreads();

        if (nrg == 0) continue;  // wave-uniform; no barrier follows before the next segment's
        // the weight ring: step j of this wave is superblock j % NSB of its
        // fragment in group g0 + wave + NW * (j / NSB) (rows past n read row
        // n - 1, their outputs are not stored)
        const uint8_t *__restrict__ wl =
            (PAIR && li >= 8 ? a.w2 : a.w) + (size_t)esel * n * row_bytes;  // this lane's bank
        const int rl = PAIR ? (li & 7) : li;                                 // its row in the fragment
        auto load_step = [&](Q4rRaw &R, int j) {
            const int i = j / NSB, s = j - i * NSB;
            const int row = min(CW * (g0 + wave + NW * i) + rl, n - 1);
            const uint8_t *p = wl + (size_t)row * row_bytes + 144 * s;
            R.hdr = ld16(p);
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) R.qc[pp] = *reinterpret_cast<const uint2 *>(p + 16 + 32 * pp + 8 * lq);
        };
        const int J = nrg * NSB;  // steps of this wave
        Q4rRaw R[D];
#pragma unroll
        for (int q = 0; q < D; ++q) {
            load_step(R[q], min(q, J - 1));
            __builtin_amdgcn_sched_barrier(0);
        }

        // the wave's steps with NF 16-slot fragments (uniform per segment)
        auto run = [&](auto NFc) {
            constexpr int NF = decltype(NFc)::value;
            v4f out[NF];
            auto compute = [&](const Q4rRaw &Rs, int s) {
                const float dl = h2f(Rs.hdr.x), dml = h2f(Rs.hdr.x >> 16);
                uint32_t sc2[4], mn2[4];
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) q4k_scales(Rs.hdr.y, Rs.hdr.z, Rs.hdr.w, pp, &sc2[pp], &mn2[pp]);
                // d of the lane's output rows 4lq + r; the min-term operand of
                // row li, blocks 4i + lq (bit selects rather than an indexed
                // array, which the compiler would place in scratch)
                float dout[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) dout[r] = __shfl(dl, 4 * lq + r);
                float amn[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t lo = mn2[2 * i], hi = mn2[2 * i + 1];
                    const uint32_t pr = lo ^ ((lo ^ hi) & (0u - (uint32_t)(lq >> 1)));
                    amn[i] = -dml * (float)((pr >> (8 * (lq & 1))) & 0xFFu);
                }
                // xs of the lane's slots (column li of each fragment), four
                // blocks at a time. Software-pipelined over the blocks: the
                // fragments of block jb + 1 are read from LDS while jb is
                // decoded, and the products of jb - 1 are added after the
                // matrix instructions of jb are issued (Tp: the pending ones).
                const float *xsp = &sxs[li * XP + 8 * s];
                const uint8_t *abase = act + li * PITCH + 512 * s + 16 * lq;
                // per pair of blocks, the two sub-block scales as an f16 pair
                // (exact: the halves 1024 + sc, minus 1024), and from them
                // the multipliers and offsets of the code conversion. The
                // high nibbles stay in place (16q), which the odd block's
                // pair absorbs: (1024 + 16q)*(sc/16) - 64*sc = q*sc.
                h2 mulp[4], addp[4];
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const h2 scp = as_h2(__builtin_amdgcn_perm(0x64646464u, sc2[pp], 0x04010400u)) + splat(-1024.0f);
                    mulp[pp] = scp * h2{(_Float16)1.0f, (_Float16)0.0625f};
                    addp[pp] = scp * h2{(_Float16)-1024.0f, (_Float16)-64.0f};
                }
                v4f acc[NF], xv[NF], Tp[NF];
                h8 bn[NF];
#pragma unroll
                for (int t = 0; t < NF; ++t) bn[t] = *reinterpret_cast<const h8 *>(abase + 16 * t * PITCH);
#pragma unroll
                for (int jb = 0; jb < 8; ++jb) {
                    h8 bf[NF];
#pragma unroll
                    for (int t = 0; t < NF; ++t) bf[t] = bn[t];
                    if (jb + 1 < 8) {
#pragma unroll
                        for (int t = 0; t < NF; ++t)
                            bn[t] = *reinterpret_cast<const h8 *>(abase + 16 * t * PITCH + 64 * (jb + 1));
                    }
                    // the block's multiplier and offset, one half of its pair's
                    const h2 mul = (jb & 1) ? h2{mulp[jb / 2].y, mulp[jb / 2].y} : h2{mulp[jb / 2].x, mulp[jb / 2].x};
                    const h2 add = (jb & 1) ? h2{addp[jb / 2].y, addp[jb / 2].y} : h2{addp[jb / 2].x, addp[jb / 2].x};
                    const uint2 cw = Rs.qc[jb / 2];
                    const uint32_t msk = (jb & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
                    const uint2 v0 = q4x4_to_f16(cw.x & msk, mul, add);
                    const uint2 v1 = q4x4_to_f16(cw.y & msk, mul, add);
                    const h8 af = __builtin_bit_cast(h8, make_uint4(v0.x, v0.y, v1.x, v1.y));
                    v4f Tn[NF];
#pragma unroll
                    for (int t = 0; t < NF; ++t)
                        Tn[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[t], (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if (jb > 0) {
#pragma unroll
                        for (int t = 0; t < NF; ++t)
                            acc[t] = jb == 1 ? xv[t][0] * Tp[t] : xv[t][(jb - 1) & 3] * Tp[t] + acc[t];
                    }
                    if ((jb & 3) == 0) {
#pragma unroll
                        for (int t = 0; t < NF; ++t) xv[t] = *reinterpret_cast<const v4f *>(xsp + 16 * t * XP + jb);
                    }
                    // the additions stay here: left to itself the compiler
                    // issues every product of the step first and spills them
#pragma unroll
                    for (int t = 0; t < NF; ++t) {
                        if (jb > 0) asm volatile("" : "+v"(acc[t]));
                        Tp[t] = Tn[t];
                    }
                }
#pragma unroll
                for (int t = 0; t < NF; ++t) acc[t] = xv[t][3] * Tp[t] + acc[t];
#pragma unroll
                for (int t = 0; t < NF; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) out[t][r] = dout[r] * acc[t][r] + out[t][r];
                // the min term: xsum of the lane's slot column, blocks 4i + lq
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int t = 0; t < NF; ++t)
                        out[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            amn[i], sxm[(16 * t + li) * XP + 8 * s + 4 * i + lq], out[t], 0, 0, 0);
            };
            const bool vec = !PAIR && (((uintptr_t)Y & 15) == 0) && (n & 3) == 0;
            for (int j0 = 0; j0 < J; j0 += D) {
#pragma unroll
                for (int q = 0; q < D; ++q) {
                    const int j = j0 + q, i = j / NSB, s = j - i * NSB;
                    if (s == 0) {
#pragma unroll
                        for (int t = 0; t < NF; ++t) out[t] = (v4f){0.f, 0.f, 0.f, 0.f};
                    }
                    compute(R[q], s);
                    __builtin_amdgcn_sched_barrier(0);
                    load_step(R[q], min(j + D, J - 1));
                    __builtin_amdgcn_sched_barrier(0);
                    if (s == NSB - 1 && i < nrg) {
                        const int cg = g0 + wave + NW * i;  // the wave's column group
                        if constexpr (PAIR) {
                            // lanes l and l + 32: gate and up of h columns
                            // CW*cg + 4(lq & 1) + r, slot column li; lanes
                            // below 32 store fragment 0, the others fragment 1
                            float hv[NF][4];
#pragma unroll
                            for (int t = 0; t < NF; ++t)
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const float x = out[t][r];
                                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                                    const float p = __uint_as_float(lane < 32 ? sw[1] : sw[0]);
                                    const float g = lane < 32 ? x : p, up = lane < 32 ? p : x;
                                    hv[t][r] = silu(g) * up;
                                }
                            const int uo = lane >> 5;
                            const int col = CW * cg + 4 * (lq & 1);
                            if (uo < NF) {
                                const int slot = s_slot[16 * uo + li];
                                float4 o;
                                o.x = uo ? hv[NF - 1][0] : hv[0][0];
                                o.y = uo ? hv[NF - 1][1] : hv[0][1];
                                o.z = uo ? hv[NF - 1][2] : hv[0][2];
                                o.w = uo ? hv[NF - 1][3] : hv[0][3];
                                if (slot >= 0 && col < n) *reinterpret_cast<float4 *>(Y + (size_t)slot * n + col) = o;
                            }
                        } else {
                            const int col = CW * cg + 4 * lq;
#pragma unroll
                            for (int t = 0; t < NF; ++t) {
                                const int slot = s_slot[16 * t + li];
                                if (slot < 0) continue;
                                float *dst = Y + (size_t)slot * n + col;
                                if (vec && col + 3 < n) {
                                    *reinterpret_cast<v4f *>(dst) = out[t];
                                } else {
#pragma unroll
                                    for (int r = 0; r < 4; ++r)
                                        if (col + r < n) dst[r] = out[t][r];
                                }
                            }
                        }
                    }
                }
            }
        };
        if (s_slot[16] >= 0) run(std::integral_constant<int, 2>{});
        else run(std::integral_constant<int, 1>{});
    }
}

// k_qmm4r, one workgroup per CU (k <= 2048): GROUPED derives its 32-slot
// segments from ids, otherwise they come from the tile table (nseg,
// seg_off, tiles of bmt slots).
template <bool PAIR, bool GROUPED>
void launch_q4r(const QmmArgs &a, const int *nseg, const int *seg_off, int bmt, hipStream_t s) {
    static thread_local int c_dev = -1, c_cus = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != c_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
        c_dev = dev;
        c_cus = cus;
    }
    const dim3 grid((unsigned)c_cus), block(1024);
    switch (a.k / 256) {
        case 1: hipLaunchKernelGGL((k_qmm4r<1, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 2: hipLaunchKernelGGL((k_qmm4r<2, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 3: hipLaunchKernelGGL((k_qmm4r<3, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 4: hipLaunchKernelGGL((k_qmm4r<4, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 5: hipLaunchKernelGGL((k_qmm4r<5, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 6: hipLaunchKernelGGL((k_qmm4r<6, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        case 7: hipLaunchKernelGGL((k_qmm4r<7, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
        default: hipLaunchKernelGGL((k_qmm4r<8, PAIR, GROUPED>), grid, block, 0, s, a, nseg, seg_off, bmt); break;
    }
}

int check_q6k_shape(int64_t n, int64_t k) {
    if (n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (n > (1 << 24) || k > (1 << 20)) return QMV_EUNSUPPORTED;
    return QMV_OK;
}

}  // namespace

extern "C" int qmm_q6k(const void *w, const int8_t *xq, const float *xs, float *y, int64_t m, int64_t n, int64_t k,
                       qmv_stream_t stream) {
    if (!w || !xq || !xs || !y || m < 1) return QMV_EINVAL;
    int rc = check_q6k_shape(n, k);
    if (rc != QMV_OK) return rc;
    if (m > (1 << 24) || m * k > ((int64_t)1 << 34)) return QMV_EUNSUPPORTED;
    if (!aligned(w, 2) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(y, 4)) return QMV_EALIGN;
    Qmm6Args a{static_cast<const uint8_t *>(w), xq, xs, nullptr, y, (int)m, (int)n, (int)k, nullptr, 1, 1};
    const dim3 grid((unsigned)div_up(n, 128), (unsigned)div_up(m, 64));
    hipLaunchKernelGGL((k_qmm_q6k<QMM6_DENSE, ACT_Q8, false>), grid, dim3(512), 0, (hipStream_t)stream, a);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

namespace {
int check_moe6(const void *bank, const int32_t *ids, float *y, int64_t x_div, int64_t nslots, int64_t n, int64_t k,
               int64_t E) {
    if (!bank || !ids || !y || x_div < 1 || nslots < 1 || E < 1) return QMV_EINVAL;
    int rc = check_q6k_shape(n, k);
    if (rc != QMV_OK) return rc;
    if (E > QMM_MOE_MAX_E || nslots > QMM_MOE_MAX_SLOTS || E * n * (k / 256) * 210 > ((int64_t)1 << 40))
        return QMV_EUNSUPPORTED;
    if (!aligned(bank, 2) || !aligned(ids, 4) || !aligned(y, 4)) return QMV_EALIGN;
    return QMV_OK;
}
}  // namespace

extern "C" int moe_qmm_q6k(const void *bank, const int8_t *xq, const float *xs, int64_t x_div, const int32_t *ids,
                           float *y, int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream) {
    if (!xq || !xs) return QMV_EINVAL;
    int rc = check_moe6(bank, ids, y, x_div, nslots, n, k, E);
    if (rc != QMV_OK) return rc;
    if (!aligned(xq, 16) || !aligned(xs, 4)) return QMV_EALIGN;
    Qmm6Args a{static_cast<const uint8_t *>(bank), xq, xs, nullptr, y, (int)nslots, (int)n, (int)k, ids, (int)E,
               (int)x_div};
    if (QMV_Q6R && k <= 256 * Q6R_MAX_NSB) {
        // the f32 form's resident GEMM, staging each value as xq * xs
        // (48-slot segments where they apply, as for f32: at 4,096 slots over
        // 128 experts, k = 768, 85 us against 108 us with 32-slot ones)
        launch_q6r<true, true>(a, nullptr, nullptr, Q6R_SLOTS, q6r_segment_slots(nslots, E, k), (hipStream_t)stream);
    } else {
        const dim3 grid((unsigned)div_up(n, QMM6_MOE_BN),
                        (unsigned)(div_up(nslots, QMM6_MOE_BM) + std::min(E, nslots)));
        hipLaunchKernelGGL((k_qmm_q6k<QMM6_MOE, ACT_Q8, true>), grid, dim3(QMM6_MOE_NT), 0, (hipStream_t)stream, a);
    }
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

extern "C" int moe_qmm_q6k_f32(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                               int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream) {
    if (!x) return QMV_EINVAL;
    int rc = check_moe6(bank, ids, y, x_div, nslots, n, k, E);
    if (rc != QMV_OK) return rc;
    if (!aligned(x, 16)) return QMV_EALIGN;
    Qmm6Args a{static_cast<const uint8_t *>(bank), nullptr, nullptr, x, y, (int)nslots, (int)n, (int)k, ids, (int)E,
               (int)x_div};
    if (QMV_Q6R && k <= 256 * Q6R_MAX_NSB) {
        // segments grouped in the kernel, the activation resident in LDS
        launch_q6r<true>(a, nullptr, nullptr, Q6R_SLOTS, q6r_segment_slots(nslots, E, k), (hipStream_t)stream);
    } else {
        const dim3 grid((unsigned)div_up(n, QMM6_MOEF_BN),
                        (unsigned)(div_up(nslots, QMM6_MOEF_BM) + std::min(E, nslots)));
        hipLaunchKernelGGL((k_qmm_q6k<QMM6_MOEF, ACT_F32, true, false, QMM6_MOEF_KP>), grid, dim3(QMM6_MOEF_NT), 0,
                           (hipStream_t)stream, a);
    }
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

// ============================================================ prefill layer
// The MoE layer at m > 1 (the prefill twin of moe_ffn_q4k_q6k): the token
// activations are quantized once (quantize_act_q8), the slots are grouped
// by expert once into a table of 32-slot tiles shared by both projections,
// gate and up run as one paired expert-indexed Q4_K GEMM whose epilogue
// writes h = silu(gate) * up per slot, the down projection is the f32-
// activation Q6_K GEMM on h, and the weighted combine sums each token's
// slots in slot order.
namespace {

// Slots per tile in the layer (both projections share the tile table): 48
// from QMV_PF48_LO to QMV_PF48_HI slots per expert on average, else 32 below
// a mean of 32 and 64 above (measured: the 64-slot eight-wave tiles were
// faster than 32-slot ones from 32 slots per expert up, the 32-slot ones at
// 8).
#ifndef QMV_PF48_LO
#define QMV_PF48_LO 24
#define QMV_PF48_HI 40
#endif

// One workgroup builds the tile table: per-expert slot counts (LDS
// atomics), an exclusive prefix of the per-expert tile counts, the tile ->
// expert map with the pad of each expert's last tile set to -1, then every
// valid slot is placed in its expert's tiles. The order of an expert's slots
// within its tiles follows the atomics and may differ between runs; every
// output row depends only on its own slot, so the results do not. It also
// lists the 32-slot segments of the table (and, given nseg48, the 48-slot
// ones the same way): nseg, and for each its slot count
// c (1..32) and the offset o in tile_slots of its first slot, as
// c << 25 | o (an expert's slots are packed from the start of its first
// tile, so its segment j starts 32 j past it; with 48-slot tiles a
// segment's 32 entries can pass the end of its expert's tiles, so only its
// first c entries are its slots).
template <int BM>
__global__ __launch_bounds__(1024) void k_group_tiles(const int32_t *__restrict__ ids, int S, int E,
                                                      int *__restrict__ ntiles, int *__restrict__ tile_e,
                                                      int *__restrict__ tile_slots, int *__restrict__ nseg,
                                                      int *__restrict__ seg_off, int *__restrict__ nseg48,
                                                      int *__restrict__ seg_off48) {
    __shared__ int s_cnt[QMM_MOE_MAX_E], s_off[QMM_MOE_MAX_E], s_wtot[16], s_wseg[16], s_wseg48[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
    __syncthreads();
    for (int sl = tid; sl < S; sl += 1024) {
        const int e = ids[sl];
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    const int cnt = tid < E ? s_cnt[tid] : 0;
    const int nt = (cnt + BM - 1) / BM, ns = (cnt + 31) / 32, ns48 = (cnt + 47) / 48;
    int inc = nt, incs = ns, incs48 = ns48;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(inc, d), vs = __shfl_up(incs, d), vs48 = __shfl_up(incs48, d);
        if (lane >= d) {
            inc += v;
            incs += vs;
            incs48 += vs48;
        }
    }
    if (lane == 63) {
        s_wtot[wave] = inc;
        s_wseg[wave] = incs;
        s_wseg48[wave] = incs48;
    }
    __syncthreads();
    int base = 0, bases = 0, bases48 = 0;
    for (int w = 0; w < wave; ++w) {
        base += s_wtot[w];
        bases += s_wseg[w];
        bases48 += s_wseg48[w];
    }
    const int off = base + inc - nt, offs = bases + incs - ns, offs48 = bases48 + incs48 - ns48;
    if (tid < E) {
        s_off[tid] = off;
        for (int i = 0; i < nt; ++i) tile_e[off + i] = tid;
        for (int j = cnt; j < nt * BM; ++j) tile_slots[(size_t)off * BM + j] = -1;
        for (int j = 0; j < ns; ++j) seg_off[offs + j] = (min(32, cnt - 32 * j) << Q6R_SEG_SHIFT) | (off * BM + 32 * j);
        if (seg_off48)
            for (int j = 0; j < ns48; ++j)
                seg_off48[offs48 + j] = (min(48, cnt - 48 * j) << Q6R_SEG_SHIFT) | (off * BM + 48 * j);
        s_cnt[tid] = 0;  // now the running position of the expert's slots
    }
    if (tid == 1023) {
        ntiles[0] = base + inc;
        nseg[0] = bases + incs;
        if (nseg48) nseg48[0] = bases48 + incs48;
    }
    __syncthreads();
    for (int sl = tid; sl < S; sl += 1024) {
        const int e = ids[sl];
        if (e >= 0 && e < E) {
            const int pos = atomicAdd(&s_cnt[e], 1);
            tile_slots[(size_t)s_off[e] * BM + pos] = sl;
        }
    }
}

// y[t, :] = sum_j wts[t, j] * d[t*topk + j, :] over the slots whose expert is
// in [0, E), in slot order; four columns per thread.
__global__ __launch_bounds__(256) void k_moe_combine(const float *__restrict__ d, const int32_t *__restrict__ ids,
                                                     const float *__restrict__ wts, float *__restrict__ y,
                                                     int topk, int hidden, int E) {
    const int t = blockIdx.y;
    const int c4 = blockIdx.x * 256 + threadIdx.x;
    if (4 * c4 >= hidden) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < topk; ++j) {
        const int e = ids[t * topk + j];
        if (e < 0 || e >= E) continue;
        const float w = wts[t * topk + j];
        const float4 v = *reinterpret_cast<const float4 *>(d + (size_t)(t * topk + j) * hidden + 4 * c4);
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
    }
    *reinterpret_cast<float4 *>(y + (size_t)t * hidden + 4 * c4) = acc;
}

struct PrefillWs {
    int8_t *xq;
    float *xs, *xsum, *h, *d;
    int *ntiles, *tile_e, *tile_slots, *nseg, *seg_off, *nseg48, *seg_off48;
    int64_t bytes;
};

#ifndef QMV_PF_GATHER_SLOTS
#define QMV_PF_GATHER_SLOTS 256  // the layer runs on the decode gathers up to this many slots
#endif
int pf_bm(int64_t S, int64_t E, int64_t T, int64_t hidden, int64_t inter) {
    // 48-slot tiles need the weight-side gate/up tile (its 32-bit lane
    // offsets) and the resident-activation down GEMM
    const bool w48 = inter * (hidden / 256) * 144 < ((int64_t)1 << 32) && T * hidden < ((int64_t)1 << 32) &&
                     QMV_Q6R && inter <= 256 * Q6R_MAX_NSB;
    if (w48 && S >= QMV_PF48_LO * E && S < QMV_PF48_HI * E) return 48;
    return S < 32 * E ? 32 : 64;
}
int64_t pf_max_tiles(int64_t S, int64_t E, int bm) { return div_up(S, bm) + std::min(E, S); }

PrefillWs prefill_ws(uint8_t *base, int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E) {
    const int64_t S = T * topk, bm = pf_bm(S, E, T, hidden, inter), mt = pf_max_tiles(S, E, (int)bm);
    PrefillWs w{};
    int64_t o = 0;
    auto take = [&](int64_t nbytes) {
        uint8_t *p = base ? base + o : nullptr;
        o += div_up(nbytes, 256) * 256;
        return p;
    };
    w.xq = reinterpret_cast<int8_t *>(take(T * hidden));
    w.xs = reinterpret_cast<float *>(take(4 * T * (hidden / 32)));
    w.xsum = reinterpret_cast<float *>(take(4 * T * (hidden / 32)));
    w.ntiles = reinterpret_cast<int *>(take(4));
    w.tile_e = reinterpret_cast<int *>(take(4 * mt));
    w.tile_slots = reinterpret_cast<int *>(take(4 * mt * bm));
    w.nseg = reinterpret_cast<int *>(take(4));
    w.seg_off = reinterpret_cast<int *>(take(4 * pf_max_tiles(S, E, 32)));
    w.nseg48 = reinterpret_cast<int *>(take(4));
    w.seg_off48 = reinterpret_cast<int *>(take(4 * pf_max_tiles(S, E, 48)));
    w.h = reinterpret_cast<float *>(take(4 * S * inter));
    w.d = reinterpret_cast<float *>(take(4 * S * hidden));
    w.bytes = o;
    return w;
}

}  // namespace

extern "C" int64_t moe_ffn_prefill_workspace_bytes(int64_t T, int64_t topk, int64_t hidden, int64_t inter,
                                                   int64_t E) {
    if (T < 1 || topk < 1 || hidden < 1 || inter < 1 || E < 1) return 0;
    return prefill_ws(nullptr, T, topk, hidden, inter, E).bytes;
}

extern "C" int moe_ffn_prefill_q4k_q6k(const void *gate, const void *up, const void *down, const float *x,
                                       const int32_t *ids, const float *wts, float *y, void *ws, int64_t ws_bytes,
                                       int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E,
                                       qmv_stream_t stream) {
    if (!gate || !up || !down || !x || !ids || !wts || !y || !ws) return QMV_EINVAL;
    if (T < 1 || topk < 1 || E < 1 || hidden < 256 || inter < 256 || hidden % 256 || inter % 256) return QMV_EINVAL;
    if (ws_bytes < moe_ffn_prefill_workspace_bytes(T, topk, hidden, inter, E)) return QMV_EINVAL;
    const int64_t S = T * topk;
    if (E > QMM_MOE_MAX_E || S > QMM_MOE_MAX_SLOTS || T > 65535 || hidden > 65536 || inter > 65536 ||
        E * inter * (hidden / 256) * 144 > ((int64_t)1 << 40) || E * hidden * (inter / 256) * 210 > ((int64_t)1 << 40))
        return QMV_EUNSUPPORTED;
    if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(down, 2) || !aligned(x, 16) || !aligned(ids, 4) ||
        !aligned(wts, 4) || !aligned(y, 16) || !aligned(ws, 256))
        return QMV_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    const PrefillWs w = prefill_ws(static_cast<uint8_t *>(ws), T, topk, hidden, inter, E);
    const int bm = pf_bm(S, E, T, hidden, inter);
    const int64_t mt = pf_max_tiles(S, E, bm);
    // gate/up on the resident-activation GEMM over the table's 32-slot segments
    const bool q4r = QMV_Q4R && hidden <= 256 * Q4R_MAX_NSB;
    int rc = quantize_act_q8(x, w.xq, w.xs, w.xsum, T, hidden, stream);
    if (rc != QMV_OK) return rc;
    // Up to 256 slots the expert-grouped decode gathers stream the bank
    // faster than the GEMMs (128 experts of [768, 2048]: 135.6 against
    // 158 us at 256 slots; at 288 the GEMMs win, 162 against 200 us, and at
    // 512 by 170 against 251); same arithmetic, h in the same workspace.
    // (the decode down pass holds at most 64 slots of a token)
    if (S <= QMV_PF_GATHER_SLOTS && topk <= 64 && hidden <= 4096 && inter <= 4096 && aligned(down, 16))
        return qmv_internal::moe_layer_q8x_f32h(gate, up, down, w.xq, w.xs, w.xsum, ids, wts, y, w.h, T, topk,
                                                hidden, inter, E, s);
    QmmArgs gu{static_cast<const uint8_t *>(gate), w.xq, w.xs, w.xsum, w.h, (int)S, (int)inter, (int)hidden, ids,
               (int)E, (int)topk, w.ntiles, w.tile_e, w.tile_slots, static_cast<const uint8_t *>(up)};
    Qmm6Args dn{static_cast<const uint8_t *>(down), nullptr, nullptr, w.h, w.d, (int)S, (int)hidden, (int)inter, ids,
                (int)E, 1, w.ntiles, w.tile_e, w.tile_slots};
    // the down GEMM's segments: 48 slots where the experts average more
    // than 16 (k_group_tiles lists them beside the 32-slot ones)
    const int sl6 = q6r_segment_slots(S, E, inter);
    int *const n48 = sl6 == 48 ? w.nseg48 : nullptr, *const s48 = sl6 == 48 ? w.seg_off48 : nullptr;
    const int *const nseg6 = sl6 == 48 ? w.nseg48 : w.nseg, *const segoff6 = sl6 == 48 ? w.seg_off48 : w.seg_off;
    if (bm == 32) {
        hipLaunchKernelGGL((k_group_tiles<32>), dim3(1), dim3(1024), 0, s, ids, (int)S, (int)E, w.ntiles, w.tile_e,
                           w.tile_slots, w.nseg, w.seg_off, n48, s48);
        QMV_LAUNCH_CHECK();
        if (q4r)
            launch_q4r<true, false>(gu, w.nseg, w.seg_off, 32, s);
        else
            hipLaunchKernelGGL((k_qmm_q4k<QMM_MOE32, true, true, true>), dim3((unsigned)div_up(inter, 64), (unsigned)mt),
                               dim3(256), 0, s, gu);
        QMV_LAUNCH_CHECK();
        if (QMV_Q6R && inter <= 256 * Q6R_MAX_NSB)
            launch_q6r<false>(dn, nseg6, segoff6, 32, sl6, s);
        else
            hipLaunchKernelGGL((k_qmm_q6k<QMM6_PF32, ACT_F32, true, true>),
                               dim3((unsigned)div_up(hidden, 256), (unsigned)mt), dim3(512), 0, s, dn);
    } else if (bm == 48) {
        // every expert's slots fit one tile up to 48 slots per expert: a
        // quarter less padding than 64-slot tiles where experts hold 20-47
        hipLaunchKernelGGL((k_group_tiles<48>), dim3(1), dim3(1024), 0, s, ids, (int)S, (int)E, w.ntiles, w.tile_e,
                           w.tile_slots, w.nseg, w.seg_off, n48, s48);
        QMV_LAUNCH_CHECK();
        if (q4r)
            launch_q4r<true, false>(gu, w.nseg, w.seg_off, 48, s);
        else
            hipLaunchKernelGGL((k_qmm2_q4k<4, 1, 2, 1, 3>), dim3((unsigned)div_up(inter, 64), (unsigned)mt), dim3(512),
                               0, s, gu, 0);
        QMV_LAUNCH_CHECK();
        launch_q6r<false>(dn, nseg6, segoff6, 48, sl6, s);
    } else {
        hipLaunchKernelGGL((k_group_tiles<64>), dim3(1), dim3(1024), 0, s, ids, (int)S, (int)E, w.ntiles, w.tile_e,
                           w.tile_slots, w.nseg, w.seg_off, n48, s48);
        QMV_LAUNCH_CHECK();
        // weight-side tile while its 32-bit lane offsets hold (an expert's
        // rows and the activation rows below 2^32 bytes)
        if (q4r)
            launch_q4r<true, false>(gu, w.nseg, w.seg_off, 64, s);
        else if (inter * (hidden / 256) * 144 < ((int64_t)1 << 32) && T * hidden < ((int64_t)1 << 32))
            hipLaunchKernelGGL((k_qmm2_q4k<4, 1, 2, 1>), dim3((unsigned)div_up(inter, 64), (unsigned)mt), dim3(512),
                               0, s, gu, 0);
        else
            hipLaunchKernelGGL((k_qmm_q4k<QMM_MOE64, true, true, true>),
                               dim3((unsigned)div_up(inter, QMM_MOE64_BN / 2), (unsigned)mt), dim3(QMM_MOE64_NT), 0, s,
                               gu);
        QMV_LAUNCH_CHECK();
        if (QMV_Q6R && inter <= 256 * Q6R_MAX_NSB)
            launch_q6r<false>(dn, nseg6, segoff6, 64, sl6, s);
        else
            hipLaunchKernelGGL((k_qmm_q6k<QMM6_PF64, ACT_F32, true, true>),
                               dim3((unsigned)div_up(hidden, 128), (unsigned)mt), dim3(512), 0, s, dn);
    }
    QMV_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)div_up(hidden, 1024), (unsigned)T), dim3(256), 0, s, w.d, ids,
                       wts, y, (int)topk, (int)hidden, (int)E);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}

// ==================================================================== Q8_0
// Q8_0 prefill GEMM on a q8 activation (hanzo-ml `src/vulkan_backend.rs`: the
// native Q8_0 blocks of `matvec_q8_0_gpu`, prefill as `matmul_q4_0_gpu` does
// for Q4_0 -- weights stay quantized, each decoded value serves a tile of
// rows):
//   Y[i, r] = sum_b xs[i, b] * d[r, b] * T[i, r, b],  T = sum_{l<32} xq * q.
// Both codes are int8, exact in f16, and T (|T| <= 32*127*128) is exact on
// the f16 matrix cores (one v_mfma_f32_16x16x32_f16 per 16x16 tile and
// block); the epilogue is d * T, then one FMA with xs, per output and block.
// Tiles of 64 x 128 on eight waves, phases of 64 values (two blocks), the
// double-buffered staging of the Q6_K kernel; rows of 34-byte blocks are
// 2-byte aligned and read with 8-byte loads.
namespace {

template <int BM, int BN, int MT, int NT, int NTHREADS>
__global__ __launch_bounds__(NTHREADS) void k_qmm_q8_0(const uint8_t *__restrict__ w, const int8_t *__restrict__ xq,
                                                       const float *__restrict__ xs, float *__restrict__ Y, int m,
                                                       int n, int k) {
    constexpr int KP = 64, NBP = 2;              // values and blocks per phase
    constexpr int WM = 16 * MT, WN = 16 * NT;
    constexpr int WGM = BM / WM, WGN = BN / WN;
    static_assert(WGM * WGN == NTHREADS / 64, "the waves tile the workgroup");
    constexpr int ST = KP + 8;
    constexpr int ACR = KP / 8;                  // 8-code activation chunks per row
    constexpr int AC = BM * ACR / NTHREADS;
    static_assert(AC >= 1 && AC * NTHREADS == BM * ACR, "activation staging");
    constexpr int BCH = BN * (KP / 8);           // 8-code weight chunks per phase
    constexpr int BCT = BCH / NTHREADS;
    static_assert(BCT >= 1 && BCT * NTHREADS == BCH && NTHREADS % BN == 0, "weight staging");
    constexpr int XC = (BM * NBP + NTHREADS - 1) / NTHREADS;

    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * ST];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * ST];
    __shared__ __attribute__((aligned(16))) float sfx[2][NBP][BM];
    __shared__ float sdq[2][NBP][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WGM, wn = wave / WGM;
    const int li = lane & 15, lq = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int kb = k / 32;
    const size_t row_bytes = (size_t)kb * 34;
    const int brow = tid % BN, bc0 = tid / BN;
    const bool bvalid = n0 + brow < n;
    const uint8_t *wrow = w + (size_t)(bvalid ? n0 + brow : 0) * row_bytes;
    int arow[AC], xrow[XC];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int r = (tid + NTHREADS * i) / ACR;
        arow[i] = m0 + r < m ? m0 + r : -1;
    }
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int idx = tid + NTHREADS * i, r = idx % BM;
        xrow[i] = (idx < BM * NBP && m0 + r < m) ? m0 + r : -1;
    }

    uint2 ra[2][AC], rb[2][BCT];
    uint32_t rd[2][BCT];
    float rxs[2][XC];

    auto prefetch = [&](int ph, int q) {
        const int k0 = ph * KP;
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c = (tid + NTHREADS * i) % ACR, gm = arow[i];
            ra[q][i] = gm >= 0 ? *reinterpret_cast<const uint2 *>(xq + (size_t)gm * k + k0 + 8 * c)
                               : make_uint2(0u, 0u);
        }
        if (bvalid) {
#pragma unroll
            for (int i = 0; i < BCT; ++i) {
                const int bc = bc0 + i * (NTHREADS / BN);  // block bc / 4 of the phase, codes 8 (bc % 4) ..
                const uint8_t *blk = wrow + (size_t)(2 * ph + (bc >> 2)) * 34;
                rb[q][i] = *reinterpret_cast<const uint2 *>(blk + 2 + 8 * (bc & 3));
                rd[q][i] = ld2(blk);
            }
        } else {
#pragma unroll
            for (int i = 0; i < BCT; ++i) rb[q][i] = make_uint2(0u, 0u), rd[q][i] = 0u;
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int bl = (tid + NTHREADS * i) / BM, gm = xrow[i];
            rxs[q][i] = gm >= 0 ? xs[(size_t)gm * kb + k0 / 32 + bl] : 0.f;
        }
    };
    auto convert_store = [&](int buf, int q) {
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int ch = tid + NTHREADS * i, row = ch / ACR, c = ch % ACR;
            const uint2 h0 = i8x4_to_f16(ra[q][i].x), h1 = i8x4_to_f16(ra[q][i].y);
            *reinterpret_cast<uint4 *>(&As[buf][row * ST + 8 * c]) = make_uint4(h0.x, h0.y, h1.x, h1.y);
        }
#pragma unroll
        for (int i = 0; i < BCT; ++i) {
            const int bc = bc0 + i * (NTHREADS / BN);
            const uint2 c0 = i8x4_to_f16(rb[q][i].x), c1 = i8x4_to_f16(rb[q][i].y);
            *reinterpret_cast<uint4 *>(&Bs[buf][brow * ST + 8 * bc]) = make_uint4(c0.x, c0.y, c1.x, c1.y);
            if ((bc & 3) == 0) sdq[buf][bc >> 2][brow] = h2f(rd[q][i]);
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int idx = tid + NTHREADS * i, row = idx % BM, bl = idx / BM;
            if (idx < BM * NBP) sfx[buf][bl][row] = rxs[q][i];
        }
    };

    v4f acc[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};

    const int nph = k / KP;  // even (k % 256 == 0)
    prefetch(0, 0);
    convert_store(0, 0);
    prefetch(1, 1);
    if (nph > 2) prefetch(2, 0);
    __syncthreads();
    for (int ph0 = 0; ph0 < nph; ph0 += 2) {
#pragma unroll
        for (int Q = 0; Q < 2; ++Q) {
            const int ph = ph0 + Q, buf = Q;
#pragma unroll
            for (int bl = 0; bl < NBP; ++bl) {
                h8 fa[MT], fb[NT];
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    fa[t] = *reinterpret_cast<const h8 *>(&As[buf][(wm * WM + 16 * t + li) * ST + 32 * bl + 8 * lq]);
#pragma unroll
                for (int u = 0; u < NT; ++u)
                    fb[u] = *reinterpret_cast<const h8 *>(&Bs[buf][(wn * WN + 16 * u + li) * ST + 32 * bl + 8 * lq]);
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const float dcol = sdq[buf][bl][wn * WN + 16 * u + li];
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const v4f T = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[t], fb[u], (v4f){0.f, 0.f, 0.f, 0.f},
                                                                             0, 0, 0);
                        const v4f fx = *reinterpret_cast<const v4f *>(&sfx[buf][bl][wm * WM + 16 * t + 4 * lq]);
                        acc[t][u] = fx * (dcol * T) + acc[t][u];
                    }
                }
            }
            if (ph + 1 < nph) {
                convert_store(buf ^ 1, Q ^ 1);
                if (ph + 3 < nph) prefetch(ph + 3, Q ^ 1);
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const int col = n0 + wn * WN + 16 * u + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WM + 16 * t + 4 * lq + r;
                if (row < m && col < n) Y[(size_t)row * n + col] = acc[t][u][r];
            }
        }
}

}  // namespace

extern "C" int qmm_q8_0(const void *w, const int8_t *xq, const float *xs, float *y, int64_t m, int64_t n, int64_t k,
                        qmv_stream_t stream) {
    if (!w || !xq || !xs || !y || m < 1 || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (m > (1 << 24) || n > (1 << 24) || k > (1 << 20) || m * k > ((int64_t)1 << 34)) return QMV_EUNSUPPORTED;
    if (!aligned(w, 2) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(y, 4)) return QMV_EALIGN;
    const dim3 grid((unsigned)div_up(n, 128), (unsigned)div_up(m, 64));
    hipLaunchKernelGGL((k_qmm_q8_0<64, 128, 2, 2, 512>), grid, dim3(512), 0, (hipStream_t)stream,
                       static_cast<const uint8_t *>(w), xq, xs, y, (int)m, (int)n, (int)k);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}
