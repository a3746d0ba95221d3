// Q4_K x q8-activation prefill GEMM on gfx950 int8 MFMA.
//
// hanzo-ml `src/vulkan_backend.rs`, `mmq_q4k_rt_gpu` / `mmq_q4k_gpu`: affine
// Q4_K weights decoded in-kernel, activation quantized to (xq, xs, xsum),
// epilogue xs*(D*dot - M*xsum) per 32-value block; `mul_mm_q4k_tiled_dp4a`:
// BM rows of the output per workgroup so cold weights are re-read m/BM times.
//
//   Y[i, r] = sum_b xs[i,b] * dsc[r,b] * S[i,r,b]  -  sum_b xsum[i,b] * dmn[r,b]
//   S[i,r,b] = sum_{l<32} xq[i,32b+l] * q[r,32b+l]    (int32, exact)
//   dsc = d*sc_j, dmn = dmin*m_j of the sub-block j holding q8 block b.
//
// Each q8 block is one v_mfma_i32_16x16x32_i8 (K = 32, one block, so the
// integer sum never mixes scales); its 16x16 int32 tile is converted and
// scaled into an f32 accumulator by the VALU. The min term is a rank-(k/32)
// f32 product done on v_mfma_f32_16x16x4_f32, four blocks per instruction.
//
// Workgroup: 256 threads, tile BM x 32 of Y. The 32 weight rows of the
// current superblock are decoded once into LDS as int8 codes (row stride
// padded to 264 bytes against bank conflicts) plus dsc/dmn; activation codes
// come straight from global memory (L2-resident); xs/xsum of the BM rows are
// staged in LDS per superblock.
#include "blocks.hpp"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = 32;
constexpr int BSTRIDE = 264;  // bytes per decoded weight row in LDS

template <int BM>
__global__ __launch_bounds__(256) void k_qmm_q4k(const uint8_t *__restrict__ w,
                                                 const int8_t *__restrict__ xq,
                                                 const float *__restrict__ xs,
                                                 const float *__restrict__ xsum,
                                                 float *__restrict__ Y, int m, int n, int k) {
    constexpr int MT = BM / 64;  // 16-row m tiles per wave (4 waves split BM)
    __shared__ __attribute__((aligned(16))) int8_t bq[BN * BSTRIDE];
    __shared__ float dsc[8][BN], dmn[8][BN];
    __shared__ __attribute__((aligned(16))) float sxs[8][BM], sxsum[8][BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * BN;
    const int mblk = blockIdx.y * BM;
    const int mw = mblk + wave * (BM / 4);  // this wave's first row
    const int kb = k / 32, nsb = k / 256;
    const int row_bytes = nsb * 144;
    const int li = lane & 15, lq = lane >> 4;

    v4f acc[MT][2];
    v4f accm[MT][2];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};
            accm[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};
        }

    for (int s = 0; s < nsb; ++s) {
        __syncthreads();
        // ---- decode 32 weight rows of superblock s into LDS: thread -> (row, chunk)
        {
            const int rr = tid >> 3, c = tid & 7;
            const int r = n0 + rr;
            uint4 q = make_uint4(0, 0, 0, 0), hd = make_uint4(0, 0, 0, 0);
            if (r < n) {
                const uint8_t *blk = w + (size_t)r * row_bytes + (size_t)s * 144;
                q = ld16(blk + 16 + 16 * c);
                hd = ld16(blk);
            }
            const int p = c >> 1, hh = c & 1;
            uint4 lo, hi;
            lo.x = q.x & 0x0F0F0F0Fu; lo.y = q.y & 0x0F0F0F0Fu; lo.z = q.z & 0x0F0F0F0Fu; lo.w = q.w & 0x0F0F0F0Fu;
            hi.x = (q.x >> 4) & 0x0F0F0F0Fu; hi.y = (q.y >> 4) & 0x0F0F0F0Fu;
            hi.z = (q.z >> 4) & 0x0F0F0F0Fu; hi.w = (q.w >> 4) & 0x0F0F0F0Fu;
            // sub-block 2p gets the low nibbles at l = 16hh.., 2p+1 the high ones
            uint32_t *dlo = reinterpret_cast<uint32_t *>(bq + rr * BSTRIDE + 32 * (2 * p) + 16 * hh);
            uint32_t *dhi = reinterpret_cast<uint32_t *>(bq + rr * BSTRIDE + 32 * (2 * p + 1) + 16 * hh);
            dlo[0] = lo.x; dlo[1] = lo.y; dlo[2] = lo.z; dlo[3] = lo.w;
            dhi[0] = hi.x; dhi[1] = hi.y; dhi[2] = hi.z; dhi[3] = hi.w;
            if (hh == 0) {
                uint32_t sc2, mn2;
                q4k_scales(hd.y, hd.z, hd.w, p, &sc2, &mn2);
                const float d = h2f(hd.x), dm = h2f(hd.x >> 16);
                dsc[2 * p][rr] = d * ubyte_f<0>(sc2);
                dsc[2 * p + 1][rr] = d * ubyte_f<1>(sc2);
                dmn[2 * p][rr] = dm * ubyte_f<0>(mn2);
                dmn[2 * p + 1][rr] = dm * ubyte_f<1>(mn2);
            }
        }
        // ---- stage xs / xsum of the BM rows for the 8 q8 blocks of superblock s
        for (int i = tid; i < 8 * BM; i += 256) {
            const int b = i / BM, mr = i % BM;
            const int gm = mblk + mr;
            float a = 0.f, z = 0.f;
            if (gm < m) {
                a = xs[(size_t)gm * kb + 8 * s + b];
                z = xsum[(size_t)gm * kb + 8 * s + b];
            }
            sxs[b][mr] = a;
            sxsum[b][mr] = z;
        }
        __syncthreads();

        // ---- 8 q8 blocks
#pragma unroll 2
        for (int b = 0; b < 8; ++b) {
            long av[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int gm = mw + 16 * t + li;
                av[t] = gm < m ? *reinterpret_cast<const long *>(xq + (size_t)gm * k + 256 * s + 32 * b + 8 * lq) : 0;
            }
            long bv[2];
            float ds[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                bv[u] = *reinterpret_cast<const long *>(bq + (16 * u + li) * BSTRIDE + 32 * b + 8 * lq);
                ds[u] = dsc[b][16 * u + li];
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float4 x4 = *reinterpret_cast<const float4 *>(&sxs[b][wave * (BM / 4) + 16 * t + 4 * lq]);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[t], bv[u], (v4i){0, 0, 0, 0}, 0, 0, 0);
                    acc[t][u][0] = fmaf((float)S[0], x4.x * ds[u], acc[t][u][0]);
                    acc[t][u][1] = fmaf((float)S[1], x4.y * ds[u], acc[t][u][1]);
                    acc[t][u][2] = fmaf((float)S[2], x4.z * ds[u], acc[t][u][2]);
                    acc[t][u][3] = fmaf((float)S[3], x4.w * ds[u], acc[t][u][3]);
                }
            }
        }
        // ---- min term: two f32 MFMAs (K = 4 blocks each) per 16x16 tile
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int b = 4 * h + lq;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float a = sxsum[b][wave * (BM / 4) + 16 * t + li];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const float bb = dmn[b][16 * u + li];
                    accm[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, accm[t][u], 0, 0, 0);
                }
            }
        }
    }
    // ---- write Y: lane holds rows 4*lq + r, column li of each 16x16 tile
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int col = n0 + 16 * u + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mw + 16 * t + 4 * lq + r;
                if (row < m && col < n) Y[(size_t)row * n + col] = acc[t][u][r] - accm[t][u][r];
            }
        }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" int qmm_q4k(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y,
                       int64_t m, int64_t n, int64_t k, int bm, qmv_stream_t stream) {
    if (!w || !xq || !xs || !xsum || !y || m < 1 || n < 1 || k < 256 || k % 256) return QMV_EINVAL;
    if (bm != 128 && bm != 256) return QMV_EINVAL;
    if (m > (1 << 24) || n > (1 << 24) || k > (1 << 20) || (int64_t)m * k > ((int64_t)1 << 34)) return QMV_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(y, 4))
        return QMV_EALIGN;
    const dim3 grid((unsigned)div_up(n, BN), (unsigned)div_up(m, bm));
    hipStream_t s = (hipStream_t)stream;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    if (bm == 128)
        hipLaunchKernelGGL(k_qmm_q4k<128>, grid, dim3(256), 0, s, wb, xq, xs, xsum, y, (int)m, (int)n, (int)k);
    else
        hipLaunchKernelGGL(k_qmm_q4k<256>, grid, dim3(256), 0, s, wb, xq, xs, xsum, y, (int)m, (int)n, (int)k);
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}
