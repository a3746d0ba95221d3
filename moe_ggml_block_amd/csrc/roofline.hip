// Streaming-read probe for the roofline denominator.
//
// The pages price their kernels against a bandwidth measured on the device
// itself (hanzo-ml `src/vulkan_backend.rs`: the roofline profiling option
// divides achieved bytes by a device-to-device copy bandwidth measured once
// at start-up). Besides such a copy, a decode matvec of a few tens of MB is
// better compared with the fastest plain READ of the same number of bytes in
// one launch: at that size the launch's ramp-up and drain are a large part of
// the time, and a copy of the same size also pays for its writes.
//
// k_stream_read: every thread reads UNR 16-byte chunks per round, the
// rounds striding over the whole buffer (the workgroups' chunks of one round
// are contiguous), and folds them into one xor; a lane writes only if the
// xor equals a value passed in that no real data produces here (so the loads
// cannot be dropped and nothing is written in practice).
#include "common.hpp"

namespace {

template <int UNR>
__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ p, int64_t n16, uint32_t never,
                                                     uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
        uint4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == never) sink[0] = acc;
}

}  // namespace

extern "C" int qmv_roofline_read(const void *buf, int64_t bytes, int64_t workgroups, int64_t unroll,
                                 uint32_t *sink, qmv_stream_t stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 || workgroups < 1 || workgroups > (1 << 20)) return QMV_EINVAL;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return QMV_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    const auto *p = static_cast<const uint4 *>(buf);
    const int64_t n16 = bytes / 16;
    const uint32_t never = 0x9E3779B9u;
    const dim3 grid((unsigned)workgroups);
    switch (unroll) {
        case 1: hipLaunchKernelGGL(k_stream_read<1>, grid, dim3(256), 0, s, p, n16, never, sink); break;
        case 2: hipLaunchKernelGGL(k_stream_read<2>, grid, dim3(256), 0, s, p, n16, never, sink); break;
        case 4: hipLaunchKernelGGL(k_stream_read<4>, grid, dim3(256), 0, s, p, n16, never, sink); break;
        case 8: hipLaunchKernelGGL(k_stream_read<8>, grid, dim3(256), 0, s, p, n16, never, sink); break;
        default: return QMV_EINVAL;
    }
    QMV_LAUNCH_CHECK();
    return QMV_OK;
}
