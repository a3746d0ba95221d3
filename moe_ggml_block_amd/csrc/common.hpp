// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv.h"

#define QMV_DEV static __device__ __forceinline__

// IEEE binary16 bits -> f32. v_cvt_f32_f16 is exact for every finite half,
// subnormals included (f16 denormals are on in the default FP mode).
QMV_DEV float h2f(uint32_t bits) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
    return (float)h;
}

// Byte b of a dword as f32 (unsigned); folds to v_cvt_f32_ubyte{b}.
template <int B>
QMV_DEV float ubyte_f(uint32_t v) {
    return (float)((v >> (8 * B)) & 0xFFu);
}

// Byte b of a dword as f32 (signed).
template <int B>
QMV_DEV float sbyte_f(uint32_t v) {
    return (float)(int32_t)(int8_t)((v >> (8 * B)) & 0xFFu);
}

// Bytes [s, s+4) of the 8-byte little-endian pair {hi:lo}, s in 0..3.
QMV_DEV uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of
// the group receives the total.
template <int G>
QMV_DEV float group_sum(float v) {
    if (G >= 64) v += __shfl_xor(v, 32);
    if (G >= 32) v += __shfl_xor(v, 16);
    if (G >= 16) v += __shfl_xor(v, 8);
    if (G >= 8) v += __shfl_xor(v, 4);
    if (G >= 4) v += __shfl_xor(v, 2);
    if (G >= 2) v += __shfl_xor(v, 1);
    return v;
}

template <int G>
QMV_DEV int group_isum(int v) {
    if (G >= 64) v += __shfl_xor(v, 32);
    if (G >= 32) v += __shfl_xor(v, 16);
    if (G >= 16) v += __shfl_xor(v, 8);
    if (G >= 8) v += __shfl_xor(v, 4);
    if (G >= 4) v += __shfl_xor(v, 2);
    if (G >= 2) v += __shfl_xor(v, 1);
    return v;
}

// Sum over aligned groups of G lanes with DPP row operations (no LDS):
// xor-1 and xor-2 quad permutes, half-row and row mirrors, then the row
// broadcasts of lanes 15 and 31. The total lands in the LAST lane of each
// group (for G <= 16 in every lane of the group). Call in wave-uniform
// control flow: every lane must execute it.
template <int CTRL, int ROW_MASK>
QMV_DEV float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return v + __int_as_float(t);
}

template <int G>
QMV_DEV float group_sum_last(float v) {
    if (G >= 2) v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    if (G >= 4) v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    if (G >= 8) v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    if (G >= 16) v = dpp_add<0x140, 0xF>(v); // row_mirror
    if (G >= 32) v = dpp_add<0x142, 0xA>(v); // row_bcast15 into rows 1, 3
    if (G >= 64) v = dpp_add<0x143, 0xC>(v); // row_bcast31 into rows 2, 3
    return v;
}

// silu(z) = z / (1 + e^-z), the division by the hardware reciprocal (1 ulp)
// instead of the correctly rounded division sequence; z below about -88
// gives e^-z = inf and -0, as the division would.
QMV_DEV float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Non-temporal-free plain 16-byte load.
QMV_DEV uint4 ld16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }
QMV_DEV uint32_t ld4(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
QMV_DEV uint32_t ld2(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

static inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

static inline int next_pow2_le64(int64_t u) {
    int g = 1;
    while (g < u && g < 64) g <<= 1;
    return g;
}

#define QMV_LAUNCH_CHECK()                                  \
    do {                                                    \
        if (hipGetLastError() != hipSuccess) return QMV_ELAUNCH; \
    } while (0)
