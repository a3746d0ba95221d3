// Library-internal entry points shared between translation units (not part
// of the C ABI).
#pragma once

#include "common.hpp"

namespace qmv_internal {

// The MoE prefill layer's arithmetic (gate/up on a q8 activation, h in f32,
// down on f32 h, weighted combine) on the decode gathers: the expert-grouped
// matvec kernels, which stream a bank faster than the prefill GEMMs when few
// slots share each expert. xq/xs/xsum hold the T quantized activation rows;
// h is scratch for T*topk*inter floats. Needs topk <= 64, T*topk <= 2048,
// hidden, inter <= 4096 and 16-byte aligned banks; returns a qmv_status.
int moe_layer_q8x_f32h(const void *gate, const void *up, const void *down, const int8_t *xq, const float *xs,
                       const float *xsum, const int32_t *ids, const float *wts, float *y, float *h, int64_t T,
                       int64_t topk, int64_t hidden, int64_t inter, int64_t E, hipStream_t s);

// All host-side checks of the f32 decode MoE layer (moe_ffn_q4k_q6k);
// returns QMV_OK or the status that entry point would return.
int check_decode_layer(const void *gate, const void *up, const void *down, const float *x, const int32_t *ids,
                       const float *wts, const float *y, const void *ws, int64_t ws_bytes, int64_t T, int64_t topk,
                       int64_t hidden, int64_t inter, int64_t E);

}  // namespace qmv_internal
