/*
 * qmv -- GGML block-quantized matrix-vector products and the indexed-MoE
 * decode path, as hand-written HIP kernels for gfx950 (MI355X).
 *
 * C ABI. Every entry point:
 *  - takes device pointers owned by the caller (the library never allocates
 *    or frees device memory) and a HIP stream (NULL = the null stream);
 *  - validates shapes and pointer alignment on the host and returns a
 *    negative qmv_status before launching anything if they are wrong;
 *  - otherwise enqueues its kernels asynchronously on `stream` and returns
 *    QMV_OK, or QMV_ELAUNCH if the HIP runtime rejected a launch;
 *  - fully overwrites its outputs (nothing is accumulated into them);
 *  - is stateless and may be called from several host threads.
 *
 * Weight blocks are the raw GGML/GGUF bytes, verbatim, row-major: row r of a
 * [n, k] matrix occupies bytes [r*(k/B)*S, (r+1)*(k/B)*S) where B is the
 * block's weight count and S its byte size. An expert bank [E, n, k] is the
 * E matrices back to back (expert e starts at byte e*n*(k/B)*S).
 *
 *   Q8_0  B = 32,  S = 34:  f16 d, int8 q[32];        w = d*q
 *   Q4_K  B = 256, S = 144: f16 d, f16 dmin, 12 bytes of 6-bit scales and
 *                           mins for 8 sub-blocks of 32, 128 bytes of 4-bit
 *                           codes;                    w = d*sc_j*q - dmin*m_j
 *   Q6_K  B = 256, S = 210: ql[128] low nibbles, qh[64] 2-bit highs,
 *                           int8 sc[16], f16 d;       w = d*sc_t*(q - 32)
 *
 * Field order and sizes: hanzo-ml `src/vulkan_backend.rs`, functions
 * `quantize_q8_blocks` (Q8_0), `quantize_q4k` / `quantize_q4k_split` (Q4_K),
 * `quantize_q6k` / `quantize_q6k_split` (Q6_K). Bit packing inside the
 * fields: the public GGML k-quant packing.
 *
 * Alignment: weight pointers 16-byte aligned; f32 activation pointers
 * 16-byte aligned; int8 activation pointers 16-byte aligned; other outputs
 * 4-byte aligned (QMV_EALIGN otherwise). Buffers allocated by hipMalloc or
 * PyTorch meet this.
 */
#ifndef QMV_H
#define QMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t; declared here so that callers need no HIP headers. */
typedef struct ihipStream_t *qmv_stream_t;

typedef enum {
    QMV_OK = 0,
    QMV_EINVAL = -1,      /* bad shape: k not a block multiple, n/m <= 0, topk out of [1,E], null pointer, workspace too small */
    QMV_EALIGN = -2,      /* a pointer does not meet the alignment above */
    QMV_ELAUNCH = -3,     /* hipGetLastError reported a failure after a launch */
    QMV_EUNSUPPORTED = -4 /* valid but outside what this build implements (e.g. E > 4096) */
} qmv_status;

/* Library version string, and a static message for a status code. */
const char *qmv_version(void);
const char *qmv_strerror(int status);

/* ------------------------------------------------------------------------
 * Dense decode matvecs, f32 activation: y[r] = sum_c W_deq[r, c] * x[c].
 * w: n*(k/B)*S bytes; x: f32[k]; y: f32[n]. Accumulation in f32.
 * Defined by `matvec_q8_0_gpu`, `matvec_q4k_gpu_off`, `matvec_q6k_gpu_off`
 * (y[nout] = Wq * x[k] over blocks read verbatim, no requantization).
 * k % 32 == 0 (Q8_0) or k % 256 == 0 (Q4_K, Q6_K); n >= 1.
 * ---------------------------------------------------------------------- */
int qmv_q8_0(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream);
int qmv_q4k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream);
int qmv_q6k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream);

/* More formats on the same decode skeleton (hanzo-ml `src/vulkan_backend.rs`):
 *   qmv_q4_0: native 18-byte Q4_0 blocks (`matvec_q4_0_gpu`: f16 d + 16 code
 *             bytes, w = d*(q - 8)); w: n*(k/32)*18 bytes, k % 32 == 0.
 *   qmv_q5k:  176-byte Q5_K superblocks (`quantize_q5k` / `matvec_q5k_gpu`: d,
 *             dmin, 12 scale bytes, 32 qh bytes, 128 qs bytes, w =
 *             d*sc_j*q - dmin*m_j with a 5-bit q); w: n*(k/256)*176 bytes,
 *             k % 256 == 0.
 * x: f32[k]; y: f32[n]; blocks read verbatim; w and x 16-byte aligned. */
int qmv_q4_0(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream);
int qmv_q5k(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * q8 activation quantizer (`quantize_act_q8`: xq int8, xs f32 scale, xsum
 * f32 dequantized block sum, per 32 consecutive values of each row).
 * x: f32[m, k]; xq: int8[m, k]; xs, xsum: f32[m, k/32]. Per block:
 *   amax = max|x|; inv = 127/amax, xs = amax/127 (inv = 0, xs = 1 if amax = 0);
 *   xq = clamp(round_half_away(x*inv), -127, 127); xsum = xs * sum(xq).
 * Every f32 step is a single correctly rounded IEEE operation, so the result
 * is bit-identical to any IEEE f32 implementation of the same steps.
 * k % 32 == 0; m >= 1.
 * ---------------------------------------------------------------------- */
int quantize_act_q8(const float *x, int8_t *xq, float *xs, float *xsum, int64_t m, int64_t k,
                    qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * qmv_q4k and quantize_act_q8 of the same activation in one call: y is
 * bit-identical to qmv_q4k(w, x, y, n, k) and (xq, xs, xsum) to
 * quantize_act_q8(x, xq, xs, xsum, 1, k) (both defined above; the q8 row is
 * what the int8-dot decode path of `matvec_q4k_gpu_off` consumes next, so a
 * decode step that runs both formats needs no quantizer launch). For
 * k <= 8192 the first workgroup of the matvec writes the q8 row from the
 * activation values it loads anyway; beyond that the two run as separate
 * launches on the stream. Buffers as in the two calls; xq, xs, xsum must not
 * overlap x, w or y. k % 256 == 0; n >= 1.
 * ---------------------------------------------------------------------- */
int qmv_q4k_qx(const void *w, const float *x, float *y, int8_t *xq, float *xs, float *xsum, int64_t n,
               int64_t k, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * Q4_K matvec against a q8 activation (the int8-dot decode path of
 * `matvec_q4k_gpu_off` / `matvec_q4k_dp4a_blk`):
 *   y[r] = sum_b ( d*sc_j*xs[b]*S[r,b] - dmin*m_j*xsum[b] ),
 *   S[r,b] = sum_{i<32} q[r, 32b+i] * xq[32b+i]  (exact int32 dot4 sums),
 * which equals W_deq . (xs*xq) up to f32 rounding.
 * w: n*(k/256)*144 bytes; xq: int8[k]; xs, xsum: f32[k/32]; y: f32[n].
 * ---------------------------------------------------------------------- */
int qmv_q4k_q8(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y,
               int64_t n, int64_t k, qmv_stream_t stream);

/* The same int8-dot Q4_K matvec from an f32 activation in one launch: every
 * workgroup quantizes x itself (the steps of quantize_act_q8, so the codes
 * and scales are the same bits) while staging it, then decodes as
 * qmv_q4k_q8 -- y is bit-identical to quantize_act_q8 followed by
 * qmv_q4k_q8 (`matvec_q4k_gpu_off` quantizes x once per call and runs the
 * int8-dot decode). w: n*(k/256)*144 bytes; x: f32[k]; y: f32[n];
 * k % 256 == 0, k <= 8192; w and x 16-byte aligned. */
int qmv_q4k_q8x(const void *w, const float *x, float *y, int64_t n, int64_t k, qmv_stream_t stream);

/* Debug export of the integer part of qmv_q4k_q8: sums[r, b] = S[r, b]
 * (int32[n, k/32]) computed by the same dot4 sequence as qmv_q4k_q8. */
int qmv_debug_blocksums_q4k_q8(const void *w, const int8_t *xq, int32_t *sums, int64_t n,
                               int64_t k, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * MoE router (`moe_route_vk`: softmax + top-k + renormalize in one kernel).
 * logits: f32[T, E]; ids: int32[T, topk]; wts: f32[T, topk].
 * Per token the topk largest logits are selected (equal values: lower
 * expert index first; NaN ranks below every number), ids are written in
 * descending-logit order and wts[j] = exp(l_j - l_max) / sum over the
 * selected of exp(l - l_max) (the softmax denominator cancels). If every
 * selected logit is -inf/NaN the weights are 1/topk.
 * 1 <= topk <= min(E, 64); 1 <= E <= 4096; T >= 1.
 * ---------------------------------------------------------------------- */
int moe_route(const float *logits, int32_t *ids, float *wts, int64_t T, int64_t E, int64_t topk,
              qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * MoE router gate + router (the "gemv" kernel of hanzo-ml
 * `src/vulkan_backend.rs`, used for the router gate at one token in place of
 * the tiled GEMM; `check_gemv` of hanzo-kernel `src/main.rs`):
 *   logits[t, e] = sum_c wr[e, c] * x[t, c]   (f32 accumulation),
 * then moe_route(logits, ids, wts, T, E, topk) on the same stream.
 * wr: f32[E, hidden] row-major (the router weight, resident); x: f32[T,
 * hidden]; logits: f32[T, E] (written, caller-owned scratch that also serves
 * as output); ids: int32[T, topk]; wts: f32[T, topk] as in moe_route.
 * 4 <= hidden <= 8192, hidden % 4 == 0; 1 <= E <= 4096; 1 <= topk <=
 * min(E, 64); 1 <= T <= 2^24. wr and x 16-byte aligned, the rest 4-byte.
 * All checks run on the host before any launch; nothing is written on error.
 * ---------------------------------------------------------------------- */
int moe_gate_route(const float *wr, const float *x, float *logits, int32_t *ids, float *wts, int64_t T,
                   int64_t E, int64_t hidden, int64_t topk, qmv_stream_t stream);

/* The MoE block from the hidden state: the router gate GEMV above (logits
 * written to `logits`), then moe_ffn_routed_q4k_q6k on those logits (router
 * fused into the gate/up gather; ids, wts written). Three launches. Operands
 * and limits as moe_gate_route and moe_ffn_q4k_q6k (hidden is both the
 * router's and the layer's input width; ws: moe_ffn_workspace_bytes()). All
 * checks run before the first launch. */
int moe_block_q4k_q6k(const float *wr, const void *gate, const void *up, const void *down, const float *x,
                      float *logits, int32_t *ids, float *wts, float *y, void *ws, int64_t ws_bytes, int64_t T,
                      int64_t topk, int64_t hidden, int64_t inter, int64_t E, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * Expert-gather matvec over a resident bank (`moe_matvec_gpu`):
 *   y[s, r] = sum_c W[ids[s], r, c] * x[s / x_div, c],  s < nslots, r < n.
 * bank: E*n*(k/B)*S bytes; x: f32[nslots/x_div rounded up, k];
 * ids: int32[nslots]; y: f32[nslots, n] in slot order.
 * Slots routed to the same expert share one read of that expert's rows.
 * A slot whose id is outside [0, E) gets a zero output row.
 * x_div >= 1 (gate/up of a routed token: x_div = topk; down: x_div = 1).
 * ---------------------------------------------------------------------- */
int moe_qmv_q4k(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream);
int moe_qmv_q6k(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y,
                int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream);
/* The same gather over a bank of native Q8_0 blocks (34 bytes per 32
 * weights; `moe_matvec_gpu` takes any resident bank format): bank
 * E*n*(k/32)*34 bytes, 2-byte aligned; limits as moe_qmv_q4k. */
int moe_qmv_q8_0(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y, int64_t nslots,
                 int64_t n, int64_t k, int64_t E, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * MoE FFN layer over routed slots s = topk*t + j, e = ids[s]
 * (the engine composition of `moe_matvec_*` gate/up, `silu_mul`, down and
 * the `broadcast_mul(scores).sum` combine):
 *   h_s = silu(W_gate[e] x_t) * (W_up[e] x_t)   gate/up: Q4_K [E, inter, hidden]
 *   d_s = W_down[e] h_s                          down:    Q6_K [E, hidden, inter]
 *   y_t = sum_j wts[t, j] * d_{topk*t + j}       (fixed j order)
 * x: f32[T, hidden]; ids: int32[T, topk]; wts: f32[T, topk]; y: f32[T, hidden].
 * ws: caller-owned device workspace of at least moe_ffn_workspace_bytes()
 * bytes (16-byte aligned); on return it holds h f32[T*topk, inter] (row s:
 * the activation slot s passed to the down projection; zero for a slot
 * whose id is outside [0, E)).
 * hidden % 256 == 0, inter % 256 == 0; hidden, inter <= 4096; T <= 65535;
 * 1 <= topk <= 64 (a token's slots are held on chip by the down pass:
 * QMV_EUNSUPPORTED above that, before any launch); T*topk <= 2048.
 * ---------------------------------------------------------------------- */
int64_t moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t hidden, int64_t inter);
int moe_ffn_q4k_q6k(const void *gate, const void *up, const void *down, const float *x,
                    const int32_t *ids, const float *wts, float *y, void *ws, int64_t ws_bytes,
                    int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E,
                    qmv_stream_t stream);

/* The same layer without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): h lives in a library-owned device array
 * of QMV_NOALLOC_SCRATCH_BYTES, one per GPU, held from the first call on
 * that GPU until the process ends; the call allocates and frees nothing.
 * Operands, limits and results as moe_ffn_q4k_q6k (the same kernels; y is
 * bit-identical to it), run on the device current at the call, which must
 * be the stream's. Needs moe_ffn_workspace_bytes(T, topk, hidden, inter) <=
 * QMV_NOALLOC_SCRATCH_BYTES, else QMV_EUNSUPPORTED before any launch.
 * Calls share their GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialized by the caller.
 * QMV_ELAUNCH also if the array's device address cannot be obtained. */
#define QMV_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_ffn_q4k_q6k_noalloc(const void *gate, const void *up, const void *down, const float *x, const int32_t *ids,
                            const float *wts, float *y, int64_t T, int64_t topk, int64_t hidden, int64_t inter,
                            int64_t E, qmv_stream_t stream);

/* The same layer with the router fused into the gate/up gather (the
 * indexed-MoE design of hanzo-ml `src/vulkan_backend.rs`: `moe_route_vk`
 * softmax + top-k + renormalize feeding `moe_matvec_gpu` with ids kept on
 * the device): every workgroup of the gather routes logits f32[T, E] itself
 * (moe_route semantics: ties to the lower expert, NaN below every number)
 * and groups the slots by expert; ids int32[T, topk] and wts f32[T, topk]
 * are written as outputs and read by the down pass. For E > 256 or T > 8
 * the router runs as its own kernel first (same ids; measured faster there). Operands otherwise as
 * moe_ffn_q4k_q6k (same workspace). */
int moe_ffn_routed_q4k_q6k(const void *gate, const void *up, const void *down, const float *x, const float *logits,
                           int32_t *ids, float *wts, float *y, void *ws, int64_t ws_bytes, int64_t T, int64_t topk,
                           int64_t hidden, int64_t inter, int64_t E, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * q8-activation MoE decode variant (the int8-dot gathers of hanzo-ml
 * `src/vulkan_backend.rs`: activation quantized once by quantize_act_q8,
 * dp4a gate/up and down over resident banks, ids on the device):
 *   moe_qmv_q4k_q8: y[s, r] = sum_c W_deq[ids[s], r, c] * xs[a, c/32] * xq[a, c]
 *                   (integer block sums of codes x xq, as in qmv_q4k_q8)
 *   moe_qmv_q6k_q8: the same over a Q6_K bank; q - 32 enters the int8 dot
 *                   as a signed byte (xsum is not needed)
 * a = s / x_div. Layout, limits and errors as moe_qmv_q4k / moe_qmv_q6k;
 * xq 16-byte aligned, xs / xsum 4-byte.
 * ---------------------------------------------------------------------- */
int moe_qmv_q4k_q8(const void *bank, const int8_t *xq, const float *xs, const float *xsum, int64_t x_div,
                   const int32_t *ids, float *y, int64_t nslots, int64_t n, int64_t k, int64_t E,
                   qmv_stream_t stream);
int moe_qmv_q6k_q8(const void *bank, const int8_t *xq, const float *xs, int64_t x_div, const int32_t *ids,
                   float *y, int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream);

/* The MoE layer with q8 activations on both projections: x quantized
 * (quantize_act_q8 per 32 values of each token row), h = silu(gate) * up
 * from int8 dots (f32), h quantized (per 32 values of each slot row), down
 * on int8 dots with the weighted combine. Up to 8 tokens two launches
 * (each workgroup quantizes the rows it stages), above that four (x and h
 * quantized by launches of their own); both use the steps of
 * quantize_act_q8, so the codes and scales are the same bits either way.
 * Same operands as moe_ffn_q4k_q6k; ws: moe_ffn_q8_workspace_bytes() bytes,
 * 256-byte aligned. Limits as moe_ffn_q4k_q6k (1 <= topk <= 64). */
int64_t moe_ffn_q8_workspace_bytes(int64_t T, int64_t topk, int64_t hidden, int64_t inter);
int moe_ffn_q4k_q6k_q8(const void *gate, const void *up, const void *down, const float *x, const int32_t *ids,
                       const float *wts, float *y, void *ws, int64_t ws_bytes, int64_t T, int64_t topk,
                       int64_t hidden, int64_t inter, int64_t E, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * Q4_K prefill GEMM (`mmq_q4k_rt_gpu`: affine Q4_K x q8 activation,
 * epilogue xs*(D*dot - M*xsum)):
 *   Y[i, r] = sum_b ( xs[i,b]*d_r*sc_rj*S[i,r,b] - xsum[i,b]*dmin_r*m_rj ),
 *   S[i,r,b] = sum_{l<32} xq[i, 32b+l] * q[r, 32b+l]  (an integer, exact),
 * each block's integer dot (with sc folded in) formed on the f16 matrix
 * cores, which hold the integer operands exactly.
 * w: n*(k/256)*144 bytes; xq: int8[m, k]; xs, xsum: f32[m, k/32];
 * Y: f32[m, n]. bm = rows of Y per workgroup tile: 64 (weights decoded
 * straight into matrix fragments, activations staged once per tile; the
 * fastest at m = 512), 128 or 256 (weights and activations both staged).
 * k % 256 == 0; m, n >= 1 (ragged tiles are masked).
 * ---------------------------------------------------------------------- */
int qmm_q4k(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y,
            int64_t m, int64_t n, int64_t k, int bm, qmv_stream_t stream);

/* The same product with each block's integer dot on the int8 matrix
 * instructions (the int8 MMQ tiles of `mul_mm_q4k_tiled_dp4a`, as
 * `mmq_q4k_rt_gpu` benches them): the bm = 64 tile of qmm_q4k with the
 * codes q and xq as int8 operands (T = sum q*xq exact in int32) and the
 * scales sc*xs applied per output and block on the vector ALU. A comparison
 * form: qmm_q4k(bm = 64) is the faster one on gfx950, because the 6-bit
 * sub-block scale rides in its f16 operand and not in an int8 one.
 * Operands and results as qmm_q4k; n*(k/256)*144 and m*k below 2^32 (else
 * QMV_EUNSUPPORTED). */
int qmm_q4k_i8(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y, int64_t m, int64_t n,
               int64_t k, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * The same Q4_K prefill product (`mmq_q4k_rt_gpu` on its q8 activation),
 *   Y[i, r] = sum_c W_deq[r, c] * xs[i, c/32] * xq[i, c],
 * formed from the dequantized activation instead of the integer block dots:
 * a pre-pass writes each row of xs*xq, scaled by a power of two that puts
 * the row's largest magnitude in [2^14, 2^15), as two f16 halves (high part
 * and the f16 of the remainder: 22 bits of each value) into ws, then one
 * GEMM accumulates whole superblocks on the f16 matrix cores (two MFMAs per
 * block, no per-block epilogue) and undoes the row scale exactly. Same
 * operands and results as qmm_q4k to f32 accuracy; two launches.
 * ws: qmm_q4k_split_workspace_bytes(m, k) bytes (m*k*4 plus row scales),
 * 256-byte aligned, caller-owned, overwritten. k % 256 == 0; m*k*2 and
 * n*(k/256)*144 below 2^32 (else QMV_EUNSUPPORTED); w and xq 16-byte
 * aligned, the rest 4-byte. */
int64_t qmm_q4k_split_workspace_bytes(int64_t m, int64_t k); /* -1 for invalid shapes */
int qmm_q4k_split(const void *w, const int8_t *xq, const float *xs, const float *xsum, float *y, void *ws,
                  int64_t ws_bytes, int64_t m, int64_t n, int64_t k, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * Expert-indexed Q4_K prefill GEMM on a q8 activation (the MoE prefill twin
 * of moe_qmv_q4k: `check_mmq_q4k_id` of hanzo-kernel `src/main.rs`,
 * expert-indexed MMQ with its slot grouping):
 *   y[s, r] = sum_c W_deq[ids[s], r, c] * xs[a, c/32] * xq[a, c],
 *   a = s / x_div (x_div = topk: one activation row per token),
 * with the epilogue of qmm_q4k (f16 matrix cores on exact integer operands).
 * bank: E*n*(k/256)*144 bytes, expert-major; xq: int8[ceil(nslots/x_div), k];
 * xs, xsum: f32[ceil(nslots/x_div), k/32] (quantize_act_q8); ids:
 * int32[nslots]; y: f32[nslots, n], every row written (a slot whose expert
 * is outside [0, E) gets a zero row). Slots are grouped by expert on the
 * device (each expert's rows are read once per tile of its slots: 32 slots
 * whose activation rows stay in LDS for k <= 2048, 64 above); no
 * workspace, no host synchronization.
 * k % 256 == 0; 1 <= E <= 1024; 1 <= nslots <= 2^20; bank and xq 16-byte
 * aligned, the rest 4-byte.
 * ---------------------------------------------------------------------- */
int moe_qmm_q4k(const void *bank, const int8_t *xq, const float *xs, const float *xsum, int64_t x_div,
                const int32_t *ids, float *y, int64_t nslots, int64_t n, int64_t k, int64_t E,
                qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * Q6_K prefill GEMM on a q8 activation (hanzo-ml `src/vulkan_backend.rs`,
 * `matmul_q6k_gpu`: weights stay quantized, each decoded value serves a
 * tile of rows; its int8 tile `mul_mm_q6k_tiled_dp4a` takes quantize_act_q8
 * output):
 *   y[i, r] = sum_c W_deq[r, c] * xs[i, c/32] * xq[i, c].
 * w: n*(k/256)*210 bytes; xq: int8[m, k]; xs: f32[m, k/32]; y: f32[m, n].
 * Each 16-value sub-block's integer dot runs on the f16 matrix cores, the
 * int8 sub-scales and xs in an exact epilogue. k % 256 == 0; xq 16-byte
 * aligned, w 2-byte, the rest 4-byte.
 * ---------------------------------------------------------------------- */
int qmm_q6k(const void *w, const int8_t *xq, const float *xs, float *y, int64_t m, int64_t n, int64_t k,
            qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * Q8_0 prefill GEMM on a q8 activation (hanzo-ml `src/vulkan_backend.rs`:
 * the native Q8_0 blocks of `matvec_q8_0_gpu`, kept quantized at m > 1 as
 * `matmul_q4_0_gpu` keeps Q4_0):
 *   y[i, r] = sum_c W_deq[r, c] * xs[i, c/32] * xq[i, c].
 * w: n*(k/32)*34 bytes (f16 d, then 32 int8 codes per block); xq: int8[m, k];
 * xs: f32[m, k/32] (quantize_act_q8); y: f32[m, n], every element written.
 * The integer dot of each 32-value block runs exactly on the f16 matrix
 * cores; d and xs scale it in the epilogue. k % 256 == 0; xq 16-byte
 * aligned, w 2-byte, the rest 4-byte. Errors: QMV_EINVAL (null pointer,
 * m or n < 1, bad k), QMV_EUNSUPPORTED (m, n > 2^24, k > 2^20 or
 * m*k > 2^34), QMV_EALIGN; nothing is launched on an error.
 * ---------------------------------------------------------------------- */
int qmm_q8_0(const void *w, const int8_t *xq, const float *xs, float *y, int64_t m, int64_t n, int64_t k,
             qmv_stream_t stream);

/* Expert-indexed Q6_K prefill GEMM (the MoE down projection at m > 1;
 * `matmul_q6k_gpu_off` on one expert's slice of a resident bank, slots
 * grouped by expert on the device as in moe_qmm_q4k):
 *   moe_qmm_q6k:     y[s, r] = sum_c W_deq[ids[s], r, c] * xs[a, c/32] * xq[a, c]
 *   moe_qmm_q6k_f32: y[s, r] = sum_c W_deq[ids[s], r, c] * x[a, c]
 * with a = s / x_div. The f32 form splits each activation into two f16
 * halves on the matrix cores, under a power of two per activation row for
 * k <= 1024 (the rows of a workgroup's 32 slots then stay in LDS) and per 32
 * values above, which keeps f32 accuracy. bank: E*n*(k/256)*210 bytes; y:
 * f32[nslots, n], every row
 * written (zero for an expert outside [0, E)). k % 256 == 0; 1 <= E <= 1024;
 * nslots <= 2^20; xq and x 16-byte aligned, bank 2-byte, the rest 4-byte. */
int moe_qmm_q6k(const void *bank, const int8_t *xq, const float *xs, int64_t x_div, const int32_t *ids, float *y,
                int64_t nslots, int64_t n, int64_t k, int64_t E, qmv_stream_t stream);
int moe_qmm_q6k_f32(const void *bank, const float *x, int64_t x_div, const int32_t *ids, float *y, int64_t nslots,
                    int64_t n, int64_t k, int64_t E, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * MoE layer at prefill (the same layer as moe_ffn_q4k_q6k at m > 1, on the
 * pages' prefill path: the token activations are quantized to q8 once and
 * the expert-indexed MMQ runs gate and up, `check_mmq_q4k_id` of
 * hanzo-kernel `src/main.rs`; the down projection is the Q6_K prefill GEMM
 * on one expert of the bank, `matmul_q6k_gpu_off` of hanzo-ml
 * `src/vulkan_backend.rs`):
 *   x_deq = quantize_act_q8(x) dequantized; for slot s = topk*t + j with
 *   e = ids[t, j] in [0, E): h = silu(Wg[e] x_deq[t]) * (Wu[e] x_deq[t]),
 *   d = Wd[e] h (h kept in f32); y[t] = sum_j wts[t, j] * d_s.
 * Same operands as moe_ffn_q4k_q6k; ws: moe_ffn_prefill_workspace_bytes()
 * bytes of device scratch (q8 activation, tile table and its 32-slot
 * segments, h, d), 256-byte
 * aligned, caller-owned, contents undefined after the call. Slots are
 * grouped by expert on the device; nothing is synchronized with the host.
 * hidden, inter: multiples of 256 (<= 65536); 1 <= E <= 1024; T <= 65535;
 * T*topk <= 2^20. gate, up, x, y 16-byte aligned; down 2-byte; rest 4-byte.
 * Any topk >= 1 is accepted. Up to 256 slots (with topk <= 64, hidden,
 * inter <= 4096 and down 16-byte aligned) the
 * same arithmetic runs on the expert-grouped decode gathers, which stream
 * the bank faster there; a token's output then agrees across batch sizes
 * to f32 rounding rather than bit for bit.
 * ---------------------------------------------------------------------- */
int64_t moe_ffn_prefill_workspace_bytes(int64_t T, int64_t topk, int64_t hidden, int64_t inter, int64_t E);
int moe_ffn_prefill_q4k_q6k(const void *gate, const void *up, const void *down, const float *x, const int32_t *ids,
                            const float *wts, float *y, void *ws, int64_t ws_bytes, int64_t T, int64_t topk,
                            int64_t hidden, int64_t inter, int64_t E, qmv_stream_t stream);

/* ------------------------------------------------------------------------
 * Measurement probe (not a step of the path): one launch that reads `bytes`
 * of device memory once with 16-byte loads and writes nothing (sink, one
 * u32, is only written for a value ordinary data does not give). The pages
 * price their kernels against a bandwidth measured on the device
 * (hanzo-ml `src/vulkan_backend.rs`, the roofline profiling option and its
 * start-up copy-bandwidth measurement); this probe gives the fastest plain
 * read of a given size to compare a matvec of that size with.
 * workgroups: grid size (256 threads each, 1 .. 2^20); unroll: loads in
 * flight per thread, 1, 2, 4 or 8. bytes % 16 == 0, buf 16-byte aligned,
 * sink 4-byte aligned; QMV_EINVAL / QMV_EALIGN otherwise.
 * ---------------------------------------------------------------------- */
int qmv_roofline_read(const void *buf, int64_t bytes, int64_t workgroups, int64_t unroll, uint32_t *sink,
                      qmv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
