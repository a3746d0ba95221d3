"""Python binding of libqmv.so (include/qmv.h): argument marshalling only.

Every function takes torch tensors that already live on a ROCm device,
passes their raw pointers and sizes to the C ABI on the current HIP stream
(or the one given) and raises QmvError on a non-zero status. All arithmetic
runs in the gfx950 kernels of libqmv.so; there is no fallback of any kind:
if the library cannot be loaded, importing this package raises.

torch is imported first so that the HIP runtime it ships (soname
libamdhip64.so.7) is the one libqmv.so binds to.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime libqmv.so links against)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -m moe_ggml_block_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGS = {
    "qmv_q8_0": [_vp, _vp, _vp, _i64, _i64, _vp],
    "qmv_q4k": [_vp, _vp, _vp, _i64, _i64, _vp],
    "qmv_q6k": [_vp, _vp, _vp, _i64, _i64, _vp],
    "qmv_q4_0": [_vp, _vp, _vp, _i64, _i64, _vp],
    "qmv_q5k": [_vp, _vp, _vp, _i64, _i64, _vp],
    "quantize_act_q8": [_vp, _vp, _vp, _vp, _i64, _i64, _vp],
    "qmv_q4k_q8": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp],
    "qmv_q4k_q8x": [_vp, _vp, _vp, _i64, _i64, _vp],
    "qmv_q4k_qx": [_vp] * 6 + [_i64, _i64, _vp],
    "qmv_debug_blocksums_q4k_q8": [_vp, _vp, _vp, _i64, _i64, _vp],
    "moe_route": [_vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "moe_gate_route": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_qmv_q4k": [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_qmv_q6k": [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_qmv_q8_0": [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_ffn_q4k_q6k": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp],
    "moe_ffn_q4k_q6k_noalloc": [_vp] * 7 + [_i64] * 5 + [_vp],
    "qmm_q4k": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp],
    "qmm_q4k_i8": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "qmm_q4k_split": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_qmm_q4k": [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "qmm_q6k": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "qmm_q8_0": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "moe_qmm_q6k": [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_qmm_q6k_f32": [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_ffn_prefill_q4k_q6k": [_vp] * 8 + [_i64] * 6 + [_vp],
    "moe_qmv_q4k_q8": [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_qmv_q6k_q8": [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "moe_ffn_q4k_q6k_q8": [_vp] * 8 + [_i64] * 6 + [_vp],
    "moe_ffn_routed_q4k_q6k": [_vp] * 9 + [_i64] * 6 + [_vp],
    "moe_block_q4k_q6k": [_vp] * 10 + [_i64] * 6 + [_vp],
    "qmv_roofline_read": [_vp, _i64, _i64, _i64, _vp, _vp],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _i32
_lib.moe_ffn_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
_lib.moe_ffn_workspace_bytes.restype = _i64
_lib.moe_ffn_prefill_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64]
_lib.moe_ffn_prefill_workspace_bytes.restype = _i64
_lib.moe_ffn_q8_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
_lib.moe_ffn_q8_workspace_bytes.restype = _i64
_lib.qmm_q4k_split_workspace_bytes.argtypes = [_i64, _i64]
_lib.qmm_q4k_split_workspace_bytes.restype = _i64
_lib.qmv_version.restype = ctypes.c_char_p
_lib.qmv_strerror.argtypes = [_i32]
_lib.qmv_strerror.restype = ctypes.c_char_p

EXPORTS = tuple(_SIGS) + ("moe_ffn_workspace_bytes", "moe_ffn_prefill_workspace_bytes",
                          "moe_ffn_q8_workspace_bytes", "qmm_q4k_split_workspace_bytes", "qmv_version",
                          "qmv_strerror")

BLOCK = {"q8_0": (32, 34), "q4k": (256, 144), "q6k": (256, 210), "q4_0": (32, 18), "q5k": (256, 176)}


class QmvError(RuntimeError):
    pass


def version() -> str:
    return _lib.qmv_version().decode()


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise QmvError(f"{name}: status {rc} ({_lib.qmv_strerror(rc).decode()})")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def row_bytes(fmt: str, k: int) -> int:
    bw, bb = BLOCK[fmt]
    return k // bw * bb


def _need(t, numel_bytes, name):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < numel_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {numel_bytes}")


# ----------------------------------------------------------------- matvecs
def _dense(name, fmt, w, x, n, k, y=None, stream=None):
    _need(w, n * row_bytes(fmt, k), "w")
    _need(x, 4 * k, "x")
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    _need(y, 4 * n, "y")
    _check(getattr(_lib, name)(_p(w), _p(x), _p(y), n, k, _stream(stream)), name)
    return y


def qmv_q8_0(w, x, n, k, y=None, stream=None):
    return _dense("qmv_q8_0", "q8_0", w, x, n, k, y, stream)


def qmv_q4k(w, x, n, k, y=None, stream=None):
    return _dense("qmv_q4k", "q4k", w, x, n, k, y, stream)


def qmv_q6k(w, x, n, k, y=None, stream=None):
    return _dense("qmv_q6k", "q6k", w, x, n, k, y, stream)


def qmv_q4_0(w, x, n, k, y=None, stream=None):
    return _dense("qmv_q4_0", "q4_0", w, x, n, k, y, stream)


def qmv_q5k(w, x, n, k, y=None, stream=None):
    return _dense("qmv_q5k", "q5k", w, x, n, k, y, stream)


def quantize_act_q8(x, m, k, out=None, stream=None):
    _need(x, 4 * m * k, "x")
    if out is None:
        out = (torch.empty((m, k), dtype=torch.int8, device=x.device),
               torch.empty((m, k // 32), dtype=torch.float32, device=x.device),
               torch.empty((m, k // 32), dtype=torch.float32, device=x.device))
    xq, xs, xsum = out
    _check(_lib.quantize_act_q8(_p(x), _p(xq), _p(xs), _p(xsum), m, k, _stream(stream)), "quantize_act_q8")
    return xq, xs, xsum


def qmv_q4k_q8(w, xq, xs, xsum, n, k, y=None, stream=None):
    _need(w, n * row_bytes("q4k", k), "w")
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=xq.device)
    _check(_lib.qmv_q4k_q8(_p(w), _p(xq), _p(xs), _p(xsum), _p(y), n, k, _stream(stream)), "qmv_q4k_q8")
    return y


def qmv_q4k_q8x(w, x, n, k, y=None, stream=None):
    """int8-dot Q4_K matvec from an f32 activation, quantized inside the kernel."""
    return _dense("qmv_q4k_q8x", "q4k", w, x, n, k, y, stream)


def qmv_q4k_qx(w, x, n, k, y=None, out=None, stream=None):
    """f32 Q4_K matvec that also returns quantize_act_q8(x) for one row: (y, (xq, xs, xsum))."""
    _need(w, n * row_bytes("q4k", k), "w")
    _need(x, 4 * k, "x")
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    _need(y, 4 * n, "y")
    if out is None:
        out = (torch.empty((1, k), dtype=torch.int8, device=x.device),
               torch.empty((1, k // 32), dtype=torch.float32, device=x.device),
               torch.empty((1, k // 32), dtype=torch.float32, device=x.device))
    xq, xs, xsum = out
    _need(xq, k, "xq")
    _need(xs, 4 * (k // 32), "xs")
    _need(xsum, 4 * (k // 32), "xsum")
    _check(_lib.qmv_q4k_qx(_p(w), _p(x), _p(y), _p(xq), _p(xs), _p(xsum), n, k, _stream(stream)), "qmv_q4k_qx")
    return y, (xq, xs, xsum)


def qmv_debug_blocksums_q4k_q8(w, xq, n, k, stream=None):
    sums = torch.empty((n, k // 32), dtype=torch.int32, device=xq.device)
    _check(_lib.qmv_debug_blocksums_q4k_q8(_p(w), _p(xq), _p(sums), n, k, _stream(stream)),
           "qmv_debug_blocksums_q4k_q8")
    return sums


# --------------------------------------------------------------------- MoE
def moe_route(logits, T, E, topk, out=None, stream=None):
    _need(logits, 4 * T * E, "logits")
    if out is None:
        out = (torch.empty((T, topk), dtype=torch.int32, device=logits.device),
               torch.empty((T, topk), dtype=torch.float32, device=logits.device))
    ids, wts = out
    _check(_lib.moe_route(_p(logits), _p(ids), _p(wts), T, E, topk, _stream(stream)), "moe_route")
    return ids, wts


def moe_gate_route(wr, x, T, E, hidden, topk, out=None, stream=None):
    """Router gate GEMV (logits = x wr^T in f32) then moe_route: (logits, ids, wts)."""
    _need(wr, 4 * E * hidden, "wr")
    _need(x, 4 * T * hidden, "x")
    if out is None:
        out = (torch.empty((T, E), dtype=torch.float32, device=x.device),
               torch.empty((T, topk), dtype=torch.int32, device=x.device),
               torch.empty((T, topk), dtype=torch.float32, device=x.device))
    logits, ids, wts = out
    _need(logits, 4 * T * E, "logits")
    _need(ids, 4 * T * topk, "ids")
    _need(wts, 4 * T * topk, "wts")
    _check(_lib.moe_gate_route(_p(wr), _p(x), _p(logits), _p(ids), _p(wts), T, E, hidden, topk,
                               _stream(stream)), "moe_gate_route")
    return logits, ids, wts


def _moe(name, fmt, bank, x, x_div, ids, nslots, n, k, E, y, stream):
    _need(bank, E * n * row_bytes(fmt, k), "bank")
    _need(ids, 4 * nslots, "ids")
    if y is None:
        y = torch.empty((nslots, n), dtype=torch.float32, device=x.device)
    _check(getattr(_lib, name)(_p(bank), _p(x), x_div, _p(ids), _p(y), nslots, n, k, E, _stream(stream)), name)
    return y


def moe_qmv_q4k(bank, x, x_div, ids, nslots, n, k, E, y=None, stream=None):
    return _moe("moe_qmv_q4k", "q4k", bank, x, x_div, ids, nslots, n, k, E, y, stream)


def moe_qmv_q6k(bank, x, x_div, ids, nslots, n, k, E, y=None, stream=None):
    return _moe("moe_qmv_q6k", "q6k", bank, x, x_div, ids, nslots, n, k, E, y, stream)


def moe_qmv_q8_0(bank, x, x_div, ids, nslots, n, k, E, y=None, stream=None):
    return _moe("moe_qmv_q8_0", "q8_0", bank, x, x_div, ids, nslots, n, k, E, y, stream)


def moe_ffn_workspace_bytes(T, topk, hidden, inter) -> int:
    return int(_lib.moe_ffn_workspace_bytes(T, topk, hidden, inter))


def moe_ffn_q4k_q6k(gate, up, down, x, ids, wts, T, topk, hidden, inter, E, y=None, ws=None, stream=None):
    nb = moe_ffn_workspace_bytes(T, topk, hidden, inter)
    if ws is None:
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((T, hidden), dtype=torch.float32, device=x.device)
    _need(gate, E * inter * row_bytes("q4k", hidden), "gate")
    _need(up, E * inter * row_bytes("q4k", hidden), "up")
    _need(down, E * hidden * row_bytes("q6k", inter), "down")
    _check(_lib.moe_ffn_q4k_q6k(_p(gate), _p(up), _p(down), _p(x), _p(ids), _p(wts), _p(y), _p(ws),
                                ws.numel() * ws.element_size(), T, topk, hidden, inter, E, _stream(stream)),
           "moe_ffn_q4k_q6k")
    return y


def roofline_read(buf, nbytes, workgroups, unroll, sink, stream=None):
    """Measurement probe: one launch reading nbytes of buf (no result)."""
    _need(buf, nbytes, "buf")
    _check(_lib.qmv_roofline_read(_p(buf), nbytes, workgroups, unroll, _p(sink), _stream(stream)),
           "qmv_roofline_read")


# the layer's scratch limit (bytes of h) for moe_ffn_q4k_q6k_noalloc
NOALLOC_SCRATCH_BYTES = 4 << 20


def moe_ffn_q4k_q6k_noalloc(gate, up, down, x, ids, wts, T, topk, hidden, inter, E, y=None, stream=None):
    """The decode MoE layer with h in the library's own per-GPU scratch (no workspace)."""
    if y is None:
        y = torch.empty((T, hidden), dtype=torch.float32, device=x.device)
    _need(gate, E * inter * row_bytes("q4k", hidden), "gate")
    _need(up, E * inter * row_bytes("q4k", hidden), "up")
    _need(down, E * hidden * row_bytes("q6k", inter), "down")
    _need(x, 4 * T * hidden, "x")
    _need(ids, 4 * T * topk, "ids")
    _need(wts, 4 * T * topk, "wts")
    _need(y, 4 * T * hidden, "y")
    _check(_lib.moe_ffn_q4k_q6k_noalloc(_p(gate), _p(up), _p(down), _p(x), _p(ids), _p(wts), _p(y), T, topk,
                                        hidden, inter, E, _stream(stream)), "moe_ffn_q4k_q6k_noalloc")
    return y


# ----------------------------------------------------------------- prefill
def qmm_q4k(w, xq, xs, xsum, m, n, k, bm=128, y=None, stream=None):
    _need(w, n * row_bytes("q4k", k), "w")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _check(_lib.qmm_q4k(_p(w), _p(xq), _p(xs), _p(xsum), _p(y), m, n, k, bm, _stream(stream)), "qmm_q4k")
    return y


def qmm_q4k_i8(w, xq, xs, xsum, m, n, k, y=None, stream=None):
    """qmm_q4k with the block dots on the int8 matrix instructions (comparison form)."""
    _need(w, n * row_bytes("q4k", k), "w")
    _need(xq, m * k, "xq")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _check(_lib.qmm_q4k_i8(_p(w), _p(xq), _p(xs), _p(xsum), _p(y), m, n, k, _stream(stream)), "qmm_q4k_i8")
    return y


def qmm_q4k_split_workspace_bytes(m, k) -> int:
    return int(_lib.qmm_q4k_split_workspace_bytes(m, k))


def qmm_q4k_split(w, xq, xs, xsum, m, n, k, y=None, ws=None, stream=None):
    """Q4_K prefill GEMM on the dequantized q8 activation split into two f16
    halves (pre-pass into ws, then one GEMM): y = deq(xq, xs) . W^T."""
    _need(w, n * row_bytes("q4k", k), "w")
    _need(xq, m * k, "xq")
    _need(xs, 4 * m * (k // 32), "xs")
    _need(xsum, 4 * m * (k // 32), "xsum")
    nb = qmm_q4k_split_workspace_bytes(m, k)
    if ws is None:
        ws = torch.empty(nb, dtype=torch.uint8, device=xq.device)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _need(y, 4 * m * n, "y")
    _check(_lib.qmm_q4k_split(_p(w), _p(xq), _p(xs), _p(xsum), _p(y), _p(ws), ws.numel() * ws.element_size(),
                              m, n, k, _stream(stream)), "qmm_q4k_split")
    return y


def moe_qmm_q4k(bank, xq, xs, xsum, x_div, ids, nslots, n, k, E, y=None, stream=None):
    """Expert-indexed Q4_K prefill GEMM: y[s] = W[ids[s]] . deq(xq, xs)[s // x_div]."""
    rows = (nslots + x_div - 1) // x_div
    _need(bank, E * n * row_bytes("q4k", k), "bank")
    _need(xq, rows * k, "xq")
    _need(xs, 4 * rows * (k // 32), "xs")
    _need(xsum, 4 * rows * (k // 32), "xsum")
    _need(ids, 4 * nslots, "ids")
    if y is None:
        y = torch.empty((nslots, n), dtype=torch.float32, device=xq.device)
    _need(y, 4 * nslots * n, "y")
    _check(_lib.moe_qmm_q4k(_p(bank), _p(xq), _p(xs), _p(xsum), x_div, _p(ids), _p(y), nslots, n, k, E,
                            _stream(stream)), "moe_qmm_q4k")
    return y


def qmm_q6k(w, xq, xs, m, n, k, y=None, stream=None):
    """Q6_K prefill GEMM on a q8 activation: y = deq(xq, xs) . W^T."""
    _need(w, n * row_bytes("q6k", k), "w")
    _need(xq, m * k, "xq")
    _need(xs, 4 * m * (k // 32), "xs")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _need(y, 4 * m * n, "y")
    _check(_lib.qmm_q6k(_p(w), _p(xq), _p(xs), _p(y), m, n, k, _stream(stream)), "qmm_q6k")
    return y


def qmm_q8_0(w, xq, xs, m, n, k, y=None, stream=None):
    """Q8_0 prefill GEMM on a q8 activation: y = deq(xq, xs) . W^T."""
    _need(w, n * row_bytes("q8_0", k), "w")
    _need(xq, m * k, "xq")
    _need(xs, 4 * m * (k // 32), "xs")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _need(y, 4 * m * n, "y")
    _check(_lib.qmm_q8_0(_p(w), _p(xq), _p(xs), _p(y), m, n, k, _stream(stream)), "qmm_q8_0")
    return y


def moe_qmm_q6k(bank, xq, xs, x_div, ids, nslots, n, k, E, y=None, stream=None):
    """Expert-indexed Q6_K prefill GEMM on a q8 activation."""
    rows = (nslots + x_div - 1) // x_div
    _need(bank, E * n * row_bytes("q6k", k), "bank")
    _need(xq, rows * k, "xq")
    _need(xs, 4 * rows * (k // 32), "xs")
    _need(ids, 4 * nslots, "ids")
    if y is None:
        y = torch.empty((nslots, n), dtype=torch.float32, device=xq.device)
    _need(y, 4 * nslots * n, "y")
    _check(_lib.moe_qmm_q6k(_p(bank), _p(xq), _p(xs), x_div, _p(ids), _p(y), nslots, n, k, E, _stream(stream)),
           "moe_qmm_q6k")
    return y


def moe_qmm_q6k_f32(bank, x, x_div, ids, nslots, n, k, E, y=None, stream=None):
    """Expert-indexed Q6_K prefill GEMM on an f32 activation."""
    rows = (nslots + x_div - 1) // x_div
    _need(bank, E * n * row_bytes("q6k", k), "bank")
    _need(x, 4 * rows * k, "x")
    _need(ids, 4 * nslots, "ids")
    if y is None:
        y = torch.empty((nslots, n), dtype=torch.float32, device=x.device)
    _need(y, 4 * nslots * n, "y")
    _check(_lib.moe_qmm_q6k_f32(_p(bank), _p(x), x_div, _p(ids), _p(y), nslots, n, k, E, _stream(stream)),
           "moe_qmm_q6k_f32")
    return y


def moe_ffn_prefill_workspace_bytes(T, topk, hidden, inter, E) -> int:
    return int(_lib.moe_ffn_prefill_workspace_bytes(T, topk, hidden, inter, E))


def moe_ffn_prefill_q4k_q6k(gate, up, down, x, ids, wts, T, topk, hidden, inter, E, y=None, ws=None,
                            stream=None):
    """MoE layer at prefill: q8 activation, expert-grouped gate/up and down GEMMs, weighted combine."""
    nb = moe_ffn_prefill_workspace_bytes(T, topk, hidden, inter, E)
    if ws is None:
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((T, hidden), dtype=torch.float32, device=x.device)
    _need(gate, E * inter * row_bytes("q4k", hidden), "gate")
    _need(up, E * inter * row_bytes("q4k", hidden), "up")
    _need(down, E * hidden * row_bytes("q6k", inter), "down")
    _need(x, 4 * T * hidden, "x")
    _need(ids, 4 * T * topk, "ids")
    _need(wts, 4 * T * topk, "wts")
    _need(y, 4 * T * hidden, "y")
    _check(_lib.moe_ffn_prefill_q4k_q6k(_p(gate), _p(up), _p(down), _p(x), _p(ids), _p(wts), _p(y), _p(ws),
                                        ws.numel() * ws.element_size(), T, topk, hidden, inter, E,
                                        _stream(stream)), "moe_ffn_prefill_q4k_q6k")
    return y


def moe_ffn_routed_q4k_q6k(gate, up, down, x, logits, T, topk, hidden, inter, E, out=None, ws=None,
                           stream=None):
    """MoE layer with the router fused into the gate/up gather: (y, ids, wts)."""
    nb = moe_ffn_workspace_bytes(T, topk, hidden, inter)
    if ws is None:
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    if out is None:
        out = (torch.empty((T, hidden), dtype=torch.float32, device=x.device),
               torch.empty((T, topk), dtype=torch.int32, device=x.device),
               torch.empty((T, topk), dtype=torch.float32, device=x.device))
    y, ids, wts = out
    _need(gate, E * inter * row_bytes("q4k", hidden), "gate")
    _need(up, E * inter * row_bytes("q4k", hidden), "up")
    _need(down, E * hidden * row_bytes("q6k", inter), "down")
    _need(x, 4 * T * hidden, "x")
    _need(logits, 4 * T * E, "logits")
    _need(ids, 4 * T * topk, "ids")
    _need(wts, 4 * T * topk, "wts")
    _need(y, 4 * T * hidden, "y")
    _check(_lib.moe_ffn_routed_q4k_q6k(_p(gate), _p(up), _p(down), _p(x), _p(logits), _p(ids), _p(wts), _p(y),
                                       _p(ws), ws.numel() * ws.element_size(), T, topk, hidden, inter, E,
                                       _stream(stream)), "moe_ffn_routed_q4k_q6k")
    return y, ids, wts


def moe_block_q4k_q6k(wr, gate, up, down, x, T, topk, hidden, inter, E, out=None, ws=None, stream=None):
    """The MoE block from the hidden state: router gate GEMV + routed layer -> (y, logits, ids, wts)."""
    nb = moe_ffn_workspace_bytes(T, topk, hidden, inter)
    if ws is None:
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    if out is None:
        out = (torch.empty((T, hidden), dtype=torch.float32, device=x.device),
               torch.empty((T, E), dtype=torch.float32, device=x.device),
               torch.empty((T, topk), dtype=torch.int32, device=x.device),
               torch.empty((T, topk), dtype=torch.float32, device=x.device))
    y, logits, ids, wts = out
    _need(wr, 4 * E * hidden, "wr")
    _need(gate, E * inter * row_bytes("q4k", hidden), "gate")
    _need(up, E * inter * row_bytes("q4k", hidden), "up")
    _need(down, E * hidden * row_bytes("q6k", inter), "down")
    _need(x, 4 * T * hidden, "x")
    for t_, nbytes, nm in ((logits, 4 * T * E, "logits"), (ids, 4 * T * topk, "ids"), (wts, 4 * T * topk, "wts"),
                           (y, 4 * T * hidden, "y")):
        _need(t_, nbytes, nm)
    _check(_lib.moe_block_q4k_q6k(_p(wr), _p(gate), _p(up), _p(down), _p(x), _p(logits), _p(ids), _p(wts), _p(y),
                                  _p(ws), ws.numel() * ws.element_size(), T, topk, hidden, inter, E,
                                  _stream(stream)), "moe_block_q4k_q6k")
    return y, logits, ids, wts


def moe_qmv_q4k_q8(bank, xq, xs, xsum, x_div, ids, nslots, n, k, E, y=None, stream=None):
    """Expert-gather Q4_K matvec on a q8 activation (int8 dot products)."""
    rows = (nslots + x_div - 1) // x_div
    _need(bank, E * n * row_bytes("q4k", k), "bank")
    _need(xq, rows * k, "xq")
    _need(xs, 4 * rows * (k // 32), "xs")
    _need(xsum, 4 * rows * (k // 32), "xsum")
    _need(ids, 4 * nslots, "ids")
    if y is None:
        y = torch.empty((nslots, n), dtype=torch.float32, device=xq.device)
    _need(y, 4 * nslots * n, "y")
    _check(_lib.moe_qmv_q4k_q8(_p(bank), _p(xq), _p(xs), _p(xsum), x_div, _p(ids), _p(y), nslots, n, k, E,
                               _stream(stream)), "moe_qmv_q4k_q8")
    return y


def moe_qmv_q6k_q8(bank, xq, xs, x_div, ids, nslots, n, k, E, y=None, stream=None):
    """Expert-gather Q6_K matvec on a q8 activation (int8 dot products)."""
    rows = (nslots + x_div - 1) // x_div
    _need(bank, E * n * row_bytes("q6k", k), "bank")
    _need(xq, rows * k, "xq")
    _need(xs, 4 * rows * (k // 32), "xs")
    _need(ids, 4 * nslots, "ids")
    if y is None:
        y = torch.empty((nslots, n), dtype=torch.float32, device=xq.device)
    _need(y, 4 * nslots * n, "y")
    _check(_lib.moe_qmv_q6k_q8(_p(bank), _p(xq), _p(xs), x_div, _p(ids), _p(y), nslots, n, k, E,
                               _stream(stream)), "moe_qmv_q6k_q8")
    return y


def moe_ffn_q8_workspace_bytes(T, topk, hidden, inter) -> int:
    return int(_lib.moe_ffn_q8_workspace_bytes(T, topk, hidden, inter))


def moe_ffn_q4k_q6k_q8(gate, up, down, x, ids, wts, T, topk, hidden, inter, E, y=None, ws=None, stream=None):
    """MoE layer with q8 activations on both projections (int8 dot products)."""
    nb = moe_ffn_q8_workspace_bytes(T, topk, hidden, inter)
    if ws is None:
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((T, hidden), dtype=torch.float32, device=x.device)
    _need(gate, E * inter * row_bytes("q4k", hidden), "gate")
    _need(up, E * inter * row_bytes("q4k", hidden), "up")
    _need(down, E * hidden * row_bytes("q6k", inter), "down")
    _need(x, 4 * T * hidden, "x")
    _need(ids, 4 * T * topk, "ids")
    _need(wts, 4 * T * topk, "wts")
    _need(y, 4 * T * hidden, "y")
    _check(_lib.moe_ffn_q4k_q6k_q8(_p(gate), _p(up), _p(down), _p(x), _p(ids), _p(wts), _p(y), _p(ws),
                                   ws.numel() * ws.element_size(), T, topk, hidden, inter, E, _stream(stream)),
           "moe_ffn_q4k_q6k_q8")
    return y


def raw(name):
    """The raw ctypes function of an export (for tests of the C ABI itself)."""
    return getattr(_lib, name)
