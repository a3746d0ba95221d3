"""CPU oracle -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``liboracle.so`` (``oracle.c``): plain single-
threaded C that decodes Q8_0 / Q4_K / Q6_K blocks exactly and accumulates in
f64, reproduces the q8 activation quantizer in f32, ranks router logits by a
full sort and composes the MoE FFN layer. Only ``tests/``, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
this package; the GPU library never does and shares no code with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

Q8_0, Q4K, Q6K, Q4_0, Q5K = 0, 1, 2, 3, 4
_FMT = {"q8_0": Q8_0, "q4k": Q4K, "q6k": Q6K, "q4_0": Q4_0, "q5k": Q5K,
        Q8_0: Q8_0, Q4K: Q4K, Q6K: Q6K, Q4_0: Q4_0, Q5K: Q5K}
BLOCK_WEIGHTS = {Q8_0: 32, Q4K: 256, Q6K: 256, Q4_0: 32, Q5K: 256}
BLOCK_BYTES = {Q8_0: 34, Q4K: 144, Q6K: 210, Q4_0: 18, Q5K: 176}


def build() -> None:
    """Compile liboracle.so: plain C, no FP contraction, no fast-math, no SIMD flags."""
    src = os.path.join(_HERE, "oracle.c")
    cmd = ["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", src, "-o", _SO + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_half.argtypes = [ctypes.c_uint16]
    lib.oracle_half.restype = ctypes.c_double
    lib.oracle_dequant.argtypes = [i32, vp, i64, vp]
    lib.oracle_matvec.argtypes = [i32, vp, vp, i64, i64, vp, i64, vp]
    lib.oracle_quantize_act_q8.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.oracle_blocksums_q4k_q8.argtypes = [vp, vp, i64, i64, vp]
    lib.oracle_matvec_q8act.argtypes = [i32, vp, vp, vp, i64, i64, vp, i64, vp]
    lib.oracle_moe_route.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.oracle_moe_qmv.argtypes = [i32, vp, vp, i64, vp, i64, i64, i64, i64, vp]
    lib.oracle_moe_ffn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.oracle_qmm.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp, i64, vp]
    lib.oracle_gemv.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.oracle_moe_qmm.argtypes = [i32, vp, vp, vp, i64, vp, i64, i64, i64, i64, vp, i64, vp]
    lib.oracle_moe_ffn_q8x.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64, vp]
    lib.oracle_moe_ffn_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64, vp, vp, vp, vp]
    for name in ("oracle_dequant", "oracle_matvec", "oracle_quantize_act_q8",
                 "oracle_blocksums_q4k_q8", "oracle_matvec_q8act", "oracle_moe_route",
                 "oracle_moe_qmv", "oracle_moe_ffn", "oracle_qmm", "oracle_gemv", "oracle_moe_qmm", "oracle_moe_ffn_q8x", "oracle_moe_ffn_q8"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: error {rc}")


def half(bits: int) -> float:
    """O1: exact IEEE binary16 value of a 16-bit pattern, as f64."""
    return float(_load().oracle_half(bits))


def dequant(fmt, blocks: np.ndarray) -> np.ndarray:
    """O2: f64 values of raw blocks (any shape, flattened), one row per block."""
    fmt = _FMT[fmt]
    b = _c(blocks, np.uint8).reshape(-1)
    nb = b.size // BLOCK_BYTES[fmt]
    out = np.empty(nb * BLOCK_WEIGHTS[fmt], dtype=np.float64)
    _check(_load().oracle_dequant(fmt, _p(b), nb, _p(out)), "dequant")
    return out


def matvec(fmt, w: np.ndarray, x: np.ndarray, n: int, k: int, rows=None) -> np.ndarray:
    """O3: f64 y = W_deq x over all rows, or the listed rows."""
    fmt = _FMT[fmt]
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    r = None if rows is None else _c(rows, np.int64)
    cnt = n if r is None else r.size
    y = np.empty(cnt, dtype=np.float64)
    _check(_load().oracle_matvec(fmt, _p(w), _p(x), n, k, _p(r), cnt, _p(y)), "matvec")
    return y


def quantize_act_q8(x: np.ndarray, m: int, k: int):
    """O4: (xq int8[m,k], xs f32[m,k/32], xsum f32[m,k/32]) per the f32 recipe."""
    x = _c(x, np.float32)
    xq = np.empty((m, k), dtype=np.int8)
    xs = np.empty((m, k // 32), dtype=np.float32)
    xsum = np.empty((m, k // 32), dtype=np.float32)
    _check(_load().oracle_quantize_act_q8(_p(x), m, k, _p(xq), _p(xs), _p(xsum)), "quantize_act_q8")
    return xq, xs, xsum


def blocksums_q4k_q8(w: np.ndarray, xq: np.ndarray, n: int, k: int) -> np.ndarray:
    """O5: int64 S[n, k/32] = per-32 sums of Q4_K codes times q8 codes."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.int8)
    S = np.empty((n, k // 32), dtype=np.int64)
    _check(_load().oracle_blocksums_q4k_q8(_p(w), _p(xq), n, k, _p(S)), "blocksums")
    return S


def matvec_q8act(fmt, w, xq, xs, n: int, k: int, rows=None) -> np.ndarray:
    """O6: f64 y = W_deq x_deq with x_deq = xs * xq."""
    fmt = _FMT[fmt]
    w, xq, xs = _c(w, np.uint8), _c(xq, np.int8), _c(xs, np.float32)
    r = None if rows is None else _c(rows, np.int64)
    cnt = n if r is None else r.size
    y = np.empty(cnt, dtype=np.float64)
    _check(_load().oracle_matvec_q8act(fmt, _p(w), _p(xq), _p(xs), n, k, _p(r), cnt, _p(y)),
           "matvec_q8act")
    return y


def moe_route(logits: np.ndarray, T: int, E: int, topk: int):
    """O7: (ids int32[T,topk], w f64[T,topk])."""
    lg = _c(logits, np.float32)
    ids = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float64)
    _check(_load().oracle_moe_route(_p(lg), T, E, topk, _p(ids), _p(w)), "moe_route")
    return ids, w


def moe_qmv(fmt, bank, x, x_div: int, ids, nslots: int, n: int, k: int, E: int) -> np.ndarray:
    """f64 y[nslots, n]: expert-gather matvec, slot s reads x row s // x_div."""
    fmt = _FMT[fmt]
    bank, x, ids = _c(bank, np.uint8), _c(x, np.float32), _c(ids, np.int32)
    y = np.empty((nslots, n), dtype=np.float64)
    _check(_load().oracle_moe_qmv(fmt, _p(bank), _p(x), x_div, _p(ids), nslots, n, k, E, _p(y)),
           "moe_qmv")
    return y


def moe_ffn(gate, up, down, x, ids, wts, T: int, topk: int, hidden: int, inter: int, E: int):
    """O8: (y f64[T,hidden], h f64[T*topk,inter], dvec f64[T*topk,hidden])."""
    gate, up, down = _c(gate, np.uint8), _c(up, np.uint8), _c(down, np.uint8)
    x, ids, wts = _c(x, np.float32), _c(ids, np.int32), _c(wts, np.float32)
    y = np.empty((T, hidden), dtype=np.float64)
    h = np.empty((T * topk, inter), dtype=np.float64)
    d = np.empty((T * topk, hidden), dtype=np.float64)
    _check(_load().oracle_moe_ffn(_p(gate), _p(up), _p(down), _p(x), _p(ids), _p(wts), T, topk,
                                  hidden, inter, E, _p(h), _p(d), _p(y)), "moe_ffn")
    return y, h, d


def qmm(fmt, w, xq, xs, m: int, n: int, k: int, mrows=None) -> np.ndarray:
    """a11: f64 Y[rows, n] = X_deq W_deq^T for all activation rows or the listed ones."""
    fmt = _FMT[fmt]
    w, xq, xs = _c(w, np.uint8), _c(xq, np.int8), _c(xs, np.float32)
    r = None if mrows is None else _c(mrows, np.int64)
    cnt = m if r is None else r.size
    Y = np.empty((cnt, n), dtype=np.float64)
    _check(_load().oracle_qmm(fmt, _p(w), _p(xq), _p(xs), m, n, k, _p(r), cnt, _p(Y)), "qmm")
    return Y


def gemv(w, x, T: int, E: int, hidden: int) -> np.ndarray:
    """Router gate: f64 logits[T, E] = x Wr^T for Wr f32[E, hidden], x f32[T, hidden]."""
    w, x = _c(w, np.float32), _c(x, np.float32)
    out = np.empty((T, E), dtype=np.float64)
    _check(_load().oracle_gemv(_p(w), _p(x), T, E, hidden, _p(out)), "gemv")
    return out


def gate_route(w, x, T: int, E: int, hidden: int, topk: int):
    """Router gate then routing: (logits f64[T, E], ids int32[T, topk], wts f64[T, topk]).

    The logits are routed as the f32 values the method stores (the f64 gate
    output rounded to f32 once); softmax and renormalization are the f64
    routing of `moe_route`.
    """
    lg = gemv(w, x, T, E, hidden)
    ids, wts = moe_route(lg.astype(np.float32), T, E, topk)
    return lg, ids, wts


def moe_qmm(fmt, bank, xq, xs, x_div: int, ids, nslots: int, n: int, k: int, E: int, slots=None) -> np.ndarray:
    """Expert-indexed prefill GEMM on a q8 activation: f64 Y[rows, n] for all slots or the listed ones;
    slot s uses expert ids[s] and activation row s // x_div (zero row for an expert outside [0, E))."""
    fmt = _FMT[fmt]
    bank, xq, xs, ids = _c(bank, np.uint8), _c(xq, np.int8), _c(xs, np.float32), _c(ids, np.int32)
    sl = None if slots is None else _c(slots, np.int64)
    cnt = nslots if sl is None else sl.size
    Y = np.empty((cnt, n), dtype=np.float64)
    _check(_load().oracle_moe_qmm(fmt, _p(bank), _p(xq), _p(xs), x_div, _p(ids), nslots, n, k, E, _p(sl), cnt,
                                  _p(Y)), "moe_qmm")
    return Y


def moe_ffn_q8x(gate, up, down, xq, xs, ids, wts, T: int, topk: int, hidden: int, inter: int, E: int,
                toks=None) -> np.ndarray:
    """MoE layer on a q8 activation (prefill): f64 y rows of all tokens or the listed ones."""
    gate, up, down = _c(gate, np.uint8), _c(up, np.uint8), _c(down, np.uint8)
    xq, xs = _c(xq, np.int8), _c(xs, np.float32)
    ids, wts = _c(ids, np.int32), _c(wts, np.float32)
    tl = None if toks is None else _c(toks, np.int64)
    cnt = T if tl is None else tl.size
    y = np.empty((cnt, hidden), dtype=np.float64)
    _check(_load().oracle_moe_ffn_q8x(_p(gate), _p(up), _p(down), _p(xq), _p(xs), _p(ids), _p(wts), T, topk,
                                      hidden, inter, E, _p(tl), cnt, _p(y)), "moe_ffn_q8x")
    return y


def moe_ffn_q8(gate, up, down, xq, xs, ids, wts, T: int, topk: int, hidden: int, inter: int, E: int, toks=None):
    """MoE layer with q8 activations on both projections: (y f64 [rows, hidden], h f64 [rows*topk, inter],
    hq int8 [rows*topk, inter], hs f32 [rows*topk, inter/32]) for all tokens or the listed ones."""
    gate, up, down = _c(gate, np.uint8), _c(up, np.uint8), _c(down, np.uint8)
    xq, xs = _c(xq, np.int8), _c(xs, np.float32)
    ids, wts = _c(ids, np.int32), _c(wts, np.float32)
    tl = None if toks is None else _c(toks, np.int64)
    cnt = T if tl is None else tl.size
    y = np.empty((cnt, hidden), dtype=np.float64)
    h = np.empty((cnt * topk, inter), dtype=np.float64)
    hq = np.empty((cnt * topk, inter), dtype=np.int8)
    hs = np.empty((cnt * topk, inter // 32), dtype=np.float32)
    _check(_load().oracle_moe_ffn_q8(_p(gate), _p(up), _p(down), _p(xq), _p(xs), _p(ids), _p(wts), T, topk,
                                     hidden, inter, E, _p(tl), cnt, _p(y), _p(h), _p(hq), _p(hs)), "moe_ffn_q8")
    return y, h, hq, hs
