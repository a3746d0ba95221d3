"""Seeded synthetic inputs shared by the oracle's tests and the GPU path.

Counter-based uniforms / normals and raw GGML-layout weight blocks
(Q8_0 34 B / 32 weights, Q4_K 144 B / 256, Q6_K 210 B / 256). Nothing in
here decodes blocks, forms dot products, quantizes activations or routes:
that arithmetic lives separately in the oracle and in the HIP kernels.

The C implementation (``synth.c``) is built into ``libsynth.so`` next to
this file by ``build()``; numpy arrays come back.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

FMT_Q8_0, FMT_Q4K, FMT_Q6K, FMT_Q4_0, FMT_Q5K = 0, 1, 2, 3, 4
BLOCK_WEIGHTS = {FMT_Q8_0: 32, FMT_Q4K: 256, FMT_Q6K: 256, FMT_Q4_0: 32, FMT_Q5K: 256}
BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q4K: 144, FMT_Q6K: 210, FMT_Q4_0: 18, FMT_Q5K: 176}
FMT_NAMES = {"q8_0": FMT_Q8_0, "q4k": FMT_Q4K, "q6k": FMT_Q6K, "q4_0": FMT_Q4_0, "q5k": FMT_Q5K}

# Stream seeds for the workloads (one stream per input, rotations offset by 100).
SEED_W, SEED_X, SEED_LOGITS = 1, 2, 3
SEED_GATE, SEED_UP, SEED_DOWN = 10, 11, 12
SEED_PREFILL_X = 20
SEED_ROUTER = 30


def build() -> None:
    """Compile libsynth.so (gcc, OpenMP, no FP contraction)."""
    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           src, "-o", _SO + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
    vp = ctypes.c_void_p
    lib.synth_uniform.argtypes = [u64, u64, i64, vp]
    lib.synth_normal.argtypes = [u64, u64, i64, vp]
    lib.synth_f32_to_f16.argtypes = [ctypes.c_float]
    lib.synth_f32_to_f16.restype = ctypes.c_uint16
    for f in (lib.synth_encode_q8_0, lib.synth_encode_q4k, lib.synth_encode_q6k, lib.synth_encode_q4_0,
              lib.synth_encode_q5k):
        f.argtypes = [vp, i64, i64, vp]
        f.restype = i32
    lib.synth_row_bytes.argtypes = [i32, i64]
    lib.synth_row_bytes.restype = i64
    lib.synth_weights.argtypes = [i32, u64, i64, i64, vp]
    lib.synth_weights.restype = i32
    lib.synth_random_blocks.argtypes = [i32, u64, i64, i32, vp]
    lib.synth_random_blocks.restype = i32
    lib.synth_pack_q4k_scales.argtypes = [vp, vp, vp]
    lib.synth_pack_q6k_codes.argtypes = [vp, vp, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def uniform(seed: int, n: int, start: int = 0) -> np.ndarray:
    """float32[n]: element i is uniform counter start+i of stream `seed`, in [-1, 1)."""
    out = np.empty(n, dtype=np.float32)
    _load().synth_uniform(seed, start, n, _ptr(out))
    return out


def normal(seed: int, n: int, start: int = 0) -> np.ndarray:
    """float32[n] ~ N(0,1) by Box-Muller (f64) over counter pairs of stream `seed`."""
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal(seed, start, n, _ptr(out))
    return out


def f32_to_f16_bits(v: float) -> int:
    return int(_load().synth_f32_to_f16(ctypes.c_float(v)))


def row_bytes(fmt: int, k: int) -> int:
    return k // BLOCK_WEIGHTS[fmt] * BLOCK_BYTES[fmt]


def encode(fmt: int, w: np.ndarray) -> np.ndarray:
    """Encode an f32 matrix [rows, k] into raw blocks, uint8[rows, row_bytes]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, k = w.shape
    out = np.empty((rows, row_bytes(fmt, k)), dtype=np.uint8)
    fn = {FMT_Q8_0: _load().synth_encode_q8_0, FMT_Q4K: _load().synth_encode_q4k,
          FMT_Q6K: _load().synth_encode_q6k, FMT_Q4_0: _load().synth_encode_q4_0,
          FMT_Q5K: _load().synth_encode_q5k}[fmt]
    if fn(_ptr(w), rows, k, _ptr(out)) != 0:
        raise ValueError(f"k={k} not a multiple of {BLOCK_WEIGHTS[fmt]}")
    return out


def weights(fmt: int, seed: int, rows: int, k: int) -> np.ndarray:
    """uint8[rows, row_bytes]: uniform[-1,1) matrix of stream `seed`, encoded to `fmt`."""
    if k % BLOCK_WEIGHTS[fmt]:
        raise ValueError(f"k={k} not a multiple of {BLOCK_WEIGHTS[fmt]}")
    out = np.empty((rows, row_bytes(fmt, k)), dtype=np.uint8)
    if _load().synth_weights(fmt, seed, rows, k, _ptr(out)) != 0:
        raise ValueError("synth_weights failed")
    return out


def weight_matrix_f32(seed: int, rows: int, k: int) -> np.ndarray:
    """The f32 matrix `weights` encodes (for quantization-error reports)."""
    return uniform(seed, rows * k).reshape(rows, k)


def random_blocks(fmt: int, seed: int, nblocks: int, subnormal_every: int = 0) -> np.ndarray:
    """uint8[nblocks, block_bytes] of random bytes with finite f16 scale fields."""
    out = np.empty((nblocks, BLOCK_BYTES[fmt]), dtype=np.uint8)
    _load().synth_random_blocks(fmt, seed, nblocks, subnormal_every, _ptr(out))
    return out


def pack_q4k_scales(sc, mn) -> np.ndarray:
    sc = np.asarray(sc, dtype=np.uint8)
    mn = np.asarray(mn, dtype=np.uint8)
    out = np.empty(12, dtype=np.uint8)
    _load().synth_pack_q4k_scales(_ptr(sc), _ptr(mn), _ptr(out))
    return out


def pack_q6k_codes(q) -> tuple[np.ndarray, np.ndarray]:
    q = np.asarray(q, dtype=np.uint8)
    ql = np.empty(128, dtype=np.uint8)
    qh = np.empty(64, dtype=np.uint8)
    _load().synth_pack_q6k_codes(_ptr(q), _ptr(ql), _ptr(qh))
    return ql, qh


def moe_logits(T: int, E: int, rotation: int = 0) -> np.ndarray:
    return normal(SEED_LOGITS + 100 * rotation, T * E).reshape(T, E)


def moe_bank(fmt: int, seed: int, E: int, n: int, k: int) -> np.ndarray:
    """Expert bank [E, n, k] encoded row-major: uint8[E*n, row_bytes]."""
    return weights(fmt, seed, E * n, k)


def router_weights(E: int, hidden: int, seed: int = SEED_ROUTER) -> np.ndarray:
    """float32[E, hidden] uniform in [-a, a), a = sqrt(3 / hidden): variance 1/hidden,
    so the logits of an x ~ N(0, 1) are about N(0, 1), the routing workload's spread."""
    a = np.float32(np.sqrt(3.0 / hidden))
    return (uniform(seed, E * hidden) * a).reshape(E, hidden)
