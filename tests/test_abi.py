"""The C ABI on the CPU: libqmv.so loads, exports every function include/qmv.h
declares, and rejects bad arguments on the host before any launch. No call
here reaches a kernel (each one fails validation first), so no GPU is used.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")
LIB = os.path.join(ROOT, "moe_ggml_block_amd", "libqmv.so")

QMV_EINVAL, QMV_EALIGN, QMV_EUNSUPPORTED = -1, -2, -4


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import moe_ggml_block_amd.build as b
        b.build()
    import torch  # noqa: F401  (same HIP runtime the binding uses)
    return ctypes.CDLL(LIB)


def test_header_declares_the_path():
    names = _declared()
    for n in ("qmv_q8_0", "qmv_q4k", "qmv_q6k", "quantize_act_q8", "qmv_q4k_q8", "moe_route",
              "moe_qmv_q4k", "moe_qmv_q6k", "moe_ffn_q4k_q6k", "qmm_q4k"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_binding_exports_match_header():
    import moe_ggml_block_amd as qmv
    assert sorted(qmv.EXPORTS) == _declared()


def test_host_validation_returns_before_launch(lib):
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.qmv_q4k.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.qmv_q4k.restype = i32
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x10001)
    assert lib.qmv_q4k(None, fake, fake, 4, 256, None) == QMV_EINVAL
    assert lib.qmv_q4k(fake, fake, fake, 4, 300, None) == QMV_EINVAL
    assert lib.qmv_q4k(fake, fake, fake, 0, 256, None) == QMV_EINVAL
    assert lib.qmv_q4k(odd, fake, fake, 4, 256, None) == QMV_EALIGN
    lib.qmv_q4k_qx.argtypes = [vp] * 6 + [i64, i64, vp]
    lib.qmv_q4k_qx.restype = i32
    assert lib.qmv_q4k_qx(fake, fake, fake, None, fake, fake, 4, 256, None) == QMV_EINVAL   # no xq
    assert lib.qmv_q4k_qx(fake, fake, fake, fake, fake, fake, 4, 288, None) == QMV_EINVAL   # k % 256
    assert lib.qmv_q4k_qx(fake, fake, fake, fake, fake, fake, 0, 256, None) == QMV_EINVAL   # n < 1
    assert lib.qmv_q4k_qx(fake, odd, fake, fake, fake, fake, 4, 256, None) == QMV_EALIGN    # x
    assert lib.qmv_q4k_qx(fake, fake, fake, odd, fake, fake, 4, 256, None) == QMV_EALIGN    # xq
    lib.qmv_q8_0.argtypes = lib.qmv_q4k.argtypes
    lib.qmv_q8_0.restype = i32
    assert lib.qmv_q8_0(fake, fake, fake, 4, 48, None) == QMV_EINVAL
    lib.moe_route.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.moe_route.restype = i32
    assert lib.moe_route(fake, fake, fake, 2, 8, 9, None) == QMV_EINVAL   # topk > E
    assert lib.moe_route(fake, fake, fake, 2, 128, 0, None) == QMV_EINVAL
    lib.moe_gate_route.argtypes = [vp] * 5 + [i64] * 4 + [vp]
    lib.moe_gate_route.restype = i32
    assert lib.moe_gate_route(fake, fake, fake, fake, fake, 2, 8, 64, 9, None) == QMV_EINVAL   # topk > E
    assert lib.moe_gate_route(fake, fake, fake, fake, fake, 2, 8, 62, 2, None) == QMV_EINVAL   # hidden % 4
    assert lib.moe_gate_route(fake, fake, fake, fake, fake, 2, 8, 8196, 2, None) == -4         # hidden > 8192
    assert lib.moe_gate_route(odd, fake, fake, fake, fake, 2, 8, 64, 2, None) == QMV_EALIGN
    lib.qmm_q4k.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.qmm_q4k.restype = i32
    assert lib.qmm_q4k(fake, fake, fake, fake, fake, 512, 4096, 4096, 32, None) == QMV_EINVAL  # bm
    lib.qmm_q8_0.argtypes = [vp] * 4 + [i64] * 3 + [vp]
    lib.qmm_q8_0.restype = i32
    assert lib.qmm_q8_0(fake, fake, fake, fake, 4, 64, 224, None) == QMV_EINVAL   # k % 256
    assert lib.qmm_q8_0(fake, fake, fake, fake, 0, 64, 256, None) == QMV_EINVAL   # m < 1
    assert lib.qmm_q8_0(fake, odd, fake, fake, 4, 64, 256, None) == QMV_EALIGN    # xq
    lib.moe_ffn_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.moe_ffn_workspace_bytes.restype = i64
    # h = silu(gate x) * (up x), f32 per slot
    assert lib.moe_ffn_workspace_bytes(16, 8, 2048, 768) == 16 * 8 * 768 * 4
    lib.moe_ffn_q4k_q6k.argtypes = [vp] * 8 + [i64] * 6 + [vp]
    lib.moe_ffn_q4k_q6k.restype = i32
    assert lib.moe_ffn_q4k_q6k(fake, fake, fake, fake, fake, fake, fake, fake, 100, 16, 8, 2048, 768, 128,
                               None) == QMV_EINVAL  # workspace too small
    lib.qmv_strerror.restype = ctypes.c_char_p
    assert b"alignment" in lib.qmv_strerror(QMV_EALIGN)


def test_layer_topk_above_64_is_rejected_on_the_host(lib):
    """The decode layers keep a token's ids and weights in 64-entry on-chip
    arrays: topk > 64 is refused before any launch (the prefill layer takes
    its GEMM route there instead)."""
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    fake = ctypes.c_void_p(0x10000)
    big = 1 << 40  # workspace size large enough to pass the size check
    for name in ("moe_ffn_q4k_q6k", "moe_ffn_q4k_q6k_q8"):
        f = getattr(lib, name)
        f.argtypes = [vp] * 8 + [i64] * 6 + [vp]
        f.restype = i32
        assert f(fake, fake, fake, fake, fake, fake, fake, fake, big, 1, 65, 2048, 768, 128, None) == QMV_EUNSUPPORTED
        assert f(fake, fake, fake, fake, fake, fake, fake, fake, big, 2, 72, 256, 256, 96, None) == QMV_EUNSUPPORTED
    f = lib.moe_ffn_routed_q4k_q6k
    f.argtypes = [vp] * 9 + [i64] * 6 + [vp]
    f.restype = i32
    assert f(fake, fake, fake, fake, fake, fake, fake, fake, fake, big, 1, 65, 2048, 768, 128, None) == QMV_EINVAL
    f = lib.moe_block_q4k_q6k
    f.argtypes = [vp] * 10 + [i64] * 6 + [vp]
    f.restype = i32
    assert f(fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, big, 1, 65, 2048, 768, 128, None) == QMV_EINVAL
    # T*topk above the layer's slot limit: refused before the gate GEMV is launched
    assert f(fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, big, 300, 8, 2048, 768, 128, None) == QMV_EUNSUPPORTED


def test_noalloc_layer_checks_its_scratch_limit_on_the_host(lib):
    """moe_ffn_q4k_q6k_noalloc keeps h in a 4 MiB library array: a call whose
    h would not fit is refused before the device is touched."""
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    fake = ctypes.c_void_p(0x10000)
    f = lib.moe_ffn_q4k_q6k_noalloc
    f.argtypes = [vp] * 7 + [i64] * 5 + [vp]
    f.restype = i32
    T = (4 << 20) // (4 * 8 * 768) + 1
    assert f(fake, fake, fake, fake, fake, fake, fake, T, 8, 2048, 768, 128, None) == QMV_EUNSUPPORTED
    assert f(fake, fake, fake, fake, fake, fake, fake, 1, 65, 2048, 768, 128, None) == QMV_EUNSUPPORTED
    assert f(None, fake, fake, fake, fake, fake, fake, 1, 8, 2048, 768, 128, None) == QMV_EINVAL
