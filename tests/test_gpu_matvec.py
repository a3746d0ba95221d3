"""GPU parity: dense matvecs, the q8 activation quantizer and the int8-dot
Q4_K matvec, against the CPU oracle on the same seeded inputs.

f32 outputs: scale-relative error <= 1e-4 (max|a-b| / max|a|, a = oracle).
Integer outputs (xq, the int32 block sums) and the quantizer's f32 scales
(single IEEE operations): bit-exact.
"""
import numpy as np
import pytest
import torch

import moe_ggml_block_amd as qmv
import oracle
import synth
from gpu_util import TOL, announce, dev, host, scalerel

pytestmark = pytest.mark.gpu

FMTS = {"q8_0": synth.FMT_Q8_0, "q4k": synth.FMT_Q4K, "q6k": synth.FMT_Q6K, "q4_0": synth.FMT_Q4_0,
        "q5k": synth.FMT_Q5K}
FN = {"q8_0": qmv.qmv_q8_0, "q4k": qmv.qmv_q4k, "q6k": qmv.qmv_q6k, "q4_0": qmv.qmv_q4_0, "q5k": qmv.qmv_q5k}


def _run_dense(fmt, w, x, n, k):
    y = FN[fmt](dev(w), dev(x), n, k)
    return host(y)


# (n, k): several tiles, ragged row tails, every unit tiling (G = 8..64,
# UPL 1..4), the generic path (Q8_0 k % 64 == 32, very long rows).
SMALL = {
    "q8_0": [(1, 32), (37, 96), (5, 64), (130, 512), (67, 2048), (29, 4096), (33, 8192), (9, 16384),
             (4133, 2048)],  # past 16 rows per CU: the two-workgroup launch form
    "q4k": [(1, 256), (37, 256), (70, 768), (65, 2048), (33, 4096), (17, 8192), (5, 12288), (3, 20480)],
    "q6k": [(1, 256), (37, 256), (70, 768), (65, 2048), (33, 4096), (17, 8192), (5, 12288), (3, 20480)],
    "q4_0": [(1, 32), (37, 96), (5, 64), (130, 512), (67, 2048), (29, 4096), (33, 8192), (9, 16384)],
    "q5k": [(1, 256), (37, 256), (70, 768), (65, 2048), (33, 4096), (17, 8192), (5, 12288), (3, 20480)],
}


@pytest.mark.parametrize("fmt", ["q8_0", "q4k", "q6k", "q4_0", "q5k"])
def test_dense_small_shapes(fmt):
    for n, k in SMALL[fmt]:
        announce(f"dense {fmt} n={n} k={k}")
        w = synth.weights(FMTS[fmt], 1, n, k)
        x = synth.normal(2, k)
        ref = oracle.matvec(fmt, w, x, n, k)
        got = _run_dense(fmt, w, x, n, k)
        assert scalerel(ref, got) <= TOL, (fmt, n, k, scalerel(ref, got))


@pytest.mark.parametrize("fmt", ["q8_0", "q4k", "q6k", "q4_0", "q5k"])
def test_dense_random_blocks(fmt):
    """Random raw bytes: every code, every 6-bit scale/min, negative Q6_K
    sub-scales, subnormal f16 scales in every 3rd block."""
    f = FMTS[fmt]
    for n, k in [(29, 512), (41, 4096), (64, 768)]:
        announce(f"dense random {fmt} n={n} k={k}")
        w = synth.random_blocks(f, 5, n * k // synth.BLOCK_WEIGHTS[f], subnormal_every=3)
        x = synth.normal(6, k)
        ref = oracle.matvec(fmt, w, x, n, k)
        got = _run_dense(fmt, w, x, n, k)
        assert scalerel(ref, got) <= TOL, (fmt, n, k, scalerel(ref, got))


def test_dense_subnormal_only_scales():
    for fmt in ("q4k", "q6k", "q8_0", "q4_0", "q5k"):
        f = FMTS[fmt]
        n, k = 16, 1024
        announce(f"dense subnormal {fmt}")
        w = synth.random_blocks(f, 8, n * k // synth.BLOCK_WEIGHTS[f], subnormal_every=1)
        x = synth.normal(9, k)
        ref = oracle.matvec(fmt, w, x, n, k)
        got = _run_dense(fmt, w, x, n, k)
        assert scalerel(ref, got) <= TOL, (fmt, scalerel(ref, got))


@pytest.mark.parametrize("fmt,n,k", [("q8_0", 4096, 4096), ("q4k", 14336, 4096), ("q6k", 128256, 4096),
                                     ("q4_0", 14336, 4096), ("q5k", 14336, 4096)])
def test_dense_full_config(fmt, n, k):
    """The full workload shapes, in the launch configuration the benchmark times."""
    announce(f"dense full {fmt} n={n} k={k}")
    w = synth.weights(FMTS[fmt], synth.SEED_W, n, k)
    x = synth.normal(synth.SEED_X, k)
    ref = oracle.matvec(fmt, w, x, n, k)
    got = _run_dense(fmt, w, x, n, k)
    assert got.shape == (n,)
    assert scalerel(ref, got) <= TOL, (fmt, scalerel(ref, got))


def test_dense_output_fully_overwritten_and_stream():
    n, k = 100, 2048
    announce("dense overwrite + side stream")
    w = dev(synth.weights(synth.FMT_Q4K, 3, n, k))
    x = dev(synth.normal(4, k))
    y = torch.full((n,), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qmv.qmv_q4k(w, x, n, k, y=y, stream=s)
    s.synchronize()
    ref = oracle.matvec("q4k", w.cpu().numpy(), x.cpu().numpy(), n, k)
    assert scalerel(ref, y.cpu().numpy()) <= TOL


def test_dense_bad_arguments_raise():
    w = torch.zeros(144, dtype=torch.uint8, device="cuda")
    x = torch.zeros(256, device="cuda")
    with pytest.raises(qmv.QmvError):
        qmv.qmv_q4k(w, x, 1, 100)  # k not a multiple of 256
    w2 = torch.zeros(160, dtype=torch.uint8, device="cuda")
    with pytest.raises(qmv.QmvError):
        qmv.qmv_q4k(w2[1:145], x, 1, 256)  # misaligned weight pointer


# --------------------------------------------------------------- q8 path
def _quant_gpu(x, m, k):
    xq, xs, xsum = qmv.quantize_act_q8(dev(x), m, k)
    return host(xq), host(xs), host(xsum)


def test_quantize_act_bit_exact():
    for m, k in [(1, 32), (1, 4096), (3, 2048), (512, 4096), (7, 96)]:
        announce(f"quantize_act m={m} k={k}")
        x = synth.normal(20, m * k).reshape(m, k)
        x[0, :32] = 0.0                                     # zero block
        if k >= 64:
            x[0, 32:64] = np.arange(32, dtype=np.float32) - 15.5  # half-way codes
            x[0, 40] = 127.0
        rq, rs, rsum = oracle.quantize_act_q8(x, m, k)
        gq, gs, gsum = _quant_gpu(x, m, k)
        assert np.array_equal(rq, gq)
        assert np.array_equal(rs.view(np.uint32), gs.view(np.uint32))
        assert np.array_equal(rsum.view(np.uint32), gsum.view(np.uint32))


def test_quantize_act_wide_dynamic_range():
    m, k = 4, 1024
    x = synth.normal(21, m * k).reshape(m, k) * np.float32(1e-3)
    x[1] *= np.float32(1e6)
    x[2, ::7] = np.float32(3e-38)
    announce("quantize_act dynamic range")
    rq, rs, rsum = oracle.quantize_act_q8(x, m, k)
    gq, gs, gsum = _quant_gpu(x, m, k)
    assert np.array_equal(rq, gq)
    assert np.array_equal(rs.view(np.uint32), gs.view(np.uint32))
    assert np.array_equal(rsum.view(np.uint32), gsum.view(np.uint32))


@pytest.mark.parametrize("n,k", [(37, 256), (65, 2048), (33, 4096), (9, 8192), (14336, 4096)])
def test_q4k_q8_blocksums_bit_exact_and_matvec(n, k):
    announce(f"q4k_q8 n={n} k={k}")
    w = synth.weights(synth.FMT_Q4K, synth.SEED_W, n, k)
    x = synth.normal(synth.SEED_X, k)
    xq, xs, xsum = oracle.quantize_act_q8(x, 1, k)
    S_ref = oracle.blocksums_q4k_q8(w, xq, n, k)
    wd, xqd = dev(w), dev(xq)
    S_gpu = host(qmv.qmv_debug_blocksums_q4k_q8(wd, xqd, n, k))
    assert np.array_equal(S_ref, S_gpu.astype(np.int64))
    y_ref = oracle.matvec_q8act("q4k", w, xq, xs, n, k)
    y_gpu = host(qmv.qmv_q4k_q8(wd, xqd, dev(xs), dev(xsum), n, k))
    assert scalerel(y_ref, y_gpu) <= TOL, scalerel(y_ref, y_gpu)


def test_q4k_q8_end_to_end_from_f32():
    """quantize on the GPU, then dot4: same as the oracle's quantize + W_deq x_deq."""
    n, k = 14336, 4096
    announce("q4k_q8 end to end")
    w = synth.weights(synth.FMT_Q4K, synth.SEED_W, n, k)
    x = synth.normal(synth.SEED_X, k)
    xq, xs, xsum = qmv.quantize_act_q8(dev(x), 1, k)
    y = host(qmv.qmv_q4k_q8(dev(w), xq, xs, xsum, n, k))
    rq, rs, _ = oracle.quantize_act_q8(x, 1, k)
    assert np.array_equal(host(xq), rq)
    y_ref = oracle.matvec_q8act("q4k", w, rq, rs, n, k)
    assert scalerel(y_ref, y) <= TOL


@pytest.mark.parametrize("n,k", [(37, 256), (65, 768), (33, 2048), (70, 4096), (9, 8192), (14336, 4096)])
def test_q4k_q8x_fused_quantize_matches_two_step(n, k):
    """qmv_q4k_q8x quantizes x inside the kernel: bit-identical to
    quantize_act_q8 + qmv_q4k_q8, and within 1e-4 of the oracle."""
    announce(f"q4k q8x fused n={n} k={k}")
    w = synth.weights(synth.FMT_Q4K, 11, n, k)
    x = synth.normal(12, k)
    x[::37] *= 100.0  # blocks with a wide spread of magnitudes
    W, X = dev(w), dev(x)
    fused = host(qmv.qmv_q4k_q8x(W, X, n, k))
    xq, xs, xsum = qmv.quantize_act_q8(X, 1, k)
    two = host(qmv.qmv_q4k_q8(W, xq, xs, xsum, n, k))
    assert np.array_equal(fused, two)
    oq, os_, _ = oracle.quantize_act_q8(x, 1, k)
    ref = oracle.matvec_q8act("q4k", w, oq[0], os_[0], n, k)
    assert scalerel(ref, fused) <= TOL


@pytest.mark.parametrize("n,k", [(1, 256), (37, 256), (70, 768), (33, 2048), (70, 4096), (9, 8192),
                                 (14336, 4096), (3, 12288)])
def test_q4k_qx_matvec_and_q8_row_bit_exact(n, k):
    """qmv_q4k_qx: y bit-identical to qmv_q4k, the q8 row bit-identical to the
    oracle's quantize_act_q8 (k = 12288 takes the two-launch form)."""
    announce(f"q4k qx n={n} k={k}")
    w = synth.weights(synth.FMT_Q4K, 13, n, k)
    x = synth.normal(14, k)
    x[::41] *= 300.0
    x[:32] = 0.0  # a zero block: scale 1, codes 0
    if k >= 64:
        x[32:64] = np.arange(32, dtype=np.float32) - 15.5  # half-way codes
    W, X = dev(w), dev(x)
    y, (xq, xs, xsum) = qmv.qmv_q4k_qx(W, X, n, k)
    y_plain = host(qmv.qmv_q4k(W, X, n, k))
    assert np.array_equal(host(y).view(np.uint32), y_plain.view(np.uint32))
    rq, rs, rsum = oracle.quantize_act_q8(x, 1, k)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(xsum).view(np.uint32), rsum.view(np.uint32))
    ref = oracle.matvec("q4k", w, x, n, k)
    assert scalerel(ref, host(y)) <= TOL


def test_q4k_qx_feeds_q8_matvec():
    """The decode step form: the q8 row written by qmv_q4k_qx drives
    qmv_q4k_q8 to the same bits as the separate quantizer launch."""
    n, k = 14336, 4096
    announce("q4k qx -> q4k_q8")
    w = synth.weights(synth.FMT_Q4K, synth.SEED_W, n, k)
    x = synth.normal(synth.SEED_X, k)
    W, X = dev(w), dev(x)
    _, (xq, xs, xsum) = qmv.qmv_q4k_qx(W, X, n, k)
    y = host(qmv.qmv_q4k_q8(W, xq, xs, xsum, n, k))
    q2, s2, m2 = qmv.quantize_act_q8(X, 1, k)
    y2 = host(qmv.qmv_q4k_q8(W, q2, s2, m2, n, k))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
