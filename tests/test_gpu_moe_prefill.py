"""GPU parity: expert-indexed Q4_K prefill GEMM (moe_qmm_q4k) against the
oracle on the same seeded inputs. f32 outputs: scale-relative error <= 1e-4;
rows of slots whose expert is out of range: exactly zero.
"""
import numpy as np
import pytest

import moe_ggml_block_amd as qmv
import oracle
import synth
from gpu_util import TOL, announce, dev, host, scalerel

pytestmark = pytest.mark.gpu


def _stride_ids(T, topk, E):
    """The pages' MMQ-ID routing: (t*t + j) mod E -- distinct within a token,
    every expert hit, uneven per-expert counts."""
    return np.array([(t * t + j) % E for t in range(T) for j in range(topk)], dtype=np.int32)


def _check(ids, n, k, E, x_div, seed, sample=None):
    ns = ids.size
    rows_x = -(-ns // x_div)
    bank = synth.moe_bank(synth.FMT_Q4K, seed, E, n, k)
    x = synth.normal(seed + 1, rows_x * k).reshape(rows_x, k)
    xq, xs, xsum = oracle.quantize_act_q8(x, rows_x, k)
    got = host(qmv.moe_qmm_q4k(dev(bank), dev(xq), dev(xs), dev(xsum), x_div, dev(ids), ns, n, k, E))
    assert got.shape == (ns, n) and np.isfinite(got).all()
    ref = oracle.moe_qmm("q4k", bank, xq, xs, x_div, ids, ns, n, k, E, slots=sample)
    g = got if sample is None else got[sample]
    assert scalerel(ref, g) <= TOL, scalerel(ref, g)
    bad = (ids < 0) | (ids >= E)
    assert np.all(got[bad] == 0.0)
    return got


def test_moe_qmm_pages_shape_per_slot_activations():
    """32 tokens x top-8 over 16 experts, [768, 2048] experts, one activation
    row per slot (the pages' MMQ-ID check shape)."""
    T, topk, E, n, k = 32, 8, 16, 768, 2048
    announce(f"moe_qmm T={T} topk={topk} E={E} n={n} k={k}")
    ids = _stride_ids(T, topk, E)
    _check(ids, n, k, E, 1, 70, sample=np.arange(0, T * topk, 3))


def test_moe_qmm_prefill_layer_shape_routed():
    """512 tokens routed top-8 over 128 experts (router on N(0,1) logits),
    gate shape [768, 2048], one activation row per token (x_div = 8)."""
    T, topk, E, n, k = 512, 8, 128, 768, 2048
    announce(f"moe_qmm routed T={T} E={E}")
    lg = synth.moe_logits(T, E)
    ids, _ = oracle.moe_route(lg, T, E, topk)
    ids = ids.reshape(-1)
    rng = np.random.default_rng(7)
    sample = np.sort(rng.choice(T * topk, 40, replace=False))
    sample = np.concatenate([[0, 1, T * topk - 1], sample])
    _check(ids, n, k, E, topk, 72, sample=sample)


@pytest.mark.parametrize("case", ["one_expert_many_tiles", "id_chunks", "bm64", "max_experts", "single"])
def test_moe_qmm_edges(case):
    if case == "one_expert_many_tiles":
        # 70 slots of one expert (two 64-row tiles, the last ragged), two
        # out-of-range ids, ragged columns
        ids = np.array([3] * 33 + [-1] + [3] * 37 + [5], dtype=np.int32)
        args = (ids, 200, 256, 5, 1, 74)
    elif case == "id_chunks":
        # more slots than one staged chunk of ids (4096)
        ids = ((np.arange(5000) * 3) % 7).astype(np.int32)
        args = (ids, 64, 512, 7, 2, 76)
    elif case == "bm64":
        # many slots per expert: several full 64-row tiles per expert
        ids = (np.arange(256) % 4).astype(np.int32)[::-1].copy()
        args = (ids, 128, 512, 4, 1, 78)
    elif case == "max_experts":
        ids = np.random.default_rng(9).integers(0, 1024, size=64).astype(np.int32)
        args = (ids, 32, 256, 1024, 1, 80)
    else:
        ids = np.zeros(1, dtype=np.int32)
        args = (ids, 16, 256, 1, 1, 82)
    announce(f"moe_qmm edge {case}")
    sample = None if args[0].size < 1000 else np.array([0, 1, 2, 4095, 4096, 4097, 4999])
    _check(*args, sample=sample)


@pytest.mark.parametrize("k", [256, 768, 1792, 2048, 2304])
def test_moe_qmm_resident_segments(k):
    """k up to 2048 runs the resident-activation GEMM (one staged row width
    per k), k = 2304 the tile GEMM. Per-expert slot counts straddle the
    16-slot fragments and the 32-slot segments (15, 16, 17, 31, 32, 33, 48,
    64, 65 slots, one expert absent), ids interleaved, x_div = 3, ragged n,
    out-of-range ids."""
    counts = [15, 16, 17, 31, 32, 33, 0, 48, 64, 65]
    ids = np.concatenate([np.full(c, e, dtype=np.int32) for e, c in enumerate(counts)] + [np.array([-1, 10, 99], dtype=np.int32)])
    ids = ids[np.random.default_rng(k).permutation(ids.size)]
    announce(f"moe_qmm resident segments k={k} slots={ids.size}")
    _check(ids, 100, k, len(counts), 3, 84 + k // 256)


def test_moe_qmm_rejects_too_many_experts():
    import torch
    t = torch.zeros(1025 * 144, dtype=torch.uint8, device="cuda")
    f = torch.zeros(64, dtype=torch.float32, device="cuda")
    i = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(qmv.QmvError):
        qmv.moe_qmm_q4k(t, t, f, f, 1, i, 4, 1, 256, 1025)


# ------------------------------------------------------------ Q6_K prefill
@pytest.mark.parametrize("m,n,k", [(1, 16, 256), (70, 200, 512), (128, 256, 768), (300, 130, 2048)])
def test_qmm_q6k_dense_small(m, n, k):
    announce(f"qmm_q6k m={m} n={n} k={k}")
    w = synth.weights(synth.FMT_Q6K, 90, n, k)
    x = synth.normal(91, m * k).reshape(m, k)
    xq, xs, _ = oracle.quantize_act_q8(x, m, k)
    ref = oracle.qmm("q6k", w, xq, xs, m, n, k)
    got = host(qmv.qmm_q6k(dev(w), dev(xq), dev(xs), m, n, k))
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)


def test_qmm_q6k_random_blocks_every_code_and_scale():
    """Random raw Q6_K blocks: every 6-bit code and every int8 sub-scale
    (including -128 and sc*(q-32) values that f16 cannot hold) occurs."""
    m, n, k = 40, 64, 1024
    announce("qmm_q6k random blocks")
    w = synth.random_blocks(synth.FMT_Q6K, 92, n * k // 256).reshape(n, -1)
    x = synth.normal(93, m * k).reshape(m, k)
    xq, xs, _ = oracle.quantize_act_q8(x, m, k)
    ref = oracle.qmm("q6k", w, xq, xs, m, n, k)
    got = host(qmv.qmm_q6k(dev(w), dev(xq), dev(xs), m, n, k))
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)


# ------------------------------------------------------------ Q8_0 prefill
@pytest.mark.parametrize("m,n,k", [(1, 16, 256), (70, 200, 512), (128, 256, 768), (300, 130, 2048)])
def test_qmm_q8_0_dense_small(m, n, k):
    announce(f"qmm_q8_0 m={m} n={n} k={k}")
    w = synth.weights(synth.FMT_Q8_0, 94, n, k)
    x = synth.normal(95, m * k).reshape(m, k)
    xq, xs, _ = oracle.quantize_act_q8(x, m, k)
    ref = oracle.qmm("q8_0", w, xq, xs, m, n, k)
    got = host(qmv.qmm_q8_0(dev(w), dev(xq), dev(xs), m, n, k))
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)


def test_qmm_q8_0_random_blocks_every_code():
    """Random raw Q8_0 blocks: every int8 code (-128 included) and scales
    across the f16 range."""
    m, n, k = 40, 64, 1024
    announce("qmm_q8_0 random blocks")
    w = synth.random_blocks(synth.FMT_Q8_0, 96, n * k // 32).reshape(n, -1)
    x = synth.normal(97, m * k).reshape(m, k)
    xq, xs, _ = oracle.quantize_act_q8(x, m, k)
    ref = oracle.qmm("q8_0", w, xq, xs, m, n, k)
    got = host(qmv.qmm_q8_0(dev(w), dev(xq), dev(xs), m, n, k))
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)


def test_qmm_q8_0_full_config_sampled_rows():
    """m=512 tokens x W[4096, 4096] in Q8_0: every output column of sampled
    rows (first/last tiles and interior) against the oracle."""
    m, n, k = 512, 4096, 4096
    announce("qmm_q8_0 full")
    w = synth.weights(synth.FMT_Q8_0, synth.SEED_W, n, k)
    x = synth.normal(synth.SEED_PREFILL_X, m * k).reshape(m, k)
    xq, xs, _ = qmv.quantize_act_q8(dev(x), m, k)
    rq, rs, _ = oracle.quantize_act_q8(x, m, k)
    assert np.array_equal(host(xq), rq)
    Y = host(qmv.qmm_q8_0(dev(w), xq, xs, m, n, k))
    rows = np.array([0, 1, 15, 16, 63, 64, 127, 128, 255, 256, 300, 383, 384, 450, 480, 509, 511])
    ref = oracle.qmm("q8_0", w, rq, rs, m, n, k, mrows=rows)
    assert scalerel(ref, Y[rows]) <= TOL, scalerel(ref, Y[rows])
    assert np.isfinite(Y).all()


def _check6(ids, n, k, E, x_div, seed, f32, sample=None):
    ns = ids.size
    rows_x = -(-ns // x_div)
    bank = synth.moe_bank(synth.FMT_Q6K, seed, E, n, k)
    x = synth.normal(seed + 1, rows_x * k).reshape(rows_x, k)
    if f32:
        got = host(qmv.moe_qmm_q6k_f32(dev(bank), dev(x), x_div, dev(ids), ns, n, k, E))
        sl = np.arange(ns) if sample is None else np.asarray(sample)
        # a slot's output depends only on its id and its activation row: the
        # sampled slots alone, one activation row each
        xs_ = np.ascontiguousarray(x[sl // x_div])
        ref = oracle.moe_qmv("q6k", bank, xs_, 1, np.ascontiguousarray(ids[sl]), sl.size, n, k, E)
    else:
        xq, xs, _ = oracle.quantize_act_q8(x, rows_x, k)
        got = host(qmv.moe_qmm_q6k(dev(bank), dev(xq), dev(xs), x_div, dev(ids), ns, n, k, E))
        sl = np.arange(ns) if sample is None else np.asarray(sample)
        ref = oracle.moe_qmm("q6k", bank, xq, xs, x_div, ids, ns, n, k, E, slots=sample)
    assert got.shape == (ns, n) and np.isfinite(got).all()
    assert scalerel(ref, got[sl]) <= TOL, scalerel(ref, got[sl])
    bad = (ids < 0) | (ids >= E)
    assert np.all(got[bad] == 0.0)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("case", ["pages", "ragged", "id_chunks", "k1024", "k1280", "layer_down"])
def test_moe_qmm_q6k(case, f32):
    if case == "layer_down":
        # the prefill layer's down shape: 512 tokens routed top-8 over 128
        # experts, [2048, 768] experts, 32 slots per expert on average
        # (48-slot segments of three 256-value superblocks)
        lg = synth.moe_logits(512, 128)
        ids, _ = oracle.moe_route(lg, 512, 128, 8)
        args = (ids.reshape(-1), 2048, 768, 128, 1, 93)
        sample = np.sort(np.random.default_rng(5).choice(4096, 24, replace=False))
    elif case == "k1024":
        # the longest rows the f32 form keeps resident in LDS, a ragged last tile
        ids = ((np.arange(300) * 7) % 5).astype(np.int32)
        args = (ids, 272, 1024, 5, 2, 97)
        sample = np.array([0, 1, 2, 150, 298, 299])
    elif case == "k1280":
        # past that limit (the staged tile GEMM)
        ids = ((np.arange(90) * 3) % 4).astype(np.int32)
        args = (ids, 80, 1280, 4, 1, 95)
        sample = None
    elif case == "pages":
        # down shape [2048, 768], 32 tokens x top-8 over 16 experts, a row per slot
        args = (_stride_ids(32, 8, 16), 2048, 768, 16, 1, 94)
        sample = np.arange(0, 256, 5)
    elif case == "ragged":
        ids = np.array([2] * 45 + [-3] + [0] * 3 + [9], dtype=np.int32)
        args = (ids, 130, 256, 3, 1, 96)
        sample = None
    else:
        ids = ((np.arange(4500) * 5) % 11).astype(np.int32)
        args = (ids, 48, 512, 11, 3, 98)
        sample = np.array([0, 1, 4095, 4096, 4499])
    announce(f"moe_qmm_q6k {case} f32={f32}")
    _check6(*args, f32, sample=sample)


def test_moe_qmm_q6k_f32_wide_dynamic_range():
    """Activation values spanning many binades (1e-6 .. 1e4) and an all-zero
    block: the power-of-two scaling and the two-half split keep f32 accuracy
    without f16 overflow."""
    E, n, k, ns = 3, 64, 512, 12
    bank = synth.moe_bank(synth.FMT_Q6K, 99, E, n, k)
    x = synth.normal(100, ns * k).reshape(ns, k)
    x *= np.float32(10.0) ** np.linspace(-6, 4, k, dtype=np.float32)[None, :]
    x[3, 64:96] = 0.0
    ids = (np.arange(ns) % E).astype(np.int32)
    announce("moe_qmm_q6k_f32 dynamic range")
    got = host(qmv.moe_qmm_q6k_f32(dev(bank), dev(x), 1, dev(ids), ns, n, k, E))
    ref = oracle.moe_qmv("q6k", bank, x, 1, ids, ns, n, k, E)
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)


# ------------------------------------------------------------ prefill layer
def _layer(T, topk, E, hidden, inter, seed, ids=None, sample=None):
    gate = synth.moe_bank(synth.FMT_Q4K, seed, E, inter, hidden)
    up = synth.moe_bank(synth.FMT_Q4K, seed + 1, E, inter, hidden)
    down = synth.moe_bank(synth.FMT_Q6K, seed + 2, E, hidden, inter)
    x = synth.normal(seed + 3, T * hidden).reshape(T, hidden)
    if ids is None:
        ids, wts = oracle.moe_route(synth.moe_logits(T, E, seed % 7), T, E, topk)
        wts = wts.astype(np.float32)
    else:
        wts = np.random.default_rng(seed).random(ids.shape).astype(np.float32)
    got = host(qmv.moe_ffn_prefill_q4k_q6k(dev(gate), dev(up), dev(down), dev(x), dev(ids), dev(wts), T, topk,
                                           hidden, inter, E))
    assert got.shape == (T, hidden) and np.isfinite(got).all()
    xq, xs, _ = oracle.quantize_act_q8(x, T, hidden)
    ref = oracle.moe_ffn_q8x(gate, up, down, xq, xs, ids, wts, T, topk, hidden, inter, E, toks=sample)
    g = got if sample is None else got[sample]
    assert scalerel(ref, g) <= TOL, scalerel(ref, g)
    return gate, up, down, x, ids, wts, got


def test_moe_prefill_layer_small_full_output():
    T, topk, E, hidden, inter = 64, 8, 16, 512, 256
    announce(f"moe prefill layer T={T} E={E} hidden={hidden} inter={inter}")
    _layer(T, topk, E, hidden, inter, 110)


@pytest.mark.parametrize("T,topk,E", [(32, 8, 16), (33, 8, 16), (64, 8, 16), (65, 8, 16), (100, 8, 128)])
def test_moe_prefill_layer_both_sides_of_the_gather_threshold(T, topk, E):
    """Up to 256 slots the layer runs on the decode gathers, above on the
    GEMMs (table tiles of 32, 48 or 64 slots by the mean slots per expert)."""
    hidden, inter = 512, 256
    announce(f"moe prefill layer T={T} topk={topk} E={E} hidden={hidden} inter={inter}")
    _layer(T, topk, E, hidden, inter, 150 + T)


@pytest.mark.parametrize("T,E,hidden,inter", [(80, 16, 1024, 512), (300, 8, 768, 256), (66, 64, 2048, 256)])
def test_moe_prefill_layer_resident_gate_up_shapes(T, E, hidden, inter):
    """The gate/up GEMM on resident activations at other staged widths
    (hidden 768, 1024, 2048) and h widths (256, 512 columns: 32 or 64 wave
    groups), with 40 to 300 slots per expert (one to ten segments; single
    column groups or whole chunks as the units)."""
    topk = 8
    announce(f"moe prefill layer T={T} E={E} hidden={hidden} inter={inter}")
    _layer(T, topk, E, hidden, inter, 180 + T, sample=np.array([0, 1, T // 2, T - 1]))


@pytest.mark.parametrize("E", [48, 24, 8])
def test_moe_prefill_layer_wide_hidden_tile_gate_up(E):
    """hidden 2304 (past the widest resident activation row): the gate/up
    GEMM runs on the tile GEMMs -- 16 slots per expert (E = 48, 32-slot
    table tiles), 32 (E = 24, 48-slot tiles on the weight-side tile) or 96
    (E = 8, 64-slot tiles on the weight-side tile)."""
    T, topk, hidden, inter = 96, 8, 2304, 256
    announce(f"moe prefill layer T={T} E={E} hidden={hidden} inter={inter}")
    _layer(T, topk, E, hidden, inter, 190 + E, sample=np.array([0, 1, 47, 48, T - 1]))


def test_moe_prefill_layer_full_shape_sampled_tokens():
    """512 tokens routed top-8 over 128 experts, gate/up [768, 2048], down
    [2048, 768]: every output column of 12 sampled tokens."""
    T, topk, E, hidden, inter = 512, 8, 128, 2048, 768
    announce(f"moe prefill layer T={T} E={E} hidden={hidden} inter={inter}")
    _layer(T, topk, E, hidden, inter, 120, sample=np.array([0, 1, 2, 63, 64, 200, 255, 256, 300, 450, 510, 511]))


def test_moe_prefill_layer_repeats_and_out_of_range_experts():
    T, topk, E, hidden, inter = 9, 3, 5, 256, 256
    ids = np.array([[4, 0, 2], [1, -1, 3], [2, 2, 0], [0, 5, 4], [3, 3, 3], [-2, -2, -2], [1, 2, 3], [0, 0, 1],
                    [4, 4, 0]], dtype=np.int32)
    announce("moe prefill layer repeats / out of range")
    got = _layer(T, topk, E, hidden, inter, 130, ids=ids)[-1]
    assert np.all(got[5] == 0.0)  # every slot of token 5 out of range


def test_moe_prefill_layer_workspace_reuse_smaller_second_call():
    import torch
    T, topk, E, hidden, inter = 40, 4, 8, 512, 256
    announce("moe prefill layer workspace reuse")
    gate, up, down, x, ids, wts, first = _layer(T, topk, E, hidden, inter, 140)
    ws = torch.empty(qmv.moe_ffn_prefill_workspace_bytes(T, topk, hidden, inter, E), dtype=torch.uint8,
                     device="cuda")
    G, U, D = dev(gate), dev(up), dev(down)
    a = host(qmv.moe_ffn_prefill_q4k_q6k(G, U, D, dev(x), dev(ids), dev(wts), T, topk, hidden, inter, E, ws=ws))
    b = host(qmv.moe_ffn_prefill_q4k_q6k(G, U, D, dev(x[:7]), dev(ids[:7]), dev(wts[:7]), 7, topk, hidden, inter,
                                         E, ws=ws))
    assert np.array_equal(a, first)   # same inputs, same bits (grouping order does not matter)
    # a token's rows agree across batch sizes to the f32 tolerance, not bit for
    # bit: the launch shape (and, across 512 slots, the kernels) set the
    # rounding order of the combine
    assert scalerel(first[:7], b) <= TOL, scalerel(first[:7], b)


@pytest.mark.parametrize("T", [32, 64])
def test_moe_prefill_layer_bench_shape_on_the_gathers(T):
    """The benched small-batch layer (top-8 over 128 experts, gate/up
    [768, 2048], down [2048, 768]; 256 slots, on the expert-grouped decode
    gathers, and 512, on the GEMMs): every output column of sampled tokens
    against the oracle."""
    topk, E, hidden, inter = 8, 128, 2048, 768
    announce(f"moe prefill layer (gathers) T={T} E={E} hidden={hidden} inter={inter}")
    _layer(T, topk, E, hidden, inter, 160 + T, sample=np.array([0, 1, T // 2, T - 2, T - 1]))


def test_moe_prefill_layer_topk_above_64_takes_the_gemm_route():
    """72 slots per token (more than the decode down pass holds on chip):
    216 slots would fit the gather route by count, but the layer must take
    the GEMM tiles, whose combine takes any topk."""
    T, topk, E, hidden, inter = 3, 72, 96, 256, 256
    announce(f"moe prefill layer T={T} topk={topk} E={E}")
    _layer(T, topk, E, hidden, inter, 170)
