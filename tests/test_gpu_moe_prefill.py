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
        # 70 slots of one expert (three row tiles, the last ragged), two
        # out-of-range ids, ragged columns
        ids = np.array([3] * 33 + [-1] + [3] * 37 + [5], dtype=np.int32)
        args = (ids, 200, 256, 5, 1, 74)
    elif case == "id_chunks":
        # more slots than one staged chunk of ids (4096)
        ids = ((np.arange(5000) * 3) % 7).astype(np.int32)
        args = (ids, 64, 512, 7, 2, 76)
    elif case == "bm64":
        # many slots per expert: the 64-row tiles
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


def test_moe_qmm_rejects_too_many_experts():
    import torch
    t = torch.zeros(1025 * 144, dtype=torch.uint8, device="cuda")
    f = torch.zeros(64, dtype=torch.float32, device="cuda")
    i = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(qmv.QmvError):
        qmv.moe_qmm_q4k(t, t, f, f, 1, i, 4, 1, 256, 1025)
