"""GPU parity: router gate GEMV + router (moe_gate_route) against the oracle.

Logits: scale-relative error <= 1e-4 and, elementwise, within the f32
summation bound of the kernel's order (per lane NV = ceil(hidden / 256)
float4 products of 4 roundings each summed with NV - 1 additions, then a
6-level tree: at most NV + 9 roundings), |err| <= (NV + 10) * 2^-24 *
sum_c |w_c x_c|.

Ids: the oracle routes its own f64 logits (rounded to f32), the GPU routes its
f32 logits, so where two logits are closer than the error bound either order is
correct. The test therefore requires (1) exact ids wherever every gap around
the top-k boundary and between selected logits exceeds twice the bound, (2)
everywhere, that position j of the GPU's choice has an oracle logit within
twice the bound of the oracle's j-th largest, with distinct in-range ids, and
(3) bit-exact ids against moe_route run on the GPU's own logits (the routing
step of the composition is the router kernel itself).
"""
import numpy as np
import pytest
import torch

import moe_ggml_block_amd as qmv
import oracle
import synth
from gpu_util import TOL, announce, dev, host, scalerel

pytestmark = pytest.mark.gpu


def _bound(W, X):
    hidden = W.shape[1]
    nv = -(-hidden // 256)
    return (nv + 10) * 2.0 ** -24 * (np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T)


def _check(W, X, T, E, hidden, topk):
    lg_ref, ids_ref, w_ref = oracle.gate_route(W, X, T, E, hidden, topk)
    lg, ids, w = qmv.moe_gate_route(dev(W), dev(X), T, E, hidden, topk)
    g_lg, g_ids, g_w = host(lg), host(ids), host(w)
    bnd = _bound(W, X)
    assert scalerel(lg_ref, g_lg) <= TOL
    assert np.all(np.abs(g_lg - lg_ref) <= bnd)
    # routing of the GPU's own logits by the router kernel: identical
    ids2, w2 = qmv.moe_route(lg, T, E, topk)
    assert np.array_equal(host(ids2), g_ids)
    assert np.array_equal(host(w2), g_w)
    exact = 0
    for t in range(T):
        row = lg_ref[t]
        tol = 2.0 * bnd[t].max() + 2.0 * np.spacing(np.float32(np.abs(row).max()))
        assert len(set(g_ids[t].tolist())) == topk
        assert g_ids[t].min() >= 0 and g_ids[t].max() < E
        srt = row[ids_ref[t]]
        assert np.all(np.abs(row[g_ids[t]] - srt) <= tol)
        nxt = np.sort(row)[::-1][: topk + 1]
        gaps = -np.diff(nxt) if topk < E else -np.diff(nxt[:topk])
        if gaps.size == 0 or gaps.min() > tol:
            assert np.array_equal(g_ids[t], ids_ref[t])
            exact += 1
    assert np.abs(g_w - w_ref).max() <= TOL
    return exact


@pytest.mark.parametrize("T,E,hidden,topk", [
    (1, 128, 2048, 8), (4, 128, 2048, 8), (16, 128, 2048, 8),  # the MoE decode layer's router
    (33, 128, 4096, 8),      # several token chunks (4 rows of 4096 per chunk)
    (3, 8, 4096, 2),         # few experts
    (5, 37, 2880, 4),        # hidden not a multiple of 256: masked lanes
    (2, 257, 8192, 8),       # largest hidden, second router kernel (E > 256)
    (1, 4096, 1024, 16),     # largest E
    (2, 5, 4, 1),            # smallest hidden: one float4, 63 idle lanes
    (7, 3, 64, 3),           # topk = E
])
def test_gate_route_matches_oracle(T, E, hidden, topk):
    announce(f"gate_route T={T} E={E} hidden={hidden} topk={topk}")
    W = synth.router_weights(E, hidden)
    X = synth.normal(synth.SEED_X, T * hidden).reshape(T, hidden)
    exact = _check(W, X, T, E, hidden, topk)
    assert exact >= (T + 1) // 2  # seeded N(0,1)-spread logits: near-ties are rare


def test_gate_route_many_chunks_grid_stride():
    """More token chunks than the grid's second dimension (1050 chunks of 2
    rows at hidden 8192): the workgroups loop over chunks."""
    T, E, hidden, topk = 2100, 4, 8192, 2
    announce(f"gate_route grid-stride T={T} E={E} hidden={hidden}")
    W = synth.router_weights(E, hidden, seed=31)
    X = synth.normal(synth.SEED_X, T * hidden).reshape(T, hidden)
    _check(W, X, T, E, hidden, topk)


def test_gate_route_one_hot_rows_exact():
    """One-hot router rows: every logit is a copy of an activation value, so
    the logits and the ids are exact (ties included, resolved by index)."""
    T, E, hidden, topk = 6, 40, 512, 8
    rng = np.random.default_rng(5)
    perm = rng.permutation(hidden)[:E]
    W = np.zeros((E, hidden), dtype=np.float32)
    W[np.arange(E), perm] = 1.0
    X = np.round(synth.normal(9, T * hidden).reshape(T, hidden) * 2).astype(np.float32)  # ties
    announce("gate_route one-hot rows")
    lg_ref, ids_ref, w_ref = oracle.gate_route(W, X, T, E, hidden, topk)
    lg, ids, w = qmv.moe_gate_route(dev(W), dev(X), T, E, hidden, topk)
    assert np.array_equal(host(lg).astype(np.float64), lg_ref)
    assert np.array_equal(host(ids), ids_ref)
    assert np.abs(host(w) - w_ref).max() <= TOL


def test_gate_route_back_to_back_reuses_buffers():
    """Two calls into the same output buffers, the second smaller: the second
    result is complete and the first call's rows beyond it are untouched."""
    E, hidden, topk = 128, 2048, 8
    W = synth.router_weights(E, hidden)
    X = synth.normal(synth.SEED_X, 16 * hidden).reshape(16, hidden)
    out = (torch.full((16, E), -7.0, device="cuda"), torch.full((16, topk), -1, dtype=torch.int32, device="cuda"),
           torch.full((16, topk), -1.0, device="cuda"))
    announce("gate_route back to back")
    qmv.moe_gate_route(dev(W), dev(X), 16, E, hidden, topk, out=out)
    first = [host(o).copy() for o in out]
    qmv.moe_gate_route(dev(W), dev(X[:3]), 3, E, hidden, topk, out=out)
    second = [host(o) for o in out]
    for a, b in zip(first, second):
        assert np.array_equal(a, b)  # same inputs on rows 0..2, rows 3.. untouched


def test_gate_route_rejects_bad_arguments():
    W = torch.zeros((8, 64), device="cuda")
    X = torch.zeros((2, 64), device="cuda")
    with pytest.raises(qmv.QmvError):
        qmv.moe_gate_route(W, X, 2, 8, 64, 9)  # topk > E
    with pytest.raises(qmv.QmvError):
        qmv.moe_gate_route(W, X, 2, 8, 62, 2)  # hidden % 4


@pytest.mark.parametrize("T", [1, 4, 16])
def test_moe_block_from_hidden_state(T):
    """Router gate GEMV + the layer with the fused router (three launches)
    against the oracle chain gemv -> route -> layer. Ids: identical to the
    router kernel on the device's own logits; against the oracle wherever the
    logit gaps exceed twice the summation bound (then y too, per token)."""
    E, hidden, inter, topk = 128, 2048, 768, 8
    announce(f"moe block T={T}")
    W = synth.router_weights(E, hidden)
    X = synth.normal(synth.SEED_X, T * hidden).reshape(T, hidden)
    gate = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, inter, hidden)
    up = synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, inter, hidden)
    down = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, hidden, inter)
    y, lg, ids, w = qmv.moe_block_q4k_q6k(dev(W), dev(gate), dev(up), dev(down), dev(X), T, topk, hidden, inter, E)
    g_y, g_lg, g_ids = host(y), host(lg), host(ids)
    lg_ref, ids_ref, w_ref = oracle.gate_route(W, X, T, E, hidden, topk)
    assert scalerel(lg_ref, g_lg) <= TOL
    ids2, _ = qmv.moe_route(lg, T, E, topk)
    assert np.array_equal(host(ids2), g_ids)
    bnd = _bound(W, X)
    y_ref, _, _ = oracle.moe_ffn(gate, up, down, X, ids_ref, w_ref.astype(np.float32), T, topk, hidden, inter, E)
    compared = 0
    for t in range(T):
        tol = 2.0 * bnd[t].max() + 2.0 * np.spacing(np.float32(np.abs(lg_ref[t]).max()))
        nxt = np.sort(lg_ref[t])[::-1][: topk + 1]
        if (-np.diff(nxt)).min() > tol:
            assert np.array_equal(g_ids[t], ids_ref[t])
            assert scalerel(y_ref[t], g_y[t]) <= TOL
            compared += 1
    assert compared >= (T + 1) // 2
