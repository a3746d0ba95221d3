"""GPU parity: the q8-activation MoE decode variant (int8-dot gathers and the
layer) against the oracle on the same seeded inputs.

Gathers: the q8 activation is an input (quantized on the host by the oracle's
quantizer), so the integer block sums are exact on both sides and the f32
outputs must be within scale-relative 1e-4.

Layer: x is quantized on the device by the bit-exact quantizer, but h (f32 on
the device, f64 in the oracle) is quantized again, and where h * 127 / amax
lies within rounding reach of a half-integer the two sides may choose
adjacent codes; both are correct. The test takes "within reach" as closer
than 2e-3 code units to a rounding boundary -- about 50 times the expected
f32 error of h at these shapes (int8 block sums are exact; the f32 epilogue
adds a few roundings per 32 values) -- and allows, on top of the 1e-4
scale-relative bar, one code step of the down projection at exactly those
positions: sum_j wts * hs_b * |W_down[e_j, r, c]| over the flagged c.
"""
import numpy as np
import pytest

import moe_ggml_block_amd as qmv
import oracle
import synth
from gpu_util import TOL, announce, dev, host, scalerel

pytestmark = pytest.mark.gpu

E, TOPK, HIDDEN, INTER = 128, 8, 2048, 768


def _ids(T, topk, E_, seed=0):
    return np.array([(i * 7 + 3 + seed) % E_ for i in range(T * topk)], dtype=np.int32)


# 32 / 33 tokens straddle the layer's switch from quantizing in the staging
# to the quantizer launches, 48 / 49 the int8 gathers' switch from one item
# per slot (up to 384 slots) to items grouped by expert
@pytest.mark.parametrize("T", [1, 4, 16, 32, 33, 49])
def test_moe_qmv_q4k_q8_gate_shape(T):
    announce(f"moe_qmv_q4k_q8 T={T}")
    bank = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, INTER, HIDDEN)
    x = synth.normal(synth.SEED_X, T * HIDDEN).reshape(T, HIDDEN)
    xq, xs, xsum = oracle.quantize_act_q8(x, T, HIDDEN)
    ids = _ids(T, TOPK, E)
    got = host(qmv.moe_qmv_q4k_q8(dev(bank), dev(xq), dev(xs), dev(xsum), TOPK, dev(ids), T * TOPK, INTER, HIDDEN, E))
    ref = oracle.moe_qmm("q4k", bank, xq, xs, TOPK, ids, T * TOPK, INTER, HIDDEN, E)
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)


@pytest.mark.parametrize("T", [1, 4, 16, 32, 33, 49])
def test_moe_qmv_q6k_q8_down_shape(T):
    announce(f"moe_qmv_q6k_q8 T={T}")
    bank = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, HIDDEN, INTER)
    ns = T * TOPK
    h = synth.normal(synth.SEED_X + 1, ns * INTER).reshape(ns, INTER)
    hq, hs, _ = oracle.quantize_act_q8(h, ns, INTER)
    ids = _ids(T, TOPK, E, 1)
    got = host(qmv.moe_qmv_q6k_q8(dev(bank), dev(hq), dev(hs), 1, dev(ids), ns, HIDDEN, INTER, E))
    ref = oracle.moe_qmm("q6k", bank, hq, hs, 1, ids, ns, HIDDEN, INTER, E)
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)


@pytest.mark.parametrize("fmt,k", [("q4k", 256), ("q4k", 8192), ("q6k", 256), ("q6k", 8192)])
def test_moe_qmv_q8_edges_random_blocks_and_bad_ids(fmt, k):
    """Random raw blocks (every code and scale pattern), ragged n, the two
    units per lane at k = 8192, and out-of-range ids (zero rows)."""
    E_, n, ns = 5, 70, 6
    sf = synth.FMT_Q4K if fmt == "q4k" else synth.FMT_Q6K
    bank = synth.random_blocks(sf, 150, E_ * n * (k // 256)).reshape(E_ * n, -1)
    x = synth.normal(151, ns * k).reshape(ns, k)
    xq, xs, xsum = oracle.quantize_act_q8(x, ns, k)
    ids = np.array([4, -1, 0, 5, 2, 4], dtype=np.int32)
    announce(f"moe_qmv_{fmt}_q8 edges k={k}")
    if fmt == "q4k":
        got = host(qmv.moe_qmv_q4k_q8(dev(bank), dev(xq), dev(xs), dev(xsum), 1, dev(ids), ns, n, k, E_))
    else:
        got = host(qmv.moe_qmv_q6k_q8(dev(bank), dev(xq), dev(xs), 1, dev(ids), ns, n, k, E_))
    ref = oracle.moe_qmm(fmt, bank, xq, xs, 1, ids, ns, n, k, E_)
    assert scalerel(ref, got) <= TOL, scalerel(ref, got)
    assert np.all(got[[1, 3]] == 0.0)


def _expert_slice(bank, fmt, e, rows, k):
    rb = synth.row_bytes(synth.FMT_Q4K if fmt == "q4k" else synth.FMT_Q6K, k)
    return oracle.dequant(fmt, bank.reshape(-1, rb)[e * rows:(e + 1) * rows]).reshape(rows, k)


@pytest.mark.parametrize("T", [1, 4, 16, 32, 33, 49])
def test_moe_layer_q8_matches_oracle_up_to_h_code_ties(T):
    announce(f"moe layer q8 T={T}")
    gate = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, INTER, HIDDEN)
    up = synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, INTER, HIDDEN)
    down = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, HIDDEN, INTER)
    x = synth.normal(synth.SEED_X, T * HIDDEN).reshape(T, HIDDEN)
    ids, wts = oracle.moe_route(synth.moe_logits(T, E), T, E, TOPK)
    wts = wts.astype(np.float32)
    got = host(qmv.moe_ffn_q4k_q6k_q8(dev(gate), dev(up), dev(down), dev(x), dev(ids), dev(wts), T, TOPK, HIDDEN,
                                      INTER, E))
    xq, xs, _ = oracle.quantize_act_q8(x, T, HIDDEN)
    y, h, hq, hs = oracle.moe_ffn_q8(gate, up, down, xq, xs, ids, wts, T, TOPK, HIDDEN, INTER, E)
    # positions where the code of h may legitimately differ by one
    hf = h.astype(np.float32).reshape(-1, INTER // 32, 32)
    amax = np.abs(hf).max(axis=2, keepdims=True)
    inv = np.where(amax > 0, np.float32(127.0) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    tv = (hf * inv).astype(np.float64)
    near = (np.abs(np.abs(tv - np.trunc(tv)) - 0.5) < 2e-3).reshape(-1, INTER)
    extra = np.zeros((T, HIDDEN))
    for s_ in np.nonzero(near.any(axis=1))[0]:
        t, e = s_ // TOPK, ids.reshape(-1)[s_]
        cols = np.nonzero(near[s_])[0]
        Wd = _expert_slice(down, "q6k", e, HIDDEN, INTER)
        extra[t] += float(wts.reshape(-1)[s_]) * (np.abs(Wd[:, cols]) * hs[s_, cols // 32]).sum(axis=1)
    bound = TOL * np.abs(y).max() + extra
    assert np.all(np.abs(got - y) <= bound), float(np.max(np.abs(got - y) - bound))
    assert near.sum() <= 0.01 * near.size  # the allowance stays rare
