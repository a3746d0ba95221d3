"""GPU: every path replayed from a captured HIP graph computes what the same
calls compute eagerly (bit for bit), on new inputs written between replays.

The benchmark times the kernels from graph replays, and the MoE paths keep
their grouping state in caller workspaces, so a kernel that relied on state
left by an earlier call (a counter, a table) would show up here. Each test
captures the calls once, then three times: writes new inputs, runs the same
calls eagerly into the outputs and keeps copies, overwrites the outputs with
NaN (eager fills, outside the graph), replays the graph and compares. All
kernels are deterministic: an output element depends only on its inputs (the
expert grouping orders slots by atomics, but every output row depends only
on its own slot).
"""
import numpy as np
import pytest
import torch

import moe_ggml_block_amd as qmv
import synth
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _nan_fill(outs):
    for o in outs:
        if o.dtype.is_floating_point:
            o.fill_(float("nan"))
        else:
            o.fill_(-7)


def _check_replays(run, set_inputs, outs, label):
    """run(): the calls, writing into outs; set_inputs(r): new inputs, eager."""
    set_inputs(0)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        set_inputs(r + 1)
        run()
        ref = [o.clone() for o in outs]
        _nan_fill(outs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"{label}: output {i} differs on replay {r}"
    del g


def test_graph_replay_decode_matvecs():
    """qmv_q4k, quantize_act_q8 + qmv_q4k_q8, qmv_q4k_q8x, qmv_q6k, qmv_q8_0."""
    announce("graph decode matvecs")
    k = 4096
    n4, n6, n8 = 1000, 777, 513
    w4 = dev(synth.weights(synth.FMT_Q4K, 11, n4, k))
    w6 = dev(synth.weights(synth.FMT_Q6K, 12, n6, k))
    w8 = dev(synth.weights(synth.FMT_Q8_0, 13, n8, k))
    xs_all = [dev(synth.normal(100 + r, k)) for r in range(REPLAYS + 1)]
    x = torch.empty(k, device="cuda")
    y4, y4q, y4x = (torch.empty(n4, device="cuda") for _ in range(3))
    y6, y8 = torch.empty(n6, device="cuda"), torch.empty(n8, device="cuda")
    xq = torch.empty(k, dtype=torch.int8, device="cuda")
    xs, xsum = torch.empty(k // 32, device="cuda"), torch.empty(k // 32, device="cuda")

    def run():
        qmv.qmv_q4k(w4, x, n4, k, y=y4)
        qmv.quantize_act_q8(x, 1, k, out=(xq, xs, xsum))
        qmv.qmv_q4k_q8(w4, xq, xs, xsum, n4, k, y=y4q)
        qmv.qmv_q4k_q8x(w4, x, n4, k, y=y4x)
        qmv.qmv_q6k(w6, x, n6, k, y=y6)
        qmv.qmv_q8_0(w8, x, n8, k, y=y8)

    _check_replays(run, lambda r: x.copy_(xs_all[r]), [y4, xq, xs, xsum, y4q, y4x, y6, y8], "decode")


E, TOPK, HIDDEN, INTER = 128, 8, 2048, 768


@pytest.fixture(scope="module")
def banks():
    gate = dev(synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, INTER, HIDDEN))
    up = dev(synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, INTER, HIDDEN))
    down = dev(synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, HIDDEN, INTER))
    wr = dev(synth.router_weights(E, HIDDEN))
    return gate, up, down, wr


@pytest.mark.parametrize("T", [1, 16])
def test_graph_replay_moe_decode_layer(banks, T):
    """Router, the f32 and q8 layers on its ids, the router-fused layer and
    the whole block from the hidden state, on new logits and activations per
    replay (new routes)."""
    announce(f"graph moe decode layer T={T}")
    gate, up, down, wr = banks
    lgs = [dev(synth.moe_logits(T, E, 40 + r)) for r in range(REPLAYS + 1)]
    xs_all = [dev(synth.normal(200 + r, T * HIDDEN)) for r in range(REPLAYS + 1)]
    lg = torch.empty((T, E), device="cuda")
    x = torch.empty(T * HIDDEN, device="cuda")
    ids = torch.empty((T, TOPK), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, TOPK), device="cuda")
    y, yq = torch.empty((T, HIDDEN), device="cuda"), torch.empty((T, HIDDEN), device="cuda")
    ws = torch.empty(qmv.moe_ffn_workspace_bytes(T, TOPK, HIDDEN, INTER), dtype=torch.uint8, device="cuda")
    wsq = torch.empty(qmv.moe_ffn_q8_workspace_bytes(T, TOPK, HIDDEN, INTER), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws)
    ws3 = torch.empty_like(ws)
    rt = (torch.empty((T, HIDDEN), device="cuda"), torch.empty((T, TOPK), dtype=torch.int32, device="cuda"),
          torch.empty((T, TOPK), device="cuda"))
    blk = (torch.empty((T, HIDDEN), device="cuda"), torch.empty((T, E), device="cuda"),
           torch.empty((T, TOPK), dtype=torch.int32, device="cuda"), torch.empty((T, TOPK), device="cuda"))

    def run():
        qmv.moe_route(lg, T, E, TOPK, out=(ids, wts))
        qmv.moe_ffn_q4k_q6k(gate, up, down, x, ids, wts, T, TOPK, HIDDEN, INTER, E, y=y, ws=ws)
        qmv.moe_ffn_q4k_q6k_q8(gate, up, down, x, ids, wts, T, TOPK, HIDDEN, INTER, E, y=yq, ws=wsq)
        qmv.moe_ffn_routed_q4k_q6k(gate, up, down, x, lg, T, TOPK, HIDDEN, INTER, E, out=rt, ws=ws2)
        qmv.moe_block_q4k_q6k(wr, gate, up, down, x, T, TOPK, HIDDEN, INTER, E, out=blk, ws=ws3)

    def set_inputs(r):
        lg.copy_(lgs[r])
        x.copy_(xs_all[r])

    _check_replays(run, set_inputs, [ids, wts, y, yq, *rt, *blk], f"moe decode T={T}")


def test_graph_replay_prefill_gemms():
    """quantize_act_q8 at m rows, then qmm_q4k at bm = 64 and 128 and the
    split-activation form, on new activations per replay."""
    announce("graph prefill gemms")
    m, n, k = 200, 640, 2048
    w = dev(synth.weights(synth.FMT_Q4K, 21, n, k))
    xs_all = [dev(synth.normal(300 + r, m * k)) for r in range(REPLAYS + 1)]
    x = torch.empty(m * k, device="cuda")
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    xs, xsum = torch.empty((m, k // 32), device="cuda"), torch.empty((m, k // 32), device="cuda")
    y64, y128, ysp = (torch.empty((m, n), device="cuda") for _ in range(3))
    ws = torch.empty(qmv.qmm_q4k_split_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")

    def run():
        qmv.quantize_act_q8(x, m, k, out=(xq, xs, xsum))
        qmv.qmm_q4k(w, xq, xs, xsum, m, n, k, bm=64, y=y64)
        qmv.qmm_q4k(w, xq, xs, xsum, m, n, k, bm=128, y=y128)
        qmv.qmm_q4k_split(w, xq, xs, xsum, m, n, k, y=ysp, ws=ws)

    _check_replays(run, lambda r: x.copy_(xs_all[r]), [xq, xs, xsum, y64, y128, ysp], "prefill")


@pytest.mark.parametrize("E_,T,hidden,inter", [(128, 64, 2048, 768), (128, 100, 2048, 768), (16, 128, 1024, 512)])
def test_graph_replay_moe_prefill_layer(E_, T, hidden, inter):
    """The MoE prefill layer (on the decode gathers at 64 tokens, 32-slot
    tiles at 100 tokens over 128 experts, 64-slot tiles at 128 tokens over
    16) and the expert-indexed Q4_K GEMM, on new routes and activations per
    replay."""
    announce(f"graph moe prefill E={E_} T={T} hidden={hidden} inter={inter}")
    topk = 8
    gate = dev(synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E_, inter, hidden))
    up = dev(synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E_, inter, hidden))
    down = dev(synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E_, hidden, inter))
    routes = []
    for r in range(REPLAYS + 1):
        i_, w_ = qmv.moe_route(dev(synth.moe_logits(T, E_, 60 + r)), T, E_, topk)
        routes.append((i_, w_))
    xs_all = [dev(synth.normal(400 + r, T * hidden)) for r in range(REPLAYS + 1)]
    ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, topk), device="cuda")
    x = torch.empty(T * hidden, device="cuda")
    y = torch.empty((T, hidden), device="cuda")
    ws = torch.empty(qmv.moe_ffn_prefill_workspace_bytes(T, topk, hidden, inter, E_), dtype=torch.uint8,
                     device="cuda")
    xq = torch.empty((T, hidden), dtype=torch.int8, device="cuda")
    xs, xsum = torch.empty((T, hidden // 32), device="cuda"), torch.empty((T, hidden // 32), device="cuda")
    ym = torch.empty((T * topk, inter), device="cuda")

    def run():
        qmv.moe_ffn_prefill_q4k_q6k(gate, up, down, x, ids, wts, T, topk, hidden, inter, E_, y=y, ws=ws)
        qmv.quantize_act_q8(x, T, hidden, out=(xq, xs, xsum))
        qmv.moe_qmm_q4k(gate, xq, xs, xsum, topk, ids, T * topk, inter, hidden, E_, y=ym)

    def set_inputs(r):
        ids.copy_(routes[r][0])
        wts.copy_(routes[r][1])
        x.copy_(xs_all[r])

    _check_replays(run, set_inputs, [y, xq, xs, xsum, ym], f"moe prefill E={E_} T={T}")
    # the routes did change between replays
    assert not np.array_equal(routes[1][0].cpu().numpy(), routes[2][0].cpu().numpy())
