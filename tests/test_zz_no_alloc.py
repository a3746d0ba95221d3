"""GPU: the allocation-free decode MoE layer (moe_ffn_q4k_q6k_noalloc), called
through the C ABI, against the workspace form of the same layer
(moe_ffn_q4k_q6k): the same kernels on the same inputs, so the outputs must
be bit-identical; and both within the f32 tolerance of the oracle. Two calls
in a row, the second smaller, share the library's per-GPU scratch array.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_ggml_block_amd as qmv
import oracle
import synth
from gpu_util import TOL, announce, dev, host, scalerel

pytestmark = pytest.mark.gpu

E, TOPK, HIDDEN, INTER = 128, 8, 2048, 768


def _noalloc_raw(G, U, D, x, ids, w, y, T):
    """The C entry point itself, through ctypes (no Python-side marshalling)."""
    f = qmv.raw("moe_ffn_q4k_q6k_noalloc")
    p = ctypes.c_void_p
    return f(p(G.data_ptr()), p(U.data_ptr()), p(D.data_ptr()), p(x.data_ptr()), p(ids.data_ptr()),
             p(w.data_ptr()), p(y.data_ptr()), T, TOPK, HIDDEN, INTER, E,
             p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_layer_matches_workspace_layer_two_calls():
    gate = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, INTER, HIDDEN)
    up = synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, INTER, HIDDEN)
    down = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, HIDDEN, INTER)
    G, U, D = dev(gate), dev(up), dev(down)
    for T, seed in ((16, 90), (3, 91)):  # the second call is smaller
        announce(f"moe_ffn_q4k_q6k_noalloc T={T} seed={seed}")
        lg = synth.normal(seed, T * E).reshape(T, E)
        x = synth.normal(seed + 100, T * HIDDEN).reshape(T, HIDDEN)
        ids_ref, w_ref = oracle.moe_route(lg, T, E, TOPK)
        ids, w = dev(ids_ref), dev(w_ref.astype(np.float32))
        xd = dev(x)
        y = torch.full((T, HIDDEN), float("nan"), device="cuda")
        assert _noalloc_raw(G, U, D, xd, ids, w, y, T) == 0
        got = host(y)
        want = host(qmv.moe_ffn_q4k_q6k(G, U, D, xd, ids, w, T, TOPK, HIDDEN, INTER, E))
        assert np.array_equal(got, want)
        y_ref, _, _ = oracle.moe_ffn(gate, up, down, x, ids_ref, w_ref.astype(np.float32), T, TOPK, HIDDEN,
                                     INTER, E)
        assert scalerel(y_ref, got) <= TOL, scalerel(y_ref, got)


def test_noalloc_layer_refuses_more_than_its_scratch():
    # T*topk*inter*4 bytes of h above the array's size: refused on the host
    T = qmv.NOALLOC_SCRATCH_BYTES // (4 * TOPK * INTER) + 1
    fake = torch.empty(4, dtype=torch.float32, device="cuda")
    y = torch.empty(4, dtype=torch.float32, device="cuda")
    announce(f"moe_ffn_q4k_q6k_noalloc over the limit T={T}")
    assert _noalloc_raw(fake, fake, fake, fake, fake, fake, y, T) == -4  # QMV_EUNSUPPORTED
