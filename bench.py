"""Benchmark of the block-quantized decode hot path on one MI355X.

Headline workload: Q4_K matvec, W[14336, 4096] (uniform[-1,1) quantized to
Q4_K, 33,030,144 packed bytes), x[4096] ~ N(0,1). One step runs every row
of the path that this workload has, on HBM-resident inputs, in two launches:
  qmv_q4k_qx       the f32-activation matvec, whose first workgroup also
                   writes quantize_act_q8(x) = (xq, xs, xsum)
  qmv_q4k_q8       int8 dot4 against the same weights
value = packed weight bytes read by the two matvecs / step time (GB/s). The
same step as three launches (qmv_q4k, quantize_act_q8, qmv_q4k_q8) is timed
and reported beside it.
Weights rotate over 32 device copies (1.06 GB) so every launch reads them
from HBM, not from the 256 MB last-level cache (warm numbers, one copy, are
reported beside).

The other workloads are measured after the headline and reported under
"others": Q8_0 4096x4096, Q6_K 128256x4096, the MoE layer (router + fused
gate/up/SiLU + down + combine, 128 experts, top-8, T = 1/4/16 tokens, in
tokens/s) and the m=512 Q4_K prefill GEMM (TOPS; its exact integer block
dots run on the f16 matrix instructions, and it is reported against both
the f16 and the int8 dense MFMA peaks).

Measured denominators beside the 8 TB/s datasheet peak: a 1 GiB
device-to-device copy, and the fastest plain read (qmv_roofline_read, a
sweep of grid sizes and loads in flight) of exactly the bytes one launch of
each dense matvec moves, over cold rotating copies.

cpu_baseline: the CPU oracle on the headline step, on one host thread and
on all the host's cores (threads over row slices), with the CPU model.

Prints ONE JSON line. `--gpus N` with N > 1 is refused: this path runs on a
single GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_I8_PEAK_TOPS = 5000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # the prefill contraction runs on f16 MFMA (exact integer products)
N2, K2 = 14336, 4096
Q4K_BYTES = N2 * (K2 // 256) * 144           # 33,030,144
# one qmv_q4k launch: every packed row (2,304 B) plus its f32 output, and x once
Q4K_LAUNCH_BYTES = Q4K_BYTES + 4 * N2 + 4 * K2  # 33,103,872
# one qmv_q4k_qx launch: the same plus the q8 row it writes (xq, xs, xsum)
QX_LAUNCH_BYTES = Q4K_LAUNCH_BYTES + K2 + 8 * (K2 // 32)  # 33,108,992
Q8_LAUNCH_BYTES = 4096 * 128 * 34 + 4 * 4096 + 4 * 4096      # Q8_0 4096x4096: 17,858,560
Q6K_LAUNCH_BYTES = 128256 * 16 * 210 + 4 * 128256 + 4 * 4096  # Q6_K 128256x4096: 431,469,568
CALIB_BYTES = 64 << 20                         # the counter-calibration copy
WARM_MS = 30.0            # untimed replays before each kernel timing
HEADLINE_WARM_MS = 100.0  # untimed steps before the headline's timed region (beyond --warmup)
TRAFFIC_JSON = os.path.join("profiles", "qmv_q4k_qx_14336x4096_traffic.json")
METRIC = "packed-weight GB/s (+% HBM peak) for Q4_K matvec 14336x4096; MoE tokens/s"
KERNEL_SOURCES = ["moe_ggml_block_amd/csrc/common.hpp",
                  "moe_ggml_block_amd/csrc/blocks.hpp", "moe_ggml_block_amd/csrc/dense.hpp",
                  "moe_ggml_block_amd/csrc/qmv_dense.hip"]


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def rotated(host_bytes, copies: int):
    """`copies` device copies of one host buffer, each 256-byte aligned."""
    import torch
    one = torch.from_numpy(host_bytes.reshape(-1)).cuda()
    nb = one.numel()
    stride = (nb + 255) // 256 * 256
    big = torch.empty(stride * copies, dtype=torch.uint8, device="cuda")
    views = []
    for i in range(copies):
        v = big[i * stride:i * stride + nb]
        v.copy_(one)
        views.append(v)
    del one
    return big, views


def capture(fn, calls: int):
    """A HIP graph of fn(0) .. fn(calls-1) launched back to back on one stream.
    Replaying it removes the host's per-launch cost from the timing."""
    import torch
    for i in range(min(calls, 3)):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    torch.cuda.synchronize()
    return g


def warm_replays(g, min_ms: float) -> int:
    """Replays g, untimed, until at least min_ms of wall time has passed (at
    least once): the GPU leaves its idle clocks during set-up phases that
    run on the host (weight generation), and the timed region should see
    the clocks a steady stream of launches runs at. Returns the replays run."""
    import time
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        g.replay()
        n += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n


def time_graph(fn, calls: int, replays: int = 20) -> float:
    """Average ms per fn call, over `replays` replays of a `calls`-call graph
    (after at least WARM_MS of untimed replays)."""
    import torch
    g = capture(fn, calls)
    warm_replays(g, WARM_MS)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) / (replays * calls)


def traffic_from_profile(kernel_hash: str):
    """HBM bytes per launch of qmv_q4k_qx from the committed PMC summary, if it was
    taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, TRAFFIC_JSON)
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("kernel_source_hash") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def host_cpu():
    """CPU model, logical CPU count and the CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


# threads the all-core oracle timing may use: the host's usable CPUs, at most
# this many (a GPU machine shares its host among its GPUs)
CPU_THREADS_MAX = 16


def cpu_baseline(seconds: float = 10.0):
    """The oracle, as it stands, on the headline step: f64 Q4_K matvec plus the
    f32 q8 quantizer and the f64 q8-activation matvec, full 14336x4096 shape,
    repeated until `seconds` of wall time have run, first on one host thread,
    then with the rows split over all usable cores (one Python thread per core,
    each calling the same single-threaded C oracle on a contiguous slice of
    rows; ctypes releases the interpreter lock during the call)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth
    w = synth.weights(synth.FMT_Q4K, synth.SEED_W, N2, K2)
    x = synth.normal(synth.SEED_X, K2)
    rb = (K2 // 256) * 144

    def rows(r0, r1, xq, xs):
        ws = w[r0 * rb:r1 * rb]
        oracle.matvec("q4k", ws, x, r1 - r0, K2)
        oracle.matvec_q8act("q4k", ws, xq, xs, r1 - r0, K2)

    def run(nthreads, budget):
        cuts = [N2 * i // nthreads for i in range(nthreads + 1)]
        steps = 0
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            t0 = time.perf_counter()
            while True:
                xq, xs, _ = oracle.quantize_act_q8(x, 1, K2)
                list(ex.map(lambda i: rows(cuts[i], cuts[i + 1], xq, xs), range(nthreads)))
                steps += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    return steps, el

    host = host_cpu()
    nthr = max(1, min(host["usable_cpus"], CPU_THREADS_MAX))
    s1, e1 = run(1, seconds / 2)
    sn, en = run(nthr, seconds / 2)
    gbs = lambda st, el: round(2 * Q4K_BYTES * st / el / 1e9, 4)
    return {"value": gbs(sn, en), "unit": "GB/s", "cores": nthr, "kind": "oracle",
            "sample": f"{sn} full oracle steps (Q4_K 14336x4096 f64 matvec + q8 quantize + f64 q8-activation "
                      f"matvec) in {en:.1f} s, rows split over {nthr} threads",
            "single_thread": {"value": gbs(s1, e1), "unit": "GB/s", "cores": 1,
                              "sample": f"{s1} full oracle steps in {e1:.1f} s on one thread"},
            "host": host}


def measured_floors(copy_bytes: int = 1 << 30):
    """Bandwidth denominators measured on this GPU: a one-shot device-to-device
    copy of copy_bytes (reported as read + write bytes per second), and, for
    each dense matvec of the bench, the fastest plain read of exactly the bytes
    one of its launches moves (qmv_roofline_read over cold rotating copies:
    1, 2, 4 or 8 workgroups of 256 per CU x 1, 2, 4 or 8 loads in flight per
    thread, best of the 16)."""
    import torch
    import moe_ggml_block_amd as qmv
    a = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    copy_ms = t0.elapsed_time(t1) / reps
    del a, b
    torch.cuda.empty_cache()
    out = {"copy_1GiB_gbs": round(2 * copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
           "copy_note": "torch copy_ of 1 GiB device to device; read + write bytes / time"}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for name, nbytes in (("qmv_q4k_14336x4096", Q4K_LAUNCH_BYTES),
                         ("qmv_q8_0_4096x4096", Q8_LAUNCH_BYTES),
                         ("qmv_q6k_128256x4096", Q6K_LAUNCH_BYTES)):
        nb = (nbytes + 15) // 16 * 16
        copies = max(3, -(-(1 << 30) // nb))
        big = torch.empty(nb * copies, dtype=torch.uint8, device="cuda")
        big.fill_(3)
        views = [big[i * nb:(i + 1) * nb] for i in range(copies)]
        best = None
        for wpc in (1, 2, 4, 8):
            for unr in (1, 2, 4, 8):
                ms = time_graph(lambda i: qmv.roofline_read(views[i % copies], nb, wpc * cus, unr, sink),
                                max(2 * copies, 16), 5)
                if best is None or ms < best[0]:
                    best = (ms, wpc, unr)
        ms, wpc, unr = best
        out[f"stream_read_{name}"] = {"bytes": nb, "us": round(ms * 1e3, 3),
                                      "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                                      "hbm_pct": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 1),
                                      "workgroups_per_cu": wpc, "loads_in_flight": unr, "copies": copies}
        del big, views
        torch.cuda.empty_cache()
    return out


def headline(steps: int, warmup: int, copies: int):
    import torch
    import moe_ggml_block_amd as qmv
    import synth

    log(f"headline: generating Q4_K {N2}x{K2} and {copies} device copies")
    w_host = synth.weights(synth.FMT_Q4K, synth.SEED_W, N2, K2)
    big, W = rotated(w_host, copies)
    x = torch.from_numpy(synth.normal(synth.SEED_X, K2)).cuda()
    y = torch.empty(N2, device="cuda")
    y8 = torch.empty(N2, device="cuda")
    xq = torch.empty(K2, dtype=torch.int8, device="cuda")
    xs = torch.empty(K2 // 32, device="cuda")
    xsum = torch.empty(K2 // 32, device="cuda")
    stream = torch.cuda.current_stream()

    # a step: the f32-activation matvec that also writes the q8 activation,
    # then the int8-dot matvec; the same work as three launches (separate
    # quantizer) and with the quantizer inside the int8 matvec's kernel
    # (qmv_q4k_q8x) is timed below as well
    def step(i):
        qmv.qmv_q4k_qx(W[i % copies], x, N2, K2, y=y, out=(xq, xs, xsum))
        qmv.qmv_q4k_q8(W[(i + copies // 2) % copies], xq, xs, xsum, N2, K2, y=y8)

    def step_three(i):
        qmv.qmv_q4k(W[i % copies], x, N2, K2, y=y)
        qmv.quantize_act_q8(x, 1, K2, out=(xq, xs, xsum))
        qmv.qmv_q4k_q8(W[(i + copies // 2) % copies], xq, xs, xsum, N2, K2, y=y8)

    def step_fused(i):
        qmv.qmv_q4k(W[i % copies], x, N2, K2, y=y)
        qmv.qmv_q4k_q8x(W[(i + copies // 2) % copies], x, N2, K2, y=y8)

    # one graph holds `copies` steps (every weight copy once per matvec);
    # the timed region replays it until exactly `steps` steps have run.
    full = capture(step, copies)
    rem = steps % copies
    tail = capture(step, rem) if rem else None
    for _ in range(max(1, warmup // copies)):
        full.replay()
    torch.cuda.synchronize()
    # more untimed steps if the requested warm-up was shorter than the clock
    # ramp (reported as warmup_steps_run)
    extra = warm_replays(full, HEADLINE_WARM_MS)
    warmup_run = max(1, warmup // copies) * copies + extra * copies
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps // copies):
        full.replay()
    if tail is not None:
        tail.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del full, tail

    # the dominant kernel alone: 4 passes over the copies per graph, on the
    # same stream, timed with events around the replays
    qx_ms = time_graph(lambda i: qmv.qmv_q4k_qx(W[i % copies], x, N2, K2, y=y, out=(xq, xs, xsum)),
                       4 * copies, 10)
    k_f32 = time_graph(lambda i: qmv.qmv_q4k(W[i % copies], x, N2, K2, y=y), 4 * copies, 10)
    k_qa = time_graph(lambda i: qmv.quantize_act_q8(x, 1, K2, out=(xq, xs, xsum)), 128, 10)
    k_q8 = time_graph(lambda i: qmv.qmv_q4k_q8(W[i % copies], xq, xs, xsum, N2, K2, y=y8), 4 * copies, 10)
    k_q8x = time_graph(lambda i: qmv.qmv_q4k_q8x(W[i % copies], x, N2, K2, y=y8), 4 * copies, 10)
    ms_fused = time_graph(step_fused, copies, 10)
    ms_three = time_graph(step_three, copies, 10)
    k_f32_warm = time_graph(lambda i: qmv.qmv_q4k(W[0], x, N2, K2, y=y), 128, 10)
    k_q8_warm = time_graph(lambda i: qmv.qmv_q4k_q8(W[0], xq, xs, xsum, N2, K2, y=y8), 128, 10)
    del big, W
    torch.cuda.empty_cache()
    return {
        "ms_per_step": ms,
        "warmup_steps_run": warmup_run,
        "qx_launch_ms": qx_ms,
        "kernels": {
            "qmv_q4k_qx_cold_us": round(qx_ms * 1e3, 3),
            "qmv_q4k_qx_cold_gbs": round(Q4K_BYTES / qx_ms / 1e6, 1),
            "qmv_q4k_cold_us": round(k_f32 * 1e3, 3),
            "qmv_q4k_cold_gbs": round(Q4K_BYTES / k_f32 / 1e6, 1),
            "qmv_q4k_warm_gbs": round(Q4K_BYTES / k_f32_warm / 1e6, 1),
            "quantize_act_q8_us": round(k_qa * 1e3, 3),
            "qmv_q4k_q8_cold_us": round(k_q8 * 1e3, 3),
            "qmv_q4k_q8_cold_gbs": round(Q4K_BYTES / k_q8 / 1e6, 1),
            "qmv_q4k_q8_warm_gbs": round(Q4K_BYTES / k_q8_warm / 1e6, 1),
            "qmv_q4k_q8x_cold_us": round(k_q8x * 1e3, 3),
            "qmv_q4k_q8x_cold_gbs": round(Q4K_BYTES / k_q8x / 1e6, 1),
            "step_three_launches_us": round(ms_three * 1e3, 3),
            "step_with_quantizer_in_int8_kernel_us": round(ms_fused * 1e3, 3),
        },
    }


def dense_other(fmt: str, n: int, k: int, copies: int):
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    f = {"q8_0": synth.FMT_Q8_0, "q6k": synth.FMT_Q6K, "q4_0": synth.FMT_Q4_0, "q5k": synth.FMT_Q5K}[fmt]
    fn = {"q8_0": qmv.qmv_q8_0, "q6k": qmv.qmv_q6k, "q4_0": qmv.qmv_q4_0, "q5k": qmv.qmv_q5k}[fmt]
    w_host = synth.weights(f, synth.SEED_W, n, k)
    nbytes = w_host.nbytes
    big, W = rotated(w_host, copies)
    del w_host
    x = torch.from_numpy(synth.normal(synth.SEED_X, k)).cuda()
    y = torch.empty(n, device="cuda")
    cold = time_graph(lambda i: fn(W[i % copies], x, n, k, y=y), max(4 * copies, 24), 10)
    warm = time_graph(lambda i: fn(W[0], x, n, k, y=y), 64, 10)
    del big, W
    torch.cuda.empty_cache()
    return {"shape": f"{n}x{k}", "packed_bytes": nbytes, "cold_us": round(cold * 1e3, 3),
            "cold_gbs": round(nbytes / cold / 1e6, 1), "cold_hbm_pct": round(nbytes / cold / 1e6 / HBM_PEAK_GBS * 100, 1),
            "warm_gbs": round(nbytes / warm / 1e6, 1), "weight_copies": copies}


def moe_other(bank_copies: int = 3, logit_sets: int = 64):
    import numpy as np
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    E, topk, hidden, inter = 128, 8, 2048, 768
    log("moe: generating banks")
    gate = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, inter, hidden)
    up = synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, inter, hidden)
    down = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, hidden, inter)
    per_expert = (gate.nbytes + up.nbytes + down.nbytes) // E
    bg, G = rotated(gate, bank_copies)
    bu, U = rotated(up, bank_copies)
    bd, D = rotated(down, bank_copies)
    del gate, up, down
    out = {}
    for T in (1, 4, 16):
        lg = [torch.from_numpy(synth.moe_logits(T, E, r)).cuda() for r in range(logit_sets)]
        x = torch.from_numpy(synth.normal(synth.SEED_X, T * hidden)).cuda()
        ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, topk), device="cuda")
        y = torch.empty((T, hidden), device="cuda")
        ws = torch.empty(qmv.moe_ffn_workspace_bytes(T, topk, hidden, inter), dtype=torch.uint8, device="cuda")

        def layer(i):
            b = i % bank_copies
            qmv.moe_route(lg[i % logit_sets], T, E, topk, out=(ids, wts))
            qmv.moe_ffn_q4k_q6k(G[b], U[b], D[b], x, ids, wts, T, topk, hidden, inter, E, y=y, ws=ws)

        ms = time_graph(layer, 2 * logit_sets, 5)
        wsq = torch.empty(qmv.moe_ffn_q8_workspace_bytes(T, topk, hidden, inter), dtype=torch.uint8, device="cuda")

        def layer_q8(i):
            b = i % bank_copies
            qmv.moe_route(lg[i % logit_sets], T, E, topk, out=(ids, wts))
            qmv.moe_ffn_q4k_q6k_q8(G[b], U[b], D[b], x, ids, wts, T, topk, hidden, inter, E, y=y, ws=wsq)

        ms_q8 = time_graph(layer_q8, 2 * logit_sets, 5)

        def layer_routed(i):
            b = i % bank_copies
            qmv.moe_ffn_routed_q4k_q6k(G[b], U[b], D[b], x, lg[i % logit_sets], T, topk, hidden, inter, E,
                                       out=(y, ids, wts), ws=ws)

        ms_rt = time_graph(layer_routed, 2 * logit_sets, 5)
        # unique experts actually routed, averaged over the logit sets
        uniq = []
        for r in range(logit_sets):
            i_, _ = qmv.moe_route(lg[r], T, E, topk)
            uniq.append(len(np.unique(i_.cpu().numpy())))
        u = float(np.mean(uniq))
        out[f"T{T}"] = {"tokens_per_s": round(T / (ms * 1e-3), 1), "layer_us": round(ms * 1e3, 3),
                        "q8_layer_us": round(ms_q8 * 1e3, 3), "q8_tokens_per_s": round(T / (ms_q8 * 1e-3), 1),
                        "routed_layer_us": round(ms_rt * 1e3, 3),
                        "routed_tokens_per_s": round(T / (ms_rt * 1e-3), 1),
                        "unique_experts": u, "gbs_unique_experts": round(u * per_expert / (ms * 1e-3) / 1e9, 1)}
    # router gate GEMV + router from the activations (a cold router matrix per
    # call: more copies than the last-level cache holds), and the whole MoE
    # block from the hidden state (gate GEMV + layer with the fused router)
    wr_host = synth.router_weights(E, hidden)
    br, R = rotated(wr_host.view(np.uint8), 320)
    for T in (1, 4, 16):
        x = torch.from_numpy(synth.normal(synth.SEED_X, T * hidden)).cuda()
        bufs = (torch.empty((T, E), device="cuda"), torch.empty((T, topk), dtype=torch.int32, device="cuda"),
                torch.empty((T, topk), device="cuda"))
        ms = time_graph(lambda i: qmv.moe_gate_route(R[i % 320], x, T, E, hidden, topk, out=bufs), 320, 5)
        out[f"T{T}"]["gate_route_us"] = round(ms * 1e3, 3)
        out[f"T{T}"]["gate_route_gbs"] = round(wr_host.nbytes / (ms * 1e-3) / 1e9, 1)
        y = torch.empty((T, hidden), device="cuda")
        ws = torch.empty(qmv.moe_ffn_workspace_bytes(T, topk, hidden, inter), dtype=torch.uint8, device="cuda")
        blk = (y,) + bufs
        ms_b = time_graph(lambda i: qmv.moe_block_q4k_q6k(R[i % 320], G[i % bank_copies], U[i % bank_copies],
                                                          D[i % bank_copies], x, T, topk, hidden, inter, E, out=blk,
                                                          ws=ws), 2 * 48, 5)
        out[f"T{T}"]["block_us"] = round(ms_b * 1e3, 3)
        out[f"T{T}"]["block_tokens_per_s"] = round(T / (ms_b * 1e-3), 1)
    del br, R, bg, bu, bd, G, U, D
    torch.cuda.empty_cache()
    return out


def prefill_other(copies: int = 64):
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    m, n, k = 512, 4096, 4096
    w_host = synth.weights(synth.FMT_Q4K, synth.SEED_W, n, k)
    big, W = rotated(w_host, copies)
    x = torch.from_numpy(synth.normal(synth.SEED_PREFILL_X, m * k)).cuda()
    xq, xs, xsum = qmv.quantize_act_q8(x, m, k)
    res = {}
    y8 = torch.empty((m, n), device="cuda")
    ms_i8 = time_graph(lambda i: qmv.qmm_q4k_i8(W[i % copies], xq, xs, xsum, m, n, k, y=y8), 2 * copies, 5)
    tops_i8 = 2.0 * m * n * k / (ms_i8 * 1e-3) / 1e12
    res["int8_mfma_tile"] = {"us": round(ms_i8 * 1e3, 2), "tops": round(tops_i8, 2),
                             "int8_peak_pct": round(tops_i8 / MFMA_I8_PEAK_TOPS * 100, 2),
                             "note": "qmm_q4k_i8: the bm=64 tile with block dots on v_mfma_i32_16x16x32_i8"}
    for bm in (64, 128, 256):
        y = torch.empty((m, n), device="cuda")
        ms = time_graph(lambda i: qmv.qmm_q4k(W[i % copies], xq, xs, xsum, m, n, k, bm=bm, y=y), 2 * copies, 5)
        tops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        res[f"bm{bm}"] = {"us": round(ms * 1e3, 2), "tops": round(tops, 2),
                          "mfma_f16_pct": round(tops / MFMA_F16_PEAK_TFLOPS * 100, 2),
                          "int8_peak_pct": round(tops / MFMA_I8_PEAK_TOPS * 100, 2)}
    ws = torch.empty(qmv.qmm_q4k_split_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    ms = time_graph(lambda i: qmv.qmm_q4k_split(W[i % copies], xq, xs, xsum, m, n, k, y=y, ws=ws), 2 * copies, 5)
    tops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    res["split"] = {"us": round(ms * 1e3, 2), "tops": round(tops, 2),
                    "mfma_f16_pct": round(tops / MFMA_F16_PEAK_TFLOPS * 100, 2),
                    "note": "qmm_q4k_split: activation pre-pass + GEMM, both launches"}
    del ws
    qa = time_graph(lambda i: qmv.quantize_act_q8(x, m, k, out=(xq, xs, xsum)), 32, 5)
    res["quantize_act_q8_us"] = round(qa * 1e3, 2)
    del big, W
    torch.cuda.empty_cache()
    # Q6_K prefill at the same shape (q8 activation)
    w6 = synth.weights(synth.FMT_Q6K, synth.SEED_W, n, k)
    big6, W6 = rotated(w6, copies)
    del w6
    y6 = torch.empty((m, n), device="cuda")
    ms6 = time_graph(lambda i: qmv.qmm_q6k(W6[i % copies], xq, xs, m, n, k, y=y6), 2 * copies, 5)
    res["q6k"] = {"us": round(ms6 * 1e3, 2), "tops": round(2.0 * m * n * k / (ms6 * 1e-3) / 1e12, 2),
                  "mfma_f16_pct": round(2.0 * m * n * k / (ms6 * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS * 100, 2)}
    del big6, W6
    torch.cuda.empty_cache()
    # Q8_0 prefill at the same shape
    w8 = synth.weights(synth.FMT_Q8_0, synth.SEED_W, n, k)
    big8, W8 = rotated(w8, copies)
    del w8
    ms8 = time_graph(lambda i: qmv.qmm_q8_0(W8[i % copies], xq, xs, m, n, k, y=y6), 2 * copies, 5)
    res["q8_0"] = {"us": round(ms8 * 1e3, 2), "tops": round(2.0 * m * n * k / (ms8 * 1e-3) / 1e12, 2),
                   "mfma_f16_pct": round(2.0 * m * n * k / (ms8 * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS * 100, 2)}
    del big8, W8
    torch.cuda.empty_cache()
    res["moe_qmm_q4k"] = moe_prefill_other()
    return res


def moe_prefill_other(bank_copies: int = 3):
    """Expert-indexed Q4_K prefill GEMM at the MoE layer's gate shape: 512
    tokens routed top-8 over 128 experts (router on N(0,1) logits), experts
    [768, 2048], one q8 activation row per token; banks rotate over cold copies."""
    import numpy as np
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    T, topk, E, n, k = 512, 8, 128, 768, 2048
    ns = T * topk
    bank = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, n, k)
    per_expert = bank.nbytes // E
    bb, B = rotated(bank, bank_copies)
    del bank
    lg = torch.from_numpy(synth.moe_logits(T, E)).cuda()
    ids, _ = qmv.moe_route(lg, T, E, topk)
    uniq = len(np.unique(ids.cpu().numpy()))
    x = torch.from_numpy(synth.normal(synth.SEED_PREFILL_X, T * k)).cuda()
    xq, xs, xsum = qmv.quantize_act_q8(x, T, k)
    y = torch.empty((ns, n), device="cuda")
    ms = time_graph(lambda i: qmv.moe_qmm_q4k(B[i % bank_copies], xq, xs, xsum, topk, ids, ns, n, k, E, y=y),
                    4 * bank_copies, 5)
    del bb, B
    torch.cuda.empty_cache()

    def line(ms, n_, k_, per_exp, shape):
        flops = 2.0 * ns * n_ * k_
        return {"shape": shape, "us": round(ms * 1e3, 2), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                "mfma_f16_pct": round(flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS * 100, 2),
                "unique_experts": uniq, "gbs_unique_experts": round(uniq * per_exp / (ms * 1e-3) / 1e9, 1)}

    res = {"moe_qmm_q4k_gate": line(ms, n, k, per_expert, f"T{T} top{topk} E{E} {n}x{k}")}
    # the down projection: Q6_K [2048, 768] experts on one f32 (and one q8) row per slot
    dbank = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, k, n)
    per_down = dbank.nbytes // E
    bd, D = rotated(dbank, bank_copies)
    del dbank
    h = torch.from_numpy(synth.normal(synth.SEED_X, ns * n)).cuda()
    hq, hs, _ = qmv.quantize_act_q8(h, ns, n)
    yd = torch.empty((ns, k), device="cuda")
    ms6 = time_graph(lambda i: qmv.moe_qmm_q6k_f32(D[i % bank_copies], h, 1, ids, ns, k, n, E, y=yd),
                     4 * bank_copies, 5)
    res["moe_qmm_q6k_f32_down"] = line(ms6, k, n, per_down, f"T{T} top{topk} E{E} {k}x{n}")
    ms6q = time_graph(lambda i: qmv.moe_qmm_q6k(D[i % bank_copies], hq, hs, 1, ids, ns, k, n, E, y=yd),
                      4 * bank_copies, 5)
    res["moe_qmm_q6k_q8_down"] = line(ms6q, k, n, per_down, f"T{T} top{topk} E{E} {k}x{n}")
    # the whole prefill layer (quantize, grouping, paired gate/up + SiLU, down, combine)
    gate = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, n, k)
    up = synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, n, k)
    bg, G = rotated(gate, bank_copies)
    bu, U = rotated(up, bank_copies)
    per_layer = (gate.nbytes + up.nbytes) // E + per_down
    del gate, up
    for TT in (32, 64, 128, 512, 2048):
        lgT = torch.from_numpy(synth.moe_logits(TT, E)).cuda()
        idsT, wT = qmv.moe_route(lgT, TT, E, topk)
        uT = len(np.unique(idsT.cpu().numpy()))
        xT = torch.from_numpy(synth.normal(synth.SEED_PREFILL_X, TT * k)).cuda()
        yT = torch.empty((TT, k), device="cuda")
        wsT = torch.empty(qmv.moe_ffn_prefill_workspace_bytes(TT, topk, k, n, E), dtype=torch.uint8, device="cuda")
        msL = time_graph(lambda i: qmv.moe_ffn_prefill_q4k_q6k(G[i % bank_copies], U[i % bank_copies],
                                                               D[i % bank_copies], xT, idsT, wT, TT, topk, k, n, E,
                                                               y=yT, ws=wsT), 2 * bank_copies, 3)
        res[f"layer_T{TT}"] = {"us": round(msL * 1e3, 1), "tokens_per_s": round(TT / (msL * 1e-3), 0),
                               "unique_experts": uT,
                               "gbs_unique_experts": round(uT * per_layer / (msL * 1e-3) / 1e9, 1),
                               "tflops": round(2.0 * TT * topk * 3 * n * k / (msL * 1e-3) / 1e12, 2)}
        del wsT
    del bd, D, bg, G, bu, U
    torch.cuda.empty_cache()
    return res


def profile_run(copies: int, other_shapes: bool = False):
    """Short eager run for rocprofv3: 64 launches each of qmv_q4k_qx, qmv_q4k
    and qmv_q4k_q8 over the rotating weight copies, 64 quantize_act_q8 calls, and
    8 launches of torch's elementwise neg over 16 Mi floats (a copy kernel
    that reads and writes exactly 64 MiB: it calibrates the FETCH_SIZE and
    WRITE_SIZE counters)."""
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    w_host = synth.weights(synth.FMT_Q4K, synth.SEED_W, N2, K2)
    big, W = rotated(w_host, copies)
    x = torch.from_numpy(synth.normal(synth.SEED_X, K2)).cuda()
    y = torch.empty(N2, device="cuda")
    xq, xs, xsum = qmv.quantize_act_q8(x, 1, K2)
    for i in range(64):
        qmv.qmv_q4k_qx(W[i % copies], x, N2, K2, y=y, out=(xq, xs, xsum))
    for i in range(64):
        qmv.qmv_q4k(W[i % copies], x, N2, K2, y=y)
    for i in range(64):
        qmv.quantize_act_q8(x, 1, K2, out=(xq, xs, xsum))
    for i in range(64):
        qmv.qmv_q4k_q8(W[i % copies], xq, xs, xsum, N2, K2, y=y)
    a = torch.ones(CALIB_BYTES // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(8):
        torch.neg(a, out=b)
    del big, W
    if other_shapes:
        for fmt, fn, n, k, reps in (("q8_0", qmv.qmv_q8_0, 4096, 4096, 32), ("q6k", qmv.qmv_q6k, 128256, 4096, 8)):
            f = {"q8_0": synth.FMT_Q8_0, "q6k": synth.FMT_Q6K}[fmt]
            bigo, Wo = rotated(synth.weights(f, synth.SEED_W, n, k), 3)
            yo = torch.empty(n, device="cuda")
            for i in range(reps):
                fn(Wo[i % 3], x, n, k, y=yo)
            del bigo, Wo
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": "qmv_q4k_qx x64, qmv_q4k x64, quantize_act_q8 x64, qmv_q4k_q8 x64, neg 64MiB x8"
                      + (", qmv_q8_0 4096x4096 x32, qmv_q6k 128256x4096 x8" if other_shapes else ""),
                      "q4k_bytes": Q4K_BYTES, "copy_bytes": CALIB_BYTES}))


def profile_q4k_run(copies: int, warm: bool):
    """For rocprofv3 kernel-trace: exactly the headline kernel's roofline timing
    (graphs of 4 x copies qmv_q4k_qx launches over the rotating cold copies,
    WARM_MS of untimed replays, then 10 replays), or with warm=True the same
    on one resident copy, so that the profiler's average duration is of one
    kind of launch only."""
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    big, W = rotated(synth.weights(synth.FMT_Q4K, synth.SEED_W, N2, K2), copies)
    x = torch.from_numpy(synth.normal(synth.SEED_X, K2)).cuda()
    y = torch.empty(N2, device="cuda")
    q8 = qmv.quantize_act_q8(x, 1, K2)
    if warm:
        ms = time_graph(lambda i: qmv.qmv_q4k_qx(W[0], x, N2, K2, y=y, out=q8), 128, 10)
    else:
        ms = time_graph(lambda i: qmv.qmv_q4k_qx(W[i % copies], x, N2, K2, y=y, out=q8), 4 * copies, 10)
    del big, W
    print(json.dumps({"profile_run": f"qmv_q4k_qx {N2}x{K2} {'warm (one copy)' if warm else f'cold ({copies} copies)'}",
                      "event_us_per_launch": round(ms * 1e3, 3)}))


def profile_moe_run(T: int, bank_copies: int = 3, calls: int = 48):
    """Short eager run for rocprofv3 counters of the MoE decode layer at T
    tokens (128 experts, top-8, gate/up Q4_K [768, 2048], down Q6_K
    [2048, 768]): `calls` x (moe_route + moe_ffn_q4k_q6k) over rotating bank
    copies and 64 logit sets, then the 64 MiB calibration copy (torch neg x8).
    Prints the unique experts of each call's routing, so that the summary can
    count the algorithmic bytes per dispatch."""
    import numpy as np
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    E, topk, hidden, inter = 128, 8, 2048, 768
    gate = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, inter, hidden)
    up = synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, inter, hidden)
    down = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, hidden, inter)
    bg, G = rotated(gate, bank_copies)
    bu, U = rotated(up, bank_copies)
    bd, D = rotated(down, bank_copies)
    lg = [torch.from_numpy(synth.moe_logits(T, E, r)).cuda() for r in range(64)]
    x = torch.from_numpy(synth.normal(synth.SEED_X, T * hidden)).cuda()
    ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, topk), device="cuda")
    y = torch.empty((T, hidden), device="cuda")
    ws = torch.empty(qmv.moe_ffn_workspace_bytes(T, topk, hidden, inter), dtype=torch.uint8, device="cuda")
    uniq = []
    for i in range(calls):
        b = i % bank_copies
        qmv.moe_route(lg[i % 64], T, E, topk, out=(ids, wts))
        qmv.moe_ffn_q4k_q6k(G[b], U[b], D[b], x, ids, wts, T, topk, hidden, inter, E, y=y, ws=ws)
        uniq.append(int(np.unique(ids.cpu().numpy()).size))
    a = torch.ones(CALIB_BYTES // 4, device="cuda")
    c = torch.empty_like(a)
    for _ in range(8):
        torch.neg(a, out=c)
    torch.cuda.synchronize()
    per_expert = (gate.nbytes + up.nbytes + down.nbytes) // E
    print(json.dumps({"profile_run": f"moe layer T={T} x{calls} (route + gate/up + down), neg 64MiB x8",
                      "unique_experts": uniq, "bytes_per_expert": per_expert,
                      "gate_up_bytes_per_expert": 2 * gate.nbytes // E, "down_bytes_per_expert": down.nbytes // E,
                      "copy_bytes": CALIB_BYTES}))


def profile_moe_prefill_run(bank_copies: int = 3, calls: int = 12):
    """Short eager run for rocprofv3 counters of the MoE prefill layer at 512
    tokens (128 experts, top-8, gate/up Q4_K [768, 2048], down Q6_K
    [2048, 768]) and of the standalone expert GEMMs at 4096 slots (the gate
    projection moe_qmm_q4k on the q8 x, the f32-activation down
    moe_qmm_q6k_f32): `calls` of each over rotating bank copies, then the
    64 MiB calibration copy (torch neg x8)."""
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    T, topk, E, hidden, inter = 512, 8, 128, 2048, 768
    ns = T * topk
    gate = synth.moe_bank(synth.FMT_Q4K, synth.SEED_GATE, E, inter, hidden)
    up = synth.moe_bank(synth.FMT_Q4K, synth.SEED_UP, E, inter, hidden)
    down = synth.moe_bank(synth.FMT_Q6K, synth.SEED_DOWN, E, hidden, inter)
    bg, G = rotated(gate, bank_copies)
    bu, U = rotated(up, bank_copies)
    bd, D = rotated(down, bank_copies)
    del gate, up, down
    lg = torch.from_numpy(synth.moe_logits(T, E)).cuda()
    ids, w = qmv.moe_route(lg, T, E, topk)
    x = torch.from_numpy(synth.normal(synth.SEED_PREFILL_X, T * hidden)).cuda()
    y = torch.empty((T, hidden), device="cuda")
    ws = torch.empty(qmv.moe_ffn_prefill_workspace_bytes(T, topk, hidden, inter, E), dtype=torch.uint8, device="cuda")
    h = torch.from_numpy(synth.normal(synth.SEED_X, ns * inter)).cuda()
    yd = torch.empty((ns, hidden), device="cuda")
    xq, xs, xsum = qmv.quantize_act_q8(x, T, hidden)
    yg = torch.empty((ns, inter), device="cuda")
    for i in range(calls):
        b = i % bank_copies
        qmv.moe_ffn_prefill_q4k_q6k(G[b], U[b], D[b], x, ids, w, T, topk, hidden, inter, E, y=y, ws=ws)
        qmv.moe_qmm_q4k(G[b], xq, xs, xsum, topk, ids, ns, inter, hidden, E, y=yg)
        qmv.moe_qmm_q6k_f32(D[b], h, 1, ids, ns, hidden, inter, E, y=yd)
    a = torch.ones(CALIB_BYTES // 4, device="cuda")
    c = torch.empty_like(a)
    for _ in range(8):
        torch.neg(a, out=c)
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": f"moe prefill layer T={T} x{calls}, moe_qmm_q4k and moe_qmm_q6k_f32 {ns} "
                                     f"slots x{calls}, neg 64MiB x8", "copy_bytes": CALIB_BYTES}))


def profile_prefill_run(copies: int = 64):
    """Short eager run for rocprofv3 counters of the Q4_K prefill GEMM:
    m=512 x W[4096, 4096], 20 launches each of qmm_q4k at bm = 64 and
    bm = 128 and of qmm_q4k_split over rotating weight copies, then the
    64 MiB calibration copy (torch neg x8)."""
    import torch
    import moe_ggml_block_amd as qmv
    import synth
    m, n, k = 512, 4096, 4096
    big, W = rotated(synth.weights(synth.FMT_Q4K, synth.SEED_W, n, k), copies)
    x = torch.from_numpy(synth.normal(synth.SEED_PREFILL_X, m * k)).cuda()
    xq, xs, xsum = qmv.quantize_act_q8(x, m, k)
    y = torch.empty((m, n), device="cuda")
    for bm in (64, 128):
        for i in range(20):
            qmv.qmm_q4k(W[i % copies], xq, xs, xsum, m, n, k, bm=bm, y=y)
    for i in range(20):
        qmv.qmm_q4k_i8(W[i % copies], xq, xs, xsum, m, n, k, y=y)
    ws = torch.empty(qmv.qmm_q4k_split_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    for i in range(20):
        qmv.qmm_q4k_split(W[i % copies], xq, xs, xsum, m, n, k, y=y, ws=ws)
    a = torch.ones(CALIB_BYTES // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(8):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": "qmm_q4k 512x4096x4096 bm=64 x20, bm=128 x20, qmm_q4k_i8 x20, qmm_q4k_split x20, "
                                     "neg 64MiB x8",
                      "copy_bytes": CALIB_BYTES}))


def counter_rows(csv_path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3
    counter_collection.csv."""
    import csv
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def write_traffic(fetch_csv: str, write_csv: str) -> dict:
    """HBM-side bytes per qmv_q4k_qx launch from two rocprofv3 --pmc runs of
    `bench.py --profile` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each
    scaled by what the counter reads for the 64 MiB neg copy. Writes the
    summary next to the other profiles and returns it."""
    import statistics

    def pick(rows, key):
        vals = [v for name, vs in rows.items() if key in name for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel named like {key!r}")
        return statistics.median(vals), len(vals)

    fetch, write = counter_rows(fetch_csv, "FETCH_SIZE"), counter_rows(write_csv, "WRITE_SIZE")
    f_q, nf = pick(fetch, "k_dense<Q4KQOutUnit, 64, 1>")
    w_q, nw = pick(write, "k_dense<Q4KQOutUnit, 64, 1>")
    f_c, _ = pick(fetch, "neg_kernel")
    w_c, _ = pick(write, "neg_kernel")
    fs, ws = CALIB_BYTES / (f_c * 1024), CALIB_BYTES / (w_c * 1024)
    hbm = f_q * 1024 * fs + w_q * 1024 * ws
    d = {"kernel": "qmv_q4k_qx (k_dense<Q4KQOutUnit, 64, 1>)", "workload": "Q4_K 14336x4096, 32 rotating weight copies",
         "kernel_source_hash": source_hash(KERNEL_SOURCES),
         "fetch_kib_median": f_q, "write_kib_median": w_q, "dispatches": [nf, nw],
         "calib_fetch_kib": f_c, "calib_write_kib": w_c, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
         "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": QX_LAUNCH_BYTES,
         "ratio_to_algorithmic": round(hbm / QX_LAUNCH_BYTES, 4)}
    with open(os.path.join(ROOT, TRAFFIC_JSON), "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--profile", action="store_true", help="short eager run for rocprofv3")
    ap.add_argument("--profile-all", action="store_true", help="--profile plus the Q8_0 and Q6_K shapes")
    ap.add_argument("--profile-prefill", action="store_true", help="short eager prefill run for rocprofv3")
    ap.add_argument("--profile-cold", action="store_true",
                    help="only the headline kernel's cold roofline timing (graph replays), for rocprofv3")
    ap.add_argument("--profile-warm", action="store_true", help="the same on one resident weight copy")
    ap.add_argument("--profile-moe", type=int, metavar="T", help="short eager MoE decode layer run at T tokens")
    ap.add_argument("--profile-moe-prefill", action="store_true", help="short eager MoE prefill layer run")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarize two rocprofv3 --pmc runs of --profile into the traffic file, then exit")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--copies", type=int, default=32)
    ap.add_argument("--no-others", action="store_true", help="headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-floors", action="store_true", help="skip the measured copy / read denominators")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    a = ap.parse_args()
    if a.write_traffic:
        print(json.dumps(write_traffic(*a.write_traffic)))
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this decode path runs on one GPU; --gpus must be 1 "
              "(multi-GPU sharding is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import moe_ggml_block_amd as qmv  # noqa: F401  (fails loudly without libqmv.so)

    if a.profile or a.profile_all:
        profile_run(a.copies, a.profile_all)
        return
    if a.profile_prefill:
        profile_prefill_run()
        return
    if a.profile_moe:
        profile_moe_run(a.profile_moe)
        return
    if a.profile_moe_prefill:
        profile_moe_prefill_run()
        return
    if a.profile_cold or a.profile_warm:
        profile_q4k_run(a.copies, a.profile_warm)
        return
    khash = source_hash(KERNEL_SOURCES)
    h = headline(a.steps, a.warmup, a.copies)
    log(f"headline done: {h['ms_per_step'] * 1e3:.2f} us/step")
    value = 2 * Q4K_BYTES / (h["ms_per_step"] * 1e-3) / 1e9
    qx_us = h["qx_launch_ms"] * 1e3
    achieved = QX_LAUNCH_BYTES / (h["qx_launch_ms"] * 1e-3) / 1e9
    traffic = traffic_from_profile(khash)
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "warmup_steps_run": h["warmup_steps_run"],
        "ms_per_step": round(h["ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Q4_K matvec 14336x4096, batch 1: f32-activation matvec (writing the q8 "
                               "activation) + int8-dot4 matvec per step",
                   "n": N2, "k": K2, "weight_copies": a.copies, "cache": "cold (rotating copies)"},
        "hbm_pct": round(value / HBM_PEAK_GBS * 100, 2),
        "roofline": {"kernel": "qmv_q4k_qx", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": QX_LAUNCH_BYTES, "avg_launch_us": round(qx_us, 3),
                     "kernel_source_hash": khash},
        "kernels": h["kernels"],
    }
    if not a.no_floors:
        log("measured floors: 1 GiB copy, plain reads of each matvec's bytes")
        fl = measured_floors()
        res["measured_floors"] = fl
        q4f = fl["stream_read_qmv_q4k_14336x4096"]["gbs"]
        res["roofline"]["frac_of_measured_read"] = round(achieved / q4f, 4)
        res["roofline"]["frac_of_copy_1GiB"] = round(achieved / fl["copy_1GiB_gbs"], 4)
        res["kernels"]["qmv_q4k_qx_cold_pct_of_measured_read"] = round(achieved / q4f * 100, 1)
        res["kernels"]["qmv_q4k_cold_pct_of_measured_read"] = round(
            Q4K_LAUNCH_BYTES / (h["kernels"]["qmv_q4k_cold_us"] * 1e-6) / 1e9 / q4f * 100, 1)
        q8a = Q4K_LAUNCH_BYTES - 4 * K2 + K2 + 8 * (K2 // 32)  # its launch: q8 x instead of f32 x
        res["kernels"]["qmv_q4k_q8_cold_pct_of_measured_read"] = round(
            q8a / (h["kernels"]["qmv_q4k_q8_cold_us"] * 1e-6) / 1e9 / q4f * 100, 1)
    if not a.no_others:
        others = {}
        log("others: q8_0")
        others["q8_0_4096x4096"] = dense_other("q8_0", 4096, 4096, 64)
        log("others: q6k")
        others["q6k_128256x4096"] = dense_other("q6k", 128256, 4096, 3)
        if "measured_floors" in res:
            fl = res["measured_floors"]
            for key, fkey, lb in (("q8_0_4096x4096", "stream_read_qmv_q8_0_4096x4096", Q8_LAUNCH_BYTES),
                                  ("q6k_128256x4096", "stream_read_qmv_q6k_128256x4096", Q6K_LAUNCH_BYTES)):
                gbs = lb / (others[key]["cold_us"] * 1e-6) / 1e9
                others[key]["cold_pct_of_measured_read"] = round(gbs / fl[fkey]["gbs"] * 100, 1)
        log("others: q4_0, q5k")
        others["q4_0_14336x4096"] = dense_other("q4_0", 14336, 4096, 32)
        others["q5k_14336x4096"] = dense_other("q5k", 14336, 4096, 32)
        log("others: moe")
        others["moe_layer"] = moe_other()
        log("others: prefill")
        others["prefill_q4k_512x4096x4096"] = prefill_other()
        res["others"] = others
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(a.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
