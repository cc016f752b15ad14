#!/usr/bin/env python3
"""Benchmark of the W4.4A8 mixed-precision linear layer on one MI355X.

One step = the whole hot path over one batch: mixllm_quant_act (fp16 activations ->
int8 + group scales) then mixllm_gemm_w4w8a8 (mixed 4/8-bit GEMM with scatter
epilogue), with inputs and packed weights already resident in HBM.  Packing is offline
(once per layer) and not part of a step.

Workload: M=512 tokens, N=K=4096, group 128, 410 of 4096 output channels (10%) 8-bit,
synthetic seeded inputs (weights N(0, 0.02) with 4 outlier channels x8, activations
N(0, 1) with 2% of input columns x20).  The step cycles through enough independent
(weights, activations, output) sets that the working set exceeds the 256 MB last-level
cache, so every step reads its weights from HBM.

Prints one JSON line.  value = 2 M N K / step time, in TOPS (int8 ops; each
multiply-add counts 2).  roofline: the GEMM kernel's own duration, measured with HIP
events on its launch stream inside the timed region, against the dense int8 MFMA peak.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
SPIN_CYCLES = 50_000_000    # head start of the timed region (about 20 ms of GPU clock)
TRAFFIC_FILE = os.path.join(HERE, "profiles", "gemm_w4w8a8_M512_N4096_K4096_p10_traffic.json")
GEMM_SRC = os.path.join(HERE, "weight_activation_quantized_amd", "csrc", "mixllm_gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: enough for >512 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--m", type=int, default=512)
    ap.add_argument("--n", type=int, default=4096)
    ap.add_argument("--k", type=int, default=4096)
    ap.add_argument("--p8", type=float, default=0.10)
    ap.add_argument("--workload", default="layer", choices=["layer", "mlp", "qkv"],
                    help="layer: the W4.4A8 layer step (default); mlp: the Llama-3.1-8B MLP block "
                         "(quantize, gate/up GEMM, SiLU*up + quantize, down GEMM) replayed as a HIP graph; "
                         "qkv: the Llama-3.1-8B q/k/v projections (one quantize, one GEMM over the three "
                         "packed as one layer)")
    ap.add_argument("--variant", default="",
                    help="time a measured variant of the tile GEMM (libmixllm_<name>.so: fold_bias, zero_pre) "
                         "instead of the library")
    ap.add_argument("--pipelined", action="store_true",
                    help="also time the same steps on two streams, the quant_act launches of the "
                         "next half of the rotating sets beside the GEMMs of this half "
                         "(reported as an extra object; the serial step stays the value)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB before the steps, as the "
                         "known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE counters")
    return ap.parse_args()


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(gemm_hash, m, n, k, n8):
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of the headline shape, or None for another shape or when absent or taken on
    a different kernel source."""
    if (m, n, k, n8) != (512, 4096, 4096, 410):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != gemm_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def algorithmic_bytes(m, n, k, n8):
    """Bytes the layer must move: 4-bit codes + 4-bit zero points + fp16 scales of the
    4-bit channels, int8 codes + fp16 scales of the 8-bit channels, a 4-byte channel
    index per output channel, int8 activations + fp32 activation scales, fp16 output."""
    g, n4 = k // 128, n - n8
    return (n4 * k / 2 + n4 * g * 2.5 + n8 * k + n8 * g * 2 + 4 * n
            + m * k + 4 * m * g + 2 * m * n)


def pipelined_steps(args, quant_on, gemm_on, sets):
    """ms per step of the same steps on two streams: chunks of half the rotating sets; the
    quant_act launches of chunk c (stream Q) wait for the GEMMs of chunk c - 2, which read
    the same buffers, and the GEMMs of chunk c (stream G) wait for chunk c's quant_act
    launches, so quantizing the next chunk overlaps this chunk's GEMMs."""
    import torch
    h = sets // 2
    if h < 1:
        raise SystemExit("--pipelined needs at least 2 rotating sets")
    chunks = [(i, min(h, args.steps - i)) for i in range(0, args.steps, h)]
    sq, sg = torch.cuda.Stream(), torch.cuda.Stream()
    eq = [torch.cuda.Event() for _ in chunks]
    eg = [torch.cuda.Event() for _ in chunks]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(sg):
        torch.cuda._sleep(SPIN_CYCLES)
    e0.record(sg)
    sq.wait_event(e0)
    rc = 0
    for c, (i0, cnt) in enumerate(chunks):
        if c >= 2:
            sq.wait_event(eg[c - 2])
        for i in range(i0, i0 + cnt):
            rc = rc or quant_on(i, sq.cuda_stream)
        eq[c].record(sq)
        sg.wait_event(eq[c])
        for i in range(i0, i0 + cnt):
            rc = rc or gemm_on(i, sg.cuda_stream)
        eg[c].record(sg)
    e1.record(sg)
    torch.cuda.synchronize()
    if rc:
        raise SystemExit(f"pipelined steps: status {rc}")
    return e0.elapsed_time(e1) / args.steps


def cpu_baseline(m, n, k, n8):
    """The CPU oracle as it stands, on the same workload (the full layer: quantize
    activations and weights, two-step dequantized GEMM)."""
    import numpy as np
    import oracle as O
    from weight_activation_quantized_amd import workloads as WL
    sh = WL.Shape(1, "p10", m, n, k, n8)
    a16, w16, idx8 = WL.make_layer_inputs(sh)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    # bounded sample: whole-layer passes until about 10 s of CPU work (at least one)
    reps, dt = 0, 0.0
    while reps == 0 or (dt < 10.0 and reps < 20):
        t0 = time.perf_counter()
        O.layer_forward(a16, w16, idx8)
        dt += time.perf_counter() - t0
        reps += 1
    out = {"value": round(2.0 * m * n * k * reps / dt / 1e12, 6), "unit": "TOPS", "cores": int(cores),
           "kind": "oracle",
           "sample": f"{reps} pass(es) of the oracle layer (quantize activations and weights + fp64 "
                     f"two-step GEMM), M={m} N={n} K={k} n8={n8}, {dt:.2f} s"}
    # the same oracle on one BLAS thread: one pass
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.layer_forward(a16, w16, idx8)
            d1 = time.perf_counter() - t0
        out["one_thread"] = {"value": round(2.0 * m * n * k / d1 / 1e12, 6), "unit": "TOPS",
                             "sample": f"1 pass, {d1:.2f} s"}
        out["blas"] = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()})
    except Exception as e:  # pragma: no cover
        out["one_thread"] = f"not measured: {e}"
    try:
        with open("/proc/cpuinfo") as f:
            out["cpu"] = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:  # pragma: no cover
        out["cpu"] = None
    out["nproc"] = os.cpu_count()
    return out


def mlp_main(args):
    """The Llama-3.1-8B MLP block at M tokens as a second workload: four launches per
    block; the blocks of every rotating set captured in sequence as one HIP graph, a step
    being one block (a replay is `sets` steps).  One graph per block and eager launches
    through the Python wrapper are reported beside it."""
    import numpy as np
    import torch
    from weight_activation_quantized_amd import mixllm as L
    from weight_activation_quantized_amd import workloads as WL

    m = args.m
    hidden, inter = WL.MLP8B["hidden"], WL.MLP8B["inter"]
    n8 = WL.llama8b_n8()
    torch.cuda.set_device(0)
    x16, wg, wu, wd, ig, iu, idn = WL.mlp_block_inputs(m, hidden, inter, n8)
    blk0 = L.MLPBlock(wg, wu, wd, ig, iu, idn)
    set_bytes = blk0.gu.blob.nbytes + blk0.down.blob.nbytes + m * (hidden + 2 * inter) * 6
    sets = args.sets or max(2, int(np.ceil(512e6 / set_bytes)))
    blocks = [blk0] + [L.MLPBlock(wg, wu, wd, ig, iu, idn) for _ in range(sets - 1)]
    xs = [torch.from_numpy(x16).cuda() for _ in range(sets)]
    bufs = [b.buffers(m) for b in blocks]
    graphs = [b.capture(x, bb) for b, x, bb in zip(blocks, xs, bufs)]
    for i in range(args.warmup):
        graphs[i % sets].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    single_ms, graph_host = timed_loop(args.steps, lambda i: graphs[i % sets].replay(), stream)
    chain = capture_chain([lambda st, b=b, x=x, bb=bb: b.forward(x, bb, st) for b, x, bb in zip(blocks, xs, bufs)])
    reps = max(1, args.steps // sets)
    chain.replay()
    step_ms, chain_host = timed_loop(reps, lambda i: chain.replay(), stream)
    step_ms, chain_host = step_ms / sets, chain_host / sets
    # the same blocks launched eagerly, for comparison
    for i in range(args.warmup):
        blocks[i % sets].forward(xs[i % sets], bufs[i % sets], stream)
    torch.cuda.synchronize()
    eager_ms, eager_host = timed_loop(
        args.steps, lambda i: blocks[i % sets].forward(xs[i % sets], bufs[i % sets], stream), stream)
    ops = 2.0 * m * 3 * inter * hidden
    out = {
        "metric": "Llama-3.1-8B MLP block TOPS (W4.4A8, HIP graph of one block per rotating set, chained)",
        "value": round(ops / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": reps * sets,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B MLP block M={m} hidden={hidden} inter={inter}: quant_act, "
                               f"gate/up GEMM (N={2 * inter}), SiLU*up + quant, down GEMM; 8-bit channels "
                               f"gate {n8['gate']}, up {n8['up']}, down {n8['down']}",
                   "M": m, "hidden": hidden, "inter": inter, "rotating_sets": sets},
        "eager_ms_per_step": round(eager_ms, 5),
        "eager_tops": round(ops / (eager_ms * 1e-3) / 1e12, 2),
        "steps_per_replay": sets,
        "chain_host_us_per_step": round(chain_host, 2),
        "single_block_graph_ms_per_step": round(single_ms, 5),
        "single_block_graph_tops": round(ops / (single_ms * 1e-3) / 1e12, 2),
        "graph_host_us_per_replay": round(graph_host, 2),
        "eager_host_us_per_step": round(eager_host, 2),
    }
    print(json.dumps(out), flush=True)


def timed_loop(steps, fn, stream=None):
    """(GPU ms per call, host us per call) of `steps` calls of fn queued behind a spin
    kernel: the GPU time is the events' span; the host time is how long the loop took to
    enqueue, which bounds the GPU time from below whenever it is the larger of the two."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    e0.record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    host_us = (time.perf_counter() - t0) * 1e6 / steps
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, host_us


def capture_chain(forwards):
    """One HIP graph of several forward passes in sequence (each f(stream) enqueues one step
    on its own buffers): the runtime leaves the GPU idle between two graph launches (about
    8 us on this stack, against none between kernels inside a graph), so chaining the steps
    of every rotating set into one graph pays that gap once per chain instead of per step."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in forwards:
            f(s)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in forwards:
            f(s)
    return g


def qkv_main(args):
    """The Llama-3.1-8B q/k/v projections at M tokens: one quant_act of the hidden state
    and one GEMM over the three projections packed as one layer (6144 channels).  The
    value is the step (both launches) by raw C calls; the same steps replayed as HIP graphs
    and launched through the Python wrapper are reported beside it with the host time each
    takes to enqueue a step."""
    import numpy as np
    import torch
    from weight_activation_quantized_amd import mixllm as L
    from weight_activation_quantized_amd import workloads as WL

    m = args.m
    hidden, nq, nkv = WL.QKV8B["hidden"], WL.QKV8B["q"], WL.QKV8B["kv"]
    n8 = WL.llama8b_n8()
    torch.cuda.set_device(0)
    x16, wq, wk, wv, iq, ik, iv = WL.qkv_inputs(m, hidden, nq, nkv, n8)
    p0 = L.QKVProjection(wq, wk, wv, iq, ik, iv)
    n = nq + 2 * nkv
    n8_all = n8["q"] + n8["k"] + n8["v"]
    set_bytes = p0.layer.blob.nbytes + m * hidden * 6 + m * n * 2
    sets = args.sets or max(2, int(np.ceil(512e6 / set_bytes)))
    projs = [p0] + [L.QKVProjection(wq, wk, wv, iq, ik, iv) for _ in range(sets - 1)]
    xs = [torch.from_numpy(x16).cuda() for _ in range(sets)]
    bufs = [pj.buffers(m) for pj in projs]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    lib = L.library_handle()
    qa_fn, gm_fn = lib.mixllm_quant_act, lib.mixllm_gemm_w4w8a8
    hdr_p = ctypes.byref(p0.layer.blob.info)
    qargs = [(x.data_ptr(), hidden, m, hidden, 128, b["aq"].data_ptr(), b["sa"].data_ptr(), b["asum"].data_ptr(),
              b["rowop"].data_ptr(), sp) for x, b in zip(xs, bufs)]
    gargs = [(b["aq"].data_ptr(), b["sa"].data_ptr(), b["asum"].data_ptr(), b["rowop"].data_ptr(), m, n, hidden,
              n8_all, hdr_p, pj.layer.blob.dev.data_ptr(), pj.layer.blob.nbytes, b["y"].data_ptr(), n, None, 0, sp)
             for pj, b in zip(projs, bufs)]

    def raw(i):
        qa_fn(*qargs[i % sets])
        gm_fn(*gargs[i % sets])

    rc = 0
    for i in range(args.warmup):
        rc = rc or qa_fn(*qargs[i % sets]) or gm_fn(*gargs[i % sets])
    torch.cuda.synchronize()
    if rc:
        raise L.MixLLMError(rc)
    step_ms, raw_host = timed_loop(args.steps, raw, stream)

    def py(i):
        projs[i % sets].forward(xs[i % sets], bufs[i % sets], stream)

    for i in range(min(args.warmup, 50)):
        py(i)
    py_ms, py_host = timed_loop(args.steps, py, stream)
    graphs = [pj.capture(x, b) for pj, x, b in zip(projs, xs, bufs)]
    for i in range(min(args.warmup, 50)):
        graphs[i % sets].replay()
    g_ms, g_host = timed_loop(args.steps, lambda i: graphs[i % sets].replay(), stream)
    chain = capture_chain([lambda st, pj=pj, x=x, b=b: pj.forward(x, b, st) for pj, x, b in zip(projs, xs, bufs)])
    reps = max(1, args.steps // sets)
    chain.replay()
    c_ms, c_host = timed_loop(reps, lambda i: chain.replay(), stream)
    c_ms, c_host = c_ms / sets, c_host / sets
    ops = 2.0 * m * n * hidden
    tops = lambda ms: round(ops / (ms * 1e-3) / 1e12, 2)
    out = {
        "metric": "Llama-3.1-8B q/k/v projection TOPS (W4.4A8)",
        "value": tops(step_ms),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B q/k/v projections M={m} hidden={hidden}: one quant_act, one GEMM "
                               f"over q|k|v packed as one layer (N={n}); 8-bit channels q {n8['q']}, k {n8['k']}, "
                               f"v {n8['v']}",
                   "M": m, "N": n, "K": hidden, "n8": n8_all, "rotating_sets": sets},
        "host_us_per_step": round(raw_host, 2),
        "python_wrapper": {"ms_per_step": round(py_ms, 5), "tops": tops(py_ms), "host_us_per_step": round(py_host, 2)},
        "hip_graph": {"ms_per_step": round(g_ms, 5), "tops": tops(g_ms), "host_us_per_replay": round(g_host, 2)},
        "hip_graph_chain": {"ms_per_step": round(c_ms, 5), "tops": tops(c_ms), "steps_per_replay": sets,
                            "host_us_per_step": round(c_host, 2)},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the path runs on one GPU: --gpus must be 1 (a multi-GPU run would "
                          "shard the output channels; it is not implemented)"}))
        sys.exit(2)
    if args.workload == "mlp":
        return mlp_main(args)
    if args.workload == "qkv":
        return qkv_main(args)

    import numpy as np
    import torch
    if args.variant:
        os.environ["MIXLLM_LIB"] = os.path.join(HERE, "weight_activation_quantized_amd",
                                                f"libmixllm_{args.variant}.so")
    from weight_activation_quantized_amd import mixllm as L
    from weight_activation_quantized_amd import workloads as WL

    m, n, k = args.m, args.n, args.k
    n8 = WL.n8_fraction(n, args.p8)
    g = k // 128
    sh = WL.Shape(1, "p10", m, n, k, n8)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # one packed layer + activations on the host, replicated into rotating device sets
    a16, w16, idx8 = WL.make_layer_inputs(sh)
    blob_host = L.mixllm_pack_weights(w16, idx8)
    set_bytes = blob_host.size + m * k * 2 + m * k + 40 * g * m + 2 * m * n
    sets = args.sets or max(4, int(np.ceil(512e6 / set_bytes)))
    base_blob = torch.from_numpy(blob_host).to(dev)
    hdr = L.blob_header(blob_host)   # the host header the GEMM checks each call against
    base_a = torch.from_numpy(a16).to(dev)
    S = []
    for _ in range(sets):
        S.append(dict(blob=base_blob.clone(), a=base_a.clone(),
                      aq=torch.empty((m, k), dtype=torch.int8, device=dev),
                      sa=torch.empty((g, m), dtype=torch.float32, device=dev),
                      asum=torch.empty((g, m), dtype=torch.int32, device=dev),
                      rowop=L.rowop_buffer(m, k, dev),
                      y=torch.empty((m, n), dtype=torch.float16, device=dev)))
    ws_bytes = L.mixllm_gemm_workspace_bytes(m, n, k, n8)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.current_stream()
    if args.copy_calib_mib:
        src = torch.ones(args.copy_calib_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Launch arguments of every set, prepared once: the timed loop makes two plain C calls
    # per step, so the host enqueues steps faster than the GPU runs them.
    lib = L.library_handle()
    qa_fn, gm_fn = lib.mixllm_quant_act, lib.mixllm_gemm_w4w8a8
    sp = stream.cuda_stream
    wsp, wsb = (ws.data_ptr(), ws.numel()) if ws is not None else (None, 0)
    qargs = [(s["a"].data_ptr(), k, m, k, 128, s["aq"].data_ptr(), s["sa"].data_ptr(), s["asum"].data_ptr(),
              s["rowop"].data_ptr(), sp) for s in S]
    hdr_p = ctypes.byref(hdr)
    gargs = [(s["aq"].data_ptr(), s["sa"].data_ptr(), s["asum"].data_ptr(), s["rowop"].data_ptr(), m, n, k, n8,
              hdr_p, s["blob"].data_ptr(), s["blob"].numel(), s["y"].data_ptr(), n, wsp, wsb, sp) for s in S]

    def quant(i):
        return qa_fn(*qargs[i % sets])

    def quant_args_on(i, st):
        return qa_fn(*(qargs[i % sets][:-1] + (st,)))

    def gemm_args_on(i, st):
        return gm_fn(*(gargs[i % sets][:-1] + (st,)))

    def gemm(i):
        return gm_fn(*gargs[i % sets])

    rc = 0
    for i in range(args.warmup):
        rc = rc or quant(i) or gemm(i)
    torch.cuda.synchronize()
    if rc:
        raise L.MixLLMError(rc)

    # Timed region: exactly `steps` steps, each quant_act + GEMM on its own batch (set).
    # The steps run in chunks of `sets`: the chunk's quant_act launches, then its GEMM
    # launches, with one HIP event on the launch stream after each run of launches, so
    # the per-kernel durations come from events without an event between every two
    # kernels (an event costs a few microseconds of queue time).  A spin kernel queued
    # first keeps the GPU busy while the host enqueues; the step clock starts at the
    # event after it.
    chunks = [(i, min(sets, args.steps - i)) for i in range(0, args.steps, sets)]
    e_start = torch.cuda.Event(enable_timing=True)
    e_q = [torch.cuda.Event(enable_timing=True) for _ in chunks]
    e_g = [torch.cuda.Event(enable_timing=True) for _ in chunks]
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    e_start.record(stream)
    for c, (i0, cnt) in enumerate(chunks):
        for i in range(i0, i0 + cnt):
            rc = rc or quant(i)
        e_q[c].record(stream)
        for i in range(i0, i0 + cnt):
            rc = rc or gemm(i)
        e_g[c].record(stream)
    torch.cuda.synchronize()
    if rc:
        raise L.MixLLMError(rc)
    step_ms = e_start.elapsed_time(e_g[-1]) / args.steps
    piped = pipelined_steps(args, quant_args_on, gemm_args_on, sets) if args.pipelined else None
    q_ms = sum((e_start if c == 0 else e_g[c - 1]).elapsed_time(e_q[c]) for c in range(len(chunks)))
    g_ms = sum(e_q[c].elapsed_time(e_g[c]) for c in range(len(chunks)))
    gemm_us = 1e3 * g_ms / args.steps
    quant_us = 1e3 * q_ms / args.steps

    ops = 2.0 * m * n * k
    value = ops / (step_ms * 1e-3) / 1e12
    gemm_tops = ops / (gemm_us * 1e-6) / 1e12
    alg_bytes = algorithmic_bytes(m, n, k, n8)
    gemm_hash = src_hash(GEMM_SRC)
    # counters were taken on the library at the headline shape
    traffic = None if args.variant else traffic_for(gemm_hash, m, n, k, n8)
    # The dominant kernel's roofline: the matrix cores when the layer's arithmetic
    # intensity (ops per algorithmic byte) is above the ridge, else HBM bandwidth.
    ridge = PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if ops / alg_bytes >= ridge:
        roofline = {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                    "unit": "TOPS", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4)}
    else:
        gbps = alg_bytes / (gemm_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    roofline.update({"traffic": traffic, "kernel": "mixllm_gemm_w4w8a8",
                     "algorithmic_ops_per_launch": ops, "algorithmic_bytes_per_launch": alg_bytes,
                     "avg_launch_us": round(gemm_us, 3)})
    out = {
        "metric": "W4.4A8 GEMM TOPS at M=512,N=K=4096; % of int8 MFMA peak / HBM BW",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"W4.4A8 mixed linear layer M={m} N={n} K={k} group=128 n8={n8} "
                               f"(p{round(100 * n8 / n)}); step = quant_act + mixed GEMM",
                   "M": m, "N": n, "K": k, "n8": n8, "group": 128, "rotating_sets": sets,
                   "variant": args.variant or None},
        "roofline": roofline,
        **({"pipelined": {"ms_per_step": round(piped, 5), "value": round(ops / (piped * 1e-3) / 1e12, 2),
                          "unit": "TOPS",
                          "schedule": "two streams: the quant_act launches of one half of the rotating "
                                      "sets run beside the GEMM launches of the other half"}}
           if piped else {}),
        "gemm_us": round(gemm_us, 3),
        "quant_act_us": round(quant_us, 3),
        "gemm_hbm_frac_algorithmic": round(alg_bytes / (gemm_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "quant_act_gbps": round(m * k * (2 + 1 + 4 / 128) / (quant_us * 1e-6) / 1e9, 1),
        "gemm_source_sha256_16": gemm_hash,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(m, n, k, n8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
