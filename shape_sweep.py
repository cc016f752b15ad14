"""Every layer shape of the four GPU workloads (headline p0..p100, Llama-3.1-8B layers,
Llama-3.1-70B layers, the decode/prefill mix), timed on the GPU, with both roofline
fractions: the GEMM's ops against the dense int8 peak and its algorithmic bytes against
HBM bandwidth, the binding one marked by the layer's arithmetic intensity.

  python shape_sweep.py [--cfgs 1,2,3,4] > table.txt

Per shape: the packed layer and the activations in rotating device sets (> 512 MB, so
the weights come from HBM), quant_act once per set, then a spin kernel and a run of GEMM
launches bracketed by HIP events on the launch stream (the host enqueues while the spin
kernel runs).  One line per shape, printed as it finishes.
"""
from __future__ import annotations

import argparse
import ctypes

import numpy as np

import bench  # the peaks and the algorithmic-bytes formula of the bench line


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--cfgs", default="1,2,3,4")
    ap.add_argument("--target-ms", type=float, default=20.0, help="GPU time per shape (approximate)")
    args = ap.parse_args(argv)
    import torch
    from weight_activation_quantized_amd import mixllm as L
    from weight_activation_quantized_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = L.library_handle()
    ridge = bench.PEAK_INT8_TOPS * 1e12 / (bench.PEAK_HBM_GBPS * 1e9)
    print(f"# {'cfg':>3s} {'layer':6s} {'M':>5s} {'N':>6s} {'K':>6s} {'n8':>5s} {'gemm_us':>9s} "
          f"{'TOPS':>8s} {'int8_frac':>9s} {'GB/s':>8s} {'hbm_frac':>8s} bound", flush=True)
    layers = {}
    for c in map(int, args.cfgs.split(",")):
        for sh in WL.config_shapes(c):
            layers.setdefault((c, sh.layer, sh.n, sh.k, sh.n8, sh.dist), []).append(sh)
    for (c, layer, n, k, n8, dist), shapes in layers.items():
        w16, idx8 = WL.make_layer_weights(shapes[0])
        blob_h = L.mixllm_pack_weights(w16, idx8)
        hdr = L.blob_header(blob_h)
        del w16
        g = k // 128
        for sh in shapes:
            m = sh.m
            a16 = WL.make_acts(m, k, sh.seed, dist)
            set_bytes = blob_h.size + m * k + 40 * g * m + 2 * m * n
            sets = max(2, min(64, int(np.ceil(600e6 / set_bytes))))
            base = torch.from_numpy(blob_h).to(dev)
            a = torch.from_numpy(a16).to(dev)
            S = []
            for i in range(sets):
                aq = torch.empty((m, k), dtype=torch.int8, device=dev)
                sa = torch.empty((g, m), dtype=torch.float32, device=dev)
                asum = torch.empty((g, m), dtype=torch.int32, device=dev)
                ro = L.rowop_buffer(m, k, dev)
                L.mixllm_quant_act(a, aq, sa, asum, ro)
                S.append((base if i == 0 else base.clone(), aq, sa, asum, ro,
                          torch.empty((m, n), dtype=torch.float16, device=dev)))
            st = torch.cuda.current_stream()
            sp = st.cuda_stream
            gargs = [(aq.data_ptr(), sa.data_ptr(), asum.data_ptr(), ro.data_ptr(), m, n, k, n8, ctypes.byref(hdr),
                      b.data_ptr(), b.numel(), y.data_ptr(), n, None, 0, sp) for b, aq, sa, asum, ro, y in S]
            rc = 0
            for i in range(3):
                rc = rc or lib.mixllm_gemm_w4w8a8(*gargs[i % sets])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = rc or lib.mixllm_gemm_w4w8a8(*gargs[0])
            e1.record(st)
            torch.cuda.synchronize()
            reps = int(max(10, min(2000, args.target_ms / max(e0.elapsed_time(e1), 1e-3))))
            torch.cuda._sleep(2 * bench.SPIN_CYCLES)
            e0.record(st)
            for i in range(reps):
                rc = rc or lib.mixllm_gemm_w4w8a8(*gargs[i % sets])
            e1.record(st)
            torch.cuda.synchronize()
            if rc:
                raise L.MixLLMError(rc)
            us = e0.elapsed_time(e1) * 1e3 / reps
            ops = 2.0 * m * n * k
            byt = bench.algorithmic_bytes(m, n, k, n8)
            tops, gbps = ops / us / 1e6, byt / us / 1e3
            bound = "mfma" if ops / byt >= ridge else "hbm"
            print(f"  {c:3d} {layer:6s} {m:5d} {n:6d} {k:6d} {n8:5d} {us:9.2f} {tops:8.1f} "
                  f"{tops / bench.PEAK_INT8_TOPS:9.4f} {gbps:8.1f} {gbps / bench.PEAK_HBM_GBPS:8.4f} {bound}",
                  flush=True)
            del S, base, a
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
