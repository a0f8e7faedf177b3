"""Throughput of the NVFP4 W4A4 linear layer on one MI355X.

One step = the whole hot path on one batch: quantize the activations to NVFP4
(per-tensor amax -> global scale -> E4M3 block scales -> E2M1 codes) and run the
block-scaled GEMM against pre-quantized, pre-packed weights, FP32 out.  Inputs
are resident in HBM before the timed region.  Steps are captured in a HIP graph
(one replay covers a whole rotation of weight copies) so the host launch rate
does not limit the measurement.

Prints one JSON line (rank 0) with the headline metric (TFLOP/s of the step,
activation quantization included), the roofline of the dominant kernel (the
GEMM) measured with HIP events on the launch stream, and the CPU oracle timed on
a bounded sample of the same workload.

Default workload: the large prefill layer, X[32768 x 16384] bf16 against
W[16384 x 16384] NVFP4 (the largest single-GPU shape: the pages quote their
single-layer speedup at the largest hidden sizes).  --config selects another
workload; decode-skinny rotates 40 weight copies (590 MB > the 256 MB Infinity
Cache) so its weight stream comes from HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 W4A4 GEMM TFLOPS incl. act-quantize; % of MFMA/HBM roofline at 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense FP16/BF16 matrix cores

CONFIG_NAMES = {"tiny": "tiny", "decode": "decode-skinny", "gdn": "gdn-fused-input-projection",
                "ngpt": "ngpt-d4096", "large": "large-prefill-d16384"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--config", default="large", choices=sorted(CONFIG_NAMES))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    p.add_argument("--minimal", action="store_true",
                   help="time only the step, the product and the quantizer (profiler runs: one shape per kernel)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB 22 times, 20 of them timed (calibrates HBM byte counters; the copy rate)")
    return p.parse_args()


def quantizer_launches(rows, K, dtype, cus=256):
    """Kernels nvfp4_quantize runs for a dense, aligned tensor with g computed (the library's rule):
    one for up to 8192 blocks (every workgroup reduces the whole tensor), one for tensors with at least
    1024 amax segments of 8192 elements that fit one workgroup per compute unit holding 1024 threads x 8
    (bf16) or 4 (FP32) blocks (the one-pass quantizer), two otherwise (amax pass, then the encoder)."""
    blocks = rows * (K // 16)
    if blocks <= 1024 * (8 if dtype == "bf16" else 4):
        return 1
    segments = -(-(rows * K) // 8192)
    if segments >= 1024 and blocks <= cus * 1024 * (8 if dtype == "bf16" else 4):
        return 1
    return 2


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel, from the committed counter runs (profiles/traffic.json),
    or None when there are none for this workload or the kernel's sources have changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec["traffic_bytes"] if h.hexdigest() == rec["sources_sha256"] else None


def copy_probe(mib):
    """A copy of known size: the HBM byte counters of its kernel scale those of the product kernels, and
    its rate (reads plus writes) is the ceiling of a pass that reads and writes HBM, as the encoder does."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):   # untimed: first touch of the destination
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 20
    print(json.dumps({"copy_probe_bytes": n, "launches": 22, "timed": 20, "us_per_copy": t * 1e6,
                      "read_plus_write_gbs": 2 * n / t / 1e9}), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch
    import nvfp4_block_scaled_03_amd as nv
    import workloads

    name = args.config
    small = name in ("tiny", "decode")
    steps = args.steps if args.steps is not None else (2000 if small else 20)
    # the big products keep speeding up over their first ~15 launches (clocks settle), so warm up past that
    warmup = args.warmup if args.warmup is not None else (200 if small else 50)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    wl = workloads.make(name)
    log(f"workload {name}: M={wl.M} K={wl.K} N={wl.N} modules={[w.shape[0] for w in wl.w]} "
        f"generated in {time.time() - t0:.1f}s")
    M, K, N = wl.M, wl.K, wl.N
    xdt = torch.bfloat16 if wl.x_dtype == "bf16" else torch.float32
    x = torch.from_numpy(wl.x).to(dev).to(xdt)
    in_dtype = nv.NVFP4_IN_BF16 if xdt == torch.bfloat16 else nv.NVFP4_IN_F32

    # weights: quantized per module (own global scale) and packed once, outside the timed region
    w_dev = [torch.from_numpy(w).to(dev).to(torch.bfloat16 if wl.w_dtype == "bf16" else torch.float32)
             for w in wl.w]
    mods = [nv.quantize(w) for w in w_dev]
    packed = nv.PackedWeight(mods, K)
    copies = 40 if name == "decode" else 1
    weights = [packed] + [packed.clone() for _ in range(copies - 1)]
    # the standard transformer's NVFP4 recipe (randomized Hadamard transform before quantization, g computed),
    # which nGPT does without: both operands transformed with the same signs, weights packed once
    extra = not args.minimal        # the variants below: g given, gates, bf16 Y, RHT, backward
    rht_on = extra and name in ("ngpt", "gdn")
    if rht_on:
        signs = workloads.rht_signs()
        packed_rht = nv.PackedWeight([nv.quantize_rht(w, signs) for w in w_dev], K)
    w_first = w_dev[0] if name == "ngpt" else None     # the nGPT backward reads W
    if not wl.quantize_w_in_step:
        del w_dev
    torch.cuda.synchronize()

    codes, scales, g = nv.empty_quantized(M, K, dev)
    ws = torch.empty((max(nv.nvfp4_quantize_workspace_bytes(M, K), 256),), dtype=torch.uint8, device=dev)
    lin_ws = nv.linear_workspace(M, xdt, packed, dev)       # zero-filled once, reused by every step
    skinny = M <= 16     # few-token path: one kernel (amax, quantize and product)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    gemm_ws = torch.zeros((max(nv.nvfp4_gemm_workspace_bytes(M, packed.desc), 256),), dtype=torch.uint8,
                          device=dev)       # (the product needs none at these shapes; a minimal one is passed)
    if wl.quantize_w_in_step:
        wq_bufs = [nv.empty_quantized(w.shape[0], K, dev) for w in w_dev]
        wq_ws = [torch.empty((max(nv.nvfp4_quantize_workspace_bytes(w.shape[0], K), 256),), dtype=torch.uint8,
                             device=dev) for w in w_dev]
        blob_step = torch.empty_like(packed.blob)

    def step(i):
        desc = weights[i % copies].desc
        if wl.quantize_w_in_step:   # tiny case: both operands quantized inside the step, the weights packed
            for w, (c, s, gg), wsb in zip(w_dev, wq_bufs, wq_ws):
                nv.nvfp4_quantize(w, c, s, gg, nv.NVFP4_G_COMPUTE, wsb)
            desc = nv.nvfp4_pack_weights(wq_bufs, K, blob_step)
        nv.nvfp4_linear(x, codes, scales, g, desc, y, lin_ws, M=M, ld_x=K, in_dtype=in_dtype, ld_y=N)

    # the decode step with one weight copy, which stays in the Infinity Cache (labelled hot-cache figure)
    step_hot = None
    if extra and copies > 1:
        codes_h, scales_h, g_h = nv.empty_quantized(M, K, dev)
        y_h = torch.empty((M, N), dtype=torch.float32, device=dev)
        lin_ws_h = nv.linear_workspace(M, xdt, packed, dev)

        def step_hot(i):
            nv.nvfp4_linear(x, codes_h, scales_h, g_h, packed.desc, y_h, lin_ws_h, M=M, ld_x=K, in_dtype=in_dtype,
                            ld_y=N)

    # the same layer without per-tensor scaling (the nGPT recipe): g given as 1, no amax pass
    codes1, scales1, g1 = nv.empty_quantized(M, K, dev)
    g1.fill_(1.0)
    y1 = torch.empty((M, N), dtype=torch.float32, device=dev)
    lin_ws1 = nv.linear_workspace(M, xdt, packed, dev)

    def step_given(i):
        nv.nvfp4_linear(x, codes1, scales1, g1, weights[i % copies].desc, y1, lin_ws1, nv.NVFP4_G_GIVEN, M=M, ld_x=K,
                        in_dtype=in_dtype, ld_y=N)

    # the GDN projection with its gate epilogue fused (decay and write-strength columns)
    gate_p = workloads.gdn_gate_params() if extra and name == "gdn" else None
    if gate_p is not None:
        gates = nv.GdnGates(gate_p.a_col, gate_p.n_a, gate_p.b_col, gate_p.n_b,
                            torch.from_numpy(gate_p.a_log).to(dev), torch.from_numpy(gate_p.dt_bias).to(dev))
        yg = torch.empty((M, N), dtype=torch.float32, device=dev)
        codes_g, scales_g, g_g = nv.empty_quantized(M, K, dev)

        def step_gated(i):
            nv.nvfp4_linear(x, codes_g, scales_g, g_g, weights[i % copies].desc, yg, lin_ws, M=M, ld_x=K,
                            in_dtype=in_dtype, ld_y=N, gates=gates)

    # training backward of the nGPT layer (nGPT trains end to end in NVFP4): dX = dY . W and dW = dY^T . X,
    # every operand quantized along its contraction axis inside the step (dY along N for dX; W, dY and X
    # along their rows, i.e. transposed), the two transposed weights packed, then the two products
    bwd = None
    if extra and name == "ngpt":
        dy_np = workloads.random_matrix(workloads.SEEDS["ngpt"] + 7, M, N, 1e-3, "bf16")
        dy = torch.from_numpy(dy_np).to(dev).to(torch.bfloat16)
        w_full = w_first

        def qbufs(rows, kdim):
            return (*nv.empty_quantized(rows, kdim, dev),
                    torch.empty((max(nv.nvfp4_quantize_workspace_bytes(rows, kdim), 256),), dtype=torch.uint8,
                                device=dev))
        a_dx, wt, a_dw, xt = qbufs(M, N), qbufs(K, N), qbufs(N, M), qbufs(K, M)
        blob_wt = torch.empty((nv.nvfp4_packed_weight_bytes([K], N),), dtype=torch.uint8, device=dev)
        blob_xt = torch.empty((nv.nvfp4_packed_weight_bytes([K], M),), dtype=torch.uint8, device=dev)
        dx = torch.empty((M, K), dtype=torch.float32, device=dev)
        dw = torch.empty((N, K), dtype=torch.float32, device=dev)

        def step_backward(i):
            # dY in both orientations from one read (one g), W and X transposed
            nv.nvfp4_quantize_both(dy, a_dx[0], a_dx[1], a_dw[0], a_dw[1], a_dx[2], nv.NVFP4_G_COMPUTE, a_dx[3])
            nv.nvfp4_quantize_t(w_full, *wt[:3], nv.NVFP4_G_COMPUTE, wt[3])
            d_wt = nv.nvfp4_pack_weights([wt[:3]], N, blob_wt)
            nv.nvfp4_gemm(M, a_dx[0], a_dx[1], a_dx[2], d_wt, dx, K, None)
            nv.nvfp4_quantize_t(x, *xt[:3], nv.NVFP4_G_COMPUTE, xt[3])
            d_xt = nv.nvfp4_pack_weights([xt[:3]], M, blob_xt)
            nv.nvfp4_gemm(N, a_dw[0], a_dw[1], a_dx[2], d_xt, dw, K, None)

        def quant_t_only(i):
            nv.nvfp4_quantize_t(x, *xt[:3], nv.NVFP4_G_COMPUTE, xt[3])

        # weight re-quantization per training step (W changes after every optimizer step): W along K, packed
        wq = qbufs(N, K)
        blob_w = torch.empty((nv.nvfp4_packed_weight_bytes([N], K),), dtype=torch.uint8, device=dev)

        def requant_w(i):
            nv.nvfp4_quantize(w_full, *wq[:3], nv.NVFP4_G_COMPUTE, wq[3], rows=N, K=K, ld_x=K,
                              in_dtype=nv.NVFP4_IN_BF16)
            nv.nvfp4_pack_weights([wq[:3]], K, blob_w)

        # both packed operands of W per step (forward along K, backward transposed), separately and fused
        blob_wt2 = torch.empty_like(blob_wt)
        g_tr = torch.empty((1,), dtype=torch.float32, device=dev)

        def requant_both_separate(i):
            requant_w(i)
            nv.nvfp4_quantize_t(w_full, *wt[:3], nv.NVFP4_G_COMPUTE, wt[3])
            nv.nvfp4_pack_weights([wt[:3]], N, blob_wt)

        def requant_both_fused(i):
            nv.nvfp4_pack_weights_train(w_full, g_tr, blob_w, blob_wt2, nv.NVFP4_G_COMPUTE, wq[3])
        bwd = (step_backward, quant_t_only, requant_w, requant_both_separate, requant_both_fused)

    if rht_on:
        codes_r, scales_r, g_r = nv.empty_quantized(M, K, dev)
        y_r = torch.empty((M, N), dtype=torch.float32, device=dev)

        def step_rht(i):
            nv.nvfp4_quantize_rht(x, signs, codes_r, scales_r, g_r, nv.NVFP4_G_COMPUTE, ws)
            nv.nvfp4_gemm(M, codes_r, scales_r, g_r, packed_rht.desc, y_r, N, gemm_ws)

        def quant_rht_only(i):
            nv.nvfp4_quantize_rht(x, signs, codes_r, scales_r, g_r, nv.NVFP4_G_COMPUTE, ws)

    # the same layer writing Y as bf16 (with the gates for the GDN projection, whose output feeds the recurrence)
    y_b = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    codes_b, scales_b, g_b = nv.empty_quantized(M, K, dev)

    def step_bf16(i):
        nv.nvfp4_linear(x, codes_b, scales_b, g_b, weights[i % copies].desc, y_b, lin_ws, M=M, ld_x=K,
                        in_dtype=in_dtype, ld_y=N, gates=gates if gate_p is not None else None)

    # the FP8 KV-cache quantizer (the page's calibrated FP8 scales), on a K-cache-shaped tensor of the GDN model
    kv = None
    if extra and name == "gdn":
        kv_np = workloads.kv_cache()
        kv_x = torch.from_numpy(kv_np).to(dev).to(torch.bfloat16)
        kv_codes = torch.empty(kv_np.shape, dtype=torch.uint8, device=dev)
        kv_s = torch.empty((1,), dtype=torch.float32, device=dev)
        kv_ws = torch.empty((max(nv.nvfp4_quantize_workspace_bytes(*kv_np.shape), 256),), dtype=torch.uint8,
                            device=dev)
        kv_codes_g = torch.empty_like(kv_codes)
        kv_sg = torch.full((1,), 0.05, dtype=torch.float32, device=dev)

        def kv_calibrated(i):
            nv.nvfp4_kv_quantize_fp8(kv_x, kv_codes, kv_s, nv.NVFP4_G_COMPUTE, kv_ws)

        def kv_given(i):
            nv.nvfp4_kv_quantize_fp8(kv_x, kv_codes_g, kv_sg, nv.NVFP4_G_GIVEN, None)
        kv = (kv_calibrated, kv_given)

    def gemm_only(i):
        nv.nvfp4_gemm(M, codes, scales, g, weights[i % copies].desc, y, N, gemm_ws)

    def quant_only(i):
        nv.nvfp4_quantize(x, codes, scales, g, nv.NVFP4_G_COMPUTE, ws, rows=M, K=K, ld_x=K, in_dtype=in_dtype)

    stream = torch.cuda.Stream()
    # steps per replayed graph: the weight rotation for the few-token case; 10 otherwise, so the ~9 us
    # launch of a graph is paid once per 10 steps, as in a captured model with many layers
    rot = copies if copies > 1 else 10

    def make_runner(fn, count):
        """Runs fn(0..count-1) once per call: as a replayed HIP graph, or eagerly."""
        if args.no_graph:
            def run():
                for i in range(count):
                    fn(i)
            return run
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for i in range(count):       # eager warm-up on the capture stream
                fn(i)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(count):
                fn(i)
        torch.cuda.synchronize()
        return graph.replay

    def timed(fn, n_steps, n_warm):
        """Run n_warm untimed then exactly n_steps steps; returns seconds for the n_steps."""
        per = rot if n_steps >= rot else n_steps
        full = make_runner(fn, per)
        rem = n_steps % per
        rem_run = make_runner(fn, rem) if rem else None
        for _ in range(max(1, n_warm // per)):
            full()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        e0.record(cur)
        for _ in range(n_steps // per):
            full()
        if rem_run:
            rem_run()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    log(f"timing {steps} steps after {warmup} warm-up steps (graph={'no' if args.no_graph else 'yes'})")
    t_step = timed(step, steps, warmup) / steps
    # dominant kernel and the quantizer alone, same launch configuration, events on the launch stream
    k_steps = max(steps, rot)
    t_gemm = timed(gemm_only, k_steps, min(warmup, k_steps)) / k_steps
    t_quant = timed(quant_only, k_steps, min(warmup, k_steps)) / k_steps
    t_given = timed(step_given, k_steps, min(warmup, k_steps)) / k_steps if extra else None
    t_hot = timed(step_hot, k_steps, min(warmup, k_steps)) / k_steps if step_hot else None
    clock = observed_gfx_clock(make_runner(step, rot)) if extra else None
    t_gated = timed(step_gated, k_steps, min(warmup, k_steps)) / k_steps if gate_p is not None else None
    t_bf16 = timed(step_bf16, k_steps, min(warmup, k_steps)) / k_steps if extra else None
    t_rht = timed(step_rht, k_steps, min(warmup, k_steps)) / k_steps if rht_on else None
    t_qrht = timed(quant_rht_only, k_steps, min(warmup, k_steps)) / k_steps if rht_on else None
    t_kv = timed(kv[0], k_steps, min(warmup, k_steps)) / k_steps if kv else None
    t_kvg = timed(kv[1], k_steps, min(warmup, k_steps)) / k_steps if kv else None
    t_bwd = timed(bwd[0], k_steps, min(warmup, k_steps)) / k_steps if bwd else None
    t_qt = timed(bwd[1], k_steps, min(warmup, k_steps)) / k_steps if bwd else None
    t_rq = timed(bwd[2], k_steps, min(warmup, k_steps)) / k_steps if bwd else None
    t_rq2 = timed(bwd[3], k_steps, min(warmup, k_steps)) / k_steps if bwd else None
    t_rqf = timed(bwd[4], k_steps, min(warmup, k_steps)) / k_steps if bwd else None

    flops = 2.0 * M * N * K
    tflops = flops / t_step / 1e12
    w_bytes = N * K * 9 // 16
    x_q_bytes = M * K * 9 // 16
    x_in_bytes = M * K * (2 if wl.x_dtype == "bf16" else 4)
    if skinny:
        # the step is one launch of the few-token kernel (amax, quantize and product): its bytes
        # are the weights (codes + scales), the activations in, their codes and scales out, and Y
        kern, t_kern = "skinny_kernel (amax + quantize + product, one launch)", t_step
        kern_bytes = w_bytes + x_in_bytes + x_q_bytes + M * N * 4
    else:
        kern, t_kern = "gemm_tile_kernel", t_gemm
        kern_bytes = w_bytes + x_q_bytes + M * N * 4
    if M <= 16:
        roof = {"bound": "hbm", "achieved": kern_bytes / t_kern / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t_kern / 1e12, "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if M > 16:   # the whole step (activation quantization included) against the same peak
        roof["step_frac"] = tflops / F16_MFMA_PEAK_TFLOPS
    roof["traffic"] = measured_traffic(CONFIG_NAMES[name])
    roof["kernel"] = kern
    roof["kernel_us"] = t_kern * 1e6
    roof["algorithmic_bytes_per_launch"] = kern_bytes

    # parity of the last step (codes bit-exact, outputs within tolerance), on sampled rows for big M
    torch.cuda.synchronize()
    from oracle import nvfp4_ref as ref
    rng = np.random.default_rng(0)
    rows = np.arange(M) if M <= 64 else np.unique(np.concatenate([[0, M - 1], rng.choice(M, 16, replace=False)]))
    gx = ref.global_scale(np.float32(np.abs(wl.x).max()))
    xq = ref.quantize(wl.x[rows], g_mode="given", g=gx)
    codes_ok = bool(np.array_equal(codes[torch.from_numpy(rows).to(dev)].cpu().numpy(), xq.codes) and
                    np.array_equal(scales[torch.from_numpy(rows).to(dev)].cpu().numpy(), xq.scales) and
                    np.float32(g.item()) == gx)
    cols = np.arange(N) if N <= 8192 else np.unique(rng.choice(N, 512, replace=False))
    parts, off = [], 0
    for w in wl.w:
        sel = cols[(cols >= off) & (cols < off + w.shape[0])] - off
        if len(sel):
            gw = ref.global_scale(np.float32(np.abs(w).max()))
            parts.append(ref.dequantize(ref.quantize(w[sel], g_mode="given", g=gw)))
        off += w.shape[0]
    y_ref, a_ref = ref.gemm_dequantized(ref.dequantize(xq), np.concatenate(parts))
    yd = y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)].cpu().numpy()
    y_ok, worst = ref.gemm_within_tolerance(yd, y_ref, a_ref)
    gated_ok, gated_worst = None, None
    if gate_p is not None:   # gate columns of the sampled rows against the gate oracle
        from oracle import gdn_gates as gref
        ia, ib = wl.module_names.index("a"), wl.module_names.index("b")
        wab = np.concatenate([ref.dequantize(ref.quantize(wl.w[ia])), ref.dequantize(ref.quantize(wl.w[ib]))])
        yab, aab = ref.gemm_dequantized(ref.dequantize(xq), wab)
        gargs = (0, gate_p.n_a, gate_p.b_col - gate_p.a_col, gate_p.n_b, gate_p.a_log.astype(np.float64),
                 gate_p.dt_bias.astype(np.float64))
        gcols = torch.arange(gate_p.a_col, gate_p.b_col + gate_p.n_b, device=dev)
        got = yg[torch.from_numpy(rows).to(dev)][:, gcols].cpu().numpy()
        gated_ok, gated_worst = gref.within(got, gref.apply_gates(yab, *gargs), gref.gates_tolerance(yab, aab, *gargs))
    rht_parity = None
    if rht_on:   # sampled rows of the transformed codes, and of the product against the transformed weights
        from oracle import rht as rref
        tx = rref.rht_blocks(wl.x, signs)
        g_t = ref.global_scale(np.float32(np.abs(tx).max()))
        txq = ref.quantize(tx[rows], "given", g_t)
        del tx
        rsel = torch.from_numpy(rows).to(dev)
        r_codes_ok = bool(np.array_equal(codes_r[rsel].cpu().numpy(), txq.codes) and
                          np.array_equal(scales_r[rsel].cpu().numpy(), txq.scales) and np.float32(g_r.item()) == g_t)
        parts_r, off = [], 0
        for w in wl.w:
            sel = cols[(cols >= off) & (cols < off + w.shape[0])] - off
            if len(sel):
                tw = rref.rht_blocks(w, signs)
                parts_r.append(ref.dequantize(ref.quantize(tw[sel], "given",
                                                           ref.global_scale(np.float32(np.abs(tw).max())))))
            off += w.shape[0]
        yr_ref, ar_ref = ref.gemm_dequantized(ref.dequantize(txq), np.concatenate(parts_r))
        yr = y_r[rsel][:, torch.from_numpy(cols).to(dev)].cpu().numpy()
        r_ok, r_worst = ref.gemm_within_tolerance(yr, yr_ref, ar_ref)
        rht_parity = {"codes_scales_bit_exact": r_codes_ok, "gemm_within_1e-5": bool(r_ok), "worst_ratio": r_worst}
    kv_parity = None
    if kv:   # every byte and the calibrated scale against the oracle
        from oracle import fp8_kv
        oc, os_ = fp8_kv.quantize_kv(kv_np)
        ocg, _ = fp8_kv.quantize_kv(kv_np, "given", 0.05)
        kv_parity = {"bytes_and_scale_bit_exact": bool(np.array_equal(kv_codes.cpu().numpy(), oc) and
                                                       np.float32(kv_s.item()) == os_),
                     "given_scale_bytes_bit_exact": bool(np.array_equal(kv_codes_g.cpu().numpy(), ocg))}
    bwd_parity = None
    if bwd:   # sampled entries of dX and dW, and sampled rows of the transposed encodings, against the oracle
        rsel = torch.from_numpy(rows).to(dev)
        csel = np.unique(np.concatenate([[0, K - 1], rng.choice(K, 14, replace=False)]))
        nsel = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 14, replace=False)]))
        g_dy = ref.global_scale(np.float32(np.abs(dy_np).max()))
        g_w = ref.global_scale(np.float32(np.abs(wl.w[0]).max()))
        g_x = ref.global_scale(np.float32(np.abs(wl.x).max()))
        dyq = ref.quantize(dy_np[rows], "given", g_dy)
        wtq = ref.quantize_t(wl.w[0][:, csel], "given", g_w)
        dx_ref, dx_a = ref.gemm_dequantized(ref.dequantize(dyq), ref.dequantize(wtq))
        dx_got = dx[rsel][:, torch.from_numpy(csel).to(dev)].cpu().numpy()
        dx_ok, dx_worst = ref.gemm_within_tolerance(dx_got, dx_ref, dx_a)
        dytq = ref.quantize_t(dy_np[:, nsel], "given", g_dy)
        xtq = ref.quantize_t(wl.x[:, csel], "given", g_x)
        dw_ref, dw_a = ref.gemm_dequantized(ref.dequantize(dytq), ref.dequantize(xtq))
        dw_got = dw[torch.from_numpy(nsel).to(dev)][:, torch.from_numpy(csel).to(dev)].cpu().numpy()
        dw_ok, dw_worst = ref.gemm_within_tolerance(dw_got, dw_ref, dw_a)
        nsel_t = torch.from_numpy(nsel).to(dev)
        t_codes_ok = bool(np.array_equal(a_dw[0][nsel_t].cpu().numpy(), dytq.codes) and
                          np.array_equal(a_dw[1][nsel_t].cpu().numpy(), dytq.scales) and
                          np.float32(a_dx[2].item()) == g_dy)
        bwd_parity = {"transposed_codes_scales_bit_exact": t_codes_ok, "dX_within_1e-5": bool(dx_ok),
                      "dX_worst_ratio": dx_worst, "dW_within_1e-5": bool(dw_ok), "dW_worst_ratio": dw_worst}
    # bf16 Y: the round-to-nearest-even of the FP32 Y of the same step (the gated FP32 Y for GDN)
    bf16_ok, given_ok = None, None
    if extra:
        y32 = yg if gate_p is not None else y
        bf16_ok = bool(torch.equal(y_b, y32.to(torch.bfloat16)))
        xq1 = ref.quantize(wl.x[rows], g_mode="given", g=1.0)
        given_ok = bool(np.array_equal(codes1[torch.from_numpy(rows).to(dev)].cpu().numpy(), xq1.codes) and
                        np.array_equal(scales1[torch.from_numpy(rows).to(dev)].cpu().numpy(), xq1.scales))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, ref)

    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 w4a4 -> f16 mfma, f32 acc",
        "data": "synthetic (seeded; distributions of the pages' workloads)",
        "config": {"workload": CONFIG_NAMES[name], "M": M, "K": K, "N": N,
                   "modules": [int(w.shape[0]) for w in wl.w], "x_dtype": wl.x_dtype,
                   "weight_copies": copies, "graph": not args.no_graph, "variants_timed": extra},
        "roofline": roof,
        "cpu_baseline": cpu,
        # launches: few tokens one kernel; otherwise the quantizer's (one or two, quantizer_launches) and
        # the product's (two when the weight has a ragged column edge, as the GDN projection); tiny adds
        # the weights' quantize and pack
        "step_breakdown_us": {"step (nvfp4_linear)": t_step * 1e6,
                              "launches_per_step": 1 if skinny else (
                                  quantizer_launches(M, K, wl.x_dtype) + (2 if N % 256 else 1)
                                  + (sum(quantizer_launches(w.shape[0], K, wl.w_dtype) for w in wl.w) + 1
                                     if wl.quantize_w_in_step else 0)),
                              "quantize alone": t_quant * 1e6, "gemm alone": t_gemm * 1e6,
                              "step with g given (no amax pass)": t_given * 1e6 if t_given else None,
                              "hot-cache step (one weight copy, resident in the Infinity Cache)":
                                  t_hot * 1e6 if t_hot else None,
                              "tflops with g given": flops / t_given / 1e12 if t_given else None,
                              "step with GDN gates fused": t_gated * 1e6 if t_gated else None,
                              "step with bf16 Y" + (" and GDN gates" if gate_p is not None else ""):
                                  t_bf16 * 1e6 if t_bf16 else None,
                              "step with RHT (both operands transformed, g computed)":
                                  t_rht * 1e6 if t_rht else None,
                              "quantize with RHT alone (g computed)": t_qrht * 1e6 if t_qrht else None,
                              "kv fp8 quantize 4096x1024 bf16 (scale calibrated)": t_kv * 1e6 if t_kv else None,
                              "kv fp8 quantize (scale given)": t_kvg * 1e6 if t_kvg else None,
                              "kv fp8 GB/s (scale given; read x, write bytes)":
                                  4096 * 1024 * 3 / t_kvg / 1e9 if t_kvg else None,
                              "backward step (dX and dW; dY both ways in one pass, W and X transposed, packed)":
                                  t_bwd * 1e6 if t_bwd else None,
                              "backward tflops": 2.0 * flops / t_bwd / 1e12 if t_bwd else None,
                              "quantize_t alone (X^T, g computed)": t_qt * 1e6 if t_qt else None,
                              "weight re-quantization per step (W quantized and packed)": t_rq * 1e6 if t_rq else None,
                              "W and W^T packed per step (quantize, quantize_t, two packs)":
                                  t_rq2 * 1e6 if t_rq2 else None,
                              "W and W^T packed per step (nvfp4_pack_weights_train, one read)":
                                  t_rqf * 1e6 if t_rqf else None,
                              "quantize_t GB/s (read x once, write codes and scales)":
                                  (x_in_bytes + x_q_bytes) / t_qt / 1e9 if t_qt else None},
        "step_gbs": (x_in_bytes + w_bytes + x_q_bytes + M * N * 4) / t_step / 1e9,
        "shader_clock_mhz_right_after_step": clock,
        "parity": {"codes_scales_bit_exact": codes_ok, "gemm_within_1e-5": bool(y_ok), "worst_ratio": worst,
                   "g_given_codes_scales_bit_exact": given_ok,
                   "gdn_gates_within_bound": gated_ok, "gdn_gates_worst_ratio": gated_worst,
                   "backward": bwd_parity, "rht": rht_parity, "kv_fp8": kv_parity, "bf16_y_is_rne_of_f32_y": bf16_ok,
                   "rows_checked": int(len(rows)), "cols_checked": int(len(cols))},
    }
    print(json.dumps(out), flush=True)


def observed_gfx_clock(run, cycles=200_000, rounds=20):
    """The shader clock right after the step has run: after each of `rounds` replays of `run`, a
    one-wave spin of `cycles` shader-clock cycles (torch.cuda._sleep, which counts the core clock)
    is timed with events on the same stream; its cycles over its time is the clock, in MHz, before
    the power management can react to the lighter load.  Untimed, after the timed region."""
    import torch
    if not hasattr(torch.cuda, "_sleep"):
        return {"error": "torch.cuda._sleep not available"}
    cur = torch.cuda.current_stream()
    mhz = []
    for _ in range(rounds):
        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        torch.cuda._sleep(cycles)
        e1.record(cur)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        if ms > 0:
            mhz.append(cycles / (ms * 1e3))
    if not mhz:
        return {"error": "no timing"}
    mhz.sort()
    return {"median": mhz[len(mhz) // 2], "min": mhz[0], "max": mhz[-1], "spins": len(mhz), "cycles": cycles}


def cpu_baseline(wl, ref, budget_s=12.0):
    """The oracle as it stands, on host cores: quantize X, dequantize, FP64 GEMM against the weights
    dequantized once beforehand (they are static, like the packed blob).  Bounded sample: whole steps
    for the small workloads; for the large ones a block of X rows against (for wide weights) a spread
    of weight rows, quantized with the whole tensors' global scales; reported in TFLOP/s of that sample."""
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    host_cores = len(os.sched_getaffinity(0))
    M, K, N = wl.M, wl.K, wl.N
    m_s = M if M <= 64 else 64
    n_cap = 2048                      # weight rows dequantized for the sample (all of them up to this)
    parts = []
    for w in wl.w:
        rows_w = w.shape[0]
        take = rows_w if N <= n_cap else max(1, rows_w * n_cap // N)
        sel = np.linspace(0, rows_w - 1, take).round().astype(np.int64) if take < rows_w else np.arange(rows_w)
        gw = ref.global_scale(np.float32(np.abs(w).max()))
        parts.append(ref.dequantize(ref.quantize(w[sel], g_mode="given", g=gw)))
    wh = np.concatenate(parts)
    n_s = wh.shape[0]
    gx = ref.global_scale(np.float32(np.abs(wl.x).max()))
    xs = wl.x[:m_s]
    n, t0 = 0, time.time()
    while True:
        xq = ref.quantize(xs, g_mode="given", g=gx)
        ref.gemm_dequantized(ref.dequantize(xq), wh)
        n += 1
        if time.time() - t0 > budget_s or n >= 1000:
            break
    dt = (time.time() - t0) / n
    return {"value": 2.0 * m_s * n_s * K / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle", "host_cores_available": host_cores, "blas_threads": int(blas_threads),
            "sample": f"{n} oracle steps of X[{m_s} x {K}] (quantize with the tensor's g, dequantize, FP64 GEMM "
                      f"with |terms|) against {n_s} of the {N} weight rows dequantized once; {dt * 1e3:.1f} ms "
                      f"per step; quantize on 1 thread, GEMM on {blas_threads} BLAS threads of {host_cores} "
                      f"host cores"}


if __name__ == "__main__":
    main()
