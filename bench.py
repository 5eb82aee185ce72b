"""Throughput of NVFP4 GPTQ + Schur Replay layer quantization on one MI355X.

One step = the whole per-layer path on inputs already resident in HBM:
  H = X^T X (bf16 MFMA)  ->  U with (H + lam I)^-1 = U^T U  ->  global scale
  ->  GPTQ sweep with Schur Replay (16 candidates per block, lazy batches of
  128 columns with an fp32 MFMA trailing update)  ->  weighted error
  tr(dW H dW^T)  ->  dequantized export.
Workload: attention-projection-shaped layer, W bf16 4096 x 4096, X bf16
262,144 tokens x 4096 (synthetic, seeded).  Metric: quantized weights per
second (Mparam/s) including the Hessian.

Prints one JSON line (see the keys below).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, K_IN, N_TOK, N_CAND = 4096, 4096, 262144, 16
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
WORKLOAD = ("attention-projection layer W 4096x4096 bf16, X 262144x4096 bf16, 16 scale candidates per "
            "16-block, lazy batch 128")

# HBM traffic of the Hessian call, from rocprofv3 FETCH_SIZE / WRITE_SIZE passes
# over this script, scaled by what the same counters read for the untimed
# device copy of CAL_COPY_BYTES that main() runs after the timed steps.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hessian_accumulate_attn_proj_4096x4096_n262144_hbm_traffic.json")
HESSIAN_SOURCES = [os.path.join(ROOT, "post_nvfp4_weight_amd", "csrc", f) for f in ("syrk.hip", "common.h")]
CAL_COPY_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline():
    """Oracle (NumPy fp64) on a bounded sample of the same workload, scaled to Mparam/s.

    Sample: Hessian over 8,192 of the 262,144 tokens (time scaled x32), the full
    4096 x 4096 factorization, the sweep + weighted error of 16 of the 4096 rows
    (time scaled x256).  Layer time = sum of the scaled stage times.
    """
    import numpy as np
    import synth
    from oracle import codec, gptq
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    W = synth.weights("attn_proj", M, K_IN, 0.02, outlier_frac=0.001)
    n_s = 8192
    X = synth.activations("attn_proj", n_s, K_IN, massive=8)
    t0 = time.perf_counter()
    H_s = gptq.hessian(X)
    t_h = (time.perf_counter() - t0) * (N_TOK / n_s)
    t0 = time.perf_counter()
    U, lam = gptq.hinv_factor(H_s)
    t_f = time.perf_counter() - t0
    rows = 16
    g = codec.global_scale(W)
    t0 = time.perf_counter()
    res = gptq.sweep(W[:rows], U, g, N_CAND)
    deq = codec.dequantize(codec.pack_codes(res["codes"]), res["scales"], g)
    gptq.weighted_error(W[:rows], deq, H_s)
    t_s = (time.perf_counter() - t0) * (M / rows)
    total = t_h + t_f + t_s
    return {"value": M * K_IN / total / 1e6, "unit": "Mparam/s", "cores": cores, "kind": "oracle",
            "sample": f"hessian on {n_s} of {N_TOK} tokens (x{N_TOK // n_s}), full {K_IN}x{K_IN} factor, "
                      f"sweep+error on {rows} of {M} rows (x{M // rows}); stage seconds "
                      f"H={t_h:.1f} factor={t_f:.1f} sweep={t_s:.1f}"}


def hessian_source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in HESSIAN_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """Measured HBM bytes per Hessian call, or None if absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != hessian_source_digest() or d.get("workload") != WORKLOAD:
        return None
    return d.get("hbm_bytes_per_call")


def summarize_pmc(fetch_csv, write_csv):
    """Per-call HBM bytes of hessian_accumulate from two rocprofv3 --pmc CSVs -> TRAFFIC_FILE."""
    import csv

    def per_dispatch(path, counter):
        d = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    e = d.setdefault(r["Dispatch_Id"], [r["Kernel_Name"], 0.0])
                    e[1] += float(r["Counter_Value"])
        return list(d.values())

    out = {"commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmcf -o fetch -- "
                        "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmcw -o write -- "
                        "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline",
                        "python3 bench.py --summarize-pmc gpurun_out/pmcf/fetch_counter_collection.csv "
                        "gpurun_out/pmcw/write_counter_collection.csv"],
           "kernel": "hessian_accumulate (syrk_main_kernel + syrk_single_kernel + syrk_reduce_kernel)",
           "workload": WORKLOAD, "source_digest": hessian_source_digest(), "unit": "bytes per call",
           "calibration_copy_bytes": CAL_COPY_BYTES}
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = per_dispatch(path, name)
        calls = sum(1 for n, _ in rows if "syrk_main_kernel" in n)
        kib = sum(v for n, v in rows if "syrk_" in n) / max(1, calls)
        copies = [v for n, v in rows if "bitwise_not" in n]
        if not calls or not copies:
            raise SystemExit(f"{path}: no Hessian or calibration-copy dispatches with {name}")
        factor = (CAL_COPY_BYTES / 1024.0) / max(copies)
        out[name] = {"kib_per_call": round(kib, 1), "copy_kib": round(max(copies), 1),
                     "scale": round(factor, 4), "bytes_per_call": round(kib * 1024.0 * factor)}
        total += kib * 1024.0 * factor
    out["hbm_bytes_per_call"] = round(total)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def streamed(nvq, Xh, dev):
    """Hessian of the benchmarked layer's X (2 GiB bf16) from host memory, in
    32768-token chunks, PCIe copies overlapped with the accumulation; against
    X resident in HBM."""
    import torch
    chunk = 32768
    Xd = Xh.to(dev)
    H = torch.zeros(K_IN, K_IN, dtype=torch.float32, device=dev)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e3

    ms_dev = timed(lambda: nvq.hessian_accumulate(Xd, H))
    del Xd
    Xpage = Xh.clone()   # pageable copy; Xh is pinned
    ms_pin = timed(lambda: nvq.hessian_accumulate_host(Xh, H, chunk=chunk))
    ms_page = timed(lambda: nvq.hessian_accumulate_host(Xpage, H, chunk=chunk))
    gb = Xh.numel() * 2 / 1e9
    print(json.dumps({"streamed_hessian": WORKLOAD, "chunk_tokens": chunk, "x_gb": round(gb, 3),
                      "ms_x_in_hbm": round(ms_dev, 3), "ms_x_pinned_host": round(ms_pin, 3),
                      "ms_x_pageable_host": round(ms_page, 3),
                      "host_to_device_gbs_pinned": round(gb / ms_pin * 1e3, 1),
                      "host_to_device_gbs_pageable": round(gb / ms_page * 1e3, 1),
                      "device_bytes_streamed": int(nvq.lib.hessian_host_workspace_size(chunk, K_IN, 1)),
                      "data": "synthetic"}))


def consumer_bench(nvq, Wd, Xd):
    """nvfp4_gemm (Y = X dequant(W)^T) on the benchmarked layer after quantization,
    for several token counts, against torch's bf16 GEMM on the dequantized weights."""
    import torch
    res = nvq.quantize_layer(Wd, Xd, n_cand=N_CAND)
    codes, scales, g = res["codes"], res["scales"], res["g"]
    Wdq = nvq.nvfp4_dequantize(codes, scales, g, torch.bfloat16)
    out = []
    for T in (1, 16, 32, 256, 2048, 8192):
        X = Xd[:T].contiguous()

        def timed(fn, reps=20):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ms = timed(lambda: nvq.nvfp4_gemm(X, codes, scales, g))
        ms_bf16 = timed(lambda: torch.matmul(X, Wdq.t()))
        flops = 2.0 * T * M * K_IN
        wbytes = M * K_IN * 0.5625
        out.append({"tokens": T, "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                    "weight_gbs": round(wbytes / ms / 1e6, 1), "ms_torch_bf16_dense": round(ms_bf16, 4)})
    print(json.dumps({"consumer": "nvfp4 weight-only GEMM, " + WORKLOAD, "results": out, "data": "synthetic"}))


def ablation(nvq, Wd, Xd):
    """Total weighted error sum_r dW_r H dW_r^T of the benchmarked layer under
    each scale-selection configuration, all on the GPU."""
    res = nvq.quantize_layer(Wd, Xd, n_cand=N_CAND)
    U, H, g = res["U"], res["H"], res["g"]
    E = {
        "rtn_absmax": nvq.gptq_nvfp4_quantize(Wd, None, H, g, 1, nvq.FLAG_RTN)["row_err"],
        "gptq_absmax": nvq.gptq_nvfp4_quantize(Wd, U, H, g, 1)["row_err"],
        "gptq_block_independent": nvq.gptq_nvfp4_quantize(Wd, U, H, g, N_CAND, nvq.FLAG_INDEP)["row_err"],
        "gptq_schur_replay": res["row_err"],
    }
    E = {k: float(v.double().sum()) for k, v in E.items()}
    ref = E["gptq_schur_replay"]
    print(json.dumps({"ablation": "block-scale selection", "workload": WORKLOAD, "n_cand": N_CAND,
                      "E_total": E, "E_relative_to_schur_replay": {k: round(v / ref, 4) for k, v in E.items()},
                      "data": "synthetic"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the Hessian's measured HBM traffic from two rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--streamed", action="store_true",
                    help="instead of the layer step, time the Hessian with X in host memory (pinned and "
                         "pageable), streamed to the device in chunks, against X resident in HBM")
    ap.add_argument("--consumer", action="store_true",
                    help="instead of the layer step, time the NVFP4 weight-only GEMM on the quantized layer")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of timing, print the layer's total weighted error under four scale-selection "
                         "configurations (RTN absmax, GPTQ absmax, GPTQ block-independent, GPTQ Schur Replay)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the per-layer path is a single-GPU workload here "
              "(several GPUs would split the tokens of the Hessian, all-reduce H, and split the rows of W, "
              "which need no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import post_nvfp4_weight_amd as nvq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs")
    W = synth.weights("attn_proj", M, K_IN, 0.02, outlier_frac=0.001)
    Wd = synth.to_bf16_tensor(W).to(dev)
    Xh = torch.empty(N_TOK, K_IN, dtype=torch.bfloat16, pin_memory=True)
    synth.activations("attn_proj", N_TOK, K_IN, massive=8, out=Xh)
    if args.streamed:
        streamed(nvq, Xh, dev)
        return
    t0 = time.perf_counter()
    Xd = Xh.to(dev, non_blocking=True)
    torch.cuda.synchronize()
    h2d_s = time.perf_counter() - t0
    del Xh
    log(f"inputs resident (H2D {h2d_s:.3f} s)")
    if args.ablation:
        ablation(nvq, Wd, Xd)
        return
    if args.consumer:
        consumer_bench(nvq, Wd, Xd)
        return

    lib = nvq.lib
    stream = nvq._stream
    P = nvq._ptr
    H = torch.empty(K_IN, K_IN, dtype=torch.float32, device=dev)
    U = torch.empty_like(H)
    lam = torch.empty(1, dtype=torch.float32, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    codes = torch.empty(M, K_IN // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(M, K_IN // 16, dtype=torch.uint8, device=dev)
    row_err = torch.empty(M, dtype=torch.float32, device=dev)
    row_loss = torch.empty(M, dtype=torch.float32, device=dev)
    deq = torch.empty(M, K_IN, dtype=torch.bfloat16, device=dev)
    ws_h_n = lib.hessian_workspace_size(N_TOK, K_IN, nvq.NVQ_DTYPE_BF16)
    ws_f_n = lib.factor_hinv_workspace_size(K_IN)
    ws_g_n = lib.nvfp4_global_scale_workspace_size(M, K_IN)
    ws_q_n = lib.gptq_nvfp4_workspace_size(M, K_IN, 0)
    ws = {n: torch.empty(max(1, b), dtype=torch.uint8, device=dev)
          for n, b in [("h", ws_h_n), ("f", ws_f_n), ("g", ws_g_n), ("q", ws_q_n)]}

    def chk(name, rc):
        if rc != 0:
            raise RuntimeError(f"{name}: {lib.nvq_last_error().decode()}")

    stages = ["hessian", "factor", "gscale", "quantize", "dequant"]

    def step(ev=None):
        s = stream()
        H.zero_()
        if ev: ev[0].record()
        chk("hessian", lib.hessian_accumulate(P(Xd), nvq.NVQ_DTYPE_BF16, N_TOK, K_IN, K_IN, P(H), P(ws["h"]),
                                              ws_h_n, s))
        if ev: ev[1].record()
        chk("factor", lib.factor_hinv(P(H), K_IN, 0.01, P(U), P(lam), P(info), P(ws["f"]), ws_f_n, s))
        if ev: ev[2].record()
        chk("gscale", lib.nvfp4_global_scale(P(Wd), nvq.NVQ_DTYPE_BF16, M, K_IN, K_IN, P(g), P(ws["g"]), ws_g_n, s))
        if ev: ev[3].record()
        chk("quantize", lib.gptq_nvfp4_quantize(P(Wd), nvq.NVQ_DTYPE_BF16, M, K_IN, K_IN, P(U), P(H), P(g), N_CAND,
                                                0, P(codes), P(scales), P(row_err), P(row_loss), P(ws["q"]),
                                                ws_q_n, s))
        if ev: ev[4].record()
        chk("dequant", lib.nvfp4_dequantize(P(codes), P(scales), P(g), M, K_IN, P(deq), nvq.NVQ_DTYPE_BF16, s))
        if ev: ev[5].record()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(info.item()) == 0, "factorization failed"

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_stage = {st: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, st in enumerate(stages)}
    ms_per_step = elapsed * 1e3 / args.steps
    value = M * K_IN / (ms_per_step / 1e3) / 1e6

    # The Hessian contraction dominates: algorithmic flops n*k*(k+1) per call.
    t_h = per_stage["hessian"] / 1e3
    flops = N_TOK * K_IN * (K_IN + 1)
    achieved = flops / t_h / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": load_traffic(),
                "kernel": "hessian_accumulate", "ms_per_call": round(per_stage["hessian"], 4)}

    # Standalone RTN encode + pack of the same W (the no-update codec path).
    rtn_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rtn_ev[0].record()
    reps = 10
    for _ in range(reps):
        chk("rtn", lib.gptq_nvfp4_quantize(P(Wd), nvq.NVQ_DTYPE_BF16, M, K_IN, K_IN, None, None, P(g), 1,
                                           nvq.FLAG_RTN | nvq.FLAG_NO_ERR, P(codes), P(scales), None, None,
                                           P(ws["q"]), ws_q_n, stream()))
    rtn_ev[1].record()
    torch.cuda.synchronize()
    rtn_ms = rtn_ev[0].elapsed_time(rtn_ev[1]) / reps

    # Untimed streaming kernel of known size (reads and writes CAL_COPY_BYTES):
    # the calibration dispatch for rocprofv3's HBM byte counters (see summarize_pmc).
    cal = torch.bitwise_not(Xd.view(torch.int32).reshape(-1)[:CAL_COPY_BYTES // 4])
    torch.cuda.synchronize()
    del cal

    out = {
        "metric": "quantized weights/sec (Mparam/s) per layer incl. Hessian",
        "value": round(value, 1), "unit": "Mparam/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16-mfma/fp32", "data": "synthetic",
        "config": {"workload": WORKLOAD,
                   "d_out": M, "d_in": K_IN, "tokens": N_TOK, "n_cand": N_CAND},
        "roofline": roofline,
        "stages_ms": {k: round(v, 3) for k, v in per_stage.items()},
        "rtn_encode_ms": round(rtn_ms, 4),
        "h2d_inputs_s": round(h2d_s, 3),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
