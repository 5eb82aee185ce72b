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

import numpy as np

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
# Counter-measured bytes of the streaming kernels (sweep batch, RTN encode, dequantize), same passes.
STREAM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sweep_rtn_dequant_hbm_traffic.json")
STREAM_SOURCES = [os.path.join(ROOT, "post_nvfp4_weight_amd", "csrc", f) for f in ("sweep.hip", "common.h")]


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
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": M * K_IN / total / 1e6, "unit": "Mparam/s", "cores": cores, "cpu_model": cpu_model,
            "kind": "oracle",
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


def stream_source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in STREAM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_stream_traffic(key):
    """Measured HBM bytes per launch of a streaming kernel, or None if absent or taken on other sources."""
    try:
        with open(STREAM_TRAFFIC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != stream_source_digest():
        return None
    return d.get("kernels", {}).get(key, {}).get("hbm_bytes")


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
                    e = d.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
                    e[1] += float(r["Counter_Value"])
        return [d[i] for i in sorted(d)]

    def hessian_calls(rows):
        # A call is a run of consecutive syrk_ dispatches (its launches and
        # reductions); calls are separated by other kernels.
        calls, prev = 0, False
        for n, _ in rows:
            cur = "syrk_" in n
            calls += cur and not prev
            prev = cur
        return calls

    out = {"commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmcf -o fetch -- "
                        "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmcw -o write -- "
                        "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline",
                        "python3 bench.py --summarize-pmc gpurun_out/pmcf/fetch_counter_collection.csv "
                        "gpurun_out/pmcw/write_counter_collection.csv"],
           "kernel": "hessian_accumulate (at k = 4096 syrk_k4_kernel twice, then syrk_reduce_k4_kernel twice; "
                     "otherwise syrk_main_kernel, syrk_single_kernel and syrk_reduce_kernel)",
           "workload": WORKLOAD, "source_digest": hessian_source_digest(), "unit": "bytes per call",
           "calibration_copy_bytes": CAL_COPY_BYTES}
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = per_dispatch(path, name)
        calls = hessian_calls(rows)
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
    # The streaming kernels: per-launch bytes of the sweep (one 128-column
    # batch of the benchmarked layer) and of the pack kernels on the 70B-class
    # W (the largest launches of rtn_kernel and dequant_kernel in the run).
    kinds = {"sweep_batch_kernel": "sweep_batch_kernel<16, float, false, true> (Cholesky-factor form; one "
                                   "128-column batch, 4096 rows)",
             "rtn_kernel": f"rtn_kernel<1> (W {PACK_M}x{PACK_K} bf16, one candidate)",
             "dequant_kernel": f"dequant_kernel<1> (W {PACK_M}x{PACK_K}, bf16 out)"}
    stream = {"commands": out["commands"], "workload": WORKLOAD, "unit": "bytes per launch",
              "source_digest": stream_source_digest(),
              "calibration_copy_bytes": CAL_COPY_BYTES, "kernels": {}}
    for key, desc in kinds.items():
        ent = {"kernel": desc}
        for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
            rows = per_dispatch(path, name)
            vals = [v for n, v in rows if key in n]
            copies = [v for n, v in rows if "bitwise_not" in n]
            factor = (CAL_COPY_BYTES / 1024.0) / max(copies)
            kib = (sum(vals) / len(vals)) if key == "sweep_batch_kernel" else max(vals)
            ent[name] = round(kib * 1024.0 * factor)
        ent["hbm_bytes"] = ent["FETCH_SIZE"] + ent["WRITE_SIZE"]
        if key != "sweep_batch_kernel":
            ent["algorithmic_bytes"] = int(PACK_M * PACK_K * 2.5625)
        stream["kernels"][key] = ent
    with open(STREAM_TRAFFIC_FILE, "w") as fh:
        json.dump(stream, fh, indent=1)
    print(json.dumps(stream))


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


WORKLOADS = {
    "attn_proj": "the attention-projection layer (headline)",
    "mlp": "MLP pair of an 8B-class block: gate+up 28672x4096 (fp32 sweep) over X 131072x4096, down "
           "4096x14336 (fp64 sweep) over its own SiLU(gate)*up activations",
    "down_proj_70b": "70B-class down projection: W 8192x28672 bf16, X 65536x28672 bf16 60% zeros (fp64 sweep)",
    "moe": "MoE layer: 256 experts, gate+up 2048x4096 each, 262144 tokens routed top-8 (Zipf 1.1)",
}


class LayerTimer:
    """Times the per-layer C-ABI calls (zero H, Hessian, factor_chol, global scale, quantize on V,
    dequantize) on device-resident inputs with events on the library's stream; buffers allocated once,
    outside timing."""

    STAGES = ["hessian", "factor", "gscale", "quantize", "dequant"]

    def __init__(self, nvq, Wd, Xd, flags, n_cand=N_CAND):
        import torch
        flags |= nvq.FLAG_CHOL_FACTOR   # factor_chol: V, no triangular inverse
        self.nvq, self.lib, self.P, self.flags, self.n_cand = nvq, nvq.lib, nvq._ptr, flags, n_cand
        self.Wd, self.Xd = Wd, Xd
        self.m, self.k = Wd.shape
        self.n = Xd.shape[0]
        dev = Wd.device
        m, k, n = self.m, self.k, self.n
        self.H = torch.empty(k, k, dtype=torch.float32, device=dev)
        self.U = torch.empty_like(self.H)
        self.lam = torch.empty(1, dtype=torch.float32, device=dev)
        self.info = torch.empty(1, dtype=torch.int32, device=dev)
        self.g = torch.empty(1, dtype=torch.float32, device=dev)
        self.codes = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(m, k // 16, dtype=torch.uint8, device=dev)
        self.row_err = torch.empty(m, dtype=torch.float32, device=dev)
        self.row_loss = torch.empty(m, dtype=torch.float32, device=dev)
        self.deq = torch.empty(m, k, dtype=torch.bfloat16, device=dev)
        lib = self.lib
        self.ws_n = {"h": lib.hessian_workspace_size(n, k, nvq.NVQ_DTYPE_BF16),
                     "f": lib.factor_chol_workspace_size(k),
                     "g": lib.nvfp4_global_scale_workspace_size(m, k),
                     "q": lib.gptq_nvfp4_workspace_size(m, k, flags)}
        self.ws = {a: torch.empty(max(1, b), dtype=torch.uint8, device=dev) for a, b in self.ws_n.items()}

    def _chk(self, name, rc):
        if rc != 0:
            raise RuntimeError(f"{name}: {self.lib.nvq_last_error().decode()}")

    def step(self, ev=None):
        lib, P, nvq, ws, wn = self.lib, self.P, self.nvq, self.ws, self.ws_n
        s = nvq._stream()
        m, k, n = self.m, self.k, self.n
        self.H.zero_()
        if ev: ev[0].record()
        self._chk("hessian", lib.hessian_accumulate(P(self.Xd), nvq.NVQ_DTYPE_BF16, n, k, self.Xd.stride(0),
                                                    P(self.H), P(ws["h"]), wn["h"], s))
        if ev: ev[1].record()
        self._chk("factor", lib.factor_chol(P(self.H), k, 0.01, P(self.U), P(self.lam), P(self.info), P(ws["f"]),
                                            wn["f"], s))
        if ev: ev[2].record()
        self._chk("gscale", lib.nvfp4_global_scale(P(self.Wd), nvq.NVQ_DTYPE_BF16, m, k, k, P(self.g), P(ws["g"]),
                                                   wn["g"], s))
        if ev: ev[3].record()
        self._chk("quantize", lib.gptq_nvfp4_quantize(P(self.Wd), nvq.NVQ_DTYPE_BF16, m, k, k, P(self.U), P(self.H),
                                                      P(self.g), self.n_cand, self.flags, P(self.codes),
                                                      P(self.scales), P(self.row_err), P(self.row_loss),
                                                      P(ws["q"]), wn["q"], s))
        if ev: ev[4].record()
        self._chk("dequant", lib.nvfp4_dequantize(P(self.codes), P(self.scales), P(self.g), m, k, P(self.deq),
                                                  nvq.NVQ_DTYPE_BF16, s))
        if ev: ev[5].record()

    def run(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        assert int(self.info.item()) == 0, "factorization failed"
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        per = {st: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, st in enumerate(self.STAGES)}
        return ms, per


PACK_M, PACK_K = 8192, 28672


def pack_roofline(nvq, lib, P, dev, reps=20):
    """RTN encode + pack (one candidate: the absmax scale) and bf16 dequantization of the 70B-class down
    projection's W (8192 x 28672 bf16, synthetic): algorithmic HBM bytes 2.5625 per weight each way
    (2 B of bf16 plus 0.5 B of codes and 1/16 B of scales), over the kernel time from events on the
    library's stream."""
    import torch
    import synth
    m, k = PACK_M, PACK_K
    W = synth.to_bf16_tensor(synth.weights("sparse", m, k, 0.01, outlier_frac=0.0005)).to(dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    codes = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(m, k // 16, dtype=torch.uint8, device=dev)
    out = torch.empty(m, k, dtype=torch.bfloat16, device=dev)
    gws_n = lib.nvfp4_global_scale_workspace_size(m, k)
    gws = torch.empty(max(1, gws_n), dtype=torch.uint8, device=dev)
    qws_n = lib.gptq_nvfp4_workspace_size(m, k, nvq.FLAG_RTN)
    qws = torch.empty(max(1, qws_n), dtype=torch.uint8, device=dev)
    s = nvq._stream()
    assert lib.nvfp4_global_scale(P(W), nvq.NVQ_DTYPE_BF16, m, k, k, P(g), P(gws), gws_n, s) == 0

    def enc():
        assert lib.gptq_nvfp4_quantize(P(W), nvq.NVQ_DTYPE_BF16, m, k, k, None, None, P(g), 1,
                                       nvq.FLAG_RTN | nvq.FLAG_NO_ERR, P(codes), P(scales), None, None, P(qws),
                                       qws_n, s) == 0

    def dec():
        assert lib.nvfp4_dequantize(P(codes), P(scales), P(g), m, k, P(out), nvq.NVQ_DTYPE_BF16, s) == 0

    res = {}
    for name, fn in (("rtn_encode", enc), ("dequant", dec)):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
    nbytes = m * k * 2.5625
    ach = {n: nbytes / (ms / 1e3) / 1e9 for n, ms in res.items()}
    worst = min(ach, key=ach.get)
    del W, codes, scales, out, qws
    torch.cuda.empty_cache()
    return {"bound": "hbm", "achieved": round(ach[worst], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach[worst] / PEAK_HBM_GBS, 4),
            "traffic": load_stream_traffic("rtn_kernel" if worst == "rtn_encode" else "dequant_kernel"),
            "kernel": f"{worst} (the slower of rtn_encode and dequant)", "workload": f"W {m}x{k} bf16",
            "bytes_per_call": int(nbytes),
            "ms_per_call": {n: round(v, 4) for n, v in res.items()},
            "gbs": {n: round(v, 1) for n, v in ach.items()}}


def hessian_roofline(n, k, ms_h):
    achieved = n * k * (k + 1) / (ms_h / 1e3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": "hessian_accumulate",
            "ms_per_call": round(ms_h, 4)}


def workload_line(name, steps, warmup):
    """One JSON line for a workload other than the headline: Mparam/s per layer including the Hessian."""
    import torch
    import post_nvfp4_weight_amd as nvq
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    if name == "mlp":
        n, d, f = 131072, 4096, 14336
        log("generating inputs")
        Xh = torch.empty(n, d, dtype=torch.bfloat16, pin_memory=True)
        synth.activations("mlp", n, d, out=Xh)
        Wg, Wu, Wdn = synth.mlp_block_weights(d, f)
        Xd = Xh.to(dev)
        del Xh
        Xdown = synth.mlp_down_activations(Xd, Wg, Wu)
        Wgu = synth.to_bf16_tensor(np.concatenate([Wg, Wu])).to(dev)
        layers = [("gate_up", Wgu, Xd, 0), ("down", synth.to_bf16_tensor(Wdn).to(dev), Xdown, nvq.FLAG_FP64)]
    elif name == "down_proj_70b":
        m, k, n = 8192, 28672, 65536
        log("generating inputs")
        Xh = torch.empty(n, k, dtype=torch.bfloat16, pin_memory=True)
        synth.activations("sparse", n, k, kind="sparse", out=Xh)
        W = synth.weights("sparse", m, k, 0.01, outlier_frac=0.0005)
        layers = [("down_proj", synth.to_bf16_tensor(W).to(dev), Xh.to(dev), nvq.FLAG_FP64)]
        del Xh
    else:
        raise SystemExit(f"unknown workload {name}")
    out = {"metric": "quantized weights/sec (Mparam/s) per layer incl. Hessian", "unit": "Mparam/s",
           "n_gpus": 1, "steps": steps, "warmup": warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16-mfma/fp32", "data": "synthetic",
           "config": {"workload": WORKLOADS[name], "n_cand": N_CAND, "factor": "cholesky"}, "layers": {}}
    tot_ms, tot_params = 0.0, 0
    for lname, Wd, Xd, flags in layers:
        log(f"{lname}: warmup {warmup}, timing {steps} steps")
        lt = LayerTimer(nvq, Wd, Xd, flags)
        ms, per = lt.run(steps, warmup)
        params = lt.m * lt.k
        tot_ms += ms
        tot_params += params
        out["layers"][lname] = {
            "d_out": lt.m, "d_in": lt.k, "tokens": lt.n, "sweep_precision": "fp64" if flags & nvq.FLAG_FP64 else "fp32",
            "ms_per_step": round(ms, 3), "mparam_s": round(params / (ms / 1e3) / 1e6, 1),
            "stages_ms": {a: round(b, 3) for a, b in per.items()},
            "roofline": hessian_roofline(lt.n, lt.k, per["hessian"])}
        del lt
        torch.cuda.empty_cache()
    out["ms_per_step"] = round(tot_ms, 3)
    out["value"] = round(tot_params / (tot_ms / 1e3) / 1e6, 1)
    print(json.dumps(out), flush=True)


def moe_line(steps, warmup):
    """The MoE layer: grouped Hessians over routed tokens, batched Cholesky factors (factor_chol_batched,
    no triangular inverse), per-expert global scales, batched quantization (fp32 sweep on V) and
    dequantization of all 256 experts; Mparam/s over all experts."""
    import torch
    import post_nvfp4_weight_amd as nvq
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    E, n, k, m, top_k = 256, 262144, 4096, 2048, 8
    log("generating inputs")
    Xh = torch.empty(n, k, dtype=torch.bfloat16, pin_memory=True)
    synth.activations("moe", n, k, out=Xh)
    idx, off = synth.moe_routing(n, E, top_k)
    Xd = Xh.to(dev)
    del Xh
    idx_d = torch.from_numpy(idx).to(dev)
    Wt = torch.empty(E, m, k, dtype=torch.bfloat16, device=dev)
    for e in range(E):
        Wt[e] = synth.to_bf16_tensor(synth.moe_expert_weights(e, m, k)).to(dev)
    lib, P = nvq.lib, nvq._ptr
    import ctypes
    offp = np.ascontiguousarray(off, dtype=np.int64)
    offc = offp.ctypes.data_as(ctypes.c_void_p)
    H = torch.empty(E, k, k, dtype=torch.float32, device=dev)
    U = torch.empty_like(H)
    lam = torch.empty(E, dtype=torch.float32, device=dev)
    info = torch.empty(E, dtype=torch.int32, device=dev)
    g = torch.empty(E, dtype=torch.float32, device=dev)
    codes = torch.empty(E, m, k // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(E, m, k // 16, dtype=torch.uint8, device=dev)
    row_err = torch.empty(E, m, dtype=torch.float32, device=dev)
    row_loss = torch.empty(E, m, dtype=torch.float32, device=dev)
    deq = torch.empty(E, m, k, dtype=torch.bfloat16, device=dev)
    # factors: 64 experts per pass (64 x 160 MiB); quantization: all 256 in one pass (256 x 68 MiB)
    qflags = nvq.FLAG_CHOL_FACTOR
    wn = {"h": lib.hessian_grouped_workspace_size(offc, E, k, nvq.NVQ_DTYPE_BF16),
          "f": 64 * lib.factor_chol_workspace_size(k), "g": lib.nvfp4_global_scale_workspace_size(m, k),
          "q": E * lib.gptq_nvfp4_workspace_size(m, k, qflags)}
    ws = {a: torch.empty(max(1, b), dtype=torch.uint8, device=dev) for a, b in wn.items()}

    def chk(name, rc):
        if rc != 0:
            raise RuntimeError(f"{name}: {lib.nvq_last_error().decode()}")

    def step(ev=None):
        s = nvq._stream()
        H.zero_()
        if ev: ev[0].record()
        chk("hessian", lib.hessian_accumulate_grouped(P(Xd), nvq.NVQ_DTYPE_BF16, n, k, k, P(idx_d), offc, E, P(H),
                                                      P(ws["h"]), wn["h"], s))
        if ev: ev[1].record()
        chk("factor", lib.factor_chol_batched(P(H), k, E, k * k, 0.01, P(U), k * k, P(lam), P(info), P(ws["f"]),
                                              wn["f"], s))
        if ev: ev[2].record()
        for e in range(E):
            chk("gscale", lib.nvfp4_global_scale(P(Wt[e]), nvq.NVQ_DTYPE_BF16, m, k, k, P(g[e:]), P(ws["g"]),
                                                 wn["g"], s))
        if ev: ev[3].record()
        chk("quantize", lib.gptq_nvfp4_quantize_batched(P(Wt), nvq.NVQ_DTYPE_BF16, E, m, k, k, m * k, P(U), k * k,
                                                        P(H), k * k, P(g), N_CAND, qflags, P(codes), P(scales),
                                                        P(row_err), P(row_loss), P(ws["q"]), wn["q"], s))
        if ev: ev[4].record()
        for e in range(E):
            chk("dequant", lib.nvfp4_dequantize(P(codes[e]), P(scales[e]), P(g[e:]), m, k, P(deq[e]),
                                                nvq.NVQ_DTYPE_BF16, s))
        if ev: ev[5].record()

    log(f"warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    assert bool(torch.all(info == 0)), "factorization failed"
    log(f"timing {steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = {st: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, st in enumerate(LayerTimer.STAGES)}
    counts = np.diff(off)
    flops = float(np.sum(counts.astype(np.float64) * k * (k + 1)))
    ach = flops / (per["hessian"] / 1e3) / 1e12
    out = {"metric": "quantized weights/sec (Mparam/s) per layer incl. Hessian",
           "value": round(E * m * k / (ms / 1e3) / 1e6, 1), "unit": "Mparam/s", "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16-mfma/fp32", "data": "synthetic",
           "config": {"workload": WORKLOADS["moe"], "experts": E, "d_out": m, "d_in": k, "tokens": n,
                      "top_k": top_k, "assignments": int(off[-1]), "tokens_per_expert_min": int(counts.min()),
                      "tokens_per_expert_max": int(counts.max()), "n_cand": N_CAND, "sweep_precision": "fp32"},
           "stages_ms": {a: round(b, 3) for a, b in per.items()},
           "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "kernel": "hessian_accumulate_grouped", "ms_per_call": round(per["hessian"], 4)}}
    print(json.dumps(out), flush=True)


def device_peaks():
    """Micro-benchmarked device peaks from libnvq_peaks.so, printed as one JSON line: the bf16 and fp32
    MFMA issue rates and the fp32 FMA rate (register operands only, 4 workgroups of 256 per CU, each
    launch about 30 ms at the nominal peak; the third of three launches, after the clock has settled),
    and HBM bandwidth of a 16-byte-vector copy of 1 GiB (read + write bytes over its time; the best of 1, 4
    or 8 vectors in flight per thread and 1024 to 16384 workgroups, with torch's copy beside it)."""
    import ctypes
    import torch
    here = os.path.dirname(os.path.abspath(__file__))
    lib = ctypes.CDLL(os.path.join(here, "post_nvfp4_weight_amd", "libnvq_peaks.so"))
    lib.nvq_peak_compute.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.nvq_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    grid = 1024
    out = torch.empty(grid * 256, dtype=torch.float32, device=dev)

    def timed(fn, reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ms = []
        for _ in range(3):
            ev[0].record()
            for _ in range(reps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]) / reps)
        return ms[-1]

    def chk(rc):
        if rc != 0:
            raise RuntimeError(f"peak kernel launch failed: hipError {rc}")

    # (name, kind, flops per iteration of the whole grid, iterations, nominal TFLOP/s)
    kinds = [("bf16_mfma", 0, grid * 4 * 4 * 32768, 131072, PEAK_BF16_TFLOPS),
             ("fp32_mfma", 1, grid * 4 * 4 * 4096, 65536, 157.3),
             ("fp32_fma_nonpacked", 2, grid * 256 * 16 * 2, 262144, 78.6)]
    res = {}
    for name, kind, fpi, iters, nominal in kinds:
        ms = timed(lambda: chk(lib.nvq_peak_compute(kind, grid, iters, ctypes.c_void_p(out.data_ptr()), s)), 1)
        tf = fpi * iters / (ms / 1e3) / 1e12
        res[name] = {"tflops": round(tf, 1), "nominal": nominal, "frac_of_nominal": round(tf / nominal, 4),
                     "implied_clock_ghz": round(2.4 * tf / nominal, 3), "ms": round(ms, 3)}
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    best = None
    sweep = {}
    for unroll in (1, 4, 8):
        for cgrid in (1024, 2048, 4096, 8192, 16384):
            ms = timed(lambda: chk(lib.nvq_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                                     nbytes, cgrid, unroll, s)), 10)
            sweep[f"u{unroll}_g{cgrid}"] = round(2 * nbytes / (ms / 1e3) / 1e9, 1)
            if best is None or ms < best[0]:
                best = (ms, unroll, cgrid)
    ms, unroll, cgrid = best
    gbs = 2 * nbytes / (ms / 1e3) / 1e9
    res["hbm_copy"] = {"gbs": round(gbs, 1), "nominal": PEAK_HBM_GBS, "frac_of_nominal": round(gbs / PEAK_HBM_GBS, 4),
                       "bytes_per_copy": 2 * nbytes, "ms": round(ms, 4), "unroll": unroll, "grid": cgrid,
                       "sweep_gbs": sweep}
    ms = timed(lambda: dst.copy_(src), 10)
    res["torch_copy_gbs"] = round(2 * nbytes / (ms / 1e3) / 1e9, 1)
    print(json.dumps({"device_peaks": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="attn_proj", choices=sorted(WORKLOADS),
                    help="attn_proj (default) is the headline line; the others print one line each for the "
                         "larger layer shapes (their own default steps: 3, warmup 1)")
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
    ap.add_argument("--peaks", action="store_true",
                    help="instead of the layer step, micro-benchmark the device's MFMA, FMA and HBM copy peaks")
    args = ap.parse_args()
    if args.peaks:
        device_peaks()
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the per-layer path is a single-GPU workload here "
              "(several GPUs would split the tokens of the Hessian, all-reduce H, and split the rows of W, "
              "which need no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload != "attn_proj":
        steps = args.steps if "--steps" in sys.argv else 3
        warmup = args.warmup if "--warmup" in sys.argv else 1
        if args.workload == "moe":
            moe_line(steps, warmup)
        else:
            workload_line(args.workload, steps, warmup)
        return

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
    # The Cholesky-factor form: factor_chol (no triangular inverse) and the sweep on V.
    qflags = nvq.FLAG_CHOL_FACTOR
    ws_f_n = lib.factor_chol_workspace_size(K_IN)
    ws_g_n = lib.nvfp4_global_scale_workspace_size(M, K_IN)
    ws_q_n = lib.gptq_nvfp4_workspace_size(M, K_IN, qflags)
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
        chk("factor", lib.factor_chol(P(H), K_IN, 0.01, P(U), P(lam), P(info), P(ws["f"]), ws_f_n, s))
        if ev: ev[2].record()
        chk("gscale", lib.nvfp4_global_scale(P(Wd), nvq.NVQ_DTYPE_BF16, M, K_IN, K_IN, P(g), P(ws["g"]), ws_g_n, s))
        if ev: ev[3].record()
        chk("quantize", lib.gptq_nvfp4_quantize(P(Wd), nvq.NVQ_DTYPE_BF16, M, K_IN, K_IN, P(U), P(H), P(g), N_CAND,
                                                qflags, P(codes), P(scales), P(row_err), P(row_loss), P(ws["q"]),
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

    # The NVFP4 pack and unpack kernels at a size where HBM, not launch latency,
    # bounds them: the 70B-class down projection's W (8192 x 28672 bf16).
    roofline_pack = pack_roofline(nvq, lib, P, dev)

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
                   "d_out": M, "d_in": K_IN, "tokens": N_TOK, "n_cand": N_CAND, "factor": "cholesky"},
        "roofline": roofline,
        "roofline_pack": roofline_pack,
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
