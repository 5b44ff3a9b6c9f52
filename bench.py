#!/usr/bin/env python3
"""Benchmark of the online 2:4 activation-sparse linear layer on one MI355X.

One step = one pass of the whole hot path over one batch: rtl_sparse_linear
(pre-pass: 2:4 selection, compensation scale, compression, LoRA-down; then
the structured-sparse GEMM with the scale and LoRA-up epilogue) on the DiT
MLP up-projection X[4096, 3072] -> Y[4096, 12288] with rank-64 LoRA, inputs
already resident in HBM.  The split into the two kernels is timed in a
second loop through rtl_sparse_linear_prepare / _apply.  Prints one JSON line on stdout; progress goes to
stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

value = effective TFLOP/s = 2 M N K / (time per step): dense-equivalent
flops, LoRA flops excluded from the numerator, LoRA time included.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "eff. TFLOP/s + speedup vs dense bf16 GEMM, M=4096 K=3072 N=12288; %MFMA peak"
PEAK_BF16_DENSE_TFLOPS = 2516.6      # 256 CU x 2048 MAC/clk x 2 x 2.4 GHz (AMD: 2.5 PF)
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "activation_sparse_gemm_token_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources that make up the structured-sparse GEMM kernel (its code and
# the workspace layout it reads).
GEMM_SOURCES = ("sparse_gemm.hip", "gemm_common.hpp", "rtl_common.hpp", "rtl_kernels.hpp")


def kernel_source_hash() -> str:
    """Hash of the GEMM kernel's sources: counter readings are only reported
    for the kernel they were taken on."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    path = os.path.join(PROFILES, f"traffic_sparse_gemm_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        log(f"[bench] {path} was taken on other kernel sources: traffic reported as null")
        return None
    return t


def traffic_from_counters(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """HBM bytes per launch of the structured-sparse GEMM from two rocprofv3
    --pmc runs of ``bench.py --counters`` (FETCH_SIZE, then WRITE_SIZE; KiB
    per dispatch).  Each counter is scaled by what it reads for the plain
    256 MiB device-to-device copy in the same run (the HIP runtime's
    copyBuffer kernel: the calibration kernel)."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                key = ("sparse_gemm" if "sparse_gemm_kernel" in name else
                       "copy" if "copybuffer" in name.lower() else None)
                if key:
                    vals.setdefault(key, []).append(float(row["Counter_Value"]))
        if "sparse_gemm" not in vals or "copy" not in vals:
            raise SystemExit(f"{d}: no {counter} rows for the sparse GEMM and the copy kernel")
        # the runtime's blit kernel also serves the smaller input uploads:
        # the calibration copies are the largest dispatches
        top = max(vals["copy"])
        vals["copy"] = [v for v in vals["copy"] if v >= 0.75 * top]
        return {k: statistics.median(v) for k, v in vals.items()}

    copy_bytes = float(256 << 20)
    f = per_kernel(fetch_dir, "FETCH_SIZE")
    w = per_kernel(write_dir, "WRITE_SIZE")
    f_scale = copy_bytes / (f["copy"] * 1024.0)
    w_scale = copy_bytes / (w["copy"] * 1024.0)
    hbm = f["sparse_gemm"] * 1024.0 * f_scale + w["sparse_gemm"] * 1024.0 * w_scale
    return {"workload": workload, "kernel": "sparse_gemm_kernel (rtl_sparse_linear_apply)",
            "fetch_size_kib": f["sparse_gemm"], "write_size_kib": w["sparse_gemm"],
            "copy_fetch_size_kib": f["copy"], "copy_write_size_kib": w["copy"],
            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
            "hbm_bytes_per_launch": round(hbm), "kernel_source_hash": kernel_source_hash()}


def cpu_baseline(x, w, a, b, reps: int):
    """The oracle as it stands, on the host cores, same inputs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max(i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        cores = len(os.sched_getaffinity(0))
    m, k = x.shape
    n = w.shape[0]
    times = []
    for i in range(reps):
        t0 = time.perf_counter()
        oracle.sparse_linear_ref(x, w, a, b, 1.0)
        times.append(time.perf_counter() - t0)
        log(f"[bench] cpu oracle rep {i}: {times[-1]:.2f} s")
    t = statistics.median(times)
    return {"value": 2.0 * m * n * k / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole {m}x{k}x{n} r={a.shape[0]} layer, NumPy fp64, median of {reps} runs "
                      f"({t:.2f} s each)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: the GPU clock takes ~40 ms of sustained work to ramp up, so
    # 300 untimed steps (~65 ms) come before 300 timed ones.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="mlp_up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=8)
    ap.add_argument("--counters", action="store_true",
                    help="a short launch sequence for rocprofv3 --pmc passes: 3 x (prepare, apply, dense, "
                         "sparsify) and 3 plain 256 MiB copies (the calibration kernel); prints no JSON")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_sparse_gemm_<workload>.json from the two rocprofv3 --pmc "
                         "output folders of --counters runs (FETCH_SIZE, WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.traffic_from:
        t = traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.workload)
        path = os.path.join(PROFILES, f"traffic_sparse_gemm_{args.workload}.json")
        with open(path, "w") as fh:
            json.dump(t, fh, indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer runs on a single MI355X; "
              "multi-GPU runs are not part of it (see DESIGN.md on how it would shard)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_sparse_gemm_token_amd as rtl
    from workloads import gen

    cfg = gen.config(args.workload)
    m, k, n, r = cfg.m, cfg.k, cfg.n, cfg.r
    log(f"[bench] workload {cfg.name}: M={m} K={k} N={n} r={r}")
    x, w, a, b = gen.make_config(cfg)
    dev = "cuda:0"

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    xd, wd, ad, bd = up(x), up(w), up(a), up(b)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((rtl.sparse_linear_workspace_bytes(m, k, r),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        rtl.sparse_linear(xd, wd, ad, bd, 1.0, out=y, workspace=ws)

    if args.counters:
        src = torch.empty((256 << 20,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        vals = torch.empty((m, k // 2), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((m, (k // 4 + 1) // 2), dtype=torch.uint8, device=dev)
        scale = torch.empty((m,), dtype=torch.float32, device=dev)
        for _ in range(3):
            step()
            rtl.dense_linear(xd, wd, out=y)
            rtl.sparsify_2of4(xd)
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] counter sequence done")
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps of rtl_sparse_linear (pre-pass + GEMM), HIP
    # events on the launch stream around the whole loop.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    # The two halves, K more steps with events around each launch.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        p = rtl.prepare(xd, ad, 1.0, workspace=ws)
        ev[i][1].record(stream)
        rtl.apply(p, wd, bd, out=y)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    prep_ms = [e[0].elapsed_time(e[1]) for e in ev]
    apply_ms = [e[1].elapsed_time(e[2]) for e in ev]
    prep_avg = sum(prep_ms) / len(prep_ms)
    apply_avg = sum(apply_ms) / len(apply_ms)

    flops_dense_eq = 2.0 * m * n * k
    value = flops_dense_eq / (ms_step * 1e-3) / 1e12
    log(f"[bench] sparse step {ms_step * 1e3:.1f} us (prepare {prep_avg * 1e3:.1f} us, apply "
        f"{apply_avg * 1e3:.1f} us): {value:.1f} eff. TFLOP/s")

    # In-house dense baseline and hipBLASLt (torch.matmul) for context.
    yd = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def time_fn(fn, reps):
        for _ in range(max(3, args.warmup)):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    dense_ms = time_fn(lambda: rtl.dense_linear(xd, wd, out=yd), args.steps)
    wt = wd.t()
    blas_ms = time_fn(lambda: torch.matmul(xd, wt, out=yd), args.steps)
    vals = torch.empty((m, k // 2), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((m, (k // 4 + 1) // 2), dtype=torch.uint8, device=dev)
    scale = torch.empty((m,), dtype=torch.float32, device=dev)
    lib = rtl.lib()
    sp_ms = time_fn(lambda: lib.rtl_sparsify_2of4(xd.data_ptr(), m, k, vals.data_ptr(), idx.data_ptr(),
                                                   scale.data_ptr(), 0, stream.cuda_stream), args.steps)
    sp_bytes = 2 * m * k + m * k + m * ((k // 4 + 1) // 2) + 4 * m
    log(f"[bench] dense in-house {dense_ms * 1e3:.1f} us, hipBLASLt {blas_ms * 1e3:.1f} us, "
        f"sparsify {sp_ms * 1e3:.1f} us")

    # Roofline of the dominant kernel: the structured-sparse GEMM (apply).
    # Algorithmic flops per launch: the kept half of the product, M N K
    # (2 flops x M N K/2 kept MACs), plus the LoRA-up 2 M N r; priced
    # against the dense bf16 peak (the sparse instruction's useful rate).
    alg_flops = float(m) * n * k + 2.0 * m * n * r
    achieved = alg_flops / (apply_avg * 1e-3) / 1e12
    traffic = load_traffic(cfg.name)
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_DENSE_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_DENSE_TFLOPS, 4),
                "traffic": traffic["hbm_bytes_per_launch"] if traffic else None}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, w, a, b, args.cpu_reps)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded DiT-shaped activations (8% large channels), Gaussian W and LoRA",
        "config": {"workload": f"{cfg.name}: DiT MLP up-projection M={m} K={k} N={n}, LoRA r={r}",
                   "M": m, "K": k, "N": n, "r": r},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {
            "speedup_vs_inhouse_dense": round(dense_ms / ms_step, 3),
            "speedup_vs_hipblaslt": round(blas_ms / ms_step, 3),
            "inhouse_dense_tflops": round(flops_dense_eq / (dense_ms * 1e-3) / 1e12, 1),
            "hipblaslt_tflops": round(flops_dense_eq / (blas_ms * 1e-3) / 1e12, 1),
            "frac_dense_peak": round(value / PEAK_BF16_DENSE_TFLOPS, 4),
            "frac_sparse_peak": round(value / (2 * PEAK_BF16_DENSE_TFLOPS), 4),
            "prepare_us": round(prep_avg * 1e3, 2),
            "apply_us": round(apply_avg * 1e3, 2),
            "prepare_share": round(prep_avg / (prep_avg + apply_avg), 4),
            "sparsify_2of4_us": round(sp_ms * 1e3, 2),
            "sparsify_2of4_GBs": round(sp_bytes / (sp_ms * 1e-3) / 1e9, 1),
            "sparsify_2of4_frac_hbm": round(sp_bytes / (sp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
