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

Before anything is timed, at least RAMP_MS of untimed layer calls bring the
GPU clock up, whatever --warmup says (the clock needs tens of ms of load).

`detail` adds: speedups over the in-house dense GEMM and hipBLASLt (the three
timed in interleaved blocks, order rotated, medians); useful
TFLOP/s (M N K + LoRA flops); per-call median / min / p90 of the step and
its two halves; the layer without LoRA (r = 0) and its unfused form
(rtl_sparsify_2of4, then rtl_sparse_linear_compressed); cold timings (MALL and L2
flushed by a 512 MB write before every call) for the layer and both dense
GEMMs, and the same with X read back into the caches after the flush (weights
cold, input warm); the graphics clock the driver reports under this load and the
fractions of the peak rescaled to it; the standalone sparsify; CPU context
(the oracle's selection step alone, NumPy fp32 dense GEMM).
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
RAMP_MS = 150.0         # untimed load before any timed loop (the clock's ramp)
BLOCKS = 6              # interleaved timing blocks per leg for the speedups
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


def cpu_context(x, w):
    """CPU figures beside the oracle: its selection + scale step alone
    (vectorised NumPy, one thread) on the whole X, and a plain NumPy fp32
    dense X W^T on the host's BLAS threads."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.sparsify(x)
        t_sel = time.perf_counter() - t0
    xf = oracle.bf16_bits_to_f64(x).astype(np.float32)
    wf = oracle.bf16_bits_to_f64(w).astype(np.float32)
    xf @ wf[:64].T
    t0 = time.perf_counter()
    xf @ wf.T
    t_mm = time.perf_counter() - t0
    m, k = x.shape
    n = w.shape[0]
    return {"oracle_select_scale_s_1thread": round(t_sel, 3),
            "numpy_fp32_dense_tflops": round(2.0 * m * n * k / t_mm / 1e12, 3)}


class ClockSampler:
    """Samples the graphics clock the driver reports (amdsmi GPU metrics,
    one reading per XCD) from a host thread, with host timestamps, so that
    the readings taken while a given loop ran can be picked out."""

    def __init__(self):
        import threading
        self.samples = []                 # (perf_counter seconds, MHz)
        self._stop = threading.Event()
        self._th = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:          # no metrics interface: the figures are reported as null
            log(f"[bench] no clock readings: {e!r}")
            self._amdsmi = None

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
                # entries outside 100-5000 MHz are the interface's "not available" markers
                c = [v for v in m.get("current_gfxclks", []) if isinstance(v, (int, float)) and 100 <= v <= 5000]
                if c:
                    self.samples.append((time.perf_counter(), sum(c) / len(c)))
            except Exception:
                pass
            self._stop.wait(0.001)

    def start(self):
        if self._amdsmi is not None:
            import threading
            self._th = threading.Thread(target=self._run, daemon=True)
            self._th.start()
        return self

    def stop(self):
        if self._th is not None:
            self._stop.set()
            self._th.join()

    def window(self, t0, t1):
        """Median, min and max of the readings taken between host times t0
        and t1, or None if there were none."""
        s = [v for t, v in self.samples if t0 <= t <= t1]
        if not s:
            return None
        return {"median": round(statistics.median(s), 1), "min": round(min(s), 1), "max": round(max(s), 1),
                "readings": len(s)}


def peak_at_clock(sclk_mhz, dense_rates_tflops):
    """The dense bf16 peak rescaled to an observed graphics clock, and a note.
    A reading below the clock that measured dense-rate work needs (kept MACs
    of the sparse GEMM, the dense GEMMs: none can beat the peak at the clock
    it ran at) is not that clock (a stale or idle figure from the driver):
    then no rescaled peak, and the note says why."""
    if not sclk_mhz:
        return None, None
    peak = PEAK_BF16_DENSE_TFLOPS * sclk_mhz / 2400.0
    need = max(dense_rates_tflops)
    if need > peak:
        return None, (f"driver clock reading {sclk_mhz} MHz is below the "
                      f"{need / PEAK_BF16_DENSE_TFLOPS * 2400:.0f} MHz the measured dense rates need; not used")
    return peak, None


def dist(ms_list):
    """median / min / p90 / mean of per-launch times, in microseconds."""
    v = sorted(ms_list)
    p90 = v[min(len(v) - 1, int(round(0.9 * (len(v) - 1))))]
    return {"median": round(statistics.median(v) * 1e3, 2), "min": round(v[0] * 1e3, 2),
            "p90": round(p90 * 1e3, 2), "mean": round(sum(v) / len(v) * 1e3, 2)}


SUITE = ("tiny", "attn_proj", "mlp_up", "mlp_down", "textimg_p05", "textimg_p10", "textimg_p25",
         "mlp_up_share8", "textimg_share8", "textimg_share2")


def queued_ms(fn, reps: int, stream) -> float:
    """Mean time of `reps` back-to-back calls of fn, enqueued behind a GPU-side
    wait (about 2 ms, or 30 us per call) so that the host has issued them all
    before the first runs: a 13 us pre-pass can outrun the host's issue of C calls
    (validation, device query, launch), and the events then see kernel
    time only."""
    import torch
    torch.cuda._sleep(max(1 << 22, 60_000 * reps))     # shader-clock cycles: ~2 ms, 30 us per call
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_suite(reps: int, warmup: int):
    """Every linear-layer workload, warm, one JSON line each: the layer
    (pre-pass + apply), its halves, the in-house dense GEMM, hipBLASLt and
    the standalone sparsify;
    then Q, K and V sharing one input (one pre-pass, three applies) and the
    time-weighted speedup over one DiT block's linears (Q, K, V, output
    projection, MLP up, MLP down)."""
    import numpy as np
    import torch

    import activation_sparse_gemm_token_amd as rtl
    from workloads import gen

    dev = "cuda:0"
    stream = torch.cuda.current_stream()

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def mean_ms(fn):
        for _ in range(warmup):
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

    def interleaved_ms(legs):
        """Median time per call of each leg over BLOCKS blocks of `reps`
        back-to-back calls, the legs' order rotated from block to block."""
        # warm-up: the legs in turn for at least a third of RAMP_MS (the
        # clock's ramp), and at least `warmup` calls of each
        t0, calls = time.perf_counter(), 0
        while calls < warmup or (time.perf_counter() - t0) * 1e3 < RAMP_MS / 3:
            for fn in legs.values():
                fn()
            calls += 1
            if calls % 10 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        order = list(legs)
        blocks = {kk: [] for kk in legs}
        for bi in range(BLOCKS):
            for kk in order[bi % len(order):] + order[:bi % len(order)]:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    legs[kk]()
                e1.record(stream)
                torch.cuda.synchronize()
                blocks[kk].append(e0.elapsed_time(e1) / reps)
        return {kk: statistics.median(v) for kk, v in blocks.items()}

    res = {}
    for name in SUITE:
        cfg = gen.config(name)
        x, w, a, b = gen.make_config(cfg)
        xd, wd, ad, bd = up(x), up(w), up(a), up(b)
        m, k, n, r = cfg.m, cfg.k, cfg.n, cfg.r
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((rtl.sparse_linear_workspace_bytes(m, k, r),), dtype=torch.uint8, device=dev)
        wt = wd.t()
        # the layer and both dense GEMMs in interleaved blocks (no leg gains
        # from coming after the others)
        t = interleaved_ms({"layer": lambda: rtl.sparse_linear(xd, wd, ad, bd, 1.0, out=y, workspace=ws),
                            "dense": lambda: rtl.dense_linear(xd, wd, out=y),
                            "blas": lambda: torch.matmul(xd, wt, out=y)})
        t_layer, t_dense, t_blas = t["layer"], t["dense"], t["blas"]
        # the halves through the C entry points, arguments marshalled once;
        # the pre-pass (shorter than a call's host time) queued behind a wait
        clib, sp = rtl.lib(), stream.cuda_stream
        prep_args = (xd.data_ptr(), ad.data_ptr(), m, k, r, 1.0, ws.data_ptr(), ws.numel(), sp)
        apply_args = (ws.data_ptr(), ws.numel(), wd.data_ptr(), bd.data_ptr(), m, n, k, r, y.data_ptr(), sp)
        prep = rtl.prepare(xd, ad, 1.0, workspace=ws)
        t_apply = mean_ms(lambda: clib.rtl_sparse_linear_apply(*apply_args))
        # the standalone sparsify into the canonical layout, queued likewise
        vals = torch.empty((m, k // 2), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((m, (k // 4 + 1) // 2), dtype=torch.uint8, device=dev)
        scale = torch.empty((m,), dtype=torch.float32, device=dev)
        sp_args = (xd.data_ptr(), m, k, vals.data_ptr(), idx.data_ptr(), scale.data_ptr(), 0, sp)
        for _ in range(warmup):
            clib.rtl_sparsify_2of4(*sp_args)
        t_sp = queued_ms(lambda: clib.rtl_sparsify_2of4(*sp_args), reps, stream)
        sp_bytes = 2 * m * k + m * k + m * ((k // 4 + 1) // 2) + 4 * m
        # last: its GPU-side wait lets the clock drop
        t_prep = queued_ms(lambda: clib.rtl_sparse_linear_prepare(*prep_args), reps, stream)
        f = 2.0 * m * n * k
        line = {"workload": name, "M": m, "K": k, "N": n, "r": r,
                "layer_us": round(t_layer * 1e3, 2), "prepare_us": round(t_prep * 1e3, 2),
                "apply_us": round(t_apply * 1e3, 2), "inhouse_dense_us": round(t_dense * 1e3, 2),
                "hipblaslt_us": round(t_blas * 1e3, 2),
                "eff_tflops": round(f / (t_layer * 1e-3) / 1e12, 1),
                "speedup_vs_inhouse_dense": round(t_dense / t_layer, 3),
                "speedup_vs_hipblaslt": round(t_blas / t_layer, 3),
                "frac_dense_peak": round(f / (t_layer * 1e-3) / 1e12 / PEAK_BF16_DENSE_TFLOPS, 4),
                "sparsify_us": round(t_sp * 1e3, 2),
                "sparsify_GBs": round(sp_bytes / (t_sp * 1e-3) / 1e9, 1),
                "sparsify_frac_hbm": round(sp_bytes / (t_sp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        res[name] = line
        print(json.dumps(line), flush=True)
        del xd, wd, ad, bd, y, ws, prep, vals, idx, scale

    # Q, K, V: three 3072 x 3072 projections of one input sharing the
    # LoRA-down (one pre-pass), each with its own W and LoRA-up.
    cfg = gen.config("attn_proj")
    x, _, a, _ = gen.make_config(cfg)
    rng = np.random.default_rng(101)
    ws3 = [up(gen.gaussian_bits(rng, (cfg.n, cfg.k), 0.02)) for _ in range(3)]
    bs3 = [up(gen.gaussian_bits(rng, (cfg.n, cfg.r), 0.01)) for _ in range(3)]
    xd, ad = up(x), up(a)
    ys = [torch.empty((cfg.m, cfg.n), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    ws = torch.empty((rtl.sparse_linear_workspace_bytes(cfg.m, cfg.k, cfg.r),), dtype=torch.uint8, device=dev)

    def qkv_sparse():
        p = rtl.prepare(xd, ad, 1.0, workspace=ws)
        for i in range(3):
            rtl.apply(p, ws3[i], bs3[i], out=ys[i])

    def qkv_dense():
        for i in range(3):
            rtl.dense_linear(xd, ws3[i], out=ys[i])

    wts = [t.t() for t in ws3]

    def qkv_blas():
        for i in range(3):
            torch.matmul(xd, wts[i], out=ys[i])

    t = interleaved_ms({"s": qkv_sparse, "d": qkv_dense, "b": qkv_blas})
    t_s, t_d, t_b = t["s"], t["d"], t["b"]
    qkv = {"workload": "qkv_shared_input", "M": cfg.m, "K": cfg.k, "N": f"3 x {cfg.n}", "r": cfg.r,
           "layer_us": round(t_s * 1e3, 2), "inhouse_dense_us": round(t_d * 1e3, 2),
           "hipblaslt_us": round(t_b * 1e3, 2),
           "speedup_vs_inhouse_dense": round(t_d / t_s, 3), "speedup_vs_hipblaslt": round(t_b / t_s, 3)}
    print(json.dumps(qkv), flush=True)

    block = [("qkv", qkv), ("out_proj", res["attn_proj"]), ("mlp_up", res["mlp_up"]),
             ("mlp_down", res["mlp_down"])]
    tot_s = sum(v["layer_us"] for _, v in block)
    tot_d = sum(v["inhouse_dense_us"] for _, v in block)
    tot_b = sum(v["hipblaslt_us"] for _, v in block)
    print(json.dumps({"workload": "dit_block_linears (qkv, out_proj, mlp_up, mlp_down; 4096 tokens)",
                      "sparse_us": round(tot_s, 2), "inhouse_dense_us": round(tot_d, 2),
                      "hipblaslt_us": round(tot_b, 2),
                      "speedup_vs_inhouse_dense": round(tot_d / tot_s, 3),
                      "speedup_vs_hipblaslt": round(tot_b / tot_s, 3)}), flush=True)


def run_variants(reps: int, warmup: int):
    """The compensation and LoRA-input variants: for every workload, the
    relative rms deviation of Y from the dense product X W^T (the quantity
    the compensation is meant to shrink) with r = 0; then on the headline
    all 12 variants with its rank-64 LoRA (random factors: the branch adds a
    term here instead of restoring one), with their times.  One JSON line
    each.  The deviation is measured with torch on the device, in fp32."""
    import numpy as np
    import torch

    import activation_sparse_gemm_token_amd as rtl
    from workloads import gen

    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    comps = {"token": rtl.COMP_TOKEN, "none": rtl.COMP_NONE, "tensor": rtl.COMP_TENSOR, "group": rtl.COMP_GROUP}
    loras = {"residual": rtl.LORA_RESIDUAL, "pruned": rtl.LORA_PRUNED, "input": rtl.LORA_INPUT}

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def rel_dev(y, yd):
        d = (y.float() - yd.float()).pow(2).mean().sqrt()
        return float(d / yd.float().pow(2).mean().sqrt())

    def mean_ms(fn):
        for _ in range(warmup):
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

    for name in SUITE:
        cfg = gen.config(name)
        x, w, _, _ = gen.make_config(cfg, with_lora=False)
        xd, wd = up(x), up(w)
        yd = rtl.dense_linear(xd, wd)
        ws = torch.empty((rtl.sparse_linear_workspace_bytes(cfg.m, cfg.k, 0),), dtype=torch.uint8, device=dev)
        line = {"workload": name, "r": 0, "x_law": cfg.x_law}
        for cn, cv in comps.items():
            y = rtl.apply(rtl.prepare(xd, None, 1.0, workspace=ws, variant=cv), wd)
            line[f"dev_{cn}"] = round(rel_dev(y, yd), 5)
        print(json.dumps(line), flush=True)
        del xd, wd, yd, ws

    cfg = gen.config("mlp_up")
    x, w, a, b = gen.make_config(cfg)
    xd, wd, ad, bd = up(x), up(w), up(a), up(b)
    yd = rtl.dense_linear(xd, wd)
    y = torch.empty_like(yd)
    ws = torch.empty((rtl.sparse_linear_workspace_bytes(cfg.m, cfg.k, cfg.r),), dtype=torch.uint8, device=dev)
    clib, sp = rtl.lib(), stream.cuda_stream
    for cn, cv in comps.items():
        for ln, lv in loras.items():
            v = cv | lv
            # through the C entry point, arguments marshalled once (a wrapped
            # call's host time exceeds a 13 us pre-pass)
            pv_args = (xd.data_ptr(), ad.data_ptr(), cfg.m, cfg.k, cfg.r, 1.0, v, ws.data_ptr(), ws.numel(), sp)
            t_prep = mean_ms(lambda: clib.rtl_sparse_linear_prepare_variant(*pv_args))
            p = rtl.prepare(xd, ad, 1.0, workspace=ws, variant=v)
            t_app = mean_ms(lambda: rtl.apply(p, wd, bd, out=y))
            rtl.apply(p, wd, bd, out=y)
            print(json.dumps({"workload": "mlp_up", "r": cfg.r, "comp": cn, "lora": ln,
                              "prepare_us": round(t_prep * 1e3, 2), "apply_us": round(t_app * 1e3, 2),
                              "dev_vs_dense": round(rel_dev(y, yd), 5)}), flush=True)


MFMA_KINDS = (
    # kind, instruction, dense-equivalent flops, nominal cycles per SIMD at
    # the dense peak (2048 dense MACs per CU per clock; the structured-sparse
    # instructions at twice the dense-equivalent rate)
    (0, "v_mfma_f32_16x16x32_bf16", 2 * 16 * 16 * 32, 16),
    (1, "v_mfma_f32_32x32x16_bf16", 2 * 32 * 32 * 16, 32),
    (2, "v_smfmac_f32_16x16x64_bf16", 2 * 16 * 16 * 64, 16),
    (3, "v_smfmac_f32_32x32x32_bf16", 2 * 32 * 32 * 32, 32),
)


def run_mfma_rates(iters: int = 2048):
    """Issue rate of the bf16 matrix instructions (microbench/mfma_rates.hip):
    one line per instruction and wavefronts per SIMD, with the cycles per
    instruction per SIMD from the shader clock, the dense-equivalent TFLOP/s
    from events, the clock, and the fraction of the nominal rate."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "activation_sparse_gemm_token_amd", "libmfma_rates.so")
    mb = ctypes.CDLL(path)
    fn = mb.mb_mfma_rate
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    dev = "cuda:0"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    for kind, name, flops, nominal in MFMA_KINDS:
        for waves in (4, 8):
            blocks = cus
            cyc = torch.zeros((blocks * waves,), dtype=torch.int64, device=dev)
            sink = torch.zeros((blocks * 64 * waves,), dtype=torch.float32, device=dev)

            def launch():
                st = fn(kind, blocks, waves, iters, cyc.data_ptr(), sink.data_ptr(), stream.cuda_stream)
                if st != 0:
                    raise RuntimeError(f"mb_mfma_rate launch failed: {st}")

            t0 = time.perf_counter()
            while time.perf_counter() - t0 < RAMP_MS * 1e-3:
                launch()
                torch.cuda.synchronize()
            times, cycles = [], []
            for _ in range(5):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e-3)
                # the longest loop of each CU: with two wavefronts per SIMD
                # they share the matrix core unevenly, the last to finish
                # spans the whole issue
                per_cu = cyc.view(blocks, waves).max(dim=1).values
                cycles.append(statistics.median(per_cu.cpu().tolist()))
            t = statistics.median(times)
            c = statistics.median(cycles)
            per_simd = waves // 4
            instr = blocks * waves * iters * 8
            cpi = c / (iters * 8 * per_simd)
            tflops = instr * flops / t / 1e12
            mhz = c / t / 1e6
            print(json.dumps({"instruction": name, "wavefronts_per_simd": per_simd,
                              "cycles_per_instruction_per_simd": round(cpi, 2), "nominal_cycles": nominal,
                              "frac_of_nominal_rate": round(nominal / cpi, 4),
                              "dense_equivalent_tflops": round(tflops, 1), "shader_clock_mhz": round(mhz, 1),
                              "cus": cus, "iters": iters}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The clock ramp does not depend on these (RAMP_MS of untimed calls
    # always come first); 300 timed steps keep the event overhead small.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="mlp_up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=12)
    ap.add_argument("--counters", action="store_true",
                    help="a short launch sequence for rocprofv3 --pmc passes: 3 x (prepare, apply, dense, "
                         "sparsify) and 3 plain 256 MiB copies (the calibration kernel); prints no JSON")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_sparse_gemm_<workload>.json from the two rocprofv3 --pmc "
                         "output folders of --counters runs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--variants", action="store_true",
                    help="deviation from the dense product and time of every compensation / LoRA-input variant")
    ap.add_argument("--mfma-rates", action="store_true",
                    help="issue rate of the bf16 dense and structured-sparse matrix instructions; one JSON line each")
    ap.add_argument("--suite", action="store_true",
                    help="time every linear-layer workload and one DiT block's linears; one JSON line each")
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
              "multi-GPU runs are not part of it (it would shard by token, with no communication)",
              file=sys.stderr)
        sys.exit(2)
    if args.suite:
        run_suite(args.steps, args.warmup)
        return
    if args.mfma_rates:
        run_mfma_rates()
        return
    if args.variants:
        run_variants(min(args.steps, 100), min(args.warmup, 100))
        return

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

    # Clock ramp: the GPU clock needs tens of milliseconds of sustained load
    # to reach its working frequency, so at least RAMP_MS of untimed layer
    # calls run before anything is timed, whatever --warmup asks; then the
    # --warmup steps.
    clk = ClockSampler().start()
    t_ramp0 = time.perf_counter()
    ramp_calls = 0
    while (time.perf_counter() - t_ramp0) * 1e3 < RAMP_MS:
        for _ in range(25):
            step()
        ramp_calls += 25
        torch.cuda.synchronize()
    ramp_ms = (time.perf_counter() - t_ramp0) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps of rtl_sparse_linear (pre-pass + GEMM), HIP
    # events on the launch stream around the whole loop; the clock readings
    # taken meanwhile are kept.
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
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]

    # Average launch duration of each half: K back-to-back launches of it
    # between two events (an event between every launch inflates a 13 us
    # kernel by several us), issued through the C entry points with their
    # arguments marshalled once, so that the host keeps ahead of a 13 us
    # kernel.
    def block_ms(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # The pre-pass block as issued, and below (before the cold timings, whose
    # idle waits it shares) queued behind a GPU-side wait (queued_ms): a
    # 13 us kernel can outrun the host's issue of C calls.
    clib = rtl.lib()
    sp = stream.cuda_stream
    prep_args = (xd.data_ptr(), ad.data_ptr(), m, k, r, 1.0, ws.data_ptr(), ws.numel(), sp)
    apply_args = (ws.data_ptr(), ws.numel(), wd.data_ptr(), bd.data_ptr(), m, n, k, r, y.data_ptr(), sp)
    prep_eager = block_ms(lambda: clib.rtl_sparse_linear_prepare(*prep_args))
    apply_avg = block_ms(lambda: clib.rtl_sparse_linear_apply(*apply_args))

    flops_dense_eq = 2.0 * m * n * k
    value = flops_dense_eq / (ms_step * 1e-3) / 1e12
    log(f"[bench] sparse step {ms_step * 1e3:.1f} us (prepare {prep_eager * 1e3:.1f} us, apply "
        f"{apply_avg * 1e3:.1f} us): {value:.1f} eff. TFLOP/s")

    def time_fn(fn, reps):
        """Mean time per call of `reps` back-to-back calls (warm)."""
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

    # The same layer through the layer policy with the streamed-weights hint
    # (the GEMM instance that probes W into L2 ahead of its copies), warm
    # here and cold below: the trade it makes.  Both legs through the C
    # entry points, the clock still ramped.
    from activation_sparse_gemm_token_amd import layers as rtl_layers
    streamed = rtl_layers.LayerPolicy(1, stream_weights=True)
    ll = rtl_layers._fn()
    ll_args = (streamed.modes, 1, 0, xd.data_ptr(), wd.data_ptr(), ad.data_ptr(), bd.data_ptr(), m, n, k, r, 1.0,
               y.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream)
    plain_args = (xd.data_ptr(), wd.data_ptr(), ad.data_ptr(), bd.data_ptr(), m, n, k, r, 1.0, y.data_ptr(),
                  ws.data_ptr(), ws.numel(), stream.cuda_stream)

    def step_stream_w():
        ll(*ll_args)

    def step_plain_c():
        clib.rtl_sparse_linear(*plain_args)

    # Both warmed first (the probing instance's first launch loads it), then
    # interleaved blocks in alternating order, medians.
    for _ in range(3):
        step_stream_w()
    torch.cuda.synchronize()
    sw_blocks = {"plain": [], "stream_w": []}
    sw_legs = (("plain", step_plain_c), ("stream_w", step_stream_w))
    for bi in range(BLOCKS):
        for name, fn in (sw_legs if bi % 2 == 0 else sw_legs[::-1]):
            sw_blocks[name].append(block_ms(fn))
    warm_plain_ms = statistics.median(sw_blocks["plain"])
    warm_stream_w_ms = statistics.median(sw_blocks["stream_w"])

    # The same layer without the LoRA branch (r = 0): the bare sparse GEMM
    # path (pre-pass without LoRA-down, GEMM without LoRA-up).
    r0_ms = time_fn(lambda: rtl.sparse_linear(xd, wd, None, None, 1.0, out=y, workspace=ws), args.steps)

    # The speedups: the layer, the in-house dense GEMM and hipBLASLt
    # (torch.matmul) timed in interleaved blocks of K back-to-back calls,
    # the order rotated from block to block, so that no leg gains from
    # coming after the others (clock, caches); medians over the blocks.
    yd = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    wt = wd.t()
    legs = {"sparse": step,
            "dense": lambda: rtl.dense_linear(xd, wd, out=yd),
            "hipblaslt": lambda: torch.matmul(xd, wt, out=yd)}
    for fn in legs.values():
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    blocks = {name: [] for name in legs}
    order = list(legs)
    for bi in range(BLOCKS):
        for name in order[bi % len(order):] + order[:bi % len(order)]:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                legs[name]()
            e1.record(stream)
            torch.cuda.synchronize()
            blocks[name].append(e0.elapsed_time(e1) / args.steps)
    sparse_blk_ms = statistics.median(blocks["sparse"])
    dense_ms = statistics.median(blocks["dense"])
    blas_ms = statistics.median(blocks["hipblaslt"])
    vals = torch.empty((m, k // 2), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((m, (k // 4 + 1) // 2), dtype=torch.uint8, device=dev)
    scale = torch.empty((m,), dtype=torch.float32, device=dev)
    lib = rtl.lib()
    sp_ms = time_fn(lambda: lib.rtl_sparsify_2of4(xd.data_ptr(), m, k, vals.data_ptr(), idx.data_ptr(),
                                                   scale.data_ptr(), 0, stream.cuda_stream), args.steps)
    sp_bytes = 2 * m * k + m * k + m * ((k // 4 + 1) // 2) + 4 * m
    prep_bytes = 2 * m * k + 2 * r * k + m * k + m * k // 8 + 4 * m + 4 * m * r
    # The unfused form of the layer without LoRA: sparsify to the canonical
    # compressed X in HBM, then the GEMM on it (its repack included).
    ws0 = torch.empty((rtl.sparse_linear_workspace_bytes(m, k, 0),), dtype=torch.uint8, device=dev)

    def unfused():
        lib.rtl_sparsify_2of4(xd.data_ptr(), m, k, vals.data_ptr(), idx.data_ptr(), scale.data_ptr(), 0,
                              stream.cuda_stream)
        lib.rtl_sparse_linear_compressed(vals.data_ptr(), idx.data_ptr(), scale.data_ptr(), wd.data_ptr(),
                                         m, n, k, y.data_ptr(), ws0.data_ptr(), ws0.numel(), stream.cuda_stream)

    unf_ms = time_fn(unfused, args.steps)
    comp_ms = time_fn(lambda: lib.rtl_sparse_linear_compressed(
        vals.data_ptr(), idx.data_ptr(), scale.data_ptr(), wd.data_ptr(), m, n, k, y.data_ptr(),
        ws0.data_ptr(), ws0.numel(), stream.cuda_stream), args.steps)
    log(f"[bench] r=0 {r0_ms * 1e3:.1f} us, dense in-house {dense_ms * 1e3:.1f} us, hipBLASLt "
        f"{blas_ms * 1e3:.1f} us, sparsify {sp_ms * 1e3:.1f} us, unfused {unf_ms * 1e3:.1f} us")

    prep_queued = queued_ms(lambda: clib.rtl_sparse_linear_prepare(*prep_args), args.steps, stream)
    clib.rtl_sparse_linear_prepare(*prep_args)     # the workspace of the layer's own inputs again
    prep_avg = min(prep_eager, prep_queued)

    # Cold: the MALL (256 MB) and the L2s flushed before every call by
    # writing 512 MB; events around the call only.
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)

    def time_cold(fn, reps=30, warm_x=False):
        out = []
        for i in range(reps):
            flush.fill_(i & 0xFF)
            if warm_x:
                # Weights cold, input warm: X read back into the caches
                # (the usual case for a layer whose input the previous
                # layer just wrote while the weights stream from HBM).
                torch.sum(xd)
            # A GPU-side wait (no memory traffic) while the host enqueues
            # the call, so that the events bracket GPU time only and not
            # the host's launch overhead of a single call.
            torch.cuda._sleep(1 << 21)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return dist(out)

    cold_step = time_cold(step)
    cold_dense = time_cold(lambda: rtl.dense_linear(xd, wd, out=yd))
    cold_blas = time_cold(lambda: torch.matmul(xd, wt, out=yd))
    wcold_step = time_cold(step, warm_x=True)
    cold_stream_w = time_cold(step_stream_w)
    wcold_stream_w = time_cold(step_stream_w, warm_x=True)
    wcold_dense = time_cold(lambda: rtl.dense_linear(xd, wd, out=yd), warm_x=True)
    wcold_blas = time_cold(lambda: torch.matmul(xd, wt, out=yd), warm_x=True)
    del flush

    # Graphics clock under this load, read from the driver while ~1 s of
    # steps runs (its metrics lag by a few hundred ms: a loop of a few ms is
    # too short for them, and a clock read on the GPU right after the loop
    # sees the clock rise as the load drops); the peaks rescaled to it say
    # how much of the gap to the nominal 2.4 GHz peak is the clock.
    for _ in range(200):
        step()
    torch.cuda.synchronize()
    h2 = time.perf_counter()
    for _ in range(max(1, int(1.0 / (ms_step * 1e-3)))):
        step()
    torch.cuda.synchronize()
    h3 = time.perf_counter()
    clk.stop()
    sclk_obs = clk.window(h2, h3)
    sclk = sclk_obs["median"] if sclk_obs else None
    log(f"[bench] cold step {cold_step['median']} us, dense {cold_dense['median']} us; sclk {sclk_obs} MHz")

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
    useful_flops = float(m) * n * k + 2.0 * m * k * r + 2.0 * m * n * r

    cpu = None
    cpu_ctx = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, w, a, b, args.cpu_reps)
        cpu_ctx = cpu_context(x, w)
    peak_at_sclk, sclk_note = peak_at_clock(
        sclk, (achieved, flops_dense_eq / (dense_ms * 1e-3) / 1e12, flops_dense_eq / (blas_ms * 1e-3) / 1e12))
    if sclk_note:
        log(f"[bench] {sclk_note}")

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
            "ramp_ms": round(ramp_ms, 1),
            "ramp_calls": ramp_calls,
            "speedup_vs_inhouse_dense": round(dense_ms / sparse_blk_ms, 3),
            "speedup_vs_hipblaslt": round(blas_ms / sparse_blk_ms, 3),
            "speedup_timing": f"medians of {BLOCKS} interleaved blocks of {args.steps} calls per leg",
            "interleaved_us": {k: [round(v * 1e3, 2) for v in vs] for k, vs in blocks.items()},
            "inhouse_dense_tflops": round(flops_dense_eq / (dense_ms * 1e-3) / 1e12, 1),
            "hipblaslt_tflops": round(flops_dense_eq / (blas_ms * 1e-3) / 1e12, 1),
            "inhouse_dense_frac_peak": round(flops_dense_eq / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_DENSE_TFLOPS, 4),
            "hipblaslt_frac_peak": round(flops_dense_eq / (blas_ms * 1e-3) / 1e12 / PEAK_BF16_DENSE_TFLOPS, 4),
            "frac_dense_peak": round(value / PEAK_BF16_DENSE_TFLOPS, 4),
            "frac_sparse_peak": round(value / (2 * PEAK_BF16_DENSE_TFLOPS), 4),
            "prepare_us": round(prep_avg * 1e3, 2),
            "prepare_us_eager_calls": round(prep_eager * 1e3, 2),
            "prepare_us_queued_calls": round(prep_queued * 1e3, 2),
            "apply_us": round(apply_avg * 1e3, 2),
            "prepare_share": round(prep_avg / (prep_avg + apply_avg), 4),
            # the pre-pass's HBM roofline: X and A read once, the workspace
            # (operand words, position fields, s, alpha T / s) written once
            "prepare_alg_bytes": prep_bytes,
            "prepare_frac_hbm": round(prep_bytes / (prep_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "sparsify_2of4_us": round(sp_ms * 1e3, 2),
            "sparsify_2of4_GBs": round(sp_bytes / (sp_ms * 1e-3) / 1e9, 1),
            "sparsify_2of4_frac_hbm": round(sp_bytes / (sp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "useful_tflops": round(useful_flops / (ms_step * 1e-3) / 1e12, 1),
            "step_us_per_call": dist(step_ms),
            "prepare_us_per_call": dist(prep_ms),
            "apply_us_per_call": dist(apply_ms),
            "r0_step_us": round(r0_ms * 1e3, 2),
            "r0_eff_tflops": round(flops_dense_eq / (r0_ms * 1e-3) / 1e12, 1),
            "r0_speedup_vs_inhouse_dense": round(dense_ms / r0_ms, 3),
            "r0_speedup_vs_hipblaslt": round(blas_ms / r0_ms, 3),
            "sparsify_over_sparse_linear": round(sp_ms / ms_step, 4),
            "unfused_r0_us": round(unf_ms * 1e3, 2),
            "compressed_gemm_us": round(comp_ms * 1e3, 2),
            "unfused_over_fused_r0": round(unf_ms / r0_ms, 4),
            "cold_step_us": cold_step,
            "cold_inhouse_dense_us": cold_dense,
            "cold_hipblaslt_us": cold_blas,
            "cold_speedup_vs_inhouse_dense": round(cold_dense["median"] / cold_step["median"], 3),
            "cold_speedup_vs_hipblaslt": round(cold_blas["median"] / cold_step["median"], 3),
            "wcold_step_us": wcold_step,
            "wcold_inhouse_dense_us": wcold_dense,
            "wcold_hipblaslt_us": wcold_blas,
            "wcold_speedup_vs_inhouse_dense": round(wcold_dense["median"] / wcold_step["median"], 3),
            "wcold_speedup_vs_hipblaslt": round(wcold_blas["median"] / wcold_step["median"], 3),
            "stream_w_cold_step_us": cold_stream_w,
            "stream_w_wcold_step_us": wcold_stream_w,
            "stream_w_warm_step_us": round(warm_stream_w_ms * 1e3, 2),
            "plain_warm_step_us_c": round(warm_plain_ms * 1e3, 2),
            "stream_w_cold_speedup_vs_hipblaslt": round(cold_blas["median"] / cold_stream_w["median"], 3),
            "stream_w_wcold_speedup_vs_hipblaslt": round(wcold_blas["median"] / wcold_stream_w["median"], 3),
            "sclk_mhz_observed": sclk_obs,
            "sclk_note": sclk_note,
            "frac_dense_peak_at_sclk": round(value / peak_at_sclk, 4) if peak_at_sclk else None,
            "apply_frac_peak_at_sclk": round(achieved / peak_at_sclk, 4) if peak_at_sclk else None,
            "cpu_context": cpu_ctx,
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
