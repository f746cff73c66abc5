"""Benchmark of the Wan DiT attention forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu]
python bench.py --backward-only NAME | --linear-only NAME | --vsa-only NAME   (one path alone, for profiling)
python bench.py --mfma-ceiling   (sustained matrix-core rate of each MFMA instruction, the practical ceiling)

One step = one call of the C ABI's wan_attn_fwd on the workload's full shape, inputs already in
HBM.  Prints ONE JSON line: the headline is the bf16 self-attention of the Wan-14B-shaped 720p,
81-frame sequence (b=2 for cond/uncond, 40 heads, 75,600 tokens, head_dim 128), in TFLOP/s
counted as 4*b*heads*s_q*s_kv*head_dim; "configs" adds every other workload (480p frame,
Wan-1.3B 480p, text cross-attention, the 8-bit path at the 720p shape) measured the same way, and
the bf16 attention backward (dQ, dK, dV from the forward's output and row log-sum-exp) at the
Wan-1.3B 480p and Wan-14B 720p shapes, in TFLOP/s counted as 8*b*heads*s_q*s_kv*head_dim, and the
FP8 GEMM of the DiT linear layers (per-token activation quantisation + GEMM, the weights quantised
once beforehand) at the Wan-14B and Wan-1.3B width-preserving projections, in TFLOP/s counted as
2*m*n*k against the 5.0 PFLOP/s dense fp8 peak, and the block-sparse (VSA-style) attention at the
Wan-1.3B 16x28x52 and Wan-14B 720p shapes (87.5% of the 64-token key blocks dropped), in TFLOP/s of
the attended keys, with its speed-up over the dense forward at the same shape.  "roofline" is for the dominant kernel, "cpu_baseline" times the plain fp64 CPU oracle on a
bounded sample of query rows of the same workload.
"""

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import threading
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "attention fwd TFLOP/s and % of MFMA peak at Wan 480p/720p token lengths"
HEADLINE = "wan14b_720p81f_self"
PEAK_TFLOPS = {"bf16": 2500.0, "int8_fp8": 5000.0}     # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0
NOMINAL_MHZ = 2400.0           # the clock the dense peaks are quoted at
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "bf16": ["attn_bf16.hip"],
    "int8_fp8": ["attn8_fwd.hip"],
}


def source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(HERE, "video_diffusion_transformer_wan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class ClockSampler:
    """Samples the GPU's current shader clock in a background thread while a timed region runs; the
    median of the samples is the clock the chip held there.  It reads the driver's pp_dpm_sclk file
    (the level marked '*' is the current clock) of the one GPU in sysfs -- no process is started.
    summary() is None when there is no such single file or fewer than 3 samples landed after the first
    (regions shorter than about 40 ms)."""

    def __init__(self, period_s=0.01):
        self.period_s = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = files[0] if len(files) == 1 else None

    def read_mhz(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*mhz", line, flags=re.I)
                        return int(m.group(1)) if m else None
        except (OSError, TypeError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self.read_mhz()
            if v:
                self.samples.append(v)
            self._stop.wait(self.period_s)

    def __enter__(self):
        if self.path is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=5)

    def summary(self):
        # the first sample can predate the first launch (the idle clock): dropped; a region with fewer
        # than 3 samples after it reports no clock
        kept = self.samples[1:]
        if len(kept) < 3:
            return None
        return {"median_mhz": statistics.median(kept), "min_mhz": min(kept),
                "max_mhz": max(kept), "samples": len(kept), "source": self.path}


def at_clock(frac, clock):
    """Fraction of the peak scaled to the measured clock (the peak at that clock instead of 2.4 GHz)."""
    if clock is None or frac is None:
        return None
    return frac * NOMINAL_MHZ / clock["median_mhz"]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_traffic(kind, workload):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if they were taken
    on the kernel source as it is now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kind}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kind):
        return None
    return rec.get("bytes_per_launch")


# Untimed warm-up of the workloads other than the headline, in ms of GPU work: the first ≈20 ms of
# sustained matrix-core work in a process run up to ≈30% slower (a GEMM sequence measured 1.70, 2.13,
# 2.03, 1.84 ... 1.71 ms per call before settling at ≈1.60 ms, whatever kernel preceded it), so a
# workload timed over a few ms right after a lighter one would report that transient, not its
# sustained rate.  The headline keeps exactly its `--warmup` steps.
SECONDARY_WARM_MS = 100.0


def time_calls(fn, steps, warmup, stream, clock=None, min_warm_ms=0.0):
    """Mean ms per call over `steps` calls after `warmup`; `clock`, if given, is a ClockSampler run
    across the timed region.  With `min_warm_ms`, the untimed warm-up continues (at most 2,000 more
    calls) until that much GPU time has passed."""
    import contextlib
    import math
    import torch
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(warmup):
        fn()
    w1.record(stream)
    torch.cuda.synchronize()
    spent = w0.elapsed_time(w1)
    if warmup > 0 and spent < min_warm_ms:
        per = max(spent / warmup, 1e-3)
        for _ in range(min(2000, int(math.ceil((min_warm_ms - spent) / per)))):
            fn()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with (clock if clock is not None else contextlib.nullcontext()):
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def step_stats(fn, steps, stream):
    """Median and minimum of `steps` individually timed calls (HIP events on `stream`), in ms; run after
    the timed region, which they do not change."""
    import statistics
    import torch
    times = []
    for _ in range(max(1, steps)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b))
    return statistics.median(times), min(times)


def cpu_baseline(w, q, k, v, budget_s=12.0, single_budget_s=None, all_rows=False):
    """The oracle as it stands, on a bounded sample of seeded query rows of the workload (every row
    when `all_rows`): with every BLAS thread, then (a smaller budget) with one."""
    res = _cpu_baseline_run(w, q, k, v, budget_s, all_rows)
    res["cpu_model"] = cpu_model()
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = _cpu_baseline_run(w, q, k, v, budget_s / 3 if single_budget_s is None else single_budget_s, all_rows)
        res["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"],
                                "seconds": one["seconds"]}
    except Exception as e:  # report, do not hide the baseline
        res["single_thread"] = {"error": str(e)}
    return res


def _cpu_baseline_run(w, q, k, v, budget_s, all_rows=False):
    import numpy as np
    import oracle
    import wan_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    if all_rows:
        rows_all = np.array([[bb, hh, i] for bb in range(w.batch) for hh in range(w.heads) for i in range(w.s_q)])
    else:
        rows_all = wan_inputs.sample_rows(w, 4096).numpy()
    # host copies of the heads the sample touches, converted exactly from bf16
    def host(t, bh):
        return {p: t[p[0], :, p[1], :].float().cpu().numpy() for p in bh}
    n = 8
    done_rows, elapsed = 0, 0.0
    while True:
        sel = rows_all[done_rows:done_rows + n]
        if len(sel) == 0:
            break
        bh = sorted({(int(r[0]), int(r[1])) for r in sel})
        qh, kh, vh = host(q, bh), host(k, bh), host(v, bh)
        t0 = time.perf_counter()
        for (bb, hh) in bh:
            idx = sel[(sel[:, 0] == bb) & (sel[:, 1] == hh)][:, 2]
            # [1, s, 1, d] views so that the oracle sees its usual layout
            oracle.attention_rows(qh[(bb, hh)][None, :, None, :], kh[(bb, hh)][None, :, None, :],
                                  vh[(bb, hh)][None, :, None, :],
                                  np.stack([np.zeros_like(idx), np.zeros_like(idx), idx], 1))
        elapsed += time.perf_counter() - t0
        done_rows += len(sel)
        if elapsed >= budget_s or done_rows >= len(rows_all):
            break
        n = min(len(rows_all) - done_rows, max(8, int(n * 2)))
    flops = 4 * done_rows * w.s_kv * w.head_dim
    total_rows = w.batch * w.heads * w.s_q
    what = "every query row" if all_rows and done_rows == total_rows else f"{done_rows} seeded query rows"
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{what} of {w.name} (fp64 two-pass oracle, "
                      f"{done_rows / elapsed:.2f} rows/s; full workload extrapolates to "
                      f"{total_rows / (done_rows / elapsed):.1f} s)",
            "rows": int(done_rows), "seconds": round(elapsed, 2),
            "full_workload_s": round(total_rows / (done_rows / elapsed), 1)}


CEILING_KINDS = [  # (kind, instruction, operations per wave-iteration, dense peak in TFLOP/s at 2.4 GHz)
    (0, "v_mfma_f32_32x32x16_bf16", 8 * 32768, 2500.0),
    (1, "v_mfma_f32_16x16x32_bf16", 16 * 16384, 2500.0),
    (2, "v_mfma_f32_32x32x64_f8f6f4 (e4m3)", 8 * 131072, 5000.0),
    (3, "v_mfma_i32_32x32x32_i8", 8 * 65536, 5000.0),
    (4, "v_mfma_f32_16x16x128_f8f6f4 (e4m3)", 16 * 65536, 5000.0),
    (5, "v_mfma_i32_16x16x64_i8", 16 * 32768, 5000.0),
]


def run_mfma_ceiling(target_ms=150.0, launches=5):
    """Sustained matrix-core rate: one wave per SIMD on every compute unit streaming independent MFMAs
    with operands from registers (random bf16 / e4m3 / int8 bit patterns that change between
    instructions), each launch about target_ms long so that the chip settles at the clock its power
    limit gives that load; HIP events on the launch stream, the shader clock sampled meanwhile."""
    import ctypes
    import torch
    from video_diffusion_transformer_wan_amd import build as wan_build
    if not os.path.exists(wan_build.CEILING_LIB):
        raise RuntimeError(f"{wan_build.CEILING_LIB} is not built (python -m video_diffusion_transformer_wan_amd.build)")
    lib = ctypes.CDLL(wan_build.CEILING_LIB)
    lib.wan_mfma_ceiling_run.restype = ctypes.c_int
    lib.wan_mfma_ceiling_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    n_wg = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cpu").manual_seed(7)
    out = torch.empty(n_wg * 4, dtype=torch.float32, device="cuda")
    res = {"workgroups": n_wg, "waves_per_simd": 1, "launch_ms_target": target_ms, "kinds": []}
    for kind, name, ops, peak in CEILING_KINDS:
        if kind in (0, 1):      # N(0,1) bf16 values
            src = torch.randn(64 * 8 * 16, generator=g).to(torch.bfloat16).view(torch.uint8)
        elif kind in (2, 4):    # N(0,1) e4m3 values (finite codes)
            src = torch.randn(64 * 8 * 32, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
        else:                   # uniform int8
            src = torch.randint(-127, 128, (64 * 8 * 32,), generator=g, dtype=torch.int8).view(torch.uint8)
        src = src.to("cuda")

        def launch(iters):
            rc = lib.wan_mfma_ceiling_run(kind, src.data_ptr(), out.data_ptr(), n_wg, iters, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"wan_mfma_ceiling_run returned {rc}")
        probe_iters = 20000
        ms = time_calls(lambda: launch(probe_iters), 1, 1, stream)
        iters = int(min(2 ** 30, max(probe_iters, probe_iters * target_ms / ms)))
        clock = ClockSampler()
        ms = time_calls(lambda: launch(iters), launches, 1, stream, clock=clock)
        flops = n_wg * 4 * iters * ops
        tf = flops / (ms * 1e-3) / 1e12
        clk = clock.summary()
        res["kinds"].append({"instruction": name, "iters": iters, "ms": round(ms, 3), "tflops": round(tf, 1),
                             "frac_of_peak": round(tf / peak, 4), "clock": clk,
                             "frac_at_measured_clock": at_clock(tf / peak, clk)})
        print(json.dumps(res["kinds"][-1]), flush=True)
    return res


def run_workload(name, steps, warmup, cpu_budget_s=0.0, min_warm_ms=0.0):
    import torch
    import video_diffusion_transformer_wan_amd as wan
    import wan_inputs
    w = wan_inputs.WORKLOADS[name]
    q, k, v = wan_inputs.make_qkv(w, device="cuda")
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    fn = lambda: wan.wan_attn_fwd(q, k, v, out, w.batch, w.heads, w.s_q, w.s_kv, w.head_dim, w.path,
                                  stream)
    clock = ClockSampler()
    ms = time_calls(fn, steps, warmup, stream, clock, min_warm_ms)
    med, mn = step_stats(fn, steps, stream)
    res = {"workload": name, "path": w.path, "ms": ms, "tflops": w.flops / (ms * 1e-3) / 1e12,
           "ms_median": med, "ms_min": mn}
    res["frac_of_peak"] = res["tflops"] / PEAK_TFLOPS[w.path]
    res["clock"] = clock.summary()
    res["frac_of_peak_at_measured_clock"] = at_clock(res["frac_of_peak"], res["clock"])
    kernel_ms = ms
    if w.path == "int8_fp8":
        # the attention kernel alone, from pre-quantised operands
        z = wan.attention8_quantize(q, k, v)
        fk = lambda: wan.attention8_from_quantized(z, w.batch, w.heads, w.s_q, w.s_kv, out=out)
        kernel_ms = time_calls(fk, steps, max(1, warmup), stream, min_warm_ms=min_warm_ms)
        res["kernel_ms"] = kernel_ms
        res["kernel_tflops"] = w.flops / (kernel_ms * 1e-3) / 1e12
        res["kernel_frac_of_peak"] = res["kernel_tflops"] / PEAK_TFLOPS[w.path]
        res["kernel_frac_of_peak_at_measured_clock"] = at_clock(res["kernel_frac_of_peak"], res["clock"])
        # the softmax's VALU floor (measured per-instruction costs beside a busy matrix core, per
        # 64-key tile and wave: 32 v_fma_f32 x 7.5 + 32 v_exp_f32 x 13.2 + 16 v_cvt_pk_fp8_f32 x 12.6 +
        # 16 v_max3_f32 x 8.6 + 12 others x 8 cycles), at the measured clock
        if res["clock"] is not None:
            cyc = 32 * 7.5 + 32 * 13.2 + 16 * 12.6 + 16 * 8.6 + 12 * 8
            wave_tiles = w.batch * w.heads * w.s_q * w.s_kv / (32 * 64)
            res["valu_floor_ms"] = wave_tiles / 1024 * cyc / (res["clock"]["median_mhz"] * 1e6) * 1e3
        del z
    if cpu_budget_s > 0:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, cpu_budget_s, cpu_budget_s / 2,
                                           all_rows=w.batch * w.heads * w.s_q <= 4096)
    return w, (q, k, v), res, kernel_ms


def run_backward(name, steps, warmup, min_warm_ms=SECONDARY_WARM_MS):
    """The bf16 backward at a workload's shape: one step = one wan_attn_bwd call (the forward that
    produces o and lse runs once, before the timed region)."""
    import torch
    import video_diffusion_transformer_wan_amd as wan
    import wan_inputs
    w = wan_inputs.WORKLOADS[name]
    q, k, v = wan_inputs.make_qkv(w, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(w.seed + 11)
    d_o = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o, lse = wan.attention_with_lse(q, k, v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()
    fn = lambda: wan.wan_attn_bwd(q, k, v, o, d_o, lse, dq, dk, dv, w.batch, w.heads, w.s_q, w.s_kv,
                                  w.head_dim, stream)
    ms = time_calls(fn, steps, warmup, stream, min_warm_ms=min_warm_ms)
    flops = 2.0 * w.flops   # the pages' beta = 8 against the forward's 4
    return {"workload": name, "path": "bf16 backward", "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "frac_of_peak": flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
            "mfma_tflops": 3.5 * w.flops / (ms * 1e-3) / 1e12}


def run_linear(name, steps, warmup, min_warm_ms=SECONDARY_WARM_MS):
    """The FP8 linear at a projection shape: one step = per-token quantisation of x plus the GEMM
    (wan_fp8_quantize_rows + wan_fp8_gemm); the weight is quantised once, before the timed region.
    The GEMM alone is timed as well."""
    import torch
    import video_diffusion_transformer_wan_amd as wan
    import wan_inputs
    w = wan_inputs.LINEAR_WORKLOADS[name]
    x, wt = wan_inputs.make_linear(w, device="cuda")
    wc, ws = wan.fp8_quantize_tensor(wt)
    xc = torch.empty((w.m, w.k), dtype=torch.uint8, device="cuda")
    xs = torch.empty((w.m,), dtype=torch.float32, device="cuda")
    y = torch.empty((w.m, w.n), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        wan.wan_fp8_quantize_rows(x, w.m, w.k, xc, xs, stream)
        wan.wan_fp8_gemm(xc, xs, wc, ws, y, w.m, w.n, w.k, stream)

    ms = time_calls(step, steps, warmup, stream, min_warm_ms=min_warm_ms)
    gemm_ms = time_calls(lambda: wan.wan_fp8_gemm(xc, xs, wc, ws, y, w.m, w.n, w.k, stream), steps, warmup, stream,
                         min_warm_ms=min_warm_ms)
    tf = w.flops / (ms * 1e-3) / 1e12
    gtf = w.flops / (gemm_ms * 1e-3) / 1e12
    return {"workload": name, "path": "fp8 linear", "m": w.m, "n": w.n, "k": w.k, "ms": ms, "tflops": tf,
            "frac_of_peak": tf / PEAK_TFLOPS["int8_fp8"], "gemm_ms": gemm_ms, "gemm_tflops": gtf,
            "gemm_frac_of_peak": gtf / PEAK_TFLOPS["int8_fp8"]}


def run_vsa(name, steps, warmup, min_warm_ms=SECONDARY_WARM_MS):
    """Block-sparse (VSA-style) attention at a Wan shape: one step = the coarse stage (block means,
    scores, top-keep selection) plus the fine block-sparse attention (wan_vsa_select + wan_vsa_attn).
    The fine stage alone, the coarse stage alone and the dense bf16 forward at the same shape are
    timed as well.  TFLOP/s count 4 * d * (query rows x attended keys) of the selection made."""
    import torch
    import video_diffusion_transformer_wan_amd as wan
    import wan_inputs
    w = wan_inputs.VSA_WORKLOADS[name]
    q, k, v = wan_inputs.make_vsa(w, device="cuda")
    b, H, s = w.batch, w.heads, w.s
    n_qb = -(-s // 64)
    idx = torch.empty((b, H, n_qb, w.keep), dtype=torch.int32, device="cuda")
    scratch = torch.empty(wan.wan_vsa_select_scratch_bytes(b, H, s, s) // 4, dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    d = wan_inputs.HEAD_DIM

    def coarse():
        wan.wan_vsa_select(q, k, b, H, s, s, d, w.keep, idx, scratch, stream)

    def fine():
        wan.wan_vsa_attn(q, k, v, idx, o, b, H, s, s, d, w.keep, stream)

    def both():
        coarse()
        fine()

    ms = time_calls(both, steps, warmup, stream, min_warm_ms=min_warm_ms)
    fine_ms = time_calls(fine, steps, warmup, stream, min_warm_ms=min_warm_ms)
    coarse_ms = time_calls(coarse, steps, warmup, stream, min_warm_ms=min_warm_ms)
    dense_ms = time_calls(lambda: wan.wan_attn_fwd(q, k, v, o, b, H, s, s, d, wan.WAN_ATTN_BF16, stream),
                          max(2, steps // 2), 1, stream, min_warm_ms=min_warm_ms)
    both()
    keys = torch.clamp(s - 64 * idx.long(), max=64).sum(dim=-1)                  # [b, H, n_qb]
    rows = torch.clamp(s - 64 * torch.arange(n_qb, device="cuda"), max=64)      # [n_qb]
    flops = float(4 * d * (keys * rows).sum().item())
    gathered = float(keys.sum().item()) * 2 * d * 2    # K and V rows of the attended keys, per query block
    tf = flops / (ms * 1e-3) / 1e12
    ftf = flops / (fine_ms * 1e-3) / 1e12
    return {"workload": name, "path": "vsa block-sparse bf16", "batch": b, "heads": H, "s": s, "keep": w.keep,
            "sparsity": 1.0 - w.keep / -(-s // 64), "ms": ms, "tflops": tf, "fine_ms": fine_ms,
            "fine_tflops": ftf, "fine_frac_of_peak": ftf / PEAK_TFLOPS["bf16"], "coarse_ms": coarse_ms,
            "dense_ms": dense_ms, "speedup_vs_dense": dense_ms / ms, "fine_speedup_vs_dense": dense_ms / fine_ms,
            "flops": flops, "gathered_bytes": gathered, "gather_tbps": gathered / (fine_ms * 1e-3) / 1e12,
            "fine_hbm": vsa_fine_hbm(name, fine_ms)}


def vsa_fine_hbm(name, fine_ms):
    """The fine stage against the HBM roofline it is bound by: the bytes it fetches from beyond L2 per
    launch (rocprofv3 FETCH_SIZE, scaled by the copy calibration; profiles/traffic.json, used only while
    vsa.hip is the source the counters were taken on) over its time, against 8 TB/s."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"vsa_fine:{name}")
    except (OSError, ValueError):
        return None
    h = hashlib.sha256(open(os.path.join(HERE, "video_diffusion_transformer_wan_amd", "csrc", "vsa.hip"), "rb").read())
    if not rec or rec.get("source_hash") != h.hexdigest()[:16]:
        return None
    gbs = rec["fetch_bytes"] / (fine_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": rec["fetch_bytes"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--backward-only", default=None, metavar="WORKLOAD",
                    help="only time the bf16 backward at this workload's shape (for profiling)")
    ap.add_argument("--linear-only", default=None, metavar="WORKLOAD",
                    help="only time the FP8 linear at this projection shape (for profiling)")
    ap.add_argument("--vsa-only", default=None, metavar="WORKLOAD",
                    help="only time the block-sparse attention at this shape (for profiling)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the sustained matrix-core rate of each MFMA instruction the kernels use")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "context-parallel path is not built", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_mib:
        # a plain copy of known size: reads and writes exactly copy_mib MiB per dispatch
        x = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(max(1, args.steps)):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mib, "dispatches": max(1, args.steps)}), flush=True)
        return
    if args.mfma_ceiling:
        print(json.dumps(run_mfma_ceiling()), flush=True)
        return
    if args.backward_only or args.linear_only or args.vsa_only:
        res = (run_backward(args.backward_only, args.steps, args.warmup) if args.backward_only
               else run_linear(args.linear_only, args.steps, args.warmup) if args.linear_only
               else run_vsa(args.vsa_only, args.steps, args.warmup))
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in res.items()}), flush=True)
        return
    import video_diffusion_transformer_wan_amd as wan
    import wan_inputs
    if not os.path.exists(wan.LIB_PATH):
        from video_diffusion_transformer_wan_amd import build
        build.build()
    wan.lib()

    w, qkv, head, kernel_ms = run_workload(args.workload, args.steps, args.warmup)
    clock = head.get("clock")
    flops = w.flops
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    # secondary ceiling: one exponential per score, at the v_exp_f32 rate measured on gfx950 (28.4 lane
    # results per clock per CU), 256 CUs at the nominal 2.4 GHz
    exps = w.batch * w.heads * w.s_q * w.s_kv
    exp_ms = exps / (28.4 * 256 * 2.4e9) * 1e3
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[w.path],
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[w.path], 4),
            "traffic": measured_traffic(w.path, w.name),
            "clock": clock, "frac_at_measured_clock": at_clock(achieved / PEAK_TFLOPS[w.path], clock),
            "kernel": "attn_fwd_bf16_kernel" if w.path == "bf16" else "attn8_fwd_kernel",
            "flops_per_launch": flops,
            "exp_ceiling": {"exps_per_launch": exps, "ms_at_exp_rate": round(exp_ms, 3),
                            "mfma_ms_at_peak": round(flops / (PEAK_TFLOPS[w.path] * 1e12) * 1e3, 3)}}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, *qkv)
    del qkv
    torch.cuda.empty_cache()

    configs = {w.name: head}
    if not args.no_extra:
        for name in wan_inputs.WORKLOADS:
            if name == w.name:
                continue
            small = wan_inputs.WORKLOADS[name].flops < 1e13
            try:
                _, _, res, _ = run_workload(name, args.steps * (10 if small else 1),
                                            args.warmup * (5 if small else 1),
                                            cpu_budget_s=0.0 if args.no_cpu else 3.0,
                                            min_warm_ms=SECONDARY_WARM_MS)
            except Exception as e:  # report, do not hide the headline
                res = {"workload": name, "error": str(e)}
            configs[name] = res
            torch.cuda.empty_cache()
        for name in ("wan1.3b_480p81f_self", HEADLINE):
            try:
                small = wan_inputs.WORKLOADS[name].flops < 1e13
                res = run_backward(name, max(2, args.steps // 2) * (5 if small else 1), 1)
            except Exception as e:
                res = {"workload": name, "error": str(e)}
            configs[name + ":backward"] = res
            torch.cuda.empty_cache()
        for name in wan_inputs.LINEAR_WORKLOADS:
            try:
                res = run_linear(name, args.steps, args.warmup)
            except Exception as e:
                res = {"workload": name, "error": str(e)}
            configs[name] = res
            torch.cuda.empty_cache()
        for name in wan_inputs.VSA_WORKLOADS:
            try:
                res = run_vsa(name, args.steps, args.warmup)
            except Exception as e:
                res = {"workload": name, "error": str(e)}
            configs[name] = res
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.path == "bf16" else "int8/fp8",
        "data": "synthetic (seeded N(0,1) Q/K/V in bf16 at Wan token lengths; no weights needed)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "s_q": w.s_q,
                   "s_kv": w.s_kv, "head_dim": w.head_dim, "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(head["frac_of_peak"], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                    for k, r in configs.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
