"""Throughput of the fused W8A8 linear on one MI355X.

One step is the whole hot path for the full linear set of a 1024px DiT block
with classifier-free-guidance batch 2 (8192 tokens): for each of the QKV
(3072->9216), out (3072->3072), MLP-up (3072->12288) and MLP-down
(12288->3072) linears, per-token activation quantization of a bf16 input
followed by the fused int8 GEMM + dequant/bias epilogue that writes bf16.
Weights are quantized per output channel once, before timing (an offline
step of the method).  Inputs are seeded synthetic tensors already resident in
HBM.  `value` is int8 TOPS of the whole step: sum of 2*M*N*K over the four
linears / step time.

Besides the contract fields the JSON line carries the roofline of the
dominant kernel (the GEMM, timed per launch with HIP events on its stream;
with the matrix cores' ceiling on the step's own codes, and the fraction of
the peak scaled to the gfx clock read under load, since the package runs at
its power limit well below the nominal 2.4 GHz),
the CPU oracle timed on a bounded sample on the host, the quantize kernel's
HBM rate, cold-cache timings, the same linears through the dequantize-to-bf16
path the method replaces, a same-shape bf16 torch GEMM, and the GEMM rates
of the other workloads (768px attention projection and MLP pair, 1024px QKV
with outlier channels).

    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--no-cpu] [--no-cold]
                    [--no-other] [--copy-calibration]

From idle the GPU needs about 25 ms of continuous load before the step rate
settles (20 steps after a 5-step warm-up from idle ran about 8% below the
steady rate), so the comparators and variants run first and the headline
steps (their own warm-up, then the timed steps) follow on a GPU already
under load; with --only-step they follow the warm-up alone.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402

WORKLOAD = datagen.WORKLOADS[4]
MFMA_INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 matrix peak (5.0 POPS)
NOMINAL_SCLK_MHZ = 2400.0      # the clock that peak is quoted at
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "w8a8_int8_quantized_token_amd", "csrc", "gemm_i8.hip")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-rows", type=int, default=4096, help="tokens per linear in the CPU sample")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-cache GEMM / quantize timings")
    p.add_argument("--no-other", action="store_true", help="skip timing the other workloads' linears")
    p.add_argument("--only-step", action="store_true",
                   help="time the step only: no comparators, variants, cold or other workloads "
                        "(for profiler runs, whose GEMM dispatches must be the step's alone)")
    p.add_argument("--with-ceiling", action="store_true",
                   help="with --only-step: also run the matrix-core ceiling diagnostic after the "
                        "steps (a kernel of its own name, for counter runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain 1 GiB streaming copy 3 times (the reference kernel "
                        "for scaling HBM byte counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_traffic():
    """HBM bytes (read + write, calibrated) of the four GEMM launches of one
    step, measured with rocprofv3 counters, if they were taken on the current
    kernel source (else None)."""
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    digest = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if rec.get("gemm_source_sha256") != digest:
        return None
    return rec.get("bytes_per_step")


COPY_BYTES = 1 << 30


def copy_calibration(dev):
    """A plain streaming copy of known size (bitwise_not of 1 GiB of uint8:
    reads and writes COPY_BYTES each): its byte counters give the factor
    that turns counter readings into bytes."""
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


# A spin of about 1 ms queued ahead of each timed launch keeps the host's
# launch latency out of the events: the launch is in the queue before the GPU
# reaches the first event, as it is inside a stream of work.
SPIN_CYCLES = 2_000_000


def gpu_ms(fn, stream, n):
    """Median over n runs of the GPU time of fn()'s launches (HIP events on
    `stream`, with the queue kept busy ahead of the first event)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(n):
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def step_loop(layer_calls, stream, steps, warmup=10):
    """Run `steps` steps of a path the way the timed step runs the fused one:
    per linear, its launches back to back (layer_calls[i] = list of callables),
    one chain of HIP events per step (before the first launch and after
    each).  Returns (wall ms per step, mean ms of each linear's each launch)."""
    nl, nph = len(layer_calls), len(layer_calls[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nl * nph + 1)] for _ in range(steps)]
    for _ in range(warmup):
        for calls in layer_calls:
            for c in calls:
                c()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        for i, calls in enumerate(layer_calls):
            for j, c in enumerate(calls):
                c()
                ev[k][i * nph + j + 1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) / steps * 1e3
    ms = np.array([[[ev[k][i * nph + j].elapsed_time(ev[k][i * nph + j + 1]) for j in range(nph)]
                    for i in range(nl)] for k in range(steps)]).mean(axis=0)
    return wall_ms, ms


def power_cap_w() -> float | None:
    """The board's package power limit (`rocm-smi --showmaxpower`), or None."""
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower", "--json"], capture_output=True, text=True,
                           timeout=20)
        for card in json.loads(r.stdout).values():
            for k, v in card.items():
                if "power" in k.lower():
                    return float(v)
    except (OSError, ValueError, AttributeError, subprocess.SubprocessError):
        pass
    return None


def _smi_sample():
    """One `amd-smi metric --clock --power` reading: (mean gfx clock over the
    XCDs in MHz, socket power in W), or None."""
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--power", "--json"], capture_output=True,
                           text=True, timeout=20)
        if r.returncode != 0:
            return None
        data = json.loads(r.stdout)
        gpus = data["gpu_data"] if isinstance(data, dict) else data
        clk = gpus[0]["clock"]
        xcd = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_")]
        pw = gpus[0].get("power", {}).get("socket_power", {}).get("value")
        if not xcd or not isinstance(pw, (int, float)):
            return None
        return sum(xcd) / len(xcd), float(pw)
    except (OSError, ValueError, KeyError, IndexError, TypeError, AttributeError,
            subprocess.SubprocessError):
        return None


def at_clock(achieved: float, mhz) -> dict | None:
    """The int8 peak scaled to the gfx clock read under load, and `achieved`
    (TOPS) as a fraction of it: how much of the matrix cores' rate at the
    clock the package actually ran at the kernel reaches."""
    if not mhz:
        return None
    peak = MFMA_INT8_PEAK_TOPS * float(mhz) / NOMINAL_SCLK_MHZ
    return {"mhz": int(mhz), "peak": round(peak, 1), "frac": round(achieved / peak, 4),
            "note": "5.0 POPS x (median gfx clock read by amd-smi with the step loop running) / 2400 MHz"}


def loaded_samples(samples, t0: float, t1: float, cap: float | None) -> list:
    """(clock, power) of the readings (time, clock, power) taken between t0
    and t1 with socket power at or above half the package limit `cap` (any
    power when the limit is unknown)."""
    thresh = 0.5 * cap if cap else 0.0
    return [(c, w) for t, c, w in samples if t0 <= t <= t1 and w >= thresh]


def sample_sclk(step, ms_per_step: float, seconds: float = 4.0) -> dict | None:
    """Shader clock and socket power under the step loop.  A thread reads
    `amd-smi` over and over while the main thread keeps about `seconds` of
    steps queued; only readings taken while the load was on (socket power at
    or above half the package limit, and the last reading before the queue
    drained) are kept as loaded.  None if the tool is missing or fails."""
    import threading
    cap = power_cap_w()
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            v = _smi_sample()
            if v is None:
                break
            samples.append((time.perf_counter(), *v))

    n_steps = max(50, int(seconds * 1e3 / max(ms_per_step, 1e-3)))
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    for _ in range(n_steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stop.set()
    th.join(timeout=30)
    if not samples:
        return None
    loaded = loaded_samples(samples, t0, t1, cap)
    return {"loaded_mhz": [round(c) for c, _ in loaded], "loaded_w": [round(w) for _, w in loaded],
            "median_loaded_mhz": round(float(np.median([c for c, _ in loaded]))) if loaded else None,
            "all_mhz": [round(c) for _, c, _ in samples], "all_w": [round(w) for _, _, w in samples],
            "power_cap_w": cap, "load_s": round(t1 - t0, 2), "steps": n_steps,
            "source": "amd-smi metric --clock --power (mean over the XCDs' gfx clocks; socket power), "
                      "polled from a thread while the steps ran; loaded = socket power >= half the "
                      "package limit (rocm-smi --showmaxpower). Instantaneous readings, not averages."}


def mfma_ceiling(w8, L, stream, iters: int = 4000, launches: int = 5) -> dict:
    """The matrix cores' rate on this GPU for the GEMM's own inner loop and
    codes (w8a8_mfma_ceiling on the timed step's QKV activation and weight
    codes): `launches` back-to-back launches of about 4 ms each under the same
    sustained load as the steps; the median of the last three."""
    from w8a8_int8_quantized_token_amd.ops import CEILING_MFMAS_PER_ITER
    ops = CEILING_MFMAS_PER_ITER * iters * 65536
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
    ev[0].record(stream)
    for i in range(launches):
        w8.mfma_ceiling(L["xq"], L["wq"], iters)
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(launches - 3, launches))[1]
    tops = ops / ms / 1e9
    return {"tops": round(tops, 1), "frac_of_peak": round(tops / MFMA_INT8_PEAK_TOPS, 4),
            "kernel": "mfma_ceiling_kernel (the GEMM's K step on one LDS-resident stage, no memory "
                      "traffic, barriers or epilogue)",
            "codes": f"{L['shape'].name} activation and weight codes of the timed step"}


def time_cold(fn, stream, scrub, reps=5):
    """Median time of fn() with the caches flushed before each run (a 512 MB
    write between runs evicts L2 and the 256 MB Infinity Cache)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        scrub.zero_()
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_backend() -> str:
    """torch's BLAS backend for the bf16 comparator (on ROCm "Cublaslt" is hipBLASLt)."""
    b = str(torch.backends.cuda.preferred_blas_library()).split(".")[-1]
    return {"Cublaslt": "hipBLASLt", "Cublas": "rocBLAS"}.get(b, b)


def cpu_baseline(rows: int) -> dict:
    """The oracle, as it stands, on the first `rows` tokens of each linear."""
    import oracle
    ops = 0
    elapsed = 0.0
    for li, shape in enumerate(WORKLOAD.linears):
        x = datagen.gen_act(shape, WORKLOAD.seed, li, rows=np.arange(rows))
        w, b = datagen.gen_weight(shape, WORKLOAD.seed, li)
        wq, ws = oracle.quantize_rows_ref(w)            # offline, not timed
        oracle.int_gemm_ref(wq[:1], wq[:1])             # load the library outside the clock
        t0 = time.perf_counter()
        xq, xs = oracle.quantize_rows_ref(x)
        acc = oracle.int_gemm_ref(xq, wq)
        y = oracle.dequant_ref(acc, xs, ws, b)
        oracle.f32_to_bf16_bits(y)
        elapsed += time.perf_counter() - t0
        ops += 2 * rows * shape.N * shape.K
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": round(ops / elapsed / 1e12, 4), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"first {rows} of {WORKLOAD.linears[0].M} tokens of each of the 4 linears "
                      f"(full N and K), quantize + int32 GEMM + fp32 dequant + bf16; "
                      f"{ops / 1e9:.1f} G int8 ops in {elapsed:.1f} s"}


def time_other_workloads(w8, dev, stream, iters: int = 10) -> dict:
    """GEMM and quantize times of the other workloads' linears (the 768px
    attention projection and MLP pair, the 1024px QKV with outliers): median
    of `iters` launches each, HIP events on the launch stream.  The GEMM is
    timed as it runs inside a model: the caches scrubbed (the weights cold),
    then the activation quantized, then the GEMM (`gemm_us`); the same launch
    repeated with everything cache-resident is `gemm_warm_us`."""
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def med(fn):
        fn()
        torch.cuda.synchronize()
        return gpu_ms(fn, stream, iters)

    def med_cold(fn, prep):
        ts = []
        for _ in range(iters):
            scrub.zero_()
            prep()
            ts.append(gpu_ms(fn, stream, 1))
        return float(np.median(ts))

    out = {}
    for wl in datagen.WORKLOADS[1:4]:
        lin = []
        for li, shape in enumerate(wl.linears):
            if shape.act == "gelu_of_prev":   # timing only: any bf16 input of the shape
                x = datagen.random_bf16((shape.M, shape.K), wl.seed * 100 + li).to(dev)
            else:
                x = datagen.gen_act(shape, wl.seed, li).to(dev)
            wbf, b = datagen.gen_weight(shape, wl.seed, li)
            wq, ws = w8.quantize_weight(wbf.to(dev))
            b = b.to(dev)
            xq, xs = w8.quantize_act(x)
            y = torch.empty((shape.M, shape.N), dtype=torch.bfloat16, device=dev)
            feeds_gelu = li + 1 < len(wl.linears) and wl.linears[li + 1].act == "gelu_of_prev"
            gemm = lambda: w8.linear(xq, xs, wq, ws, b, y=y, gelu=feeds_gelu)
            g = med_cold(gemm, lambda: w8.quantize_act(x, xq, xs))
            g_warm = med(gemm)
            q = med(lambda: w8.quantize_act(x, xq, xs))
            ops = 2 * shape.M * shape.N * shape.K
            rec = {"linear": shape.name, "M": shape.M, "K": shape.K, "N": shape.N,
                   "plan": w8.select_tile(shape.M, shape.N, shape.K),
                   "gemm_us": round(g * 1e3, 2), "gemm_tops": round(ops / g / 1e9, 1),
                   "gemm_warm_us": round(g_warm * 1e3, 2), "quant_us": round(q * 1e3, 2)}
            if feeds_gelu:
                # the GELU before the next linear runs in this GEMM's epilogue; the
                # unfused alternative is the plain epilogue plus a separate GELU pass
                g0 = med(lambda: w8.linear(xq, xs, wq, ws, b, y=y))
                glue = med(lambda: torch.nn.functional.gelu(y))
                rec.update(gemm_gelu_epilogue_us=rec["gemm_warm_us"], gemm_plain_us=round(g0 * 1e3, 2),
                           separate_gelu_us=round(glue * 1e3, 2))
            lin.append(rec)
        g_us = sum(l["gemm_us"] for l in lin)
        q_us = sum(l["quant_us"] for l in lin)
        out[wl.name] = {"gemm_tops": round(wl.ops / g_us / 1e6, 1),
                        "frac": round(wl.ops / g_us / 1e6 / MFMA_INT8_PEAK_TOPS, 4),
                        "linear_tops": round(wl.ops / (g_us + q_us) / 1e6, 1), "linears": lin}
    del scrub
    return out


def time_fp8_variant(w8, layers, stream, steps: int) -> dict:
    """The same step with e4m3 codes (the fp8 variant): per linear, the fp8
    activation quantizer and the fp8 GEMM with the same epilogue, timed like
    the int8 step; weights quantized to e4m3 once, before timing."""
    fp = []
    for L in layers:
        cw, sw = w8.quantize_weight_fp8(L["wbf"])
        cx, sx = w8.quantize_act_fp8(L["x"])
        fp.append((cw, sw, cx, sx))
    calls = [[lambda L=L, f=f: w8.quantize_act_fp8(L["x"], f[2], f[3]),
              lambda L=L, f=f: w8.linear_fp8(f[2], f[3], f[0], f[1], L["b"], y=L["y"])]
             for L, f in zip(layers, fp)]
    wall_ms, ms = step_loop(calls, stream, steps)
    per, ops_tot = [], 0
    for L, (q, g) in zip(layers, ms):
        s = L["shape"]
        ops = 2 * s.M * s.N * s.K
        per.append({"linear": s.name, "gemm_us": round(g * 1e3, 2), "gemm_tops": round(ops / g / 1e9, 1),
                    "quant_us": round(q * 1e3, 2)})
        ops_tot += ops
    g_tot, q_tot = float(ms[:, 1].sum()), float(ms[:, 0].sum())
    del fp
    return {"value": round(ops_tot / wall_ms / 1e9, 1), "ms_per_step": round(wall_ms, 4),
            "gemm_tops": round(ops_tot / g_tot / 1e9, 1),
            "frac_of_fp8_peak": round(ops_tot / g_tot / 1e9 / MFMA_INT8_PEAK_TOPS, 4),
            "linear_tops": round(ops_tot / (g_tot + q_tot) / 1e9, 1), "per_linear": per,
            "note": "e4m3 codes, v_mfma_f32_32x32x64_f8f6f4, same tiles and epilogue; "
                    "MI355X dense fp8 peak = int8 peak = 5.0 P"}


def bf16_comparator(layers, per, stream, steps) -> tuple:
    """torch F.linear (hipBLASLt bf16) on the same shapes, run as a step like
    the fused one.  Returns (sum of per-linear mean ms, wall ms per step)."""
    calls = [[lambda L=L: torch.nn.functional.linear(L["x"], L["wbf"], L["b"])] for L in layers]
    wall_ms, ms = step_loop(calls, stream, steps)
    for p, t in zip(per, ms[:, 0]):
        p["bf16_us"] = round(float(t) * 1e3, 2)
    return float(ms[:, 0].sum()), wall_ms


def cold_timings(w8, layers, per, stream, dev, step_ops, q_bytes) -> dict:
    log("cold-cache timings")
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    g_sum = q_sum = 0.0
    for p, L in zip(per, layers):
        s = L["shape"]
        g = time_cold(lambda: w8.linear(L["xq"], L["xs"], L["wq"], L["ws"], L["b"], y=L["y"]), stream, scrub)
        q = time_cold(lambda: w8.quantize_act(L["x"], L["xq"], L["xs"]), stream, scrub)
        p["gemm_cold_us"] = round(g * 1e3, 2)
        p["quant_cold_us"] = round(q * 1e3, 2)
        p["quant_cold_gbs"] = round((3 * s.M * s.K + 4 * s.M) / q / 1e6, 1)
        g_sum += g
        q_sum += q
    del scrub
    return {"gemm_tops": round(step_ops / g_sum / 1e9, 1),
            "linear_tops": round(step_ops / (g_sum + q_sum) / 1e9, 1),
            "quant_gbs": round(q_bytes / q_sum / 1e6, 1),
            "note": "median of 5 runs per launch, 512 MB cache scrub before each"}


def slow_path(w8, layers, per, stream, steps) -> tuple:
    """The same linears through quantize -> dequantize to bf16 -> bf16 GEMM,
    run as a step.  Returns (sum of per-linear mean ms, wall ms per step)."""
    scratch = [{} for _ in layers]
    calls = [[lambda L=L, sc=sc: w8.dequant_bf16_linear(L["x"], L["wq"], L["ws"], L["b"], sc)]
             for L, sc in zip(layers, scratch)]
    wall_ms, ms = step_loop(calls, stream, steps)
    for p, t in zip(per, ms[:, 0]):
        p["dequant_bf16_us"] = round(float(t) * 1e3, 2)
    del scratch
    return float(ms[:, 0].sum()), wall_ms


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU; --gpus must be 1 "
                          "(the multi-GPU sharding is described in the design notes, not built)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    import w8a8_int8_quantized_token_amd as w8

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        log(f"copy calibration: 3 x {COPY_BYTES} B streaming copy")
        copy_calibration(dev)

    # ---- inputs, resident in HBM; weights quantized offline ----
    layers = []
    for li, shape in enumerate(WORKLOAD.linears):
        log(f"inputs {shape.name} M={shape.M} K={shape.K} N={shape.N}")
        x = datagen.gen_act(shape, WORKLOAD.seed, li).to(dev)
        wbf, b = datagen.gen_weight(shape, WORKLOAD.seed, li)
        wbf, b = wbf.to(dev), b.to(dev)
        wq, ws = w8.quantize_weight(wbf)
        xq = torch.empty((shape.M, shape.K), dtype=torch.int8, device=dev)
        xs = torch.empty((shape.M,), dtype=torch.float32, device=dev)
        y = torch.empty((shape.M, shape.N), dtype=torch.bfloat16, device=dev)
        layers.append(dict(shape=shape, x=x, wbf=wbf, b=b, wq=wq, ws=ws, xq=xq, xs=xs, y=y,
                           tile=w8.select_tile(shape.M, shape.N, shape.K)))
    torch.cuda.synchronize()
    step_ops = WORKLOAD.ops

    nl = len(layers)
    # one chain of events per step: before the first launch and after each
    # (launch 2i quantizes linear i, launch 2i+1 is its GEMM)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nl + 1)] for _ in range(args.steps)]

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        for i, L in enumerate(layers):
            w8.quantize_act(L["x"], L["xq"], L["xs"])
            if events is not None:
                events[2 * i + 1].record(stream)
            w8.linear(L["xq"], L["xs"], L["wq"], L["ws"], L["b"], y=L["y"])
            if events is not None:
                events[2 * i + 2].record(stream)

    extras = not args.only_step
    # ---- comparators and variants first: they also bring the GPU to a
    # steady loaded state (clocks and power management settle after tens of
    # ms of continuous load), so the headline steps below are not timed
    # from an idle GPU ----
    other = None
    if extras and not args.no_other:
        log("other workloads")
        other = time_other_workloads(w8, dev, stream)

    cold = None
    per_cold = [dict() for _ in layers]
    if extras and not args.no_cold:
        cold = cold_timings(w8, layers, per_cold, stream, dev, step_ops,
                            sum(3 * L["shape"].M * L["shape"].K + 4 * L["shape"].M for L in layers))

    bf_total = None
    per_bf = [dict() for _ in layers]
    if extras:
        log("bf16 comparator")
        bf_total, bf_wall = bf16_comparator(layers, per_bf, stream, args.steps)

    slow_total = None
    if extras:
        log("dequantize-to-bf16 comparator")
        slow_total, slow_wall = slow_path(w8, layers, per_bf, stream, args.steps)

    fp8 = None
    if extras:
        log("fp8 variant")
        fp8 = time_fp8_variant(w8, layers, stream, args.steps)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = step_ops * args.steps / elapsed / 1e12

    # per-launch kernel times from the events (the stream the kernels run on)
    q_ms = np.array([[ev[k][2 * i].elapsed_time(ev[k][2 * i + 1]) for i in range(nl)] for k in range(args.steps)])
    g_ms = np.array([[ev[k][2 * i + 1].elapsed_time(ev[k][2 * i + 2]) for i in range(nl)]
                     for k in range(args.steps)])
    per = []
    for i, L in enumerate(layers):
        s = L["shape"]
        ops = 2 * s.M * s.N * s.K
        gm = float(np.mean(g_ms[:, i]))
        qm = float(np.mean(q_ms[:, i]))
        per.append({"linear": s.name, "M": s.M, "K": s.K, "N": s.N, "tile": L["tile"],
                    "gemm_us": round(gm * 1e3, 2), "gemm_tops": round(ops / gm / 1e9, 1),
                    "quant_us": round(qm * 1e3, 2),
                    "quant_gbs": round((3 * s.M * s.K + 4 * s.M) / qm / 1e6, 1),
                    "linear_tops": round(ops / (gm + qm) / 1e9, 1)})
    gemm_total_ms = float(g_ms.mean(axis=0).sum())
    gemm_tops = step_ops / gemm_total_ms / 1e9
    q_bytes = sum(3 * L["shape"].M * L["shape"].K + 4 * L["shape"].M for L in layers)
    q_total_ms = float(q_ms.mean(axis=0).sum())

    for p, pc, pb in zip(per, per_cold, per_bf):
        p.update(pc)
        p.update(pb)
    ceiling = mfma_ceiling(w8, layers[0], stream) if extras or args.with_ceiling else None
    sclk = sample_sclk(step, ms_per_step) if extras else None

    traffic = gemm_traffic()
    alg_bytes = sum(L["shape"].M * L["shape"].K + L["shape"].N * L["shape"].K
                    + 2 * L["shape"].M * L["shape"].N + 4 * L["shape"].M + 4 * L["shape"].N
                    + 2 * L["shape"].N for L in layers)
    roofline = {"bound": "mfma", "kernel": "gemm_i8_kernel (fused W8A8 linear)",
                "achieved": round(gemm_tops, 1), "peak": MFMA_INT8_PEAK_TOPS, "unit": "TOPS",
                "frac": round(gemm_tops / MFMA_INT8_PEAK_TOPS, 4), "traffic": traffic,
                "algorithmic_bytes": alg_bytes,
                "ceiling": None if ceiling is None else dict(
                    ceiling, frac_of_ceiling=round(gemm_tops / ceiling["tops"], 4)),
                "at_loaded_clock": at_clock(gemm_tops, (sclk or {}).get("median_loaded_mhz")),
                "per_launch": "sum of 2MNK over the four GEMM launches / sum of their mean durations; "
                              "traffic and algorithmic_bytes are summed over the same four launches"}

    result = {
        "metric": "fused W8A8 linear int8 TOPS and % of MI355X int8 MFMA peak; speedup vs bf16",
        "value": round(value, 1),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD.name, "tokens": WORKLOAD.linears[0].M,
                   "linears": [f"{L['shape'].name} {L['shape'].K}->{L['shape'].N}" for L in layers],
                   "ops_per_step": step_ops, "weights": "pre-quantized per output channel",
                   "inputs": "bf16 N(0,1) activations, N(0,0.02) weights, N(0,0.01) bias, seed 4"},
        "frac_of_peak": round(value / MFMA_INT8_PEAK_TOPS, 4),
        "roofline": roofline,
        "quantize": {"bound": "hbm", "achieved": round(q_bytes / q_total_ms / 1e6, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(q_bytes / q_total_ms / 1e6 / HBM_PEAK_GBS, 4)},
        "cold": cold,
        "sclk": sclk,
        "other_workloads": other,
        "fp8_variant": fp8,
        "vs_dequant_bf16_path": None if slow_total is None else {
            "tops": round(step_ops / slow_total / 1e9, 1),
            "speedup_full_linear": round(slow_total / (gemm_total_ms + q_total_ms), 3),
            "step_ms": round(slow_wall, 4), "speedup_step": round(slow_wall / ms_per_step, 3),
            "path": "quantize_act + dequantize X and W to bf16 + torch F.linear"},
        "vs_bf16": None if bf_total is None else {
            "bf16_torch_linear_tops": round(step_ops / bf_total / 1e9, 1),
            "step_ms": round(bf_wall, 4), "speedup_step": round(bf_wall / ms_per_step, 3),
            "speedup_full_linear": round(bf_total / (gemm_total_ms + q_total_ms), 3),
            "speedup_gemm_only": round(bf_total / gemm_total_ms, 3),
            "blas_backend": blas_backend()},
        "per_linear": per,
    }
    if not args.no_cpu:
        log(f"cpu oracle baseline on {args.cpu_rows} tokens per linear")
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
