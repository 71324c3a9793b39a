#!/usr/bin/env python3
"""Benchmark of the int4 GPTQ small-M products on one MI355X.

A step is one pass over the small-M workload: Y = X . W^T with GPTQ int4
weights (group 128) for (k, n) in {(4096, 4096), (2048, 8192)} and m in
{1, 8, 15} tokens -- six calls through the C ABI, each taking its dispatch
path (GEMV for m = 1, the fused small-M kernel otherwise).

Inputs are resident in HBM before timing starts.  In the default cold regime
every call reads a different copy of its weights, rotating through enough
copies (>= 512 MiB per shape, twice the 256 MB Infinity Cache) that the
weights stream from HBM; --regime warm reuses one copy (cache-resident).

Prints ONE JSON line: effective GB/s over the whole step (algorithmic bytes /
time), per-call microseconds and GB/s, the roofline of the dominant kernel
measured live with HIP events on the launch stream, the rest of the metric
per call (``configs``: the int4 prefill and large-weight shapes, the bf16 dense
training trio), and the CPU oracle timed on a bounded sample of the same
workload.  ``--suite FILE`` also times every int4 and dense workload shape and
writes them to FILE.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qgemm µs & eff. HBM GB/s at m=1/8; TFLOPS (% MFMA peak) at m>=512"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X published dense fp32 (matrix and vector)
LLC_BYTES = 256 << 20
# HBM traffic of the small-M kernels, measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
# and scaled by the same counters on a copy of known size; valid only while the
# kernel sources hash to the value recorded with the counters.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "skinny_lds_small_m_traffic.md")
KERNEL_SOURCES = ["int4_weight_only_gptq_amd/csrc/int4_kernels.hip",
                  "int4_weight_only_gptq_amd/csrc/common.hpp",
                  "int4_weight_only_gptq_amd/csrc/launch.hpp",
                  "int4_weight_only_gptq_amd/build.py"]

SMALL_M = [(4096, 4096), (2048, 8192)]
SMALL_M_TOKENS = [1, 8, 15]


def int4_bytes(m, k, n, zeros=True):
    """Algorithmic bytes of one int4 call: every tensor touched once."""
    g = k // 128
    return k * n // 2 + g * n * 2 + (g * n // 2 if zeros else 0) + 2 * m * k + 2 * m * n


def dense_bytes(M, N, K):
    return 2 * (M * K + N * K + M * N)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--regime", choices=["cold", "warm"], default="cold")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="wall time budget of the CPU oracle sample (0 disables)")
    p.add_argument("--suite", default=None, help="also time all workload shapes into this JSON file")
    p.add_argument("--suite-kinds", default="int4,int4_nozero,dense,int4_lora,dense_fp32,attention",
                   help="comma-separated row kinds the suite times")
    return p.parse_args()


class Int4Case:
    """One int4 product with `copies` resident copies of its weights."""

    def __init__(self, qg, torch, m, k, n, seed, copies, zeros=True):
        from qgemm_inputs import int4_inputs
        import numpy as np

        self.m, self.k, self.n = m, k, n
        d = int4_inputs(m, k, n, seed=seed)
        self.host = d
        dev = torch.device("cuda")
        self.x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        qw = torch.from_numpy(d["qweight"].view(np.int32)).to(dev)
        sc = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
        qz = torch.from_numpy(d["qzeros"].view(np.int32)).to(dev) if zeros else None
        self.w = [(qw, sc, qz)] + [(qw.clone(), sc.clone(), None if qz is None else qz.clone())
                                   for _ in range(copies - 1)]
        self.y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        self.i = 0
        self.qg = qg
        self.kernel = qg.describe_int4(m, n, k).split(" ")[0]
        self.bytes = int4_bytes(m, k, n, zeros)
        self.flops = 2 * m * n * k

    def launch(self, path="auto"):
        qw, sc, qz = self.w[self.i % len(self.w)]
        self.i += 1
        self.qg.qgemm_int4(self.x, qw, sc, qz, out=self.y, path=path)


def copies_for(bytes_per_copy, regime):
    if regime == "warm":
        return 1
    return max(2, -(-2 * LLC_BYTES // bytes_per_copy))


WARM_S = 0.03   # untimed replays (or calls) before each timing, so that the clocks have left idle


def time_us(torch, fn, iters, graph=True, reps=7, min_calls=1):
    """Microseconds per call of fn() over n = max(iters, min_calls) back-to-back
    calls: the median of `reps` timed repetitions.

    With graph=True the n calls are captured once into a HIP graph on the
    launch stream and each repetition is one replay of it, so host launch cost
    (Python, ctypes) is not on the clock; HIP events bracket each replay on the
    same stream.  graph=False times eager launches from Python.  A caller that
    rotates over R buffer copies passes min_calls=R, so every replay touches all
    of them (the cold regime: R copies span at least twice the LLC).  Before the
    timed repetitions the same replays (calls) run untimed for WARM_S seconds:
    after host-side set-up the GPU clocks start from idle and take milliseconds
    to rise, which otherwise shows as the first measurement of a pair reading
    slower.
    """
    import statistics
    import time

    n = max(iters, min_calls)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()                       # warm replays
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < WARM_S:
            g.replay()
            torch.cuda.synchronize()
        for _ in range(reps):
            e0.record(s)
            g.replay()
            e1.record(s)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / n)
        del g
        return statistics.median(times)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARM_S:
        fn()
        torch.cuda.synchronize()
    for _ in range(reps):
        e0.record(s)
        for _ in range(n):
            fn()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / n)
    return statistics.median(times)


def kernel_source_sha256():
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter profile, or None
    when there is none for it or the kernel sources changed since it was taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    data = json.loads(text[start + 7:end])
    if data.get("source_sha256") != kernel_source_sha256():
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else int(k["fetch_bytes"] + k["write_bytes"])


def bandwidth_peaks(qg, torch, nbytes=4 << 30):
    """Measured HBM bandwidth with the library's 16-byte lane probes over nbytes
    (4 GiB, sixteen times the LLC): a copy (read + write bytes / time) and a
    read-only stream.  Best of 5 launches, HIP events on the launch stream."""
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    src.fill_(0x5A5A5A5A)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(5):
            e0.record(s)
            fn()
            e1.record(s)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return min(ms)

    copy_ms = best(lambda: qg.probe_copy(src, dst))
    read_ms = best(lambda: qg.probe_read(src, sink))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbps": round(2 * nbytes / copy_ms / 1e6, 1), "read_gbps": round(nbytes / read_ms / 1e6, 1),
            "bytes": nbytes, "kernels": "copy16_kernel, read16_kernel (16-byte lane loads/stores, grid-stride)"}


def same_size_reference(qg, torch, nbytes, regime, iters):
    """The library's read and copy probes over the same number of bytes as one
    launch of the dominant kernel, in the same regime (cold: rotating copies
    spanning twice the LLC, every copy touched in each replay), graph-replayed
    back to back.  Microseconds per launch each."""
    nbytes = max(16, nbytes // 16 * 16)
    copies = copies_for(nbytes, regime)
    src = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(i) for i in range(copies)]
    dst = [torch.empty_like(src[0]) for _ in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = {"i": 0}

    def read():
        qg.probe_read(src[st["i"] % copies], sink)
        st["i"] += 1

    def copy():
        qg.probe_copy(src[st["i"] % copies], dst[st["i"] % copies])
        st["i"] += 1

    for _ in range(3):
        read()
        copy()
    r = time_us(torch, read, iters, min_calls=copies)
    c = time_us(torch, copy, iters, min_calls=copies)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "read_us": round(r, 3), "copy_us": round(c, 3), "copies": copies,
            "kernels": "read16_kernel (reads the bytes), copy16_kernel (reads and writes them)"}


def gpu_state(qg, torch):
    """Shader clock under a short MFMA load (cycle counter against the 100 MHz
    constant counter) and the temperatures rocm-smi reports, logged per config
    (the BC-250 post found sysfs clocks wrong and benchmarked from a known
    thermal state)."""
    import subprocess

    import numpy as np

    clocks = qg.probe_mfma_bf16(256, 400)
    torch.cuda.synchronize()
    c = clocks.cpu().numpy().astype("float64")
    ticks = c[:, 3] - c[:, 1]
    mhz = float(np.median(100.0 * (c[:, 2] - c[:, 0]) / np.where(ticks > 0, ticks, np.nan)))
    out = {"sclk_mhz": round(mhz, 1)}
    try:
        # rocm-smi is a Python script: start it under this interpreter as a child
        # process, so that no launcher in between replaces itself with exec()
        import shutil

        smi = shutil.which("rocm-smi")
        if smi is None:
            raise OSError("rocm-smi not found")
        smi = os.path.realpath(smi)
        with open(smi, "rb") as f:
            first = f.readline()
        cmd = ([sys.executable, smi] if b"python" in first else [smi]) + ["--showtemp", "--json"]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=15)
        data = json.loads(res.stdout)
        temps = {}
        for card, vals in data.items():
            for key, v in vals.items():
                if "emperature" in key:
                    try:
                        temps[key.replace("Temperature (Sensor ", "").rstrip(")").replace(") (C", "")] = float(v)
                    except (TypeError, ValueError):
                        pass
            break
        out["temp_c"] = temps or None
    except Exception:       # no rocm-smi or no JSON: the clock alone
        out["temp_c"] = None
    return out


def mfma_probe(qg, torch, blocks=1024, iters=4000):
    """Sustained bf16 MFMA rate of a register-only loop and the shader clock under it.

    1024 workgroups of 4 waves (4 per CU: one per SIMD) each run 8 independent
    16x16x32 bf16 MFMA chains; the clock is the median over workgroups of 100 MHz x
    shader cycles / constant-counter ticks between the loop's start and end.
    """
    flops = blocks * 4 * iters * 8 * 16384
    clocks = qg.probe_mfma_bf16(blocks, iters)          # warm-up launch
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(5):
        e0.record(stream)
        qg.probe_mfma_bf16(blocks, iters, clocks=clocks)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    c = clocks.cpu().numpy().astype("float64")
    import numpy as np

    ticks = c[:, 3] - c[:, 1]
    mhz = float(np.median(100.0 * (c[:, 2] - c[:, 0]) / np.where(ticks > 0, ticks, np.nan)))
    tflops = flops / (best * 1e-3) / 1e12
    return {"tflops": round(tflops, 1), "frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "sclk_mhz": round(mhz, 1), "ms": round(best, 4), "blocks": blocks, "iters": iters,
            "kernel": "mfma_probe_kernel (register-only 16x16x32 bf16 MFMA chains)"}


def cpu_baseline(cases, seconds):
    """The C++ CPU oracle, as it stands, on the same inputs until `seconds` have passed.

    It runs on std::threads over output columns; the thread count is the
    host's CPU share (OMP_NUM_THREADS when set, else the hardware threads, at
    most 16).
    """
    from oracle import cpu

    threads = cpu.default_threads()
    t0 = time.perf_counter()
    done_bytes, done_flops, calls = 0, 0, 0
    while True:
        for c in cases:
            d = c.host
            cpu.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], c.m, c.k, c.n, threads=threads)
            done_bytes += c.bytes
            done_flops += c.flops
            calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    # the same oracle on one thread, on the GEMV workload (m = 1, k = 896, n = 4864)
    from qgemm_inputs import int4_inputs

    g = int4_inputs(1, 896, 4864, seed=1000 * 65536)
    t1, n1 = time.perf_counter(), 0
    while time.perf_counter() - t1 < 1.0:
        cpu.qgemm_int4(g["x"], g["qweight"], g["scales"], g["qzeros"], 1, 896, 4864, threads=1)
        n1 += 1
    el1 = time.perf_counter() - t1
    # one pass over the six small-M products on one thread
    t2 = time.perf_counter()
    for c in cases:
        d = c.host
        cpu.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], c.m, c.k, c.n, threads=1)
    el2 = time.perf_counter() - t2
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "us_per_call": round(el / calls * 1e6, 1),
            "gflops": round(done_flops / el / 1e9, 3), "cpu_model": model,
            "hardware_threads": cpu.hardware_threads(),
            "single_thread_gemv_us": round(el1 / n1 * 1e6, 1),
            "single_thread_step_s": round(el2, 3),
            "sample": "%d calls of the C++ oracle (dequantise to fp32, accumulate in fp64, %d std::threads "
                      "over output columns) cycling over the six small-M products, %.1f s"
                      % (calls, threads, el)}


class DeviceWeights:
    """`copies` resident copies of one (k, n) int4 weight set drawn on the device
    from a seeded torch generator (timing only: the parity tests draw the same
    distributions from the host generator).  q and z uniform 0..15 (random
    words), s = fp16(0.005 + |N(0, 0.01)|)."""

    def __init__(self, torch, k, n, seed, copies):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        self.k, self.n = k, n
        self.w = []
        for _ in range(copies):
            qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (k // 8, n), generator=g, dtype=torch.int32, device="cuda")
            sc = (0.005 + (torch.randn((k // 128, n), generator=g, device="cuda") * 0.01).abs()).to(torch.float16)
            qz = torch.randint(-2 ** 31, 2 ** 31 - 1, (k // 128, n // 8), generator=g, dtype=torch.int32,
                               device="cuda")
            self.w.append((qw, sc, qz))
        self.i = 0

    def next(self):
        w = self.w[self.i % len(self.w)]
        self.i += 1
        return w


def time_configs(qg, torch, args, bw):
    """The rest of the metric, per call in the cold regime: the prefill shapes
    (25600 x 5120, 5120 x 25600) at m = 16, 512, 2048 and the large-weight shapes
    (4096 x 28672, 4096 x 14336, 8192 x 8192) at m = 1, 8, 16; each row with its
    kernel, µs, GB/s of algorithmic bytes, TFLOP/s and the fraction of its
    roofline (MFMA-bound rows: of the 2.5 PFLOP/s bf16 peak; the others: of the
    measured copy), plus the shader clock and temperatures after each shape;
    then the bf16 dense training trio (forward NT, input gradient NN, weight
    gradient TN at 1024 / 2048 / 4096 tokens for both weight orientations),
    with the library's default workspace (the k split where it applies)."""
    from qgemm_inputs.configs import dense_cases, seed_for

    rows, states = [], []
    for cfg, shapes, tokens in ((2, [(25600, 5120), (5120, 25600)], [16, 512, 2048]),
                                (4, [(4096, 28672), (4096, 14336), (8192, 8192)], [1, 8, 16])):
        for si, (k, n) in enumerate(shapes):
            w = DeviceWeights(torch, k, n, seed_for(cfg, 100 + si), copies_for(int4_bytes(0, k, n), args.regime))
            g = torch.Generator(device="cuda")
            g.manual_seed(seed_for(cfg, 200 + si))
            for m in tokens:
                x = torch.randn((m, k), generator=g, device="cuda").to(torch.bfloat16)
                y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

                def launch(x=x, y=y):
                    qw, sc, qz = w.next()
                    qg.qgemm_int4(x, qw, sc, qz, out=y)

                for _ in range(3):
                    launch()
                us = time_us(torch, launch, args.steps, min_calls=len(w.w))
                nb, fl = int4_bytes(m, k, n), 2 * m * n * k
                row = {"config": cfg, "m": m, "k": k, "n": n, "kernel": qg.describe_int4(m, n, k).split(" ")[0],
                       "us": round(us, 3), "gbps": round(nb / us / 1e3, 1), "tflops": round(fl / us / 1e6, 1),
                       "bytes": nb}
                ridge = bw["copy_gbps"] * 1e-3 * fl / nb           # TFLOP/s the copy bandwidth allows
                if ridge >= MFMA_BF16_PEAK_TFLOPS:
                    row.update(bound="mfma", frac_of_mfma_peak=round(row["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4))
                else:
                    row.update(bound="hbm", frac_of_copy=round(row["gbps"] / bw["copy_gbps"], 4))
                rows.append(row)
                print("config", row, file=sys.stderr, flush=True)
                del x, y
            del w
            torch.cuda.empty_cache()
            st = gpu_state(qg, torch)
            st.update(config=cfg, k=k, n=n)
            states.append(st)
    # config 3, bf16: operands N(0, 0.02^2) drawn on the device (timing only; the
    # parity tests use the host generator)
    g = torch.Generator(device="cuda")
    for case in dense_cases(3, with_lora=False):
        if case["dtype"] != "bf16":
            continue
        lay, M, N, K = case["layout"], case["M"], case["N"], case["K"]
        g.manual_seed(case["seed"])
        a = (torch.randn((K, M) if lay == "TN" else (M, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        b = (torch.randn((N, K) if lay == "NT" else (K, N), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        out = qg.gemm_dense(lay, a, b)
        us = time_us(torch, lambda: qg.gemm_dense(lay, a, b, out=out), args.steps)
        fl = 2 * M * N * K
        rows.append({"config": 3, "role": case["role"], "layout": lay, "M": M, "N": N, "K": K,
                     "us": round(us, 3), "tflops": round(fl / us / 1e6, 1), "bound": "mfma",
                     "frac_of_mfma_peak": round(fl / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "k_split": qg.dense_workspace_size(lay, "bf16", M, N, K) > 0})
        print("config", rows[-1], file=sys.stderr, flush=True)
        del a, b, out
    torch.cuda.empty_cache()
    return rows, states


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import int4_weight_only_gptq_amd as qg

    qg.load()
    torch.cuda.init()

    cases = []
    for si, (k, n) in enumerate(SMALL_M):
        for mi, m in enumerate(SMALL_M_TOKENS):
            nb = int4_bytes(0, k, n)
            cases.append(Int4Case(qg, torch, m, k, n, seed=(1001 * 65536) + 3 * si + mi,
                                  copies=copies_for(nb, args.regime)))
    torch.cuda.synchronize()
    state0 = gpu_state(qg, torch)

    # per-call timing (each case back to back, every weight copy touched in each
    # replay), then the whole step
    for c in cases:
        for _ in range(args.warmup):
            c.launch()
    per_case = []
    for c in cases:
        us = time_us(torch, c.launch, args.steps, min_calls=len(c.w))
        per_case.append({"m": c.m, "k": c.k, "n": c.n, "kernel": c.kernel, "us": round(us, 3),
                         "gbps": round(c.bytes / us / 1e3, 1), "tflops": round(c.flops / us / 1e6, 2),
                         "bytes": c.bytes,
                         "calls_per_replay": max(args.steps, len(c.w)),
                         "bytes_per_replay": max(args.steps, len(c.w)) * c.bytes})
        print("case", per_case[-1], file=sys.stderr, flush=True)
    state1 = gpu_state(qg, torch)
    # context: the warm regime (one weight copy, resident in the LLC), same timing
    warm = []
    for c in cases:
        w0 = c.w[0]

        def warm_launch(c=c, w0=w0):
            c.qg.qgemm_int4(c.x, w0[0], w0[1], w0[2], out=c.y)

        us = time_us(torch, warm_launch, args.steps)
        warm.append({"m": c.m, "k": c.k, "n": c.n, "us": round(us, 3), "gbps": round(c.bytes / us / 1e3, 1)})
    # floor: the smallest kernel the same entry point launches (k = 0 -> a zero fill of 1 x 8)
    fx = torch.empty((1, 0), dtype=torch.bfloat16, device="cuda")
    fw = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    fs = torch.empty((0, 8), dtype=torch.float16, device="cuda")
    fz = torch.empty((0, 1), dtype=torch.int32, device="cuda")
    fy = torch.empty((1, 8), dtype=torch.bfloat16, device="cuda")
    floor_us = time_us(torch, lambda: qg.qgemm_int4(fx, fw, fs, fz, out=fy), args.steps)

    def step():
        for c in cases:
            c.launch()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the step: exactly K steps in one timed region (one graph replay between events)
    step_us = time_us(torch, step, args.steps, reps=1)
    step_bytes = sum(c.bytes for c in cases)
    value = step_bytes / step_us / 1e3
    print("step", {"us": step_us, "gbps": value}, file=sys.stderr, flush=True)
    bw = bandwidth_peaks(qg, torch)
    print("bandwidth", bw, file=sys.stderr, flush=True)

    # dominant kernel: largest share of the step; its average launch duration is
    # the event-timed average over its calls in the per-call runs above
    agg = {}
    for pc in per_case:
        a = agg.setdefault(pc["kernel"], {"us": 0.0, "bytes": 0, "launches": 0})
        a["us"] += pc["us"]
        a["bytes"] += pc["bytes"]
        a["launches"] += 1
    dom = max(agg, key=lambda name: agg[name]["us"])
    a = agg[dom]
    avg_us, avg_bytes = a["us"] / a["launches"], a["bytes"] / a["launches"]
    achieved = avg_bytes / avg_us / 1e3
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "avg_launch_us": round(avg_us, 3), "bytes_per_launch": int(avg_bytes),
                "traffic": measured_traffic(dom)}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "int4 GPTQ small-M: k x n in {4096x4096, 2048x8192}, m in "
                               "{1, 8, 15}, group 128, bf16 activations",
                   "regime": args.regime, "calls_per_step": len(cases),
                   "parallelism": "none (1 GPU)"},
        "cases": per_case,
        "timing": "HIP graph replay of back-to-back launches, HIP events on the launch stream; the step: one "
                  "replay of exactly K steps; per-case, floor, reference and config figures: median of 7 "
                  "replays, each touching every weight copy (>= 2x the LLC per replay in the cold regime); "
                  "warm_cases: the same calls on one weight copy (LLC-resident), context only",
        "warm_cases": warm,
        "floor_us": round(floor_us, 3),
        "copy_gbps": bw["copy_gbps"],
        "read_gbps": bw["read_gbps"],
        "bandwidth_probe": bw,
        "roofline": roofline,
    }
    roofline["frac_of_copy"] = round(achieved / bw["copy_gbps"], 4)
    roofline["frac_of_read"] = round(achieved / bw["read_gbps"], 4)
    # the same bytes through the library's read and copy probes: how far launch
    # and latency, not bandwidth, bound a launch of this size
    same = same_size_reference(qg, torch, int(avg_bytes), args.regime, args.steps)
    out["same_size_reference"] = same
    roofline["time_vs_same_size_copy"] = round(avg_us / same["copy_us"], 3)
    roofline["time_vs_same_size_read"] = round(avg_us / same["read_us"], 3)
    # the MFMA-bound denominators beside the datasheet peak: a register-only
    # bf16 MFMA loop and the shader clock it runs at
    out["mfma_probe"] = mfma_probe(qg, torch)
    # the m >= 512 TFLOP/s and the large-weight GB/s halves of the metric
    rows, states = time_configs(qg, torch, args, bw)
    out["configs"] = rows
    out["gpu_state"] = [dict(state0, at="start"), dict(state1, at="after the small-M cases")] + states
    # context only (another codec on another GPU, so no vs_baseline): the fused
    # small-M kernel times the GPTQModel NF12 pull request reports on an R9700
    # (gfx1201) for the same shapes, beside this path's per-call times
    pages = {(1, 4096, 4096): 20.45, (8, 4096, 4096): 24.15, (1, 2048, 8192): 18.49, (8, 2048, 8192): 23.87}
    out["pages_context"] = [
        {"m": c["m"], "k": c["k"], "n": c["n"], "us": c["us"], "pages_us_r9700_nf12": pages[(c["m"], c["k"], c["n"])],
         "ratio": round(pages[(c["m"], c["k"], c["n"])] / c["us"], 2)}
        for c in per_case if (c["m"], c["k"], c["n"]) in pages]
    if args.suite:
        out["suite_file"] = args.suite
        run_suite(qg, torch, args, args.suite)
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(cases, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def run_suite(qg, torch, args, path):
    """Time every int4 and dense workload shape (auto path) into a JSON file."""
    import numpy as np
    from qgemm_inputs import dense_cases, dense_inputs, int4_cases

    rows = []
    iters = max(10, args.steps // 4)
    kinds = set(args.suite_kinds.split(","))
    for cfg in ((0, 1, 2, 4) if "int4" in kinds else ()):
        for (_, m, k, n, seed) in int4_cases(cfg):
            c = Int4Case(qg, torch, m, k, n, seed, copies_for(int4_bytes(0, k, n), args.regime))
            for _ in range(3):
                c.launch()
            us = time_us(torch, c.launch, iters, min_calls=len(c.w))
            rows.append({"kind": "int4", "m": m, "k": k, "n": n, "kernel": c.kernel, "us": us,
                         "gbps": c.bytes / us / 1e3, "tflops": c.flops / us / 1e6,
                         "mfma_frac": c.flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS})
            print("suite int4", rows[-1], file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
    # weights without a zero point (qzeros NULL) on the small-M and prefill shapes
    for cfg in ((1, 2) if "int4_nozero" in kinds else ()):
        for (_, m, k, n, seed) in int4_cases(cfg):
            c = Int4Case(qg, torch, m, k, n, seed, copies_for(int4_bytes(0, k, n, False), args.regime),
                         zeros=False)
            for _ in range(3):
                c.launch()
            us = time_us(torch, c.launch, iters, min_calls=len(c.w))
            rows.append({"kind": "int4_nozero", "m": m, "k": k, "n": n, "kernel": c.kernel, "us": us,
                         "gbps": c.bytes / us / 1e3, "tflops": c.flops / us / 1e6,
                         "mfma_frac": c.flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS})
            print("suite int4_nozero", rows[-1], file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
    for case in (dense_cases(3) if "dense" in kinds else ()):
        d = dense_inputs(case["layout"], case["dtype"], case["M"], case["N"], case["K"], case["seed"])
        dt = torch.bfloat16 if case["dtype"] == "bf16" else torch.float16
        a = torch.from_numpy(d["a"].view(np.int16)).cuda().view(dt)
        b = torch.from_numpy(d["b"].view(np.int16)).cuda().view(dt)
        out = qg.gemm_dense(case["layout"], a, b)
        us = time_us(torch, lambda: qg.gemm_dense(case["layout"], a, b, out=out), iters)
        M, N, K = case["M"], case["N"], case["K"]
        rows.append({"kind": "dense", "role": case["role"], "layout": case["layout"],
                     "dtype": case["dtype"], "M": M, "N": N, "K": K, "us": us,
                     "gbps": dense_bytes(M, N, K) / us / 1e3, "tflops": 2 * M * N * K / us / 1e6,
                     "mfma_frac": 2 * M * N * K / us / 1e6 / MFMA_BF16_PEAK_TFLOPS})
        if "dense_vendor" in kinds and min(M, N) > 16:
            # context: the vendor library (torch.mm -> hipBLASLt) on the same operands
            # and layout, same timing; 2-D products only
            lay = case["layout"]
            lhs = a.t() if lay == "TN" else a
            rhs = b.t() if lay == "NT" else b
            ref = torch.empty((M, N), dtype=dt, device="cuda")
            torch.mm(lhs, rhs, out=ref)
            vus = time_us(torch, lambda: torch.mm(lhs, rhs, out=ref), iters)
            rows[-1].update({"vendor_us": vus, "vendor_tflops": 2 * M * N * K / vus / 1e6,
                             "vendor": "torch.mm (hipBLASLt)"})
            del ref
        print("suite dense", rows[-1], file=sys.stderr, flush=True)
    # a rank-16 LoRA add in the epilogue (U = X A^T launched first) on the same shapes
    for cfg in ((1, 2) if "int4_lora" in kinds else ()):
        for (_, m, k, n, seed) in int4_cases(cfg):
            c = Int4Case(qg, torch, m, k, n, seed, copies_for(int4_bytes(0, k, n), args.regime))
            g = torch.Generator(device="cuda")
            g.manual_seed(seed)
            la = (torch.randn((16, k), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
            lb = (torch.randn((n, 16), generator=g, device="cuda") * 0.05).to(torch.bfloat16)

            def launch(c=c, la=la, lb=lb):
                qw, sc, qz = c.w[c.i % len(c.w)]
                c.i += 1
                qg.qgemm_int4_lora(c.x, qw, sc, qz, la, lb, 2.0, out=c.y)

            for _ in range(3):
                launch()
            us = time_us(torch, launch, iters, min_calls=len(c.w))
            nbytes = c.bytes + 2 * 16 * (k + n)
            rows.append({"kind": "int4_lora", "m": m, "k": k, "n": n, "kernel": c.kernel, "us": us,
                         "gbps": nbytes / us / 1e3, "tflops": c.flops / us / 1e6,
                         "mfma_frac": c.flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS})
            print("suite int4_lora", rows[-1], file=sys.stderr, flush=True)
            del c, la, lb
            torch.cuda.empty_cache()
    # the FP32 training trio (fp32 products and accumulation) against the fp32 peak
    for case in (dense_cases(3, with_lora=False) if "dense_fp32" in kinds else ()):
        if case["dtype"] != "bf16":
            continue
        M, N, K, layout = case["M"], case["N"], case["K"], case["layout"]
        sa = (M, K) if layout != "TN" else (K, M)
        sb = (N, K) if layout == "NT" else (K, N)
        g = torch.Generator(device="cuda")
        g.manual_seed(case["seed"])
        a = torch.randn(sa, generator=g, device="cuda", dtype=torch.float32) * 0.02
        b = torch.randn(sb, generator=g, device="cuda", dtype=torch.float32) * 0.02
        out = qg.gemm_dense(layout, a, b)
        us = time_us(torch, lambda: qg.gemm_dense(layout, a, b, out=out), iters)
        rows.append({"kind": "dense_fp32", "role": case["role"], "layout": layout, "dtype": "fp32",
                     "M": M, "N": N, "K": K, "us": us, "gbps": 2 * dense_bytes(M, N, K) / us / 1e3,
                     "tflops": 2 * M * N * K / us / 1e6,
                     "fp32_frac": 2 * M * N * K / us / 1e6 / FP32_PEAK_TFLOPS})
        print("suite dense_fp32", rows[-1], file=sys.stderr, flush=True)
        del a, b, out
    # batched attention products; operands drawn on the device from a seeded
    # generator (timing only: the parity tests use the host generator)
    from qgemm_inputs import attention_cases
    for case in (attention_cases() if "attention" in kinds else ()):
        dt = torch.bfloat16 if case["dtype"] == "bf16" else torch.float16
        bt, M, N, K, layout = case["batch"], case["M"], case["N"], case["K"], case["layout"]
        sa = (bt, M, K) if layout != "TN" else (bt, K, M)
        sb = (bt, N, K) if layout == "NT" else (bt, K, N)
        g = torch.Generator(device="cuda")
        g.manual_seed(case["seed"])
        a = torch.randn(sa, generator=g, device="cuda", dtype=torch.float32).to(dt)
        b = torch.randn(sb, generator=g, device="cuda", dtype=torch.float32).to(dt)
        out = qg.gemm_dense_batched(layout, a, b)
        us = time_us(torch, lambda: qg.gemm_dense_batched(layout, a, b, out=out), iters)
        rows.append({"kind": "attention", "role": case["role"], "layout": layout, "dtype": case["dtype"],
                     "batch": bt, "M": M, "N": N, "K": K, "us": us,
                     "gbps": bt * dense_bytes(M, N, K) / us / 1e3, "tflops": 2 * bt * M * N * K / us / 1e6,
                     "mfma_frac": 2 * bt * M * N * K / us / 1e6 / MFMA_BF16_PEAK_TFLOPS})
        print("suite attention", rows[-1], file=sys.stderr, flush=True)
        del a, b, out
        torch.cuda.empty_cache()
    probe = mfma_probe(qg, torch)
    for r in rows:
        if "tflops" in r and r.get("kind") != "dense_fp32":
            r["frac_of_mfma_probe"] = r["tflops"] / probe["tflops"]
    with open(path, "w") as f:
        json.dump({"regime": args.regime, "mfma_probe": probe, "rows": rows}, f, indent=1)


if __name__ == "__main__":
    main()
