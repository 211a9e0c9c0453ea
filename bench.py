#!/usr/bin/env python3
"""Benchmark of the compressed linear forward on one MI355X.

Default workload: the LLaMA-70B layer set at batch 1 -- GQA qkv 8192->10240,
up 8192->28672, down 28672->8192 -- with 3-bit per-row LUT codes (ten per
32-bit word), 0.45% fp16 CSR outliers and a rank-64 bf16 low-rank
correction, bf16 activations, seeded synthetic weights and activations (the
largest workload that fits one GPU).  One step is one forward of every layer
of the set (one decode launch per layer).  Packed weights rotate over enough
copies (>= 1 GiB) that no step finds its weights in the 256 MB last-level
cache.

Prints one JSON line on stdout:
  value            effective HBM GB/s on algorithmic bytes (packed weights + x + y)
  roofline         the decode kernel against the 8 TB/s HBM peak (and against the
                   streaming-read ceiling measured in the same run)
  cpu_baseline     the fp64 CPU oracle on a bounded sample of the same layers
  streaming_read_ceiling, launch_floor
                   one read-only kernel per layer-sized buffer, and back-to-back
                   empty launches: what one launch per layer can reach here
  other_workloads  the 4096x4096 LUT3, LLaMA-7B LUT4 and SLiM INT4 2:4 + int4
                   rank-128 workloads at batch 1 (default run only)

Other workloads (`--config 1..5`, `--M`) are for measurement sweeps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "batch-1 µs/layer & effective HBM GB/s (% of peak) for compressed GEMV"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16 matrix-core peak
ROTATE_BYTES = 1 << 30
# counter summaries of HBM traffic per workload (committed under profiles/), each
# valid only for the kernel sources it was taken with
TRAFFIC_FILES = {(5, 1): os.path.join(ROOT, "profiles", "decode_lut3_lr_llama70b_b1_traffic.txt"),
                 (2, 1): os.path.join(ROOT, "profiles", "decode_lut4_llama7b_b1_traffic.txt"),
                 (3, 1): os.path.join(ROOT, "profiles", "decode_int4_24_lr128_b1_traffic.txt")}
KERNEL_SOURCES = ["compressed_linear_amd/csrc/decode_rows.h", "compressed_linear_amd/csrc/unpack.h",
                  "compressed_linear_amd/csrc/decode.hip", "compressed_linear_amd/csrc/layout.h",
                  "compressed_linear_amd/csrc/lowrank.h", "compressed_linear_amd/csrc/decode_stream.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(cfg: int, M: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload, or None.

    The summary holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the decode
    kernel, the same counters for a copy kernel of known size (calibration), and
    the hash of the kernel sources it was taken with; a different hash means the
    kernel changed since, and the figure no longer applies.
    """
    path = TRAFFIC_FILES.get((cfg, M))
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_]+)\s*[:=]\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def batch1_kernel(l, acct) -> str:
    """The kernel a batch-1 forward of layer l runs on the auto path: the
    streaming kernel for layers of 28 MiB of code chunks or more, or with a
    rank term (the library's rule in decode.hip), the row-wise kernel
    otherwise."""
    stream = acct["codes"] >= (28 << 20) or bool(l.rank)
    return "decode_stream_kernel" if stream else "decode_rows_kernel"


def roofline(cfg: int, M: int, path: str, built, set_bytes: int, us_per_launch: float, graph: bool) -> dict:
    """Roofline entry for the launches of one layer (mean over the layers of a step).

    Decode (M <= 32) is priced on algorithmic HBM bytes (packed weights + x + y)
    against the 8 TB/s peak; prefill on algorithmic flops (2*M*K*N for the
    weight product, 2*M*r*(K+N) for a rank term) against the dense fp16/bf16
    matrix-core peak.  The counter-based HBM traffic figure comes from the
    committed summary of the workload (batch 1, one decode kernel per layer),
    else it is null.
    """
    n = len(built)
    if M > 32:
        flops = sum(2.0 * M * l.K * l.N + (2.0 * M * l.rank * (l.K + l.N) if l.rank else 0.0) for l, _, _ in built) / n
        achieved = flops / (us_per_launch * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": f"prefill (weight tiles dequantised into LDS, 16-bit matrix cores), M {M}",
                "flops_per_launch": int(flops), "us_per_launch": round(us_per_launch, 3)}
    bytes_per_launch = set_bytes / n
    achieved = bytes_per_launch / us_per_launch / 1e3
    if M == 1 and path == "auto":
        kind = built[0][0].dense.upper()
        names = sorted({batch1_kernel(l, acct) for l, acct, _ in built})
        kernel = f"{' + '.join(names)} ({kind}, batch 1; one launch per layer, rank prologue inside)"
    elif path == "decode_valu":
        kernel = f"vector-ALU decode, batch {M} (all launches of a layer)"
    else:
        kernel = f"decode, batch {M}, path {path} (all launches of a layer)"
    traffic = read_traffic(cfg, M) if (path == "auto" and not graph) else None
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kernel, "bytes_per_launch": int(bytes_per_launch), "us_per_launch": round(us_per_launch, 3)}


def layer_bytes(acct: dict, K: int, N: int, M: int) -> int:
    return int(acct["total"]) + 2 * M * K + 4 * M * N


def _host_description():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = sorted({f"{d.get('internal_api')} ({d.get('user_api')})" for d in threadpool_info()})
    except Exception:  # noqa: BLE001 -- optional
        pass
    return model, blas


def cpu_baseline(layers, xs, frac: float = 1.0 / 32):
    """The fp64 oracle as it stands on a row sample of each layer: all the
    process's cores (BLAS threads), then one thread; scaled to whole layers."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    env_cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    if env_cap > 0:
        cores = min(cores, env_cap)
    runs = {}
    rows_total, rows_all = 0, 0
    for threads in (cores, 1):
        with threadpool_limits(limits=threads):
            used = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
            t_total, bytes_total = 0.0, 0.0
            per_layer_us = []
            rows_total, rows_all = 0, 0
            for (layer, acct), x in zip(layers, xs):
                n_rows = max(64, int(layer.N * frac))
                rows = np.arange(n_rows)
                t0 = time.perf_counter()
                oracle.forward(layer, x, rows)
                dt = time.perf_counter() - t0
                scale = layer.N / n_rows
                t_total += dt * scale
                bytes_total += layer_bytes(acct, layer.K, layer.N, x.shape[0])
                per_layer_us.append(dt * scale * 1e6)
                rows_total += n_rows
                rows_all += layer.N
        runs[threads] = (bytes_total / t_total / 1e9, float(np.mean(per_layer_us)), used)
    model, blas = _host_description()
    v_all, us_all, used_all = runs[cores]
    v_one, us_one, _ = runs[1]
    return {
        "value": round(v_all, 4), "unit": "GB/s", "cores": int(used_all), "kind": "oracle",
        "us_per_layer": round(us_all, 1),
        "single_thread": {"value": round(v_one, 4), "unit": "GB/s", "us_per_layer": round(us_one, 1)},
        "cpu_model": model, "blas": blas,
        "sample": f"fp64 reconstruct + x W^T of the first {frac:.4g} of the rows of each layer "
                  f"({rows_total} of {rows_all} rows), with {used_all} BLAS threads and with one, "
                  f"scaled to whole layers",
    }


def to_dev_x(x, x_dtype, dev):
    import torch
    if x_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x.astype(np.float16))).to(dev)


def build_layers(cfg: int, M: int, act_scale: float = 0.0):
    from synth.layers import CONFIGS, make_layer, make_x, with_act_scale
    import compressed_linear_amd as cla
    out, xs = [], []
    for li, (name, K, N) in enumerate(CONFIGS[cfg]["layers"]):
        layer = make_layer(cfg, li, M_for_clamp=M)
        if act_scale > 0:
            layer = with_act_scale(layer, seed=li, frac=act_scale)
        blob, acct = cla.pack(layer)
        out.append((layer, acct, blob))
        xs.append(make_x(cfg, li, M))
    return out, xs


def bench_fit_int(a, dev):
    """--fit int: the data-free int4 2:4 packer (cl_fit_int) on the 4096 -> 11008 projection."""
    import torch
    import compressed_linear_amd as cla
    N, K, grid = 11008, 4096, 100
    r = np.random.default_rng(2027)
    w = r.normal(0, 0.02, (N, K))
    w = np.where(r.random((N, K)) < 0.002, r.normal(0, 0.3, (N, K)), w).astype(np.float16)
    Wd = torch.from_numpy(w.view(np.int16)).view(torch.float16).to(dev)
    cla.fit_int(Wd, 4, "2:4", grid)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(3, a.steps // 40)
    e0.record(stream)
    for _ in range(reps):
        cla.fit_int(Wd, 4, "2:4", grid)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # ALU bound: one element-candidate (a kept weight under one scale candidate) = an fp64
    # division (about 8 operations), rint, the clamp, an integer multiply-subtract and a
    # 128-bit square-accumulate: about 20 operations at 39.3 T operations/s
    ec = N * (K // 2) * grid
    peak = 39.3e12 / 20
    cpu = None
    if not a.no_cpu_baseline:
        from oracle import fit_oracle as F
        t0 = time.perf_counter()
        F.fit_int(w[:2], 4, "2:4", grid)
        dt = time.perf_counter() - t0
        cpu = {"value": round(2 * K / dt / 1e6, 4), "unit": "M weights/s", "cores": 1, "kind": "oracle",
               "sample": f"the packer oracle on the first 2 rows ({2 * K} weights), Python integers, one process"}
    out = {
        "metric": "data-free int4 2:4 packing throughput (cl_fit_int)",
        "value": round(N * K / ms / 1e6, 3), "unit": "G weights/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 in, f64 division, 128-bit integer errors", "data": "synthetic (seeded)",
        "config": {"workload": f"up projection {K}->{N}, int4, magnitude 2:4, clip grid of {grid}"},
        "roofline": {"bound": "alu", "achieved": round(ec / ms / 1e6, 2), "peak": round(peak / 1e9, 2),
                     "unit": "G element-candidates/s", "frac": round(ec / ms * 1e3 / peak, 4), "traffic": None,
                     "kernel": "fit_int_kernel<7>"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_fit(a, dev):
    """--fit: the data-free LUT packer (cl_fit_lut) on one LLaMA-7B projection."""
    import torch
    import compressed_linear_amd as cla
    if a.fit == "int":
        return bench_fit_int(a, dev)
    N, K, bits, frac, iters = 11008, 4096, 4, 0.0045, 30
    r = np.random.default_rng(2026)
    w = r.normal(0, 0.02, (N, K))
    w = np.where(r.random((N, K)) < 0.003, r.normal(0, 0.3, (N, K)), w).astype(np.float16)
    n_out = int(round(frac * N * K))
    Wd = torch.from_numpy(w.view(np.int16)).view(torch.float16).to(dev)
    for _ in range(max(1, a.warmup // 10)):
        cla.fit_lut(Wd, bits, n_out, iters)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(3, a.steps // 40)
    stats = {}
    e0.record(stream)
    for _ in range(reps):
        cla.fit_lut(Wd, bits, n_out, iters, stats)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # ALU bound: one element-iteration = the weight's 2^b - 1 boundary compares in fp64 (and its
    # cluster sum), against MI355X's fp64 vector rate of 39.3 T operations/s (78.6 TFLOP/s counting
    # an FMA as two), i.e. 39.3e12 / (2^b - 1) element-iterations per second
    elem_iters = stats["total_iters"] * (K - n_out / N)
    peak_ei = 39.3e12 / ((1 << bits) - 1)
    # algorithmic bytes: the weights read once, codes and LUTs written, the CSR part written
    alg = N * K * 2 + N * K + N * (1 << bits) * 2 + (N + 1) * 4 + n_out * 6
    cpu = None
    if not a.no_cpu_baseline:
        from oracle import fit_oracle as F
        rows = 64
        t0 = time.perf_counter()
        F.fit_lut(w[:rows], bits, int(round(frac * rows * K)), iters)
        dt = time.perf_counter() - t0
        cpu = {"value": round(rows * K / dt / 1e6, 3), "unit": "M weights/s", "cores": 1, "kind": "oracle",
               "sample": f"the packer oracle on the first {rows} rows ({rows * K} weights), numpy, one process"}
    out = {
        "metric": "data-free LUT packing throughput (cl_fit_lut)",
        "value": round(N * K / ms / 1e6, 3), "unit": "G weights/s", "n_gpus": 1, "steps": reps,
        "warmup": max(1, a.warmup // 10), "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16 in, f64 sums", "data": "synthetic (seeded)",
        "config": {"workload": f"LLaMA-7B gate projection {K}->{N}, {bits}-bit LUT, {frac:.2%} outliers, "
                               f"{iters} Lloyd iterations at most"},
        "roofline": {"bound": "alu", "achieved": round(elem_iters / ms / 1e6, 2), "peak": round(peak_ei / 1e9, 2),
                     "unit": "G element-iterations/s", "frac": round(elem_iters / ms * 1e3 / peak_ei, 4),
                     "traffic": None, "kernel": "cl_fit_lut (all kernels of one call)",
                     "lloyd_iterations_per_row": round(stats["total_iters"] / N, 2),
                     "hbm_GBps_on_algorithmic_bytes": round(alg / ms / 1e6, 1), "bytes_per_call": alg},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def measure(cfg, M, a, dev, steps, warmup, per_layer=False, graph=False, act_scale=0.0):
    """Time `steps` steps of workload `cfg` at batch M (one forward of every layer
    per step, weights rotating over >= 1 GiB of packed copies); events on the
    stream the kernels run on."""
    import torch
    import compressed_linear_amd as cla
    from synth.layers import CONFIGS

    log(f"building config {cfg} M={M}")
    built, xs_np = build_layers(cfg, M, act_scale)
    set_bytes = sum(layer_bytes(acct, l.K, l.N, M) for l, acct, _ in built)
    weight_bytes = sum(int(acct["total"]) for _, acct, _ in built)
    R = max(2, -(-ROTATE_BYTES // weight_bytes))
    log(f"layer set: {len(built)} layers, {set_bytes / 1e6:.2f} MB algorithmic per step, {R} rotating copies")
    max_M = max(M, 2) if a.path == "decode_mfma" else max(M, 1)  # the matrix-core decode needs a batch workspace
    mods = [[cla.CompressedLinear(blob, max_M=max_M, device=dev) for (_, _, blob) in built] for _ in range(R)]
    xs = [[to_dev_x(x, l.x_dtype, dev) for (l, _, _), x in zip(built, xs_np)] for _ in range(R)]
    ys = [[torch.empty((M, l.N), dtype=torch.float32, device=dev) for (l, _, _) in built] for _ in range(R)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ptrs = [[(m._h, x.data_ptr(), y.data_ptr()) for m, x, y in zip(mods[r], xs[r], ys[r])] for r in range(R)]
    path = cla.PATH[a.path]
    fwd = cla.lib().cl_forward_path

    def step(i):
        for h, xp, yp in ptrs[i % R]:
            st = fwd(h, M, xp, yp, sp, path)
            if st != 0:
                raise cla.ClError(st, "cl_forward", cla.lib().cl_last_error().decode())

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        # one pass over the rotating copies recorded into a HIP graph, replayed
        gs = torch.cuda.Stream(device=dev)
        gsp = gs.cuda_stream

        def steps_on(handle):
            for i in range(R):
                for h, xp, yp in ptrs[i]:
                    st = fwd(h, M, xp, yp, handle, path)
                    if st != 0:
                        raise cla.ClError(st, "cl_forward", cla.lib().cl_last_error().decode())
        with torch.cuda.stream(gs):
            steps_on(gsp)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            steps_on(gsp)
        torch.cuda.synchronize()
        reps = max(1, -(-steps // R))
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        steps = reps * R
    else:
        e0.record(stream)
        for i in range(steps):
            step(warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps
    n_launch = len(built)
    gbs = set_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"config {cfg} M={M}: {ms_per_step * 1e3:.2f} us/step, {ms_per_step * 1e3 / n_launch:.2f} us/layer, "
        f"{gbs:.1f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak)")
    layers_out = []
    if per_layer:
        for li, (l, acct, _) in enumerate(built):
            reps = max(20, steps)
            for i in range(5):
                h, xp, yp = ptrs[i % R][li]
                fwd(h, M, xp, yp, sp, path)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(reps):
                h, xp, yp = ptrs[i % R][li]
                fwd(h, M, xp, yp, sp, path)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            b = layer_bytes(acct, l.K, l.N, M)
            layers_out.append({"layer": CONFIGS[cfg]["layers"][li][0], "K": l.K, "N": l.N, "us": round(us, 3),
                               "GBps": round(b / us / 1e3, 1), "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                               "bytes": b})
            log(f"  {layers_out[-1]}")
    for r in mods:
        for m in r:
            m.close()
    del mods, xs, ys
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"built": built, "xs_np": xs_np, "set_bytes": set_bytes, "ms_per_step": ms_per_step, "gbs": gbs,
            "n_launch": n_launch, "rotating": R, "steps": steps, "per_layer": layers_out}


def streaming_ceiling(dev, sizes, reps=60):
    """One read-only kernel per buffer of each size (cl_probe_read), back to back
    over >= 1 GiB of rotating slices: the best one launch of that size reaches."""
    import torch
    import compressed_linear_amd as cla
    L = cla.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    out = []
    for sz in sizes:
        sz16 = (int(sz) + 255) // 256 * 256
        copies = max(4, -(-ROTATE_BYTES // sz16))
        buf = torch.ones(copies * sz16 // 4, dtype=torch.int32, device=dev)
        sink = torch.zeros(int(L.cl_probe_read_sink_words(sz16)) + 1, dtype=torch.int32, device=dev)
        base, sk = buf.data_ptr(), sink.data_ptr()
        for i in range(copies):
            assert L.cl_probe_read(base + i * sz16, sz16, sk, sp) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            L.cl_probe_read(base + (i % copies) * sz16, sz16, sk, sp)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out.append({"bytes": int(sz), "us": round(us, 3), "GBps": round(sz / us / 1e3, 1)})
        del buf, sink
    torch.cuda.empty_cache()
    return out


def launch_floor(dev, reps=2000):
    """Back-to-back empty one-wavefront kernels (cl_probe_empty): us per launch."""
    import torch
    import compressed_linear_amd as cla
    L = cla.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    for _ in range(50):
        L.cl_probe_empty(sp)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        L.cl_probe_empty(sp)
    e1.record(stream)
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / reps, 3)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--path", default="auto")
    ap.add_argument("--graph", action="store_true",
                    help="record one pass over the rotating copies into a HIP graph and time its replays")
    ap.add_argument("--act-scale", type=float, default=0.0,
                    help="scale this fraction of each layer's input channels (SLiM's output-error variant)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads, the streaming-read ceiling and the launch floor")
    ap.add_argument("--per-layer", action="store_true", help="also time each layer alone")
    ap.add_argument("--fit", nargs="?", const="lut", choices=["lut", "int"],
                    help="time a data-free packer (LUT k-means, or the int4 2:4 clip search) instead of the forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for the byte counters)")
    a = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU; multi-GPU runs (--gpus > 1) are not part of it.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from synth.layers import CONFIGS

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}), flush=True)
        return
    if a.fit:
        return bench_fit(a, dev)
    cfg, M = a.config, a.M
    default_run = cfg == 5 and M == 1 and a.path == "auto" and not a.graph and a.act_scale == 0

    res = measure(cfg, M, a, dev, a.steps, a.warmup, per_layer=a.per_layer or default_run, graph=a.graph,
                  act_scale=a.act_scale)
    built = res["built"]
    us_per_layer = res["ms_per_step"] * 1e3 / res["n_launch"]
    roof = roofline(cfg, M, a.path, built, res["set_bytes"], us_per_layer, a.graph)

    extras = {}
    if not a.no_extras and M <= 32:
        sizes = [layer_bytes(acct, l.K, l.N, M) for l, acct, _ in built]
        ceil = streaming_ceiling(dev, sizes)
        ceil_us = sum(c["us"] for c in ceil) / len(ceil)
        extras["streaming_read_ceiling"] = {
            "per_layer": ceil, "us_per_layer": round(ceil_us, 3),
            "GBps": round(res["set_bytes"] / len(ceil) / ceil_us / 1e3, 1),
            "kernel": "cl_probe_read: one read-only kernel per layer-sized buffer, 16-byte nontemporal loads, "
                      "back to back over >= 1 GiB of rotating slices"}
        roof["frac_of_streaming_ceiling"] = round(ceil_us / us_per_layer, 4)
        extras["launch_floor"] = {"us_per_launch": launch_floor(dev),
                                  "kernel": "cl_probe_empty: back-to-back empty one-wavefront launches"}
        log(f"streaming ceiling {ceil_us:.2f} us/layer, launch floor {extras['launch_floor']['us_per_launch']} us")
    if default_run and not a.no_extras:
        other = {}
        for c in (1, 2, 3):
            r = measure(c, 1, a, dev, max(50, a.steps // 2), a.warmup)
            usl = r["ms_per_step"] * 1e3 / r["n_launch"]
            other[f"config {c}"] = {
                "workload": CONFIGS[c]["desc"] + ": " + ", ".join(f"{n} {K}->{N}" for n, K, N in CONFIGS[c]["layers"]),
                "batch": 1, "us_per_layer": round(usl, 3), "GBps": round(r["gbs"], 1),
                "frac_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_step": int(r["set_bytes"]),
                "traffic": read_traffic(c, 1)}
        extras["other_workloads"] = other

    cpu = None
    if not a.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        cpu = cpu_baseline([(l, acct) for l, acct, _ in built], res["xs_np"])
        log(f"  {cpu}")

    dtype = "bf16 x, fp16 weights, f32 acc" if built[0][0].x_dtype == "bf16" else "f16"
    layers_desc = ", ".join(f"{n} {K}->{N}" for n, K, N in CONFIGS[cfg]["layers"])
    gbs = res["gbs"]
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": a.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "us_per_layer": round(us_per_layer, 3),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; LLaMA layer shapes, random codes/LUTs/outliers/factors)",
        "config": {"workload": f"{CONFIGS[cfg]['desc']}: {layers_desc}"
                   + (" (HIP graph replay)" if a.graph else "")
                   + (f", {a.act_scale:.1%} of input channels scaled" if a.act_scale > 0 else ""), "batch": M,
                   "layers_per_step": res["n_launch"], "rotating_copies": res["rotating"],
                   "algorithmic_bytes_per_step": int(res["set_bytes"])},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_layer": res["per_layer"],
    }
    out.update(extras)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
