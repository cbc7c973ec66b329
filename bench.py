"""Benchmark: remapped-position RoPE attention on one MI355X.

A step is one bifocal prefill over the 64K workload (B=1, 32 query / 8 KV
heads, d=128, w0=4096, s=2, bf16): every prefill step of the hot path
(rotation-index maps, fused RoPE tile loads, QK^T, online softmax, PV, the
bifocal merge). The same JSON line also carries the 128K bifocal prefill and
the 128K-cache bifocal decode (batch 1 and 8), each timed the same way.

Prints ONE JSON line. Inputs are seeded synthetic N(0,1) tensors (workloads/),
resident in HBM before timing starts. Each leg runs ~150 ms of warm-up steps;
its time per step is one pair of HIP events on the stream the kernels run on,
around all timed steps (exactly --steps for the headline leg, at least 100 ms
of work for the short legs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (% bf16 MFMA peak) at 64K/128K; decode KV GB/s at 128K"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector ALU (the fp32 prefill path)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def n_pairs(S: int, window_left: int) -> int:
    """Kept (i, j) pairs of causal attention with i - j <= window_left (-1: none)."""
    if window_left < 0 or window_left >= S - 1:
        return S * (S + 1) // 2
    w = window_left + 1
    return w * (w + 1) // 2 + (S - w) * w


def prefill_flops(w) -> float:
    left = w.window_left if w.mode != "bifocal" else -1  # every causal pair counts once in bifocal
    return 4.0 * w.d * w.Hq * w.B * n_pairs(w.S, left)


def prefill_bytes(w) -> float:
    """Compulsory HBM bytes of one prefill launch: q, k, v (and the ids) read
    once, o written once; no LSE (the bench does not request it)."""
    el = 2 if w.dtype == "bf16" else 4
    ids = 4 * w.B * w.S if w.mode != "nope" else 0
    return float(el * w.B * w.S * w.d * (2 * w.Hq + 2 * w.Hkv) + ids)


def roofline_time_us(flops: float, nbytes: float, peak_tflops: float):
    """The roofline's lower bound on a launch's time (us) and the unit that sets it."""
    t_mfma = flops / (peak_tflops * 1e12) * 1e6
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e6
    return (t_mfma, "mfma") if t_mfma >= t_hbm else (t_hbm, "hbm")


def kernel_source_sha(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "position_remapped_rope_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(tag: str, sha: str):
    """HBM traffic per launch from committed rocprofv3 PMC runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", f"{tag}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != sha:
        return None
    return t.get("bytes_per_launch")


def warm_for(fn, seconds: float):
    """Run fn back to back for about `seconds` (synchronising every 16 calls):
    after a host-side pause (input generation) the device first runs its
    short kernels at lower, changing clocks, which a few warm-up steps of a
    100 us kernel do not cover."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_steady(fn, steps: int, warmup: int, min_seconds: float = 0.0):
    """After ~150 ms of warm-up, time `steps` steps, or more if they would
    take under `min_seconds` (a 100 us step is short next to the device's
    clock changes). Returns (ms per step, steps timed)."""
    warm_for(fn, 0.15)
    if min_seconds > 0:
        est, _ = time_launches(fn, 3, 0)
        steps = max(steps, math.ceil(min_seconds * 1e3 / max(est, 1e-4)))
    avg, _ = time_launches(fn, steps, warmup)
    return avg, steps


def time_launches(fn, steps: int, warmup: int):
    """Average ms per step over `steps` steps, from one pair of events on the
    launch stream around all of them (synchronised on both sides), and the
    host wall time. A marker per step would put ~10 us of command-processor
    work between consecutive kernels, which a 100 us decode step cannot hide."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def item_trace_summary(step, launches=50):
    """Item phases of the bf16 prefill kernel from a trace build
    (`python -m position_remapped_rope_amd.build --trace OUT.so`, loaded with
    PROPE_LIB_PATH=OUT.so): `launches` back-to-back launches, then the
    timestamps of the last one, per workgroup and item, as medians in us. The
    kernel's 100 MHz real-time counter gives 10 ns resolution."""
    import ctypes
    import numpy as np
    import torch
    import position_remapped_rope_amd as P
    L = P.lib()
    if not hasattr(L, "prope_item_trace_read"):
        raise SystemExit("--item-trace needs the trace build: python -m position_remapped_rope_amd.build "
                         "--trace OUT.so, then PROPE_LIB_PATH=OUT.so")
    L.prope_item_trace_read.restype = ctypes.c_int
    L.prope_item_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    wgs, slots = 1024, 64
    buf = np.zeros(wgs * slots, dtype=np.uint64)
    torch.cuda.synchronize()
    assert L.prope_item_trace_read(buf.ctypes.data, buf.nbytes) == 0  # clears the table
    for i in range(launches):
        step(i)
    torch.cuda.synchronize()
    assert L.prope_item_trace_read(buf.ctypes.data, buf.nbytes) == 0
    return {"launches": launches, **summarize_item_trace(buf.reshape(wgs, slots))}


def summarize_item_trace(table, per_item=5):
    """Medians (us) of the item phases in an item-trace table: one row per
    workgroup of 100 MHz counter values, slot 0 at entry, slots 1 + 5k .. 5 + 5k
    for item k (start after the claim, end of the load and rotation setup,
    start of the tile loop, end of the loop, end of the item) and the last slot
    at exit; zero where nothing was recorded. non_loop_share is the part of the
    time from entry to the end of the last traced item spent outside tile
    loops (launch ramp, setup, prologue, finalize, claims)."""
    import numpy as np
    tr = np.asarray(table).astype(np.int64)
    slots = tr.shape[1]
    used = tr[:, 0] > 0
    tr = tr[used]
    t0 = tr[:, 0].min()
    us = lambda x: float(x) / 100.0
    names = ("setup", "prologue", "loop", "finalize")
    phases = {n: [] for n in names}
    gaps, overhead_share = [], []
    for r in tr:
        items = [r[1 + per_item * k: 1 + per_item * (k + 1)] for k in range((slots - 2) // per_item)]
        items = [it for it in items if (it > 0).all()]
        busy_loop = 0
        for k, it in enumerate(items):
            for n, d in zip(names, np.diff(it)):
                phases[n].append(us(d))
            busy_loop += it[3] - it[2]
            if k + 1 < len(items):
                gaps.append(us(items[k + 1][0] - it[4]))
        if items:  # share of the time from entry to the end of the last traced item
            overhead_share.append(1.0 - busy_loop / float(items[-1][4] - r[0]))
    med = lambda v: round(float(np.median(v)), 3) if v else None
    return {"workgroups": int(used.sum()), "items_traced": len(phases["loop"]),
            "median_us": {**{n: med(v) for n, v in phases.items()}, "claim_gap": med(gaps)},
            "launch_span_us": round(us(tr[:, slots - 1].max() - t0), 2),
            "workgroup_exit_us": [round(us(np.percentile(tr[:, slots - 1] - t0, q)), 2) for q in (0, 50, 100)],
            "non_loop_share_median": med(overhead_share)}


def bench_prefill(name, steps, warmup, unfused=False, min_seconds=0.0, item_trace=False):
    import torch
    import position_remapped_rope_amd as P
    import workloads as W
    w = W.get(name)
    log(f"{name}: generating inputs")
    inp = W.make_prefill_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, pos = (inp[n].to(dev) for n in ("q", "k", "v", "pos"))
    o = torch.empty_like(q)
    if w.mode == "bifocal":
        kw = dict(rope_base=w.rope_base, remap_scale=w.remap_scale, window_left=w.window_left)
    elif w.mode == "rope":
        kw = dict(rope_base=w.rope_base, period=w.period, window_left=w.window_left)
    else:
        kw = dict(window_left=w.window_left)
        pos = None

    if unfused:  # the pages' three-call construction merged by Eq. (7), for comparison
        ws = torch.empty(P.bifocal_unfused_workspace_size(w.B, w.S, w.Hq, w.d), dtype=torch.uint8, device=dev)

        def step(_):
            P.prefill_bifocal_unfused(q, k, v, pos, out=o, workspace=ws, **kw)
    else:
        def step(_):
            P.prefill(q, k, v, pos, mode=w.mode, out=o, **kw)

    log(f"{name}: timing" + (" (unfused)" if unfused else ""))
    avg, steps = time_steady(step, steps, warmup, min_seconds)
    flops = prefill_flops(w)
    tflops = flops / (avg * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_VECTOR_TFLOPS
    nbytes = prefill_bytes(w)
    t_roof, bound = roofline_time_us(flops, nbytes, peak)
    r = dict(avg_ms=avg, steps_timed=steps, flops=flops, tflops=tflops, frac=tflops / peak, bytes=nbytes,
             roofline_us=t_roof, roofline_bound=bound, frac_roofline=t_roof / (avg * 1e3))
    if item_trace:
        r["item_trace"] = item_trace_summary(step, launches=max(2, min(50, int(200.0 / max(avg, 1e-3)))))
    return w, inp, r


def bench_decode(name, steps, warmup, S=None):
    import torch
    import position_remapped_rope_amd as P
    import workloads as W
    w = W.get(name) if S is None else W.get(name).with_(S=S)
    log(f"{name}: generating inputs")
    inp = W.make_decode_inputs(w)
    dev = torch.device("cuda:0")
    kv_bytes = inp["k_cache"].numel() * 2 * 2
    # rotate between cache copies so the timed reads are not served by the 256 MB MALL
    copies = max(1, math.ceil(1.5e9 / kv_bytes))
    caches = []
    for c in range(copies):
        caches.append((inp["k_cache"].to(dev), inp["v_cache"].to(dev)))
    q = inp["q"].to(dev)
    kv_len = inp["kv_len"].to(dev)
    o = torch.empty_like(q)
    ws = torch.empty(P.decode_workspace_size(w.B, w.S, w.Hq, w.d), dtype=torch.uint8, device=dev)
    kw = dict(rope_base=w.rope_base, remap_scale=w.remap_scale, window_left=w.window_left)

    def step(i):
        kc, vc = caches[i % copies]
        P.decode(q, kc, vc, kv_len, mode="bifocal", out=o, workspace=ws, **kw)

    log(f"{name}: timing over {copies} cache copies")
    avg, steps = time_steady(step, steps, warmup, min_seconds=0.1)
    gbs = kv_bytes / (avg * 1e-3) / 1e9
    return dict(avg_ms=avg, bytes=kv_bytes, gbs=gbs, frac=gbs / PEAK_HBM_GBS, copies=copies, steps_timed=steps)


def bench_copy(steps, warmup, nbytes=1 << 30):
    """A plain streaming copy of known size (y = 1 * x, fp32, torch's elementwise kernel):
    the yardstick that converts the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    x = torch.randn(nbytes // 4, device="cuda:0")
    y = torch.empty_like(x)

    def step(_):
        torch.mul(x, 1.0, out=y)

    avg, _ = time_steady(step, steps, warmup, min_seconds=0.1)
    return dict(avg_ms=avg, read_bytes=nbytes, write_bytes=nbytes, gbs=2 * nbytes / (avg * 1e-3) / 1e9)


def bench_rope_apply(steps, warmup, S=131072, H=8, d=128):
    """prope_rope_apply on a 128K-token, 8-head bf16 K tensor (the base-rotated
    cache of the decode workload), out of place: bytes = read x + write y."""
    import torch
    import position_remapped_rope_amd as P
    g = torch.Generator(device="cuda:0").manual_seed(0)
    x = torch.randn(1, S, H, d, device="cuda:0", generator=g).to(torch.bfloat16)
    y = torch.empty_like(x)
    pos = torch.arange(S, dtype=torch.int32, device="cuda:0").reshape(1, S)

    def step(_):
        P.rope_apply(x, pos, 1e6, out=y)

    avg, _ = time_steady(step, steps, warmup, min_seconds=0.1)
    nbytes = 2 * x.numel() * x.element_size()
    return dict(avg_ms=avg, bytes=nbytes, gbs=nbytes / (avg * 1e-3) / 1e9)


def bench_gemm(steps, warmup, n=8192):
    """Ceiling reference for the MFMA roofline: a large bf16 GEMM through torch
    (hipBLASLt), 2 n^3 flop per launch. Not part of the measured path."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)

    def step(_):
        torch.mm(a, b, out=c)

    avg, _ = time_steady(step, steps, warmup)
    return dict(avg_ms=avg, tflops=2.0 * n ** 3 / (avg * 1e-3) / 1e12)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, n_rows: int):
    """The fp64 oracle, as it stands, on a bounded sample of query rows of the same workload.
    Its matrix products run on the BLAS thread pool (the `cores` figure); its
    elementwise steps (rotations, exp) on one thread."""
    import numpy as np
    import oracle as O
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = affinity
    rng = np.random.default_rng(12345)
    rows = np.sort(rng.choice(w.S, size=n_rows, replace=False))
    q, k, v = (inp[n].double().numpy() for n in ("q", "k", "v"))
    pos = inp["pos"].numpy()
    t0 = time.perf_counter()
    O.prefill_ref(q, k, v, pos, "bifocal", rope_base=w.rope_base, remap_scale=w.remap_scale,
                  window_left=w.window_left, operand_round="bf16", rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * w.Hq * w.B * float(np.sum(rows + 1))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_rows} uniformly drawn query rows x all {w.Hq} heads of {w.name} "
                      f"({flops:.3e} algorithmic flop in {dt:.1f} s, fp64 NumPy)",
            "seconds": dt, "cpu_model": cpu_model(), "affinity_cpus": affinity, "blas_threads": int(threads)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-extra", action="store_true", help="skip the 128K prefill and decode lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--only", choices=["prefill_64k", "prefill_128k", "prefill_64k_unfused", "prope_local_8k",
                                       "nope_global_8k", "endprompt_fp32", "decode_b1", "decode_b8", "rope_apply",
                                       "copy"],
                    help="time one leg only and print its figures (for profiler runs)")
    ap.add_argument("--item-trace", action="store_true",
                    help="with --only on a bf16 prefill leg and a trace build: per-item phase times")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on a single GPU (no multi-GPU path); --gpus must be 1"}))
        sys.exit(2)

    import torch
    import position_remapped_rope_amd as P
    P.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.only:
        if args.only == "copy":
            name = "copy_1GiB_fp32"
            r = bench_copy(args.steps, args.warmup)
        elif args.only == "rope_apply":
            name = "rope_apply_128k_k"
            r = bench_rope_apply(args.steps, args.warmup)
        elif args.only in ("prope_local_8k", "nope_global_8k", "endprompt_fp32"):
            name = args.only
            _, _, r = bench_prefill(name, args.steps, args.warmup, min_seconds=0.1,
                                    item_trace=args.item_trace and name != "endprompt_fp32")
        elif args.only.startswith("prefill"):
            name = "bifocal_128k" if args.only == "prefill_128k" else "bifocal_64k"
            _, _, r = bench_prefill(name, args.steps, args.warmup, unfused=args.only.endswith("unfused"),
                                    item_trace=args.item_trace and not args.only.endswith("unfused"))
        else:
            name = "bifocal_decode_128k_b1" if args.only == "decode_b1" else "bifocal_decode_128k_b8"
            r = bench_decode(name, args.steps, args.warmup)
        print(json.dumps({"only": args.only, "workload": name, **r}), flush=True)
        return

    w, inp, pre = bench_prefill("bifocal_64k", args.steps, args.warmup)
    sha = kernel_source_sha(["prefill_bf16.hip", "prefill_common.hpp", "common.hpp", "internal.hpp"])
    traffic = load_traffic("prefill_bf16_bifocal_64k", sha)
    result = {
        "metric": METRIC,
        "value": round(pre["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["avg_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "mode": "bifocal", "w0": w.window_left, "s": w.remap_scale, "rope_base": w.rope_base,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(pre["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre["frac"], 4), "traffic": traffic,
                     "kernel": "prefill_bf16_kernel<128, BIFOCAL>",
                     "algorithmic_flop_per_launch": pre["flops"]},
    }
    extra = {}
    if not args.no_extra:
        w4, _, pre4 = bench_prefill("bifocal_128k", max(3, args.steps // 2), 1)
        extra["bifocal_128k"] = {"tflops": round(pre4["tflops"], 2), "frac_bf16_peak": round(pre4["frac"], 4),
                                 "avg_ms": round(pre4["avg_ms"], 3), "flop": pre4["flops"]}
        torch.cuda.empty_cache()
        _, _, unf = bench_prefill("bifocal_64k", max(3, args.steps // 2), 1, unfused=True)
        extra["bifocal_64k_unfused_eq7"] = {"tflops": round(unf["tflops"], 2), "avg_ms": round(unf["avg_ms"], 3),
                                            "fused_speedup": round(unf["avg_ms"] / pre["avg_ms"], 3)}
        # the other prefill workloads: P-RoPE local + NoPE global layers at 8K, EndPrompt in fp32
        for name, st in (("prope_local_8k", 20), ("nope_global_8k", 20), ("endprompt_fp32", 50)):
            _, _, r = bench_prefill(name, st, 3, min_seconds=0.1)
            extra[name] = {"tflops": round(r["tflops"], 2), "avg_ms": round(r["avg_ms"], 4), "flop": r["flops"],
                           "frac_peak": round(r["frac"], 4),
                           "peak": "bf16 MFMA 2500" if name != "endprompt_fp32" else "fp32 vector 157.3",
                           # the larger of the compute time at that peak and the
                           # compulsory q/k/v/ids/o traffic at 8 TB/s
                           "hbm_bytes": r["bytes"], "roofline_us": round(r["roofline_us"], 2),
                           "roofline_bound": r["roofline_bound"], "frac_roofline": round(r["frac_roofline"], 4)}
        for name, st in (("bifocal_decode_128k_b1", 50), ("bifocal_decode_128k_b8", 10)):
            d = bench_decode(name, st, 3)
            extra[name] = {"gbs": round(d["gbs"], 1), "frac_hbm_peak": round(d["frac"], 4),
                           "avg_us": round(d["avg_ms"] * 1e3, 2), "steps_timed": d["steps_timed"],
                           "kv_bytes": d["bytes"],
                           "cache_copies": d["copies"]}
            torch.cuda.empty_cache()
        # not a benchmark configuration: the same decode on a 16K cache, where the
        # launch shrinks its chunks to keep the chip busy (latency-bound, for scale)
        d = bench_decode("bifocal_decode_128k_b1", 50, 3, S=16384)
        extra["bifocal_decode_16k_b1"] = {"gbs": round(d["gbs"], 1), "frac_hbm_peak": round(d["frac"], 4),
                                          "avg_us": round(d["avg_ms"] * 1e3, 2), "kv_bytes": d["bytes"],
                                          "note": "16K cache, not a benchmark configuration"}
        torch.cuda.empty_cache()
        ra = bench_rope_apply(20, 3)
        extra["rope_apply_128k_k"] = {"gbs": round(ra["gbs"], 1), "frac_hbm_peak": round(ra["gbs"] / PEAK_HBM_GBS, 4),
                                      "avg_us": round(ra["avg_ms"] * 1e3, 2), "bytes": ra["bytes"]}
        # what this machine reaches on plain library work, for scale: a bf16 GEMM
        # (MFMA ceiling in practice) and a 1 GiB streaming copy (HBM ceiling in practice)
        gm = bench_gemm(20, 3)
        cp = bench_copy(20, 3)
        props = torch.cuda.get_device_properties(0)
        extra["ceilings"] = {"bf16_gemm_8192_tflops": round(gm["tflops"], 1),
                             "copy_1GiB_gbs": round(cp["gbs"], 1),
                             "device": props.name, "compute_units": props.multi_processor_count}
        torch.cuda.empty_cache()
    result["extra"] = extra
    if not args.no_cpu:
        log("cpu baseline (oracle on sampled rows)")
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
