"""Throughput of the attention forward pass on one MI355X.

One step = one fa_fwd call over the whole workload (all heads, all query tiles) with
Q, K, V, O, L resident in HBM. Default workload: causal bf16, B=4, H=16, N=4096,
d=128. Prints one JSON line. ``value`` is algorithmic TFLOP/s: 4 d FLOP per
admissible (query, key) pair -- 2d for the score, 2d for the weighted value row --
with N(N+1)/2 pairs per head when causal.

The roofline object compares the kernel against the MI355X published dense bf16
MFMA peak; ``traffic`` is the HBM traffic measured by rocprofv3 counters for the
same kernel source (null when the kernel source has changed since). The CPU
baseline times the fp64 oracle on a bounded sample of query rows on the host cores
of the machine that runs the benchmark, and checks the sampled rows of the GPU output
against it.

``--pass bwd`` times the backward pass instead (one fa_bwd call: the dQ and dK/dV
kernels, plus a preprocessing kernel for fp32) on the same workload with a seeded dO, with algorithmic
FLOP = 8 d per admissible pair (the products dV = P^T dO, dP = dO V^T, dQ = dS K and
dK = dS^T Q), and times the fp64 backward oracle on one head for the CPU baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % MFMA peak (bf16, causal, B4 H16 N4096 d128)"
METRIC_BWD = "attn bwd TFLOP/s & % MFMA peak (bf16, causal, B4 H16 N4096 d128)"


def metric_name(which: str, w) -> str:
    """The metric string for a pass and workload (METRIC / METRIC_BWD for the default one)."""
    mask = "causal" if w.causal else "non-causal"
    n = f"Nq{w.N} Nk{w.keys}" if w.keys != w.N else f"N{w.N}"
    return f"attn {which} TFLOP/s & % MFMA peak ({w.dtype}, {mask}, B{w.B} H{w.H} {n} d{w.d})"
# MI355X published dense peaks, TFLOP/s: 256 CUs x 2.4 GHz x 4096 bf16 FLOP/clk/CU;
# fp32 matrix 157.3.
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
# The forward kernel's sources: the device headers and the host source that launches them.
KERNEL_SOURCES = [os.path.join(ROOT, "tiled_online_softmax_amd", "csrc", f)
                  for f in ("fa_device.h", "fa_fwd_kernels.h", "fa_fwd.hip")]
# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, per workload and kernel source.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_kernel_{}_traffic.json")


def device_info(fa) -> dict:
    """The device as HIP reports it, beside the published peak the roofline uses: name,
    architecture, compute units and peak engine clock, and the dense peaks they imply
    (4096 bf16 / 256 fp32 matrix FLOP per clock and CU)."""
    import ctypes

    import torch

    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", "").split(":")[0],
            "compute_units": props.multi_processor_count}
    # hipDeviceGetAttribute from the HIP runtime the library is linked against;
    # attribute 5 is hipDeviceAttributeClockRate (peak engine clock, kHz).
    try:
        get = ctypes.CDLL(fa.LIB_PATH).hipDeviceGetAttribute
    except (OSError, AttributeError):
        return info
    get.restype = ctypes.c_int
    get.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    khz = ctypes.c_int(0)
    if get(ctypes.byref(khz), 5, 0) == 0 and khz.value > 0:
        ghz = khz.value / 1e6
        info["peak_sclk_ghz"] = round(ghz, 3)
        cu = props.multi_processor_count
        info["implied_peak_tflops"] = {"bf16": round(cu * ghz * 4096 / 1e3, 1), "f32": round(cu * ghz * 256 / 1e3, 1)}
    return info


def source_digest() -> str:
    """sha256 over the forward kernel's source files, in a fixed order."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    try:
        with open(TRAFFIC_FILE.format(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("source_sha256") != source_digest():
        return None
    return entry.get("bytes_per_launch")


def cpu_baseline(w, q, k, v, O, L, target_s: float):
    """Time the oracle on evenly spaced query rows of every head; check those rows."""
    import numpy as np

    import oracle

    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    heads = w.B * w.H

    def run(nrows):
        rows = np.unique(np.linspace(0, w.N - 1, nrows).round().astype(np.int64))
        t0 = time.perf_counter()
        Oref, Lref = oracle.attention(qn, kn, vn, w.causal, w.scale, rows=rows)
        return rows, Oref, Lref, time.perf_counter() - t0

    nrows = 8
    rows, Oref, Lref, t = run(nrows)
    # Grow the sample until it takes at least half the target time (or covers every row).
    while t < 0.5 * target_s and len(rows) < w.N:
        nrows = int(min(w.N, max(2 * nrows, nrows * target_s / max(t, 1e-3))))
        rows, Oref, Lref, t = run(nrows)
    pairs = (rows + 1).sum() if w.causal else len(rows) * w.N
    flops = 4.0 * w.d * float(pairs) * heads
    o = O.double().cpu().numpy()[:, :, rows]
    l = L.double().cpu().numpy()[:, :, rows]
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{len(rows)} evenly spaced query rows of each of the {heads} heads "
                  f"(full rows of S and P in fp64), {t:.1f} s",
        "seconds": t,
        "sampled_rows_max_abs_err": {"O": float(np.max(np.abs(o - Oref))),
                                     "L": float(np.max(np.abs(l - Lref)))},
    }


def cpu_baseline_cross(w, q, k, v, O, L, target_s: float):
    """Time the cross-attention oracle on whole heads, one after another, until about
    half the target time has passed; check those heads."""
    import numpy as np

    import oracle

    o = O.double().cpu().numpy()
    l = L.double().cpu().numpy()
    t, heads, eo, el = 0.0, 0, 0.0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            args = [x[sl].double().numpy() for x in (q, k, v)]
            t0 = time.perf_counter()
            Oref, Lref = oracle.attention_cross(*args, w.causal, w.scale)
            t += time.perf_counter() - t0
            heads += 1
            eo = max(eo, float(np.max(np.abs(o[sl] - Oref))))
            el = max(el, float(np.max(np.abs(l[sl] - Lref))))
            if t >= 0.5 * target_s:
                break
        if t >= 0.5 * target_s:
            break
    flops = 4.0 * w.d * float(w.pairs()) * heads
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{heads} whole heads of {w.B * w.H} (full Nq x Nk S and P in fp64), {t:.1f} s",
        "seconds": t,
        "sampled_heads_max_abs_err": {"O": eo, "L": el},
    }


def cpu_baseline_bwd(w, q, k, v, do, dQ, dK, dV):
    """Time the backward oracle on the first head (all rows: dK and dV need every
    query); check that head of the GPU gradients against it."""
    import numpy as np

    import oracle

    sl = (slice(0, 1), slice(0, 1))
    args = [t[sl].double().numpy() for t in (q, k, v, do)]
    t0 = time.perf_counter()
    ref = oracle.attention_bwd(*args, w.causal, w.scale)
    t = time.perf_counter() - t0
    flops = 8.0 * w.d * float(w.pairs())
    errs = {}
    for name, g, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        a = g[sl].double().cpu().numpy()
        errs[name] = float(np.max(np.abs(a - r)))
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"head (0, 0) of {w.B * w.H}, every row (full N x N S, P, dP, dS in fp64), {t:.1f} s",
        "seconds": t,
        "sampled_head_max_abs_err": errs,
    }


def copy_calibration(mib: int):
    """Three device-to-device copies of a known size: each reads and writes `mib` MiB.

    The sizes exceed the last-level cache, so every byte crosses HBM once each way;
    the counters' readings for these dispatches give the factor between the
    counter units and bytes.
    """
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": n * 4}), flush=True)


def vs_sdpa(names, steps: int, warmup_seconds: float, bwd: bool = False):
    """fa_fwd (or, with `bwd`, fa_bwd) beside torch's scaled_dot_product_attention (the
    fused attention PyTorch ships for this GPU; its backward through autograd with the
    graph kept) on the given workloads: HIP events on the launch stream around `steps`
    calls of each after a clock warm-up, and the largest difference between their
    outputs. Context for the pages' comparison with SDPA; one JSON line per workload."""
    import torch
    import torch.nn.functional as F

    import tiled_online_softmax_amd as fa
    from workloads import WORKLOADS

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warmup_seconds:
            for _ in range(16):
                fn()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    for name in names:
        w = WORKLOADS[name]
        if w.keys != w.N:
            raise SystemExit(f"--vs-sdpa takes self-attention workloads ({name} has N_k != N)")
        q, k, v = (t.to(dev) for t in w.make())
        O = torch.empty_like(q)
        L = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        if bwd:
            fa.fa_fwd(q, k, v, O, L, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)
            g = torch.Generator().manual_seed(1000 + w.seed)
            do = torch.randn((w.B, w.H, w.N, w.d), generator=g).to(q.dtype).to(dev)
            grads = [torch.empty_like(q) for _ in range(3)]
            work = torch.empty(2 * w.B * w.H * w.N, dtype=torch.float32, device=dev)
            ms_fa = timed(lambda: fa.fa_bwd(q, k, v, O, L, do, *grads, work, w.B, w.H, w.N, w.d, w.causal,
                                            w.scale, stream))
            qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
            out = F.scaled_dot_product_attention(qg, kg, vg, is_causal=w.causal, scale=w.scale)
            ms_sdpa = timed(lambda: torch.autograd.grad(out, (qg, kg, vg), do, retain_graph=True))
            ref = torch.autograd.grad(out, (qg, kg, vg), do, retain_graph=True)
            fa.fa_bwd(q, k, v, O, L, do, *grads, work, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)
            torch.cuda.synchronize()
            flops = 2 * w.flops()  # 8 d per pair: dV, dP, dQ, dK
            print(json.dumps({"vs_sdpa": name, "pass": "bwd", "dtype": w.dtype, "steps": steps,
                              "fa_bwd_us": round(ms_fa * 1e3, 2),
                              "fa_bwd_tflops": round(flops / (ms_fa * 1e-3) / 1e12, 1),
                              "sdpa_bwd_us": round(ms_sdpa * 1e3, 2),
                              "sdpa_bwd_tflops": round(flops / (ms_sdpa * 1e-3) / 1e12, 1),
                              "sdpa_over_fa": round(ms_sdpa / ms_fa, 2),
                              "max_abs_diff_dQ_dK_dV": [float((a.float() - r.float()).abs().max())
                                                        for a, r in zip(grads, ref)],
                              "torch": torch.__version__}), flush=True)
            continue
        ms_fa = timed(lambda: fa.fa_fwd(q, k, v, O, L, w.B, w.H, w.N, w.d, w.causal, w.scale, stream))
        ms_sdpa = timed(lambda: F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale))
        ref = F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale)
        fa.fa_fwd(q, k, v, O, L, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)
        torch.cuda.synchronize()
        flops = w.flops()
        print(json.dumps({"vs_sdpa": name, "dtype": w.dtype, "steps": steps,
                          "fa_fwd_us": round(ms_fa * 1e3, 2), "fa_fwd_tflops": round(flops / (ms_fa * 1e-3) / 1e12, 1),
                          "sdpa_us": round(ms_sdpa * 1e3, 2), "sdpa_tflops": round(flops / (ms_sdpa * 1e-3) / 1e12, 1),
                          "sdpa_over_fa": round(ms_sdpa / ms_fa, 2),
                          "max_abs_diff_O": float((O.float() - ref.float()).abs().max()),
                          "torch": torch.__version__}), flush=True)


def small_sweep(reps: int):
    """The pages' small-shape sweep: per configuration, the median latency of one
    fa_fwd call, of torch's scaled_dot_product_attention and of the explicit
    softmax(Q K^T) V in torch, all fp32 on this GPU; one JSON line each."""
    import statistics

    import torch

    import tiled_online_softmax_amd as fa
    from workloads import SMALL_SWEEP

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    F = torch.nn.functional

    def explicit(q, k, v, causal, scale):
        s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
        if causal:
            n = s.shape[-1]
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool, device=s.device).triu(1), float("-inf"))
        return torch.matmul(torch.softmax(s, dim=-1), v)

    def timed(fn):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        dev_us, host_us = [], []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            host_us.append((time.perf_counter() - t0) * 1e6)
            dev_us.append(a.elapsed_time(b) * 1e3)
        return statistics.median(dev_us), statistics.median(host_us)

    rows = []
    for w in SMALL_SWEEP:
        q, k, v = (t.to(dev) for t in w.make())
        O = torch.empty_like(q)
        L = torch.empty((1, 1, w.N), dtype=torch.float32, device=dev)
        ours = timed(lambda: fa.fa_fwd(q, k, v, O, L, 1, 1, w.N, w.d, w.causal, w.scale, stream))
        # The same call captured once into a HIP graph and replayed (no Python or
        # argument checks per launch).
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fa.fa_fwd(q, k, v, O, L, 1, 1, w.N, w.d, w.causal, w.scale)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fa.fa_fwd(q, k, v, O, L, 1, 1, w.N, w.d, w.causal, w.scale)
        replay = timed(graph.replay)
        sdpa = timed(lambda: F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale))
        expl = timed(lambda: explicit(q, k, v, w.causal, w.scale))
        ref = F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        rec = {"sweep": "small_shapes_f32", "workload": w.name, "N": w.N, "d": w.d, "causal": w.causal,
               "fa_fwd_us": round(ours[0], 2), "sdpa_us": round(sdpa[0], 2), "explicit_us": round(expl[0], 2),
               "fa_fwd_host_us": round(ours[1], 2), "sdpa_host_us": round(sdpa[1], 2),
               "fa_fwd_graph_replay_us": round(replay[0], 2), "fa_fwd_graph_replay_host_us": round(replay[1], 2),
               "explicit_host_us": round(expl[1], 2),
               "max_abs_diff_vs_sdpa": float((O - ref).abs().max()), "reps": reps}
        rows.append(rec)
        print(json.dumps(rec), flush=True)
    faster = sum(1 for r in rows if r["fa_fwd_us"] < r["sdpa_us"])
    print(json.dumps({"sweep": "small_shapes_f32", "configs": len(rows), "fa_fwd_faster_than_sdpa": faster,
                      "median_speedup_vs_sdpa": round(statistics.median(r["sdpa_us"] / r["fa_fwd_us"] for r in rows), 3),
                      "timing": "median over reps of HIP events around one call on the current stream "
                                "(*_host_us: host wall time of one call including launch and synchronisation)"}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed launches before the timed region (after the clock warm-up)")
    ap.add_argument("--warmup-seconds", type=float, default=1.0, metavar="S",
                    help="first keep launching untimed steps for S seconds of wall time: the GPU "
                         "clock ramps up over the first tens of milliseconds of sustained load, so "
                         "a short --warmup alone leaves it ramping inside the timed region")
    ap.add_argument("--workload", default=None, help="workload name (default: the causal bf16 B4 H16 N4096 d128)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=8, metavar="K",
                    help="record a HIP event pair around every K-th timed launch (per-launch kernel time)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward pass")
    ap.add_argument("--layout", choices=("contiguous", "bshd"), default="contiguous",
                    help="forward only: bshd stores Q, K, V, O as [B, N, H, d] and calls fa_fwd_strided")
    ap.add_argument("--specialize", action="store_true",
                    help="forward only: call fa_fwd_specialized (kernel compiled at run time for this shape)")
    ap.add_argument("--vs-sdpa", action="store_true",
                    help="instead of the benchmark, time fa_fwd (with --pass bwd: fa_bwd) beside torch's "
                         "scaled_dot_product_attention (its backward) on --workload (default: the large bf16 "
                         "workloads) and print one JSON line per workload")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark, run the small-shape fp32 sweep against torch SDPA")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run three plain device copies of MIB MiB each "
                         "(reference dispatches for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads are independent: each GPU would run this kernel on its share).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.vs_sdpa:
        names = ([args.workload] if args.workload else
                 ["causal_bf16_b4h16n4096d128", "long_causal_bf16_h32n16384d64"] + (
                     [] if args.which == "bwd" else ["ragged_wide_logits_bf16_n1000"]))
        vs_sdpa(names, steps=max(args.steps if args.which == "fwd" else min(args.steps, 100), 1),
                warmup_seconds=args.warmup_seconds, bwd=args.which == "bwd")
        return
    if args.sweep:
        small_sweep(reps=200)
        return

    import tiled_online_softmax_amd as fa
    from workloads import HEADLINE, WORKLOADS

    w = WORKLOADS[args.workload or HEADLINE]
    strided = args.layout == "bshd" or w.keys != w.N
    if args.specialize and (strided or args.which == "bwd"):
        print("--specialize applies to the contiguous forward pass", file=sys.stderr)
        sys.exit(2)
    if args.which == "bwd" and strided:
        print("the backward pass takes contiguous [B, H, N, d] tensors with Nq = Nk", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    q, k, v = w.make()
    if args.layout == "bshd":
        # [B, N, H, d] storage, viewed as [B, H, N, d]
        qd, kd, vd = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q, k, v))
    else:
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O = torch.empty_like(qd)
    L = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.which == "bwd":
        fa.fa_fwd(qd, kd, vd, O, L, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)
        g = torch.Generator().manual_seed(1000 + w.seed)
        do = torch.randn((w.B, w.H, w.N, w.d), generator=g).to(q.dtype)
        dod = do.to(dev)
        dQ, dK, dV = (torch.empty_like(qd) for _ in range(3))
        work = torch.empty(2 * w.B * w.H * w.N, dtype=torch.float32, device=dev)

        def step():
            fa.fa_bwd(qd, kd, vd, O, L, dod, dQ, dK, dV, work, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)
    elif strided:
        def step():
            fa.fa_fwd_strided(qd, kd, vd, O, L, w.causal, w.scale, stream)
    elif args.specialize:
        def step():
            fa.fa_fwd_specialized(qd, kd, vd, O, L, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)

        t_jit = time.perf_counter()
        step()  # compiles and loads the kernel for this shape
        torch.cuda.synchronize()
        t_jit = time.perf_counter() - t_jit
    else:
        def step():
            fa.fa_fwd(qd, kd, vd, O, L, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)

    # Clock warm-up: untimed steps until S seconds have passed (checked every 16 launches,
    # so the queue never runs dry), then the W counted warm-up steps.
    clock_steps = 0
    t_clock = time.perf_counter()
    while time.perf_counter() - t_clock < args.warmup_seconds:
        for _ in range(16):
            step()
        clock_steps += 16
        torch.cuda.synchronize()
    t_clock = time.perf_counter() - t_clock
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: HIP events on the stream the kernel is enqueued on, around the whole
    # region and around every `event_every`-th launch (the per-launch event pairs add a
    # few microseconds between launches, so the others run back to back).
    every = max(1, args.event_every)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(0, args.steps, every)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if i % every == 0:
            a, b = per[i // every]
            a.record(stream)
            step()
            b.record(stream)
        else:
            step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    launch_ms = sorted(a.elapsed_time(b) for (a, b) in per)
    ms_per_step = total_ms / args.steps
    avg_launch_ms = sum(launch_ms) / len(launch_ms)

    bwd = args.which == "bwd"
    flops = 2 * w.flops() if bwd else w.flops()  # backward: 8 d per pair
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = None if (bwd or strided or args.specialize) else measured_traffic(w.name)
    # backward: Q, K, V, O, dO read and dQ, dK, dV written once, plus L
    n_rows = w.B * w.H * w.N
    io_bytes = (2 * (w.io_bytes() - 4 * n_rows) + 4 * n_rows) if bwd else w.io_bytes()

    rec = {
        "metric": metric_name(args.which, w),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs, cast to the workload dtype)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel_ms": {"avg": round(avg_launch_ms, 5), "median": round(launch_ms[len(launch_ms) // 2], 5),
                          "min": round(launch_ms[0], 5), "max": round(launch_ms[-1], 5),
                          "launches_timed": len(launch_ms)},
            "algorithmic_flop_per_launch": flops,
            "algorithmic_bytes_per_launch": io_bytes,
        },
        "wall_s_timed": round(t_wall, 4),
        "clock_warmup": {"seconds": round(t_clock, 3), "steps": clock_steps,
                         "why": "untimed steps before the warm-up steps: the GPU clock ramps up "
                                "under sustained load"},
        "cpu_baseline": None,
        "device": device_info(fa),
    }
    if bwd:
        rec["roofline"]["kernel_ms"]["covers"] = ("one fa_bwd call: dQ and dK/dV kernels" +
                                                  (" and the preprocessing kernel" if w.dtype == "f32" else ""))
    if args.specialize:
        rec["config"]["specialized"] = True
        rec["jit_first_call_s"] = round(t_jit, 3)
        rec["roofline"]["kernel_ms"]["covers"] = "one fa_fwd_specialized call (kernel compiled for this shape)"
    if strided:
        rec["config"]["Nk"] = w.keys
        rec["config"]["layout"] = args.layout
        rec["roofline"]["kernel_ms"]["covers"] = "one fa_fwd_strided call"
    if not args.no_cpu_baseline:
        if bwd:
            rec["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, do, dQ, dK, dV)
        elif w.keys != w.N:
            rec["cpu_baseline"] = cpu_baseline_cross(w, q, k, v, O, L, args.cpu_seconds)
        else:
            rec["cpu_baseline"] = cpu_baseline(w, q, k, v, O, L, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
