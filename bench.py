#!/usr/bin/env python3
"""Benchmark of the grouped tril mask softmax on one MI355X.

One step is one call of the whole operation (gtms_forward: decomposition, padded rows,
prefix loads, max, exp/sum, normalise, zero tails) over one batch of synthetic scores that
are already resident in HBM. The default workload is the larger of the README's two timed
binary32 shapes, X[12, 64, 1000, 1000] (its A10 timing at B = 12), with seeded lengths; the
other workloads are parity-test shapes and can be measured with --workload.

Prints ONE JSON line. value = effective HBM throughput over the algorithmic bytes of a
step: the kept lower-triangle reads plus the full S*S writes,
    bytes = esize * (sum_b M * L_b (L_b + 1) / 2 + B * M * S^2)
(--op backward: gtms_backward instead, reading two kept triangles, y and dy).
--variant band / mask measure the mask variants of the ScaledMaskSoftmax article instead:
a band lo <= c - r <= hi (default: a causal window of 512 columns), or an explicit byte
mask (default: the article's window mask tril(w), one [S, S] mask shared by every plane).
Their bytes count the reads of each row's column interval (the band itself; [0, L_b - 1]
for an explicit mask, which the kernel cannot narrow without reading the mask), the mask's
own bytes once, and the full writes.
The roofline object reports the same bytes over the kernel's average duration measured
with HIP events on the launch stream, against the 8 TB/s HBM peak of the MI355X. The
cpu_baseline object times the fp64 CPU oracle on the same workload on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix-core peak, published
METRIC = "ms and effective HBM GB/s (% of peak) for [B,M,S,S] masked softmax"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# the sources each kernel family is built from; a traffic figure is valid while they are
# unchanged
KERNEL_SOURCES = {
    family: [os.path.join(ROOT, "variable_length_causal_amd", "csrc", f) for f in files]
    for family, files in (
        ("softmax", ("device_common.h", "forward_kernels.h", "backward_kernels.h",
                     "gtms_api.hip", "launch.h", "launch_kind.hip")),
        ("attention", ("device_common.h", "attention_kernels.h", "gtms_api.hip", "launch.h",
                       "launch_attention.hip")))
}


def algorithmic_bytes(w: workloads.Workload, lens, op: str = "forward") -> int:
    """Kept-triangle reads (one tensor forward, y and dy backward) plus full writes."""
    S = w.S
    reads = sum(w.M * min(max(int(L), 0), S) * (min(max(int(L), 0), S) + 1) // 2 for L in lens)
    writes = w.B * w.M * S * S
    return w.esize * ((2 if op == "backward" else 1) * reads + writes)


def variant_bytes(w: workloads.Workload, lens, variant: str, lo: int, hi: int,
                  op: str = "forward", mask_bytes: int = 0) -> int:
    """Algorithmic bytes of a mask variant: interval reads (x forward; y and dy backward),
    the mask's bytes once, full writes."""
    S = w.S
    reads = 0
    for L in lens:
        Lc = min(max(int(L), 0), S)
        if variant == "band":
            r = np.arange(Lc)
            c0 = np.maximum(0, r + lo)
            c1 = np.minimum(Lc - 1, r + hi)
            reads += int(np.maximum(c1 - c0 + 1, 0).sum())
        else:
            reads += Lc * Lc
    reads *= w.M
    writes = w.B * w.M * S * S
    return w.esize * ((2 if op == "backward" else 1) * reads + writes) + mask_bytes


def attention_flops(w: workloads.AttnWorkload, lens) -> int:
    """Multiply-adds x 2 of the kept pairs (query r < L, key c <= r): D for q.k and D for
    the weighted sum of v, per pair."""
    pairs = sum(w.M * min(max(int(L), 0), w.S) * (min(max(int(L), 0), w.S) + 1) // 2
                for L in lens)
    return 4 * w.D * pairs


def plain_ceilings(xs, ys, n, stream, tensor_bytes):
    """Same-run rates of torch's own plain kernels on tensors of the workload's size, as
    context for the roofline fraction: a fill (stores only) and a copy (half reads). Each
    is timed like the step, n back-to-back launches between two events on the stream."""
    import torch
    out = {}
    for name, nbytes, op in (
            ("plain_fill_gbs", tensor_bytes, lambda i: ys[i % len(ys)].fill_(1.0)),
            ("plain_copy_gbs", 2 * tensor_bytes,
             lambda i: ys[i % len(ys)].copy_(xs[(i + 1) % len(xs)]))):
        for i in range(3):
            op(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            op(i)
        b.record(stream)
        torch.cuda.synchronize()
        out[name] = round(nbytes / (a.elapsed_time(b) / n * 1e-3) / 1e9, 1)
    out["what"] = ("torch fill_ and copy_ of one tensor of the workload's size, same GPU and "
                   "run; bytes = stores (fill), reads + stores (copy)")
    return out


def bench_attention(args):
    import torch
    import variable_length_causal_amd as g
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.ATTN_WORKLOADS[args.workload]
    lens = workloads.seq_lens(w)
    sl = torch.as_tensor(lens).to(dev)
    flops = attention_flops(w, lens)
    nsets = 2
    qkv = [[workloads.scores_device(w.shape, w.dtype, 1.0, w.x_seed + 3 * i + j, dev)
            for j in range(3)] for i in range(nsets)]
    outs = [torch.empty_like(qkv[0][0]) for _ in range(nsets)]
    torch.cuda.synchronize()

    def step(i):
        q, k, v = qkv[i % nsets]
        g.attention(q, k, v, sl, w.scale, out=outs[i % nsets], split=args.split)

    for i in range(args.warmup):
        step(i)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    achieved = flops / (avg_kernel_ms * 1e-3) / 1e12
    # after the timed region: per-launch events for the spread of single launch times
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(args.steps, 50))]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    if args.copy_calibration:  # plain copy of a known size, outside the timed region
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out = {
        "metric": "TFLOP/s of the fused attention with the grouped tril mask",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": workloads.DTYPE_NAMES[w.dtype],
        "data": "synthetic (seeded normal q, k, v generated on the device, seeded lengths)",
        "config": {"workload": w.name, "op": "attention", "split": args.split,
                   "B": w.B, "M": w.M, "S": w.S,
                   "D": w.D, "seq_lens": [int(v) for v in lens], "scale": w.scale,
                   "x_seed": w.x_seed, "len_seed": None if w.fixed_lens else w.len_seed,
                   "flops_per_step": flops,
                   "kernel_ms_min": round(float(np.min(kernel_ms)), 5),
                   "kernel_ms_median": round(float(np.median(kernel_ms)), 5)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(
                         f"{w.name}:attention" + ("" if args.split == "auto" else f":split-{args.split}"))},
        "cpu_baseline": None,
        "device": device_info(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_attention(qkv[0], outs[0], lens, w, args.cpu_budget)
    print(json.dumps(out), flush=True)


def cpu_baseline_attention(qkv_dev, o_dev, lens, w: workloads.AttnWorkload, budget_s: float):
    """Time the CPU oracle's attention, as it stands, on whole heads of the same input: one
    oracle call per head on T host threads, over the first k heads of every batch, k as many
    as fit the time budget (wall seconds). After the timing, the oracle's fp64 output of
    those heads is compared with the GPU's output o_dev of the same input: the largest
    absolute difference is reported."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    T = host_threads()
    probe_b = int(np.argmax(lens))
    one = [workloads.to_storage(t[probe_b:probe_b + 1, :1].cpu()) for t in qkv_dev]
    t0 = time.perf_counter()
    oracle.attention_f64(*one, lens[probe_b:probe_b + 1], w.scale, w.dtype)
    per_head = max(time.perf_counter() - t0, 1e-6)
    k = int(max(1, min(w.M, budget_s * T / (per_head * w.B))))
    qs, ks, vs = (workloads.to_storage(t[:, :k].contiguous().cpu()) for t in qkv_dev)
    tasks = [(b, m) for b in range(w.B) for m in range(k)]

    outs = {}

    def run(task):
        b, m = task
        outs[task] = oracle.attention_f64(qs[b:b + 1, m:m + 1], ks[b:b + 1, m:m + 1],
                                          vs[b:b + 1, m:m + 1], lens[b:b + 1], w.scale, w.dtype)

    with ThreadPoolExecutor(max_workers=T) as pool:
        t0 = time.perf_counter()
        list(pool.map(run, tasks))
        dt = time.perf_counter() - t0
    diff = 0.0
    for (b, m), ref in outs.items():
        got = o_dev[b, m].double().cpu().numpy()
        diff = max(diff, float(np.max(np.abs(got - ref[0, 0]))))
    sub = workloads.AttnWorkload(w.name, w.B, k, w.S, w.D, w.dtype, w.len_lo, w.len_hi)
    flops = attention_flops(sub, lens)
    what = "all heads" if k == w.M else f"heads m < {k} of every batch"
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": T,
        "kind": "oracle",
        "sample": f"{what} ({w.B * k} of {w.B * w.M} heads, {flops / 1e9:.2f} GFLOP) of the "
                  f"same seeded input, fp64 C oracle (single-threaded), one call per head on "
                  f"{T} host threads, {dt:.2f} s wall",
        "cpu": cpu_model(),
        "max_abs_diff_vs_gpu": diff,
    }


# hipDeviceAttribute_t ordinals (hip/hip_runtime_api.h, ROCm 7)
_HIP_ATTR_MEMORY_BUS_WIDTH, _HIP_ATTR_MEMORY_CLOCK_RATE, _HIP_ATTR_MULTIPROCESSOR_COUNT = 59, 60, 63


def device_info() -> dict:
    """What the runtime reports about GPU 0: name, compute units, and the HBM interface (memory
    clock in kHz, bus width in bits). The roofline's peak stays AMD's published 8 TB/s; these
    are context. The attribute ordinals are trusted only if the compute-unit count they give
    matches torch's."""
    import ctypes
    import torch
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "hbm_peak_published_gbs": HBM_PEAK_GBS}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return info
    v = ctypes.c_int()

    def attr(code):
        return v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), code, 0) == 0 else None
    if attr(_HIP_ATTR_MULTIPROCESSOR_COUNT) == props.multi_processor_count:
        info["hbm_clock_khz_reported"] = attr(_HIP_ATTR_MEMORY_CLOCK_RATE)
        info["hbm_bus_bits_reported"] = attr(_HIP_ATTR_MEMORY_BUS_WIDTH)
    return info


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_sources_hash(family: str = "softmax") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or
    None if there is none for this workload or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    family = "attention" if ":attention" in key else "softmax"
    if not ent or ent.get("kernel_sources_sha256") != kernel_sources_hash(family):
        return None
    return ent.get("hbm_bytes_per_launch")


def host_threads() -> int:
    """Host threads for the oracle baseline: the CPUs this process may run on, at most 16
    (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return int(max(1, min(16, n)))


def cpu_baseline(x_dev, y_dev, lens, w: workloads.Workload, budget_s: float,
                 max_host_bytes: int = 4 << 30):
    """Time the CPU oracle, as it stands, on whole planes of the same input: all planes if
    they fit the time budget (wall seconds) and the host-memory cap, else planes m < k of
    every batch. The oracle is single-threaded; independent planes run concurrently, one
    oracle call per plane, on T host threads (ctypes releases the GIL during each call).
    After the timing, the oracle's (rounded) output of those planes is compared with the
    GPU's output y_dev of the same input: the largest absolute difference is reported."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import torch
    T = host_threads()
    # estimate the per-plane cost from one plane of the largest length
    probe_b = int(np.argmax(lens))
    xs = workloads.to_storage(x_dev[probe_b:probe_b + 1, :1].cpu())
    t0 = time.perf_counter()
    oracle.softmax(xs, lens[probe_b:probe_b + 1], w.scale, w.dtype)
    per_plane = max(time.perf_counter() - t0, 1e-6)
    plane_bytes = w.S * w.S * w.esize
    k = int(max(1, min(w.M, budget_s * T / (per_plane * w.B),
                       max_host_bytes // (w.B * plane_bytes))))
    sample = workloads.to_storage(x_dev[:, :k].contiguous().cpu())
    torch.cuda.synchronize()
    tasks = [(b, m) for b in range(w.B) for m in range(k)]

    outs = {}

    def run(task):
        b, m = task
        outs[task] = oracle.softmax(sample[b:b + 1, m:m + 1], lens[b:b + 1], w.scale, w.dtype)

    with ThreadPoolExecutor(max_workers=T) as pool:
        t0 = time.perf_counter()
        list(pool.map(run, tasks))
        dt = time.perf_counter() - t0
    diff = 0.0
    for (b, m), ref in outs.items():
        got = y_dev[b, m].double().cpu()
        want = workloads.from_storage(ref[0, 0], w.dtype).double()
        diff = max(diff, float((got - want).abs().max()))
    sub = workloads.Workload(w.name, w.B, k, w.S, w.dtype, w.sigma, w.scale)
    nbytes = algorithmic_bytes(sub, lens)
    what = "all planes" if k == w.M else f"planes m < {k} of every batch"
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "sample": f"{what} ({w.B * k} of {w.B * w.M} planes, {nbytes / 1e6:.1f} MB "
                  f"algorithmic) of the same seeded input, fp64 C oracle (single-threaded), "
                  f"one call per plane on {T} host threads, {dt:.2f} s wall",
        "cpu": cpu_model(),
        "max_abs_diff_vs_gpu": diff,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    choices=sorted(k for k in workloads.WORKLOADS if "example" not in k) +
                    sorted(workloads.ATTN_WORKLOADS))
    ap.add_argument("--op", default="forward", choices=["forward", "backward", "attention"],
                    help="the forward (the headline), its backward, or the fused attention")
    ap.add_argument("--variant", default="tril", choices=["tril", "band", "mask"],
                    help="the grouped tril mask (the headline), a band, or an explicit mask")
    ap.add_argument("--band", default="-511,0",
                    help="band: lo,hi (kept when lo <= c - r <= hi); mask: hi = the w of "
                         "the window mask tril(w)")
    ap.add_argument("--path", default="auto", choices=["auto", "wave", "block", "stream"])
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--split", default="auto", choices=["auto", "off", "on"],
                    help="attention: the key split of each query tile (head size 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of known size (for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the operation shards by planes with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import variable_length_causal_amd as g

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.op == "attention":
        args.workload = args.workload or "attn_bf16_32x8x4096_d64"
        if args.workload not in workloads.ATTN_WORKLOADS:
            ap.error("--op attention takes an attention workload")
        return bench_attention(args)
    args.workload = args.workload or "readme_f32_12x64x1000"
    if args.workload not in workloads.WORKLOADS:
        ap.error(f"--op {args.op} takes a softmax workload")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.workload]
    lens = workloads.seq_lens(w)
    sl = torch.as_tensor(lens).to(dev)
    lo, hi = (int(v) for v in args.band.split(","))
    mask = None
    if args.variant == "mask":  # the window mask tril(w): kept where c - r <= hi
        mask = torch.ones(w.S, w.S, dtype=torch.uint8, device=dev).tril(hi)[None, None]
        lo = -w.S
    if args.variant == "tril":
        step_bytes = algorithmic_bytes(w, lens, args.op)
    else:
        step_bytes = variant_bytes(w, lens, args.variant, lo, hi, args.op,
                                   0 if mask is None else mask.numel())
    tensor_bytes = w.B * w.M * w.S * w.S * w.esize

    # rotate over enough (input, output) pairs that consecutive uses of one pair are
    # separated by far more than the 256 MB last-level cache; the inputs are resident
    # before the timed region starts
    nsets = int(min(4, max(1, (3 << 30) // tensor_bytes + 1)))
    if args.op == "backward":  # and one upstream gradient per set
        nsets = int(min(4, max(1, (3 << 30) // (2 * tensor_bytes) + 1)))
    xs = [workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed + i, dev) for i in range(nsets)]
    ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
    gs = []
    if args.op == "backward":
        for i in range(nsets):  # y = the forward's output, dy = normal
            if args.variant == "band":
                g.forward_band(xs[i], sl, lo, hi, w.scale, out=ys[i])
            elif args.variant == "mask":
                g.forward_masked(xs[i], mask, sl, w.scale, out=ys[i])
            else:
                g.forward(xs[i], sl, w.scale, out=ys[i])
            gs.append(workloads.scores_device(w.shape, w.dtype, 1.0, w.x_seed + 100 + i, dev))
    torch.cuda.synchronize()

    def step(i):
        x, y = xs[i % nsets], ys[i % nsets]
        if args.op == "backward":
            dy = gs[i % nsets]
            if args.variant == "band":
                g.backward_band(y, dy, sl, lo, hi, w.scale, out=x, path=args.path,
                                flags=args.flags)
            elif args.variant == "mask":
                g.backward_masked(y, dy, mask, sl, w.scale, out=x, path=args.path,
                                  flags=args.flags)
            else:
                g.backward(y, dy, sl, w.scale, out=x, path=args.path, flags=args.flags)
        elif args.variant == "band":
            g.forward_band(x, sl, lo, hi, w.scale, out=y, path=args.path, flags=args.flags)
        elif args.variant == "mask":
            g.forward_masked(x, mask, sl, w.scale, out=y, path=args.path, flags=args.flags)
        else:
            g.forward(x, sl, w.scale, out=y, path=args.path, flags=args.flags)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed region: K back-to-back steps; two events on the launch stream bracket it,
    # so the average launch duration is their interval over K (gaps between launches
    # included, which makes it slightly pessimistic)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    # after the timed region: per-launch events for the spread of single launch times
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(args.steps, 50))]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in ev]

    ceilings = plain_ceilings(xs, ys, min(args.steps, 50), stream, tensor_bytes)

    if args.copy_calibration:  # plain copy of a known size, outside the timed region
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (avg_kernel_ms * 1e-3) / 1e9
    key = args.workload + ("" if args.op == "forward" else ":backward") + \
        ("" if args.variant == "tril" else f":{args.variant}{lo},{hi}")
    traffic = measured_traffic(key)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic the kernels compute in: fp32 for every element type (the element
        # type of the tensors is config.io_dtype)
        "dtype": "f32",
        "data": "synthetic (seeded normal scores generated on the device, seeded lengths)",
        "config": {
            "workload": w.name,
            "op": args.op,
            "variant": args.variant if args.variant == "tril" else
            (f"band lo={lo} hi={hi}" if args.variant == "band" else f"mask tril({hi}) [1,1,S,S]"),
            "B": w.B, "M": w.M, "S": w.S,
            "io_dtype": workloads.DTYPE_NAMES[w.dtype],
            "seq_lens": [int(v) for v in lens],
            "scale": w.scale,
            "x_seed": w.x_seed,
            "len_seed": None if w.fixed_lens else w.len_seed,
            "path": args.path,
            "bytes_per_step": step_bytes,
            "kernel_ms_min": round(float(np.min(kernel_ms)), 5),
            "kernel_ms_median": round(float(np.median(kernel_ms)), 5),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
        "context": ceilings,
        "device": device_info(),
    }
    # the CPU oracle runs whole planes; planes beyond 2^26 elements (the 65536-wide rows) would
    # take minutes and tens of GB of host memory, so their lines carry no baseline
    if not args.no_cpu_baseline and args.op == "forward" and args.variant == "tril" \
            and w.S * w.S <= (1 << 26):
        step(0)  # the context kernels above overwrote ys: the forward of xs[0] again
        torch.cuda.synchronize()
        out["cpu_baseline"] = cpu_baseline(xs[0], ys[0], lens, w, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
