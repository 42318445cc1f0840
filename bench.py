#!/usr/bin/env python3
"""Benchmark of the fused tensor-parallel BF16 GEMM + reduction on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the fused kernel over one batch of synthetic input
already resident in HBM.  The default workload is the M=4096, N=6288, K=7168
GEMM-AR with 7 emulated peer partials.  W untimed steps run first, then K
steps are timed back to back with HIP events on the stream the kernel is
launched on; one JSON line goes to stdout.

Besides the throughput, the line carries
  roofline      the kernel's algorithmic flops per launch over its measured
                average launch time, against the MI355X dense bf16 MFMA peak,
                and the HBM traffic per launch measured by rocprofv3 counters
                (profiles/traffic.json; null when the kernel source changed
                since the counters were taken)
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
                on this host's cores (a reported baseline, not the target)

One GPU only: there is no multi-GPU path, and --gpus above 1 exits.
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "TFLOP/s + % bf16 MFMA peak, fused GEMM-AR at M=4096,N=6288,K=7168"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "tensor_bf16_gemm_amd", "csrc", f)
                  for f in ("gc_kernel.hpp", "gemm_coll.hip")]


def source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Each operand once: A, B, the peer rows actually read, the outputs."""
    e = 2
    if w.mode == "ag":
        return e * (w.R * w.M * w.K + w.K * w.N + w.R * w.M * w.N)
    base = e * (w.M * w.K + w.K * w.N)
    if w.mode == "ar":
        return base + e * ((w.R - 1) * w.M * w.N + w.M * w.N)
    P = -(-w.M // w.R)
    lo, hi = min(w.rank * P, w.M), min(w.rank * P + P, w.M)
    owned = hi - lo
    if w.mode == "ar2":   # peers of the slice in; ws, out slice and R-1 peer slices out
        return base + e * ((w.R - 1) * owned * w.N + (w.M - owned) * w.N + w.R * owned * w.N)
    return base + e * ((w.R - 1) * owned * w.N + P * w.N + (w.M - owned) * w.N)


def make_step(w, x):
    import torch
    import tensor_bf16_gemm_amd as gc
    dev = x["B"].device
    if w.mode == "ar":
        out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        return lambda: gc.gemm_ar(x["A"], x["B"], x["peers"], out, R=w.R, rank=w.rank)
    if w.mode == "rs":
        P = -(-w.M // w.R)
        out = torch.empty((P, w.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        return lambda: gc.gemm_rs(x["A"], x["B"], x["peers"], ws, out, R=w.R, rank=w.rank)
    if w.mode == "ar2":
        out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        peer_out = torch.empty((w.R - 1, w.M, w.N), dtype=torch.bfloat16, device=dev)
        return lambda: gc.gemm_ar_two_shot(x["A"], x["B"], x["peers"], ws, peer_out, out, R=w.R,
                                           rank=w.rank)
    out = torch.empty((w.R * w.M, w.N), dtype=torch.bfloat16, device=dev)
    flags = torch.ones(w.R, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    return lambda: gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, out, R=w.R,
                              rank=w.rank, epoch=1)


def read_traffic(w, kernel_us: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source for this workload."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(w.name)
    if not entry or entry.get("source_digest") != source_digest():
        return None
    return entry.get("bytes_per_launch")


def _counter_means(run_dir: str, counter: str) -> dict:
    """Mean value of `counter` per kernel name over the dispatches recorded in
    a rocprofv3 --pmc run directory (its *counter_collection.csv files); rows
    of one dispatch (one per counter instance, where the tool splits them)
    are summed first."""
    import csv
    import glob
    per: dict = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    key = (f, r["Dispatch_Id"])
                    name, v = per.get(key, (r["Kernel_Name"], 0.0))
                    per[key] = (name, v + float(r["Counter_Value"]))
    vals: dict = {}
    for name, v in per.values():
        vals.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in vals.items()}


def ingest_counters(name: str, fetch_dir: str, write_dir: str, cal_fetch_dir: str,
                    cal_write_dir: str) -> dict:
    """HBM bytes per step of the fused path from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of this benchmark, and the
    same two counters for `--calibrate-copy` (a 1 GiB device copy, so 1 GiB
    read and 1 GiB written).  Each counter is divided by what it reads for the
    copy per byte moved.  A step is one launch of each gc_kernel instance the
    call makes (two where full rounds of whole tiles precede a split tail),
    so the per-instance means are summed.  Writes the entry into
    profiles/traffic.json."""
    n = 1 << 30

    def kernel_kib(d, counter):
        m = _counter_means(d, counter)
        ks = [k for k in m if "gc_kernel" in k]
        if not ks:
            raise SystemExit(f"{d}: no gc_kernel entry for {counter}")
        return sum(m[k] for k in ks), {k: m[k] for k in ks}

    def copy_kib(d, counter):
        m = _counter_means(d, counter)
        if not m:
            raise SystemExit(f"{d}: no {counter} records")
        return max(m.values())          # the 1 GiB copy dominates every other kernel

    f_fetch = copy_kib(cal_fetch_dir, "FETCH_SIZE") * 1024 / n
    f_write = copy_kib(cal_write_dir, "WRITE_SIZE") * 1024 / n
    fk, fparts = kernel_kib(fetch_dir, "FETCH_SIZE")
    wk, wparts = kernel_kib(write_dir, "WRITE_SIZE")
    fetch = fk * 1024 / f_fetch
    write = wk * 1024 / f_write
    entry = {"source_digest": source_digest(), "bytes_per_launch": fetch + write,
             "fetch_bytes": fetch, "write_bytes": write,
             "copy_factor_fetch": f_fetch, "copy_factor_write": f_write,
             "instances": {k: {"fetch_bytes": fparts[k] * 1024 / f_fetch,
                               "write_bytes": wparts.get(k, 0.0) * 1024 / f_write}
                           for k in fparts}}
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        t = {}
    t.setdefault("workloads", {})[name] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return entry


def unfused_parts(w, x) -> dict:
    """The unfused pipeline on the same inputs: a library GEMM (torch.matmul,
    hipBLASLt) writing the local product in bf16, then the reduction kernel
    gemm_coll_peer_sum over the rows this rank keeps (AR: all; RS and
    two-shot AR: its slice, the local product being the published partial;
    two-shot AR also copies the slice into the R-1 peer outputs).  AG: the
    all-gather's data movement on one GPU -- a copy of the R shards (the
    other ranks' from the receive buffer, this rank's from A) into one
    [R*Ms, K] buffer -- then one GEMM on it.  Returns the whole step and its
    parts as callables."""
    import torch
    import tensor_bf16_gemm_amd as gc
    dev = x["B"].device
    B = x["B"]
    copies = None
    pre = None
    if w.mode == "ag":
        gathered = torch.empty((w.R, w.M, w.K), dtype=torch.bfloat16, device=dev)
        r = w.rank

        def gather():
            # contiguous slice copies (the other ranks' shards), then A
            if r > 0:
                gathered[:r].copy_(x["shards"][:r])
            if r + 1 < w.R:
                gathered[r + 1:].copy_(x["shards"][r + 1:])
            gathered[r].copy_(x["A"])
        pre = gather
        a_in = gathered.view(w.R * w.M, w.K)
        local = torch.empty((w.R * w.M, w.N), dtype=torch.bfloat16, device=dev)
        reduce = None
    else:
        a_in = x["A"]
        local = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        if w.mode == "ar":
            out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
            reduce = lambda: gc.peer_sum(local, x["peers"], out)
        else:
            P = -(-w.M // w.R)
            lo, hi = min(w.rank * P, w.M), min(w.rank * P + P, w.M)
            out = torch.empty((hi - lo, w.N), dtype=torch.bfloat16, device=dev)
            reduce = lambda: gc.peer_sum(local[lo:hi], x["peers"][:, lo:hi], out)
            if w.mode == "ar2":
                peer_out = torch.empty((w.R - 1, w.M, w.N), dtype=torch.bfloat16, device=dev)
                copies = lambda: peer_out[:, lo:hi].copy_(out.unsqueeze(0).expand(w.R - 1, -1, -1))
    gemm = lambda: torch.matmul(a_in, B, out=local)

    def step():
        if pre is not None:
            pre()
        gemm()
        if reduce is not None:
            reduce()
        if copies is not None:
            copies()

    what = ("torch.matmul (hipBLASLt) to a bf16 local product, then gemm_coll_peer_sum"
            + (" and the slice copies" if copies is not None else "")
            if w.mode != "ag" else "copy of the R shards into one buffer (the all-gather's "
            "data movement), then torch.matmul (hipBLASLt) on it")
    return {"step": step, "gemm": gemm, "reduce": reduce, "gather": pre, "what": what}


def read_sclk() -> list:
    """Active shader-clock levels (MHz) of the driver's sysfs tables
    pp_dpm_sclk (the lines marked '*'); empty where they are not readable.
    (A file read: no other program is started from this process.)"""
    import glob
    import re
    out = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as fh:
                for line in fh:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            out.append(int(m.group(1)))
        except OSError:
            pass
    return out


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if v else None


def compare_fused_unfused(w, x, fused_step, blocks: int = 12, per_block: int = 20,
                          warm: int = 60) -> dict:
    """Fused against unfused in one window, so that both see the same clock:
    `warm` launches of each (a fixed warm-up, past the power-limit transient
    of about 60 launches), then `blocks` timed blocks of `per_block` launches
    alternating in the order F U U F F U U F ... (each leg equally often
    first).  Each block is timed with HIP events on the launch stream and
    nothing else runs on the host meanwhile.  Reports the median block of
    each leg, times the unfused parts alone (30 warm-up launches, then 40),
    and reads the shader clock from sysfs during one more, untimed block of
    each leg.  (A sysfs clock read inside a timed block slowed that block by
    up to 15 %.)"""
    import torch
    parts = unfused_parts(w, x)
    legs = {"fused": fused_step, "unfused": parts["step"]}
    st = torch.cuda.current_stream()
    est = {}
    for name, f in legs.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(warm):
            f()
        e1.record(st)
        torch.cuda.synchronize()
        est[name] = e0.elapsed_time(e1) / warm * 1e-3      # seconds per launch
    times = {"fused": [], "unfused": []}
    for b in range(blocks):
        name = ("fused", "unfused", "unfused", "fused")[b % 4]
        f = legs[name]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(per_block):
            f()
        e1.record(st)
        torch.cuda.synchronize()
        times[name].append(e0.elapsed_time(e1) / per_block * 1e3)

    def alone(f, n=40, warm_n=30):
        if f is None:
            return 0.0
        for _ in range(warm_n):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(n):
            f()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    # The unfused parts alone, right after the blocks (same window).
    part_us = {k: alone(parts[k]) for k in ("gemm", "reduce", "gather")}
    clocks = {"fused": [], "unfused": []}
    for name, f in legs.items():
        # At least 40 ms of work is queued; the clock is read as soon as it is
        # (for short launches the host only just keeps ahead of the GPU).
        n = max(per_block, int(0.04 / max(est[name], 1e-6)))
        for _ in range(n):
            f()
        clocks[name] += read_sclk()
        torch.cuda.synchronize()

    fu, uu = _median(times["fused"]), _median(times["unfused"])
    return {"fused_us": fu, "us_per_step": uu, "fused_speedup": uu / fu,
            "fused_blocks_us": times["fused"], "unfused_blocks_us": times["unfused"],
            "sclk_mhz_fused": _median(clocks["fused"]), "sclk_mhz_unfused": _median(clocks["unfused"]),
            "gemm_us": part_us["gemm"], "reduce_us": part_us["reduce"],
            "gather_us": part_us["gather"], "what": parts["what"],
            "method": f"one window: {warm} warm-up launches of each leg, then {blocks} blocks of "
                      f"{per_block} launches alternating F U U F ...; median block per leg; sclk "
                      "read from sysfs during one more, untimed block of each leg"}


def ag_arrival(w, x, resident_us: float, iters: int = 10, warmup: int = 3) -> dict:
    """AG-GEMM with the shards arriving during the call: ag_push_shards copies
    the other ranks' shards into a receive buffer through the DMA engines,
    raising each flag after its shard, in ring order.  Timed three ways per
    iteration (a fresh epoch each): the pushes alone; the pushes and then the
    kernel on one stream; the kernel with the pushes on a side stream, which
    it consumes as they land (streams joined between iterations, so the
    receive buffer is never rewritten while it is read)."""
    import torch
    import tensor_bf16_gemm_amd as gc
    dev = x["B"].device
    R, rank = w.R, w.rank
    recv = torch.zeros_like(x["shards"])
    flags = torch.zeros(R, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((R * w.M, w.N), dtype=torch.bfloat16, device=dev)
    n_ep = 3 * (iters + warmup) + 1
    epochs = torch.arange(1, n_ep + 1, dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ep = [0]

    def push(stream):
        e = ep[0]
        gc.ag_push_shards(x["shards"], recv, flags, epochs[e:e + 1], R=R, rank=rank, stream=stream)

    def kernel(stream):
        gc.ag_gemm(x["A"], x["B"], recv, flags, status, out, R=R, rank=rank, epoch=ep[0] + 1,
                   stream=stream)

    def copy_only():
        push(main)
        ep[0] += 1

    def serial():
        push(main)
        kernel(main)
        ep[0] += 1

    def overlapped():
        side.wait_stream(main)
        kernel(main)
        push(side)
        main.wait_stream(side)
        ep[0] += 1

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(main)
        for _ in range(iters):
            f()
        s1.record(main)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / iters * 1e3

    copy_us = timed(copy_only)
    res = {"copy_only_us": copy_us, "copy_then_gemm_us": timed(serial), "overlapped_us": timed(overlapped),
           "resident_us": resident_us,
           "copy_GBps": (R - 1) * w.M * w.K * 2 / (copy_us * 1e-6) / 1e9,
           "status": int(status.item()),
           "what": "ag_push_shards (DMA-engine copies + flag per shard, ring order) on a side stream "
                   "while ag_gemm polls the flags, against copies then GEMM, and shards resident"}
    return res


def sample_sclk(step, seconds: float = 1.0) -> dict | None:
    """The shader clock while the step runs back to back: the active level of
    the driver's sysfs table pp_dpm_sclk, read half-way through about
    `seconds` of launches.  The chip is power-limited, so the clock under
    load is below the 2.4 GHz of the peak figures.  None where the file is
    not readable."""
    import torch
    if not read_sclk():
        return None
    t0 = time.perf_counter()
    samples = []
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        if time.perf_counter() - t0 > seconds / 2 and len(samples) < 8:
            samples.append(read_sclk())      # launches queued ahead keep the GPU busy
        torch.cuda.synchronize()
    vals = [v for s_ in samples for v in s_]
    if not vals:
        return None
    return {"sclk_mhz": max(set(vals), key=vals.count), "samples": vals[:8],
            "source": "active level of pp_dpm_sclk (sysfs) while the step runs back to back"}


def cpu_baseline(w, x, target_s: float):
    """Time the CPU oracle on leading rows of the workload (about target_s)."""
    import torch
    from oracle.oracle import load
    from workloads import bits
    orc = load()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    B = bits(x["B"].cpu())
    if w.mode == "ag":
        src = x["A"]
        peer_fn = lambda rows: None
        total_rows = w.R * w.M
    else:
        src = x["A"]
        peer_fn = lambda rows: bits(x["peers"][:, :rows].cpu().contiguous())
        total_rows = w.M

    def run(rows):
        A = bits(src[:rows].cpu().contiguous())
        P = peer_fn(rows)
        t0 = time.perf_counter()
        orc.ar_rows(A, B, P)
        return time.perf_counter() - t0

    probe = min(16, src.shape[0])
    dt = run(probe)
    rows = max(probe, min(src.shape[0], int(probe * target_s / max(dt, 1e-6))))
    dt = run(rows)
    flops = 2.0 * rows * w.N * w.K
    peers = "" if w.mode == "ag" else f", {w.R - 1} peer partials"
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of {total_rows} ({w.name}: all {w.N} columns, "
                  f"K={w.K}{peers}); {dt:.1f} s; {orc.acc} accumulation, plain loops",
        "seconds": dt,
        "rows": rows,
        "cpu": cpu_model(),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    # The clock settles within about 60 back-to-back launches at M=4096 (the
    # first ones run at a higher clock, then the power limit pulls it down
    # and it recovers): the default warmup runs past that transient.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock under load (sysfs pp_dpm_sclk)")
    ap.add_argument("--no-arrival", action="store_true",
                    help="AG only: skip the run with shards arriving during the call")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the unfused baseline (library GEMM + peer-sum kernel)")
    ap.add_argument("--profile", action="store_true",
                    help="for profiler runs: only the W warm-up and K timed steps (no unfused "
                         "comparison, cold launches, clock sampling, arrival or CPU baseline)")
    ap.add_argument("--cold-launches", type=int, default=30,
                    help="launches timed one by one after a 512 MiB write that evicts the L2 "
                         "and last-level caches (0 = skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="rocprofv3 --pmc run directories (FETCH_SIZE and WRITE_SIZE of this "
                         "benchmark, then of --calibrate-copy): write profiles/traffic.json")
    args = ap.parse_args(argv)
    if args.profile:
        # A profiler serializes dispatches: the AG arrival leg (a kernel that
        # polls flags raised by copies on another stream) would then wait out
        # its time-outs, and the other legs only add kernels to the trace.
        args.no_cpu_baseline = args.no_clock = args.no_arrival = args.no_unfused = True
        args.cold_launches = 0

    if args.ingest_counters:
        import workloads as wl
        name = args.workload or wl.HEADLINE
        print(json.dumps({name: ingest_counters(name, *args.ingest_counters)}))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the peer ranks are emulated by buffers in this GPU's memory); "
              "run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import tensor_bf16_gemm_amd as gc
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    gc.lib()  # fail loudly if the library is missing

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return 0

    name = args.workload or wl.HEADLINE
    w = wl.WORKLOADS[name]
    x = wl.make_inputs(w, device="cuda")
    step = make_step(w, x)
    # The fused-versus-unfused comparison runs first, in a window of its own
    # with a fixed warm-up (see compare_fused_unfused).  The W warm-up steps
    # and the K timed steps follow it directly.
    comparison = None
    if not args.no_unfused:
        comparison = compare_fused_unfused(w, x, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / max(args.steps, 1)

    # Cold launches: each one timed alone after a write of 512 MiB (twice
    # the last-level cache) has evicted A, B and the peers from the caches.
    cold = None
    if args.cold_launches > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_launches)]
        for i, (e0, e1) in enumerate(evs):
            flush.fill_(i & 255)
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        med = us[len(us) // 2]
        cold = {"launches": len(us), "median_us": med, "min_us": us[0],
                "median_tflops": w.flops / (med * 1e-6) / 1e12,
                "flush": "512 MiB device write before each launch, outside the events"}
        del flush

    flops = w.flops
    tflops = flops / (ms * 1e-3) / 1e12
    abytes = algorithmic_bytes(w)
    traffic = read_traffic(w, ms * 1e3)
    # The roofline that bounds this workload: the MFMA peak or, where the
    # algorithmic bytes take longer at the HBM peak than the flops at the
    # MFMA peak (small M), the HBM bandwidth.
    hbm_bound = abytes / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_BF16_TFLOPS * 1e12)
    gbs = abytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC if name == wl.HEADLINE else f"TFLOP/s, fused {w.mode.upper()} {name}",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "mode": w.mode, "M": w.M, "N": w.N, "K": w.K, "R": w.R,
                   "rank": w.rank, "global_batch": w.M * (w.R if w.mode == "ag" else 1),
                   "parallelism": f"tp{w.R} emulated on 1 GPU"},
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "achieved": gbs if hbm_bound else tflops,
            "peak": PEAK_HBM_GBS if hbm_bound else PEAK_BF16_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": gbs / PEAK_HBM_GBS if hbm_bound else tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "algorithmic_bytes": abytes,
            "hbm_frac_of_step": (abytes / (ms * 1e-3)) / (PEAK_HBM_GBS * 1e9),
            "kernel": f"gc_kernel mode {w.mode}",
            "timing": "HIP events on the launch stream around the timed steps",
        },
        "cold": cold,
        "preceded_by": None if comparison is None else
        "the fused/unfused comparison in unfused_baseline (its own warm-up and blocks), then "
        "the W warm-up steps",
        "wall_s": wall,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_clock:
        line["sclk"] = sample_sclk(step)
    if comparison is not None:
        line["unfused_baseline"] = comparison
    if w.mode == "ag" and not args.no_arrival:
        line["arrival"] = ag_arrival(w, x, ms * 1e3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
