"""Throughput of the fused attention forward (or backward) on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload c3] [--pass fwd|bwd]

(The short launches l1, c1, c2 and c4 default to 200 warm-up and 200 timed steps.)

A step is one call of attn_fwd (the whole fused forward: Q tile load, K/V
staging, both matrix products, online softmax, normalisation, O and lse
stores) over one batch of seeded synthetic inputs already resident in HBM.
The default workload is causal bf16 attention with B=2, H=32, N=8192, d=128.
Prints one JSON line: throughput in TFLOP/s at the algorithmic count
4*B*H*N^2*d (halved when causal), the kernel's roofline figures, and the fp64
CPU oracle timed on a bounded sample of the same workload on the host cores.

With --pass bwd a step is one call of attn_bwd (D = rowsum(dO o O), then the
dQ and dK/dV kernels) on the forward's o and lse, counted at 2.5 times the
forward's flops (five N x N x d products instead of two).

With --workload m1|m2|m3 a step is one call of attn_fwd_masked (unequal query and
key lengths, a boolean mask packed once before timing), counted at 4*d flops per
visible (query, key) pair.

With --workload l1 a step is one call of attn_linear_fwd (causal linear
attention, fp32; with E = M = 64 the one-pass form: per 128-token span its own
products and state, the prefix of the earlier spans through the workspace, the
outputs; the workspace is allocated before timing), bound by HBM: the value is
algorithmic GB/s (read q, k, v and write o once) against the 8 TB/s peak.

The MFMA-bound lines also report, under roofline.practical_ceiling, this board's dense bf16
MFMA rate on random operands (the probe below, run for --practical-seconds right after the
bench) and the kernel's fraction of it.

With --probes it runs only the rate probes of libattn_probe.so (dense bf16 MFMA on
random and on constant operands; LDS reads as ds_read_b128, ds_read_b64 and
ds_read_b64_tr_b16) and prints one JSON line: each probe's rate, the shader clock
amd-smi reads while it runs, and the rate per compute unit and clock.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_c3_hbm_traffic.txt")
TRAFFIC_FILE_LINEAR = os.path.join(ROOT, "profiles", "attn_linear_fwd_l1_hbm_traffic.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "exact_attention_96_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch (per call of the entry point) from the committed counter
    summary, if it was taken on the current kernel source and this workload; else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.lstrip().startswith("#"):
                k, v = ln.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash() or kv.get("workload") != workload_name:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_avg(path: str, counter: str, name_part: str) -> float:
    """Mean per-dispatch value of a rocprofv3 --pmc counter for kernels whose name contains name_part."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {counter} rows for '{name_part}' in {path}")
    return sum(vals) / len(vals)


def _counter_step(path: str, counter: str, name_part: str) -> float:
    """Sum over the kernels whose name contains name_part of each one's mean per-dispatch
    counter value: the counter per call of an entry point that launches each once."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"no {counter} rows for '{name_part}' in {path}")
    return sum(sum(v) / len(v) for v in per.values())


def summarize_traffic(args) -> None:
    """Write the HBM traffic summary from two attention runs (FETCH_SIZE, WRITE_SIZE) and the
    same two counters on a plain device copy of known size (calibration)."""
    from exact_attention_96_amd.workloads import LINEAR_WORKLOADS, WORKLOADS
    # the launches of one call of the entry point (a step), summed: one kernel for the
    # forward and for the one-pass linear form, three for the chunked linear form
    if args.workload in LINEAR_WORKLOADS:
        w = LINEAR_WORKLOADS[args.workload]
        kern = "attn_linear_"
    else:
        w = WORKLOADS[args.workload]
        kern = "attn_fwd_"
    fetch_kib = _counter_step(args.fetch_csv, "FETCH_SIZE", kern)
    write_kib = _counter_step(args.write_csv, "WRITE_SIZE", kern)
    copy_fetch_kib = _counter_avg(args.copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    copy_write_kib = _counter_avg(args.copy_write_csv, "WRITE_SIZE", "copyBuffer")
    fetch_factor = args.copy_bytes / (copy_fetch_kib * 1024)
    write_factor = args.copy_bytes / (copy_write_kib * 1024)
    hbm = fetch_kib * 1024 * fetch_factor + write_kib * 1024 * write_factor
    lines = [
        f"# HBM traffic of {kern}* (every launch of one call) on {w.name}",
        "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch (rocprofv3 --pmc, one counter per run),",
        "# scaled by the ratio of known bytes to counter bytes on a device copy of copy_bytes.",
        f"workload = {w.name}",
        f"kernel_source_sha = {kernel_source_hash()}",
        f"fetch_kib_per_dispatch = {fetch_kib:.1f}",
        f"write_kib_per_dispatch = {write_kib:.1f}",
        f"copy_bytes = {args.copy_bytes}",
        f"copy_fetch_kib = {copy_fetch_kib:.1f}",
        f"copy_write_kib = {copy_write_kib:.1f}",
        f"fetch_factor = {fetch_factor:.4f}",
        f"write_factor = {write_factor:.4f}",
        f"hbm_bytes_per_launch = {hbm:.0f}",
        f"algorithmic_bytes_per_launch = {w.io_bytes}",
        f"traffic_over_algorithmic = {hbm / w.io_bytes:.3f}",
    ]
    if args.commands:
        lines += ["# commands:"] + [f"#   {c}" for c in args.commands]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _smi_gfx_clocks():
    """Current shader clocks (MHz, one per XCD) from amd-smi, or [] if unavailable."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi")
    if not exe:
        return []
    try:
        out = subprocess.run([exe, "metric", "--clock", "--json"], capture_output=True, text=True,
                             timeout=10).stdout
        data = json.loads(out)
    except (subprocess.SubprocessError, ValueError, OSError):
        return []
    gpus = data.get("gpu_data", data) if isinstance(data, dict) else data
    clocks = []
    for g in gpus if isinstance(gpus, list) else []:
        for name, c in (g.get("clock") or {}).items():
            if name.startswith("gfx_") and isinstance(c, dict):
                v = (c.get("clk") or {}).get("value")
                if isinstance(v, (int, float)):
                    clocks.append(float(v))
    return clocks


def sustained_clock(step, seconds: float = 1.5):
    """Shader clock (MHz) sampled with amd-smi while the same step runs back to back for
    `seconds` right after the timed region (the timed region itself is too short for the
    tool): per sample the mean of the per-XCD readings (the chip's aggregate clock; the
    highest reading is kept too), then the median over samples.  Returns a dict, or None
    without amd-smi."""
    import threading
    import torch
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            c = _smi_gfx_clocks()
            if not c:
                return
            samples.append(c)

    t = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    t.start()
    # steps are enqueued back to back; the host waits only every ~20 ms of work, so the
    # GPU does not idle between batches while it is sampled
    ev = torch.cuda.Event()
    while time.perf_counter() - t0 < seconds or (t.is_alive() and not samples and time.perf_counter() - t0 < 15):
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < 0.02:
            step()
        ev.record()
        ev.synchronize()
    torch.cuda.synchronize()
    stop.set()
    t.join(timeout=15)
    # readings below the lowest active DPM level (500 MHz) are an idle XCD
    kept = [[x for x in c if x >= 500.0] for c in samples]
    kept = [c for c in kept if c]
    if not kept:
        return None
    mean = sorted(sum(c) / len(c) for c in kept)
    top = sorted(max(c) for c in kept)
    low = sorted(min(c) for c in kept)
    return {"mhz_median": round(mean[len(mean) // 2], 1), "mhz_min": mean[0], "mhz_max": mean[-1],
            "mhz_fastest_xcd_median": top[len(top) // 2], "mhz_slowest_xcd_median": low[len(low) // 2],
            "samples": len(kept),
            "source": "amd-smi metric --clock (per-XCD gfx clocks) polled while the step repeats for "
                      f"{seconds:.1f} s right after the timed region; per sample the mean over the XCDs, "
                      "median over samples"}


def cpu_baseline(w, q, k, v, seconds: float):
    """The fp64 oracle (as it stands) on whole heads of the same workload, head after
    head until `seconds` of wall time have been spent (at least one head)."""
    import oracle
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        oracle.attn_rows(q[b, h], k[b, h], v[b, h], w.scale, w.causal, range(w.N))
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    flops = w.flops * done / (w.B * w.H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} of {w.B * w.H} heads, all {w.N} query rows each "
                      f"({flops:.3e} algorithmic flops in {dt:.1f} s)"}


def cpu_baseline_bwd(w, q, k, v, do, seconds: float):
    """The fp64 oracle backward on whole heads of the same workload, as many at once as
    the oracle has threads (it runs heads in parallel), batch after batch until
    `seconds` of wall time have been spent (at least one batch)."""
    import oracle
    T = max(1, oracle.num_threads())
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    while done < len(heads):
        batch = heads[done:done + T]
        sel = lambda x: x[[b for b, _ in batch], [h for _, h in batch]][None]  # noqa: E731
        oracle.attn_bwd(sel(q), sel(k), sel(v), sel(do), w.scale, w.causal)
        done += len(batch)
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    flops = 2.5 * w.flops * done / (w.B * w.H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": T, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} of {w.B * w.H} heads, whole heads, {min(T, done)} at a time "
                      f"({flops:.3e} algorithmic flops in {dt:.1f} s)"}


def visible_pairs(mw, mask) -> int:
    """Visible (query, key) pairs of one head: the mask (if any) and the bottom-right
    causal triangle (key j visible to query i iff j <= i + Nk - Nq)."""
    import torch
    vis = torch.ones((mw.Nq, mw.Nk), dtype=torch.bool) if mask is None else mask[0, 0].clone()
    if mw.causal:
        i = torch.arange(mw.Nq).view(-1, 1) + (mw.Nk - mw.Nq)
        vis &= torch.arange(mw.Nk).view(1, -1) <= i
    return int(vis.sum())


def cpu_baseline_masked(mw, q, k, v, mask, pairs: int, seconds: float):
    """The fp64 oracle's general-mask form on whole heads of the same workload, head
    after head until `seconds` of wall time have been spent (at least one head)."""
    import oracle
    heads = [(b, h) for b in range(mw.B) for h in range(mw.H)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attn_masked(q[sl], k[sl], v[sl], mw.scale, mw.causal, mask)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * mw.d * pairs * done
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} of {mw.B * mw.H} heads, all {mw.Nq} query rows each "
                      f"({flops:.3e} algorithmic flops in {dt:.1f} s)"}


def copy_probe(nbytes: int, steps: int):
    """A plain device copy of known size (counter calibration run)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "steps": steps}), flush=True)


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "exact_attention_96_amd", "libattn_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m exact_attention_96_amd.build)")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_mfma_bf16.argtypes = [vp, vp, ci, ci, vp]
    lib.attn_probe_lds_read.argtypes = [vp, ci, ci, ci, vp]
    return lib


def _probe_rate(launch, units_per_launch: float, seconds: float, clock_seconds: float):
    """Launches back to back for `seconds` (warm-up: the board settles at its clock for
    the load), then times 20 launches with one event pair; then the clock while the
    same launches repeat.  Returns (units per second, clock dict or None)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        launch()
        torch.cuda.synchronize()
    _, ms = time_steps(launch, 20, 0)
    rate = units_per_launch / (ms[0] * 1e-3)
    clock = sustained_clock(launch, clock_seconds) if clock_seconds > 0 else None
    return rate, clock


def run_probes(clock_seconds: float) -> None:
    """Sustained rates of the matrix cores and of LDS reads on this board (one JSON line).
    The published peaks assume the 2.4 GHz peak clock; under load the board holds a
    power-limited clock, and what a compute unit does per clock at that clock is what
    the attention kernels can be held to."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"probes": {}, "cus": cus, "device": torch.cuda.get_device_name(0)}
    # matrix cores: 1024 workgroups of 4 waves (two per SIMD), 2048 iterations of 8 products
    blocks, iters = 1024, 2048
    flops = blocks * 4 * iters * 8 * 32 * 32 * 16 * 2
    res = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    g = torch.Generator().manual_seed(20260101)
    operands = {"mfma_bf16_random": torch.randn(256 * 8 * 8, generator=g).to(torch.bfloat16),
                "mfma_bf16_ones": torch.ones(256 * 8 * 8, dtype=torch.bfloat16)}
    for name, ops in operands.items():
        opd = ops.to("cuda:0")

        def launch():
            rc = lib.attn_probe_mfma_bf16(opd.data_ptr(), res.data_ptr(), blocks, iters, stream)
            assert rc == 0, rc
        rate, clock = _probe_rate(launch, flops, 1.0, clock_seconds)
        tf = rate / 1e12
        entry = {"tflops": round(tf, 1), "frac_of_2516_6": round(tf / PEAK_MFMA_BF16_TFLOPS, 4)}
        if clock:
            entry["clock"] = clock
            entry["flop_per_clk_per_cu"] = round(rate / (cus * clock["mhz_median"] * 1e6), 1)
        out["probes"][name] = entry
        print(f"[probe] {name}: {json.dumps(entry)}", file=sys.stderr, flush=True)
    # LDS reads: 2048 workgroups of 8 waves with 64 KiB of LDS each (two per CU at a time)
    blocks, iters = 2048, 512
    resu = torch.empty(blocks * 512, dtype=torch.int32, device="cuda:0")
    for mode, (name, piece) in enumerate((("lds_read_b128", 16), ("lds_read_b64", 8), ("lds_read_b64_tr_b16", 8))):
        nbytes = blocks * 512 * iters * 8 * piece

        def launch():
            rc = lib.attn_probe_lds_read(resu.data_ptr(), blocks, iters, mode, stream)
            assert rc == 0, rc
        rate, clock = _probe_rate(launch, nbytes, 1.0, clock_seconds)
        entry = {"tb_per_s": round(rate / 1e12, 2)}
        if clock:
            entry["clock"] = clock
            entry["bytes_per_clk_per_cu"] = round(rate / (cus * clock["mhz_median"] * 1e6), 1)
        out["probes"][name] = entry
        print(f"[probe] {name}: {json.dumps(entry)}", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def practical_ceiling(seconds: float):
    """This board's dense bf16 MFMA rate on random operands (libattn_probe.so, the probe of
    --probes), launched back to back for `seconds` and then timed: the most a bf16 kernel
    with real data reaches here at the clock the board holds under that load.  None
    without the probe library."""
    import torch
    try:
        lib = _probe_lib()
    except (RuntimeError, OSError):
        return None
    blocks, iters = 1024, 2048
    flops = blocks * 4 * iters * 8 * 32 * 32 * 16 * 2
    res = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    g = torch.Generator().manual_seed(20260101)
    ops = torch.randn(256 * 8 * 8, generator=g).to(torch.bfloat16).to("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.attn_probe_mfma_bf16(ops.data_ptr(), res.data_ptr(), blocks, iters, stream)
        assert rc == 0, rc
    rate, _ = _probe_rate(launch, flops, seconds, 0.0)
    return rate / 1e12


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 200 for the sub-0.2 ms launches l1, c1, c2, c4)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 10; 200 for l1, c1, c2, c4: short launches "
                         "take ~100 calls to bring the board to its working clock)")
    ap.add_argument("--workload", default="c3",
                    help="c1..c5 (default: c3, the headline), m1..m3 (masked / unequal lengths), "
                         "or l1 (causal linear attention)")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time the CPU oracle runs whole heads for cpu_baseline (0: skip)")
    ap.add_argument("--cpu-heads", type=int, default=None, help="(0: skip the cpu_baseline leg)")
    ap.add_argument("--practical-seconds", type=float, default=1.0,
                    help="seconds of the random-operand MFMA probe for the practical ceiling "
                         "of the MFMA-bound lines (0: skip)")
    ap.add_argument("--clock-seconds", type=float, default=1.5,
                    help="seconds of repeated steps while amd-smi samples the shader clock (0: skip)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a device copy of this many bytes (counter calibration)")
    ap.add_argument("--probes", action="store_true",
                    help="only run the matrix-core and LDS rate probes (libattn_probe.so)")
    ap.add_argument("--summarize-traffic", action="store_true",
                    help="write the HBM traffic summary from rocprofv3 counter CSVs and exit")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--copy-fetch-csv")
    ap.add_argument("--copy-write-csv")
    ap.add_argument("--copy-bytes", type=int, default=268435456)
    ap.add_argument("--out", default=TRAFFIC_FILE)
    ap.add_argument("--commands", nargs="*", default=[])
    args = ap.parse_args()
    short = args.workload in ("l1", "c1", "c2", "c4") and args.which == "fwd"
    if args.steps is None:
        args.steps = 200 if short else 50
    if args.warmup is None:
        args.warmup = 200 if short else 10

    if args.summarize_traffic:
        summarize_traffic(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward is not sharded across "
              "GPUs in this library (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_96_amd as ea
    from exact_attention_96_amd.workloads import (LINEAR_WORKLOADS, MASKED_WORKLOADS, WORKLOADS, make_inputs,
                                                  random_grad)

    if args.copy_probe:
        copy_probe(args.copy_probe, max(args.steps, 1))
        return
    if args.probes:
        run_probes(args.clock_seconds)
        return
    if args.workload in LINEAR_WORKLOADS:
        if args.which != "fwd":
            print("linear attention times the forward only", file=sys.stderr)
            sys.exit(2)
        bench_linear(args, LINEAR_WORKLOADS[args.workload])
        return
    if args.workload in MASKED_WORKLOADS:
        if args.which != "fwd":
            print("masked workloads time the forward only", file=sys.stderr)
            sys.exit(2)
        bench_masked(args, MASKED_WORKLOADS[args.workload])
        return

    w = WORKLOADS[args.workload]
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v = make_inputs(w)
    dev = "cuda:0"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    bwd = args.which == "bwd"
    if bwd:
        if w.dtype == "f32":
            print("the backward runs in bf16/fp16 only", file=sys.stderr)
            sys.exit(2)
        do = random_grad(w.B, w.H, w.N, w.d, w.dtype, w.seed + 1000, std=w.std)
        dod = do.to(dev)
        ea.attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
        delta = torch.empty_like(lse)

        def step():
            ea.attn_bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                        delta=delta)
    else:
        def step():
            ea.attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    wall, kernel_ms = time_steps(step, args.steps, 0)
    avg_kernel_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    flops = 2.5 * w.flops if bwd else w.flops
    value = flops * args.steps / wall / 1e12

    achieved = flops / avg_kernel_s / 1e12
    peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_MFMA_BF16_TFLOPS
    traffic = None if bwd else measured_traffic(w.name)
    out = {
        # the headline workload carries the headline metric's name; others name themselves
        "metric": (("attention bwd TFLOP/s (bf16 causal, N=8192 d=128) and % of MFMA peak" if bwd else
                    "attention fwd TFLOP/s (bf16 causal, N=8192 d=128) and % of MFMA peak")
                   if args.workload == "c3" else
                   f"attention {'bwd' if bwd else 'fwd'} TFLOP/s ({w.name}) and % of "
                   f"{'fp32 vector' if w.dtype == 'f32' else 'MFMA'} peak"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_mfma_peak": round(100 * value / peak, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded randn inputs, see exact_attention_96_amd/workloads.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     # backward: q, k, v, o, dO and lse read, dq, dk, dv written, once each
                     "algorithmic_bytes": (8 * w.B * w.H * w.N * w.d * w.elt + 4 * w.B * w.H * w.N
                                           if bwd else w.io_bytes),
                     "kernel_ms_avg": round(avg_kernel_s * 1e3, 4),
                     "kernel_source_sha": kernel_source_hash()},
    }
    if args.clock_seconds > 0 and w.dtype != "f32":
        print(f"[bench] shader clock: amd-smi for ~{args.clock_seconds:.1f} s", file=sys.stderr, flush=True)
        clk = sustained_clock(step, args.clock_seconds)
        if clk is not None:
            # the dense MFMA peak scales with the shader clock: 256 CU x clock x 4096 flop/clk
            peak_at = PEAK_MFMA_BF16_TFLOPS * clk["mhz_median"] / 2400.0
            clk["peak_at_clock_tflops"] = round(peak_at, 1)
            clk["frac_at_clock"] = round(achieved / peak_at, 4)
        out["roofline"]["sustained_clock"] = clk
    if args.practical_seconds > 0 and w.dtype != "f32":
        print(f"[bench] practical ceiling: MFMA probe for ~{args.practical_seconds:.1f} s", file=sys.stderr,
              flush=True)
        pc = practical_ceiling(args.practical_seconds)
        if pc is not None:
            out["roofline"]["practical_ceiling"] = {
                "tflops": round(pc, 1), "frac": round(achieved / pc, 4),
                "source": "dense bf16 v_mfma_f32_32x32x16 on every SIMD with random operands "
                          "(libattn_probe.so), timed on this board right after the bench"}
    if args.cpu_seconds > 0 and args.cpu_heads != 0:
        print(f"[bench] cpu baseline: oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = (cpu_baseline_bwd(w, q, k, v, do, args.cpu_seconds) if bwd else
                               cpu_baseline(w, q, k, v, args.cpu_seconds))
    print(json.dumps(out), flush=True)


def cpu_baseline_linear(lw, q, k, v, seconds: float):
    """The fp64 oracle's causal linear attention on whole heads of the same workload,
    head after head until `seconds` of wall time have been spent (at least one head)."""
    import oracle
    heads = [(b, h) for b in range(lw.B) for h in range(lw.H)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.linear_attn(q[sl], k[sl], v[sl], lw.feature_map, lw.eps)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    nbytes = lw.io_bytes * done / (lw.B * lw.H)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} of {lw.B * lw.H} heads, all {lw.N} tokens each "
                      f"({nbytes:.3e} algorithmic bytes in {dt:.1f} s; the oracle sums every "
                      f"key of every row, O(N^2) per head)"}


def bench_linear(args, lw):
    import torch
    import exact_attention_96_amd as ea
    print(f"[bench] workload {lw.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v = lw.inputs()
    dev = "cuda:0"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(vd)
    # the chunked form's workspace, allocated once outside the timed region
    ws = torch.empty(ea.linear_workspace_bytes(lw.B, lw.H, lw.N, lw.E, lw.M), dtype=torch.uint8, device=dev)

    def step():
        ea.attn_linear_fwd(qd, kd, vd, feature_map=lw.feature_map, eps=lw.eps, out=o, workspace=ws)

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    wall, kernel_ms = time_steps(step, args.steps, args.warmup)
    avg_kernel_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    value = lw.io_bytes * args.steps / wall / 1e9
    achieved = lw.io_bytes / avg_kernel_s / 1e9
    out = {
        "metric": "causal linear attention fwd: algorithmic HBM GB/s (fp32) and % of the 8 TB/s peak",
        "value": round(value, 1), "unit": "GB/s", "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded randn inputs, see exact_attention_96_amd/workloads.py)",
        "config": {"workload": lw.name, "B": lw.B, "H": lw.H, "N": lw.N, "E": lw.E, "M": lw.M,
                   "feature_map": lw.feature_map, "eps": lw.eps},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(lw.name, TRAFFIC_FILE_LINEAR),
                     "algorithmic_bytes": lw.io_bytes, "kernel_ms_avg": round(avg_kernel_s * 1e3, 4),
                     "fp32_tflops": round(lw.flops / avg_kernel_s / 1e12, 2),
                     "workspace_bytes": ws.numel(),
                     "kernel_source_sha": kernel_source_hash()},
    }
    if args.cpu_seconds > 0 and args.cpu_heads != 0:
        print(f"[bench] cpu baseline: oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_linear(lw, q, k, v, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def time_steps(step, steps: int, warmup: int):
    """Warmup, then `steps` timed calls: wall seconds, and the average launch duration in
    ms (one entry per call) from one pair of HIP events around the timed calls on the
    current stream (the stream the library is given).  The calls run back to back, so
    the average is kernel time plus the GPU's launch-to-launch gap; events around each
    call would add their own gap to every call (about 10 us per call on a 0.2 ms
    kernel)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [start.elapsed_time(end) / steps] * steps


def bench_masked(args, mw):
    import torch
    import exact_attention_96_amd as ea
    print(f"[bench] workload {mw.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v, mask = mw.inputs()
    dev = "cuda:0"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((mw.B, mw.H, mw.Nq), dtype=torch.float32, device=dev)
    bits = None
    pack_ms = None
    if mask is not None:
        md = mask.to(dev)
        bits = ea.pack_mask(md)  # bits and tile summary, once, outside the timed region
        torch.cuda.synchronize()
        _, pk = time_steps(lambda: ea.pack_mask(md), 10, 2)
        pack_ms = sum(pk) / len(pk)

    def step():
        ea.attn_fwd_masked(qd, kd, vd, mask_bits=bits, causal=mw.causal, scale=mw.scale, out=o, lse=lse)

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    wall, kernel_ms = time_steps(step, args.steps, args.warmup)
    pairs = visible_pairs(mw, mask)
    flops = 4.0 * mw.d * pairs * mw.B * mw.H
    avg_kernel_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    value = flops * args.steps / wall / 1e12
    achieved = flops / avg_kernel_s / 1e12
    peak = PEAK_MFMA_BF16_TFLOPS
    out = {
        "metric": "attention fwd TFLOP/s (masked / unequal lengths) and % of MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "pct_of_mfma_peak": round(100 * value / peak, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": mw.dtype,
        "data": "synthetic (seeded randn inputs and mask patterns, see exact_attention_96_amd/workloads.py)",
        "config": {"workload": mw.name, "B": mw.B, "H": mw.H, "Nq": mw.Nq, "Nk": mw.Nk, "d": mw.d,
                   "causal": mw.causal, "mask": mw.mask_kind, "mask_w": mw.mask_w, "scale": mw.scale,
                   "visible_pairs_per_head": pairs},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "algorithmic_bytes": mw.io_bytes + (0 if bits is None else bits.bits.numel() * 8),
                     "kernel_ms_avg": round(avg_kernel_s * 1e3, 4),
                     "kernel_source_sha": kernel_source_hash()},
        "mask_pack_ms": None if pack_ms is None else round(pack_ms, 4),
    }
    if args.cpu_seconds > 0 and args.cpu_heads != 0:
        print(f"[bench] cpu baseline: oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_masked(mw, q, k, v, mask, pairs, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
