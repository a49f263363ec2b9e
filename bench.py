#!/usr/bin/env python3
"""Attention-forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one ``attn_fwd`` call (the whole hot path: Q-tile load, K/V tile
stream, scores, mask, online softmax, P.V, epilogue) over the workload's
synthetic inputs, which are generated on the host from a fixed seed and are
resident in HBM before timing starts.  The default workload is causal
prefill B=1, H=32, S=4096, d=128 in bf16 with fp32 accumulation.

Prints one JSON line with the throughput in TFLOP/s (4*B*H*Sq*Skv*d, halved
for causal), a ``roofline`` object for the attention kernel (MFMA-bound;
achieved TFLOP/s from HIP events around each launch on the launch stream,
against the MI355X dense bf16 MFMA peak) and a ``cpu_baseline`` object (the
fp64 oracle timed on a bounded sample of the same workload on the host).

``--copy-probe BYTES`` instead times a plain device-to-device copy of BYTES
bytes; its rocprofv3 FETCH_SIZE / WRITE_SIZE readings calibrate the HBM
counters against a transfer of known size.  ``--gemm-probe N`` times a
dense N x N x N bf16 torch.matmul on random and on all-zero operands (the
chip's matrix-core rate under its power limit, for data that toggle like
the benchmark's and for data that do not).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % MFMA peak (bf16 H=32 S=4096 d=128 causal)"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "f64": 78.6}
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_h32_s4096_d128.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_busy_prefill_h32_s4096_d128.json")
# MI355X: 256 compute units of 4 SIMDs each, in 8 XCDs
N_SIMDS, N_XCDS = 1024, 8
KERNEL_SOURCES = ["attn_bf16.hip", "attn_device.h", "attn_api.hip"]


def code_text(src: str) -> str:
    """The source without comments and blank lines (so that comment edits do
    not invalidate measurements taken on the same code)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in src.splitlines()]
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_source_hash(read=None) -> str:
    """Hash of the code of the kernel sources (see ``code_text``)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        path = os.path.join(ROOT, "tiled_online_softmax_05_amd", "csrc", name)
        if read is None:
            with open(path) as f:
                text = f.read()
        else:
            text = read(path)
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel source (else None)."""
    if workload != "prefill_h32_s4096_d128" or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# The counter runs behind the two records (run from the repository root; DIR
# is the folder passed to --record-counters).
COUNTER_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_fetch -o run -- "
    "python3 -u bench.py --steps 20 --warmup 100 --cpu-budget 0",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc_write -o run -- "
    "python3 -u bench.py --steps 20 --warmup 100 --cpu-budget 0",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_copy_fetch -o run -- "
    "python3 -u bench.py --copy-probe 1073741824 --steps 3",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc_copy_write -o run -- "
    "python3 -u bench.py --copy-probe 1073741824 --steps 3",
    "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
    "-d DIR/pmc_mfma -o run -- python3 -u bench.py --steps 20 --warmup 100 --cpu-budget 0",
]


def measured_mfma_busy(workload: str):
    """Fraction of the launch's cycles in which a SIMD's matrix core is busy,
    from rocprofv3 counters taken on the current kernel source (else None):
    SQ_VALU_MFMA_BUSY_CYCLES per SIMD over GRBM_GUI_ACTIVE per XCD."""
    if workload != "prefill_h32_s4096_d128" or not os.path.exists(MFMA_FILE):
        return None
    with open(MFMA_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("mfma_busy_frac")


def read_counters(path: str, kernel_key: str = "attn_fwd_bf16_kernel", last: int = 20):
    """Mean per dispatch of each counter in a rocprofv3 counter_collection.csv,
    over the last ``last`` dispatches of the kernel whose name contains
    ``kernel_key`` (the timed launches come last).  Returns (kernel name,
    {counter: mean})."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if kernel_key not in r["Kernel_Name"]:
                continue
            rows.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], {}))[1][r["Counter_Name"]] = \
                float(r["Counter_Value"])
    if not rows:
        raise SystemExit(f"{path}: no dispatch of a kernel named *{kernel_key}*")
    ids = sorted(rows)[-last:]
    name = rows[ids[-1]][0]
    means = {}
    for c in rows[ids[-1]][1]:
        means[c] = sum(rows[i][1][c] for i in ids) / len(ids)
    return name, means


def record_counters(d: str, commands: list) -> None:
    """Write the traffic and MFMA-busy records from the rocprofv3 counter runs
    under ``d`` (pmc_fetch, pmc_write, pmc_copy_fetch, pmc_copy_write,
    pmc_mfma, each with a run_counter_collection.csv), keyed on the current
    kernel source."""
    def csv_in(sub):
        return os.path.join(d, sub, "run_counter_collection.csv")
    name, fetch = read_counters(csv_in("pmc_fetch"))
    _, write = read_counters(csv_in("pmc_write"))
    _, cfetch = read_counters(csv_in("pmc_copy_fetch"), kernel_key="", last=1)
    _, cwrite = read_counters(csv_in("pmc_copy_write"), kernel_key="", last=1)
    _, mf = read_counters(csv_in("pmc_mfma"))
    # the copy reads and writes copy_bytes once each: bytes per counted byte
    copy_bytes = 1 << 30
    fscale = copy_bytes / (cfetch["FETCH_SIZE"] * 1024)
    wscale = copy_bytes / (cwrite["WRITE_SIZE"] * 1024)
    h = kernel_source_hash()
    rd = round(fetch["FETCH_SIZE"] * 1024 * fscale)
    wr = round(write["WRITE_SIZE"] * 1024 * wscale)
    traffic = {"workload": "prefill_h32_s4096_d128", "kernel": name, "kernel_source_sha256_16": h,
               "fetch_size_kib_per_launch": round(fetch["FETCH_SIZE"], 1),
               "write_size_kib_per_launch": round(write["WRITE_SIZE"], 1),
               "copy_probe_bytes": copy_bytes,
               "copy_fetch_size_kib": round(cfetch["FETCH_SIZE"], 4),
               "copy_write_size_kib": round(cwrite["WRITE_SIZE"], 4),
               "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5),
               "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
               "hbm_bytes_per_launch": rd + wr, "commands": commands[:4]}
    busy = mf["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMDS
    active = mf["GRBM_GUI_ACTIVE"] / N_XCDS
    mfma = {"workload": "prefill_h32_s4096_d128", "kernel": name, "kernel_source_sha256_16": h,
            "sq_valu_mfma_busy_cycles": mf["SQ_VALU_MFMA_BUSY_CYCLES"],
            "grbm_gui_active": mf["GRBM_GUI_ACTIVE"], "simds": N_SIMDS, "xcds": N_XCDS,
            "mfma_busy_cycles_per_simd": round(busy, 1), "active_cycles_per_xcd": round(active, 1),
            "mfma_busy_frac": round(busy / active, 4), "commands": commands[4:]}
    for path, rec in ((TRAFFIC_FILE, traffic), (MFMA_FILE, mfma)):
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(f"wrote {path}")


def cpu_baseline(q, k, v, causal: bool, budget_s: float) -> dict:
    """The fp64 oracle, as it stands, on whole heads of the same inputs,
    for about ``budget_s`` seconds; scaled to TFLOP/s with the same FLOP
    formula as the GPU figure."""
    import oracle
    from seeded_inputs import to_f64
    from tiled_online_softmax_05_amd.accounting import attention_flops
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                         for i in info if i.get("user_api") == "blas") or "none loaded"
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    _, H, Sq, d = q.shape
    Skv = k.shape[2]
    per_head = attention_flops(1, 1, Sq, Skv, d, causal)
    heads = [(to_f64(q[0, h]), to_f64(k[0, h]), to_f64(v[0, h])) for h in range(H)]
    # whole passes over the heads of the first batch entry until the budget
    # is spent, reporting the median pass (a workload too large for one pass
    # stops inside it and reports the rate over the heads done)
    rates, done, t_all = [], 0, time.perf_counter()
    while True:
        t0, n = time.perf_counter(), 0
        for qh, kh, vh in heads:
            oracle.direct_attention(qh, kh, vh, scale=1.0 / math.sqrt(d), causal=causal)
            n += 1
            if time.perf_counter() - t_all > budget_s and not rates:
                break
        rates.append(n * per_head / (time.perf_counter() - t0))
        done = max(done, n)
        if n < H or time.perf_counter() - t_all > budget_s:
            break
    dt = time.perf_counter() - t_all
    value = sorted(rates)[len(rates) // 2] if done == H else rates[0]
    how = (f"median of {len(rates)} passes over {H} heads" if done == H
           else f"{done} of {H} heads")
    return {"value": round(value / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "host_cpus": os.cpu_count(), "blas": blas,
            "kind": "oracle",
            "sample": f"{how} (B=1, Sq={Sq}, Skv={Skv}, d={d}, causal={causal}), fp64 numpy "
                      f"direct attention, {dt:.1f} s"}


def copy_probe(nbytes: int, steps: int) -> None:
    import torch
    dev = torch.device("cuda", 0)
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "steps": steps}), flush=True)


def gemm_probe(n: int, steps: int) -> None:
    """Dense bf16 GEMM rate (torch.matmul, n x n x n) on random and on all-zero
    operands: the same instructions, different bit toggling.  Under a power
    limit the random-operand rate is the attainable matrix-core rate for
    data like the benchmark's."""
    import torch
    dev = torch.device("cuda", 0)
    g = torch.Generator(device="cpu").manual_seed(7)
    res = {"gemm_probe": n, "steps": steps, "dtype": "bf16"}
    for name in ("random", "zeros"):
        if name == "random":
            a = (torch.rand(n, n, generator=g) * 1.6 - 0.8).to(torch.bfloat16).to(dev)
            b = (torch.rand(n, n, generator=g) * 1.6 - 0.8).to(torch.bfloat16).to(dev)
        else:
            a = torch.zeros(n, n, dtype=torch.bfloat16, device=dev)
            b = torch.zeros(n, n, dtype=torch.bfloat16, device=dev)
        c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
        for _ in range(max(3, steps // 4)):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.matmul(a, b, out=c)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}
    print(json.dumps(res), flush=True)


def mfma_probe(iters: int, grid: int = 512) -> None:
    """Sustained bf16 matrix-core rate from libattn_probe.so (see
    include/attn_probe.h): MFMA streams with zero or random operands, with and
    without 1 KiB of LDS operand reads per MFMA, two 256-thread workgroups per
    compute unit.  Three untimed launches, then five timed back to back
    between one HIP event pair on torch's current stream."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "tiled_online_softmax_05_amd", "libattn_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m tiled_online_softmax_05_amd.build`")
    lib = ctypes.CDLL(path)
    vp, ip = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_mfma.argtypes = [ip, ip, ip, vp, vp]
    lib.attn_probe_mfma.restype = ip
    lib.attn_probe_mfma_flops.argtypes = [ip, ip, ip]
    lib.attn_probe_mfma_flops.restype = ctypes.c_double
    dev = torch.device("cuda", 0)
    out = torch.zeros(grid, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    names = ["mfma_zero", "mfma_random", "mfma_lds_zero", "mfma_lds_random"]
    res = {"mfma_probe_iters": iters, "grid": grid, "dtype": "bf16"}
    for kind, name in enumerate(names):
        def launch():
            st = lib.attn_probe_mfma(kind, iters, grid, out.data_ptr(), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"attn_probe_mfma({kind}) returned {st}")
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            launch()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / 5
        tf = lib.attn_probe_mfma_flops(kind, iters, grid) / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}
    print(json.dumps(res), flush=True)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU raises its clocks over the first tens of milliseconds of load, so
    # the default warm-up (~50 ms of launches) precedes the timed region
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="prefill_h32_s4096_d128")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline (0 disables it)")
    ap.add_argument("--tiles", default=None,
                    help="force BMxBN, e.g. 128x64; 'auto' = the selector's tiles even "
                         "where the workload forces its own")
    ap.add_argument("--splits", type=int, default=None,
                    help="time attn_fwd_split with this many key chunks (0 = library choice)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES")
    ap.add_argument("--zero-inputs", action="store_true",
                    help="diagnostic: all-zero Q, K, V of the workload's shape (same instructions, "
                         "no operand bit toggling); not the benchmark")
    ap.add_argument("--gemm-probe", type=int, default=0, metavar="N",
                    help="time an N x N x N bf16 torch.matmul on random and on zero operands")
    ap.add_argument("--mfma-probe", type=int, default=0, metavar="ITERS",
                    help="time bare bf16 MFMA streams (zero / random operands, with and "
                         "without LDS operand reads) from libattn_probe.so")
    ap.add_argument("--launch-series", type=int, default=0, metavar="N",
                    help="diagnostic: N launches from a cold start (no warm-up), each "
                         "between its own event pair, printed as one JSON line of "
                         "per-launch times (the GPU's clock ramp)")
    ap.add_argument("--flush", action="store_true",
                    help="overwrite a 1 GiB buffer before each timed launch (outside the "
                         "per-launch events), so K/V start outside L2 and Infinity Cache; "
                         "value then comes from the events")
    ap.add_argument("--record-counters", metavar="DIR", default=None,
                    help="no GPU: write the traffic and MFMA-busy records from the rocprofv3 "
                         "counter runs under DIR (see profiles/) for the current kernel source")
    a = ap.parse_args(argv)

    if a.record_counters:
        record_counters(a.record_counters, COUNTER_COMMANDS)
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if a.copy_probe:
        copy_probe(a.copy_probe, max(1, a.steps))
        return 0
    if a.gemm_probe:
        gemm_probe(a.gemm_probe, max(1, a.steps))
        return 0
    if a.mfma_probe:
        mfma_probe(a.mfma_probe)
        return 0

    from seeded_inputs import WORKLOADS, make_tensors
    from tiled_online_softmax_05_amd import binding
    from tiled_online_softmax_05_amd.accounting import attention_flops, compulsory_bytes

    w = WORKLOADS[a.workload]
    causal = True in w.causal_modes
    dev = torch.device("cuda", 0)
    q_h, k_h, v_h = make_tensors(w)
    if a.zero_inputs:
        # diagnostic: the same launches on operands that do not toggle
        q_h, k_h, v_h = (torch.zeros_like(x) for x in (q_h, k_h, v_h))
        a.cpu_budget = 0
    q, k, v = q_h.to(dev), k_h.to(dev), v_h.to(dev)
    # the split path runs the selector's tiles: a workload's own forced tiles
    # give way to them (only an explicit --tiles conflicts with --splits)
    if a.tiles == "auto":
        tiles = None
    else:
        tiles = (tuple(int(x) for x in a.tiles.split("x")) if a.tiles
                 else (None if a.splits is not None else w.tiles))
    odt = q.dtype
    out = torch.empty(q.shape, dtype=odt, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    code = {torch.float32: binding.F32, torch.bfloat16: binding.BF16,
            torch.float16: binding.F16}[odt]
    dtype_name = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[odt]
    scale = 1.0 / math.sqrt(w.d)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    if tiles is None:
        tiles_used = binding.select_tiles(w.d, w.Sq, w.Skv, w.B * w.H, code, causal)[:2]
    else:
        tiles_used = tiles
    n_splits = None
    if a.splits is not None:
        if tiles is not None:
            print("--tiles and --splits cannot be combined", file=sys.stderr)
            return 2
        n_splits = a.splits or binding.select_splits(w.d, w.Sq, w.Skv, w.B * w.H, code, causal)[0]
        ws_bytes = binding.split_workspace_bytes(w.B, w.H, w.Sq, w.d, n_splits)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)   # 256-byte aligned

    def step():
        if n_splits is None:
            binding.fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), w.B, w.H, w.Sq, w.Skv, w.d, scale, causal, code, sp,
                            tiles)
        else:
            binding.fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), w.B, w.H, w.Sq, w.Skv, w.d, scale, causal, code,
                                  sp, n_splits, ws.data_ptr(), ws_bytes)

    if a.launch_series:
        # back to back on the launch stream, one event pair per launch
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(a.launch_series)]
        torch.cuda.synchronize()
        for s0, s1 in pairs:
            s0.record(stream)
            step()
            s1.record(stream)
        torch.cuda.synchronize()
        us = [round(s0.elapsed_time(s1) * 1e3, 2) for s0, s1 in pairs]

        def mean(lo, hi):
            part = us[lo:hi]
            return round(sum(part) / len(part), 2) if part else None
        print(json.dumps({"launch_series": a.launch_series, "workload": a.workload,
                          "us_mean": {"1-5": mean(0, 5), "6-25": mean(5, 25),
                                      "26-100": mean(25, 100), "101-300": mean(100, 300),
                                      "last 100": mean(len(us) - 100, len(us))},
                          "us": us}), flush=True)
        return 0

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` launches back to back, one HIP event pair
    # around the region on the launch stream.  With --flush a scrub of the
    # caches runs before every launch, so each launch gets its own events and
    # the scrubs stay outside the timed intervals.
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev) if a.flush else None
    if scrub is not None:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    else:
        region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if scrub is None:
        region[0].record(stream)
        for _ in range(a.steps):
            step()
        region[1].record(stream)
    else:
        for i in range(a.steps):
            scrub.fill_(float(i))
            starts[i].record(stream)
            step()
            ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if scrub is None:
        avg_ms = region[0].elapsed_time(region[1]) / a.steps
        # after the timed region: 31 launches, each bracketed by its own events
        # (the events add their own overhead to every interval), for the median
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(31)]
        for s0, s1 in pairs:
            s0.record(stream)
            step()
            s1.record(stream)
        torch.cuda.synchronize()
        med_ms = sorted(s0.elapsed_time(s1) for s0, s1 in pairs)[15]
    else:
        launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
        avg_ms = sum(launch_ms) / len(launch_ms)
        med_ms = sorted(launch_ms)[len(launch_ms) // 2]

    flops = attention_flops(w.B, w.H, w.Sq, w.Skv, w.d, causal)
    # with --flush the wall clock also holds the scrubs: use the launch events
    ms_per_step = avg_ms if a.flush else wall * 1e3 / a.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype_name]
    in_b = 4 if dtype_name == "f32" else 2
    comp = compulsory_bytes(w.B, w.H, w.Sq, w.Skv, w.d, in_b, in_b)
    # counters were taken on the default launch (selector tiles, one key chunk, warm cache)
    default_launch = tiles == w.tiles and n_splits is None and not a.flush
    traffic = measured_traffic(a.workload) if default_launch else None
    mfma_busy = measured_mfma_busy(a.workload) if default_launch else None

    # bound: MFMA above the ridge point (peak FLOP/s over HBM bytes/s), HBM below
    if flops / comp >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                    "mfma_busy_frac": mfma_busy}
    else:
        gbs = comp / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 5), "traffic": traffic,
                    "mfma_tflops": round(achieved, 4), "mfma_peak": peak}
    rec = {
        "metric": METRIC if a.workload == "prefill_h32_s4096_d128" else f"attention fwd TFLOP/s ({a.workload})",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": {"workload": a.workload, "B": w.B, "H": w.H, "Sq": w.Sq, "Skv": w.Skv,
                   "d": w.d, "causal": causal, "tiles": list(tiles_used),
                   "key_chunks": n_splits or 1, "cache": "flushed" if a.flush else "warm",
                   "input_dist": "zeros" if a.zero_inputs else w.dist, "seed": w.seed},
        "roofline": roofline,
    }
    roofline.update({"launch_ms_avg": round(avg_ms, 5),
                     "launch_ms_median": None if med_ms is None else round(med_ms, 5),
                     "flops_per_launch": flops, "compulsory_bytes_per_launch": comp,
                     "compulsory_GBps": round(comp / (avg_ms * 1e-3) / 1e9, 1),
                     "hbm_peak_GBps": PEAK_HBM_GBS})
    if a.cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(q_h, k_h, v_h, causal, a.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
