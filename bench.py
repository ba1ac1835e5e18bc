"""Benchmark: batched, row-wise, stride-correct top-k index selection on one GPU.

One step = one call of the library's top-k over the whole batch (all rows),
with the inputs already resident in HBM.  Before its W warm-up steps each
timed workload runs its own launches untimed for 0.25 s (`clock_settle_s`):
the GPU's clocks need about 10 ms of sustained load to leave their idle
level, which a run of a few dozen launches would otherwise measure.  Copies of the input are used in
turn, enough that more than 600 MB (twice the L2 caches plus the 256 MB
last-level cache) is touched between two uses of one copy, so that no step
finds its input in a cache (2 copies for the prefill batch, 21 for the
long-context batch).  The timed region is K launches back to back between two
HIP events on the launch stream; a separate pass with an event pair around
each launch gives the spread of single launches.  For context the line also
carries `read_ceiling`: a plain max (torch.amax) over the same bytes and input
copies (rows cut into pieces when there are few), timed the same way, i.e.
what a simple streaming read of the batch reaches on this GPU (also for the
long-context workload in `configs`);
`warm_cache`: the same launches on one reused input copy; `paged_output`:
the same launches writing KV-cache slots through a page table (the index
transform fused into the stores); and `value_order`: the selection followed by
the kernel that ranks each row's columns by value.  `configs` times the
other four workloads the same way (long with its own read ceiling), and
`c128a_metadata` the C128A metadata kernel at the shapes the adaptive-width
page times.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload prefill]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
METRIC = "rows/s and achieved HBM GB/s (% of peak), batched strided top-k, k=2048"
DESCRIPTIONS = {
    "prefill": "causal prefill indexer: 4096 rows, L_i = 28672+i+1, row stride 32768, "
               "N(0,1) + per-row offset U(-3,3), k=2048",
    "long": "small-batch long context: 8 rows, L_i = 900000, row stride 900096, "
            "N(0,1) with 0.5% N(4,1) outliers, k=2048",
    "decode": "decode batch: 64 rows, L_i ~ U{1..60000}, row stride 60160, bf16-rounded N(0,1), k=1024",
    "adversarial": "adversarial mix: 256 rows, row stride 131072, k=1024",
    "tiny": "tiny: 4 rows x 4096, k=512",
}
KERNEL_SOURCES = ["row_wise_top_topk_amd/csrc/topk_kernels.hip",
                  "row_wise_top_topk_amd/csrc/select_device.hpp",
                  "row_wise_top_topk_amd/csrc/wave64.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the copy-calibrated FETCH_SIZE/WRITE_SIZE
    counters in profiles/traffic.json, or None when the kernel sources have
    changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    h = kernel_source_hash()
    for t in json.load(open(TRAFFIC_FILE)):
        if t.get("kernel_hash") == h and t.get("workload") == workload:
            return t.get("bytes_per_launch")
    return None


# ---------------------------------------------------------------- CPU oracle leg
_CPU = {}


def cpu_share() -> int:
    """Host threads this process may keep busy: the OMP_NUM_THREADS the
    machine sets for one GPU's share of its cores (16 if unset)."""
    try:
        return max(1, int(os.environ.get("OMP_NUM_THREADS", "16")))
    except ValueError:
        return 16


def _oracle_rows(rows):
    from oracle import oracle_topk_row, row_view
    w = _CPU["w"]
    flat = _CPU["flat"]
    lengths = _CPU["lengths"]
    for r in rows:
        oracle_topk_row(row_view(flat, w.row_stride, int(lengths[r]), r), w.k)
    return len(rows)


def cpu_baseline(w, max_rows: int) -> dict:
    """The CPU oracle, as it stands, over a bounded sample of the same rows."""
    affinity = len(os.sched_getaffinity(0))
    cores = min(affinity, cpu_share())
    _CPU["w"] = w
    _CPU["flat"], _CPU["lengths"] = workloads.to_numpy(w)
    rows = list(range(min(max_rows, w.num_rows)))
    parts = [rows[i::cores] for i in range(cores)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        done = sum(pool.map(_oracle_rows, parts))
    dt = time.perf_counter() - t0
    one = rows[:512]
    t1 = time.perf_counter()
    n1 = _oracle_rows(one)
    d1 = time.perf_counter() - t1
    return {"value": done / dt, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "affinity_cores": affinity,
            "sample": f"first {done} rows of the {w.name} workload, one pass, "
                      f"numpy stable argsort per row across a {cores}-process pool "
                      f"({dt:.2f} s wall)",
            "value_1core": n1 / d1,
            "sample_1core": f"first {n1} rows on one core ({d1:.2f} s)"}


# ---------------------------------------------------------------- GPU leg
def gpu_env() -> dict:
    env = {}
    try:
        env["gpu"] = torch.cuda.get_device_name(0)
    except Exception:
        pass
    env["hip"] = getattr(torch.version, "hip", None)
    try:
        env["git"] = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                                    capture_output=True, text=True).stdout.strip() or None
    except Exception:
        env["git"] = None
    return env


COLD_BYTES = 600e6   # bytes touched between two uses of one input copy
MAX_COPIES = 64
SETTLE_S = 0.25      # untimed load before the warm-up steps (clock settling)


def settle(fn, seconds: float | None = None) -> int:
    """Run `fn` back to back, untimed, for `seconds` of wall time.  After idling
    the GPU's clocks are low and take about 10 ms of sustained load to reach
    their working level (on MI355X, consecutive batches of 20 prefill launches
    from idle measured 124, 117, 113, 110, 109, 109 us per launch, and again
    116 us after 2 s idle), so every timed workload is preceded by this much
    of its own work before its warm-up steps.  Returns the launches made."""
    seconds = SETTLE_S if seconds is None else seconds
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def input_copies(w) -> int:
    """Copies of the input that keep every step cold in the caches."""
    footprint = 4.0 * w.num_rows * w.row_stride
    return int(min(MAX_COPIES, max(2, -(-COLD_BYTES // footprint))))


def time_workload(w, steps: int, warmup: int, copies: int = 2, paging: dict | None = None,
                  order: str = "column", path: str = "auto"):
    import row_wise_top_topk_amd as mt
    dev = torch.device("cuda:0")
    pg = {} if paging is None else {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
                                    for k, v in paging.items()}
    if order != "column":
        pg["order"] = order
    if path != "auto":
        pg["path"] = path
    bufs = []
    for _ in range(copies):
        flat = w.flat.to(dev)
        bufs.append(flat.as_strided((w.num_rows, w.row_stride), (w.row_stride, 1)))
    lengths = w.lengths.to(dev)
    out = torch.empty((w.num_rows, w.k), dtype=torch.int32, device=dev)
    need = mt.workspace_size(w.num_rows, w.row_stride, w.k, path=path)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev) if need else None
    it = [0]

    def one():
        mt.topk_indices(bufs[it[0] % copies], lengths, w.k, out=out, workspace=ws, **pg)
        it[0] += 1
    settle(one)
    for i in range(warmup):
        mt.topk_indices(bufs[i % copies], lengths, w.k, out=out, workspace=ws, **pg)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the stream the library launches on
    # per-launch event pairs, for the spread of single launches
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        starts[i].record(stream)
        mt.topk_indices(bufs[i % copies], lengths, w.k, out=out, workspace=ws, **pg)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    # the timed region: `steps` launches back to back between two events
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        mt.topk_indices(bufs[i % copies], lengths, w.k, out=out, workspace=ws, **pg)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = t_start.elapsed_time(t_end)
    err = mt.workspace_error(ws) if ws is not None else 0
    if err:
        raise RuntimeError("a cross-workgroup barrier wait gave up during the benchmark")
    return total_ms, per_launch_ms, wall


def paging_for(w, page_size: int = 64, seed: int = 7) -> dict:
    """Every row a token of one request whose pages are a random permutation:
    the page table of a single long sequence in a paged KV cache."""
    g = torch.Generator().manual_seed(seed)
    pages = -(-w.row_stride // page_size)
    table = torch.randperm(4 * pages, generator=g)[:pages].to(torch.int32).reshape(1, pages)
    return {"block_table": table, "page_size": page_size,
            "row_to_req": torch.zeros(w.num_rows, dtype=torch.int32)}


def read_ceiling(w, steps: int, warmup: int, copies: int):
    """A plain streaming read of the same bytes for context: torch.amax over
    the batch's full strides, on the same rotation of cold input copies,
    timed like the top-k launches (back to back between two events).  Rows
    are cut into f pieces (f a power of two dividing the stride) until there
    are at least 2048 pieces, none below 1024 entries, so that a batch of a
    few long rows still spreads over the whole GPU."""
    dev = torch.device("cuda:0")
    f = 1
    while (w.num_rows * f < 2048 and w.row_stride % (2 * f) == 0
           and w.row_stride // (2 * f) >= 1024):
        f *= 2
    shape = (w.num_rows * f, w.row_stride // f)
    bufs = [w.flat.to(dev).as_strided(shape, (shape[1], 1)) for _ in range(copies)]
    it = [0]

    def one():
        torch.amax(bufs[it[0] % copies], dim=1)
        it[0] += 1
    settle(one)
    for i in range(warmup):
        torch.amax(bufs[i % copies], dim=1)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(steps):
        torch.amax(bufs[i % copies], dim=1)
    t_end.record(stream)
    torch.cuda.synchronize()
    us = t_start.elapsed_time(t_end) / steps * 1e3
    nbytes = 4.0 * w.num_rows * w.row_stride
    del bufs
    return {"kernel": "torch.amax(dim=1) over the full row strides", "view": list(shape),
            "us_per_launch": us,
            "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
            "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def rows_sweep(name: str, steps: int, warmup: int) -> None:
    """The workload's rows repeated or cut to several batch sizes, timed like
    the bench line: a straight-line fit of time against rows separates the
    per-row (streaming) cost from the fixed cost of a launch (start-up and the
    last rows' drain).  One JSON line per size, then the fit."""
    base = workloads.make(name)
    xs, ys = [], []
    for rows in (768, 1536, 2304, 3072, 3840, 4608, 5376):
        reps = -(-rows // base.num_rows)
        flat = (base.flat.view(base.num_rows, base.row_stride).repeat(reps, 1)[:rows]
                .reshape(-1).contiguous())
        lens = base.lengths.repeat(reps)[:rows].contiguous()
        w = workloads.Workload(f"{name}-rows{rows}", flat, base.row_stride, lens, rows, base.k)
        t, _, _ = time_workload(w, steps, warmup, copies=input_copies(w))
        us = t / steps * 1e3
        xs.append(rows)
        ys.append(us)
        print(json.dumps({"rows": rows, "us_per_launch": us,
                          "achieved_gbs": w.algorithmic_bytes() / (us * 1e-6) / 1e9}), flush=True)
    slope, icpt = np.polyfit(np.array(xs, dtype=float), np.array(ys), 1)
    per_row_bytes = base.algorithmic_bytes() / base.num_rows
    print(json.dumps({"fit": "us = intercept + slope * rows", "intercept_us": icpt,
                      "slope_ns_per_row": slope * 1e3,
                      "marginal_gbs": per_row_bytes / (slope * 1e-6) / 1e9}), flush=True)


def calibrate_copy() -> None:
    """A plain copy of known size, to scale the HBM byte counters by."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "copies": 5}), flush=True)


# The page's own timings of the C128A metadata build (context 32768, capacity
# 8192, active width 256; Triton do_bench medians, hardware not stated):
# tokens -> (fixed-width us, adaptive-width us).
C128A_PAGE_US = {512: (9.22, 7.20), 2048: (15.39, 7.20), 8192: (44.00, 11.30), 32768: (150.56, 25.79)}


def time_c128a(steps: int, warmup: int) -> dict:
    """The C128A metadata kernel at the page's shapes: prefill tokens at
    positions 32768 - T .. 32767, capacity 8192, the fixed width (8192)
    and the adaptive width (256).  `us`: launches back to back between two
    events through the C ABI with the arguments marshalled once (so the
    figure is the GPU's, not Python's); `us_single`: the median of an event
    pair around each launch, as the page's do_bench times one call."""
    import ctypes
    import row_wise_top_topk_amd as mt
    lib = mt.load_library()
    dev = torch.device("cuda:0")
    context, ratio, capacity = 32768, 128, 8192
    active = mt.c128a_active_width(context, ratio)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    rows = []
    for T in sorted(C128A_PAGE_US):
        pos = torch.arange(context - T, context, dtype=torch.int64, device=dev)
        pbuf = torch.empty((T, capacity), dtype=torch.int32, device=dev)
        for label, width, page_us in (("fixed", capacity, C128A_PAGE_US[T][0]),
                                      ("adaptive", active, C128A_PAGE_US[T][1])):
            args = (ctypes.c_void_p(pos.data_ptr()), T, ratio, 0, None, None, 0, 2, None, 0, None,
                    ctypes.c_void_p(pbuf.data_ptr()), capacity, width, sp)
            fn = lib.c128a_topk_metadata
            settle(lambda: fn(*args))
            for _ in range(warmup):
                if fn(*args) != 0:
                    raise RuntimeError("c128a_topk_metadata failed")
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                fn(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(steps)]
            for a, b in pairs:
                a.record(stream)
                fn(*args)
                b.record(stream)
            torch.cuda.synchronize()
            single = float(np.median([a.elapsed_time(b) for a, b in pairs])) * 1e3
            nbytes = 4 * T * width + 8 * T       # rows written, positions read
            rows.append({"tokens": T, "width": label, "entries_per_row": width, "us": us,
                         "us_single": single, "gbs": nbytes / (us * 1e-6) / 1e9,
                         "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "page_us": page_us})
        del pbuf
    return {"kernel": "c128a_metadata_kernel", "context": context, "compress_ratio": ratio,
            "capacity": capacity, "active_width": active, "rows": rows,
            "note": "page_us: the page's Triton do_bench medians (hardware not stated), context only"}


def time_config(name: str, steps: int, warmup: int, with_read_ceiling: bool = False) -> dict:
    """One named workload through the automatic path, cold inputs, K launches
    back to back between two events."""
    w = workloads.make(name)
    c = input_copies(w)
    t, pl, _ = time_workload(w, steps, warmup, copies=c)
    b = w.algorithmic_bytes()
    m = t / steps
    res = {"workload": DESCRIPTIONS[name], "input_copies": c, "rows": w.num_rows,
           "row_stride": w.row_stride, "k": w.k, "valid_elements": w.valid_elements,
           "rows_with_length_below_k": int((w.lengths.to(torch.int64).clamp(0, w.row_stride)
                                            < w.k).sum()),
           "algorithmic_bytes": b,
           "launch_us_mean": m * 1e3,
           "launch_us_p50": float(np.percentile(pl, 50)) * 1e3,
           "rows_per_s": w.num_rows / (m * 1e-3),
           "achieved_gbs": b / (m * 1e-3) / 1e9,
           "frac": b / (m * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "traffic": measured_traffic(name)}
    tp, _, _ = time_workload(w, steps, warmup, copies=c, path="persist")
    res["persistent_grid"] = {"launch_us_mean": tp / steps * 1e3,
                              "over_plain_us": (tp - t) / steps * 1e3}
    if with_read_ceiling:
        rc = read_ceiling(w, steps, warmup, c)
        res["read_ceiling"] = {"us_per_launch": rc["us_per_launch"], "gbs": rc["gbs"], "frac": rc["frac"],
                               "topk_over_read_time": m * 1e3 / rc["us_per_launch"]}
    return res


def main() -> None:
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--others", default="long,decode,adversarial,tiny",
                    help="the other workloads timed for the line's `configs` ('' to skip)")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the workload the CPU oracle leg processes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip paged output, value order, warm cache, read ceiling and C128A")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB five times (HBM counter calibration)")
    ap.add_argument("--rows-sweep", action="store_true",
                    help="only time the workload at several row counts and fit time against rows")
    ap.add_argument("--c128a-only", action="store_true",
                    help="only time the C128A metadata kernel at the page's shapes")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="untimed load before each workload's warm-up (clock settling)")
    args = ap.parse_args()
    SETTLE_S = args.settle_s
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.rows_sweep:
        rows_sweep(args.workload, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): rows are independent, "
              "so the path shards by rows with no exchange; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.c128a_only:
        print(json.dumps(time_c128a(args.steps, args.warmup)), flush=True)
        return

    w = workloads.make(args.workload)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_rows)   # before the GPU is initialised (fork pool)

    copies = input_copies(w)
    total_ms, per_launch, wall = time_workload(w, args.steps, args.warmup, copies=copies)
    ms_per_step = total_ms / args.steps
    alg_bytes = w.algorithmic_bytes()
    avg_launch_ms = ms_per_step   # launches back to back in the timed region
    achieved = alg_bytes / (avg_launch_ms * 1e-3) / 1e9
    rows_per_s = w.num_rows / (ms_per_step * 1e-3)

    traffic = measured_traffic(args.workload)

    result = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.workload], "rows": w.num_rows,
                   "row_stride": w.row_stride, "k": w.k, "valid_elements": w.valid_elements,
                   "rows_with_length_below_k": int((w.lengths.to(torch.int64).clamp(0, w.row_stride)
                                                    < w.k).sum()),
                   "algorithmic_bytes": alg_bytes, "input_copies": copies,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "cpu_baseline": cpu,
        "gbs_per_step": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "launch_us": {"mean": avg_launch_ms * 1e3,
                      "single_mean": float(np.mean(per_launch)) * 1e3,
                      "p10": float(np.percentile(per_launch, 10)) * 1e3,
                      "p50": float(np.percentile(per_launch, 50)) * 1e3,
                      "p90": float(np.percentile(per_launch, 90)) * 1e3},
        "host_wall_s": wall,
        "clock_settle_s": SETTLE_S,
        "env": gpu_env(),
    }
    others = [n for n in args.others.split(",") if n and n != args.workload]
    if others:
        result["configs"] = {n: time_config(n, args.steps, args.warmup, with_read_ceiling=(n == "long"))
                             for n in others}
    if not args.no_extras:
        paged_ms, _, _ = time_workload(w, args.steps, args.warmup, copies=copies, paging=paging_for(w))
        result["paged_output"] = {"page_size": 64, "requests": 1,
                                  "launch_us_mean": paged_ms / args.steps * 1e3,
                                  "over_plain_us": (paged_ms / args.steps - avg_launch_ms) * 1e3,
                                  "note": "topk_indices_paged: columns written as KV-cache slots "
                                          "through a random page table, fused into the stores"}
        vo_ms, _, _ = time_workload(w, args.steps, args.warmup, copies=copies, order="value")
        result["value_order"] = {"launch_us_mean": vo_ms / args.steps * 1e3,
                                 "over_plain_us": (vo_ms / args.steps - avg_launch_ms) * 1e3,
                                 "note": "topk_indices(order='value'): the selection with each "
                                         "row's columns ranked by value"}
        pers_ms, _, _ = time_workload(w, args.steps, args.warmup, copies=copies, path="persist")
        result["persistent_grid"] = {"launch_us_mean": pers_ms / args.steps * 1e3,
                                     "over_plain_us": (pers_ms / args.steps - avg_launch_ms) * 1e3,
                                     "note": "path='persist': the same kernel on a fixed grid of the "
                                             "workgroups the device holds at once"}
        warm_ms, _, _ = time_workload(w, args.steps, args.warmup, copies=1)
        result["warm_cache"] = {"input_copies": 1, "launch_us_mean": warm_ms / args.steps * 1e3,
                                "achieved_gbs": alg_bytes / (warm_ms / args.steps * 1e-3) / 1e9,
                                "note": "one input copy reused: parts of it may be served from the caches"}
        rc = read_ceiling(w, args.steps, args.warmup, copies)
        rc["topk_over_read_time"] = avg_launch_ms * 1e3 / rc["us_per_launch"]
        rc["topk_gbs_over_read_gbs"] = achieved / rc["gbs"]
        result["read_ceiling"] = rc
        result["c128a_metadata"] = time_c128a(args.steps, args.warmup)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
