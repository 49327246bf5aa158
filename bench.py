"""Throughput of exact per-row top-k on one MI355X.

One step = one call of the whole path (one kernel launch per batch) over one
batch of synthetic input already resident in HBM.  The timed K steps are
captured once into a HIP graph and replayed, so host launch overhead is not
measured.  Each step reads a different copy of the inputs from a ring of at
least 512 MiB, so the 256 MiB last-level cache cannot serve the scores.

Prints one JSON line: rows/s (value) plus effective HBM GB/s against the
8 TB/s peak (roofline) and the CPU oracle's rows/s on the host (cpu_baseline).
After the headline workload (C3 by default), every named workload C1 .. C5 is
timed the same way over max(K, 200) calls (per_config), each with its empty
launch and read-only floors; none of that is inside the headline's timed
region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "rows/sec and effective HBM GB/s (% of peak), top-k k=1024/2048, 1 GPU"
HBM_PEAK_GBS = 8000.0
RING_BYTES = 512 << 20
KERNEL_SOURCE = os.path.join(ROOT, "exact_top_selection_amd", "csrc", "ets_topk.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(w) -> int:
    """Bytes the method must move per call: each valid score read once, the
    k outputs written, the length read, the touched page-table entries (paged)
    or the row start (ragged)."""
    n = w.row_lengths.astype(np.int64)
    total = 4 * n + 4 * w.k + 4
    if w.api == "paged":
        total += 4 * ((n + w.page_size - 1) // w.page_size)
    if w.api == "ragged":
        total += 4
    return int(total.sum())


def kernel_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, budget_s: float):
    """The CPU oracle on the host cores over repeated full batches, with as
    many threads as the host offers (at most 16), then on one thread."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    oracle.build()

    def once(nt):
        if w.api == "raw":
            oracle.topk_raw(w.scores, w.k, w.lens, threads=nt)
        elif w.api == "paged":
            oracle.topk_paged(w.scores, w.lens, w.page_table, w.page_size, w.k, threads=nt)
        else:
            oracle.topk_ragged(w.scores, w.row_starts, w.lengths, w.k, threads=nt)

    def rate(nt, budget):
        once(nt)  # warm
        reps = 0
        t0 = time.perf_counter()
        while True:
            once(nt)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 10000:
                return reps, el

    reps, el = rate(threads, budget_s)
    reps1, el1 = rate(1, budget_s / 2)
    rows, rows1 = reps * w.B, reps1 * w.B
    return {"value": rows / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "value_1thread": rows1 / el1,
            "sample": "%d full batches of %s (%d rows) in %.1f s on %d threads, and %d batches "
                      "in %.1f s on 1 thread; %s, %d logical CPUs"
                      % (reps, w.name, rows, el, threads, reps1, el1, cpu_model(),
                         os.cpu_count() or 0)}


COPY_BYTES = 256 << 20


def calibrate_copy(torch, steps: int) -> int:
    """A plain device-to-device copy of COPY_BYTES per launch: the reference for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(max(steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "launches": max(steps, 1)}))
    return 0


def _pmc_per_dispatch(path: str, counter: str, name_part: str):
    """Mean counter value per dispatch of kernels whose name contains name_part."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Dispatch_Id"], 0.0)
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        return None, 0
    return sum(vals.values()) / len(vals), len(vals)


def traffic_report(d: str, workload: str, seed: int) -> int:
    """Reads DIR/{fetch,write,copy_fetch,copy_write}/*counter_collection.csv."""
    import glob
    import workloads

    def one(sub, counter, part):
        files = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter csv under %s/%s" % (d, sub))
        return _pmc_per_dispatch(files[0], counter, part)

    kf, nkf = one("fetch", "FETCH_SIZE", "topk_kernel")
    kw, nkw = one("write", "WRITE_SIZE", "topk_kernel")
    cf, ncf = one("copy_fetch", "FETCH_SIZE", "copy")
    cw, ncw = one("copy_write", "WRITE_SIZE", "copy")
    # counters are in KiB per dispatch; scale each by the copy kernel's reading
    sf = COPY_BYTES / (cf * 1024.0)
    sw = COPY_BYTES / (cw * 1024.0)
    fetch_b = kf * 1024.0 * sf
    write_b = kw * 1024.0 * sw
    w = workloads.make(workload, seed=seed)
    rec = {"kernel_sha": kernel_hash(), "bytes_per_launch": fetch_b + write_b,
           "fetch_bytes": fetch_b, "write_bytes": write_b,
           "fetch_kib_raw": kf, "write_kib_raw": kw, "copy_fetch_scale": sf,
           "copy_write_scale": sw, "algorithmic_bytes": algorithmic_bytes(w),
           "dispatches": [nkf, nkw, ncf, ncw]}
    try:
        with open(TRAFFIC_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec[w.name] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    print(json.dumps({w.name: rec}, indent=1))
    return 0



def timed(torch, step, steps: int, warmup: int, eager: bool) -> float:
    """Milliseconds for exactly `steps` calls of step(i), after `warmup` untimed
    ones; the timed calls are one captured graph unless `eager`.  HIP events on
    the stream the calls run on."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if not eager:
        graph = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        cap_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap_stream):
            with torch.cuda.graph(graph, stream=cap_stream):
                for i in range(steps):
                    step(warmup + i)
        torch.cuda.current_stream().wait_stream(cap_stream)
        torch.cuda.synchronize()
        graph.replay()  # uploads the graph; untimed
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if eager:
        for i in range(steps):
            step(warmup + i)
    else:
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop)

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="C3", help="C1 .. C5 (default C3)")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-floors", action="store_true",
                    help="skip the empty-launch and read-only floors")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload lines (C1 .. C5) after the headline")
    ap.add_argument("--sweep", choices=["batch", "k", "spread", "split"],
                    help="instead of the headline: one JSON line per point of a sweep, "
                         "'batch' = paged decode rows of 32768 scores, k = 1024, B in "
                         "1 .. 512 (HIP graph and eager launches); 'k' = the C3 workload with "
                         "k in 1 .. 2048; 'spread' = raw rows of up to 262144 scores, "
                         "k = 2048, B in 4 .. 64, lengths all L or uniform in [L/2, L] or "
                         "[L/8, L], the split heuristic's choice against forced "
                         "workgroups per row (ETS_ROW_SPLIT); 'split' = raw rows of one "
                         "length, k = 2048, B in 1 .. 512, L in 65536 .. 262144, the "
                         "heuristic's choice against forced workgroups per row")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of replaying a HIP graph")
    ap.add_argument("--host-overhead", action="store_true",
                    help="instead of the headline: host time per eager call of the headline "
                         "workload, through the Python binding and as a direct C call with "
                         "prepared arguments (one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain device copy of known size (counter calibration) and exit")
    ap.add_argument("--traffic-report", metavar="DIR",
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE csv runs under DIR into "
                         "profiles/traffic.json and print a summary (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_report:
        return traffic_report(args.traffic_report, args.workload, args.seed)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the top-k rows are independent, so a batch "
              "shards across GPUs by row blocks with no exchange, and the library has no "
              "multi-GPU path of its own (run with --gpus 1)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    import exact_top_selection_amd as ets
    import workloads

    if args.calibrate_copy:
        return calibrate_copy(torch, args.steps)
    if args.sweep:
        return sweep(torch, ets, workloads, args)
    if args.host_overhead:
        return host_overhead(torch, ets, workloads, args)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    limits = ets.device_limits()
    aux_steps = max(args.steps, 200)  # floors and per-config lines

    # ---- the headline workload
    w = workloads.make(args.workload, seed=args.seed)
    rig = Rig(torch, ets, w, dev, limits)
    ms_total = timed(torch, rig.step, args.steps, args.warmup, args.eager)
    us_per_step = ms_total * 1e3 / args.steps
    rows_per_s = w.B / (us_per_step * 1e-6)
    abytes = algorithmic_bytes(w)
    achieved = abytes / (us_per_step * 1e-6) / 1e9  # GB/s; one kernel launch per step
    result = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": us_per_step * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": "%s: %s" % (w.name, w.note),
            "api": w.api, "B": w.B, "L": int(w.L or w.max_len), "k": w.k,
            "page_size": w.page_size or None, "seed": args.seed,
            "input_ring_copies": rig.R,
            "launch": "eager launches" if args.eager else "hip graph of K steps",
            "algorithmic_bytes_per_step": abytes,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(w.name),
            "kernel": rig.kernel,
            # one kernel per step: HIP events on the launching stream around the
            # K replayed steps, divided by K
            "us_per_launch": us_per_step,
        },
    }
    if not args.no_floors:
        result["floors"] = rig.floors(aux_steps, args.warmup, args.eager)
    del rig
    torch.cuda.empty_cache()

    # ---- every workload, timed the same way (outside the headline's timed region)
    if not args.no_configs:
        per = {}
        for name in workloads.NAMES:
            wc = workloads.make(name, seed=args.seed)
            rc = Rig(torch, ets, wc, dev, limits)
            us = timed(torch, rc.step, aux_steps, args.warmup, args.eager) * 1e3 / aux_steps
            ab = algorithmic_bytes(wc)
            gbs = ab / (us * 1e-6) / 1e9
            per[name] = {"us_per_call": us, "rows_per_s": wc.B / (us * 1e-6), "gb_per_s": gbs,
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": ab,
                         "kernel": rc.kernel, "calls": aux_steps}
            if not args.no_floors:
                per[name]["floors"] = rc.floors(aux_steps, args.warmup, args.eager)
            del rc
            torch.cuda.empty_cache()
        result["per_config"] = per
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def sweep_spread(torch, ets, workloads, args, dev, limits, steps) -> int:
    """The split heuristic sees only the longest row (the lengths stay on the
    device): rows whose lengths spread below it, timed with the heuristic's
    choice and with each forced number of workgroups per row."""
    from workloads import Workload
    L, k = 262144, 2048
    forced = (None, 0, 4, 8, 16, 32)
    old = os.environ.get("ETS_ROW_SPLIT")
    try:
        for B in (4, 16, 64):
            for lo_div in (1, 2, 8):
                rng = np.random.Generator(np.random.PCG64(args.seed + 1000 * B + lo_div))
                x = workloads.normal_dense(rng, B, L)
                lens = (np.full(B, L, dtype=np.int32) if lo_div == 1 else
                        rng.integers(L // lo_div, L, size=B, endpoint=True).astype(np.int32))
                spread = "all L" if lo_div == 1 else "U[L/%d, L]" % lo_div
                for g in forced:
                    if g is None:
                        os.environ.pop("ETS_ROW_SPLIT", None)
                    else:
                        os.environ["ETS_ROW_SPLIT"] = str(g)
                    w = Workload("spread-B%d-L%d-%s" % (B, L, spread), "raw", k, B, x, L=L,
                                 lens=lens, note="raw, N(0,1), lengths " + spread)
                    rig = Rig(torch, ets, w, dev, limits)
                    us_g = timed(torch, rig.step, steps, args.warmup, False) * 1e3 / steps
                    if rig.ws is not None:
                        assert ets.workspace_error(rig.ws) == 0, "a bounded wait expired"
                    ab = algorithmic_bytes(w)
                    print(json.dumps({"point": w.name, "B": B, "L": L, "k": k, "lengths": spread,
                                      "mean_len": float(lens.mean()),
                                      "split": "heuristic" if g is None else "forced",
                                      "groups": rig.split, "us_per_call_graph": us_g,
                                      "gb_per_s": ab / (us_g * 1e-6) / 1e9, "calls": steps}),
                          flush=True)
                    del rig
                    torch.cuda.empty_cache()
    finally:
        if old is None:
            os.environ.pop("ETS_ROW_SPLIT", None)
        else:
            os.environ["ETS_ROW_SPLIT"] = old
    return 0


def sweep_split(torch, ets, workloads, args, dev, limits, steps) -> int:
    """The (B, L) grid behind the split heuristic: raw N(0,1) rows all of
    length L, k = 2048, timed with the heuristic's choice and with each forced
    number of workgroups per row that the device allows (ETS_ROW_SPLIT)."""
    from workloads import Workload
    k = 2048
    points = [(B, L) for L in (65536, 131072, 262144)
              for B in (1, 4, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512)]
    cap = ets.group_cap(*limits)
    # the heuristic's own point last: the first launches after a new shape
    # (new ring buffers) can run slow
    forced = [0] + [g for g in (2, 3, 4, 5, 6, 8, 10, 12, 16, 32) if g <= cap] + [None]
    old = os.environ.get("ETS_ROW_SPLIT")
    try:
        for B, L in points:
            rng = np.random.Generator(np.random.PCG64(args.seed + 7 * B + L))
            x = workloads.normal_dense(rng, B, L)
            for g in forced:
                if g is None:
                    os.environ.pop("ETS_ROW_SPLIT", None)
                else:
                    os.environ["ETS_ROW_SPLIT"] = str(g)
                w = Workload("split-B%d-L%d" % (B, L), "raw", k, B, x, L=L,
                             lens=np.full(B, L, dtype=np.int32), note="raw, N(0,1), all rows L")
                rig = Rig(torch, ets, w, dev, limits)
                us_g = timed(torch, rig.step, steps, args.warmup, False) * 1e3 / steps
                if rig.ws is not None:
                    assert ets.workspace_error(rig.ws) == 0, "a bounded wait expired"
                ab = algorithmic_bytes(w)
                print(json.dumps({"point": w.name, "B": B, "L": L, "k": k,
                                  "split": "heuristic" if g is None else "forced",
                                  "groups": rig.split, "us_per_call_graph": us_g,
                                  "gb_per_s": ab / (us_g * 1e-6) / 1e9, "calls": steps}),
                      flush=True)
                del rig
                torch.cuda.empty_cache()
    finally:
        if old is None:
            os.environ.pop("ETS_ROW_SPLIT", None)
        else:
            os.environ["ETS_ROW_SPLIT"] = old
    return 0


def sweep(torch, ets, workloads, args) -> int:
    """Latency against batch size (the decode caller's flat region), against
    k, or against the spread of row lengths under the split heuristic."""
    from workloads import Workload
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    limits = ets.device_limits()
    steps = max(args.steps, 200)
    if args.sweep == "spread":
        return sweep_spread(torch, ets, workloads, args, dev, limits, steps)
    if args.sweep == "split":
        return sweep_split(torch, ets, workloads, args, dev, limits, steps)
    points = []
    if args.sweep == "batch":
        L, k, ps = 32768, 1024, 64
        for B in (1, 8, 32, 64, 128, 256, 512):
            rng = np.random.Generator(np.random.PCG64(args.seed + B))
            x = workloads.normal_dense(rng, B, L)
            pt = np.stack([rng.permutation(L // ps) for _ in range(B)]).astype(np.int32)
            w = Workload("decode-B%d" % B, "paged", k, B, x, L=L,
                         lens=np.full(B, L, dtype=np.int32), page_table=pt, page_size=ps,
                         note="paged, seq_lens all %d, k %d, N(0,1)" % (L, k))
            points.append(w)
    else:
        base = workloads.make("C3", seed=args.seed)
        for k in (1, 64, 256, 512, 1024, 2048):
            points.append(Workload("C3-k%d" % k, "paged", k, base.B, base.scores, L=base.L,
                                   lens=base.lens, page_table=base.page_table,
                                   page_size=base.page_size, note=base.note))
    for w in points:
        rig = Rig(torch, ets, w, dev, limits)
        us_g = timed(torch, rig.step, steps, args.warmup, False) * 1e3 / steps
        us_e = timed(torch, rig.step, steps, args.warmup, True) * 1e3 / steps
        ab = algorithmic_bytes(w)
        print(json.dumps({"point": w.name, "B": w.B, "k": w.k, "L": w.L,
                          "us_per_call_graph": us_g, "us_per_call_eager": us_e,
                          "rows_per_s": w.B / (us_g * 1e-6), "gb_per_s": ab / (us_g * 1e-6) / 1e9,
                          "frac": ab / (us_g * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "algorithmic_bytes": ab, "kernel": rig.kernel, "calls": steps}),
              flush=True)
        del rig
        torch.cuda.empty_cache()
    return 0


def host_overhead(torch, ets, workloads, args) -> int:
    """Host microseconds per eager call: the loop's time before the stream is
    drained (host-bound when above the kernel's time), and with the drain."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make(args.workload, seed=args.seed)
    if w.api != "paged":
        raise SystemExit("--host-overhead times the paged call (C1, C2, C3)")
    s = torch.from_numpy(w.scores).to(dev)
    lens = torch.from_numpy(w.lens).to(dev)
    pt = torch.from_numpy(w.page_table).to(dev)
    out = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
    ws = ets.new_workspace(w.B, w.L, w.k, dev)
    n = max(args.steps, 3000)
    lib = ets._load()
    prepared = (s.data_ptr(), s.stride(0), w.B, w.L, lens.data_ptr(), pt.data_ptr(), pt.stride(0),
                w.page_size, w.k, out.data_ptr(), out.stride(0),
                ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                torch.cuda.current_stream(dev).cuda_stream)

    def binding():
        ets.topk_paged(s, lens, pt, out, w.page_size, workspace=ws)

    def direct():
        lib.ets_topk_paged(*prepared)

    res = {}
    for name, f in (("binding", binding), ("direct_c", direct)):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            f()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        res[name] = {"host_us_per_call": (t1 - t0) / n * 1e6,
                     "us_per_call_with_drain": (t2 - t0) / n * 1e6}
    print(json.dumps({"host_overhead": res, "workload": w.name, "calls": n,
                      "eager_launches": True}), flush=True)
    return 0


class Rig:
    """One workload's inputs resident in HBM as a ring of copies (>= 512 MiB,
    so the 256 MiB last-level cache cannot serve the scores), its output and
    workspace, and one step = one call on copy i % R."""

    def __init__(self, torch, ets, w, dev, limits):
        self.w, self.dev, self.torch, self.ets = w, dev, torch, ets
        per_copy = w.scores.nbytes
        self.R = R = max(1, -(-RING_BYTES // per_copy))
        scores0 = torch.from_numpy(w.scores).to(dev)
        self.ring = ring = torch.empty((R,) + tuple(scores0.shape), dtype=torch.float32, device=dev)
        ring.copy_(scores0.unsqueeze(0).expand_as(ring))
        del scores0
        self.out = out = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
        self.max_len = w.max_len if w.api == "ragged" else w.L
        # one zero-filled workspace for every step (each call leaves it zero)
        self.ws = ws = ets.new_workspace(w.B, self.max_len, w.k, dev)
        self.split = ets.row_split(w.B, self.max_len, *limits)
        self.kernel = ("group_topk_kernel (%d workgroups per row)" % self.split if self.split
                       else "row_topk_kernel")
        if w.api == "paged":
            self.lens = lens = torch.from_numpy(w.lens).to(dev)
            pt = torch.from_numpy(w.page_table).to(dev)

            def step(i):
                ets.topk_paged(ring[i % R], lens, pt, out, w.page_size, workspace=ws)
        elif w.api == "raw":
            self.lens = lens = torch.from_numpy(w.lens).to(dev) if w.lens is not None else None

            def step(i):
                ets.topk_raw(ring[i % R], w.k, lens, out=out, workspace=ws)
        else:
            self.starts = starts = torch.from_numpy(w.row_starts).to(dev)
            self.lens = lengths = torch.from_numpy(w.lengths).to(dev)
            max_len = w.max_len

            def step(i):
                ets.topk_ragged(ring[i % R], starts, lengths, w.k, max_len=max_len, out=out,
                                workspace=ws)
        self.step = step

    def floors(self, steps, warmup, eager):
        """Per call: the same grid launched empty, and the same grid reading the
        same bytes and forming keys (one max per workgroup), timed the same way
        over the same input ring."""
        torch, ets, w, R, ring = self.torch, self.ets, self.w, self.R, self.ring
        sink = torch.empty(w.B * max(1, self.split), dtype=torch.int32, device=self.dev)
        if w.api == "ragged":
            starts, lengths, max_len = self.starts, self.lens, self.max_len

            def read_step(i):
                ets.floor_read(ring[i % R], lengths, starts, max_len, sink=sink)
        else:
            lens = self.lens

            def read_step(i):
                ets.floor_read(ring[i % R], lens, sink=sink)
        dev, B, max_len = self.dev, w.B, self.max_len

        def launch_step(i):
            ets.floor_launch(B, max_len, dev)
        return {"launch_us": timed(torch, launch_step, steps, warmup, eager) * 1e3 / steps,
                "read_us": timed(torch, read_step, steps, warmup, eager) * 1e3 / steps,
                "calls": steps,
                "what": "per call: an empty launch of the same grid; the same grid reading "
                        "the same bytes and forming keys, one max per workgroup"}


if __name__ == "__main__":
    sys.exit(main())
