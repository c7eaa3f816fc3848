"""Benchmark of mixed FP8/TQ3 paged decode on one MI355X.

One step = one mkv_decode call over the whole batch of the workload (all
partial kernels and the merge, schedule cached), with the cache already
resident in HBM.  The default workload is the 131072-token long-context case
(B=1, Hq=48, Hkv=8, d=128, 16-token pages, last 4096 tokens FP8, the rest
TQ3).  The cache is held in R identical replicas, one pool each (like the
per-layer caches of a model), at different seeded physical pages; consecutive
steps decode different replicas, so the 256 MB last-level cache cannot serve
a step from the previous one.  Workloads whose live KV already exceeds a few GB
use one pool with their own slab sizes.

Prints one JSON line:
  value        KV GB/s = algorithmic bytes per step / step time (mean over the
               timed steps; config adds per-step p10 / p50 / p90 from a pass
               with an event pair around every step, and the KV GB/s as a share
               of a plain 1 GiB device copy's read + write rate)
  roofline     the dominant kernel (the partial kernel, which reads every KV
               byte of the step in one launch): its algorithmic bytes per
               launch / its mean launch time from HIP events recorded on the
               decode stream during a second timed region of the same steps
               (the first, without library events, gives value), against 8 TB/s
  cpu_baseline the CPU oracle on the same workload (bounded repetitions)
  comparison   the same rows as a dense BF16 control cache and as an all-FP8
               cache (no demotion), decoded the same way: their us/step, the
               mixed cache's throughput relative to each (the control ratio
               of the Minima-KV summary's canary test) and KV bytes per live
               token (its compression relative to BF16 and FP8); and the
               materialising profile (every step expands the cache into dense
               bf16 rows of a control pool, then decodes that copy)

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long] [--no-compare]
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

METRIC = "mixed FP8/TQ3 paged decode: µs/step and achieved KV HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0
# Sources of the decode kernels: the partial kernel's own (its HBM traffic
# record is keyed to these) and, with the merge, those of a whole decode step
# (the per-dispatch duration records).
PARTIAL_SOURCES = ["kernels_partial.hip", "mkv_device.hpp", "mkv_kernels.hpp"]
KERNEL_SOURCES = PARTIAL_SOURCES + ["kernels_merge.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_src_hash(names=None) -> str:
    """Hash of the kernel sources with comments and blank lines left out, so a
    record made with the kernels stays keyed to them when only their comments
    change."""
    import re
    h = hashlib.sha256()
    for name in names or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_mixed_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(text.encode())
    return h.hexdigest()[:16]


def workload(name):
    from decode_attention_mixed_amd import workloads as W
    if name.startswith("sweep"):
        return W.sweep(int(name[5:]) / 100.0)
    if name.startswith("canary"):
        return W.canary(int(name[6:] or 16))
    return getattr(W, name)()


def describe(wl) -> str:
    if wl.B == 1:
        L = f"L={int(wl.lengths[0])}"
    else:
        L = f"L in [{int(wl.lengths.min())},{int(wl.lengths.max())}]"
    fp8 = sum(len(a) for a in wl.anchors)
    tot = sum(wl.n_pages(b) for b in range(wl.B))
    return (f"{wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} d={wl.d} page={wl.P} {L}, "
            f"{fp8}/{tot} pages FP8 (e4m3) and the rest TQ3")


def kv_bytes(wl):
    """Algorithmic bytes per decode step and per format (codes, TQ3 group
    scales, FP8 page-head scales of every live token of the batch)."""
    fp8 = tq3 = 0
    for b in range(wl.B):
        L = int(wl.lengths[b])
        anchors = set(int(p) for p in wl.anchors[b])
        for lp in range(wl.n_pages(b)):
            n = min(wl.P, L - lp * wl.P)
            if lp in anchors:
                fp8 += n * 2 * wl.Hkv * wl.d + 8 * wl.Hkv
            else:
                tq3 += n * wl.Hkv * wl.d * 7 // 8
    return fp8, tq3


def cpu_baseline(wl, per_step_bytes, budget_s=20.0):
    """Time the CPU oracle's decode step on the same workload (bounded)."""
    import numpy as np
    from oracle import attention as A
    from oracle import pool_model as PM
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    models = []
    for b in range(wl.B):
        k, v = wl.kv(b)
        m = PM.SeqModel(wl.Hkv, wl.d, wl.P)
        m.append(k, v)
        for lp in wl.demote_pages(b):
            m.demote(int(lp))
        models.append(m)
        del k, v
    reps = 0
    t0 = time.perf_counter()
    while True:
        for b in range(wl.B):
            A.decode_seq(models[b], wl.q_bits[b], wl.tau)
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 50:
            break
    dt = (time.perf_counter() - t0) / reps
    model_name = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model_name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": per_step_bytes / dt / 1e9, "unit": "GB/s", "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{reps} full decode step(s) of the same workload, {dt:.3f} s/step "
                  f"({per_step_bytes / dt / 1e6:.1f} MB/s); numpy fp64 on '{model_name}', "
                  f"BLAS threads {blas_threads}, host cpus {os.cpu_count()}",
    }


def load_traffic(kernel: str, wl_name: str):
    """HBM bytes per launch measured by rocprofv3 counters (see write_traffic),
    if taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{wl_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_src_hash(PARTIAL_SOURCES):
        return None
    return t.get("bytes_per_launch")


def _pmc_means(csv_path: str, name_part: str, counter: str):
    """Per-dispatch mean of a rocprofv3 counter over the kernels whose name
    contains name_part (counter_collection.csv of one --pmc pass)."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"{csv_path}: no {counter} samples for kernels matching {name_part!r}")
    return sum(vals) / len(vals), len(vals)


def _req_bytes(rd_csv, wr_csv, name_part):
    """HBM bytes per dispatch of the kernels matching name_part from the
    L2-to-memory request counters: reads 32/64/128 B per request by size
    class, writes 64 B (TCC_EA0_WRREQ_64B) or 32 B (the rest of
    TCC_EA0_WRREQ)."""
    n32, nd = _pmc_means(rd_csv, name_part, "TCC_EA0_RDREQ_32B_sum")
    n64, _ = _pmc_means(rd_csv, name_part, "TCC_EA0_RDREQ_64B_sum")
    n128, _ = _pmc_means(rd_csv, name_part, "TCC_EA0_RDREQ_128B_sum")
    nrd, _ = _pmc_means(rd_csv, name_part, "TCC_EA0_RDREQ_sum")
    w64, nw = _pmc_means(wr_csv, name_part, "TCC_EA0_WRREQ_64B_sum")
    wall, _ = _pmc_means(wr_csv, name_part, "TCC_EA0_WRREQ_sum")
    rd = 32 * n32 + 64 * n64 + 128 * n128
    wr = 64 * w64 + 32 * (wall - w64)
    return {"read_bytes": rd, "write_bytes": wr, "read_requests": nrd,
            "read_requests_by_size": [n32, n64, n128], "unsized_read_requests": nrd - n32 - n64 - n128,
            "write_requests": wall, "write_requests_64B": w64, "dispatches": [nd, nw]}


def write_traffic(rd_csv, wr_csv, copy_rd_csv, copy_wr_csv, copy_bytes, wl_name, commands=None):
    """HBM bytes per launch of the partial kernel from two rocprofv3 --pmc
    passes (read-request counters by size, write-request counters), checked on
    a plain copy of copy_bytes bytes (read and written once), whose counted
    bytes are reported beside the true ones rather than used as a scale.
    Writes profiles/traffic_partial_<workload>.json."""
    k = _req_bytes(rd_csv, wr_csv, "partial_mixed")
    c = _req_bytes(copy_rd_csv, copy_wr_csv, "copyBuffer")
    out = {
        "kernel": "partial", "workload": wl_name, "kernel_src_sha": kernel_src_hash(PARTIAL_SOURCES),
        "bytes_per_launch": round(k["read_bytes"] + k["write_bytes"]),
        "read_bytes_per_launch": round(k["read_bytes"]), "write_bytes_per_launch": round(k["write_bytes"]),
        "read_requests_32_64_128B": [round(x) for x in k["read_requests_by_size"]],
        "unsized_read_requests": round(k["unsized_read_requests"]),
        "write_requests": round(k["write_requests"]), "write_requests_64B": round(k["write_requests_64B"]),
        "dispatches": k["dispatches"],
        "copy_check": {"bytes": copy_bytes, "counted_read_bytes": round(c["read_bytes"]),
                       "counted_write_bytes": round(c["write_bytes"]),
                       "read_ratio": round(c["read_bytes"] / copy_bytes, 4),
                       "write_ratio": round(c["write_bytes"] / copy_bytes, 4)},
        "commands": list(commands or []),
    }
    path = os.path.join(ROOT, "profiles", f"traffic_partial_{wl_name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def kernel_stats(trace_csv, wl_name, steps, commands=None):
    """Per-dispatch durations of the partial and merge kernels from a
    rocprofv3 --kernel-trace CSV of a bench run (the last `steps` dispatches
    of each, i.e. the timed steps): mean and percentiles, and the same for
    their sum per step.  Writes profiles/kernel_durations_<workload>.json."""
    import csv
    import numpy as np
    rows = list(csv.DictReader(open(trace_csv)))
    def durs(part):
        d = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
             for r in rows if part in r["Kernel_Name"]]
        d.sort()
        return np.array([x[1] for x in d[-steps:]], dtype=np.float64) / 1e3
    part, merge = durs("partial_mixed"), durs("merge")
    n = min(len(part), len(merge))
    step = part[-n:] + merge[-n:]
    def summ(x):
        return {"mean": round(float(x.mean()), 3),
                **{f"p{k}": round(float(np.percentile(x, k)), 3) for k in (10, 50, 90, 99)}}
    out = {"workload": wl_name, "kernel_src_sha": kernel_src_hash(), "dispatches": int(n),
           "partial_us": summ(part[-n:]), "merge_us": summ(merge[-n:]), "partial_plus_merge_us": summ(step),
           "commands": list(commands or [])}
    path = os.path.join(ROOT, "profiles", f"kernel_durations_{wl_name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def load_kernel_stats(wl_name):
    path = os.path.join(ROOT, "profiles", f"kernel_durations_{wl_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    return t if t.get("kernel_src_sha") == kernel_src_hash() else None


def read_ceiling(mkv, torch, nbytes=4 * 2**30, reps=10):
    """Read ceiling of the device: the library's read-only calibration kernel
    over nbytes (16-byte loads), GB/s."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(7)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    for _ in range(3):
        mkv.debug_read_bandwidth(src, sink)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mkv.debug_read_bandwidth(src, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, sink
    torch.cuda.empty_cache()
    return gbs


def copy_calibration(nbytes: int, steps: int):
    """A plain copy kernel of known size: reads and writes nbytes per launch."""
    import torch
    torch.cuda.set_device(0)
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    print(json.dumps({"copy_bytes": nbytes, "launches": steps + 3, "ms_per_copy": round(ms, 6),
                      "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--replicas", type=int, default=0, help="0: 8, or 1 for multi-GB workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the BF16-control and all-FP8 comparison runs")
    ap.add_argument("--serve", type=int, default=0, metavar="N",
                    help="also run N mkv_decode_step calls: each appends one token to every "
                         "sequence, converts the pages the library's anchor policy releases and decodes")
    ap.add_argument("--layer-calls", type=int, default=0, metavar="N",
                    help="also time the batch as N calls over consecutive entries (a multi-layer "
                         "workload decoded layer by layer instead of in one call)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes --steps "
                         "times (reference for the HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=5, metavar=("RDREQ_CSV", "WRREQ_CSV", "COPY_RDREQ_CSV",
                                                          "COPY_WRREQ_CSV", "COPY_BYTES"),
                    help="only turn rocprofv3 --pmc request-counter files (TCC_EA0_RDREQ{,_32B,_64B,"
                         "_128B}_sum; TCC_EA0_WRREQ{,_64B}_sum) into the partial kernel's HBM "
                         "traffic record under profiles/ (no GPU needed)")
    ap.add_argument("--kernel-stats", metavar="KERNEL_TRACE_CSV",
                    help="only turn a rocprofv3 --kernel-trace CSV of a bench run into per-dispatch "
                         "duration percentiles under profiles/ (no GPU needed; --steps = the run's)")
    ap.add_argument("--profile-command", action="append", default=[], metavar="TEXT",
                    help="with --kernel-stats / --write-traffic: the profiler command that made "
                         "each input file, recorded in the summary (repeatable, in input order)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this library "
              "has no multi-GPU path; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.write_traffic:
        f1, f2, f3, f4, nb = args.write_traffic
        write_traffic(f1, f2, f3, f4, int(nb), args.workload, args.profile_command)
        return
    if args.kernel_stats:
        kernel_stats(args.kernel_stats, args.workload, args.steps, args.profile_command)
        return

    import numpy as np
    import torch

    import decode_attention_mixed_amd as mkv
    from decode_attention_mixed_amd import harness as H

    torch.cuda.set_device(0)
    wl = workload(args.workload)
    fp8_b, tq3_b = kv_bytes(wl)
    step_bytes = fp8_b + tq3_b
    R = args.replicas if args.replicas > 0 else (8 if step_bytes < 2**30 else 1)
    log(f"workload {describe(wl)}; {step_bytes} KV bytes/step; {R} replicas")

    # R pools, each holding one replica of the batch at its own (seeded, scattered)
    # physical pages, like the per-layer caches of a model; step i decodes pool i % R.
    n_anchor = sum(len(a) for a in wl.anchors)
    all_pages = sum(wl.n_pages(b) for b in range(wl.B))
    n_tq3 = all_pages - n_anchor
    max_pages = max(wl.n_pages(b) for b in range(wl.B))
    kvs = [wl.kv(b) for b in range(wl.B)] if wl.B * max_pages * wl.P * wl.Hkv * wl.d <= 2**29 else None
    q = H.q_tensor(wl)
    out = torch.empty(wl.B, wl.Hq, wl.d, device="cuda")
    lse = torch.empty(wl.B, wl.Hq, device="cuda")
    batch = list(range(wl.B))
    tau = float(wl.tau)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    build_rates = {}

    def build(kind):
        """R pools of one kind: "mixed" (anchors FP8, the rest demoted to TQ3),
        "bf16" (control pool) or "fp8" (mixed pool, nothing demoted)."""
        t0 = time.perf_counter()
        pools = []
        grow = (args.serve // wl.P + 2) if kind == "mixed" and args.serve > 0 else 0   # serve headroom
        for r in range(R):
            if kind == "mixed" and R == 1:
                desc = H.pool_desc(wl, max_pages_per_seq=max_pages + grow,
                                   fp8_pages=wl.fp8_pages + wl.B * grow,
                                   tq3_pages=wl.tq3_pages + wl.B * grow)
            elif kind == "mixed":
                desc = H.pool_desc(wl, fp8_pages=n_anchor + max_pages + 16 + wl.B * grow,
                                   tq3_pages=n_tq3 + 16 + wl.B * grow,
                                   max_pages_per_seq=max_pages + grow,
                                   placement_seed=wl.placement_seed + r)
            else:
                desc = H.pool_desc(wl, kind=kind, fp8_pages=all_pages + 16,
                                   placement_seed=wl.placement_seed + r)
            pools.append(H.DevicePool(desc))
        # replica 0 of the mixed cache is built with events around each
        # sequence's append and conversion (the cache-write kernels' rates)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        t_app = t_dem = 0.0
        n_dem = 0
        if kind == "mixed":
            mkv.profile_enable(pools[0].handle, True)
        for b in range(wl.B):
            kv = kvs[b] if kvs is not None else wl.kv(b)
            for r in range(R):
                if kind == "mixed" and r == 0:
                    kd = torch.from_numpy(kv[0]).cuda().contiguous()
                    vd = torch.from_numpy(kv[1]).cuda().contiguous()
                    dem = wl.demote_pages(b)
                    torch.cuda.synchronize()
                    ev[0].record()
                    mkv.append(pools[0].handle, b, kd, vd)
                    ev[1].record()
                    if dem.size:
                        mkv.demote(pools[0].handle, b, dem)
                    ev[2].record()
                    torch.cuda.synchronize()
                    t_app += ev[0].elapsed_time(ev[1])
                    t_dem += ev[1].elapsed_time(ev[2])
                    n_dem += int(dem.size)
                    del kd, vd
                else:
                    H.load_sequence(pools[r], wl, b, kv=kv, demote=(kind == "mixed"))
        torch.cuda.synchronize()
        st = mkv.pool_stats(pools[0].handle)
        log(f"{kind} cache built in {time.perf_counter() - t0:.1f} s: {st}")
        if kind == "mixed":
            kprof = mkv.profile_read(pools[0].handle)
            mkv.profile_enable(pools[0].handle, False)
            toks = int(sum(int(x) for x in wl.lengths))
            app_bytes = toks * wl.Hkv * wl.d * (2 * 4 + 2)        # fp32 K, V read; FP8 codes written
            dem_bytes = n_dem * (2 * wl.Hkv * wl.P * wl.d + 2 * wl.Hkv * wl.P * (wl.d // 32) * 14)
            ka, kd = kprof["ms_append"], kprof["ms_demote"]
            build_rates.update({
                "what": "replica 0 of the cache: kernel time from the library's events around the "
                        "append and conversion launches; call time from events around each mkv_append "
                        "and mkv_demote call (host metadata and uploads included)",
                "append_kernel_us": round(ka * 1e3, 1),
                "append_kernel_gbs": round(app_bytes / (ka * 1e-3) / 1e9, 1) if ka else None,
                "append_kernel_frac": round(app_bytes / (ka * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if ka else None,
                "append_call_us": round(t_app * 1e3, 1),
                "demote_pages": n_dem,
                "demote_kernel_us": round(kd * 1e3, 1),
                "demote_kernel_gbs": round(dem_bytes / (kd * 1e-3) / 1e9, 1) if kd else None,
                "demote_kernel_frac": round(dem_bytes / (kd * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if kd else None,
                "demote_call_us": round(t_dem * 1e3, 1),
                "bytes": {"append": app_bytes, "demote": dem_bytes}})
        return pools, st

    def timed_steps(pools):
        torch.cuda.synchronize()
        ev0.record()
        t0 = time.perf_counter()
        for i in range(args.steps):
            mkv.decode(pools[i % R].handle, batch, q, tau, out, lse)
        host_s = time.perf_counter() - t0
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / args.steps, host_s / args.steps

    def warm(pools):
        for i in range(max(args.warmup, R)):
            mkv.decode(pools[i % R].handle, batch, q, tau, out, lse)
        torch.cuda.synchronize()

    pools, mixed_stats = build("mixed")
    warm(pools)
    sched = mkv.debug_schedule(pools[0].handle, arrays=False)
    log(f"decode schedule: {sched}")
    # Timed region 1: the step as a caller sees it (no library events).
    ms, host_s = timed_steps(pools)
    # Timed region 2: the same steps with the library's per-kernel HIP events
    # recorded on the decode stream (kernel durations for the roofline).
    for p in pools:
        mkv.profile_enable(p.handle, True)
        mkv.profile_read(p.handle)
    ms_ev, _ = timed_steps(pools)
    prof = {}
    for p in pools:
        for k2, v2 in mkv.profile_read(p.handle).items():
            prof[k2] = prof.get(k2, 0) + v2
        mkv.profile_enable(p.handle, False)
    log(f"step {ms * 1e3:.2f} us (host {host_s * 1e6:.1f} us per call; {ms_ev * 1e3:.2f} us with "
        f"kernel events); kernel profile {prof}")
    multi = None
    if args.layer_calls > 0:
        assert wl.B % args.layer_calls == 0
        per = wl.B // args.layer_calls
        groups = [(batch[i * per:(i + 1) * per], q[i * per:(i + 1) * per].contiguous(),
                   out[i * per:(i + 1) * per], lse[i * per:(i + 1) * per])
                  for i in range(args.layer_calls)]
        def layer_steps(n):
            torch.cuda.synchronize()
            ev0.record()
            for i in range(n):
                for ids, qg, og, lg in groups:
                    mkv.decode(pools[i % R].handle, ids, qg, tau, og, lg)
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / n
        layer_steps(max(args.warmup, R))
        ms_layers = layer_steps(args.steps)
        multi = {"calls": args.layer_calls, "entries_per_call": per,
                 "us_per_step_one_call": round(ms * 1e3, 3),
                 "us_per_step_per_call": round(ms_layers * 1e3, 3),
                 "one_call_speedup": round(ms_layers / ms, 4)}
        log(f"layer by layer: {multi}")
    materialised = None
    if not args.no_compare:
        # Materialising profile: each step expands the whole batch of replica
        # i % R into dense bf16 rows of a control pool and decodes that copy.
        dpools = [H.DevicePool(H.pool_desc(wl, kind="bf16", fp8_pages=all_pages + 16,
                                           placement_seed=wl.placement_seed + r)) for r in range(R)]

        def mat_steps(n, with_decode):
            torch.cuda.synchronize()
            ev0.record()
            for i in range(n):
                src, dst = pools[i % R], dpools[i % R]
                for b in batch:
                    mkv.seq_reset(dst.handle, b)
                    mkv.materialize(src.handle, b, dst.handle, b)
                if with_decode:
                    mkv.decode(dst.handle, batch, q, tau, out, lse)
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / n

        mat_steps(max(args.warmup, R), True)
        mat_only = mat_steps(args.steps, False)
        mat_step = mat_steps(args.steps, True)
        materialised = {"materialise_us": round(mat_only * 1e3, 3),
                        "us_per_step": round(mat_step * 1e3, 3),
                        "mixed_throughput_ratio": round(mat_step / ms, 4)}
        log(f"materialising profile: {materialised}")
        for p in dpools:
            p.close()
        del dpools
    serve = None
    if args.serve > 0:
        # Decode-step loop: the recent window is the workload's FP8 tail; anchors
        # older than it stay protected (FP8) for good.
        # The library applies the anchor policy (mkv_set_anchor_window, with the
        # workload's older anchors protected) inside each mkv_decode_step call.
        window = {"long": 4096, "throughput": 1024, "ragged": 512}.get(wl.name, 1024)
        for p in pools:
            mkv.set_anchor_window(p.handle, window)
            for b in range(wl.B):
                L = int(wl.lengths[b])
                mkv.protect_pages(p.handle, b, [a for a in wl.anchors[b] if (a + 1) * wl.P <= L - window])
        tq3_before = sum(mkv.pool_stats(p.handle)["tq3_pages_live"] for p in pools)
        gen = torch.Generator(device="cuda").manual_seed(7)
        rows_k = torch.randn(16, wl.B, wl.Hkv, wl.d, device="cuda", generator=gen)
        rows_v = torch.randn(16, wl.B, wl.Hkv, wl.d, device="cuda", generator=gen)
        torch.cuda.synchronize()
        ev0.record()
        t0 = time.perf_counter()
        for i in range(args.serve):
            mkv.decode_step(pools[i % R].handle, batch, rows_k[i % 16], rows_v[i % 16], q, tau, out, lse)
        host = (time.perf_counter() - t0) / args.serve
        ev1.record()
        torch.cuda.synchronize()
        ms_serve = ev0.elapsed_time(ev1) / args.serve
        n_dem = sum(mkv.pool_stats(p.handle)["tq3_pages_live"] for p in pools) - tq3_before
        serve = {"steps": args.serve, "window_tokens": window,
                 "us_per_step": round(ms_serve * 1e3, 3),
                 "host_us_per_step": round(host * 1e6, 2),
                 "decode_only_us_per_step": round(ms * 1e3, 3),
                 "ratio_to_decode_only": round(ms_serve / ms, 3),
                 "pages_demoted": n_dem}
        log(f"serve: {serve}")
    for p in pools:
        p.close()
    del pools
    torch.cuda.empty_cache()

    comparison = None
    if not args.no_compare:
        tokens = int(mixed_stats["live_tokens"])
        comparison = {"mixed": {"us_per_step": round(ms * 1e3, 3),
                                "kv_bytes_per_token": round(mixed_stats["bytes_per_token"], 2)}}
        for kind, label in (("bf16", "bf16_control"), ("fp8", "all_fp8")):
            cpools, cst = build(kind)
            warm(cpools)
            cms, _ = timed_steps(cpools)
            comparison[label] = {
                "us_per_step": round(cms * 1e3, 3),
                "kv_bytes_per_token": round(cst["bytes_per_token"], 2),
                "kv_gbs": round(cst["kv_bytes"] / (cms * 1e-3) / 1e9, 2),
                "mixed_throughput_ratio": round(cms / ms, 4),
                "mixed_compression": round(cst["bytes_per_token"] / mixed_stats["bytes_per_token"], 4),
            }
            assert int(cst["live_tokens"]) == tokens
            log(f"{kind}: {comparison[label]}")
            for p in cpools:
                p.close()
            del cpools
            torch.cuda.empty_cache()
        comparison["materialising_profile"] = materialised
    del kvs

    # Practical HBM ceiling on this device: a 1 GiB device-to-device copy,
    # counting the bytes read and written (context for the KV GB/s).
    src = torch.empty(2**30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(10):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    copy_ceiling = 2.0 * 2**30 * 10 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    read_ceil = read_ceiling(mkv, torch)

    kernel_ms = {"partial": prof["ms_partial"] / max(1, prof["n_partial"]),
                 "merge": prof["ms_merge"] / max(1, prof["n_merge"])}
    # the dominant kernel: the partial kernel, one launch reads every KV byte
    dom = "partial"
    dom_bytes = step_bytes
    achieved = dom_bytes / (kernel_ms[dom] * 1e-3) / 1e9 if kernel_ms[dom] > 0 else 0.0
    value = step_bytes / (ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_step": round(ms * 1e3, 3),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: seeded N(0,1) fp32 K/V (outlier channels x8), bf16 N(0,1) query",
        "config": {
            "workload": describe(wl),
            "arithmetic": "f16 MFMA operands (exact FP8/TQ3 codes, hi/lo split probabilities), "
                          "f32 accumulation and softmax",
            "kv_bytes_per_step": step_bytes,
            "kv_bytes_fp8": fp8_b,
            "kv_bytes_tq3": tq3_b,
            "split_k": {"chunks": sched["n_chunks"], "work_items": sched["n_items"],
                        "most_chunks_per_entry": sched["max_seq_chunks"],
                        "kv_heads_per_workgroup": sched["heads_per_wave"],
                        "resident_waves": sched["resident_waves"]},
            "replicas_rotated": R,
            "kernel_us": {k: round(v * 1e3, 3) for k, v in kernel_ms.items()},
            "host_us_per_call": round(host_s * 1e6, 2),
            "us_per_step_with_kernel_events": round(ms_ev * 1e3, 3),
            "kernel_durations_rocprof": load_kernel_stats(wl.name),
            "copy_ceiling_gbs": round(copy_ceiling, 1),
            "pct_of_copy_ceiling": round(100.0 * value / copy_ceiling, 2) if copy_ceiling else None,
            "read_ceiling_gbs": round(read_ceil, 1),
            "pct_of_read_ceiling": round(100.0 * value / read_ceil, 2) if read_ceil else None,
            "cache_build": build_rates,
        },
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(dom, wl.name),
            "algorithmic_bytes_per_launch": dom_bytes,
        },
    }
    if comparison is not None:
        result["comparison"] = comparison
    if multi is not None:
        result["multi_layer"] = multi
    if serve is not None:
        result["serve"] = serve
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, step_bytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
