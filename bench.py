"""Benchmark of the activation-compression hot path on one MI355X.

Headline (`value`): ZVC compress + ZVC decompress of one resident 4 GiB fp32
activation buffer (2^30 elements, zero fraction 0.5, the sparsity sweep's
largest workload), in GB/s of uncompressed input per round trip.  One step is
one round trip; the steps run back to back with the inputs already in HBM.

Rows beside it, each timed in a block of its own (HIP events on the launch
stream, no PCIe transfer running before them):
  * zvc_compress / zvc_decompress of the step, with their fraction of the
    8 TB/s HBM peak counted on algorithmic bytes (the roofline object names
    the longer of the two);
  * the other codecs on the same buffer: RLE, interleaved ZVC, fused ReLU + ZVC;
  * the sparsity sweep: ZVC and RLE both ways at zero fraction
    0 / 0.25 / 0.5 / 0.75 / 0.9 / 0.99 / 1 of the 4 GiB buffer, each call
    cold (the 256 MB last-level cache emptied before it);
  * the named CNN-like workloads (single map, AlexNet conv1, the VGG-16 stack,
    fp16 map), ZVC and RLE both ways, warm and cold;
  * the PCIe-bound stages: compressed offload and prefetch against raw copies.
The CPU oracle (single-threaded and on all host cores) is timed last.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--zero-frac S]

`python bench.py --summarize-profile DIR --out FILE` turns rocprofv3 output
(kernel trace with --stats, or a --pmc counter run) into a short text summary.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
N_ELEMS = 1 << 30
CHUNK = 1 << 24
SLOTS = 3
SPIN_CYCLES = 400_000  # ~0.2 ms of device-side spin ahead of a timed call
FLUSH_BYTES = 1 << 30  # read before a cold call: 4x the 256 MB last-level cache
CPU_ST_SAMPLE = 1 << 27  # elements for the single-threaded oracle (about 2 s per round trip)
CPU_MT_SAMPLE = 1 << 30  # elements for the oracle on all host cores (the whole buffer)
KERNEL_SOURCES = ("sparse_activation_compression_amd/csrc/zvc_compress.hpp",
                  "sparse_activation_compression_amd/csrc/zvc_decompress.hpp",
                  "sparse_activation_compression_amd/csrc/zvc_common.hpp",
                  "sparse_activation_compression_amd/csrc/device_common.hpp",
                  "sparse_activation_compression_amd/csrc/kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "zvc_kernels_sweep4GiB_s0.5_traffic.md")
ALGO_ID = {"zvc": 0, "rle": 1, "zvci": 2}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch of the two ZVC kernels from the committed counter
    summary ({'zvc_compress': B, 'zvc_decompress': B}), or {} if the file is
    missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return {}
    out = {}
    for k in ("zvc_compress", "zvc_decompress"):
        try:
            out[k] = float(vals[f"hbm_bytes_per_launch_{k}"])
        except (KeyError, ValueError):
            pass
    return out


# ----------------------------------------------------------------------------
# rocprofv3 summaries
# ----------------------------------------------------------------------------

def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _newest(d: str, pattern: str) -> list:
    """Files under d matching pattern, newest first (a rerun into the same
    directory leaves the older run's files beside the new ones)."""
    return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True), key=os.path.getmtime, reverse=True)


def summarize_profile(d: str, out: str, command: str, calib_bytes: float | None) -> None:
    lines = [f"# rocprofv3 summary: {os.path.basename(out)}", "", f"Command: `{command}`", ""]
    stats = _newest(d, "*kernel_stats.csv")
    counters = _newest(d, "*counter_collection.csv")
    if stats:
        rows = _read_csv(stats[0])
        lines += ["| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
        for r in rows:
            name = r.get("Name", "?")
            short = name.split("(")[0][:90]
            lines.append(f"| `{short}` | {r.get('Calls')} | {float(r.get('AverageNs', 0)) / 1e3:.1f} | "
                         f"{float(r.get('MinNs', 0)) / 1e3:.1f} | {float(r.get('MaxNs', 0)) / 1e3:.1f} | "
                         f"{float(r.get('Percentage', 0)):.1f}% |")
    if counters:
        rows = _read_csv(counters[0])
        per = {}
        for r in rows:
            name = r.get("Kernel_Name", "?").split("(")[0]
            cname = r.get("Counter_Name", "?")
            per.setdefault((name, cname), []).append(float(r.get("Counter_Value", 0)))
        lines += ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
        for (name, cname), v in sorted(per.items()):
            lines.append(f"| `{name[:90]}` | {cname} | {len(v)} | {statistics.mean(v):.4g} |")
        if calib_bytes:
            lines += ["", f"Calibration copy bytes: {calib_bytes:.0f}"]
    lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)


def summarize_traffic(fetch_dir: str, write_dir: str, out: str, command: str, calib_bytes: float) -> None:
    """HBM bytes per dispatch from a FETCH_SIZE run and a WRITE_SIZE run of
    the same program, each scaled by what the counter reads for the plain
    device copy of calib_bytes that the program ran (--calibrate-copy)."""
    def load(d, counter):
        f = _newest(d, "*counter_collection.csv")[0]
        by_id = {}
        for r in _read_csv(f):
            if r.get("Counter_Name") == counter:
                by_id[int(r["Dispatch_Id"])] = (r["Kernel_Name"].split("(")[0], float(r["Counter_Value"]))
        return by_id

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    calib_kib = calib_bytes / 1024
    ids = [i for i, (k, v) in write.items() if "copy" in k.lower() and abs(v - calib_kib) < 1e-3 * calib_kib]
    f_scale = calib_kib / statistics.mean(fetch[i][1] for i in ids)
    w_scale = calib_kib / statistics.mean(write[i][1] for i in ids)
    lines = [f"# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE): {os.path.basename(out)}", "",
             f"Command: `{command}`", "",
             f"Calibration: a plain device-to-device copy of {calib_bytes:.0f} bytes reads back as "
             f"FETCH_SIZE {calib_kib / f_scale:.1f} KiB and WRITE_SIZE {calib_kib / w_scale:.1f} KiB, "
             f"so FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f} "
             f"(dispatches {ids}).", "",
             "| kernel | fetched (GB, scaled) | written (GB, scaled) | total (GB) |", "|---|---|---|---|"]
    per = {}
    for i, (k, v) in fetch.items():
        if i in write and "cdma" in k:
            per.setdefault(k, []).append((v * f_scale * 1024, write[i][1] * w_scale * 1024))
    for k, v in sorted(per.items()):
        fb, wb = statistics.mean(a for a, _ in v), statistics.mean(b for _, b in v)
        lines.append(f"| `{k}` | {fb / 1e9:.4f} | {wb / 1e9:.4f} | {(fb + wb) / 1e9:.4f} |")

    def total(*names):
        tot = 0.0
        for name in names:
            v = [a + b for k, vv in per.items() if name in k for a, b in vv]
            if not v:
                return None
            tot += statistics.mean(v)
        return tot

    comp = total("zvc_compress_kernel<4, 0>")
    dec = total("zvc_count_kernel", "zvc_scan_kernel", "zvc_expand_kernel<4, 4>")
    lines += ["", "Machine-readable (read by bench.py; valid only for the kernel sources hashed here):", ""]
    if comp is not None:
        lines.append(f"- hbm_bytes_per_launch_zvc_compress: `{comp:.0f}`")
    if dec is not None:
        lines.append(f"- hbm_bytes_per_launch_zvc_decompress: `{dec:.0f}`")
    lines += [f"- kernel_source_sha256: `{kernel_source_hash()}`", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)


# ----------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


class Timer:
    """Times one call at a time with HIP events on the launch stream.  A short
    device-side spin is queued first so the events time GPU work, not launch
    latency; with cold=True a 1 GiB buffer is read first so nothing of the
    inputs is left in the last-level cache.  Reading it (not writing it)
    leaves clean lines there, so no write-back of the flush lands in the
    timed call."""

    def __init__(self, torch, stream, dev):
        self.torch, self.stream, self.dev = torch, stream, dev
        self._flush = None
        self._sink = None

    def flush(self):
        if self._flush is None:
            self._flush = self.torch.ones(FLUSH_BYTES // 4, dtype=self.torch.int32, device=self.dev)
            self._sink = self.torch.zeros(1, dtype=self.torch.int64, device=self.dev)
        self._sink.add_(self._flush.sum())

    def __call__(self, fn, reps: int, warmup: int = 1, cold: bool = False):
        torch = self.torch
        ts = []
        for r in range(warmup + reps):
            if cold:
                self.flush()
            torch.cuda._sleep(SPIN_CYCLES)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            e1.synchronize()
            if r >= warmup:
                ts.append(e0.elapsed_time(e1) * 1e3)
        return ts


def _row(us_list, in_bytes, alg_bytes):
    us = statistics.median(us_list)
    row = {"us": round(us, 2), "us_min": round(min(us_list), 2),
           "gbs_uncompressed": round(in_bytes / us / 1e3, 1)}
    if alg_bytes is not None:
        row["gbs_algorithmic"] = round(alg_bytes / us / 1e3, 1)
        row["hbm_frac"] = round(alg_bytes / us / 1e3 / PEAK_HBM_GBS, 4)
    return row


def codec_rows(cdma, torch, timer, x, esz, algos, reps, dirs=("c", "d"), cold=False, check=True):
    """Compress and decompress x (a flat int32/int16 device tensor) with each
    codec; returns {f"{algo}_compress": row, f"{algo}_decompress": row, ...}
    with sizes and ratios, after checking each round trip exactly."""
    dev = x.device
    n = x.numel()
    in_bytes = esz * n
    out = {}
    ws = torch.empty(max(256, max(cdma.cdma_workspace_bytes(ALGO_ID[a], esz, n) for a in algos)),
                     dtype=torch.uint8, device=dev)
    sz = torch.zeros(1, dtype=torch.int64, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    rec = torch.empty_like(x)
    for algo in algos:
        a = ALGO_ID[algo]
        dst = torch.empty(max(16, cdma.cdma_max_compressed_bytes(a, esz, n)), dtype=torch.uint8, device=dev)
        tc = timer(lambda: cdma.compress(x, algo, dst=dst, out_bytes=sz, ws=ws), reps, cold=cold)
        size = int(sz.item())
        td = timer(lambda: cdma.decompress(dst, n, esz, algo, src_bytes=sz, out=rec, error=err, ws=ws),
                   reps, cold=cold)
        ok = True
        if check:
            ok = int(err.item()) == 0 and torch.equal(rec, x)
        alg = in_bytes + size  # read the map and write the stream, or the reverse
        out[f"{algo}_compress"] = dict(_row(tc, in_bytes, alg), bytes=size, ratio=round(in_bytes / size, 4),
                                       ok=bool(ok))
        out[f"{algo}_decompress"] = dict(_row(td, in_bytes, alg), ok=bool(ok))
        del dst
    return out


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same buffer
# ----------------------------------------------------------------------------

def cpu_baseline(x_dev, st_sample: int, mt_sample: int):
    """ZVC compress + decompress round trip of the oracle on the first
    elements of the same buffer: single-threaded, and two-phase over window
    ranges on every host core.  Median of 3 runs each."""
    import numpy as np
    import oracle

    threads = os.cpu_count() or 1

    def run(sample, t):
        bits = x_dev[:sample].cpu().numpy().view(np.uint32)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            if t == 1:
                z = oracle.zvc_compress(bits)
                oracle.zvc_decompress(z, bits.size, 4)
            else:
                z = oracle.zvc_compress_mt(bits, t)
                oracle.zvc_decompress_mt(z, bits.size, 4, t)
            times.append(time.perf_counter() - t0)
        return 4 * sample / statistics.median(times) / 1e9, times

    st_gbs, st_t = run(st_sample, 1)
    mt_gbs, mt_t = run(mt_sample, threads)
    return {
        "value": round(mt_gbs, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"ZVC compress + decompress round trip of the first {mt_sample} elements "
                   f"({4 * mt_sample / 2**20:.0f} MiB) of the same 4 GiB buffer on {threads} threads "
                   f"(the oracle's two-phase form over window ranges), median of 3; gcc -O2 C oracle"),
        "seconds": [round(t, 2) for t in mt_t],
        "single_thread": {"value": round(st_gbs, 4), "unit": "GB/s", "cores": 1,
                          "sample": f"first {st_sample} elements ({4 * st_sample / 2**20:.0f} MiB), median of 3",
                          "seconds": [round(t, 2) for t in st_t]},
        "host_cpu": _cpu_model(),
        "host_cpus_visible": threads,
    }


# ----------------------------------------------------------------------------
# layout study: the same maps in three layouts, both codecs
# ----------------------------------------------------------------------------

def layout_study(max_elems: int) -> int:
    """One JSON line per (workload, layout) with both codecs' compressed sizes
    and ratios, computed by the HIP library on the device; the layout change
    itself is input preparation (a torch permute of the NCHW map)."""
    import numpy as np
    import torch
    import sparse_activation_compression_amd as cdma
    from synth import LAYOUTS, WORKLOADS, workload

    dev = torch.device("cuda:0")
    names = [k for k, v in WORKLOADS.items() if v["kind"] in ("clustered", "iid")]
    for name in names:
        x = workload(name, scale_n=max_elems)
        sig = x.view(np.int32 if x.dtype.itemsize == 4 else np.int16)
        xd = torch.from_numpy(sig).to(dev)
        row = {"workload": name, "shape_nchw": list(x.shape), "elements": int(x.size),
               "bytes": int(x.nbytes)}
        for layout, perm in LAYOUTS.items():
            y = xd.permute(*perm).contiguous().view(-1)
            sizes = {}
            for algo in ("zvc", "rle"):
                _, nb = cdma.compress(y, algo)
                torch.cuda.synchronize()
                sizes[algo] = int(nb.item())
            row[layout] = {a: {"bytes": b, "ratio": round(x.nbytes / b, 4)} for a, b in sizes.items()}
            del y
        print(json.dumps(row), flush=True)
        del xd
        torch.cuda.empty_cache()
    return 0


# ----------------------------------------------------------------------------
# the benchmark
# ----------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--zero-frac", type=float, default=0.5)
    ap.add_argument("--reps", type=int, default=10, help="timed calls per row")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sections", default="rows,sweep,configs,pcie",
                    help="row blocks to run after the timed steps: rows, sweep, configs, pcie")
    ap.add_argument("--only-workload", default=None,
                    help="in the configs block, run only workloads whose name contains this")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--layout-study", action="store_true",
                    help="ZVC and RLE ratios of the CNN-like workloads in NCHW, NHWC and CHWN, then exit")
    ap.add_argument("--layout-elems", type=int, default=1 << 25,
                    help="elements per workload in the layout study (the batch is cut to fit)")
    ap.add_argument("--summarize-profile", metavar="DIR")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--out")
    ap.add_argument("--command", default="")
    ap.add_argument("--calib-bytes", type=float)
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.out, args.command, args.calib_bytes or float(1 << 30))
        return 0
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.out, args.command, args.calib_bytes)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by independent chunks, with no communication)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import __graft_entry__
    __graft_entry__.ensure_built()
    import sparse_activation_compression_amd as cdma
    from synth import SWEEP_SEEDS, SWEEP_ZERO_FRACTIONS, WORKLOADS, sweep_bits_device, workload

    if args.layout_study:
        return layout_study(args.layout_elems)

    sections = set(s for s in args.sections.split(",") if s)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream, dev)
    s = args.zero_frac
    seeds = dict(zip(SWEEP_ZERO_FRACTIONS, SWEEP_SEEDS))
    seed = seeds.get(s, 52)
    n = N_ELEMS
    x = sweep_bits_device(n, s, seed, device=dev)
    torch.cuda.synchronize()
    nnz = int(torch.count_nonzero(x).item())
    W = (n + 31) // 32
    in_bytes = 4 * n
    zvc_alg = in_bytes + 4 * W + 4 * nnz  # read the map, write masks and values (or the reverse)

    # ---- the timed steps: ZVC compress -> ZVC decompress, back to back -----
    zcap = cdma.cdma_max_compressed_bytes(0, 4, n)
    zdst = torch.empty(zcap, dtype=torch.uint8, device=dev)
    zsz = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(cdma.cdma_workspace_bytes(a, 4, n) for a in (0, 1, 2)), dtype=torch.uint8, device=dev)
    zout = torch.empty_like(x)
    zerr = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(evs):
        evs[0].record(stream)
        cdma.compress(x, "zvc", dst=zdst, out_bytes=zsz, ws=ws)
        evs[1].record(stream)
        cdma.decompress(zdst, n, 4, "zvc", src_bytes=zsz, out=zout, error=zerr, ws=ws)
        evs[2].record(stream)

    for _ in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    tc = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    td = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    t_gpu = evs[0][0].elapsed_time(evs[-1][2]) * 1e3  # first event to last, device clock (us)
    zsize = int(zsz.item())
    step_ok = zsize == 4 * W + 4 * nnz and int(zerr.item()) == 0 and torch.equal(zout, x)
    ms_per_step = t_total / args.steps * 1e3

    rows = {
        "zvc_compress": dict(_row(tc, in_bytes, zvc_alg), us_mean=round(statistics.mean(tc), 2),
                             kernels="workspace clear + zvc_compress_kernel", bytes=zsize,
                             ratio=round(in_bytes / zsize, 4)),
        "zvc_decompress": dict(_row(td, in_bytes, zvc_alg), us_mean=round(statistics.mean(td), 2),
                               kernels="zvc_count_kernel + zvc_scan_kernel + zvc_expand_kernel"),
    }
    rows["zvc_round_trip"] = {"us": round(statistics.median([a + b for a, b in zip(tc, td)]), 2),
                              "gbs_uncompressed": round(in_bytes / statistics.mean([a + b for a, b in zip(tc, td)])
                                                        / 1e3, 1),
                              "device_ms_per_step": round(t_gpu / 1e3 / args.steps, 3)}

    if args.calibrate_copy:  # a plain copy of known size, for the counter scale factor
        a = torch.empty(1 << 28, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    checks = {"step": bool(step_ok)}

    # ---- the other codecs on the same buffer --------------------------------
    if "rows" in sections:
        r = codec_rows(cdma, torch, timer, x, 4, ("rle", "zvci"), args.reps)
        rows.update(r)
        checks["rows"] = all(v.get("ok", True) for v in r.values())
        # fused producer epilogue: ReLU of pre-activations coded straight into
        # the ZVC stream (plus the dense ReLU output), against a separate ReLU
        # pass followed by the plain compressor.  Pre-activations are the map
        # with -1.0 where it is zero, so ReLU(pre) is the map.
        pre = torch.where(x == 0, torch.tensor(-0x40800000, dtype=torch.int32, device=dev), x).view(torch.float32)
        act = torch.empty_like(pre)
        fdst = torch.empty_like(zdst)
        fsz = torch.zeros(1, dtype=torch.int64, device=dev)
        tf = timer(lambda: cdma.relu_compress(pre, "zvc", act=act, dst=fdst, out_bytes=fsz, ws=ws), args.reps)

        def unfused():
            torch.clamp_min(pre, 0.0, out=act)
            cdma.compress(act.view(torch.int32), "zvc", dst=zdst, out_bytes=zsz, ws=ws)
        tu = timer(unfused, args.reps)
        fsize = int(fsz.item())
        fused_ok = fsize == zsize and torch.equal(fdst[:fsize], zdst[:fsize]) and torch.equal(act.view(torch.int32), x)
        f_alg = 8 * n + 4 * W + 4 * nnz  # read x, write ReLU(x) densely, write the stream
        rows["relu_zvc_compress"] = dict(_row(tf, in_bytes, f_alg), unfused_us=round(statistics.median(tu), 1),
                                         speedup_vs_unfused=round(statistics.median(tu) / statistics.median(tf), 3),
                                         unfused="torch.clamp_min then zvc compress", ok=bool(fused_ok))
        checks["relu"] = bool(fused_ok)
        del pre, act, fdst

    # ---- sparsity sweep of the 4 GiB buffer ---------------------------------
    sweep = {}
    if "sweep" in sections:
        y = torch.empty_like(x)
        for zf in SWEEP_ZERO_FRACTIONS:
            sweep_bits_device(n, zf, seeds[zf], device=dev, out=y)
            r = codec_rows(cdma, torch, timer, y, 4, ("zvc", "rle"), args.reps, cold=True)
            sweep[f"s{zf}"] = r
            checks[f"sweep_s{zf}"] = all(v.get("ok", True) for v in r.values())
        del y

    # ---- the named CNN-like workloads, warm and cold ------------------------
    configs = {}
    if "configs" in sections:
        torch.cuda.empty_cache()
        names = [k for k, v in WORKLOADS.items() if v["kind"] != "sweep"]
        if args.only_workload:
            names = [k for k in names if args.only_workload in k]
        for name in names:
            host = workload(name)
            esz = host.dtype.itemsize
            xd = torch.from_numpy(host.reshape(-1).view(np.int32 if esz == 4 else np.int16)).to(dev)
            del host
            warm = codec_rows(cdma, torch, timer, xd, esz, ("zvc", "rle"), args.reps)
            cold = codec_rows(cdma, torch, timer, xd, esz, ("zvc", "rle"), max(3, args.reps // 2), cold=True)
            configs[name] = {"elements": xd.numel(), "element_bytes": esz, "warm": warm, "cold": cold}
            checks[name] = all(v.get("ok", True) for v in list(warm.values()) + list(cold.values()))
            del xd
            torch.cuda.empty_cache()
        # the VGG-16 stack as one workload: bytes of all five maps over the sum of their times
        vgg = [k for k in configs if k.startswith("vgg16_")]
        if len(vgg) == 5:
            stack = {}
            for temp in ("warm", "cold"):
                for key in ("zvc_compress", "zvc_decompress", "rle_compress", "rle_decompress"):
                    us = sum(configs[k][temp][key]["us"] for k in vgg)
                    inb = sum(4 * configs[k]["elements"] for k in vgg)
                    alg = sum(4 * configs[k]["elements"] + configs[k][temp][key.split("_")[0] + "_compress"]["bytes"]
                              for k in vgg)
                    stack.setdefault(temp, {})[key] = _row([us], inb, alg)
            configs["vgg16_stack_fp32"] = stack

    # ---- PCIe-bound stages: compressed offload and prefetch ----------------
    pcie = {}
    if "pcie" in sections:
        host_img = torch.empty(zcap, dtype=torch.uint8, pin_memory=True)
        scratch = torch.empty(cdma.cdma_offload_scratch_bytes(0, 4, CHUNK, SLOTS), dtype=torch.uint8, device=dev)
        cstream = torch.cuda.Stream(device=dev)
        pstream = torch.cuda.Stream(device=dev)
        off_t, totals, sizes = [], [], []
        for r in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            job = cdma.offload(x, host_img, CHUNK, "zvc", SLOTS, scratch=scratch, compute_stream=cstream,
                               copy_stream=pstream)
            rc, total, sizes = job.wait()
            off_t.append((time.perf_counter() - t0) * 1e6)
            totals.append(total)
            if rc != 0:
                raise RuntimeError(f"offload failed: {rc}")
        expect = sum(4 * ((min(CHUNK, n - lo) + 31) // 32) + 4 * int(torch.count_nonzero(x[lo:lo + CHUNK]).item())
                     for lo in range(0, n, CHUNK))
        off_ok = all(t == expect for t in totals)
        # first chunk's compression: the only part with no copy running beside it
        cdst = torch.empty(cdma.cdma_max_compressed_bytes(0, 4, CHUNK), dtype=torch.uint8, device=dev)
        csz = torch.zeros(1, dtype=torch.int64, device=dev)
        cws = torch.empty(cdma.cdma_workspace_bytes(0, 4, CHUNK), dtype=torch.uint8, device=dev)
        first = timer(lambda: cdma.compress(x[:CHUNK], "zvc", dst=cdst, out_bytes=csz, ws=cws), 5)
        off_us = statistics.median(off_t)
        checks["offload"] = bool(off_ok)
        # prefetch of the offloaded image back into device memory
        pout = torch.empty_like(x)
        perr = torch.zeros(1, dtype=torch.int32, device=dev)
        pscratch = torch.empty(cdma.cdma_prefetch_scratch_bytes(0, 4, n, CHUNK, SLOTS), dtype=torch.uint8,
                               device=dev)
        pre_t = []
        for r in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            job = cdma.prefetch(host_img, sizes, n, 4, CHUNK, "zvc", SLOTS, out=pout, error=perr,
                                scratch=pscratch, compute_stream=cstream, copy_stream=pstream)
            rc, _, _ = job.wait()
            pre_t.append((time.perf_counter() - t0) * 1e6)
            if rc != 0:
                raise RuntimeError(f"prefetch failed: {rc}")
        torch.cuda.synchronize()
        pre_ok = int(perr.item()) == 0 and torch.equal(pout, x)
        # raw copies of the dense buffer for comparison (the host image is
        # free to overwrite once the prefetch has been checked)
        raw = []
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            host_img[: in_bytes].copy_(x.view(torch.uint8), non_blocking=True)
            torch.cuda.synchronize()
            raw.append(time.perf_counter() - t0)
        raw_gbs = in_bytes / min(raw) / 1e9
        raw_h2d = []
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            pout.view(torch.uint8).copy_(host_img[: in_bytes], non_blocking=True)
            torch.cuda.synchronize()
            raw_h2d.append(time.perf_counter() - t0)
        raw_h2d_gbs = in_bytes / min(raw_h2d) / 1e9
        pcie["offload"] = {"us": round(off_us, 1), "gbs_uncompressed": round(in_bytes / off_us / 1e3, 2),
                           "raw_pcie_d2h_gbs": round(raw_gbs, 2), "host_bytes": totals[0],
                           "speedup_vs_raw_copy": round((in_bytes / raw_gbs / 1e3) / off_us, 3),
                           "compression_ratio": round(in_bytes / totals[0], 4),
                           "first_chunk_compress_us": round(statistics.median(first), 1),
                           "chunk_elems": CHUNK, "slots": SLOTS, "ok": bool(off_ok)}
        pre_us = statistics.median(pre_t)
        pcie["prefetch"] = {"us": round(pre_us, 1), "gbs_uncompressed": round(in_bytes / pre_us / 1e3, 2),
                            "raw_pcie_h2d_gbs": round(raw_h2d_gbs, 2), "host_bytes": sum(sizes),
                            "speedup_vs_raw_copy": round((in_bytes / raw_h2d_gbs / 1e3) / pre_us, 3),
                            "ok": bool(pre_ok)}
        checks["prefetch"] = bool(pre_ok)
        del host_img, scratch, pout, pscratch, cdst, cws

    # what PyTorch's own streaming kernels reach on the same buffer: context
    # for the HBM fractions (mixed read/write traffic peaks well below the
    # 8 TB/s interface figure on this part)
    def moved(fn, nbytes):
        return round(nbytes / statistics.median(timer(fn, 3)) / 1e3, 1)
    hbm_context = {"torch_copy_gbs": moved(lambda: zout.copy_(x), 8 * n),
                   "torch_fill_gbs": moved(lambda: zout.fill_(7), 4 * n),
                   "torch_amax_gbs": moved(lambda: torch.amax(x), 4 * n),
                   "note": "read+write bytes per second of torch's copy_, fill_ and amax on the same buffer"}

    # roofline of the longer of the step's two calls, from the step's events
    c_mean, d_mean = statistics.mean(tc), statistics.mean(td)
    dom, dom_us = ("zvc_decompress", d_mean) if d_mean >= c_mean else ("zvc_compress", c_mean)
    traffic = stored_traffic().get(dom)
    roofline = {
        "kernel": dom + (" (zvc_count_kernel + zvc_scan_kernel + zvc_expand_kernel)" if dom == "zvc_decompress"
                         else " (workspace clear + zvc_compress_kernel)"),
        "bound": "hbm",
        "achieved": round(zvc_alg / dom_us / 1e3, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(zvc_alg / dom_us / 1e3 / PEAK_HBM_GBS, 4),
        "traffic": round(traffic) if traffic else None,
        "algorithmic_bytes_per_launch": zvc_alg,
        "avg_launch_us": round(dom_us, 1),
        "other": {"zvc_compress" if dom == "zvc_decompress" else "zvc_decompress":
                  {"avg_launch_us": round(c_mean if dom == "zvc_decompress" else d_mean, 1),
                   "frac": round(zvc_alg / (c_mean if dom == "zvc_decompress" else d_mean) / 1e3 / PEAK_HBM_GBS,
                                 4)}},
    }

    ok = all(checks.values())
    result = {
        "metric": "ZVC compress/decompress GB/s (uncompressed) and % HBM peak; compression ratio",
        "value": round(in_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": f"sweep_fp32_4GiB_s{s}",
            "elements": n,
            "element": "fp32 bit patterns",
            "zero_fraction": s,
            "generator": "counter-based hash, seed %d, forced all-zero/all-dense windows" % seed,
            "step": ["zvc_compress", "zvc_decompress"],
            "value": "uncompressed bytes per step (one compress + one decompress) / step time",
            "parallelism": "single GPU",
        },
        "compression_ratio": {"zvc": round(in_bytes / zsize, 4)},
        "rows": rows,
        "roofline": roofline,
        "sweep": sweep,
        "configs": configs,
        "pcie": pcie,
        "hbm_context": hbm_context,
        "checks": checks,
        "ok": bool(ok),
    }
    if "rle_compress" in rows:
        result["compression_ratio"]["rle"] = rows["rle_compress"]["ratio"]
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(x, CPU_ST_SAMPLE, CPU_MT_SAMPLE)
    print(json.dumps(result), flush=True)
    del x, zdst, zsz, ws, zout, zerr
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
