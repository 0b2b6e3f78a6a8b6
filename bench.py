"""Benchmark of the MXFP8 master-weight writeback on one MI355X.

One step is the whole path over a 16384x6144 master weight (BF16 by default) held as four
contiguous fragments whose boundaries fall inside 32-value blocks (cuts at N/4+17, N/2+17,
3N/4+17), as four ranks would hold it: zero-fill of one packed amax buffer per fragment,
partial amax of every fragment, MAX-combine of the four buffers, then E8M0 scales (one call
over the whole weight) and the in-place partial cast of every fragment to E4M3 row-wise and
column-wise data, the four calls of the pages' design; ``--fused`` derives the scales inside
the cast instead (mxfp8_scales_and_cast, one pass per fragment).  Inputs are resident in HBM
before timing.  Steps walk over several distinct weights
(buffer sets, >= 1.2 GB in all) like a writeback over a model: step i runs the amax side on
weight i and the cast of weight i - 1, so no kernel reads an input another kernel has just
left in the 256 MB Infinity Cache.

Prints one JSON line: ``value`` is the step's algorithmic HBM bytes / wall time (GB/s);
``roofline`` is for the dominant kernel (the cast, or with ``--fused`` the fused one), from
timing-only HIP events (no system-scope fence) that the runtime stamps at the cast kernel's
start and end on every fourth timed step (and, for comparison, events recorded on the launch
stream around the call on the steps halfway between);
``kernels`` is the per-call table (partial amax, partial cast and the fused scales + cast;
full input and the quarter fragment at offset 17, BF16 and FP32; at 16384x6144 also the quarter
fragment in one rank's own buffers, ``*_partial_own``: input and fragment-sized outputs in
allocations of their own); ``cpu_baseline`` times
the oracle on the host over a band-aligned sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CAST_SAMPLE = 4  # timed steps per cast-duration sample
CPU_LEG_SECONDS = 10.0  # CPU work of the oracle leg, one thread
METRIC = "µs/call and achieved HBM GB/s (% of peak) for partial amax + cast"
KERNEL_SRC = os.path.join(ROOT, "mxfp8_block_scaled_partial_amd", "csrc", "kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first: an idle GPU takes a few tens of ms of work to "
                         "reach its steady clocks")
    ap.add_argument("--dtype", choices=["bf16", "fp32"], default="bf16")
    ap.add_argument("--min-footprint-gb", type=float, default=1.2,
                    help="distinct input/output sets rotate until this many GB are in use")
    ap.add_argument("--kernel-table", dest="kernel_table", action="store_true", default=True)
    ap.add_argument("--no-kernel-table", dest="kernel_table", action="store_false")
    ap.add_argument("--table-shapes", default="16384x6144,4096x4096,1024x1024,160x96",
                    help="matrices of the per-call table, comma-separated ROWSxCOLS")
    ap.add_argument("--table-runs", default="full,partial,partial_own,full_rowonly",
                    help="runs of the per-call table: full, partial (quarter at offset 17), "
                         "partial_own (the quarter in a rank's own buffers, 16384x6144 only), "
                         "full_rowonly (16384x6144 only)")
    ap.add_argument("--kernel-calls", type=int, default=140,
                    help="graph replays (10 calls each) per kernel-table entry (7 rounds of 20)")
    ap.add_argument("--cpu-baseline", dest="cpu", action="store_true", default=True)
    ap.add_argument("--no-cpu-baseline", dest="cpu", action="store_false")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="rows of the weight (a band-aligned sample) the oracle processes")
    ap.add_argument("--fused", dest="fused", action="store_true", default=False,
                    help="derive the scales inside the cast (one call) instead of the scales "
                         "call followed by the cast call")
    ap.add_argument("--single-pass", dest="single_pass", action="store_true", default=True,
                    help="also time the writeback that quantizes whole bands in one pass")
    ap.add_argument("--no-single-pass", dest="single_pass", action="store_false")
    ap.add_argument("--layer-batch", dest="layer_batch", action="store_true", default=True,
                    help="also time the transformer-layer batch (4 weights, 8 fragments): the "
                         "whole writeback with one shared packed buffer and with 8 buffers + "
                         "combine, and one rank's fragment")
    ap.add_argument("--no-layer-batch", dest="layer_batch", action="store_false")
    ap.add_argument("--ablation", action="store_true", default=False,
                    help="also time the runtime-guard ablation library (build.py --ablation) "
                         "against the product's compile-time specialization: amax and cast, "
                         "row-only and bidirectional, full input and quarter fragment, BF16 and "
                         "FP32 at 16384x6144")
    ap.add_argument("--copy-probe", dest="copy_probe", action="store_true", default=True,
                    help="also time a plain device copy (the achievable read + write ceiling, "
                         "and the counter calibration kernel); on by default")
    ap.add_argument("--no-copy-probe", dest="copy_probe", action="store_false")
    ap.add_argument("--counter-pass", metavar="MANIFEST", default=None,
                    help="run for a rocprofv3 counter pass: every launch of the step "
                         "(--warmup + --steps steps) and of the per-call table (--counter-calls "
                         "eager calls per entry) with no timing, plus the copy probe; writes "
                         "the launch order (labels, calls, algorithmic bytes) to MANIFEST")
    ap.add_argument("--counter-calls", type=int, default=4,
                    help="eager calls per table entry in --counter-pass")
    ap.add_argument("--summarize-counters", metavar="RUN", default=None,
                    help="(no GPU) summarize the rocprofv3 passes of --counter-pass runs as "
                         "markdown: RUN_fetch/ (FETCH_SIZE) and RUN_write/ (WRITE_SIZE), "
                         "optionally RUN_wrreq/ (TCC_EA0_WRREQ_sum, TCC_EA0_WRREQ_64B_sum), "
                         "each with its manifest RUN_<pass>.json; to --out")
    ap.add_argument("--summarize-trace", metavar="RUN", default=None,
                    help="(no GPU) summarize the rocprofv3 --kernel-trace run of a "
                         "--counter-pass workload (RUN_trace/ and RUN_trace.json) as markdown, "
                         "to --out")
    ap.add_argument("--summarize-stats", metavar="DIR", default=None,
                    help="(no GPU) summarize a rocprofv3 --kernel-trace --stats run of the "
                         "benchmark (DIR, with its JSON line in DIR.log) as markdown, to --out")
    ap.add_argument("--out", default=None)
    return ap.parse_args()


def hip_runtime_path() -> str:
    """Path of the HIP runtime library this process has loaded (torch maps its own at import,
    and the library resolves to it), read from /proc/self/maps, so the benchmark talks to the
    same runtime instance whatever its file name or soname."""
    import torch  # noqa: F401

    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1] if len(line.split()) >= 6 else ""
            if os.path.basename(path).startswith("libamdhip64.so"):
                return path
    raise RuntimeError("the HIP runtime (libamdhip64) is not loaded in this process")


def hip_event_flag(name: str, fallback: int) -> int:
    """Value of a hipEvent* flag macro from the HIP headers of the ROCm install, if present
    (the documented value otherwise)."""
    for root in (os.environ.get("ROCM_PATH"), "/opt/rocm"):
        hdr = os.path.join(root or "", "include", "hip", "hip_runtime_api.h")
        if root and os.path.exists(hdr):
            m = re.search(r"#define\s+" + name + r"\s+(0x[0-9a-fA-F]+|\d+)", open(hdr).read())
            if m:
                return int(m.group(1), 0)
    return fallback


class TimingEvent:
    """A HIP event used for timing only, created with hipEventDisableSystemFence.

    Recording a default event makes the command processor write back and invalidate the
    caches at system scope, which lengthens the stream by a few µs at every marker; without
    that fence the marker only takes its timestamp, so the time between two markers is close
    to the kernel durations a profiler reports.  torch.cuda.Event cannot set the flag, so this
    calls the HIP runtime torch has already loaded (found in the process's mappings, so the
    same instance) and records on torch's current stream, where the library launches.
    """
    _hip = None
    _flag = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            cls._flag = hip_event_flag("hipEventDisableSystemFence", 0x20000000)
            h = ctypes.CDLL(hip_runtime_path())
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for f in (h.hipEventCreateWithFlags, h.hipEventRecord, h.hipEventElapsedTime,
                      h.hipEventDestroy):
                f.restype = ctypes.c_int
            cls._hip = h
        return cls._hip

    @staticmethod
    def _ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def __init__(self):
        self.ev = ctypes.c_void_p()
        self._ok(self._rt().hipEventCreateWithFlags(ctypes.byref(self.ev), self._flag),
                 "hipEventCreateWithFlags")

    def record(self):
        import torch
        self._ok(self._rt().hipEventRecord(self.ev, torch.cuda.current_stream().cuda_stream),
                 "hipEventRecord")

    def elapsed_time(self, end: "TimingEvent") -> float:
        """Milliseconds from this event to ``end``; both must have completed."""
        ms = ctypes.c_float()
        self._ok(self._rt().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev),
                 "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        try:
            if self.ev and self._hip is not None:
                self._hip.hipEventDestroy(self.ev)
        except Exception:  # interpreter shutdown
            pass


def kernel_sha() -> str:
    """Hash of the kernel source without its comments and blank space, so that a counter
    summary stays valid across comment edits; the build embeds the same hash in the library
    (mxfp8_build_id)."""
    from mxfp8_block_scaled_partial_amd import build as hip_build

    return hip_build.kernel_source_hash(KERNEL_SRC)


def library_matches_source() -> tuple:
    """(build id of the loaded library, whether it was built from the current kernel
    source): a library left over from another source would measure other kernels."""
    from mxfp8_block_scaled_partial_amd import binding as B

    bid = B.mxfp8_build_id()
    return bid, bid == kernel_sha()


def counter_blocks():
    """The JSON blocks of the committed rocprofv3 counter summaries (profiles/*_counters.md)."""
    out = []
    for f in sorted(glob.glob(os.path.join(PROFILES, "*_counters.md"))):
        m = re.search(r"```json\n(.*?)\n```", open(f).read(), re.S)
        if m:
            out.append(json.loads(m.group(1)))
    return out


def traffic_from_counters(dtype: str, fused: bool, label: str, library_id: str | None = None):
    """Calibrated HBM bytes per launch of the step stage ``label`` (e.g. ``step_cast``) from the
    committed counter summary of the same step (dtype, fused), if it was taken on the current
    kernel source and (``library_id``: the running library's build id) the running library was
    built from it; None otherwise."""
    sha = kernel_sha()
    if library_id is not None and library_id != sha:
        return None
    for d in counter_blocks():
        if (d.get("dtype"), d.get("fused")) == (dtype, fused) and \
                d.get("kernel_source_sha256_16") == sha and label in d.get("hbm_bytes_per_launch", {}):
            return d["hbm_bytes_per_launch"][label]
    return None


def _counter_dispatches(d):
    """The dispatches of one rocprofv3 --pmc run (output directory ``d``), in dispatch order:
    kernel name, grid, workgroup and the summed value of each counter."""
    import csv

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {files}")
    disp = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            e = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                        "grid": int(r["Grid_Size"]),
                                                        "wg": int(r["Workgroup_Size"]), "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def _short_kernel(name: str) -> str:
    m = re.search(r"(\w+_kernel)<([^()]*)>", name)
    if not m:
        return name.split("(")[0][-60:]
    a = [x.strip() for x in m.group(2).split(",")]
    t = {"unsigned short": "bf16", "unsigned int": "fp32"}.get(a[0], a[0])
    rest = ", ".join(a[1:])
    return f"{m.group(1)}<{t}{', ' + rest if rest else ''}>"


MARKER = "FillFunctor<short>"  # LaunchLog's marker kernel


def _attribute(man, disp):
    """Splits a run's dispatches at LaunchLog's markers into the manifest's items: each item's
    library dispatches (namespace mxfp8), in order, and the copy probe's copies.  Checks the
    counts."""
    spans = []
    for i, d in enumerate(disp):
        if MARKER in d["name"]:
            spans.append([])
        elif spans:
            spans[-1].append(i)
    spans = spans[1:]  # the first fill is the marker tensor's zero-fill, before any item
    items = man["items"]
    if len(spans) != len(items):
        raise SystemExit(f"{len(spans)} marked spans, {len(items)} manifest items")
    runs, probe = [], None
    for it, sp in zip(items, spans):
        if it.get("aux"):
            runs.append([])
            continue
        if it["label"] == "copy_probe":
            # the probe's copies come first, back to back (later ones set up the next item)
            n = man["copy_probe"]["launches"]
            probe = [i for i in sp if "copyBuffer" in disp[i]["name"]][:n]
            if len(probe) != n or probe[-1] - probe[0] != n - 1 or \
                    len({(disp[i]["grid"], disp[i].get("wg")) for i in probe}) != 1:
                raise SystemExit(f"copy probe: expected {n} consecutive copies of one shape")
            runs.append([])
            continue
        lib = [i for i in sp if "mxfp8::" in disp[i]["name"]]
        if not lib or len(lib) % it["calls"]:
            raise SystemExit(f"{it['label']}: {len(lib)} launches for {it['calls']} calls")
        runs.append(lib)
    return runs, probe


COUNTER_PASSES = (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"),
                  ("wrreq", "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum"))


ITEM_NOTES = (
    "Items: `step_*` are the stages of the 4-fragment step; the others are the per-call "
    "table's entries at 16384x6144, or at the matrix their name starts with (`full`, "
    "`partial`: the quarter fragment at offset 17, "
    "`partial_own`: the quarter in a rank's own input and fragment-sized output allocations, "
    "`full_rowonly`: column-wise outputs absent), each as eager calls rotating over its buffer "
    "sets, the layer batch's stages (`layer_k_buffers_*`: 8 packed buffers and a K = 8 combine, "
    "`layer_shared_buffer_*`: one shared buffer) and one rank's fragment of it (`rank_*`: "
    "fragment 2, in place and into fragment-sized outputs), and with --ablation the runtime-guard "
    "ablation's calls (`abl_compile_time_*`: the product library, `abl_runtime_guard_*`: the "
    "ablation library built by `build.py --ablation`).")


def _load_runs(run, kinds):
    """The manifests of a counter or trace run's passes, checked to hold the same launches."""
    mans = {k: json.load(open(f"{run}_{k}.json")) for k in kinds}
    man = mans[kinds[0]]
    for k in kinds:
        if [(i["label"], i["calls"]) for i in mans[k]["items"]] != \
                [(i["label"], i["calls"]) for i in man["items"]] or \
                mans[k]["kernel_source_sha256_16"] != man["kernel_source_sha256_16"]:
            raise SystemExit(f"the {k} pass ran other launches or another kernel source")
    return man


def _by_label(man):
    """Item indices by label, in first-seen order (the copy probe left out)."""
    seen = {}
    for k, it in enumerate(man["items"]):
        if it["label"] != "copy_probe" and not it.get("aux"):
            seen.setdefault(it["label"], []).append(k)
    return seen


def _per_call(vals, calls):
    """Median over the calls of the sum over each call's launches, and launches per call."""
    lpc = len(vals) // calls
    return statistics.median(sum(vals[j * lpc:(j + 1) * lpc]) for j in range(calls)), lpc


def _kernels(disp, idx):
    names = []
    for i in idx:
        n = _short_kernel(disp[i]["name"])
        if n not in names:
            names.append(n)
    return ", ".join(f"`{n}`" for n in names)


def _commands(man, run, kinds, what):
    argv = list(man["argv"])
    j = argv.index("--counter-pass")
    del argv[j:j + 2]
    name = os.path.basename(run)
    out = []
    for k, ctr in what:
        if k not in kinds:
            continue
        prof = (f"timeout -s KILL 600 rocprofv3 --pmc {ctr}" if ctr else
                "timeout -k 10 600 rocprofv3 --kernel-trace --stats")
        out.append(f"cd /tmp && export TMPDIR=/tmp && {prof} --output-format csv -d "
                   f"$R/gpurun_out/cnt/{name}_{k} -o p -- python -u $R/bench.py {' '.join(argv)} "
                   f"--counter-pass $R/gpurun_out/cnt/{name}_{k}.json")
    return out, name


def _workload(man):
    """What a --counter-pass run covered, from its manifest."""
    argv = man["argv"]
    w = (f"16384x6144 {man['dtype']} step, 4 fragments, bidirectional, "
         + ("fused scales + cast" if man["fused"] else "scales then cast"))
    extra = [what for flag, on, what in (
        ("--no-kernel-table", False, "the per-call table"),
        ("--no-layer-batch", False, "the layer batch"),
        ("--ablation", True, "the runtime-guard ablation")) if (flag in argv) == on]
    return w + ("; " + ", ".join(extra) if extra else "")


def _write(args, md):
    text = "\n".join(md)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        print(text)


def summarize_counters(args):
    """Markdown summary of the counter passes of one --counter-pass workload (``RUN_fetch``,
    ``RUN_write`` and optionally ``RUN_wrreq``, each a rocprofv3 output directory next to the
    manifest its run wrote): calibrated HBM bytes per call of every item against its
    algorithmic bytes, and the JSON block ``traffic_from_counters`` reads."""
    run = args.summarize_counters
    kinds = [k for k, _ in COUNTER_PASSES if os.path.isdir(f"{run}_{k}")]
    if "fetch" not in kinds or "write" not in kinds:
        raise SystemExit(f"need {run}_fetch/ and {run}_write/")
    man = _load_runs(run, kinds)
    passes = {k: _counter_dispatches(f"{run}_{k}") for k in kinds}
    att = {k: _attribute(man, v) for k, v in passes.items()}

    nb_kib = man["copy_probe"]["read_bytes"] / 1024
    f_probe = statistics.median(passes["fetch"][i]["c"]["FETCH_SIZE"] for i in att["fetch"][1])
    w_probe = statistics.median(passes["write"][i]["c"]["WRITE_SIZE"] for i in att["write"][1])
    ff, wf = nb_kib / f_probe, (man["copy_probe"]["write_bytes"] / 1024) / w_probe

    rows, blob = [], {}
    for label, ks in _by_label(man).items():
        it = man["items"][ks[0]]

        def med(kind, counter):
            return statistics.median(
                _per_call([passes[kind][i]["c"][counter] for i in att[kind][0][k]],
                          it["calls"])[0] for k in ks)
        fk, wk = med("fetch", "FETCH_SIZE"), med("write", "WRITE_SIZE")
        lpc = len(att["fetch"][0][ks[0]]) // it["calls"]
        kname = _kernels(passes["fetch"], att["fetch"][0][ks[0]])
        rd, wr = fk * 1024 * ff, wk * 1024 * wf
        w64 = None
        if "wrreq" in passes:
            tot = med("wrreq", "TCC_EA0_WRREQ_sum")
            w64 = med("wrreq", "TCC_EA0_WRREQ_64B_sum") / tot if tot else float("nan")
        rows.append((label, kname, lpc, len(ks) * it["calls"], fk, wk, rd, wr, it["alg_bytes"],
                     w64))
        blob[label] = int(round((rd + wr) / lpc))

    has_w = "wrreq" in passes
    hdr = ("| item | kernels | launches per call | calls | FETCH_SIZE KiB per call | "
           "WRITE_SIZE KiB per call | HBM read MB | HBM write MB | total MB | algorithmic MB | "
           "total / algorithmic |" + (" 64-byte share of write requests |" if has_w else ""))
    lines = [hdr, "|" + "---|" * (hdr.count("|") - 1)]
    for label, kname, lpc, n, fk, wk, rd, wr, alg, w64 in rows:
        lines.append(f"| {label} | {kname} | {lpc} | {n} | {fk:.0f} | {wk:.0f} | "
                     f"{rd / 1e6:.2f} | {wr / 1e6:.2f} | {(rd + wr) / 1e6:.2f} | {alg / 1e6:.2f} | "
                     f"{(rd + wr) / alg:.4f} |" + (f" {w64:.4f} |" if has_w else ""))
    workload = _workload(man)
    block = {"workload": workload, "dtype": man["dtype"], "fused": man["fused"],
             "kernel_source_sha256_16": man["kernel_source_sha256_16"],
             "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
             "hbm_bytes_per_launch": blob}
    cmds, name = _commands(man, run, kinds, COUNTER_PASSES)
    md = [f"# HBM traffic per call: rocprofv3 counters, {workload}", "",
          "One MI355X (gfx950), ROCm 7.2.  `bench.py --counter-pass` runs every launch untimed "
          "in a fixed order, a marker kernel before each item, and writes that order to a "
          "manifest; each counter set is a rocprofv3 run of its own ($R is the repository "
          "root):", "", "```", *cmds, "```", "",
          f"This summary is `python bench.py --summarize-counters gpurun_out/cnt/{name} --out "
          f"<this file>`, which splits each run's dispatches at the markers into the manifest's "
          "items and checks the counts.  " + ITEM_NOTES, "",
          f"Calibration: the copy probe (torch `copy_` of 256 MiB, `__amd_rocclr_copyBuffer`) "
          f"reads {f_probe:.0f} KiB of FETCH_SIZE and {w_probe:.0f} KiB of WRITE_SIZE per launch "
          f"for {nb_kib:.0f} KiB read and written: fetch factor {ff:.4f}, write factor {wf:.4f}.",
          "",
          "Per call: the median over the item's calls of the sum over the call's launches.  "
          "Algorithmic bytes follow `mxfp8_block_scaled_partial_amd/bytes_model.py` (the input "
          "once, touched amax entries or scale bytes once, one E4M3 byte per element and "
          "direction).  A ratio near 1.00 means no re-reads and no staging traffic." +
          (" The last column is the share of HBM write requests (TCC_EA0_WRREQ) that are whole "
           "64-byte requests." if has_w else ""), "", *lines, "",
          "`bench.py` reads `roofline.traffic` from this block while the kernel source hash "
          "matches:", "", "```json", json.dumps(block, indent=1), "```", ""]
    _write(args, md)


def _trace_dispatches(d):
    """The dispatches of one rocprofv3 --kernel-trace run (output directory ``d``), in
    dispatch order: kernel name, grid and duration (µs)."""
    import csv

    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_trace.csv under {d}, found {files}")
    disp = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            disp[int(r["Dispatch_Id"])] = {
                "name": r["Kernel_Name"], "grid": int(r["Grid_Size_X"]),
                "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3}
    return [disp[k] for k in sorted(disp)]


def summarize_trace(args):
    """Markdown summary of the kernel trace of one --counter-pass workload (``RUN_trace``, a
    rocprofv3 --kernel-trace output directory next to its manifest): kernel-only µs per call
    of every item, and its algorithmic GB/s and fraction of the 8 TB/s peak."""
    run = args.summarize_trace
    man = _load_runs(run, ["trace"])
    disp = _trace_dispatches(f"{run}_trace")
    runs, probe = _attribute(man, disp)
    lines = ["| item | kernels | launches per call | calls | µs per call (median) | min | max | "
             "algorithmic MB | GB/s | fraction of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|---|"]
    for label, ks in _by_label(man).items():
        it = man["items"][ks[0]]
        per = []
        for k in ks:
            v = [disp[i]["us"] for i in runs[k]]
            lpc = len(v) // it["calls"]
            per += [sum(v[j * lpc:(j + 1) * lpc]) for j in range(it["calls"])]
        us = statistics.median(per)
        gbs = it["alg_bytes"] / (us * 1e-6) / 1e9
        lines.append(f"| {label} | {_kernels(disp, runs[ks[0]])} | {lpc} | {len(per)} | "
                     f"{us:.2f} | {min(per):.2f} | {max(per):.2f} | {it['alg_bytes'] / 1e6:.2f} | "
                     f"{gbs:.1f} | {gbs / HBM_PEAK_GBS:.4f} |")
    cp = statistics.median(disp[i]["us"] for i in probe)
    cmds, name = _commands(man, run, ["trace"], (("trace", None),))
    workload = _workload(man)
    md = [f"# Kernel durations per call: rocprofv3 kernel trace, {workload}", "",
          "One MI355X (gfx950), ROCm 7.2.  `bench.py --counter-pass` runs every launch untimed "
          "in a fixed order, a marker kernel before each item, and writes that order to a "
          "manifest ($R is the repository root):", "", "```", *cmds, "```", "",
          f"This summary is `python bench.py --summarize-trace gpurun_out/cnt/{name} --out "
          "<this file>`, which splits the traced dispatches at the markers into the manifest's "
          "items and checks the counts.  " + ITEM_NOTES, "",
          "Per call: the sum of the call's launch durations (kernel only, from the trace's "
          "timestamps; no dispatch gap); median, min and max over the item's calls.  The calls "
          "run eagerly, one item after another with a synchronization between items, so these "
          "are the kernels' own times, without the per-call overhead that graph replays of the "
          "per-call table include.  Algorithmic bytes follow "
          "`mxfp8_block_scaled_partial_amd/bytes_model.py`.", "", *lines, "",
          f"Copy probe (256 MiB device copy, read + write), median of {len(probe)} launches: "
          f"{cp:.2f} µs, {2 * COPY_PROBE_BYTES / (cp * 1e-6) / 1e9:.1f} GB/s.", "",
          f"Kernel source: `kernels.hip` sha256 prefix `{man['kernel_source_sha256_16']}`.", ""]
    _write(args, md)


STATS_NAMES = {"FillFunctor<c10::BFloat16>": "torch fill, bf16 (zero-fill of the packed amax buffers)",
               "FillFunctor<float>": "torch fill, fp32 (zero-fill of the packed amax buffers)",
               "FillFunctor<unsigned char>": "torch fill, u8 (buffer set-up)",
               "FillFunctor<long>": "torch fill, i64 (set-up)",
               "__amd_rocclr_copyBuffer": "__amd_rocclr_copyBuffer (device copy: the 256 MiB copy "
                                          "probe and the input-set clones)"}


def summarize_stats(args):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of the benchmark: the kernel
    durations of ``DIR/*_kernel_stats.csv``, the same run's JSON line (``DIR.log``) and the
    dominant kernel's kernel-only fraction of peak."""
    import csv

    d = args.summarize_stats.rstrip("/")
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_stats.csv under {d}, found {files}")
    rows = list(csv.DictReader(open(files[0])))
    b = json.loads([ln for ln in open(d + ".log") if ln.startswith("{")][-1])
    fused = "fused" in b["roofline"]["kernel"]
    t = "unsigned short" if b["dtype"] == "bf16" else "unsigned int"
    pattern = f"cast_vec_kernel<{t}, true, false, {'true' if fused else 'false'}"
    dom = [r for r in rows if pattern in r["Name"]]
    if len(dom) != 1:
        raise SystemExit(f"no single {pattern} row in {files[0]}")
    avg = float(dom[0]["AverageNs"]) / 1e3
    alg = b["roofline"]["alg_bytes_per_launch"]
    argv = ([] if b["dtype"] == "bf16" else ["--dtype", b["dtype"]]) + (["--fused"] if fused else [])
    if b["steps"] != 200:
        argv += ["--steps", str(b["steps"])]
    if b["warmup"] != 1000:
        argv += ["--warmup", str(b["warmup"])]
    for key, flag in (("kernels", "--no-kernel-table"), ("cpu_baseline", "--no-cpu-baseline"),
                      ("single_pass_step", "--no-single-pass"), ("layer_batch", "--no-layer-batch")):
        if key not in b:
            argv.append(flag)
    if "ablation" in b:
        argv.append("--ablation")
    name = os.path.basename(d)
    cmd = (f"cd /tmp && export TMPDIR=/tmp && timeout -k 10 600 rocprofv3 --kernel-trace --stats "
           f"--output-format csv -d $R/gpurun_out/stats/{name} -o step -- python -u $R/bench.py "
           f"{' '.join(argv)}")

    def label(n):
        for k, v in STATS_NAMES.items():
            if k in n:
                return v
        return "`" + _short_kernel(n) + "`"
    md = [f"# Kernel durations: rocprofv3 --kernel-trace --stats, {b['config']['rows']}x"
          f"{b['config']['cols']} {b['dtype'].upper()} writeback step", "",
          f"Workload: {b['config']['workload']}; {b['warmup']} warm-up and {b['steps']} timed steps, "
          "then the stage-breakdown pass and the steps replayed from graphs, plus the copy probe.  "
          "One MI355X (gfx950), ROCm 7.2 ($R is the repository root on the GPU box):", "", "```",
          cmd + f" > $R/gpurun_out/stats/{name}.log 2>&1", "```", "",
          f"This summary is `python bench.py --summarize-stats gpurun_out/stats/{name} --out <this "
          "file>`.  From `step_kernel_stats.csv` (µs):", "",
          "| kernel | calls | average | min | max |", "|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {label(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    rl = b["roofline"]
    md += ["", "The same run's `bench.py` line (under the profiler, whose serialization slows every "
           "launch a little and the event-marked ones more): stage breakdown pass (µs, an event "
           "before every stage) " + ", ".join(f"{k} {v}" for k, v in
                                              b["stage_us_breakdown_pass"].items())
           + f"; one step replayed from a graph {b['graph_us_per_step']} µs; the cast from the "
           f"events stamped at its kernel's start and end {rl['launch_us']} µs, from markers "
           f"around the call {rl.get('launch_us_with_dispatch')} µs.", "",
           f"Kernel only, the step's cast moves {alg / 1e6:.1f} MB (algorithmic) in {avg:.2f} µs on "
           f"average = {alg / (avg * 1e-6) / 1e12:.2f} TB/s ({alg / (avg * 1e-6) / 8e12 * 100:.1f}% of "
           "8 TB/s).  `roofline.achieved` divides the same bytes by the mean of the kernel-stamped "
           "events over the timed steps.", "",
           f"Kernel source: `kernels.hip` sha256 prefix "
           f"`{b.get('library', {}).get('build_id', kernel_sha())}` (the build id the library "
           "reported).", ""]
    _write(args, md)


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_stats:
        summarize_stats(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the writeback runs on a single MI355X "
              "(the cross-rank MAX all-reduce is replaced by an on-device combine); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mxfp8_block_scaled_partial_amd import binding as B
    from mxfp8_block_scaled_partial_amd import bytes_model as BM
    from mxfp8_block_scaled_partial_amd import workloads as wl
    from mxfp8_block_scaled_partial_amd import writeback as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    dev = torch.device("cuda:0")
    rows, cols = 16384, 6144
    n = rows * cols
    tdt = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    s_in = 2 if args.dtype == "bf16" else 4

    log(f"generating {rows}x{cols} {args.dtype} input")
    m = wl.matrix_large(args.dtype)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x0 = to_dev(m.data)
    cuts = [0, n // 4 + 17, n // 2 + 17, 3 * n // 4 + 17, n]
    frags = [(cuts[i], cuts[i + 1] - cuts[i]) for i in range(4)]
    spec = W.WeightSpec(rows, cols, True)

    set_bytes = n * s_in + 2 * n + 4 * (spec.amax_row_entries + spec.amax_col_entries) * s_in
    n_sets = max(2, int(np.ceil(args.min_footprint_gb * 1e9 / set_bytes)))
    log(f"{n_sets} buffer sets of {set_bytes / 1e6:.0f} MB")
    sets = []
    for i in range(n_sets):
        x = x0 if i == 0 else x0.clone()
        wb = W.Writeback([spec], tdt, dev, frags, shared=False, fused=args.fused)
        plan = wb.plan([x[s:s + l] for s, l in frags])
        sets.append((x, wb, plan))
    for p in sets[0][2].amax:
        assert B.mxfp8_query_path(p, 0) == 1
    for p in sets[0][2].cast:
        assert B.mxfp8_query_path(p, 2 if args.fused else 1) == 1

    # algorithmic bytes of one step
    per = [BM.piece_bytes(rows, cols, s, l, s_in, True) for s, l in frags]
    packed = spec.amax_row_entries + spec.amax_col_entries
    stage_bytes = {
        "zero": BM.zero_bytes(4, packed, s_in),
        "amax": sum(p["amax"] for p in per),
        "combine": BM.combine_bytes(4, packed, s_in),
    }
    if args.fused:
        stage_bytes["scales_cast"] = sum(p["scales_cast"] for p in per)
    else:
        stage_bytes["scales"] = BM.piece_bytes(rows, cols, 0, n, s_in, True)["scales"]
        stage_bytes["cast"] = sum(p["cast"] for p in per)
    step_bytes = sum(stage_bytes.values())

    # Step i runs zero / amax / combine (/ scales) on buffer set i and the cast of set i - 1,
    # the weight before it: as in a writeback over many weights, a fragment's cast never
    # directly follows its own amax, so the cast reads its input from HBM and not from the
    # Infinity Cache the amax just filled.  Every step still runs every stage once.
    stage_names = [name for name, _ in sets[0][2].stages()]
    stages = [s[2].stages() for s in sets]

    def step(i, ev=None, cast_ev=None, kernel_ev=None):
        """One step; ``ev`` times every stage (the breakdown pass), ``cast_ev`` brackets the
        cast call with markers on the stream, ``kernel_ev`` has the library stamp the cast's
        own kernel start and end (the timed steps: each marker costs the stream a few µs)."""
        seq = stages[i % n_sets][:-1] + [stages[(i - 1) % n_sets][-1]]
        last = len(seq) - 1
        for j, (_, fn) in enumerate(seq):
            if ev is not None:
                ev[j].record()
            if cast_ev is not None and j == last:
                cast_ev[0].record()
            if kernel_ev is not None and j == last:
                B.mxfp8_time_next_call(kernel_ev[0].ev.value, kernel_ev[1].ev.value)
            fn()
        if ev is not None:
            ev[-1].record()
        if cast_ev is not None:
            cast_ev[1].record()

    lib_id, lib_ok = library_matches_source()
    if not lib_ok:
        if args.counter_pass:
            raise SystemExit(f"the library was built from kernel source {lib_id}, not from the "
                             f"current {kernel_sha()}: rebuild it before a counter pass")
        log(f"WARNING: the library was built from kernel source {lib_id}, not from the current "
            f"{kernel_sha()}; roofline.traffic stays null")

    if args.counter_pass:
        counter_pass(args, stages, n_sets, stage_bytes, m, dev)
        return

    log(f"warmup {args.warmup} steps")
    for i in range(max(2, args.warmup)):
        step(i)
    torch.cuda.synchronize()

    # the timed steps: wall clock over all of them.  The cast call of every CAST_SAMPLE-th
    # step is timed by HIP events that the runtime stamps at its kernel's start and end
    # (mxfp8_time_next_call: hipExtLaunchKernel events), and that of the steps halfway between
    # by events recorded on the stream around the call, which also hold its dispatch (each
    # marker costs the stream a few µs, so sampling keeps the measurement from lengthening the
    # steps it measures)
    kev = {i: (TimingEvent(), TimingEvent()) for i in range(0, args.steps, CAST_SAMPLE)}
    cev = {i: (TimingEvent(), TimingEvent())
           for i in range(CAST_SAMPLE // 2, args.steps, CAST_SAMPLE)}
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, cast_ev=cev.get(i), kernel_ev=kev.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    cast_ms_mean = sum(a.elapsed_time(b) for a, b in kev.values()) / len(kev)
    cast_ms_bracket = sum(a.elapsed_time(b) for a, b in cev.values()) / len(cev)

    # the stage breakdown, from a separate pass with an event before every stage
    # (informational: the markers themselves lengthen that pass's steps)
    evs = [[TimingEvent() for _ in range(len(stage_names) + 1)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    stage_ms = {name: statistics.median(e[j].elapsed_time(e[j + 1]) for e in evs)
                for j, name in enumerate(stage_names)}

    # dominant kernel: the cast (with --fused, the fused one).  The library launches
    # the pieces of one call that share a kernel specialization together, up to 16 per
    # launch: here the 4 fragments of the weight (all on the vector path, checked above) go
    # out as one launch.
    cast_stage = stage_names[-1]
    kname = (f"cast_vec_kernel<{args.dtype}, colwise, fused scales>" if args.fused
             else f"cast_vec_kernel<{args.dtype}, colwise>")
    n_cast = -(-sets[0][2].n_cast // 16)
    cast_launch_us = cast_ms_mean * 1e3 / n_cast
    cast_bytes_launch = stage_bytes[cast_stage] / n_cast
    achieved = cast_bytes_launch / (cast_launch_us * 1e-6) / 1e9
    traffic = traffic_from_counters(args.dtype, bool(args.fused), "step_" + cast_stage, lib_id)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": kname,
                "launch_us": round(cast_launch_us, 2),
                "launch_us_with_dispatch": round(cast_ms_bracket * 1e3 / n_cast, 2),
                "timing": f"mean over {len(kev)} timed steps of HIP events stamped at the "
                          "cast kernel's start and end (hipExtLaunchKernel); "
                          "launch_us_with_dispatch: events recorded around the call on the "
                          f"stream, {len(cev)} other timed steps",
                "alg_bytes_per_launch": int(cast_bytes_launch)}

    # the same steps replayed from captured graphs (no host launch gaps)
    def graph_step(j):
        seq = stages_now(j % n_sets)[:-1] + [stages_now((j - 1) % n_sets)[-1]]
        for _, fn in seq:
            fn()

    def stages_now(j):  # built at call time, so inside a capture they use its stream
        return sets[j][2].stages()

    graph_us = graph_step_us(args, [lambda j=j: graph_step(j) for j in range(n_sets)])

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"{rows}x{cols} {args.dtype} master weight as 4 contiguous "
                               "fragments (cuts at N/4+17, N/2+17, 3N/4+17), bidirectional "
                               "MXFP8 writeback: zero, partial amax, combine K=4, "
                               + ("scales fused into the partial cast" if args.fused
                                  else "scales, partial cast"),
                   "rows": rows, "cols": cols, "fragments": frags, "buffer_sets": n_sets,
                   "step_alg_bytes": step_bytes},
        "library": {"build_id": lib_id, "kernel_source": kernel_sha(), "matches_source": lib_ok},
        "graph_us_per_step": graph_us,
        "graph_GBps": round(step_bytes / (graph_us * 1e-6) / 1e9, 1),
        "stage_us_breakdown_pass": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "stage_alg_GBps": {k: round(stage_bytes[k] / (stage_ms[k] * 1e-3) / 1e9, 1)
                           for k in stage_names},
        "roofline": roofline,
    }

    if args.single_pass:
        out["single_pass_step"] = {
            "k_buffers": single_pass_step(args, sets, spec, frags, s_in, dev, tdt, False),
            "shared_buffer": single_pass_step(args, sets, spec, frags, s_in, dev, tdt, True)}

    if args.copy_probe:
        out["copy_probe"] = copy_probe(dev)

    if args.kernel_table:
        out["kernels"], out["kernels_other_shapes"] = kernel_table(args, m, dev)
        # the bar: partial amax and partial cast each at >= 70% of HBM peak on the full
        # 16384x6144 input, BF16 and FP32 (per-call table, graph replays)
        k = out["kernels"]
        names = ("amax_bf16_full", "cast_bf16_full", "amax_fp32_full", "cast_fp32_full")
        if all(nm in k for nm in names) and roofline is not None:
            roofline["bar"] = {nm: {"us": k[nm]["us"], "frac": k[nm]["frac_of_peak"]}
                               for nm in names}
            roofline["bar"]["target_frac"] = 0.70
            roofline["bar"]["all_met"] = all(k[nm]["frac_of_peak"] >= 0.70 for nm in names)

    if args.layer_batch:
        out["layer_batch"] = layer_batch(args, dev)

    if args.ablation:
        out["ablation"] = ablation(args, dev)

    if args.cpu:
        # the oracle leg runs after every GPU measurement (the GPU idles meanwhile): it times
        # the oracle on the host and checks the outputs the steps left for weight 0 (the same
        # input and fragments; every step writes the same bytes) bit for bit
        wb0 = sets[0][1]
        ar0, ac0 = wb0.combined.views(0)
        st0 = wb0.storage[0]
        gpu0 = {"amax_row": ar0, "amax_col": ac0, "scale_row": st0.scale_row,
                "scale_col": st0.scale_col, "data_row": st0.data_row, "data_col": st0.data_col}
        out["cpu_baseline"] = cpu_baseline(m, args.cpu_rows, s_in,
                                           gpu0 if args.cpu_rows == rows else None)

    print(json.dumps(out), flush=True)


COPY_PROBE_BYTES = 256 << 20
COPY_PROBE_LAUNCHES = 24


def copy_probe(dev):
    """A plain device-to-device copy of known size (256 MiB per launch, rotating over four
    buffer pairs so it streams from HBM): the achievable read + write ceiling on this machine, and
    the kernel the rocprofv3 FETCH_SIZE / WRITE_SIZE counters are calibrated on.  24 launches:
    4 untimed, then 20 between HIP events."""
    import torch

    nb = COPY_PROBE_BYTES
    pairs = [(torch.empty(nb, dtype=torch.uint8, device=dev),
              torch.empty(nb, dtype=torch.uint8, device=dev)) for _ in range(4)]
    for a, b in pairs:
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = TimingEvent(), TimingEvent()
    reps = COPY_PROBE_LAUNCHES - 4
    e0.record()
    for i in range(reps):
        a, b = pairs[i % 4]
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del pairs
    return {"bytes_per_launch": 2 * nb, "read_bytes": nb, "write_bytes": nb,
            "us": round(us, 2), "GBps": round(2 * nb / (us * 1e-6) / 1e9, 1)}


class LaunchLog:
    """The order of the launches of a counter or trace run (--counter-pass): each item is
    preceded by a marker, a one-element int16 fill (a kernel nothing else here launches), so
    the summaries can split the profiled dispatches into items whatever kernels an item runs.
    The marker tensor's own zero-fill, when the log is made, is one more such fill: it opens
    the span of everything before the first item."""

    def __init__(self, dev):
        import torch

        self.items = []
        self._t = torch.zeros(1, dtype=torch.int16, device=dev)

    def run(self, label, calls, alg_bytes, fn, aux=False):
        """The marker, then fn(i) for i < calls, then a synchronization.  An ``aux`` item (work
        between measured items, such as a check) only delimits: the summaries skip it."""
        import torch

        self._t.fill_(1)
        for i in range(calls):
            fn(i)
        torch.cuda.synchronize()
        self.items.append({"label": label, "calls": calls, "alg_bytes": int(alg_bytes)})
        if aux:
            self.items[-1]["aux"] = True


def counter_pass(args, stages, n_sets, stage_bytes, m, dev):
    """The launches a rocprofv3 counter or trace pass attributes, untimed and in a fixed order:
    the steps (each stage but the zero-fill, which is torch's, as an item of one call), the
    copy probe, then (unless --no-kernel-table) every entry of the per-call table as
    ``--counter-calls`` eager calls rotating over its buffer sets, and (unless
    --no-layer-batch) the layer batch's stages and one rank's calls.  Writes the order to the
    manifest for ``summarize_counters`` and ``summarize_trace``."""
    L = LaunchLog(dev)
    for i in range(max(2, args.warmup) + args.steps):
        seq = stages[i % n_sets][:-1] + [stages[(i - 1) % n_sets][-1]]
        for name, fn in seq:
            if name == "zero":
                fn()
            else:
                L.run(f"step_{name}", 1, stage_bytes[name], lambda i, fn=fn: fn())
    L.run("copy_probe", 1, 2 * COPY_PROBE_BYTES, lambda i: copy_probe(dev))
    if args.kernel_table:
        kernel_table(args, m, dev, L)
    if args.layer_batch:
        layer_batch(args, dev, L)
    if args.ablation:
        ablation(args, dev, L=L)
    man = {"argv": sys.argv[1:], "dtype": args.dtype, "fused": bool(args.fused),
           "kernel_source_sha256_16": library_matches_source()[0],
           "copy_probe": {"launches": COPY_PROBE_LAUNCHES, "read_bytes": COPY_PROBE_BYTES,
                          "write_bytes": COPY_PROBE_BYTES},
           "items": L.items}
    with open(args.counter_pass, "w") as f:
        json.dump(man, f, indent=1)
    log(f"counter pass: {len(L.items)} items -> {args.counter_pass}")


def single_pass_step(args, sets, spec, frags, s_in, dev, tdt, shared):
    """The same writeback with ``single_pass``: each fragment's whole 32-row bands are
    quantized in one pass (input read once) on a side stream, overlapped with the partial
    chain for the bands at the cuts (amax -> combine of just their entries -> scales + cast;
    with ``shared`` the cut blocks merge atomically into one buffer and there is no combine).
    Same outputs, fewer bytes moved.  Timed with HIP events around each whole step, eagerly
    and replayed from a captured graph, over the rotating buffer sets."""
    import torch

    from mxfp8_block_scaled_partial_amd import bytes_model as BM
    from mxfp8_block_scaled_partial_amd import writeback as W

    plans = []
    for x, _, _ in sets:
        wb = W.Writeback([spec], tdt, dev, frags, shared=shared, single_pass=True)
        plans.append(wb.plan([x[s:s + l] for s, l in frags]))
    p0 = plans[0]
    k = 1 if shared else len(frags)
    rows, cols = spec.rows, spec.cols
    packed = spec.amax_row_entries + spec.amax_col_entries
    part = [BM.piece_bytes(rows, cols, a, b - a, s_in, True) for _, a, b in p0.partial_ranges]
    quant = [BM.piece_bytes(rows, cols, a, b - a, s_in, True) for _, a, b in p0.quant_ranges]
    shared_entries = 0 if shared else sum(c for _, _, c in p0.wb.combine_calls)
    stage_bytes = {"zero": BM.zero_bytes(k, packed, s_in),
                   "amax": sum(p["amax"] for p in part),
                   "quantize": sum(p["quantize"] for p in quant),
                   "scales_cast": sum(p["scales_cast"] for p in part)}
    if not shared:
        stage_bytes["combine"] = BM.combine_bytes(k, shared_entries, s_in)
    total = sum(stage_bytes.values())

    # one linear pass with events per stage (no overlap), for the breakdown
    names = [n for n, _ in p0.stages()]
    ev = [TimingEvent() for _ in range(len(names) + 1)]
    stage_runs = []
    for i in range(args.warmup + 5):
        for j, (_, fn) in enumerate(plans[i % len(plans)].stages()):
            ev[j].record()
            fn()
        ev[-1].record()
        torch.cuda.synchronize()
        stage_runs.append([ev[j].elapsed_time(ev[j + 1]) * 1e3 for j in range(len(names))])
    stage_us = {n: round(statistics.median(r[j] for r in stage_runs[args.warmup:]), 2)
                for j, n in enumerate(names)}

    # the overlapped step, eager
    for i in range(args.warmup):
        plans[i % len(plans)].run()
    torch.cuda.synchronize()
    evs = [(TimingEvent(), TimingEvent())
           for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        plans[(args.warmup + i) % len(plans)].run()
        e1.record()
    torch.cuda.synchronize()
    step_us = statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    graph_us = graph_step_us(args, [lambda p=p: p.run() for p in plans])
    return {"us": round(step_us, 2), "graph_us": graph_us, "alg_bytes": total,
            "GBps": round(total / (step_us * 1e-6) / 1e9, 1),
            "graph_GBps": round(total / (graph_us * 1e-6) / 1e9, 1),
            "stage_us_serial": stage_us, "stage_alg_bytes": stage_bytes,
            "quantize_pieces": p0.n_quant, "partial_pieces": p0.n_cast,
            "combined_entries": shared_entries,
            "note": "same outputs as the step; whole bands of each fragment go through the "
                    "single-pass quantize (input read once) on a second stream, overlapped "
                    "with the partial chain for the bands at the cuts"}


def layer_batch(args, dev, L=None):
    """The transformer-layer batch: QKV 4096x12288 (bidirectional), out-proj 4096x4096
    (row-only), up 4096x14336 (bidirectional), down 14336x4096 (row-only), BF16, end to end in
    one flat buffer of 184 549 376 elements cut into 8 equal fragments (fragments 2 and 5 span
    weight boundaries).

    ``steps``: the whole writeback per step, with one packed buffer per fragment + a K = 8
    MAX-combine (as 8 ranks would hold them), and with one shared packed buffer whose cut
    blocks merge atomically (no combine).  Two buffer sets; step i runs the amax side on set i
    and the cast of set i - 1, as in the main step.  Timed with events around each whole step
    (eager) and from graph replays; a separate pass with a marker before every stage gives
    each stage's µs and its GB/s / fraction of peak on the stage's algorithmic bytes.

    ``rank_fragment``: one rank's share, fragment 2 (its pieces of QKV, out-proj and up), per
    call like the kernel table (graph replays of 10 calls over rotating buffer sets): its
    partial amax, and its cast in place and into fragment-sized outputs.

    With a LaunchLog ``L`` (a counter pass) nothing is timed: the steps' stages and the
    rank's calls run as items of the log."""
    import numpy as np
    import torch

    from mxfp8_block_scaled_partial_amd import binding as B
    from mxfp8_block_scaled_partial_amd import bytes_model as BM
    from mxfp8_block_scaled_partial_amd import workloads as wl
    from mxfp8_block_scaled_partial_amd import writeback as W

    log("generating the layer batch")
    b = wl.layer_batch()
    specs = [W.WeightSpec(r, c, cw) for _, r, c, cw in b.tensors]
    frags = b.fragments
    x0 = torch.from_numpy(b.data.view(np.int16)).view(torch.bfloat16).to(dev)
    del b
    packed = sum(sp.amax_row_entries + sp.amax_col_entries for sp in specs)

    def piece_sum(frag_list, key):
        tot = 0
        for fs, fl in frag_list:
            for (i, st, n, _) in W.split_fragment(specs, fs, fl):
                tot += BM.piece_bytes(specs[i].rows, specs[i].cols, st, n, 2,
                                      specs[i].colwise)[key]
        return tot

    scale_bytes = sum(BM.piece_bytes(sp.rows, sp.cols, 0, sp.numel, 2, sp.colwise)["scales"]
                      for sp in specs)
    res = {"workload": "QKV 4096x12288 bi, out 4096x4096 row, up 4096x14336 bi, down "
                       "14336x4096 row; BF16; 184549376 elements in 8 fragments",
           "packed_entries": packed}
    xs = [x0, x0.clone()]
    for mode, shared in (("k_buffers", False), ("shared_buffer", True)):
        k = 1 if shared else len(frags)
        stage_bytes = {"zero": BM.zero_bytes(k, packed, 2), "amax": piece_sum(frags, "amax")}
        if not shared:
            stage_bytes["combine"] = BM.combine_bytes(k, packed, 2)
        stage_bytes["scales"] = scale_bytes
        stage_bytes["cast"] = piece_sum(frags, "cast")
        total = sum(stage_bytes.values())
        plans = []
        for x in xs:
            wb = W.Writeback(specs, torch.bfloat16, dev, frags, shared=shared)
            plans.append(wb.plan([x[s:s + l] for s, l in frags]))
        names = [nm for nm, _ in plans[0].stages()]
        assert names[-1] == "cast" and list(stage_bytes) == names, names

        def step(i, ev=None):
            seq = plans[i % 2].stages()[:-1] + [plans[(i - 1) % 2].stages()[-1]]
            for j, (_, fn) in enumerate(seq):
                if ev is not None:
                    ev[j].record()
                fn()
            if ev is not None:
                ev[-1].record()

        if L is not None:
            for i in range(max(2, args.warmup) + max(4, args.steps // 2)):
                for nm, fn in plans[i % 2].stages()[:-1] + [plans[(i - 1) % 2].stages()[-1]]:
                    if nm == "zero":
                        fn()
                    else:
                        L.run(f"layer_{mode}_{nm}", 1, stage_bytes[nm], lambda i, fn=fn: fn())
            del plans
            torch.cuda.empty_cache()
            continue

        for i in range(max(2, args.warmup)):
            step(i)
        torch.cuda.synchronize()
        steps = max(4, args.steps // 2)
        tev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
        for i, (e0, e1) in enumerate(tev):
            e0.record()
            step(i)
            e1.record()
        torch.cuda.synchronize()
        step_us = statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in tev)
        evs = [[TimingEvent() for _ in range(len(names) + 1)] for _ in range(steps)]
        for i in range(steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        stage_us = {nm: statistics.median(e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs)
                    for j, nm in enumerate(names)}

        def graph_fn(j):
            def fn():
                for _, f in (plans[j % 2].stages()[:-1] + [plans[(j - 1) % 2].stages()[-1]]):
                    f()
            return fn

        graph_us = graph_step_us(args, [graph_fn(0), graph_fn(1)])
        res[mode] = {
            "us": round(step_us, 2), "graph_us": graph_us, "alg_bytes": total,
            "GBps": round(total / (step_us * 1e-6) / 1e9, 1),
            "stages": {nm: {"us": round(stage_us[nm], 2), "alg_bytes": stage_bytes[nm],
                            "GBps": round(stage_bytes[nm] / (stage_us[nm] * 1e-6) / 1e9, 1),
                            "frac_of_peak": round(stage_bytes[nm] / (stage_us[nm] * 1e-6) / 1e9
                                                  / HBM_PEAK_GBS, 4)}
                       for nm in names},
            "pieces": {"amax": plans[0].n_amax, "cast": plans[0].n_cast},
            "note": "stage times from a pass with a marker before every stage; launches per "
                    "call: the kernel trace summary"}
        del plans
        torch.cuda.empty_cache()

    # one rank's fragment, per call
    f = 2
    fs, fl = frags[f]
    rank = {"fragment": [fs, fl], "pieces": [[i, st, n] for (i, st, n, _) in
                                              W.split_fragment(specs, fs, fl)]}
    per_set = fl * 2 * 2 + 2 * packed * 3
    n_sets = max(2, min(10, int(np.ceil(args.min_footprint_gb * 1e9 / per_set))))
    for name, fo in (("in_place", False), ("fragment_outputs", True)):
        plans = []
        for i in range(n_sets):
            x = x0[fs:fs + fl].clone()  # the rank's shard in an allocation of its own
            wb = W.Writeback(specs, torch.bfloat16, dev, [(fs, fl)], shared=True,
                             fragment_outputs=fo)
            plans.append(wb.plan([x]))
        lib = B.lib()
        calls = [("cast", lambda p, sp: lib.mxfp8_partial_cast(p.cast, p.n_cast, sp))]
        if not fo:
            calls.insert(0, ("amax", lambda p, sp: lib.mxfp8_partial_amax(p.amax, p.n_amax, sp)))
        for kname, call in calls:
            def fn(i, call=call):
                assert call(plans[i % n_sets], torch.cuda.current_stream().cuda_stream) == 0
            nb = piece_sum([(fs, fl)], kname)
            if L is not None:
                L.run(f"rank_{kname}_{name}", args.counter_calls, nb, fn)
                continue
            us = per_call_us(args, fn, 10)
            rank[f"{kname}_{name}"] = {"us": round(us, 2), "alg_bytes": nb,
                                       "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                                       "frac_of_peak": round(nb / (us * 1e-6) / 1e9
                                                             / HBM_PEAK_GBS, 4),
                                       "pieces": len(rank["pieces"]), "buffer_sets": n_sets}
        del plans
        torch.cuda.empty_cache()
    res["rank_fragment"] = rank
    return None if L is not None else res


def ablation(args, dev, rounds=3, L=None):
    """The PR page's one design measurement ("Bidirectional kernel performance": an earlier
    version whose amax selected the column-wise work with runtime pointer guards was 21-35%
    slower) redone on MI355X with the current kernels: the product's compile-time
    specialization (one kernel per direction) against libmxfp8partial_guards.so (one kernel per
    dtype for both, the column-wise work selected at run time by the column-wise pointer).
    16384x6144 BF16 and FP32, full input and the quarter fragment at offset 17, row-only and
    bidirectional, amax and cast; per call from graph replays of 10 calls over rotating buffer
    sets, the two builds interleaved over ``rounds`` rounds (median).  Each case also checks
    that the two builds write the same bytes.  With a LaunchLog ``L`` (a counter pass) nothing
    is timed: each case's calls run as one item per build (``abl_<build>_<case>``)."""
    import numpy as np
    import torch

    from mxfp8_block_scaled_partial_amd import binding as B
    from mxfp8_block_scaled_partial_amd import build as hip_build
    from mxfp8_block_scaled_partial_amd import bytes_model as BM
    from mxfp8_block_scaled_partial_amd import workloads as wl

    libs = {"compile_time": B.lib(), "runtime_guard": B.load_library(hip_build.GUARDS_LIB)}
    out = {"note": "µs per call; ratio = runtime_guard / compile_time"}
    for dtype in ("bf16", "fp32"):
        log(f"ablation: {dtype}")
        m = wl.matrix_large(dtype)
        rows, cols = m.rows, m.cols
        n = rows * cols
        nb, nbands = B.nblocks(cols), B.nblocks(rows)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        s_in = 2 if dtype == "bf16" else 4
        x0 = (torch.from_numpy(m.data.view(np.int16)).view(torch.bfloat16) if dtype == "bf16"
              else torch.from_numpy(m.data)).to(dev)
        for run, (s, l) in (("full", (0, n)), ("quarter", (17, n // 4))):
            lead = s % 32  # input - s and data - s stay aligned, as in the per-call table
            per_set = l * s_in + 2 * l + (rows * nb + nbands * cols) * (s_in + 1)
            n_sets = max(2, min(10, int(np.ceil(args.min_footprint_gb * 1e9 / per_set))))
            sets = []
            for i in range(n_sets):
                xb = torch.empty(l + 32, dtype=tdt, device=dev)
                xb[lead:lead + l] = x0[s:s + l]
                bufs = dict(x=xb[lead:lead + l], xb=xb,
                            ar=torch.zeros(rows, nb, dtype=tdt, device=dev),
                            ac=torch.zeros(nbands, cols, dtype=tdt, device=dev),
                            sr=torch.full((rows, nb), 120, dtype=torch.uint8, device=dev),
                            sc=torch.full((nbands, cols), 120, dtype=torch.uint8, device=dev),
                            drb=torch.zeros(l + 32, dtype=torch.uint8, device=dev),
                            dcb=torch.zeros(l + 32, dtype=torch.uint8, device=dev))
                sets.append(bufs)
            for colwise in (True, False):
                arrs = {"amax": [], "cast": []}
                for b in sets:
                    dr, dc = b["drb"][lead:lead + l], b["dcb"][lead:lead + l]
                    arrs["amax"].append(B._array([B.make_piece(
                        rows, cols, s, b["x"], amax_row=b["ar"],
                        amax_col=b["ac"] if colwise else None)])[0])
                    arrs["cast"].append(B._array([B.make_piece(
                        rows, cols, s, b["x"], scale_row=b["sr"], scale_col=b["sc"],
                        data_row=dr, data_col=dc if colwise else None)])[0])
                for kname in ("amax", "cast"):
                    # same bytes from both builds (set 0, outputs cleared before each)
                    outs = []

                    def check(_):
                        for name, lb in libs.items():
                            b = sets[0]
                            for t in (b["ar"], b["ac"], b["drb"], b["dcb"]):
                                t.zero_()
                            f = getattr(lb, f"mxfp8_partial_{kname}")
                            assert f(arrs[kname][0], 1,
                                     torch.cuda.current_stream().cuda_stream) == 0
                            torch.cuda.synchronize()
                            outs.append([t.clone() for t in (b["ar"], b["ac"], b["drb"], b["dcb"])])
                    if L is not None:
                        L.run(f"abl_check_{kname}_{dtype}_{run}_{colwise}", 1, 0, check, aux=True)
                    else:
                        check(0)
                    same = all(torch.equal(a, c) for a, c in zip(*outs))
                    key = f"{kname}_{dtype}_{run}_{'bidirectional' if colwise else 'rowonly'}"
                    if L is not None:
                        assert same, key
                        nb_alg = BM.piece_bytes(rows, cols, s, l, s_in, colwise)[kname]
                        for name, lib in libs.items():
                            f = getattr(lib, f"mxfp8_partial_{kname}")
                            L.run(f"abl_{name}_{key}", args.counter_calls, nb_alg,
                                  lambda i, f=f, a=arrs[kname]: f(
                                      a[i % n_sets], 1, torch.cuda.current_stream().cuda_stream))
                        continue
                    times = {name: [] for name in libs}
                    for _ in range(rounds):
                        for name, lb in libs.items():
                            f = getattr(lb, f"mxfp8_partial_{kname}")

                            def fn(i, f=f, a=arrs[kname]):
                                assert f(a[i % n_sets], 1,
                                         torch.cuda.current_stream().cuda_stream) == 0
                            times[name].append(per_call_us(args, fn, 10))
                    ct = statistics.median(times["compile_time"])
                    rg = statistics.median(times["runtime_guard"])
                    out[key] = {"compile_time_us": round(ct, 2), "runtime_guard_us": round(rg, 2),
                                "ratio": round(rg / ct, 3), "same_bytes": same,
                                "buffer_sets": n_sets}
            del sets
            torch.cuda.empty_cache()
    return out


def per_call_us(args, fn, per_graph):
    """Median µs per call of ``fn(i)`` (call i on buffer set i), from HIP events around
    replays of a captured graph of ``per_graph`` calls, as in the per-call table."""
    import torch

    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(args.kernel_calls)]
    for e0, e1 in ev:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    us = statistics.median(e0.elapsed_time(e1) * 1e3 / per_graph for e0, e1 in ev)
    del g
    return us


def graph_step_us(args, step_fns):
    """Median µs of one step replayed from a captured HIP graph (one graph per buffer set,
    replayed in turn), so no host launch gap sits between the step's kernels."""
    import torch

    graphs = []
    for fn in step_fns:
        fn()  # outside capture first: nothing is first-touched inside the graph
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()  # the library reads torch's current stream: the capture stream here
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        graphs[i % len(graphs)].replay()
        e1.record()
    torch.cuda.synchronize()
    us = statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    del graphs
    return round(us, 2)


def kernel_table(args, m_default, dev, L=None):
    """Per-call µs and GB/s of partial amax and partial cast, the pages' table, plus the fused
    scales + cast and (full input only) the single-pass quantize, for every matrix of that
    table (16384x6144, 4096x4096, 1024x1024, 160x96): full input and the quarter fragment
    starting at offset 17, both directions, BF16 and FP32.  Timed like the pages: HIP events
    around replays of a captured graph of 50 calls (up to 4 M elements) or 10 calls (larger),
    median per call over the replays.  Calls rotate over distinct buffer sets, as many as
    reach the footprint option but at most one per call of the graph (full runs: whole
    matrices; partial runs: quarter-size fragments placed so that input - 17 elements stays
    16-byte aligned): the two large matrices stream from HBM, the small ones stay in the 256 MB
    Infinity Cache like any repeated small call.  Returns the 16384x6144 entries and, by
    shape, the others.  With a LaunchLog ``L`` (a counter pass) nothing is timed: each entry
    makes ``--counter-calls`` eager calls as an item of the log."""
    import torch

    from mxfp8_block_scaled_partial_amd import workloads as wl

    table, by_shape = {}, {}
    shapes = [tuple(int(v) for v in t.split("x")) for t in args.table_shapes.split(",") if t]
    for rows, cols in shapes:
        for dtype in ("bf16", "fp32"):
            if (rows, cols) == (16384, 6144):
                if dtype == args.dtype:
                    m = m_default
                else:
                    log(f"generating {rows}x{cols} {dtype} input for the kernel table")
                    m = wl.matrix_large(dtype)
            else:  # N(0,1) times a per-column 2^U[-8, 8], the 4096x4096 recipe
                m = wl.matrix_square(dtype, rows=rows, cols=cols)
            entries = time_shape(args, m, dev, L)
            if (rows, cols) == (16384, 6144):
                table.update(entries)
            else:
                by_shape.setdefault(f"{rows}x{cols}", {}).update(entries)
            torch.cuda.empty_cache()
    return table, by_shape


def time_shape(args, m, dev, L=None):
    """The table's entries for one matrix in one dtype (see ``kernel_table``)."""
    import numpy as np
    import torch

    from mxfp8_block_scaled_partial_amd import binding as B
    from mxfp8_block_scaled_partial_amd import bytes_model as BM

    rows, cols, dtype = m.rows, m.cols, m.dtype
    n = rows * cols
    nb, nbands = B.nblocks(cols), B.nblocks(rows)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s_in = 2 if dtype == "bf16" else 4
    per_graph = 50 if n <= 4 * 1024 * 1024 else 10
    x0 = (torch.from_numpy(m.data.view(np.int16)).view(torch.bfloat16) if dtype == "bf16"
          else torch.from_numpy(m.data)).to(dev)
    out = {}
    runs = [("full", (0, n)), ("partial", (17, n // 4))]
    if (rows, cols) == (16384, 6144):
        # one rank's own buffers: the quarter fragment's input and its fragment-sized E4M3
        # outputs in allocations of their own, so input - 17 and data - 17 lose their alignment
        # (BF16 input 2 bytes off a dword; outputs off their 128-byte lines: the cast's
        # line-owned tiles)
        runs.append(("partial_own", (17, n // 4)))
        # row-only (column-wise outputs absent: the kColwise = false kernels), full input
        runs.append(("full_rowonly", (0, n)))
    keep_runs = set(args.table_runs.split(","))
    for run, (s, l) in runs:
        if run not in keep_runs:
            continue
        colwise = run != "full_rowonly"
        # element offset that keeps input - s (and data - s) aligned; 0 for a rank's own buffers
        lead = 0 if run == "partial_own" else s % 32
        per_set = l * s_in + 2 * l + (rows * nb + nbands * cols) * (s_in + 1)
        n_sets = max(2, min(per_graph, int(np.ceil(args.min_footprint_gb * 1e9 / per_set))))
        amax_p, cast_p, fused_p, keep = [], [], [], []
        for i in range(n_sets):
            xb = torch.empty(l + 32, dtype=tdt, device=dev)
            xb[lead:lead + l] = x0[s:s + l]
            x = xb[lead:lead + l]
            ar = torch.zeros(rows, nb, dtype=tdt, device=dev)
            ac = torch.zeros(nbands, cols, dtype=tdt, device=dev)
            sr = torch.full((rows, nb), 120, dtype=torch.uint8, device=dev)
            sc = torch.full((nbands, cols), 120, dtype=torch.uint8, device=dev)
            drb = torch.empty(l + 32, dtype=torch.uint8, device=dev)
            dcb = torch.empty(l + 32, dtype=torch.uint8, device=dev)
            dr, dc = drb[lead:lead + l], dcb[lead:lead + l]
            keep.append((xb, ar, ac, sr, sc, drb, dcb))
            if not colwise:  # empty handles for the absent direction
                ac = dc = None
            amax_p.append(B.make_piece(rows, cols, s, x, amax_row=ar, amax_col=ac))
            cast_p.append(B.make_piece(rows, cols, s, x, scale_row=sr, scale_col=sc,
                                       data_row=dr, data_col=dc))
            fused_p.append(B.make_piece(rows, cols, s, x, amax_row=ar, amax_col=ac,
                                        scale_row=sr, scale_col=sc, data_row=dr,
                                        data_col=dc))
            assert B.mxfp8_query_path(amax_p[-1], 0) == 1
            # a rank's own output buffers sit off the 128-byte lines: line-owned cast tiles
            assert B.mxfp8_query_path(cast_p[-1], 1) == (2 if run == "partial_own" else 1)
            assert B.mxfp8_query_path(fused_p[-1], 2) == 1
            assert run != "full" or B.mxfp8_query_path(fused_p[-1], 3) == 1
        pb = BM.piece_bytes(rows, cols, s, l, s_in, colwise)
        # the amax runs first, so the fused call reads real amax entries; the single-pass
        # quantize needs whole bands, so it runs on the full input only
        kernels = [("amax", amax_p, B.mxfp8_partial_amax),
                   ("cast", cast_p, B.mxfp8_partial_cast)]
        if run in ("full", "partial"):
            kernels.append(("scales_cast", fused_p, B.mxfp8_scales_and_cast))
        if run == "full":
            kernels.append(("quantize", fused_p, B.mxfp8_quantize))
        for kname, pieces, fn in kernels:
            if L is not None:
                shape = "" if (rows, cols) == (16384, 6144) else f"{rows}x{cols}_"
                L.run(f"{shape}{kname}_{dtype}_{run}", args.counter_calls, pb[kname],
                      lambda i, fn=fn, pieces=pieces: fn(pieces[i % n_sets]))
                continue
            for i in range(3):
                fn(pieces[i % n_sets])
            torch.cuda.synchronize()
            # the pages' method: HIP-event timing of graph replays (each call on the next
            # buffer set), median per call over the replays
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(per_graph):
                    fn(pieces[i % n_sets])
            g.replay()
            torch.cuda.synchronize()
            ev = [(TimingEvent(), TimingEvent()) for _ in range(args.kernel_calls)]
            for e0, e1 in ev:
                e0.record()
                g.replay()
                e1.record()
            torch.cuda.synchronize()
            us = statistics.median(e0.elapsed_time(e1) * 1e3 / per_graph for e0, e1 in ev)
            del g
            gbs = pb[kname] / (us * 1e-6) / 1e9
            entry = {"us": round(us, 2), "GBps": round(gbs, 1),
                     "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "alg_bytes": pb[kname], "buffer_sets": n_sets, "calls_per_graph": per_graph}
            # the same call on one buffer set over and over: what stays in the 256 MB
            # Infinity Cache between calls is not re-read from HBM (cache-resident figure)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(per_graph):
                    fn(pieces[0])
            g.replay()
            torch.cuda.synchronize()
            for e0, e1 in ev:
                e0.record()
                g.replay()
                e1.record()
            torch.cuda.synchronize()
            hot = statistics.median(e0.elapsed_time(e1) * 1e3 / per_graph for e0, e1 in ev)
            del g
            entry["hot_us_cache_resident"] = round(hot, 2)
            out[f"{kname}_{dtype}_{run}"] = entry
        del keep, amax_p, cast_p, fused_p
        torch.cuda.empty_cache()
    return out


def cpu_baseline(m, cpu_rows, s_in, gpu=None):
    """The oracle (plain C) over the first ``cpu_rows`` rows of the same weight, cut into 4
    fragments like the GPU step, through the whole path: once on one thread, then with the
    rows split into groups of whole 32-row bands, one group per host core (blocks never cross
    a band, so each group is an independent writeback of its rows with the cuts that fall in
    them; the oracle releases the GIL inside its C calls)."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    import oracle
    from mxfp8_block_scaled_partial_amd import bytes_model as BM

    rows, cols = cpu_rows, m.cols
    n = rows * cols
    cuts = [0, n // 4 + 17, n // 2 + 17, 3 * n // 4 + 17, n]
    frags = [(cuts[i], cuts[i + 1] - cuts[i]) for i in range(4)]
    x = m.data[:n]
    oracle.lib()
    # the one-thread leg repeats the whole sample until about 10 s of CPU work have run
    t0 = time.perf_counter()
    want = oracle.writeback(x, rows, cols, frags, colwise=True)
    reps = 1
    while time.perf_counter() - t0 < CPU_LEG_SECONDS:
        oracle.writeback(x, rows, cols, frags, colwise=True)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    check = "not run (sample is not the whole weight)"
    if gpu is not None:
        import numpy as np
        bad = []
        for k, t in gpu.items():
            g = t.detach().cpu()
            g = g.view(torch.int16).numpy().view(np.uint16) if g.dtype == torch.bfloat16 else g.numpy()
            w = want[k]
            if g.dtype == np.float32:
                g, w = g.view(np.uint32), w.view(np.uint32)
            if not np.array_equal(g, w):
                bad.append(f"{k}: {int(np.count_nonzero(g != w))} bytes differ")
        check = "bit-exact" if not bad else "MISMATCH " + "; ".join(bad)
        if bad:
            log("GPU step outputs differ from the oracle: " + check)
    packed = rows * ((cols + 31) // 32) + ((rows + 31) // 32) * cols
    per = [BM.piece_bytes(rows, cols, s, l, s_in, True) for s, l in frags]
    total = (BM.zero_bytes(4, packed, s_in) + sum(p["amax"] + p["cast"] for p in per)
             + BM.combine_bytes(4, packed, s_in)
             + BM.piece_bytes(rows, cols, 0, n, s_in, True)["scales"])

    cores = min(16, len(os.sched_getaffinity(0)))
    nbands = rows // 32
    edges = [round(i * nbands / cores) * 32 for i in range(cores + 1)]

    def group(g):
        r0, r1 = edges[g], edges[g + 1]
        lo, hi = r0 * cols, r1 * cols
        pieces = [(max(s, lo) - lo, min(s + l, hi) - max(s, lo)) for s, l in frags
                  if max(s, lo) < min(s + l, hi)]
        oracle.writeback(x[lo:hi], r1 - r0, cols, pieces, colwise=True)

    t0 = time.perf_counter()
    reps_all = 0
    with ThreadPoolExecutor(cores) as ex:
        while reps_all == 0 or time.perf_counter() - t0 < CPU_LEG_SECONDS / 4:
            list(ex.map(group, range(cores)))
            reps_all += 1
    dt_all = (time.perf_counter() - t0) / reps_all
    sample = (f"first {rows} of 16384 rows ({rows}x{cols}, {n} elements), 4 fragments, whole "
              "path (amax, combine, scales, cast), C oracle")
    return {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt * reps, 2), "runs": reps,
            "sample": sample + f", one thread, {reps} runs of the sample",
            "gpu_step_vs_oracle": check,
            "all_cores": {"value": round(total / dt_all / 1e9, 3), "unit": "GB/s",
                          "cores": cores, "seconds": round(dt_all * reps_all, 2),
                          "runs": reps_all,
                          "sample": sample + f", {cores} threads over groups of 32-row bands"},
            "host_cpus": len(os.sched_getaffinity(0)), "host_cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
