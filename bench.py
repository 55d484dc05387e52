"""Benchmark: GAE over 4096 envs x T=128 fp32 rollouts on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the hot path over one synthetic rollout batch: one
rlca_gae call (rewards, values [N,T+1], terminated, truncated + truncation
bootstraps -> advantages and value targets).  Inputs are drawn once (seeded),
copied to the GPU into R rotating buffer sets whose total size exceeds the
256 MB Infinity Cache, so every step reads its inputs from HBM.  The K timed
steps are captured once in a HIP graph (one kernel launch per step, each on
the next buffer set) and replayed between two events on the launch stream.

Output: one JSON line with env-steps/s, the roofline of the kernel (algorithmic
bytes per launch / average launch time against the 8 TB/s HBM peak) and the
CPU oracle timed on the host cores on a bounded sample.

--window times the window form of the same call (rlca_X_chunk: a per-row
carry read, the outgoing carry and the carry map written) on the same inputs.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "env-steps/sec and achieved HBM GB/s (% of peak), GAE 4096 envs × T=128 fp32"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources each kernel family is built from (with the host code that picks
# its launch configuration): a committed traffic figure is used only while
# these are unchanged.
_CSRC = os.path.join(ROOT, "reverse_linear_recurrence_amd", "csrc")
KERNEL_SOURCES = {
    "scan": ("scan_kernels.hpp", "kernel_table.hpp", "variants.hpp", "kernels_plain.hip",
             "kernels_window.hip", "kernels_chain.hip", "rlca.hip"),
    "probs": ("scan_kernels.hpp", "probs_kernels.hpp", "variants.hpp", "kernels_probs.hip",
              "rlca.hip"),
    "materialized": ("scan_kernels.hpp", "materialized.hpp", "kernels_materialized.hip",
                     "rlca.hip"),
}


def kernel_family(workload_key):
    if workload_key.endswith("/materialized"):
        return "materialized"
    return "probs" if "_probs_" in workload_key else "scan"


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_text(src):
    """C++ source with comments removed and whitespace runs collapsed: what a
    comment-only edit leaves unchanged.  (No kernel source puts // or /* in a
    string literal.)"""
    return " ".join(_COMMENT.sub(" ", src).split())


def traffic_key(workload, window=False, materialized=False, split_form=None):
    """The profiles/traffic.json key of a timed configuration: the workload,
    then the entry point (window or materialized form) and the form a split
    call took (chained or three-launch; an unsplit call adds nothing)."""
    return workload + ("/window" if window else "") + (
        "/materialized" if materialized else "") + {
        "chained": "/chained", "three-launch": "/three-launch"}.get(split_form, "")


def kernel_source_hash(family="scan"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(_CSRC, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="gae_4096x128")
    ap.add_argument("--rotate-mb", type=float, default=1024.0,
                    help="total size of the rotating buffer sets (defeats the 256 MB MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time for the oracle baseline (0: skip)")
    ap.add_argument("--no-graph", action="store_true",
                    help="plain eager launches from Python (same as --timing eager)")
    ap.add_argument("--timing", choices=["auto", "queued", "graph", "eager"], default="auto",
                    help="how the K steps are timed (auto: queued for K <= %d, else graph)"
                    % 1000)
    ap.add_argument("--variant", type=int, default=-1, help="force a tiling variant")
    ap.add_argument("--window", action="store_true",
                    help="time the window entry point (carry in; carry and carry map out)")
    ap.add_argument("--materialized", action="store_true",
                    help="time the materialized doubling scan (rlca_X_materialized, the "
                         "pages' comparison baseline re-created in HIP) instead of the fused "
                         "kernel")
    ap.add_argument("--split", action="store_true",
                    help="call the window form with a workspace (and, without --window, no "
                         "carries), so that calls on few long rows split every row into "
                         "segments")
    ap.add_argument("--no-chain", action="store_true",
                    help="with --split: the three-launch form of split calls instead of the "
                         "chained one (rlca_set_chained(False))")
    ap.add_argument("--spread-replays", type=int, default=11,
                    help="after the timed region, time the same K steps this many more "
                         "times, each block alone, for median / p10 / p90 (0: skip)")
    ap.add_argument("--body-blocks", type=int, default=30,
                    help="blocks of steps timed through the instrumented library for the "
                         "kernel body (0: skip)")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip timing a plain copy kernel of the same byte count")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script into profiles/traffic.json, then exit")
    ap.add_argument("--summarize-profile", nargs=2, metavar=("RUN_DIR", "OUT_MD"),
                    help="write the profile summary of one workload (see summarize_profile), "
                         "then exit")
    return ap.parse_args()


def algorithmic_bytes(w, N, T, window=False):
    """Bytes the method must move per step: one read of every input element
    it uses and one write of every output element (truncation bootstraps,
    read only at truncations, are not counted).  A window call adds its
    per-row carry in (4 B), carry out (4 B) and carry map (8 B) per launch."""
    if window:
        return algorithmic_bytes(w, N, T) + 16 * N * launches_per_step_of(w)
    es = 2 if w.dtype == "bf16" else 4
    if w.algo in ("gae",):
        return (2 * es + 2 + 8) * N * T + es * N  # r, V, 2 flags, adv+targets; V_T
    if w.algo == "td_lambda":
        flags = 2 if w.p_trunc is not None else 1
        return (2 * es + flags + 4) * N * T + es * N
    if w.algo == "returns":
        return (es + 1 + 4) * N * T
    if w.algo == "vtrace+retrace":
        vt = (3 * es + 1 + 8) * N * T + es * N          # r, V, log_rho, term; vs, pg
        rt = (4 * es + 1 + 4) * N * T                  # r, Q, EQ, log_rho, term; q_ret
        return vt + rt
    if w.algo in ("eligibility", "cumsum"):
        flags = 2 if w.p_trunc is not None else 1
        return (es + flags + 4) * N * T                # x, flags; output
    flags = 2 if w.p_trunc is not None else 1
    A = w.num_actions
    if w.algo == "retrace_probs":
        # r, action, the taken behaviour entry, flags, q_ret per step; every
        # entry of the q and log_pi slices 1..T (E_pi Q), and the taken entries
        # of slice 0.
        return (es + 4 + es + flags + 4 + 2 * A * es) * N * T + 2 * es * N
    if w.algo == "vtrace_probs":
        # r, V, action, the two taken entries, flags, vs + pg per step; V_T.
        return (2 * es + 4 + 2 * es + flags + 8) * N * T + es * N
    raise ValueError(w.algo)


def stream_mixes(w):
    """The byte mix of each launch of a step, as (fp32 arrays, 16-bit arrays,
    byte arrays, fp32 outputs) of N*T elements each, for the streaming-ceiling
    leg: the arrays the method must read and write (algorithmic_bytes), or None
    where the ceiling kernel has no such mix."""
    flags = 2 if w.p_trunc is not None else 1
    mixes = {"returns": [(1, 0, flags, 1)], "gae": [(2, 0, 2, 2)],
             "td_lambda": [(2, 0, flags, 1)], "vtrace+retrace": [(3, 0, 1, 2), (4, 0, 1, 1)],
             "eligibility": [(1, 0, flags, 1)], "cumsum": [(1, 0, flags, 1)]}.get(w.algo)
    if mixes is None:
        return None
    if w.dtype == "bf16":
        mixes = [(0, nf, nb, no) for nf, _, nb, no in mixes]
    known = {(1, 0, 1, 1), (2, 0, 2, 2), (2, 0, 1, 1), (2, 0, 2, 1), (3, 0, 1, 2), (4, 0, 1, 1),
             (0, 2, 2, 2), (1, 0, 2, 1)}
    return mixes if all(m in known for m in mixes) else None


def launches_per_step_of(w):
    return 2 if w.algo == "vtrace+retrace" else 1


def summarize_pmc(fetch_dir, write_dir):
    """Per-launch HBM traffic of each kernel from two rocprofv3 --pmc runs of
    `bench.py --no-graph` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
    scaled by the counter reading of the known-size copy kernel in the same
    runs.  Writes profiles/traffic.json keyed by workload."""
    import csv
    import glob
    import statistics

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter_collection.csv under %s" % d)
        vals = {}
        for f in files:
            for row in csv.DictReader(open(f)):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Kernel_Name"], row["Grid_Size"])
                vals.setdefault(key, []).append(float(row["Counter_Value"]))
        return {k: statistics.median(v) for k, v in vals.items()}

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    meta_path = os.path.join(fetch_dir, "bench_meta.json")
    with open(meta_path) as f:
        meta = json.load(f)
    half = meta["copy_bytes_per_launch"] / 2
    # The calibration copy: the runtime's copy kernel whose dispatches write
    # exactly the known size (input uploads use the same kernel name).
    copies = [k for k in write if "copyBuffer" in k[0] and abs(write[k] * 1024 - half) < 0.01 * half]
    scan_name = [k for k in fetch if "rlca::" in k[0]]
    if len(copies) != 1 or not scan_name:
        raise SystemExit("expected one calibration copy and the library's kernel(s): %s"
                         % list(write))
    cn = copies[0]
    f_scale = half / (fetch[cn] * 1024.0)
    w_scale = half / (write[cn] * 1024.0)
    traffic = sum(fetch[k] * 1024.0 * f_scale + write[k] * 1024.0 * w_scale for k in scan_name)
    traffic /= len(scan_name)
    out = {}
    if os.path.exists(TRAFFIC_FILE):
        out = json.load(open(TRAFFIC_FILE))
    out[meta["workload"]] = {
        "kernel_source_hash": kernel_source_hash(kernel_family(meta["workload"])),
        "bytes_per_launch": traffic,
        "fetch_kib_per_launch": {"%s [grid %s]" % k: fetch[k] for k in scan_name},
        "write_kib_per_launch": {"%s [grid %s]" % k: write[k] for k in scan_name},
        "copy_kernel": "%s [grid %s]" % cn,
        "copy_fetch_kib": fetch[cn], "copy_write_kib": write[cn],
        "copy_bytes_read": half, "copy_bytes_written": half,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "algorithmic_bytes_per_launch": meta["algorithmic_bytes_per_launch"],
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out[meta["workload"]], indent=1))


# The commands of one workload's profile, run from the repository root; {opts}
# stands for the bench options of the workload, {d} for the run directory.
PROFILE_COMMANDS = (
    ("bench", "python3 bench.py {opts} > {d}/bench.json"),
    ("trace", "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats "
              "--output-format csv -d {d}/trace -o t -- python3 <repo>/bench.py {opts} "
              "--steps 2000 --warmup 100 --cpu-seconds 0 --body-blocks 0 --spread-replays 0"),
    ("fetch", "cd /tmp && export TMPDIR=/tmp && RLCA_BENCH_META_DIR={d}/fetch rocprofv3 --pmc "
              "FETCH_SIZE --output-format csv -d {d}/fetch -o p -- python3 <repo>/bench.py "
              "{opts} --steps 20 --warmup 2 --cpu-seconds 0 --no-graph --rotate-mb 64 "
              "--body-blocks 0 --spread-replays 0"),
    ("write", "(the same with WRITE_SIZE into {d}/write)"),
    ("busy", "(the same with SQ_BUSY_CYCLES SQ_WAVES into {d}/busy)"),
    ("summary", "python3 bench.py --summarize-profile {d} profiles/<this file>"),
)
SE_COUNT = 32          # shader engines: 4 per XCD, 8 XCDs
SCLK_GHZ = 2.4         # MI355X peak engine clock


def summarize_profile(run_dir, out_md):
    """One workload's profile summary (markdown) from a run directory holding
    args.txt (the bench options), bench.json (the unprofiled bench line),
    trace/ (rocprofv3 --kernel-trace), fetch/ and write/ (--pmc FETCH_SIZE,
    WRITE_SIZE; also written to profiles/traffic.json) and busy/ (--pmc
    SQ_BUSY_CYCLES SQ_WAVES)."""
    import csv
    import glob
    import statistics

    opts = open(os.path.join(run_dir, "args.txt")).read().split()
    b = json.load(open(os.path.join(run_dir, "bench.json")))
    traffic = None
    if os.path.isdir(os.path.join(run_dir, "fetch")):
        summarize_pmc(os.path.join(run_dir, "fetch"), os.path.join(run_dir, "write"))
        entry = b["config"]["entry"]
        key = traffic_key(b["config"]["workload"], entry.startswith("window"),
                          entry.startswith("material"), b["config"].get("split_form"))
        traffic = json.load(open(TRAFFIC_FILE))[key]

    def rows_of(d, name):
        out = []
        import gzip
        for f in glob.glob(os.path.join(run_dir, d, "**", name), recursive=True) + glob.glob(
                os.path.join(run_dir, d, "**", name + ".gz"), recursive=True):
            out += list(csv.DictReader(gzip.open(f, "rt") if f.endswith(".gz") else open(f)))
        return out

    def q(v, f):
        v = sorted(v)
        return v[min(len(v) - 1, int(f * len(v)))]

    def short(name):
        name = re.sub(r"\(void const\*.*$", "", name)
        return name if len(name) < 90 else name[:87] + "..."

    trace = rows_of("trace", "*kernel_trace.csv")
    groups = {}
    for r in trace:
        n = r["Kernel_Name"]
        if "rlca::" in n:
            k = short(n)
        elif "copyBuffer" in n:
            k = "copy (`__amd_rocclr_copyBuffer`, grid %s)" % r["Grid_Size_X"]
        elif "spin_kernel" in n:
            k = "empty kernel (`torch.cuda._sleep`)"
        else:
            continue
        groups.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    # the calibration copy: the copy grid with the most dispatches
    copies = sorted((k for k in groups if k.startswith("copy")), key=lambda k: -len(groups[k]))
    for k in copies[1:]:
        del groups[k]
    busy = {}
    for r in rows_of("busy", "*counter_collection.csv"):
        if "rlca::" in r["Kernel_Name"]:
            busy.setdefault((short(r["Kernel_Name"]), r["Counter_Name"]), []).append(
                float(r["Counter_Value"]))

    rf, kb, fl, cp, sp = (b["roofline"], b.get("kernel_body"), b.get("launch_floor"),
                          b.get("copy_ceiling"), b.get("step_us_spread"))
    L = b["config"]["launches_per_step"]
    d = "<run>"
    o = " ".join(opts)
    lines = ["# librlca, workload `%s`%s" % (b["config"]["workload"], {
                 "plain": ""}.get(b["config"]["entry"], " (%s)" % b["config"]["entry"])), "",
             "MI355X, one GPU: %d x %d %s inputs, %d launch%s per step." % (
                            b["config"]["num_envs"], b["config"]["T"],
                            b["config"]["input_dtype"], L, "" if L == 1 else "es"), "",
             "Commands (repository root on the GPU box; `<run>` is a scratch directory):", "",
             "```"]
    for _, c in PROFILE_COMMANDS:
        lines.append(c.format(opts=o, d=d))
    lines += ["```", "",
              "## Per-launch time, unprofiled (the bench line)", "",
              "| quantity | median | p10 | p90 |", "|---|---|---|---|"]
    if sp:
        per = 1e0 / L
        lines.append("| library, back to back: µs per launch over %d blocks of %d steps (%s) "
                     "| %.3f | %.3f | %.3f |" % (sp["blocks"], sp["steps_per_block"],
                                                 b["config"]["timing"], sp["median"] * per,
                                                 sp["p10"] * per, sp["p90"] * per))
    if kb:
        lines.append("| kernel body, µs: first wavefront's start to the last wavefront's "
                     "completed stores (instrumented build, %d samples, %d wavefronts) "
                     "| %.3f | %.3f | %.3f |" % (kb["samples"], kb["wavefronts"],
                                                 kb["median_us"], kb["p10_us"], kb["p90_us"]))
    lines += ["", "| quantity | value |", "|---|---|",
              "| timed region: µs per step (K = %d) | %.3f |" % (b["steps"],
                                                                  b["ms_per_step"] * 1e3),
              "| µs per launch | %.3f |" % rf["avg_launch_us"],
              "| algorithmic bytes per launch | %d |" % rf["algorithmic_bytes_per_launch"],
              "| achieved (algorithmic bytes / µs per launch) | %.0f GB/s, %.1f%% of 8 TB/s |"
              % (rf["achieved"], 100 * rf["frac"])]
    if rf.get("kernel_only_frac"):
        lines.append("| kernel-only (algorithmic bytes / kernel body) | %.0f GB/s, %.1f%% |"
                     % (rf["kernel_only_frac"] * HBM_PEAK_GBPS, 100 * rf["kernel_only_frac"]))
    if fl:
        lines.append("| launch floor: an almost empty kernel, µs per launch | %.3f |"
                     % fl["avg_launch_us"])
    if cp:
        lines.append("| copy ceiling: torch copy of %d bytes (half read, half written), µs per "
                     "launch | %.3f (%.0f GB/s) |" % (cp["bytes_per_launch"], cp["avg_launch_us"],
                                                      cp["GBps"]))
    sc = b.get("stream_ceiling")
    if sc:
        lines.append("| streaming ceiling: the same byte mix streamed with no recurrence "
                     "(libstream_ceiling.so, best of 9 launch shapes), µs per step | %.3f "
                     "(%.0f GB/s) |" % (sc["step_us"], sc["GBps"]))
        lines.append("| this call's speed relative to the streaming ceiling | %.1f%% |"
                     % (100 * rf["frac_of_stream_ceiling"]))
    lines += ["", "## rocprofv3 kernel trace (durations of single dispatches, ns)", "",
              "The timed region of the traced run is one HIP graph replay of 2000 steps. "
              "The tracer takes each dispatch alone, so a duration here is one launch's "
              "latency from the command processor's start of the dispatch to its "
              "end-of-kernel signal, with no overlap with the launches before and after "
              "it: for a short kernel it is longer than its share of a back-to-back "
              "stream, and so are the copy and empty kernels of the same run.", "",
              "| kernel | dispatches | median | p10 | p90 |", "|---|---|---|---|---|"]
    for k, v in sorted(groups.items(), key=lambda kv: -len(kv[1])):
        lines.append("| %s | %d | %d | %d | %d |" % (k, len(v), q(v, 0.5), q(v, 0.1), q(v, 0.9)))
    if busy:
        lines += ["", "## Shader-engine busy time (rocprofv3 --pmc SQ_BUSY_CYCLES SQ_WAVES)", "",
                  "SQ_BUSY_CYCLES counts, per shader engine, the cycles in which any "
                  "wavefront of the dispatch is resident; the sum over the %d engines / %d "
                  "is the mean engine's busy time, at the %.1f GHz peak clock a lower bound "
                  "of the kernel's time with waves on the GPU." % (SE_COUNT, SE_COUNT,
                                                                   SCLK_GHZ), "",
                  "| kernel | wavefronts | busy cycles per engine | µs at %.1f GHz |" % SCLK_GHZ,
                  "|---|---|---|---|"]
        for (k, c), v in sorted(busy.items()):
            if c != "SQ_BUSY_CYCLES":
                continue
            waves = statistics.median(busy.get((k, "SQ_WAVES"), [0]))
            per_se = statistics.median(v) / SE_COUNT
            lines.append("| %s | %d | %.0f | %.3f |" % (k, waves, per_se,
                                                         per_se / SCLK_GHZ / 1e3))
    if traffic is None:
        with open(out_md, "w") as f:
            f.write("\n".join(lines + ["", "(No counter runs for this workload.)", ""]))
        print("wrote", out_md)
        return
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              "| quantity | value |", "|---|---|"]
    for k, v in traffic["fetch_kib_per_launch"].items():
        lines.append("| FETCH_SIZE per dispatch (KiB), %s | %.1f |" % (short(k), v))
    for k, v in traffic["write_kib_per_launch"].items():
        lines.append("| WRITE_SIZE per dispatch (KiB), %s | %.1f |" % (short(k), v))
    lines += ["| calibration copy bytes read / written | %d / %d |"
              % (traffic["copy_bytes_read"], traffic["copy_bytes_written"]),
              "| its FETCH_SIZE / WRITE_SIZE (KiB) | %.1f / %.1f |"
              % (traffic["copy_fetch_kib"], traffic["copy_write_kib"]),
              "| scale: FETCH / WRITE | %.3f / %.3f |" % (traffic["fetch_scale"],
                                                          traffic["write_scale"]),
              "| HBM bytes per launch (scaled; mean over the library's kernels) | %.0f |"
              % traffic["bytes_per_launch"],
              "| algorithmic bytes per launch | %d |" % traffic["algorithmic_bytes_per_launch"],
              "| ratio | %.3f |" % (traffic["bytes_per_launch"]
                                   / traffic["algorithmic_bytes_per_launch"]),
              "| kernel source hash | `%s` |" % traffic["kernel_source_hash"], ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("wrote", out_md)


def host_threads():
    """Host cores this process may run on, capped at 16 (one GPU's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Timed regions of at most this many steps are timed as eager launches
# queued behind a spin kernel; longer ones as one HIP graph replay.  A graph
# replay carries a fixed cost of about 8 us on this runtime, which 20 steps
# do not amortize; the queue of a stream holds a few thousand launches.
QUEUED_MAX_STEPS = 1000
MAX_SETS = 1024
TIMING_DESC = {
    "queued": "K eager launches queued behind a spin kernel (the GPU runs them back to back; "
              "events bracket exactly the K launches)",
    "graph": "HIP graph replay of K launches",
    "eager": "eager launches from Python",
}


def spin_rate(stream):
    """Cycles of torch.cuda._sleep per microsecond on this GPU."""
    import torch
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(2_000_000)
    b.record(stream)
    b.synchronize()
    return 2e6 / (a.elapsed_time(b) * 1e3)


def make_timed(fn, K, mode, stream, rate):
    """A function that runs K launches, fn(i) for K consecutive values of i,
    between two events on `stream`, with the device synchronized before and
    after, and returns the average microseconds per step.  i keeps counting
    from one call to the next, so that fn can rotate through buffer sets
    without any block reusing the sets of the block before (which the 256 MB
    Infinity Cache could still hold).

    queued: the launches are enqueued while a spin kernel (torch.cuda._sleep,
    bounded) keeps the GPU busy, long enough to cover the host's enqueue
    time, so the GPU runs the K launches back to back and the start event is
    taken when the spin ends; graph: one replay of a HIP graph of the K
    launches (captured and replayed once untimed here; every replay repeats
    the same K values of i); eager: plain launches."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    if mode == "graph":
        dev = torch.cuda.current_device()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(K):
                    fn(i)
        torch.cuda.synchronize()
        g.replay()  # untimed: the first replay uploads the graph
        torch.cuda.synchronize()

        def once():
            torch.cuda.synchronize()
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / K
        once.graph = g
        return once
    ctr = [0]
    host_us = 0.0
    if mode == "queued":
        n = min(K, 50)
        t0 = time.perf_counter()
        for i in range(n):
            fn(ctr[0] + i)
        host_us = (time.perf_counter() - t0) / n * 1e6
        ctr[0] += n
        torch.cuda.synchronize()

    def once():
        torch.cuda.synchronize()
        if mode == "queued":
            torch.cuda._sleep(int((2.0 * K * host_us + 300.0) * rate))
        i0 = ctr[0]
        a.record(stream)
        for i in range(i0, i0 + K):
            fn(i)
        b.record(stream)
        ctr[0] = i0 + K
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / K
    return once


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only; multi-GPU runs are not part of this "
              "library (rows shard across GPUs with no communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import reverse_linear_recurrence_amd as rl
    from reverse_linear_recurrence_amd.synth import WORKLOADS, fp32_param, make_workload

    if not os.path.exists(rl.lib_path()):
        from reverse_linear_recurrence_amd import build as hip_build
        hip_build.build()
    rl.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    w = WORKLOADS[args.workload]
    N, T = w.num_envs, w.T
    gamma, lam = fp32_param(w.gamma), fp32_param(w.lam)
    clips = {k: fp32_param(v) for k, v in w.clips.items()}
    dev = torch.device("cuda:0")
    host = make_workload(w)
    set_bytes = sum(x.numel() * x.element_size() for x in host.values()) + 2 * 4 * N * T
    # (at most MAX_SETS: a tiny batch would otherwise take tens of thousands of
    # sets, and as many untimed pre-touch calls; such a batch is latency-bound
    # and sits in the caches whatever the rotation)
    R = max(2, min(MAX_SETS, int(np.ceil(args.rotate_mb * 2 ** 20 / set_bytes))))
    print("workload %s: %d x %d %s, %d rotating sets of %.2f MB" %
          (w.name, N, T, w.dtype, R, set_bytes / 2 ** 20), file=sys.stderr, flush=True)

    # Window calls: a seeded per-row carry entering every window.
    carry_in = torch.from_numpy(np.random.Generator(np.random.PCG64(w.seed + 1))
                                .standard_normal(N).astype(np.float32))
    sets = []
    for _ in range(R):
        d = {k: v.to(dev) for k, v in host.items()}
        d["_o0"] = torch.empty(N, T, dtype=torch.float32, device=dev)
        d["_o1"] = torch.empty(N, T, dtype=torch.float32, device=dev)
        d["_o2"] = torch.empty(N, T, dtype=torch.float32, device=dev)
        d["_cin"] = carry_in.to(dev)
        d["_cout"] = torch.empty(N, dtype=torch.float32, device=dev)
        d["_cmap"] = torch.empty(N, 2, dtype=torch.float32, device=dev)
        d["_cout2"] = torch.empty(N, dtype=torch.float32, device=dev)
        d["_cmap2"] = torch.empty(N, 2, dtype=torch.float32, device=dev)
        sets.append(d)
    torch.cuda.synchronize()
    rl.rlca_set_variant(args.variant)
    split_segments = 1
    workspace = None
    if args.split:
        if w.algo in ("retrace_probs", "vtrace_probs", "vtrace+retrace"):
            print("--split: the workload must be one call of the scan family", file=sys.stderr)
            sys.exit(2)
        split_segments = rl.rlca_split_segments(N, T)
        workspace = rl.split_workspace(N, T, dev)
    if args.no_chain:
        rl.rlca_set_chained(False)

    def window_step(d):
        if args.window:
            c = dict(carry_in=d["_cin"], carry_out=d["_cout"], carry_map=d["_cmap"])
        else:  # --split alone: the plain call's results through the window form
            c = dict(with_carry_out=False, with_map=False)
        c["workspace"] = workspace
        if w.algo == "gae":
            rl.rlca_gae_chunk(d["rewards"], d["values"], d["terminated"], d.get("truncated"),
                              d.get("trunc_values"), gamma=gamma, lam=lam, advantages=d["_o0"],
                              targets=d["_o1"], **c)
        elif w.algo == "td_lambda":
            rl.rlca_td_lambda_chunk(d["rewards"], d["values"], d["terminated"],
                                    d.get("truncated"), d.get("trunc_values"), gamma=gamma,
                                    lam=lam, out=d["_o0"], **c)
        elif w.algo == "returns":
            rl.rlca_returns_chunk(d["rewards"], d["terminated"], gamma=gamma, out=d["_o0"], **c)
        elif w.algo == "eligibility":
            rl.rlca_eligibility_trace_chunk(d["rewards"], d["terminated"], d.get("truncated"),
                                            gamma=gamma, lam=lam, out=d["_o0"], **c)
        elif w.algo == "cumsum":
            rl.rlca_episodic_cumsum_chunk(d["rewards"], d["terminated"], d.get("truncated"),
                                          out=d["_o0"], **c)
        elif w.algo == "vtrace+retrace":
            rl.rlca_vtrace_chunk(d["rewards"], d["values"], d["log_rhos"], d["terminated"],
                                 gamma=gamma, lam=lam, vs=d["_o0"], pg_advantages=d["_o1"],
                                 **clips, **c)
            rl.rlca_retrace_chunk(d["rewards"], d["q_taken"], d["exp_q_next"], d["log_rhos"],
                                  d["terminated"], gamma=gamma, lam=lam, c_bar=clips["c_bar"],
                                  out=d["_o2"], carry_in=d["_cin"], carry_out=d["_cout2"],
                                  carry_map=d["_cmap2"])
        else:
            raise ValueError(w.algo)

    mat_ws = None
    if args.materialized:
        if args.window or args.split or w.algo not in ("returns", "gae", "td_lambda",
                                                       "vtrace+retrace"):
            print("--materialized: a plain call of returns, GAE, TD(lambda), V-trace or "
                  "Retrace", file=sys.stderr)
            sys.exit(2)
        mat_ws = torch.empty(rl.rlca_materialized_workspace_bytes(N, T) // 4,
                             dtype=torch.float32, device=dev)

    def materialized_step(d):
        kw = dict(workspace=mat_ws)
        if w.algo == "gae":
            rl.rlca_gae_materialized(d["rewards"], d["values"], d["terminated"],
                                     d.get("truncated"), d.get("trunc_values"), gamma=gamma,
                                     lam=lam, advantages=d["_o0"], targets=d["_o1"], **kw)
        elif w.algo == "td_lambda":
            rl.rlca_td_lambda_materialized(d["rewards"], d["values"], d["terminated"],
                                           d.get("truncated"), d.get("trunc_values"),
                                           gamma=gamma, lam=lam, out=d["_o0"], **kw)
        elif w.algo == "returns":
            rl.rlca_returns_materialized(d["rewards"], d["terminated"], gamma=gamma,
                                         out=d["_o0"], **kw)
        else:
            rl.rlca_vtrace_materialized(d["rewards"], d["values"], d["log_rhos"],
                                        d["terminated"], gamma=gamma, lam=lam, vs=d["_o0"],
                                        pg_advantages=d["_o1"], **clips, **kw)
            rl.rlca_retrace_materialized(d["rewards"], d["q_taken"], d["exp_q_next"],
                                         d["log_rhos"], d["terminated"], gamma=gamma, lam=lam,
                                         c_bar=clips["c_bar"], out=d["_o2"], **kw)

    def step(d):
        if args.materialized:
            materialized_step(d)
            return
        if args.window or args.split:
            window_step(d)
            return
        if w.algo == "retrace_probs":
            rl.rlca_retrace_probs(d["rewards"], d["q_values"], d["actions"], d["log_pi"],
                                  d["log_mu"], d["terminated"], d.get("truncated"),
                                  d.get("trunc_eq"), gamma=gamma, lam=lam, out=d["_o0"], **clips)
            return
        if w.algo == "vtrace_probs":
            rl.rlca_vtrace_probs(d["rewards"], d["values"], d["actions"], d["log_pi"],
                                 d["log_mu"], d["terminated"], d.get("truncated"),
                                 d.get("trunc_values"), gamma=gamma, lam=lam, vs=d["_o0"],
                                 pg_advantages=d["_o1"], **clips)
            return
        if w.algo == "gae":
            rl.rlca_gae(d["rewards"], d["values"], d["terminated"], d.get("truncated"),
                        d.get("trunc_values"), gamma=gamma, lam=lam, advantages=d["_o0"],
                        targets=d["_o1"])
        elif w.algo == "td_lambda":
            rl.rlca_td_lambda(d["rewards"], d["values"], d["terminated"], d.get("truncated"),
                              d.get("trunc_values"), gamma=gamma, lam=lam, out=d["_o0"])
        elif w.algo == "returns":
            rl.rlca_returns(d["rewards"], d["terminated"], gamma=gamma, out=d["_o0"])
        elif w.algo == "eligibility":
            rl.rlca_eligibility_trace(d["rewards"], d["terminated"], d.get("truncated"),
                                      gamma=gamma, lam=lam, out=d["_o0"])
        elif w.algo == "cumsum":
            rl.rlca_episodic_cumsum(d["rewards"], d["terminated"], d.get("truncated"),
                                    out=d["_o0"])
        elif w.algo == "vtrace+retrace":
            rl.rlca_vtrace(d["rewards"], d["values"], d["log_rhos"], d["terminated"], gamma=gamma,
                           lam=lam, vs=d["_o0"], pg_advantages=d["_o1"], **clips)
            rl.rlca_retrace(d["rewards"], d["q_taken"], d["exp_q_next"], d["log_rhos"],
                            d["terminated"], gamma=gamma, lam=lam, c_bar=clips["c_bar"],
                            out=d["_o2"])
        else:
            raise ValueError(w.algo)

    # ---- parity of the timed configuration against the oracle (set 0)
    import oracle
    step(sets[0])
    torch.cuda.synchronize()
    launches_per_call = rl.rlca_last_launches()  # of the step's (last) library call
    segments_per_row = rl.rlca_last_segments()
    win = dict(carry_in=carry_in, chunk=True) if args.window else {}
    if args.window and w.algo in ("returns",):
        win = dict(chunk=True)
    if w.algo in ("retrace_probs", "vtrace_probs") and args.window:
        print("the policy-table calls have no window form", file=sys.stderr)
        sys.exit(2)
    if w.algo == "retrace_probs":
        ref = oracle.retrace_probs(host["rewards"], host["q_values"], host["actions"],
                                   host["log_pi"], host["log_mu"], host["terminated"],
                                   host.get("truncated"), host.get("trunc_eq"), gamma=gamma,
                                   lam=lam, **clips)
        outs = (sets[0]["_o0"],)
    elif w.algo == "vtrace_probs":
        ref = oracle.vtrace_probs(host["rewards"], host["values"], host["actions"],
                                  host["log_pi"], host["log_mu"], host["terminated"],
                                  host.get("truncated"), host.get("trunc_values"), gamma=gamma,
                                  lam=lam, **clips)
        outs = (sets[0]["_o0"], sets[0]["_o1"])
    elif w.algo == "gae":
        ref = oracle.gae(host["rewards"], host["values"], host["terminated"],
                         host.get("truncated"), host.get("trunc_values"), gamma=gamma, lam=lam,
                         **win)
        outs = (sets[0]["_o0"], sets[0]["_o1"])
    elif w.algo == "td_lambda":
        ref = oracle.td_lambda(host["rewards"], host["values"], host["terminated"],
                               host.get("truncated"), host.get("trunc_values"), gamma=gamma,
                               lam=lam, **win)
        outs = (sets[0]["_o0"],)
    elif w.algo == "returns":
        ref = oracle.returns(host["rewards"], host["terminated"],
                             bootstrap=carry_in if args.window else None, gamma=gamma, **win)
        outs = (sets[0]["_o0"],)
    elif w.algo == "eligibility":
        ref = oracle.eligibility_trace(host["rewards"], host["terminated"], host.get("truncated"),
                                       carry_in if args.window else None, gamma=gamma, lam=lam,
                                       **({"chunk": True} if args.window else {}))
        outs = (sets[0]["_o0"],)
    elif w.algo == "cumsum":
        ref = oracle.episodic_cumsum(host["rewards"], host["terminated"], host.get("truncated"),
                                     carry_in if args.window else None,
                                     **({"chunk": True} if args.window else {}))
        outs = (sets[0]["_o0"],)
    else:
        vs = oracle.vtrace(host["rewards"], host["values"], host["log_rhos"], host["terminated"],
                           gamma=gamma, lam=lam, **clips, **win)
        qr = oracle.retrace(host["rewards"], host["q_taken"], host["exp_q_next"],
                            host["log_rhos"], host["terminated"], gamma=gamma, lam=lam,
                            c_bar=clips["c_bar"], **win)
        outs = (sets[0]["_o0"], sets[0]["_o1"], sets[0]["_o2"])
        if args.window:
            ref = (vs[0], vs[1], vs[2], vs[3], qr[0], qr[1], qr[2])
            outs = (sets[0]["_o0"], sets[0]["_o1"], sets[0]["_cout"], sets[0]["_cmap"],
                    sets[0]["_o2"], sets[0]["_cout2"], sets[0]["_cmap2"])
        else:
            ref = (vs[0], vs[1], qr)
    if not isinstance(ref, tuple):
        ref = (ref,)
    if args.window and w.algo != "vtrace+retrace":
        # outputs, then carry_out [N] and carry map [N, 2]
        outs = outs + (sets[0]["_cout"], sets[0]["_cmap"])
    per_output = [float(np.max(np.abs(o.double().cpu().numpy() - r)) / np.max(np.abs(r)))
                  for o, r in zip(outs, ref)]
    parity = max(per_output)
    tol = 1e-2 if w.dtype == "bf16" else 1e-4
    variant = rl.rlca_last_variant()
    print("parity max|err|/max|ref| = %.3g (tolerance %g), variant %d" % (parity, tol, variant),
          file=sys.stderr, flush=True)
    if not parity <= tol:
        print("parity check failed", file=sys.stderr)
        sys.exit(1)

    # ---- warmup, then K timed steps.  Before the W warmup steps, one
    # untimed call per rotation set: a training loop calls the library on
    # buffers it has used before, so every set is read once by the kernel
    # (its pages mapped in the GPU's address translation caches) before any
    # step is timed; the sets stay too large in total for the Infinity Cache.
    stream = torch.cuda.current_stream(dev)
    for d in sets:
        step(d)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    K = args.steps
    mode = args.timing
    if mode == "auto":
        mode = "eager" if args.no_graph else ("queued" if K <= QUEUED_MAX_STEPS else "graph")
    rate = spin_rate(stream) if mode == "queued" else None
    # (every block, warmup included, moves on through the R rotating sets)
    once = make_timed(lambda i: step(sets[(args.warmup + i) % R]), K, mode, stream, rate)
    torch.cuda.synchronize()
    ms_per_step = once() / 1e3  # the timed region: exactly K steps
    timing = TIMING_DESC[mode]

    # ---- spread: the same K steps timed again, each block alone, for the
    # median / p10 / p90 of the per-step average over blocks.
    spread = None
    if args.spread_replays > 0:
        per = sorted(once() for _ in range(args.spread_replays))

        def pick(f):
            return per[min(len(per) - 1, int(f * len(per)))]
        spread = {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9),
                  "blocks": len(per), "steps_per_block": K}

    # ---- floors, timed the same way: a plain copy kernel (torch's) moving
    # the same number of bytes (half read, half written), the practical
    # ceiling for one launch of this size, and an almost empty kernel
    # (torch.cuda._sleep(0)), the per-launch cost of the runtime and the
    # command processor.  Under --no-graph the copy also serves as the
    # known-size calibration kernel of the counter runs (see --summarize-pmc).
    copy = floor = None
    if not args.no_copy_ceiling:
        half = algorithmic_bytes(w, N, T, args.window) // launches_per_step_of(w) // 2 // 16 * 16
        RC = max(2, min(MAX_SETS, int(np.ceil(args.rotate_mb * 2 ** 20 / (2 * half)))))
        bufs = [(torch.empty(half // 4, dtype=torch.float32, device=dev),
                 torch.empty(half // 4, dtype=torch.float32, device=dev)) for _ in range(RC)]
        for a, _ in bufs:
            a.fill_(1.0)
        KC = min(K, QUEUED_MAX_STEPS)
        mode_c = "eager" if mode == "eager" else ("queued" if rate is not None else "graph")
        torch.cuda.synchronize()
        cus = make_timed(lambda i: bufs[i % RC][1].copy_(bufs[i % RC][0]), KC, mode_c, stream,
                         rate)()
        copy = {"bytes_per_launch": 2 * half, "avg_launch_us": cus,
                "GBps": 2 * half / (cus * 1e-6) / 1e9, "kernel": "torch copy_ (float32)",
                "timing": TIMING_DESC[mode_c]}
        del bufs
        fus = make_timed(lambda i: torch.cuda._sleep(0), KC, mode_c, stream, rate)()
        floor = {"avg_launch_us": fus, "kernel": "torch.cuda._sleep(0), an almost empty kernel",
                 "timing": TIMING_DESC[mode_c]}
    # ---- streaming ceiling: the workload's byte mix (the arrays the method
    # must read and write, N*T elements each) streamed by a kernel with no
    # recurrence (libstream_ceiling.so), timed the same way over a few launch
    # shapes; the best is the practical ceiling of one launch of this size.
    ceiling = None
    mixes = stream_mixes(w)
    from reverse_linear_recurrence_amd import build as hip_build
    if (not args.no_copy_ceiling and mixes and not args.window
            and os.path.exists(hip_build.LIB_CEILING)):
        import ctypes
        clib = ctypes.CDLL(hip_build.LIB_CEILING)
        clib.stream_ceiling.restype = ctypes.c_int
        E = N * T
        KC = min(K, QUEUED_MAX_STEPS)
        mode_c = "eager" if mode == "eager" else ("queued" if rate is not None else "graph")
        per_launch, shapes = [], []
        for nf, nh, nb, no in mixes:
            mix_bytes = E * (4 * nf + 2 * nh + nb + 4 * no)
            RS = max(2, min(MAX_SETS, int(np.ceil(args.rotate_mb * 2 ** 20 / mix_bytes))))
            P4 = ctypes.c_void_p * 4
            csets = []
            for _ in range(RS):
                arrs = ([torch.empty(E, dtype=torch.float32, device=dev) for _ in range(nf)],
                        [torch.zeros(E, dtype=torch.int16, device=dev) for _ in range(nh)],
                        [torch.zeros(E, dtype=torch.uint8, device=dev) for _ in range(nb)],
                        [torch.empty(E, dtype=torch.float32, device=dev) for _ in range(no)])
                for a in arrs[0]:
                    a.fill_(1.0)
                ptrs = [P4(*([x.data_ptr() for x in group] + [None] * (4 - len(group))))
                        for group in arrs]
                csets.append((ptrs, arrs))
            best = None
            for u in (1, 2, 4):
                for blk in (256, 512, 1024):
                    def cstep(i, u=u, blk=blk):
                        pt = csets[i % RS][0]
                        rc = clib.stream_ceiling(nf, nh, nb, no, pt[0], pt[1], pt[2], pt[3],
                                                 ctypes.c_int64(E), u, blk, ctypes.c_void_p(
                                                     torch.cuda.current_stream().cuda_stream))
                        if rc != 0:
                            raise RuntimeError("stream_ceiling failed (%d)" % rc)
                    for i in range(RS):
                        cstep(i)
                    torch.cuda.synchronize()
                    us = make_timed(cstep, KC, mode_c, stream, rate)()
                    if best is None or us < best[0]:
                        best = (us, u, blk)
            per_launch.append(best[0])
            shapes.append({"slots_per_thread": best[1], "workgroup": best[2],
                           "bytes_per_launch": mix_bytes})
            del csets
        torch.cuda.synchronize()
        ceil_us = sum(per_launch)
        ceiling = {"step_us": ceil_us, "per_launch_us": per_launch, "launches": shapes,
                   "GBps": algorithmic_bytes(w, N, T) / (ceil_us * 1e-6) / 1e9,
                   "kernel": "stream_ceiling (libstream_ceiling.so): the workload's byte mix "
                             "with non-temporal loads and stores and no recurrence; best of "
                             "3 x 3 launch shapes",
                   "timing": TIMING_DESC[mode_c]}
    # ---- kernel body: the same steps through the instrumented build of the
    # library (librlca_timed.so: same sources, plus per-wavefront wall-clock
    # stamps at entry and once all loads and stores are done).  For the last
    # launch of each block of steps, the body is max(end) - min(start): the
    # kernel's time on the GPU from its first wavefront's start to its last
    # wavefront's completed stores, without the runtime's per-launch cost.
    body = None
    if (args.body_blocks > 0 and mode != "eager" and not args.materialized
            and os.path.exists(rl.TIMED_LIB_PATH)):
        with rl.use_library(rl.TIMED_LIB_PATH):
            # the per-thread settings of the timed build: the same as the library's
            rl.rlca_set_chained(not args.no_chain)
            rl.rlca_set_variant(args.variant)
            for i in range(min(args.warmup, 50)):
                step(sets[i % R])
            torch.cuda.synchronize()
            KB = min(K, 200)
            mode_b = "queued" if rate is not None else "graph"
            once_b = make_timed(lambda i: step(sets[i % R]), KB, mode_b, stream, rate)
            bodies, waves_us, spreads, steps_b = [], [], [], []
            for _ in range(args.body_blocks):
                steps_b.append(once_b())
                st = rl.rlca_timestamps().astype(np.int64)
                if st.shape[0] == 0:
                    break  # a kernel without stamps
                bodies.append(float(st[:, 1].max() - st[:, 0].min()) * 0.01)
                waves_us.append(float(np.median(st[:, 1] - st[:, 0])) * 0.01)
                spreads.append(float(st[:, 0].max() - st[:, 0].min()) * 0.01)
            n_waves = int(st.shape[0])
        bodies.sort()

        def q(v, f):
            v = sorted(v)
            return v[min(len(v) - 1, int(f * len(v)))]
        if bodies:
            body = {"median_us": q(bodies, 0.5), "p10_us": q(bodies, 0.1),
                    "p90_us": q(bodies, 0.9), "samples": len(bodies), "wavefronts": n_waves,
                    "wave_median_us": q(waves_us, 0.5), "start_spread_us": q(spreads, 0.5),
                    "instrumented_step_us": q(steps_b, 0.5),
                    "method": "librlca_timed.so (the same sources with per-wavefront 100 MHz "
                              "wall-clock stamps); last launch of each of %d blocks of %d "
                              "steps, %s" % (len(bodies), KB, TIMING_DESC[mode_b])}
    launches_per_step = launches_per_step_of(w) * launches_per_call
    split_form = None
    if args.split:
        split_form = ("unsplit" if segments_per_row == 1 else
                      "three-launch" if launches_per_call == 3 else "chained")
        split_segments = segments_per_row
    env_steps = N * T
    value = env_steps / (ms_per_step * 1e-3)
    bytes_per_step = algorithmic_bytes(w, N, T, args.window)
    tkey = traffic_key(w.name, args.window, args.materialized, split_form)
    achieved = bytes_per_step / (ms_per_step * 1e-3) / 1e9

    # ---- HBM traffic from the committed counter runs, if they match this kernel
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        entry = tr.get(tkey)
        if entry and entry.get("kernel_source_hash") == kernel_source_hash(kernel_family(tkey)):
            traffic = entry.get("bytes_per_launch")

    # ---- CPU oracle on the host cores (bounded sample of the same workload):
    # the fp64 C oracle over the whole batch, first on one thread, then on
    # every host core this process may use (at most 16, one GPU's share), one
    # contiguous slice of rows per OpenMP thread (oracle_rows.c).  Each leg
    # repeats whole batches until its time budget is spent.
    cpu = None
    if args.cpu_seconds > 0:
        params = dict(gamma=gamma, lam=lam, **clips)
        algos = {"vtrace+retrace": ("vtrace", "retrace"), "eligibility": ("eligibility_trace",),
                 "cumsum": ("episodic_cumsum",)}.get(w.algo, (w.algo,))

        def runner(threads):
            runs = [oracle.batch_runner(a, host, params, threads) for a in algos]

            def run():
                for r in runs:
                    r()
            return run

        def timed(run, budget):
            """Whole batches until the time budget is spent and at least five
            ran (the first call, untimed, touches the memory).  Returns the
            repetitions, the time spent and each batch's time, sorted."""
            run()
            each, t0 = [], time.perf_counter()
            while True:
                t1 = time.perf_counter()
                run()
                each.append(time.perf_counter() - t1)
                spent = time.perf_counter() - t0
                if spent >= budget and len(each) >= 5:
                    return len(each), spent, sorted(each)

        reps, cpu_s, each = timed(runner(1), args.cpu_seconds / 2)
        cpu = {"value": env_steps * reps / cpu_s, "unit": "env-steps/s", "cores": 1,
               "kind": "oracle",
               "sample": "the whole %dx%d batch, %d repetitions (%.1f s), single-threaded "
                         "fp64 C oracle" % (N, T, reps, cpu_s),
               "median_ms_per_batch": each[len(each) // 2] * 1e3,
               "cpu_model": cpu_model()}
        nthreads = host_threads()
        if nthreads > 1:
            reps_m, cpu_m, each_m = timed(runner(nthreads), args.cpu_seconds / 2)
            cpu["all_cores"] = {
                "value": env_steps * reps_m / cpu_m, "unit": "env-steps/s", "cores": nthreads,
                "sample": "the whole %dx%d batch, %d repetitions (%.1f s), the same oracle on "
                          "%d OpenMP threads, one contiguous slice of rows each"
                          % (N, T, reps_m, cpu_m, nthreads),
                "median_ms_per_batch": each_m[len(each_m) // 2] * 1e3,
                "speedup_over_one_thread": (reps_m / cpu_m) / (reps / cpu_s)}

    meta_dir = os.environ.get("RLCA_BENCH_META_DIR")
    if meta_dir:
        os.makedirs(meta_dir, exist_ok=True)
        with open(os.path.join(meta_dir, "bench_meta.json"), "w") as f:
            json.dump({"workload": tkey, "algorithmic_bytes_per_launch":
                       bytes_per_step / launches_per_step,
                       "copy_bytes_per_launch": copy["bytes_per_launch"] if copy else None}, f)

    out = {
        "metric": METRIC if w.name == "gae_4096x128" else "env-steps/sec, %s" % w.name,
        "value": value,
        "unit": "env-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "num_envs": N, "T": T, "input_dtype": w.dtype,
                   "gamma": w.gamma, "lam": w.lam, "p_term": w.p_term, "p_trunc": w.p_trunc,
                   "seed": w.seed, "rotation_sets": R, "timing": timing,
                   "before_warmup": "one untimed call per rotation set",
                   "launches_per_step": launches_per_step, "variant": variant,
                   "split_segments": split_segments, "split_form": split_form,
                   "entry": "window (carry in; carry and carry map out)" if args.window
                   else ("materialized doubling scan (2 + ceil(log2 T) launches through HBM)"
                         if args.materialized else "plain")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": bytes_per_step / launches_per_step,
                     "avg_launch_us": ms_per_step * 1e3 / launches_per_step,
                     "kernel_body_us": body["median_us"] if body else None,
                     "kernel_only_frac": (bytes_per_step / launches_per_step
                                          / (body["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS)
                     if body and launches_per_step == 1 else None,
                     "frac_of_stream_ceiling": (ceiling["step_us"] / (ms_per_step * 1e3))
                     if ceiling else None},
        "kernel_body": body,
        "cpu_baseline": cpu,
        "copy_ceiling": copy,
        "stream_ceiling": ceiling,
        "launch_floor": floor,
        "step_us_spread": spread,
        "parity_max_rel_err": parity,
        "parity": {"max_rel_err_per_output": per_output, "tolerance": tol,
                   "pass": parity <= tol},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
