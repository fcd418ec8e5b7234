"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole path over one batch: each sequence's new token is
appended into its block (slot T[L / B] * B + L % B), and the fused score /
online-softmax / V pass runs over every sequence's physical blocks (stage 1),
followed by the merge of segments split between workers (stage 2); the step
attends over L + 1 tokens.  By default the step is one
paged_attn_decode_shared call (prepare: the new rows and the prefix each
sequence shares with the previous one; stage 1; stage 2), which reads blocks
that forked siblings share once; ``--call fused`` runs
paged_attn_decode_append and ``--call two-launch`` paged_kv_append_at then
paged_attn_decode instead.

The default workload is the largest one that fits one GPU: copy-on-write
parallel sampling, 128 prompts of 1024 tokens each forked into 4 siblings
that share the 64 prompt blocks and own private tails of 0 .. 63 tokens
(512 sequences, 40 query / 40 kv heads, head_dim 128, bf16 K/V in 16-token
blocks).

Timing (the stated protocol): W untimed warm-up steps; then the timed region
of exactly K steps, each preceded by writing a 1 GiB buffer (beyond L2 and
MALL, so every step starts with cold caches) and bracketed by HIP events on
the launch stream; the step time is the median over the K steps (min and
10th-90th percentiles reported).  After the timed region the same number of
flushed repetitions bracket stage 1 alone, for the roofline of that kernel,
and K steps run back to back (warm caches) for comparison.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--call shared|fused|two-launch]

prints one JSON line: logical KV GB/s of the step (sum(L+1) * 2 * kv_heads *
head_dim * 2 B per median step time; shared prompt blocks counted once per
sibling, as each sibling's attention reads them), the unique-byte rate
(every physical K/V row read counted once), the roofline of stage 1, the
fp64 CPU oracle timed on the host's cores, and in ``extra`` the flushed
steps of the other workloads, a paged-against-contiguous A/B, a plain
streaming-read probe, the copy-on-write block copy, the CPU-GPU swap and the
prompt pass.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, vendor figure
FLUSH_BYTES = 1 << 30
# Host cores one GPU of the box may use for worker pools.
HOST_CORES_PER_GPU = 16

# Prompt pass measured after the step: sequences, new tokens per sequence and
# tokens held (the chunk continues an earlier context), Llama-7B heads.
PREFILL_SHAPE = {"seqs": 4, "chunk": 1024, "context": 2048, "q_heads": 32, "kv_heads": 32, "head_dim": 128,
                 "block_size": 16}


def prefill_flops(seqs: int, chunk: int, context: int, q_heads: int, head_dim: int) -> int:
    """4 D flops per (query row, head, visible key): 2 D for the score and 2 D
    for the weighted V sum; the row at position p sees p + 1 keys."""
    first = context - chunk
    keys = chunk * (first + 1) + chunk * (chunk - 1) // 2  # sum of p + 1 over the chunk's positions
    return 4 * head_dim * q_heads * keys * seqs


METRIC = "paged decode attention: KV GB/s and % of MI355X HBM peak; seq-tokens/s"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_357_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("decode.hip", "decode_shared.hip", "decode_core.h",
                                                  "pkv_internal.h")]

WORKLOADS = {"llama7b-decode": 2, "tiny-f32": 1, "gqa-lognormal": 3, "cow-parallel-sampling": 4,
             "long-context": 5}
STAGE1_KERNELS = ("decode_shared_kernel", "decode_balanced_kernel", "decode_partitioned_kernel")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cow-parallel-sampling", choices=sorted(WORKLOADS))
    ap.add_argument("--call", default="shared", choices=["shared", "fused", "two-launch"],
                    help="entry point(s) of the step")
    ap.add_argument("--deal", default="shuffled", choices=["shuffled", "identity"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences in the CPU sample (0 = all)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the chosen workload only (no other workloads, A/B, probes, copy, swap, prompt pass)")
    ap.add_argument("--extra-reps", type=int, default=10, help="flushed repetitions per extra measurement")
    ap.add_argument("--cow-pairs", type=int, default=2048,
                    help="block pairs in the copy-on-write block copy timed after the step (0 = skip)")
    ap.add_argument("--swap-blocks", type=int, default=512,
                    help="blocks swapped out to pinned host memory and back after the step (0 = skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="launch one plain copy of this size (reference kernel for byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of this "
                         "workload's run with --copy-probe-mib into its traffic summary under profiles/")
    ap.add_argument("--write-traces", metavar="TRACE_DIR",
                    help="no GPU run: summarise a rocprofv3 --kernel-trace --stats output folder of this "
                         "workload's run into profiles/ (kernel, calls, mean / min / max duration)")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the copy probe in those runs")
    ap.add_argument("--write-pmc", nargs="+", metavar="DIR_OR_NAME",
                    help="no GPU run: rocprofv3 --pmc output folders, then a summary name; writes the mean per "
                         "dispatch of every counter of --pmc-kernel to profiles/NAME.txt")
    ap.add_argument("--pmc-kernel", default="prefill_kernel", help="kernel name pattern for --write-pmc")
    ap.add_argument("--pmc-command", default="python bench.py --prefill-only --steps 5",
                    help="the profiled command, recorded in the --write-pmc summary")
    ap.add_argument("--flush-sweep", action="store_true",
                    help="stage 1 of the workload after writing buffers of 0 .. 1024 MiB before each call "
                         "(median of 10 per size); prints one line and exits")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time the prompt pass alone (--steps flushed repetitions) and print its line")
    ap.add_argument("--wave-timing", action="store_true",
                    help="per-wave timing of the shared-prefix stage 1 (libpagedkv_timing.so, --steps flushed "
                         "calls of --workload); writes profiles/wave_timing_<workload>_shared.txt")
    return ap.parse_args()


class HipEvents:
    """Timing events of the HIP runtime already loaded in this process,
    recorded on a given stream (the one the kernels are launched on).  They
    are created with hipEventDisableSystemFence: recording one then costs no
    system-scope cache writeback and invalidation, which with default events
    adds several microseconds to every step and disturbs the work that
    follows.  Used only for timing; the host synchronises with the device
    before reading them."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, stream_ptr):
        import ctypes
        path = "libamdhip64.so.7"
        with open("/proc/self/maps") as f:  # the copy torch loaded
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.stream = ctypes.c_void_p(stream_ptr)
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            self.ev.append(e)

    def record(self, i):
        rc = self.hip.hipEventRecord(self.ev[i], self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, i, j):
        t = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(t), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(t.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "min_ms": float(a.min()), "p10_ms": float(np.percentile(a, 10)),
            "p90_ms": float(np.percentile(a, 90)), "reps": int(a.size)}


def kernel_sha() -> str:
    """Hash of the stage-1 kernel sources with comments and blank lines
    dropped, so that a counter summary stays valid across comment edits."""
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_file(workload: str, call: str) -> str:
    return os.path.join(PROFILES, f"decode_stage1_{workload}_{call}_traffic.txt")


def read_traffic(workload: str, call: str):
    """HBM bytes per stage-1 launch from the committed counter summary, or
    None when it is missing or was taken on a different kernel source."""
    path = traffic_file(workload, call)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_]+)\s*[:=]\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_sha") != kernel_sha() or kv.get("workload") != workload:
        return None
    try:
        return {"fetch": float(kv["fetch_bytes_per_launch"]), "write": float(kv["write_bytes_per_launch"]),
                "hbm": float(kv["hbm_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


def unique_kv_bytes(w, lens) -> int:
    """K+V bytes of the distinct physical rows the step's attention covers:
    every (block, offset) slot of positions < L, counted once however many
    sequences read it."""
    B = w.block_size
    slots = []
    for s in range(w.num_seqs):
        L = int(lens[s])
        if L <= 0:
            continue
        pos = np.arange(L)
        slots.append(w.block_tables[s, pos // B].astype(np.int64) * B + pos % B)
    n = int(np.unique(np.concatenate(slots)).size) if slots else 0
    return n * 2 * w.kv_heads * w.head_dim * w.elt


def _counter_rows(folder, counter):
    """(kernel name, dispatch id, value) of every rocprofv3 counter row named
    `counter` in the CSV files under `folder`."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection*.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], r.get("Dispatch_Id", ""), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {folder}")
    return rows


def _per_dispatch(rows, pattern):
    """Counter value per dispatch of the kernels whose name contains `pattern`
    (rows of one dispatch, e.g. one per XCD, are summed)."""
    acc = {}
    for name, disp, val in rows:
        if pattern in name:
            acc[disp] = acc.get(disp, 0.0) + val
    return list(acc.values())


def profile_command(args, extra=""):
    return ("python bench.py --workload {wl} --call {call} --steps 3 --warmup 1 --no-cpu-baseline --no-extras"
            "{extra}").format(wl=args.workload, call=args.call, extra=extra)


def write_traffic(args):
    """Traffic summary of the stage-1 kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what it reads on the plain copy probe
    of known size run in the same process."""
    from workloads import make_config
    fetch_dir, write_dir = args.write_traffic
    w = make_config(WORKLOADS[args.workload], values=False)
    lens = (w.context_lens + 1).astype(np.int64)
    logical = w.kv_bytes(lens)
    unique = unique_kv_bytes(w, lens)
    copy_kib = args.copy_mib * 1024.0
    out = {}
    for tag, folder, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(folder, counter)
        probe = _per_dispatch(rows, "probe_copy_kernel")
        if not probe:
            raise SystemExit(f"no probe_copy_kernel dispatch under {folder}")
        scale = copy_kib / float(np.mean(probe))
        kernel = next((k for k in STAGE1_KERNELS if _per_dispatch(rows, k)), None)
        if kernel is None:
            raise SystemExit(f"no stage-1 dispatch under {folder}")
        stage1 = _per_dispatch(rows, kernel)
        out[tag] = (float(np.mean(stage1)), scale, len(stage1), kernel)
    fetch_b = out["fetch"][0] * out["fetch"][1] * 1024
    write_b = out["write"][0] * out["write"][1] * 1024
    cmd_run = profile_command(args, f" --copy-probe-mib {args.copy_mib}")
    text = f"""# HBM traffic of the stage-1 decode kernel ({out['fetch'][3]}) on the {w.name} step
# ({w.num_seqs} sequences, {w.q_heads}/{w.kv_heads} heads, head_dim {w.head_dim}, {w.dtype} KV,
# {w.block_size}-token blocks, context L+1, call {args.call}), MI355X, rocprofv3 counter collection in two passes:
#
#   cd /tmp && export TMPDIR=/tmp && cd <repository root> &&
#   timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o run --output-format csv -- \\
#       {cmd_run}
#   timeout -s KILL 180 rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o run --output-format csv -- \\
#       {cmd_run}
#   python bench.py --workload {args.workload} --call {args.call} --write-traffic gpurun_out/pmc_fetch gpurun_out/pmc_write
#
# Scaling: each counter is multiplied by (bytes the plain copy probe moves) / (what the counter reads
# on it): FETCH_SIZE x {out['fetch'][1]:.4f}, WRITE_SIZE x {out['write'][1]:.4f} ({args.copy_mib} MiB copy).
# Per stage-1 launch (mean of {out['fetch'][2]} / {out['write'][2]} dispatches): FETCH_SIZE {out['fetch'][0]:.0f} KiB,
# WRITE_SIZE {out['write'][0]:.0f} KiB.  Logical KV bytes per launch (sum(L+1) * 2 * Hkv * D * elt): {logical};
# unique KV bytes (distinct physical rows): {unique}.
workload: {args.workload}
call: {args.call}
kernel: {out['fetch'][3]}
kernel_sha: {kernel_sha()}
fetch_bytes_per_launch: {fetch_b:.0f}
write_bytes_per_launch: {write_b:.0f}
hbm_bytes_per_launch: {fetch_b + write_b:.0f}
fetch_over_logical: {fetch_b / logical:.4f}
fetch_over_unique: {fetch_b / unique:.4f}
"""
    with open(traffic_file(args.workload, args.call), "w") as f:
        f.write(text)
    print(text)


def write_pmc(args):
    """Mean per dispatch of every counter in rocprofv3 --pmc output folders,
    for the kernels whose name contains --pmc-kernel, into profiles/."""
    import csv
    import glob
    folders, name = args.write_pmc[:-1], args.write_pmc[-1]
    acc = {}
    per_folder = {}
    for folder in folders:
        for path in glob.glob(os.path.join(folder, "**", "*counter_collection*.csv"), recursive=True):
            with open(path, newline="") as f:
                for r in csv.DictReader(f):
                    per_folder.setdefault(folder, set()).add(r["Counter_Name"])
                    if args.pmc_kernel in r["Kernel_Name"]:
                        key = (folder, r.get("Dispatch_Id", ""))
                        acc.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
                        acc[key][r["Counter_Name"]] += float(r["Counter_Value"])
    if not acc:
        raise SystemExit(f"no dispatch of {args.pmc_kernel} under {folders}")
    names = sorted({c for v in acc.values() for c in v})
    mean = {c: float(np.mean([v[c] for v in acc.values() if c in v])) for c in names}
    lines = [f"# rocprofv3 counters of {args.pmc_kernel}, mean per dispatch over the listed runs, MI355X",
             "# (counters summed over the rows of a dispatch: XCDs / shader engines / SIMDs as the tool reports)",
             "#", "#   cd /tmp && export TMPDIR=/tmp && cd <repository root> &&"]
    for folder in folders:
        counters = " ".join(sorted(per_folder.get(folder, ())))
        lines.append(f"#   timeout -s KILL 90 rocprofv3 --pmc {counters} "
                     f"-d {folder} -o run --output-format csv -- {args.pmc_command}")
    lines.append(f"#   python bench.py --pmc-kernel {args.pmc_kernel} --pmc-command '{args.pmc_command}' "
                 f"--write-pmc {' '.join(folders)} {name}")
    lines.append("")
    for c in names:
        lines.append(f"{c}: {mean[c]:.6g}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, f"{name}.txt"), "w") as f:
        f.write(text)
    print(text)


def write_traces(args):
    """Per-kernel duration summary from a rocprofv3 --kernel-trace --stats
    output folder (its kernel_stats CSV), written under profiles/."""
    import csv
    import glob
    paths = glob.glob(os.path.join(args.write_traces, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {args.write_traces}")
    rows = []
    for p in paths:
        with open(p, newline="") as f:
            rows += list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    if args.prefill_only:
        cmd = f"python bench.py --prefill-only --steps {args.steps}"
        what = "prompt pass at the Llama-7B shape (4 sequences, 1024-token chunks over 2048-token contexts)"
        rerun = f"python bench.py --prefill-only --steps {args.steps} --write-traces gpurun_out/trace"
        note = [f"# The run holds 2 warm-up calls, {args.steps} timed calls each after a 1 GiB flush (fill kernel), and",
                f"# {args.steps} calls back to back."]
        out = os.path.join(PROFILES, "kernel_trace_prefill_llama7b-shape.md")
    else:
        cmd = profile_command(args)
        what = f"{args.workload} step (call {args.call})"
        rerun = f"python bench.py --workload {args.workload} --call {args.call} --write-traces gpurun_out/trace"
        note = ["# The run holds 1 warm-up and 3 timed steps, then the same number of stage-1 repetitions,",
                "# each after a 1 GiB flush (fill kernel), and 3 steps back to back."]
        out = os.path.join(PROFILES, f"kernel_trace_{args.workload}_{args.call}.md")
    lines = [f"# rocprofv3 kernel trace of the {what}, MI355X",
             "#", "#   cd /tmp && export TMPDIR=/tmp && cd <repository root> &&",
             f"#   timeout -k 10 300 rocprofv3 --kernel-trace --stats -d gpurun_out/trace -o run "
             f"--output-format csv -- {cmd}",
             f"#   {rerun}", "#", *note, "",
             "| kernel | calls | mean us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = re.sub(r"\(pkv::DecodeParams\)|\(.*\)$", "", name.replace("(anonymous namespace)::", ""))[:110]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    print(text)


# ---------------------------------------------------------------- CPU leg

_CPU = {}


def _cpu_worker(seqs):
    from threadpoolctl import threadpool_limits
    import oracle.paged_attention as pa
    a = _CPU
    with threadpool_limits(1):
        pa.oracle_decode(a["q"], a["k"], a["v"], a["tables"], a["lens"], a["scale"], a["dtype"], a["B"], seqs=seqs)
    return len(seqs)


def host_cores():
    """(cores the worker pool uses, cores in this process's affinity set,
    cgroup CPU quota or None).  The pool takes the affinity set, capped by
    the cgroup quota and by the host share of one GPU."""
    aff = len(os.sched_getaffinity(0))
    quota = None
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = max(1, int(int(q) // int(period)))
    except (OSError, ValueError):
        pass
    cores = min(aff, quota if quota else aff, HOST_CORES_PER_GPU)
    return max(1, cores), aff, quota


def cpu_baseline(w, lens, n_seqs, min_seconds=10.0):
    """The fp64 oracle over (a sample of) the same decode, sequences spread
    over a fork pool of the host's cores, one BLAS thread each; whole passes
    repeat until at least min_seconds of wall time, and the rate is the mean
    over them."""
    import multiprocessing as mp
    from workloads import raw_numpy
    seqs = list(range(w.num_seqs if n_seqs <= 0 else min(n_seqs, w.num_seqs)))
    cores, aff, quota = host_cores()
    cores = max(1, min(cores, len(seqs)))
    _CPU.update(q=raw_numpy(w.q), k=raw_numpy(w.k_cache), v=raw_numpy(w.v_cache), tables=w.block_tables,
                lens=lens, scale=w.scale, dtype=w.dtype, B=w.block_size)
    # longest first, dealt round robin, so the workers finish together
    order = sorted(seqs, key=lambda s: -int(lens[s]))
    chunks = [order[i::cores] for i in range(cores)]
    ctx = mp.get_context("fork")
    passes = 0
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        while True:  # whole passes over the sample until about 10 s have gone by
            done = sum(pool.map(_cpu_worker, chunks))
            assert done == len(seqs)
            passes += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt = (time.perf_counter() - t0) / passes
    kv = w.kv_bytes(lens[seqs])
    tokens = int(np.asarray(lens[seqs], dtype=np.int64).sum())
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle decode of sequences 0..{len(seqs) - 1} of {w.num_seqs} "
                      f"({tokens} context tokens, all {w.q_heads} q heads) at the step's lengths L+1, "
                      f"{passes} whole passes timed together",
            "cores_in_affinity": aff, "cgroup_cpu_quota": quota, "host_cores_per_gpu": HOST_CORES_PER_GPU,
            "blas_threads_per_worker": 1,
            "seconds": dt, "passes": passes, "seq_tokens_per_s": tokens / dt}


# ---------------------------------------------------------------- GPU leg

class Step:
    """One decode step of a workload resident on the GPU, with its stage split:
    pre() (launches before stage 1), stage1(), post() (stage 2)."""

    def __init__(self, pk, torch, d, w, call):
        self.pk, self.torch, self.d, self.call_name = pk, torch, d, call
        lens_step = (w.context_lens + 1).astype(np.int32)
        max_len = int(lens_step.max())
        if call == "shared":
            self.call = pk.DecodeSharedCall(d.q, d.k, d.v, d.tables, d.pos, w.scale, max_len, d.kn, d.vn)
            self.pre, self.stage1, self.post = self.call.prepare, self.call.attend, self.call.merge
            self.run = self.call.run
        elif call == "fused":
            self.call = pk.DecodeAppendCall(d.q, d.k, d.v, d.kn, d.vn, d.tables, d.pos, w.scale, max_len)
            self.pre = lambda: None
            self.stage1, self.post = self.call.partitions, self.call.reduce  # stage 1 holds the row write
            self.run = lambda: (self.call.partitions(), self.call.reduce())
        else:
            lens = torch.from_numpy(lens_step).to(d.q.device)
            self.call = pk.DecodeCall(d.q, d.k, d.v, d.tables, lens, w.scale, max_len)
            self._keep = lens
            self.pre = lambda: pk.append_at(d.k, d.v, d.kn, d.vn, d.tables, d.pos)
            self.stage1, self.post = self.call.partitions, self.call.reduce
            self.run = lambda: (self.pre(), self.call.partitions(), self.call.reduce())

    def kernel(self):
        if self.call_name == "shared" and getattr(self.call, "workspace", None) is not None:
            return "decode_shared_kernel"
        return "decode_stage1"


def flushed_reps(n, flush, stream_ptr, before, body, after):
    """n repetitions of before(); [event] body() [event]; after(), each after
    writing the flush buffer; returns the bracketed times in ms."""
    import torch
    ev = HipEvents(2 * n, stream_ptr)
    for i in range(n):
        flush.fill_(1)
        before()
        ev.record(2 * i)
        body()
        ev.record(2 * i + 1)
        after()
    torch.cuda.synchronize()
    ms = [ev.ms(2 * i, 2 * i + 1) for i in range(n)]
    ev.close()
    return ms


def on_gpu(w, dev, seed):
    """A workload's tensors on the device: lengths and tables from the
    workload; q, pools and new rows as given, or (values=False workloads)
    N(0,1) draws in the cache dtype from a seeded device generator."""
    import torch
    from types import SimpleNamespace
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    if w.k_cache.numel():
        q, kc, vc, kn, vn = (t.to(dev) for t in (w.q, w.k_cache, w.v_cache, w.k_new, w.v_new))
    else:
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        S, NB, B, H, Hq, D = w.num_seqs, w.num_blocks, w.block_size, w.kv_heads, w.q_heads, w.head_dim
        q = torch.randn((S, Hq, D), generator=g, device=dev, dtype=torch.float32).to(dt)
        kc = torch.randn((NB, B, H, D), generator=g, device=dev, dtype=torch.float32).to(dt)
        vc = torch.randn((NB, B, H, D), generator=g, device=dev, dtype=torch.float32).to(dt)
        kn = torch.randn((S, H, D), generator=g, device=dev, dtype=torch.float32).to(dt)
        vn = torch.randn((S, H, D), generator=g, device=dev, dtype=torch.float32).to(dt)
    return SimpleNamespace(q=q, k=kc, v=vc, kn=kn, vn=vn, tables=torch.from_numpy(w.block_tables).to(dev),
                           pos=torch.from_numpy(w.context_lens).to(dev))


def measure_step(pk, torch, w, d, call, reps, warmup, flush, stream_ptr):
    """Flushed step and stage-1 statistics of one workload and call (outside
    the timed region of the headline)."""
    st = Step(pk, torch, d, w, call)
    for _ in range(warmup):
        st.run()
    torch.cuda.synchronize()
    step = stats(flushed_reps(reps, flush, stream_ptr, lambda: None, st.run, lambda: None))
    s1 = stats(flushed_reps(reps, flush, stream_ptr, st.pre, st.stage1, st.post))
    lens = (w.context_lens + 1).astype(np.int64)
    logical = w.kv_bytes(lens)
    unique = unique_kv_bytes(w, lens)
    algo = unique if call == "shared" else logical
    return {"call": call, "step": step, "stage1": s1, "logical_kv_bytes": logical, "unique_kv_bytes": unique,
            "step_GBps_logical": logical / (step["median_ms"] / 1e3) / 1e9,
            "step_GBps_unique": unique / (step["median_ms"] / 1e3) / 1e9,
            "step_pct_of_hbm_peak": 100.0 * (algo / (step["median_ms"] / 1e3) / 1e9) / HBM_PEAK_GBS,
            "stage1_GBps": algo / (s1["median_ms"] / 1e3) / 1e9,
            "stage1_pct_of_hbm_peak": 100.0 * (algo / (s1["median_ms"] / 1e3) / 1e9) / HBM_PEAK_GBS,
            "algorithmic_bytes": "unique" if call == "shared" else "logical"}


def measure_prefill(pk, torch, dev, flush, stream_ptr, reps):
    """The prompt pass at PREFILL_SHAPE: flushed repetitions, median."""
    from workloads import make_workload, normal_storage
    ps = PREFILL_SHAPE
    pw = make_workload("prefill-llama7b", [ps["context"]] * ps["seqs"], ps["q_heads"], ps["kv_heads"],
                       ps["head_dim"], ps["block_size"], "bf16", 357100)
    prng = np.random.default_rng(357101)
    pq = normal_storage(prng, (ps["seqs"] * ps["chunk"], ps["q_heads"], ps["head_dim"]), "bf16").to(dev)
    pk_, pv_ = pw.k_cache.to(dev), pw.v_cache.to(dev)
    ptab = torch.from_numpy(pw.block_tables).to(dev)
    plen = torch.from_numpy(pw.context_lens).to(dev)
    pstart = torch.arange(0, ps["seqs"] + 1, dtype=torch.int32, device=dev) * ps["chunk"]
    pout = torch.empty((ps["seqs"] * ps["chunk"], ps["q_heads"], ps["head_dim"]), dtype=torch.float32, device=dev)

    def prefill():
        pk.prefill(pq, pk_, pv_, ptab, plen, pstart, pw.scale, ps["chunk"], ps["context"], out=pout)

    for _ in range(2):
        prefill()
    st = stats(flushed_reps(reps, flush, stream_ptr, lambda: None, prefill, lambda: None))
    pms = st["median_ms"]
    flops = prefill_flops(ps["seqs"], ps["chunk"], ps["context"], ps["q_heads"], ps["head_dim"])
    tf = flops / (pms / 1e3) / 1e12
    # Context: the same calls back to back (no flush between them), mean per call.
    ev = HipEvents(2, stream_ptr)
    ev.record(0)
    for _ in range(reps):
        prefill()
    ev.record(1)
    torch.cuda.synchronize()
    warm_ms = ev.ms(0, 1) / reps
    ev.close()
    return {"kernel": "prefill_kernel", "shape": ps, "flops": flops, "ms": pms, "times": st, "TFLOPs": tf,
            "bound": "mfma", "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS, "frac": tf / MFMA_BF16_PEAK_TFLOPS,
            "tokens_per_s": ps["seqs"] * ps["chunk"] / (pms / 1e3),
            "warm_back_to_back_ms": warm_ms, "warm_TFLOPs": flops / (warm_ms / 1e3) / 1e12}


def wave_timing(args):
    """Per-wave timing of the shared-prefix stage 1 from the timing build of
    the library: --steps flushed calls of the workload's step; per call the
    entry and stream-start spreads, the end times, the fluid finish (every
    wave at its measured rate with the work shared out perfectly) and the
    per-XCD mean ends; across calls, the correlation of each worker's
    duration with itself (after each XCD's mean is removed)."""
    import ctypes
    import torch
    import paged_kv_cache_357_amd as pk
    from workloads import make_config
    lib = pk.load_library(os.path.join(ROOT, "paged_kv_cache_357_amd", "libpagedkv_timing.so"))
    read = lib.pkv_wave_timing_read
    read.restype = ctypes.c_int
    read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    n_waves = 4096
    buf = np.zeros((n_waves, 4), dtype=np.uint64)

    def fetch():
        if read(buf.ctypes.data, n_waves) != 0:
            raise SystemExit("pkv_wave_timing_read failed")
        return buf.copy()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_config(WORKLOADS[args.workload], values=False)
    d = on_gpu(w, dev, 5)
    st = Step(pk, torch, d, w, "shared")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    for _ in range(3):
        st.run()
    torch.cuda.synchronize()
    fetch()
    reps = []
    for _ in range(args.steps):
        flush.fill_(1)
        st.run()
        torch.cuda.synchronize()
        reps.append(fetch())
    lines = [f"# Per-wave timing of the shared-prefix stage 1 on the {args.workload} step, MI355X",
             "# (device real-time counter at 100 MHz; times in us from the earliest wave entry of each call)", "#",
             "#   python -c 'import __graft_entry__ as g; g.build()'      # also builds libpagedkv_timing.so",
             f"#   python bench.py --workload {args.workload} --steps {args.steps} --wave-timing", "#",
             "# entry/start: spread of wave entries and of stream starts (end of the prologue); end: min / mean / "
             "max;", "# fluid: finish if every wave kept its measured rate and the work were shared out perfectly;",
             "# tail = (max end - mean end) / max end; xcd: mean end per XCD (workgroup id mod 8).", ""]
    durs, xcds = [], None
    for i, r in enumerate(reps):
        live = r[:, 2] != 0
        t = r[live].astype(np.float64)
        base = t[:, 0].min()
        entry, start, end = (t[:, 0] - base) / 100.0, (t[:, 1] - base) / 100.0, (t[:, 2] - base) / 100.0
        chunks = (r[live, 3] >> np.uint64(32)).astype(np.float64)
        wg = (r[live, 3] & np.uint64(0xffffffff)).astype(np.int64)
        xcd = wg % 8
        rate = chunks / np.maximum(end - start, 1e-3)
        fluid = start.mean() + chunks.sum() / rate.sum()
        by_x = [round(float(end[xcd == x].mean()), 1) for x in range(8)]
        lines.append(f"call {i}: waves {int(live.sum())}; entry spread {entry.max():.2f}; start {start.min():.2f} .. "
                     f"{start.max():.2f}; end {end.min():.1f} / {end.mean():.1f} / {end.max():.1f}; fluid {fluid:.1f}; "
                     f"tail {(end.max() - end.mean()) / end.max():.3f}; xcd {by_x}")
        durs.append(end - start)
        xcds = xcd
    if len(durs) > 1 and all(len(x) == len(durs[0]) for x in durs):
        D = np.stack(durs)
        R = D.copy()
        for x in range(8):
            R[:, xcds == x] -= R[:, xcds == x].mean(axis=1, keepdims=True)
        c, cr = np.corrcoef(D), np.corrcoef(R)
        off = ~np.eye(len(durs), dtype=bool)
        lines.append("")
        lines.append(f"per-wave duration, correlation across calls: {c[off].min():.2f} .. {c[off].max():.2f}; "
                     f"after removing each XCD's mean: {cr[off].min():.2f} .. {cr[off].max():.2f}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, f"wave_timing_{args.workload}_shared.txt"), "w") as f:
        f.write(text)
    print(text)


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.write_traces:
        write_traces(args)
        return
    if args.write_pmc:
        write_pmc(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (the decode shards over "
              "sequences or kv heads with no exchange; see the design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.wave_timing:
        wave_timing(args)
        return
    if args.prefill_only:
        import torch
        import paged_kv_cache_357_amd as pk
        pk.load_library()
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        res = measure_prefill(pk, torch, dev, flush, torch.cuda.current_stream(dev).cuda_stream, args.steps)
        print(json.dumps({"prefill": res}), flush=True)
        return

    from workloads import make_config
    k = WORKLOADS[args.workload]
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    # Without the CPU leg nothing needs the values on the host: they are drawn
    # on the device (same lengths and tables, other N(0,1) draws), which keeps
    # profiling runs short.
    w = make_config(k, deal=args.deal, values=not args.no_cpu_baseline)
    lens_step = (w.context_lens + 1).astype(np.int32)  # attend over the appended token too

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, lens_step, args.cpu_seqs)  # before the GPU is touched (fork pool)

    import torch
    import paged_kv_cache_357_amd as pk
    pk.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = on_gpu(w, dev, 0)
    st = Step(pk, torch, d, w, args.call)
    stream_ptr = torch.cuda.current_stream(dev).cuda_stream  # the stream every entry point launches on
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    print(f"[bench] {args.workload} call {args.call}: warm-up", file=sys.stderr, flush=True)
    if args.flush_sweep:
        for _ in range(5):
            st.run()
        torch.cuda.synchronize()
        res = {}
        for mib in (0, 8, 24, 48, 96, 192, 320, 512, 1024):
            buf = flush[: mib << 20]
            ms = flushed_reps(12, buf, stream_ptr, lambda: None, st.stage1, lambda: None) if mib else None
            if ms is None:  # warm: back to back, no write in between
                ev = HipEvents(24, stream_ptr)
                for i in range(12):
                    ev.record(2 * i)
                    st.stage1()
                    ev.record(2 * i + 1)
                torch.cuda.synchronize()
                ms = [ev.ms(2 * i, 2 * i + 1) for i in range(12)]
                ev.close()
            res[mib] = float(np.median(ms[2:])) * 1e3
        print(json.dumps({"workload": args.workload, "call": args.call, "stage1_us_by_flush_mib": res}), flush=True)
        return

    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()

    # Timed region: exactly K steps, each after a 1 GiB flush, each bracketed
    # by events on the launch stream.
    ev = HipEvents(2 * args.steps, stream_ptr)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(1)
        ev.record(2 * i)
        st.run()
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    region_s = time.perf_counter() - t0
    step_ms = [ev.ms(2 * i, 2 * i + 1) for i in range(args.steps)]
    ev.close()
    step = stats(step_ms)

    # After the timed region: stage 1 alone, flushed, and warm steps.
    s1 = stats(flushed_reps(args.steps, flush, stream_ptr, st.pre, st.stage1, st.post))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        st.run()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t1) * 1e3 / args.steps

    logical = w.kv_bytes(lens_step)
    unique = unique_kv_bytes(w, lens_step)
    tokens = int(lens_step.astype(np.int64).sum())
    ms_step = step["median_ms"]
    value = logical / (ms_step / 1e3) / 1e9
    algo = unique if args.call == "shared" else logical
    achieved = algo / (s1["median_ms"] / 1e3) / 1e9
    traffic = read_traffic(args.workload, args.call)
    kernel = st.kernel()
    if kernel == "decode_stage1":
        P, NP = st.call.plan if hasattr(st.call, "plan") else (None, None)
        kernel = "decode_balanced_kernel" if P == 0 else "decode_partitioned_kernel"

    extra = {
        "timing": "median of K steps, each after writing a 1 GiB buffer, HIP events on the launch stream",
        "step": step,
        "stage1": {**s1, "bracket": {"shared": "stage 1 kernel alone (prepare and merge outside the events)",
                                     "fused": "stage 1 kernel alone (it writes the new rows itself)",
                                     "two-launch": "stage 1 kernel alone"}[args.call]},
        "timed_region_s": region_s,
        "warm_back_to_back_ms_per_step": warm_ms,
        "logical_kv_bytes_per_step": logical,
        "unique_kv_bytes_per_step": unique,
        "step_GBps_logical": value,
        "step_GBps_unique": unique / (ms_step / 1e3) / 1e9,
        "pct_of_hbm_peak_step_unique": 100.0 * unique / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "pct_of_hbm_peak_step_logical": 100.0 * value / HBM_PEAK_GBS,
        "seq_tokens_per_s": tokens / (ms_step / 1e3),
        "decode_tokens_per_s": w.num_seqs / (ms_step / 1e3),
        "call": args.call,
        "kernel_sha": kernel_sha(),
    }

    if not args.no_extras:
        reps = args.extra_reps
        # the other workloads (values drawn on the device), shared and plain calls
        other = {}
        for name, kk in WORKLOADS.items():
            if kk in (1, k):
                continue
            print(f"[bench] extra workload {name}", file=sys.stderr, flush=True)
            wx = make_config(kk, values=False)
            dx = on_gpu(wx, dev, 357300 + kk)
            other[name] = {c: measure_step(pk, torch, wx, dx, c, reps, 2, flush, stream_ptr)
                           for c in ("shared", "fused")}
            del dx
        extra["workloads"] = other
        # the headline workload through the other calls
        extra["headline_other_calls"] = {c: measure_step(pk, torch, w, d, c, reps, 2, flush, stream_ptr)
                                         for c in ("fused", "shared") if c != args.call}
        # paged (shuffled blocks) against contiguous blocks, same lengths
        ab = {}
        for name, kk in (("llama7b-decode", 2), ("long-context", 5)):
            print(f"[bench] identity A/B {name}", file=sys.stderr, flush=True)
            res = {}
            for deal in ("shuffled", "identity"):
                wx = make_config(kk, deal=deal, values=False)
                dx = on_gpu(wx, dev, 357400 + kk)
                res[deal] = measure_step(pk, torch, wx, dx, "fused", reps, 2, flush, stream_ptr)["step"]["median_ms"]
                del dx
            ab[name] = {"shuffled_ms": res["shuffled"], "identity_ms": res["identity"],
                        "GBps_ratio_shuffled_over_identity": res["identity"] / res["shuffled"]}
        extra["paged_vs_contiguous"] = ab
        # plain streaming read and copy over 4 GiB
        import ctypes
        plib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_357_amd", "libpkv_probes.so"))
        for fn in (plib.pkv_probe_copy, plib.pkv_probe_read, plib.pkv_probe_fill):
            fn.restype = ctypes.c_int
        stream = ctypes.c_void_p(stream_ptr)
        nb = 4 << 30
        buf = torch.empty(nb, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        dst = torch.empty(nb // 2, dtype=torch.uint8, device=dev)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        probe = {}
        for pname, fn in (("read", lambda: plib.pkv_probe_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(nb),
                                                               ctypes.c_void_p(sink.data_ptr()), stream)),
                          ("copy", lambda: plib.pkv_probe_copy(ctypes.c_void_p(dst.data_ptr()),
                                                               ctypes.c_void_p(buf.data_ptr()),
                                                               ctypes.c_size_t(nb // 2), stream))):
            pev = HipEvents(12, stream_ptr)
            for i in range(6):
                pev.record(2 * i)
                assert fn() == 0
                pev.record(2 * i + 1)
            torch.cuda.synchronize()
            t = float(np.median([pev.ms(2 * i, 2 * i + 1) for i in range(1, 6)]))
            pev.close()
            probe[pname + "_GBps"] = nb / (t / 1e3) / 1e9  # read: nb read; copy: nb / 2 read + nb / 2 written
        extra["probe"] = probe
        extra["stage1_pct_of_probe_read"] = 100.0 * achieved / probe["read_GBps"]
        del buf, dst

        if args.cow_pairs > 0:
            # Copy-on-write block copy at this workload's block shape, on buffers
            # of its own: pair i copies block i to block n + i of both caches.
            n = args.cow_pairs
            shape = (2 * n, w.block_size, w.kv_heads, w.head_dim)
            ck = torch.empty(shape, dtype=d.k.dtype, device=dev)
            cv = torch.empty(shape, dtype=d.k.dtype, device=dev)
            ck.fill_(1)
            cv.fill_(2)
            src = torch.arange(n, dtype=torch.int32, device=dev)
            dsti = src + n
            for _ in range(2):
                pk.copy_blocks(ck, cv, src, dsti)
            cms = stats(flushed_reps(reps, flush, stream_ptr, lambda: None,
                                     lambda: pk.copy_blocks(ck, cv, src, dsti), lambda: None))["median_ms"]
            block_bytes = w.block_size * w.kv_heads * w.head_dim * d.k.element_size()
            moved = 2 * n * 2 * block_bytes  # K and V blocks, each read once and written once
            extra["copy_blocks"] = {"kernel": "copy_blocks_kernel", "pairs": n, "block_bytes": block_bytes,
                                    "bytes_moved": moved, "ms": cms, "GBps": moved / (cms / 1e3) / 1e9,
                                    "frac_of_hbm_peak": moved / (cms / 1e3) / 1e9 / HBM_PEAK_GBS}
            del ck, cv

        if args.swap_blocks > 0:
            # Swap scattered pool blocks out to pinned host memory and back into
            # the same blocks (the pool ends unchanged): PCIe-bound copies.
            n = min(args.swap_blocks, w.num_blocks)
            ids = np.random.default_rng(357200).permutation(w.num_blocks)[:n].astype(np.int32)
            shape = (n, w.block_size, w.kv_heads, w.head_dim)
            hk = torch.empty(shape, dtype=d.k.dtype, pin_memory=True)
            hv = torch.empty(shape, dtype=d.k.dtype, pin_memory=True)
            dt = pk.DTYPE_BF16 if d.k.dtype == torch.bfloat16 else pk.DTYPE_F32
            staging = torch.empty(pk.swap_staging_bytes(n, w.block_size, w.kv_heads, w.head_dim, dt),
                                  dtype=torch.uint8, device=dev)
            moved = 2 * n * w.block_size * w.kv_heads * w.head_dim * d.k.element_size()  # K and V
            runs = 1 + int(np.count_nonzero(np.diff(ids) != 1))
            extra["swap"] = {"blocks": n, "bytes_per_direction": moved}
            for label, stg in (("staged", staging), ("per_run", None)):
                pk.swap_out(d.k, d.v, ids, hk, hv, staging=stg)
                pk.swap_in(d.k, d.v, ids, hk, hv, staging=stg)
                torch.cuda.synchronize()
                sev = HipEvents(4 * 5, stream_ptr)
                for i in range(5):
                    sev.record(4 * i)
                    pk.swap_out(d.k, d.v, ids, hk, hv, staging=stg)
                    sev.record(4 * i + 1)
                    sev.record(4 * i + 2)
                    pk.swap_in(d.k, d.v, ids, hk, hv, staging=stg)
                    sev.record(4 * i + 3)
                torch.cuda.synchronize()
                out_ms = float(np.median([sev.ms(4 * i, 4 * i + 1) for i in range(5)]))
                in_ms = float(np.median([sev.ms(4 * i + 2, 4 * i + 3) for i in range(5)]))
                sev.close()
                extra["swap"][label] = {"copies_per_direction": 2 if stg is not None else 2 * runs,
                                        "out_ms": out_ms, "in_ms": in_ms,
                                        "out_GBps": moved / (out_ms / 1e3) / 1e9,
                                        "in_GBps": moved / (in_ms / 1e3) / 1e9}
            del hk, hv, staging

        extra["prefill"] = measure_prefill(pk, torch, dev, flush, stream_ptr, reps)

    if args.copy_probe_mib:
        import ctypes
        plib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_357_amd", "libpkv_probes.so"))
        plib.pkv_probe_copy.restype = ctypes.c_int
        nb = args.copy_probe_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dstb = torch.empty(nb, dtype=torch.uint8, device=dev)
        src.fill_(3)
        torch.cuda.synchronize()
        rc = plib.pkv_probe_copy(ctypes.c_void_p(dstb.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                 ctypes.c_size_t(nb), ctypes.c_void_p(stream_ptr))
        assert rc == 0
        torch.cuda.synchronize()
        extra["copy_probe_bytes"] = nb
        del src, dstb

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "context_tokens_per_step": tokens,
            "q_heads": w.q_heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
            "num_blocks": w.num_blocks, "block_layout": args.deal, "kv_dtype": w.dtype, "accumulate": "fp32",
            "value_bytes": "logical: sum(L+1) * 2 * Hkv * D * 2 B, shared prompt blocks once per sibling",
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": None if traffic is None else traffic["hbm"],
            "kernel": kernel,
            "algorithmic_bytes_per_launch": algo,
            "algorithmic_bytes": "unique (each physical K/V row read once)" if args.call == "shared"
                                 else "logical",
            "logical_bytes_per_launch": logical,
            "logical_GBps": logical / (s1["median_ms"] / 1e3) / 1e9,
            "stage1_ms_median": s1["median_ms"],
            "fetch_over_algorithmic": None if traffic is None else traffic["fetch"] / algo,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
