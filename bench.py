"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole path over one batch: slot mapping for every sequence's
new token and the K/V append into its block, the fused score / online-softmax /
V pass over every sequence's physical blocks (stage 1), and the merge of the
pieces of split segments (stage 2), run as one paged_attn_decode_append call:
with the vector-ALU kernels stage 1 writes the new rows itself, with the
matrix-core kernels the call writes them in a launch of its own first.
--two-launch runs paged_kv_append_at and then paged_attn_decode instead.  The
workload is the Llama-7B-shaped decode batch (64 sequences, context lengths
uniform in [128, 2048], 32 query / 32 kv heads, head_dim 128, bf16 K/V in
16-token blocks dealt from a shuffled pool 1.25x the blocks in use).  Each
step appends the token at position L and attends over L + 1 tokens.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

prints one JSON line: KV GB/s of the whole step (logical K+V bytes read by
the attention, sum(L+1) * 2 * kv_heads * head_dim * 2 B, per step time), the
roofline of the dominant kernel (stage 1, its duration from HIP events
recorded around it on the launch stream in every fifth step of the timed
region, created without the system-scope fence that default events add;
each event still leaves a bubble of a few microseconds, so the other steps
run unbracketed; its HBM
traffic from the committed rocprofv3 counter summary when that was taken on
the same kernel source), and the fp64 CPU oracle timed on the host's cores
over the same workload.
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
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_357_amd", "csrc", f) for f in ("decode.hip", "pkv_internal.h")]

WORKLOADS = {"llama7b-decode": 2, "tiny-f32": 1, "gqa-lognormal": 3, "cow-parallel-sampling": 4,
             "long-context": 5}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b-decode", choices=sorted(WORKLOADS))
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--deal", default="shuffled", choices=["shuffled", "identity"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-launch", action="store_true",
                    help="run the append as its own launch (paged_kv_append_at), then paged_attn_decode")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences in the CPU sample (0 = all)")
    ap.add_argument("--probes", action="store_true", help="also time plain HBM read / copy probes")
    ap.add_argument("--flush-reps", type=int, default=0,
                    help="also time this many single decode launches after a 1 GiB cache flush each")
    ap.add_argument("--cow-pairs", type=int, default=2048,
                    help="block pairs in the copy-on-write block copy timed after the step (0 = skip)")
    ap.add_argument("--event-every", type=int, default=5,
                    help="bracket the stage-1 launch with HIP events in every n-th timed step (each event "
                         "leaves a bubble of a few microseconds on the stream)")
    ap.add_argument("--swap-blocks", type=int, default=512,
                    help="blocks swapped out to pinned host memory and back after the step (0 = skip)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prompt-pass (prefill) attention timed after the step")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="launch one plain copy of this size (reference kernel for byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of this "
                         "workload's run with --copy-probe-mib into its traffic summary under profiles/")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the copy probe in those runs")
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


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"decode_stage1_{workload}_traffic.txt")


def read_traffic(workload: str):
    """HBM bytes per stage-1 launch from the committed counter summary, or
    None when it is missing or was taken on a different kernel source."""
    path = traffic_file(workload)
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
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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
    if not acc:
        raise SystemExit(f"no dispatch of a kernel matching {pattern!r}")
    return list(acc.values())


def write_traffic(args):
    """Traffic summary of the stage-1 kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what it reads on the plain copy probe
    of known size run in the same process."""
    from workloads import make_config
    fetch_dir, write_dir = args.write_traffic
    w = make_config(WORKLOADS[args.workload], values=False)
    lens = (w.context_lens + 1).astype(np.int64)
    algo = int(lens.sum()) * 2 * w.kv_heads * w.head_dim * w.elt
    copy_kib = args.copy_mib * 1024.0
    out = {}
    for tag, folder, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(folder, counter)
        probe = _per_dispatch(rows, "probe_copy_kernel")
        scale = copy_kib / float(np.mean(probe))
        stage1 = [v for pat in ("decode_balanced_kernel", "decode_partitioned_kernel")
                  for v in (_per_dispatch(rows, pat) if any(pat in r[0] for r in rows) else [])]
        out[tag] = (float(np.mean(stage1)), scale, len(stage1))
    fetch_b = out["fetch"][0] * out["fetch"][1] * 1024
    write_b = out["write"][0] * out["write"][1] * 1024
    cmd_run = ("python bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline "
               "--copy-probe-mib {mib}").format(wl=args.workload, mib=args.copy_mib)
    text = f"""# HBM traffic of the stage-1 decode kernel on the {w.name} step
# ({w.num_seqs} sequences, {w.q_heads}/{w.kv_heads} heads, head_dim {w.head_dim}, {w.dtype} KV,
# {w.block_size}-token blocks, context L+1), MI355X, rocprofv3 counter collection in two passes:
#
#   cd /tmp && export TMPDIR=/tmp && cd <repository root> &&
#   timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o run --output-format csv -- \
#       {cmd_run}
#   timeout -s KILL 180 rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o run --output-format csv -- \
#       {cmd_run}
#   python bench.py --workload {args.workload} --write-traffic gpurun_out/pmc_fetch gpurun_out/pmc_write
#
# Scaling: each counter is multiplied by (bytes the plain copy probe moves) / (what the counter reads
# on it): FETCH_SIZE x {out['fetch'][1]:.4f}, WRITE_SIZE x {out['write'][1]:.4f} ({args.copy_mib} MiB copy).
# Per stage-1 launch (mean of {out['fetch'][2]} / {out['write'][2]} dispatches): FETCH_SIZE {out['fetch'][0]:.0f} KiB,
# WRITE_SIZE {out['write'][0]:.0f} KiB.  Algorithmic bytes per launch (sum(L+1) * 2 * Hkv * D * elt): {algo}.
workload: {args.workload}
kernel_sha: {kernel_sha()}
fetch_bytes_per_launch: {fetch_b:.0f}
write_bytes_per_launch: {write_b:.0f}
hbm_bytes_per_launch: {fetch_b + write_b:.0f}
fetch_over_algorithmic: {fetch_b / algo:.4f}
"""
    with open(traffic_file(args.workload), "w") as f:
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


def cpu_baseline(w, lens, n_seqs, min_seconds=10.0):
    """The fp64 oracle over (a sample of) the same decode, sequences spread
    over a fork pool of the host's cores, one BLAS thread each; whole passes
    repeat until at least min_seconds of wall time, and the rate is the mean
    over them."""
    import multiprocessing as mp
    from workloads import raw_numpy
    seqs = list(range(w.num_seqs if n_seqs <= 0 else min(n_seqs, w.num_seqs)))
    cores = max(1, min(16, len(os.sched_getaffinity(0)), len(seqs)))
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
            "seconds": dt, "passes": passes, "seq_tokens_per_s": tokens / dt}


# ---------------------------------------------------------------- GPU leg

def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (the decode shards over "
              "sequences or kv heads with no exchange; see the design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from workloads import make_config
    k = WORKLOADS[args.workload]
    w = make_config(k, deal=args.deal)
    lens_step = (w.context_lens + 1).astype(np.int32)  # attend over the appended token too

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, lens_step, args.cpu_seqs)  # before the GPU is touched (fork pool)

    import torch
    import paged_kv_cache_357_amd as pk
    pk.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, kc, vc = w.q.to(dev), w.k_cache.to(dev), w.v_cache.to(dev)
    kn, vn = w.k_new.to(dev), w.v_new.to(dev)
    tables = torch.from_numpy(w.block_tables).to(dev)
    pos = torch.from_numpy(w.context_lens).to(dev)
    lens = torch.from_numpy(lens_step).to(dev)
    max_len = int(lens_step.max())
    slots = torch.empty(w.num_seqs, dtype=torch.int32, device=dev)
    two_launch = args.two_launch
    if two_launch:
        # slot mapping + K/V append in a launch of its own, then the decode of L + 1
        call = pk.DecodeCall(q, kc, vc, tables, lens, w.scale, max_len, args.partition_size)
    else:
        # one call: append and decode of L + 1 (stage 1 writes the rows itself on the vector-ALU
        # kernels; the matrix-core kernels get a launch of their own first)
        call = pk.DecodeAppendCall(q, kc, vc, kn, vn, tables, pos, w.scale, max_len, args.partition_size)
    P, NP = call.plan
    balanced = P == 0  # balanced schedule: NP is the number of worker waves

    stream_ptr = torch.cuda.current_stream(dev).cuda_stream  # the stream every entry point launches on

    def step(ev=None, i=0):
        if two_launch:
            pk.append_at(kc, vc, kn, vn, tables, pos, slots)  # slot mapping + K/V append, one launch
        if ev is not None:
            ev.record(2 * i)
        call.partitions()
        if ev is not None:
            ev.record(2 * i + 1)
        call.reduce()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps; in every n-th step two events bracket the
    # stage-1 launch (an event record leaves a bubble of a few microseconds
    # between kernels, so the other steps run back to back).
    every = max(1, args.event_every)
    sampled = list(range(0, args.steps, every))
    ev = HipEvents(2 * len(sampled), stream_ptr)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % every == 0:
            step(ev, i // every)
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    part_ms = float(np.mean([ev.ms(2 * j, 2 * j + 1) for j in range(len(sampled))]))
    ev.close()

    # After the timed region: the other launches, each bracketed alone (the
    # separate append only exists on the two-launch path; it is timed there
    # and, for comparison, also here).
    ev = HipEvents(4 * 10, stream_ptr)
    for i in range(10):
        ev.record(4 * i)
        pk.append_at(kc, vc, kn, vn, tables, pos, slots)
        ev.record(4 * i + 1)
        call.partitions()
        ev.record(4 * i + 2)
        call.reduce()
        ev.record(4 * i + 3)
    torch.cuda.synchronize()
    app_ms = float(np.mean([ev.ms(4 * i, 4 * i + 1) for i in range(10)]))
    red_ms = float(np.mean([ev.ms(4 * i + 2, 4 * i + 3) for i in range(10)]))
    ev.close()

    kv_bytes = w.kv_bytes(lens_step)
    tokens = int(lens_step.astype(np.int64).sum())
    value = kv_bytes / (ms_step / 1e3) / 1e9
    achieved = kv_bytes / (part_ms / 1e3) / 1e9
    traffic = read_traffic(args.workload)

    extra = {
        "kv_bytes_per_step": kv_bytes,
        "pct_of_hbm_peak_step": 100.0 * value / HBM_PEAK_GBS,
        "seq_tokens_per_s": tokens / (ms_step / 1e3),
        "decode_tokens_per_s": w.num_seqs / (ms_step / 1e3),
        "partition_kernel_ms": part_ms, "partition_kernel_samples": len(sampled),
        "reduce_kernel_ms_untimed": red_ms,
        "append_at_kernel_ms_untimed": app_ms,
        "append": "separate launch (append_at)" if two_launch else "paged_attn_decode_append",
        "schedule": "balanced" if balanced else "partitioned",
        "partition_size": P, "num_partitions": NP,
        "kernel_sha": kernel_sha(),
    }

    if args.cow_pairs > 0:
        # Copy-on-write block copy at this workload's block shape, on buffers
        # of its own: pair i copies block i to block n + i of both caches.
        n = args.cow_pairs
        shape = (2 * n, w.block_size, w.kv_heads, w.head_dim)
        ck = torch.empty(shape, dtype=kc.dtype, device=dev)
        cv = torch.empty(shape, dtype=kc.dtype, device=dev)
        ck.fill_(1)
        cv.fill_(2)
        src = torch.arange(n, dtype=torch.int32, device=dev)
        dst = src + n
        for _ in range(2):
            pk.copy_blocks(ck, cv, src, dst)
        cev = HipEvents(2 * 10, stream_ptr)
        for i in range(10):
            cev.record(2 * i)
            pk.copy_blocks(ck, cv, src, dst)
            cev.record(2 * i + 1)
        torch.cuda.synchronize()
        cms = float(np.mean([cev.ms(2 * i, 2 * i + 1) for i in range(10)]))
        cev.close()
        block_bytes = w.block_size * w.kv_heads * w.head_dim * kc.element_size()
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
        hk = torch.empty(shape, dtype=kc.dtype, pin_memory=True)
        hv = torch.empty(shape, dtype=kc.dtype, pin_memory=True)
        dt = pk.DTYPE_BF16 if kc.dtype == torch.bfloat16 else pk.DTYPE_F32
        staging = torch.empty(pk.swap_staging_bytes(n, w.block_size, w.kv_heads, w.head_dim, dt),
                              dtype=torch.uint8, device=dev)
        moved = 2 * n * w.block_size * w.kv_heads * w.head_dim * kc.element_size()  # K and V
        runs = 1 + int(np.count_nonzero(np.diff(ids) != 1))
        extra["swap"] = {"blocks": n, "bytes_per_direction": moved}
        for label, st in (("staged", staging), ("per_run", None)):
            pk.swap_out(kc, vc, ids, hk, hv, staging=st)
            pk.swap_in(kc, vc, ids, hk, hv, staging=st)
            torch.cuda.synchronize()
            sev = HipEvents(4 * 5, stream_ptr)
            for i in range(5):
                sev.record(4 * i)
                pk.swap_out(kc, vc, ids, hk, hv, staging=st)
                sev.record(4 * i + 1)
                sev.record(4 * i + 2)
                pk.swap_in(kc, vc, ids, hk, hv, staging=st)
                sev.record(4 * i + 3)
            torch.cuda.synchronize()
            out_ms = float(np.median([sev.ms(4 * i, 4 * i + 1) for i in range(5)]))
            in_ms = float(np.median([sev.ms(4 * i + 2, 4 * i + 3) for i in range(5)]))
            sev.close()
            extra["swap"][label] = {"copies_per_direction": 2 if st is not None else 2 * runs,
                                    "out_ms": out_ms, "in_ms": in_ms,
                                    "out_GBps": moved / (out_ms / 1e3) / 1e9, "in_GBps": moved / (in_ms / 1e3) / 1e9}
        del hk, hv, staging

    if not args.no_prefill:
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
        pout = torch.empty((ps["seqs"] * ps["chunk"], ps["q_heads"], ps["head_dim"]), dtype=torch.float32,
                           device=dev)
        for _ in range(2):
            pk.prefill(pq, pk_, pv_, ptab, plen, pstart, pw.scale, ps["chunk"], ps["context"], out=pout)
        pev = HipEvents(2 * 10, stream_ptr)
        for i in range(10):
            pev.record(2 * i)
            pk.prefill(pq, pk_, pv_, ptab, plen, pstart, pw.scale, ps["chunk"], ps["context"], out=pout)
            pev.record(2 * i + 1)
        torch.cuda.synchronize()
        pms = float(np.mean([pev.ms(2 * i, 2 * i + 1) for i in range(10)]))
        pev.close()
        flops = prefill_flops(ps["seqs"], ps["chunk"], ps["context"], ps["q_heads"], ps["head_dim"])
        tf = flops / (pms / 1e3) / 1e12
        extra["prefill"] = {"kernel": "prefill_kernel", "shape": ps, "flops": flops, "ms": pms, "TFLOPs": tf,
                            "bound": "mfma", "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                            "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                            "tokens_per_s": ps["seqs"] * ps["chunk"] / (pms / 1e3)}
        del pq, pk_, pv_, pout, pw

    if args.flush_reps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        fev = HipEvents(2 * args.flush_reps, stream_ptr)
        for i in range(args.flush_reps):
            flush.fill_(1)
            fev.record(2 * i)
            call.run()
            fev.record(2 * i + 1)
        torch.cuda.synchronize()
        med = float(np.median([fev.ms(2 * i, 2 * i + 1) for i in range(args.flush_reps)]))
        fev.close()
        extra["flushed_decode_ms_median"] = med
        extra["flushed_decode_GBps"] = kv_bytes / (med / 1e3) / 1e9
        del flush

    if args.probes or args.copy_probe_mib:
        import ctypes
        plib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_357_amd", "libpkv_probes.so"))
        for fn in (plib.pkv_probe_copy, plib.pkv_probe_read, plib.pkv_probe_fill):
            fn.restype = ctypes.c_int
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if args.copy_probe_mib:
            nb = args.copy_probe_mib << 20
            src = torch.empty(nb, dtype=torch.uint8, device=dev)
            dst = torch.empty(nb, dtype=torch.uint8, device=dev)
            src.fill_(3)
            torch.cuda.synchronize()
            rc = plib.pkv_probe_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                     ctypes.c_size_t(nb), stream)
            assert rc == 0
            torch.cuda.synchronize()
            extra["copy_probe_bytes"] = nb
            del src, dst
        if args.probes:
            nb = 4 << 30
            buf = torch.empty(nb, dtype=torch.uint8, device=dev)
            buf.fill_(1)
            dst = torch.empty(nb // 2, dtype=torch.uint8, device=dev)
            sink = torch.zeros(4, dtype=torch.int32, device=dev)
            res = {}
            for name, fn in (("read", lambda: plib.pkv_probe_read(ctypes.c_void_p(buf.data_ptr()),
                                                                 ctypes.c_size_t(nb),
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
                moved = nb if name == "read" else nb  # copy: nb/2 read + nb/2 written
                res[name + "_GBps"] = moved / (t / 1e3) / 1e9
            extra["probe"] = res
            del buf, dst

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
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": "decode_balanced_kernel" if balanced else "decode_partitioned_kernel",
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
