"""Helpers shared by the GPU tests: move a workload to the device, run the
HIP path through the binding, run the oracle on the same inputs, compare."""
from __future__ import annotations

import sys
from types import SimpleNamespace

import numpy as np
import torch

import oracle.paged_attention as pa
from workloads import raw_numpy

TOL = {"f32": 1e-4, "bf16": 5e-4}


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_gpu(w, device="cuda"):
    return SimpleNamespace(
        q=w.q.to(device), k=w.k_cache.to(device), v=w.v_cache.to(device),
        kn=w.k_new.to(device), vn=w.v_new.to(device),
        tables=torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(device),
        lens=torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(device))


def gpu_decode(pk, w, d, lens=None, partition_size=0, max_len=None, k=None, v=None, q=None, scale=None):
    lens = w.context_lens if lens is None else np.asarray(lens, dtype=np.int32)
    lens_t = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to(d.q.device)
    max_len = int(lens.max()) if max_len is None else int(max_len)
    out = pk.decode(d.q if q is None else q, d.k if k is None else k, d.v if v is None else v, d.tables, lens_t,
                    w.scale if scale is None else scale, max_len, partition_size)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_out(w, lens=None, seqs=None, k_cache=None, v_cache=None, q=None, scale=None):
    lens = w.context_lens if lens is None else lens
    return pa.oracle_decode(raw_numpy(w.q) if q is None else q,
                            raw_numpy(w.k_cache) if k_cache is None else k_cache,
                            raw_numpy(w.v_cache) if v_cache is None else v_cache,
                            w.block_tables, lens, w.scale if scale is None else scale, w.dtype, w.block_size,
                            seqs=seqs)


def max_err(gpu, ref, seqs=None):
    idx = slice(None) if seqs is None else list(seqs)
    g, r = gpu[idx].astype(np.float64), ref[idx]
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - r))) if g.size else 0.0


def assert_parity(gpu, ref, w, seqs=None, what=""):
    e = max_err(gpu, ref, seqs)
    tol = TOL[w.dtype]
    say(f"{w.name} {what}: max|gpu - oracle| = {e:.3e} (tol {tol:g})")
    assert e <= tol, (w.name, what, e)
    return e
