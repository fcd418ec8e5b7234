"""ctypes binding of libpagedkv.so (the C ABI declared in include/pagedkv.h).

Argument marshalling only: shapes are read off torch tensors, device pointers
and the current HIP stream are passed through, and non-zero status codes
become exceptions.  All computation happens in the library's HIP kernels.
PyTorch provides device memory (outputs, workspace) and streams.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedkv.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
_DTYPES = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}

_c_int, _c_i32, _c_f, _c_sz, _vp = ctypes.c_int, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); must match include/pagedkv.h
_DECODE_ARGS = [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                _c_f, _c_i32, _c_i32, _vp, _c_sz, _vp]
_DECODE_APPEND_ARGS = [_vp] * 8 + [_c_i32] * 8 + [_c_f, _c_i32, _c_i32, _vp, _c_sz, _vp]
SIGNATURES = {
    "paged_kv_slot_mapping": (_c_int, [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "paged_kv_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "paged_kv_append_at": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_i32, _vp]),
    "paged_attn_decode": (_c_int, _DECODE_ARGS),
    "paged_attn_decode_partitions": (_c_int, _DECODE_ARGS),
    "paged_attn_decode_reduce": (_c_int, _DECODE_ARGS),
    "paged_attn_decode_append": (_c_int, _DECODE_APPEND_ARGS),
    "paged_attn_decode_append_partitions": (_c_int, _DECODE_APPEND_ARGS),
    "paged_attn_decode_append_reduce": (_c_int, _DECODE_APPEND_ARGS),
    "paged_attn_decode_noalloc": (_c_int, _DECODE_ARGS[:17] + [_vp]),
    "paged_attn_decode_shared": (_c_int, _DECODE_APPEND_ARGS),
    "paged_attn_decode_shared_workspace_size": (_c_sz, [_c_i32] * 7),
    "paged_attn_decode_plan": (_c_int, [_c_i32] * 8 + [_i32p, _i32p]),
    "paged_attn_decode_workspace_size": (_c_sz, [_c_i32] * 8),
    "paged_status_str": (ctypes.c_char_p, [_c_int]),
    "paged_kv_copy_blocks": (_c_int, [_vp, _vp, _vp, _vp] + [_c_i32] * 6 + [_vp]),
    "paged_attn_prefill": (_c_int, [_vp] * 7 + [_c_i32] * 9 + [_c_f, _c_i32, _vp]),
    "pkv_bm_create": (_vp, [_c_i32] * 3),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_add_sequence": (_c_int, [_vp, _i32p]),
    "pkv_bm_fork": (_c_int, [_vp, _c_i32, _i32p]),
    "pkv_bm_free": (_c_int, [_vp, _c_i32]),
    "pkv_bm_append": (_c_int, [_vp, _c_i32, _c_i32, _i32p, _i32p, _i32p, _i32p]),
    "pkv_bm_append_batch": (_c_int, [_vp, _i32p, _c_i32, _i32p, _i32p, _i32p, _i32p, _i32p]),
    "pkv_bm_table": (_c_int, [_vp, _c_i32, _i32p, _c_i32, _i32p, ctypes.POINTER(ctypes.c_int64)]),
    "pkv_bm_tables": (_c_int, [_vp, _i32p, _c_i32, _i32p, _c_i32, _c_i32, _i32p]),
    "pkv_bm_ref_count": (_c_int, [_vp, _c_i32, _i32p]),
    "pkv_bm_free_blocks": (ctypes.c_int32, [_vp]),
    "pkv_bm_usage": (_c_int, [_vp] + [ctypes.POINTER(ctypes.c_int64)] * 4),
    "pkv_bm_swap_out": (_c_int, [_vp, _c_i32, _i32p, _c_i32, _i32p]),
    "pkv_bm_swap_in": (_c_int, [_vp, _c_i32, _i32p, _c_i32, _i32p]),
    "paged_kv_swap_out": (_c_int, [_vp, _vp, _i32p, _c_i32, _vp, _vp, _vp, _c_sz] + [_c_i32] * 5 + [_vp]),
    "paged_kv_swap_in": (_c_int, [_vp, _vp, _i32p, _c_i32, _vp, _vp, _vp, _c_sz] + [_c_i32] * 5 + [_vp]),
    "paged_kv_swap_staging_bytes": (_c_sz, [_c_i32] * 5),
}

PKV_ERR_OUT_OF_BLOCKS = -7

_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_str(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C-ABI library.  Raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_357_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().paged_status_str(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise PagedKVError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    dev = ts[0].device
    for t in ts:
        _require(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")
        _require(t.is_contiguous(), "tensors must be contiguous")
    return dev


def slot_mapping(block_tables: torch.Tensor, positions: torch.Tensor, num_blocks: int, block_size: int,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Slot of each sequence's next token (position = its current length)."""
    lib = load_library()
    _require(block_tables.dtype == torch.int32 and positions.dtype == torch.int32, "int32 tables and positions")
    S, MB = block_tables.shape
    _require(positions.shape == (S,), "positions must be [num_seqs]")
    dev = _dev(block_tables, positions)
    out = torch.empty(S, dtype=torch.int32, device=dev) if out is None else out
    _dev(out)
    _check("paged_kv_slot_mapping", lib.paged_kv_slot_mapping(_ptr(out), _ptr(block_tables), _ptr(positions), S, MB,
                                                              block_size, num_blocks, _stream(dev)))
    return out


def append(k_cache, v_cache, k_new, v_new, slot_mapping_t) -> None:
    """Write k_new[t] / v_new[t] into slot slot_mapping_t[t] of both pools."""
    lib = load_library()
    NB, B, Hkv, D = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "k_cache and v_cache differ in shape")
    N = slot_mapping_t.shape[0]
    _require(k_new.shape == (N, Hkv, D) and v_new.shape == (N, Hkv, D), "k_new/v_new must be [N, Hkv, D]")
    _require(slot_mapping_t.dtype == torch.int32, "slot_mapping must be int32")
    _require(len({k_cache.dtype, v_cache.dtype, k_new.dtype, v_new.dtype}) == 1, "mixed dtypes")
    _require(k_cache.dtype in _DTYPES, f"unsupported dtype {k_cache.dtype}")
    dev = _dev(k_cache, v_cache, k_new, v_new, slot_mapping_t)
    _check("paged_kv_append", lib.paged_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                                  _ptr(slot_mapping_t), N, NB, B, Hkv, D, _DTYPES[k_cache.dtype],
                                                  _stream(dev)))


def append_at(k_cache, v_cache, k_new, v_new, block_tables, positions, slot_mapping_out=None) -> None:
    """Write k_new[s] / v_new[s] at position positions[s] of sequence s (slot
    computed from the block table in the same launch); optionally record the
    slots in slot_mapping_out."""
    lib = load_library()
    NB, B, Hkv, D = k_cache.shape
    S, MB = block_tables.shape
    _require(v_cache.shape == k_cache.shape, "k_cache and v_cache differ in shape")
    _require(k_new.shape == (S, Hkv, D) and v_new.shape == (S, Hkv, D), "k_new/v_new must be [num_seqs, Hkv, D]")
    _require(block_tables.dtype == torch.int32 and positions.dtype == torch.int32, "int32 tables and positions")
    _require(positions.shape == (S,), "positions must be [num_seqs]")
    _require(len({k_cache.dtype, v_cache.dtype, k_new.dtype, v_new.dtype}) == 1, "mixed dtypes")
    _require(k_cache.dtype in _DTYPES, f"unsupported dtype {k_cache.dtype}")
    tensors = [k_cache, v_cache, k_new, v_new, block_tables, positions]
    if slot_mapping_out is not None:
        _require(slot_mapping_out.dtype == torch.int32 and slot_mapping_out.shape == (S,), "slots must be int32 [S]")
        tensors.append(slot_mapping_out)
    dev = _dev(*tensors)
    _check("paged_kv_append_at", lib.paged_kv_append_at(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                                        _ptr(block_tables), _ptr(positions), _ptr(slot_mapping_out),
                                                        S, MB, NB, B, Hkv, D, _DTYPES[k_cache.dtype], _stream(dev)))


def copy_blocks(k_cache, v_cache, src, dst) -> None:
    """Copy block src[i] -> dst[i] of both caches (copy-on-write copies)."""
    lib = load_library()
    NB, B, Hkv, D = k_cache.shape
    _require(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache and v_cache differ")
    _require(k_cache.dtype in _DTYPES, f"unsupported dtype {k_cache.dtype}")
    _require(src.dtype == torch.int32 and dst.dtype == torch.int32 and src.shape == dst.shape and src.dim() == 1,
             "src and dst must be int32 vectors of one length")
    dev = _dev(k_cache, v_cache, src, dst)
    _check("paged_kv_copy_blocks", lib.paged_kv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(src), _ptr(dst),
                                                            src.numel(), NB, B, Hkv, D, _DTYPES[k_cache.dtype],
                                                            _stream(dev)))


def prefill(q, k_cache, v_cache, block_tables, context_lens, q_start, scale, max_q_len, max_context_len,
            out=None) -> torch.Tensor:
    """Causal attention of new prompt rows over the paged cache; returns out
    [total_q, Hq, D] fp32."""
    lib = load_library()
    total, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    S, MB = block_tables.shape
    _require(D2 == D and v_cache.shape == k_cache.shape, "q and caches disagree")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "mixed dtypes")
    _require(q.dtype in _DTYPES, f"unsupported dtype {q.dtype}")
    _require(context_lens.shape == (S,) and q_start.shape == (S + 1,), "context_lens [S], q_start [S+1]")
    _require(block_tables.dtype == context_lens.dtype == q_start.dtype == torch.int32, "int32 index tensors")
    _require(all(t.is_contiguous() for t in (q, k_cache, v_cache, block_tables, context_lens, q_start)),
             "tensors must be contiguous")
    if out is None:
        out = torch.empty((total, Hq, D), dtype=torch.float32, device=q.device)
    _require(out.shape == (total, Hq, D) and out.dtype == torch.float32, "out must be fp32 [total_q, Hq, D]")
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens, q_start)
    _check("paged_attn_prefill", lib.paged_attn_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                        _ptr(block_tables), _ptr(context_lens), _ptr(q_start), S,
                                                        int(max_q_len), Hq, Hkv, D, B, NB, MB, int(max_context_len),
                                                        float(scale), _DTYPES[q.dtype], _stream(dev)))
    return out


def _swap(fn, k_cache, v_cache, blocks, host_k, host_v, staging):
    import numpy as np
    lib = load_library()
    NB, B, Hkv, D = k_cache.shape
    blocks = np.ascontiguousarray(blocks, dtype=np.int32)
    n = len(blocks)
    _require(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache and v_cache differ")
    _require(k_cache.dtype in _DTYPES, f"unsupported dtype {k_cache.dtype}")
    for h in (host_k, host_v):
        _require(not h.is_cuda and h.is_pinned() and h.is_contiguous(), "host buffers must be pinned CPU tensors")
        _require(h.dtype == k_cache.dtype and h.shape[0] >= n and tuple(h.shape[1:]) == (B, Hkv, D),
                 "host buffers must be [>= n_blocks, B, Hkv, D] of the cache dtype")
    dev = _dev(k_cache, v_cache)
    if staging is not None:
        _dev(k_cache, staging)
    _check(fn, getattr(lib, fn)(_ptr(k_cache), _ptr(v_cache), blocks.ctypes.data_as(_i32p), n,
                                ctypes.c_void_p(host_k.data_ptr()), ctypes.c_void_p(host_v.data_ptr()),
                                _ptr(staging), 0 if staging is None else staging.numel() * staging.element_size(),
                                NB, B, Hkv, D, _DTYPES[k_cache.dtype], _stream(dev)))


def swap_staging_bytes(n_blocks, block_size, kv_heads, head_dim, dtype) -> int:
    """Device staging bytes for a swap of n_blocks blocks."""
    return int(load_library().paged_kv_swap_staging_bytes(n_blocks, block_size, kv_heads, head_dim, dtype))


def swap_out(k_cache, v_cache, blocks, host_k, host_v, staging=None) -> None:
    """Copy device blocks blocks[i] of both caches to host slot i (pinned
    host tensors [>= n, B, Hkv, D]); asynchronous on the current stream.
    ``staging`` (a device uint8 tensor of swap_staging_bytes) batches the
    transfer into one copy per cache."""
    _swap("paged_kv_swap_out", k_cache, v_cache, blocks, host_k, host_v, staging)


def swap_in(k_cache, v_cache, blocks, host_k, host_v, staging=None) -> None:
    """Copy host slot i of both pinned host tensors to device block blocks[i]."""
    _swap("paged_kv_swap_in", k_cache, v_cache, blocks, host_k, host_v, staging)


class OutOfBlocksError(PagedKVError):
    pass


def _i32buf(n):
    import numpy as np
    return np.zeros(max(1, n), dtype=np.int32)


def _p(a):
    return a.ctypes.data_as(_i32p)


class BlockManager:
    """Host-side block manager of the library (pool, tables, reference counts,
    copy-on-write decisions).  ``append`` returns the slots of the new tokens
    and the (src, dst) block copies to run with :func:`copy_blocks` first."""

    def __init__(self, num_blocks, block_size, max_blocks_per_seq):
        self.lib = load_library()
        self.num_blocks, self.B, self.max_blocks = int(num_blocks), int(block_size), int(max_blocks_per_seq)
        self.h = self.lib.pkv_bm_create(self.num_blocks, self.B, self.max_blocks)
        if not self.h:
            raise ValueError("pkv_bm_create rejected the sizes")
        self._live = set()

    def __del__(self):
        h, self.h = getattr(self, "h", None), None
        if h:
            self.lib.pkv_bm_destroy(h)

    def _st(self, fn, st):
        if st == PKV_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocksError(fn, st)
        _check(fn, st)

    def add_sequence(self):
        out = ctypes.c_int32()
        self._st("pkv_bm_add_sequence", self.lib.pkv_bm_add_sequence(self.h, ctypes.byref(out)))
        self._live.add(out.value)
        return out.value

    def fork(self, parent):
        out = ctypes.c_int32()
        self._st("pkv_bm_fork", self.lib.pkv_bm_fork(self.h, int(parent), ctypes.byref(out)))
        self._live.add(out.value)
        return out.value

    def free(self, s):
        self._st("pkv_bm_free", self.lib.pkv_bm_free(self.h, int(s)))
        self._live.discard(int(s))

    def append(self, s, n):
        slots, src, dst, nc = _i32buf(n), _i32buf(1), _i32buf(1), ctypes.c_int32()
        self._st("pkv_bm_append", self.lib.pkv_bm_append(self.h, int(s), int(n), _p(slots), _p(src), _p(dst),
                                                         ctypes.byref(nc)))
        return [int(x) for x in slots[:n]], [(int(src[i]), int(dst[i])) for i in range(nc.value)]

    def append_batch(self, seqs):
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = len(seqs)
        slots, src, dst = _i32buf(n), _i32buf(n), _i32buf(n)
        nc, nd = ctypes.c_int32(), ctypes.c_int32()
        st = self.lib.pkv_bm_append_batch(self.h, _p(seqs), n, _p(slots), _p(src), _p(dst), ctypes.byref(nc),
                                          ctypes.byref(nd))
        self._st("pkv_bm_append_batch", st)
        return slots[:n].copy(), src[:nc.value].copy(), dst[:nc.value].copy()

    def table(self, s):
        buf, nb, ln = _i32buf(self.max_blocks), ctypes.c_int32(), ctypes.c_int64()
        self._st("pkv_bm_table", self.lib.pkv_bm_table(self.h, int(s), _p(buf), self.max_blocks, ctypes.byref(nb),
                                                       ctypes.byref(ln)))
        return [int(x) for x in buf[:nb.value]]

    def length(self, s):
        buf, nb, ln = _i32buf(self.max_blocks), ctypes.c_int32(), ctypes.c_int64()
        self._st("pkv_bm_table", self.lib.pkv_bm_table(self.h, int(s), _p(buf), self.max_blocks, ctypes.byref(nb),
                                                       ctypes.byref(ln)))
        return int(ln.value)

    def tables(self, seqs, max_blocks_per_seq=None, fill=0):
        """[len(seqs), max_blocks_per_seq] int32 table and int32 lengths (host numpy)."""
        import numpy as np
        mb = self.max_blocks if max_blocks_per_seq is None else int(max_blocks_per_seq)
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        t = np.zeros((max(1, len(seqs)), mb), dtype=np.int32)
        lens = _i32buf(len(seqs))
        self._st("pkv_bm_tables", self.lib.pkv_bm_tables(self.h, _p(seqs), len(seqs), _p(t), mb, int(fill),
                                                         _p(lens)))
        return t[:len(seqs)], lens[:len(seqs)].copy()

    def swap_out(self, s):
        """Block ids (table order) to save; the sequence leaves the device."""
        buf, nb = _i32buf(self.max_blocks), ctypes.c_int32()
        self._st("pkv_bm_swap_out", self.lib.pkv_bm_swap_out(self.h, int(s), _p(buf), self.max_blocks,
                                                             ctypes.byref(nb)))
        self._live.discard(int(s))
        return [int(x) for x in buf[:nb.value]]

    def swap_in(self, s):
        """Fresh block ids (table order) that receive the saved contents."""
        buf, nb = _i32buf(self.max_blocks), ctypes.c_int32()
        self._st("pkv_bm_swap_in", self.lib.pkv_bm_swap_in(self.h, int(s), _p(buf), self.max_blocks,
                                                           ctypes.byref(nb)))
        self._live.add(int(s))
        return [int(x) for x in buf[:nb.value]]

    def ref_count(self, block):
        out = ctypes.c_int32()
        self._st("pkv_bm_ref_count", self.lib.pkv_bm_ref_count(self.h, int(block), ctypes.byref(out)))
        return out.value

    @property
    def ref(self):
        return [self.ref_count(b) for b in range(self.num_blocks)]

    def free_blocks(self):
        return int(self.lib.pkv_bm_free_blocks(self.h))

    def usage(self):
        """(used blocks, filled slots, live sequences, held tokens)."""
        v = [ctypes.c_int64() for _ in range(4)]
        self._st("pkv_bm_usage", self.lib.pkv_bm_usage(self.h, *[ctypes.byref(x) for x in v]))
        return tuple(int(x.value) for x in v)

    def live(self):
        return sorted(self._live)


def _decode_shapes(q, k_cache, v_cache, block_tables, context_lens):
    S, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    _require(D == D2 and v_cache.shape == k_cache.shape, "q / k_cache / v_cache shapes disagree")
    _require(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32, "int32 tables and lengths")
    _require(block_tables.shape[0] == S and context_lens.shape == (S,), "tables / lengths must have num_seqs rows")
    _require(q.dtype == k_cache.dtype == v_cache.dtype and q.dtype in _DTYPES, "q, K, V must share f32/bf16")
    return S, Hq, Hkv, D, B, NB, block_tables.shape[1]


def plan(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype, partition_size=0):
    """(resolved partition size, number of partitions) for these sizes."""
    lib = load_library()
    p, n = ctypes.c_int32(), ctypes.c_int32()
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    _check("paged_attn_decode_plan", lib.paged_attn_decode_plan(num_seqs, q_heads, kv_heads, head_dim, block_size,
                                                                max_context_len, dt, partition_size,
                                                                ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value


def workspace_size(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype, partition_size=0):
    lib = load_library()
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.paged_attn_decode_workspace_size(num_seqs, q_heads, kv_heads, head_dim, block_size,
                                                    max_context_len, dt, partition_size))


class DecodeCall:
    """A prepared decode call: output and workspace allocated once, the same
    arguments reused by every invocation (what a serving loop or a benchmark
    does).  ``run()`` enqueues both stages; ``partitions()`` / ``reduce()``
    enqueue one stage each."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                 partition_size=0, out=None, workspace=None):
        S, Hq, Hkv, D, B, NB, MB = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
        self.dev = _dev(q, k_cache, v_cache, block_tables, context_lens)
        self.lib = load_library()
        dt = _DTYPES[q.dtype]
        ws = workspace_size(S, Hq, Hkv, D, B, int(max_context_len), dt, partition_size)
        if out is None:
            out = torch.empty((S, Hq, D), dtype=torch.float32, device=self.dev)
        _require(out.shape == (S, Hq, D) and out.dtype == torch.float32, "out must be fp32 [S, Hq, D]")
        _dev(out)
        if workspace is None and ws:
            workspace = torch.empty(ws, dtype=torch.uint8, device=self.dev)
        self.out, self.workspace = out, workspace
        self.plan = plan(S, Hq, Hkv, D, B, int(max_context_len), dt, partition_size)
        self._keep = (q, k_cache, v_cache, block_tables, context_lens)
        self.args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                     S, Hq, Hkv, D, B, NB, MB, int(max_context_len), float(scale), dt, int(partition_size),
                     _ptr(workspace), 0 if workspace is None else workspace.numel())

    def _call(self, name):
        _check(name, getattr(self.lib, name)(*self.args, _stream(self.dev)))
        return self.out

    def run(self):
        return self._call("paged_attn_decode")

    def partitions(self):
        return self._call("paged_attn_decode_partitions")

    def reduce(self):
        return self._call("paged_attn_decode_reduce")


class DecodeAppendCall(DecodeCall):
    """A prepared fused step: each sequence's new K/V row is written at
    position context_lens[s] and the decode attends over context_lens[s] + 1
    tokens, in the launches of one decode.  ``max_context_len`` bounds the
    attended length (L + 1)."""

    def __init__(self, q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, scale, max_context_len,
                 partition_size=0, out=None, workspace=None):
        super().__init__(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size,
                         out, workspace)
        Hkv, D = k_cache.shape[2], k_cache.shape[3]
        S = q.shape[0]
        _require(k_new.shape == (S, Hkv, D) and v_new.shape == (S, Hkv, D), "k_new / v_new must be [S, Hkv, D]")
        _require(k_new.dtype == v_new.dtype == k_cache.dtype, "k_new / v_new must have the cache dtype")
        _dev(q, k_new, v_new)
        self._keep = self._keep + (k_new, v_new)
        a = self.args
        self.args = a[:4] + (_ptr(k_new), _ptr(v_new)) + a[4:]

    def run(self):
        return self._call("paged_attn_decode_append")

    def partitions(self):
        return self._call("paged_attn_decode_append_partitions")

    def reduce(self):
        return self._call("paged_attn_decode_append_reduce")


def decode_append(q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, scale, max_context_len,
                  partition_size=0, out=None, workspace=None) -> torch.Tensor:
    """Append each sequence's new token at position context_lens[s] and decode
    over the context_lens[s] + 1 tokens; returns out [S, Hq, D] fp32."""
    return DecodeAppendCall(q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, scale, max_context_len,
                            partition_size, out, workspace).run()


STAGE_PREPARE, STAGE_ATTEND, STAGE_MERGE, STAGES_ALL = 1, 2, 4, 7  # PKV_STAGE_*


def shared_workspace_size(num_seqs, q_heads, kv_heads, head_dim, block_size, max_context_len, dtype):
    lib = load_library()
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.paged_attn_decode_shared_workspace_size(num_seqs, q_heads, kv_heads, head_dim, block_size,
                                                           max_context_len, dt))


class DecodeSharedCall:
    """A prepared paged_attn_decode_shared call: the decode (k_new = None) or
    the fused append + decode (k_new, v_new given) that reads blocks shared by
    neighbouring sequences once.  ``run()`` enqueues every stage;
    ``prepare()`` / ``attend()`` / ``merge()`` one stage each, in that order."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, k_new=None,
                 v_new=None, out=None, workspace=None):
        S, Hq, Hkv, D, B, NB, MB = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
        self.dev = _dev(q, k_cache, v_cache, block_tables, context_lens)
        self.lib = load_library()
        dt = _DTYPES[q.dtype]
        _require((k_new is None) == (v_new is None), "give both k_new and v_new, or neither")
        if k_new is not None:
            _require(k_new.shape == (S, Hkv, D) and v_new.shape == (S, Hkv, D), "k_new / v_new must be [S, Hkv, D]")
            _require(k_new.dtype == v_new.dtype == k_cache.dtype, "k_new / v_new must have the cache dtype")
            _dev(q, k_new, v_new)
        ws = shared_workspace_size(S, Hq, Hkv, D, B, int(max_context_len), dt)
        if out is None:
            out = torch.empty((S, Hq, D), dtype=torch.float32, device=self.dev)
        _require(out.shape == (S, Hq, D) and out.dtype == torch.float32, "out must be fp32 [S, Hq, D]")
        _dev(out)
        if workspace is None and ws:
            workspace = torch.empty(ws, dtype=torch.uint8, device=self.dev)
        self.out, self.workspace = out, workspace
        self._keep = (q, k_cache, v_cache, block_tables, context_lens, k_new, v_new)
        self.args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
                     _ptr(context_lens), S, Hq, Hkv, D, B, NB, MB, int(max_context_len), float(scale), dt)
        self.ws_args = (_ptr(workspace), 0 if workspace is None else workspace.numel())

    def _call(self, stages):
        _check("paged_attn_decode_shared",
               self.lib.paged_attn_decode_shared(*self.args, stages, *self.ws_args, _stream(self.dev)))
        return self.out

    def run(self):
        return self._call(STAGES_ALL)

    def prepare(self):
        return self._call(STAGE_PREPARE)

    def attend(self):
        return self._call(STAGE_ATTEND)

    def merge(self):
        return self._call(STAGE_MERGE)


def decode_shared(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, k_new=None, v_new=None,
                  out=None, workspace=None) -> torch.Tensor:
    """Paged decode (or fused append + decode) reading shared prefix blocks
    once; returns out [S, Hq, D] fp32."""
    return DecodeSharedCall(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, k_new, v_new,
                            out, workspace).run()


NOALLOC_SCRATCH_BYTES = 32 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, out,
                   partition_size=0) -> torch.Tensor:
    """paged_attn_decode_noalloc: the decode with the library's fixed device
    scratch array instead of a workspace; ``out`` [S, Hq, D] fp32 is given by
    the caller, and the call allocates nothing."""
    S, Hq, Hkv, D, B, NB, MB = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    _require(out.shape == (S, Hq, D) and out.dtype == torch.float32, "out must be fp32 [S, Hq, D]")
    lib = load_library()
    _check("paged_attn_decode_noalloc",
           lib.paged_attn_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                         _ptr(context_lens), S, Hq, Hkv, D, B, NB, MB, int(max_context_len),
                                         float(scale), _DTYPES[q.dtype], int(partition_size), _stream(dev)))
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size=0,
           out=None, workspace=None) -> torch.Tensor:
    """Paged decode attention; returns out [S, Hq, D] fp32."""
    return DecodeCall(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size,
                      out, workspace).run()
