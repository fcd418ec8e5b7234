"""Seeded synthetic workloads for paged decode attention and KV append.

Every workload is drawn from ``numpy.random.default_rng(seed)`` in a fixed
order: context lengths, then (for forked prompts) the private tail lengths,
then the physical-block permutation, then q, the K pool, the V pool and the new
token's K/V rows.  Values are N(0, 1) draws in fp32; for bf16 workloads they are
rounded to bf16 by torch's round-to-nearest-even cast, and the stored bf16 bits
are the input (nobody ever sees the pre-rounding fp32 values).

Physical blocks are handed out the way an incremental allocator would: each
sequence owns ceil((L+1)/B) blocks, room for its L context tokens plus the one
token the next append writes (the block-per-overflow rule of "PagedAttention
and vLLM Architecture", section "Why Internal Fragmentation is Bounded").  The
pool holds 1.25x the blocks in use unless a size is given.  Forked sequences
(copy-on-write parallel sampling, "PagedAttention Paper Breakdown" section 3)
alias their prompt's blocks and own only their tail blocks.

Nothing here translates logical positions to slots or computes attention.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

CONFIG_NAMES = {
    1: "tiny-f32",
    2: "llama7b-decode",
    3: "gqa-lognormal",
    4: "cow-parallel-sampling",
    5: "long-context",
}


@dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": storage type of q, K, V, k_new, v_new
    block_size: int            # B, tokens per physical block
    q_heads: int
    kv_heads: int
    head_dim: int
    num_blocks: int            # NB, blocks in the physical pool
    scale: float               # fp32 value (a Python float holding an exactly-fp32 number)
    context_lens: np.ndarray   # int32 [S]
    block_tables: np.ndarray   # int32 [S, MB]; entries at or beyond ceil((L+1)/B) are padding
    q: torch.Tensor            # CPU [S, Hq, D]
    k_cache: torch.Tensor      # CPU [NB, B, Hkv, D]
    v_cache: torch.Tensor      # CPU [NB, B, Hkv, D]
    k_new: torch.Tensor        # CPU [S, Hkv, D]: the token appended at position L
    v_new: torch.Tensor        # CPU [S, Hkv, D]
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def kv_bytes(self, lens=None) -> int:
        """Logical K+V bytes one decode call reads: sum(L) * 2 * Hkv * D * elt."""
        lens = self.context_lens if lens is None else lens
        return int(np.asarray(lens, dtype=np.int64).sum()) * 2 * self.kv_heads * self.head_dim * self.elt


def raw_numpy(t: torch.Tensor) -> np.ndarray:
    """Storage bits of a CPU tensor as numpy: uint16 for bf16, float32 for fp32."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def _to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def _normal(rng, shape, dtype):
    return _to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


def normal_storage(rng, shape, dtype: str) -> torch.Tensor:
    """N(0,1) draws from rng stored in the cache dtype ("bf16" rounds to
    nearest even), as a CPU tensor."""
    return _normal(rng, shape, dtype)


def make_workload(name, lens, q_heads, kv_heads, head_dim, block_size, dtype, seed, *,
                  rng=None, num_blocks=None, pool_factor=1.25, deal="shuffled",
                  prompts=None, tails=None, shared_q=False, pad_cols=0, values=True):
    """Build a workload.

    lens      : context lengths (ignored when ``prompts`` is given).
    prompts   : (num_prompts, siblings, prompt_len) for forked sequences; the
                sequence order is prompt-major (s = prompt * siblings + k).
    tails     : private tail lengths of forked sequences, one per sequence.
    deal      : "shuffled" (blocks dealt from a seeded permutation of the pool)
                or "identity" (sequence s owns blocks s*MB .. s*MB+need-1).
    shared_q  : forked siblings get the same q (copy-on-write identity case).
    values    : False skips drawing q / K / V (empty tensors); lengths and
                tables are unchanged because they are drawn first.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    B = int(block_size)
    if q_heads % kv_heads:
        raise ValueError("q_heads must be a multiple of kv_heads")

    if prompts is not None:
        n_prompts, n_sib, prompt_len = prompts
        if prompt_len % B:
            raise ValueError("a shared prompt must fill whole blocks")
        tails = np.asarray(tails, dtype=np.int64)
        assert tails.shape == (n_prompts * n_sib,)
        lens = prompt_len + tails
        prompt_blocks = prompt_len // B
        private_need = -(-(tails + 1) // B)
        total_need = n_prompts * prompt_blocks + int(private_need.sum())
    else:
        lens = np.asarray(lens, dtype=np.int64)
        need = -(-(lens + 1) // B)
        total_need = int(need.sum())
    S = int(lens.shape[0])

    if deal == "identity":
        if prompts is not None:
            raise ValueError("identity dealing has no shared blocks")
        MB = int(need.max()) + pad_cols if S else 1
        NB = S * MB if num_blocks is None else int(num_blocks)
        assert NB >= S * MB
        tables = np.zeros((S, MB), dtype=np.int64)
        for s in range(S):
            tables[s] = s * MB + np.arange(MB)
    else:
        NB = int(math.ceil(pool_factor * total_need)) if num_blocks is None else int(num_blocks)
        if NB < total_need:
            raise ValueError("pool too small")
        perm = rng.permutation(NB)
        nxt = 0
        if prompts is not None:
            MB = prompt_blocks + int(private_need.max()) + pad_cols
            tables = np.zeros((S, MB), dtype=np.int64)
            prompt_ids = []
            for j in range(n_prompts):
                prompt_ids.append(perm[nxt:nxt + prompt_blocks])
                nxt += prompt_blocks
            for s in range(S):
                j = s // n_sib
                tables[s, :prompt_blocks] = prompt_ids[j]
                k = int(private_need[s])
                tables[s, prompt_blocks:prompt_blocks + k] = perm[nxt:nxt + k]
                nxt += k
        else:
            MB = (int(need.max()) if S else 1) + pad_cols
            tables = np.zeros((S, MB), dtype=np.int64)
            for s in range(S):
                k = int(need[s])
                tables[s, :k] = perm[nxt:nxt + k]
                nxt += k
        # padding entries point at the first block nobody owns (or block 0 if
        # the pool is exactly full); they are never read by a correct kernel.
        unused = perm[nxt:]
        pad = int(unused[0]) if unused.size else 0
        owned = np.zeros_like(tables, dtype=bool)
        if prompts is not None:
            for s in range(S):
                owned[s, :prompt_blocks + int(private_need[s])] = True
        else:
            for s in range(S):
                owned[s, :int(need[s])] = True
        tables[~owned] = pad

    D = int(head_dim)
    if not values:
        empty = torch.empty(0)
        return Workload(name=name, dtype=dtype, block_size=B, q_heads=q_heads, kv_heads=kv_heads,
                        head_dim=D, num_blocks=NB, scale=float(np.float32(1.0 / math.sqrt(D))),
                        context_lens=lens.astype(np.int32), block_tables=tables.astype(np.int32),
                        q=empty, k_cache=empty, v_cache=empty, k_new=empty, v_new=empty, seed=seed,
                        meta={"total_need": total_need, "deal": deal,
                              **({"prompts": tuple(prompts), "prompt_blocks": prompt_blocks,
                                  "tails": tails.astype(np.int32)} if prompts is not None else {})})
    if shared_q and prompts is not None:
        qp = rng.standard_normal((n_prompts, q_heads, D), dtype=np.float32)
        q = _to_storage(np.repeat(qp, n_sib, axis=0), dtype)
    else:
        q = _normal(rng, (S, q_heads, D), dtype)
    k_cache = _normal(rng, (NB, B, kv_heads, D), dtype)
    v_cache = _normal(rng, (NB, B, kv_heads, D), dtype)
    k_new = _normal(rng, (S, kv_heads, D), dtype)
    v_new = _normal(rng, (S, kv_heads, D), dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    meta = {"total_need": total_need, "deal": deal}
    if prompts is not None:
        meta.update(prompts=tuple(prompts), prompt_blocks=prompt_blocks, tails=tails.astype(np.int32))
    return Workload(name=name, dtype=dtype, block_size=B, q_heads=q_heads, kv_heads=kv_heads,
                    head_dim=D, num_blocks=NB, scale=scale,
                    context_lens=lens.astype(np.int32), block_tables=tables.astype(np.int32),
                    q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                    seed=seed, meta=meta)


def make_config(k: int, *, deal="shuffled", shared_q=False, zero_tails=False, values=True) -> Workload:
    """The five named workloads, seeded with 357000 + k."""
    seed = 357000 + k
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[k]
    if k == 1:
        # 4 sequences, fixed lengths, fp32, pool of exactly 32 blocks.
        return make_workload(name, [5, 16, 17, 40], 4, 4, 64, 16, "f32", seed, rng=rng,
                             num_blocks=32 if deal == "shuffled" else None, deal=deal, values=values)
    if k == 2:
        lens = rng.integers(128, 2049, size=64)
        return make_workload(name, lens, 32, 32, 128, 16, "bf16", seed, rng=rng, deal=deal, values=values)
    if k == 3:
        lens = np.clip(np.rint(rng.lognormal(math.log(500.0), 1.0, size=256)), 1, 4096).astype(np.int64)
        return make_workload(name, lens, 32, 8, 128, 32, "bf16", seed, rng=rng, deal=deal, values=values)
    if k == 4:
        tails = rng.integers(0, 64, size=512)
        if zero_tails:
            tails = np.zeros_like(tails)
        return make_workload(name, None, 40, 40, 128, 16, "bf16", seed, rng=rng,
                             prompts=(128, 4, 1024), tails=tails, shared_q=shared_q, values=values)
    if k == 5:
        return make_workload(name, [32768] * 8, 64, 8, 128, 16, "bf16", seed, rng=rng, deal=deal,
                             values=values)
    raise ValueError(k)


def make_small(k: int, *, seed_offset=0, deal="shuffled", shared_q=False, zero_tails=False) -> Workload:
    """Scaled-down relatives of the five workloads: same dtype, D, B and group
    size, fewer sequences and heads, lengths that still span several 16-token
    chunks and partitions and end in ragged tails."""
    seed = 358000 + 10 * k + seed_offset
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[k] + "-small"
    if k == 1:
        return make_workload(name, [5, 16, 17, 40], 4, 4, 64, 16, "f32", seed, rng=rng,
                             num_blocks=32 if deal == "shuffled" else None, deal=deal)
    if k == 2:
        lens = rng.integers(1, 700, size=6)
        return make_workload(name, lens, 4, 4, 128, 16, "bf16", seed, rng=rng, deal=deal)
    if k == 3:
        lens = np.clip(np.rint(rng.lognormal(math.log(120.0), 1.0, size=8)), 1, 900).astype(np.int64)
        return make_workload(name, lens, 8, 2, 128, 32, "bf16", seed, rng=rng, deal=deal)
    if k == 4:
        tails = rng.integers(0, 40, size=12)
        if zero_tails:
            tails = np.zeros_like(tails)
        return make_workload(name, None, 3, 3, 128, 16, "bf16", seed, rng=rng,
                             prompts=(3, 4, 128), tails=tails, shared_q=shared_q)
    if k == 5:
        return make_workload(name, [3000, 2100], 16, 2, 128, 16, "bf16", seed, rng=rng, deal=deal)
    raise ValueError(k)


def identity_tables(w: Workload, seed=None) -> Workload:
    """A workload of the same shape whose tables are the identity layout
    (sequence s owns blocks s*MB ..), with fresh values drawn from ``seed``."""
    if "prompts" in w.meta:
        raise ValueError("forked workloads share blocks; no identity layout exists")
    seed = w.seed + 7 if seed is None else seed
    return make_workload(w.name + "-identity", w.context_lens, w.q_heads, w.kv_heads, w.head_dim,
                         w.block_size, w.dtype, seed, deal="identity")


def permute_pool(w: Workload, perm: np.ndarray) -> Workload:
    """Relabel physical blocks: block p moves to perm[p] and every table entry
    p becomes perm[p].  Attention must not change."""
    perm = np.asarray(perm, dtype=np.int64)
    assert sorted(perm.tolist()) == list(range(w.num_blocks))
    inv = np.empty_like(perm)
    inv[perm] = np.arange(w.num_blocks)
    idx = torch.from_numpy(inv)
    return replace(w, name=w.name + "-permuted",
                   k_cache=w.k_cache.index_select(0, idx).contiguous(),
                   v_cache=w.v_cache.index_select(0, idx).contiguous(),
                   block_tables=perm[w.block_tables.astype(np.int64)].astype(np.int32))


def poison_unused(w: Workload) -> Workload:
    """Fill every physical block that no sequence owns with NaN, and point every
    padding table entry at one of them.  Reading any of it shows up as NaN."""
    B = w.block_size
    owned = np.zeros(w.num_blocks, dtype=bool)
    for s in range(w.num_seqs):
        if "prompts" in w.meta:
            pb = w.meta["prompt_blocks"]
            n = pb + -(-(int(w.meta["tails"][s]) + 1) // B)
        else:
            n = -(-(int(w.context_lens[s]) + 1) // B)
        owned[w.block_tables[s, :n]] = True
    free = np.flatnonzero(~owned)
    if free.size == 0:
        raise ValueError("no free block to poison")
    k = w.k_cache.clone()
    v = w.v_cache.clone()
    fidx = torch.from_numpy(free)
    k[fidx] = float("nan")
    v[fidx] = float("nan")
    tables = w.block_tables.copy()
    for s in range(w.num_seqs):
        if "prompts" in w.meta:
            n = w.meta["prompt_blocks"] + -(-(int(w.meta["tails"][s]) + 1) // B)
        else:
            n = -(-(int(w.context_lens[s]) + 1) // B)
        tables[s, n:] = free[0]
    return replace(w, name=w.name + "-poisoned", k_cache=k, v_cache=v, block_tables=tables,
                   meta={**w.meta, "free_blocks": free})
