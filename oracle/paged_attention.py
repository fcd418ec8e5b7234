"""Plain fp64 oracle for paged decode attention and the KV slot write.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Sources (the pages this follows):
  [A] "PagedAttention Paper Breakdown: Virtual Memory Allocation for LLM KV
      Cache Serving", section 2, "Address Translation Formula": logical block
      b = floor(i / B), offset o = i mod B, and K_i lives at T[b] * B + o.
  [B] "PagedAttention and vLLM Architecture: Virtual Memory for LLM Serving",
      section 1: each physical page holds both the Key and the Value tensors of
      B tokens, so K and V share one table and one slot.
  [C] same page, section 2, "PagedAttention Attention CUDA Kernel Mechanics":
      for the decode step the query of the new token is dotted with every
      cached key, fetched block by block through the table, and an online
      softmax plus the product with the Value blocks finishes the step.  An
      online softmax reaches, up to rounding, exactly what the textbook
      softmax reaches, so the oracle is that definition written out:
          x_i = scale * <q, K_i>,  w = softmax(x),  out = sum_i w_i V_i
      over the logical positions i = 0 .. L-1.
  [D] same page, "Why Internal Fragmentation is Bounded": a sequence gets a new
      block only when a token overflows its last one; the appended token of a
      sequence with L cached tokens sits at logical position L.

Readings where the pages are silent (each one is listed in the design notes):
  * the value T[b] * B + o is a token-slot index into the pool viewed as
    [num_blocks * B] rows of [kv_heads, head_dim];
  * query head h reads kv head h // G (G = q_heads / kv_heads, contiguous
    groups);
  * decode attends to positions 0 .. L-1; the append writes position L;
  * L = 0 gives an all-zero output;
  * the stored bf16 / fp32 bits are the inputs; they are widened exactly to
    fp64 and all arithmetic is fp64, with the fp32 scale widened exactly.
"""
from __future__ import annotations

import numpy as np


def decode_storage(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to fp64 exactly.  bf16 bits are the top half of an
    IEEE binary32, so shifting them up 16 bits gives the same number as fp32."""
    if dtype == "bf16":
        assert raw.dtype == np.uint16
        return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        assert raw.dtype == np.float32
        return raw.astype(np.float64)
    raise ValueError(dtype)


def slot_of(table_row, i: int, block_size: int) -> int:
    """[A]: the slot of logical token i of a sequence whose block table is table_row."""
    b = i // block_size
    o = i % block_size
    return int(table_row[b]) * block_size + o


def kv_head_of(h: int, group: int, kv_heads: int) -> int:
    """Reading: query head h shares the kv head h // G (contiguous groups of G
    query heads per kv head, G = q_heads / kv_heads)."""
    g = h // group
    assert 0 <= g < kv_heads
    return g


def oracle_slot_mapping(block_tables: np.ndarray, positions, block_size: int) -> np.ndarray:
    """[A] + [D]: the slot each sequence's next token is written to (its logical
    position is its current length).  A negative position maps to -1 (no write)."""
    out = np.empty(len(positions), dtype=np.int64)
    for s, pos in enumerate(positions):
        pos = int(pos)
        out[s] = -1 if pos < 0 else slot_of(block_tables[s], pos, block_size)
    return out


def oracle_append(k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                  positions, k_new: np.ndarray, v_new: np.ndarray, block_size: int):
    """[B] + [D]: write each new token's K and V rows ([kv_heads, head_dim],
    stored bits, no conversion) into its slot.  Returns new pools; the inputs
    are left untouched."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    nb, bs, hkv, d = kc.shape
    assert bs == block_size
    kflat = kc.reshape(nb * bs, hkv, d)
    vflat = vc.reshape(nb * bs, hkv, d)
    for s, pos in enumerate(positions):
        pos = int(pos)
        if pos < 0:
            continue
        slot = slot_of(block_tables[s], pos, block_size)
        kflat[slot] = k_new[s]
        vflat[slot] = v_new[s]
    return kc, vc


def gather_context(cache: np.ndarray, table_row, length: int, block_size: int) -> np.ndarray:
    """[A] + [C]: the rows of logical positions 0 .. length-1, fetched one token
    at a time through the table.  Returns [length, kv_heads, head_dim] raw."""
    nb, bs, hkv, d = cache.shape
    flat = cache.reshape(nb * bs, hkv, d)
    slots = [slot_of(table_row, i, block_size) for i in range(length)]
    return flat[np.asarray(slots, dtype=np.int64)] if slots else np.zeros((0, hkv, d), cache.dtype)


def softmax_attention(q64: np.ndarray, k64: np.ndarray, v64: np.ndarray, scale64: float):
    """[C]: textbook softmax attention of one query row over L keys and values.
    q64 [D], k64 [L, D], v64 [L, D], all fp64.  Returns (out [D], weights [L])."""
    x = scale64 * (k64 @ q64)
    m = np.max(x)
    e = np.exp(x - m)
    w = e / np.sum(e)
    return w @ v64, w


def oracle_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  block_tables: np.ndarray, context_lens, scale: float, dtype: str,
                  block_size: int, seqs=None, return_weights: bool = False):
    """[C]: fp64 paged decode attention.

    q [S, Hq, D], k_cache / v_cache [NB, B, Hkv, D]: stored bits (uint16 for
    bf16, float32 for f32).  Returns out64 [S, Hq, D] (rows of sequences not in
    ``seqs`` are NaN), plus the weights {(s, h): w} if asked.
    """
    S, hq, d = q.shape
    hkv = k_cache.shape[2]
    assert hq % hkv == 0
    group = hq // hkv
    scale64 = float(np.float32(scale))
    out = np.full((S, hq, d), np.nan, dtype=np.float64)
    weights = {}
    seqs = range(S) if seqs is None else seqs
    for s in seqs:
        L = int(context_lens[s])
        if L == 0:
            out[s] = 0.0
            continue
        assert 1 <= L <= block_tables.shape[1] * block_size
        k64 = decode_storage(gather_context(k_cache, block_tables[s], L, block_size), dtype)
        v64 = decode_storage(gather_context(v_cache, block_tables[s], L, block_size), dtype)
        q64 = decode_storage(q[s], dtype)
        for h in range(hq):
            g = kv_head_of(h, group, hkv)
            o, w = softmax_attention(q64[h], k64[:, g, :], v64[:, g, :], scale64)
            out[s, h] = o
            if return_weights:
                weights[(s, h)] = w
    return (out, weights) if return_weights else out


def oracle_decode_sampled(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                          block_size, seqs):
    """Only the listed sequences (for workloads too large to check whole);
    returns {s: out64[Hq, D]}."""
    out = oracle_decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                        block_size, seqs=seqs)
    return {int(s): out[s] for s in seqs}
