"""Plain fp64 oracle for prompt (prefill) attention over the paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU leg,
never by the product path.

Sources (the pages this follows):
  [A] "PagedAttention Paper Breakdown: Virtual Memory Allocation for LLM KV
      Cache Serving", section 2, "Address Translation Formula": K_i of a
      sequence lives at slot T[i // B] * B + i % B.
  [B] "PagedAttention and vLLM Architecture: Virtual Memory for LLM Serving",
      section 3, item 1: a prompt is processed and its logical blocks are
      assigned physical blocks; section 2: attention reads the keys and values
      through the table and applies softmax to the scaled dot products.

Readings where the pages are silent (each one is listed in the design notes):
  * a prompt chunk of n new tokens of a sequence holding L tokens (the chunk
    included, its K and V already written) occupies positions L-n .. L-1;
    n = L is a whole prompt, n < L continues an earlier context;
  * causal attention: the token at position p attends to positions 0 .. p
    (itself and everything before it), as in autoregressive decoding;
  * GQA, scale and storage widening as in the decode oracle.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import decode_storage, gather_context, kv_head_of, softmax_attention


def chunk_positions(n: int, L: int) -> np.ndarray:
    """Positions of the n new tokens of a sequence holding L tokens."""
    assert 0 <= n <= L
    return np.arange(L - n, L, dtype=np.int64)


def oracle_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                   context_lens, q_start, scale: float, dtype: str, block_size: int, seqs=None,
                   tokens=None) -> np.ndarray:
    """fp64 causal attention of every new query row over its sequence's
    cached keys 0 .. p.

    q [total_q, Hq, D] stored bits; rows q_start[s] .. q_start[s+1]-1 belong
    to sequence s.  Returns out64 [total_q, Hq, D]; rows of sequences not in
    ``seqs`` (and, when ``tokens`` maps s to a list of chunk indices, rows
    not listed) are NaN.
    """
    total, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    scale64 = float(np.float32(scale))
    out = np.full((total, hq, d), np.nan, dtype=np.float64)
    S = len(context_lens)
    for s in (range(S) if seqs is None else seqs):
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        n, L = r1 - r0, int(context_lens[s])
        if n == 0:
            continue
        k64 = decode_storage(gather_context(k_cache, block_tables[s], L, block_size), dtype)
        v64 = decode_storage(gather_context(v_cache, block_tables[s], L, block_size), dtype)
        q64 = decode_storage(q[r0:r1], dtype)
        for t, p in enumerate(chunk_positions(n, L)):
            if tokens is not None and t not in tokens.get(s, ()):
                continue
            for h in range(hq):
                g = kv_head_of(h, group, hkv)
                o, _ = softmax_attention(q64[t, h], k64[:p + 1, g, :], v64[:p + 1, g, :], scale64)
                out[r0 + t, h] = o
    return out

