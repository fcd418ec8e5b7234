"""Pins of the prefill oracle (oracle/prefill.py) against things other than
itself: torch's scaled_dot_product_attention (causal, fp64) on contiguous
tables, a brute-force scalar loop, a needle that only later rows may see,
and the decode oracle for the last row of each chunk.  Planted mistakes in
the causal indexing are each caught."""
import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
import oracle.prefill as pf
from workloads import make_workload, raw_numpy


def _case(lens, n_new, hq=4, hkv=2, D=16, B=4, dtype="f32", seed=0, deal="shuffled"):
    w = make_workload(f"pf-{seed}", lens, hq, hkv, D, B, dtype, 9000 + seed, deal=deal)
    rng = np.random.default_rng(500 + seed)
    n = np.asarray(n_new, dtype=np.int64)
    q_start = np.concatenate([[0], np.cumsum(n)])
    qs = rng.standard_normal((int(q_start[-1]), hq, D)).astype(np.float32)
    if dtype == "bf16":
        qs = (torch.from_numpy(qs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    return w, q_start, qs


def _run(fn, w, q_start, qs):
    return fn(qs, raw_numpy(w.k_cache), raw_numpy(w.v_cache), w.block_tables, w.context_lens, q_start,
              w.scale, w.dtype, w.block_size)


def pin_sdpa(fn):
    for seed, (lens, n_new) in enumerate([([7, 12, 5], [7, 12, 5]), ([9, 20], [3, 8]), ([16, 1], [16, 1])]):
        w, q_start, qs = _case(lens, n_new, deal="identity", seed=seed)
        out = _run(fn, w, q_start, qs)
        k = pa.decode_storage(raw_numpy(w.k_cache), w.dtype)
        v = pa.decode_storage(raw_numpy(w.v_cache), w.dtype)
        G = w.q_heads // w.kv_heads
        for s, L in enumerate(w.context_lens):
            L = int(L)
            r0, r1 = int(q_start[s]), int(q_start[s + 1])
            n = r1 - r0
            # identity deal: the sequence's rows are consecutive slots starting at its first block
            first = int(w.block_tables[s, 0]) * w.block_size
            kk = torch.from_numpy(k.reshape(-1, w.kv_heads, w.head_dim)[first:first + L]).permute(1, 0, 2)
            vv = torch.from_numpy(v.reshape(-1, w.kv_heads, w.head_dim)[first:first + L]).permute(1, 0, 2)
            kk = kk.repeat_interleave(G, dim=0).contiguous()
            vv = vv.repeat_interleave(G, dim=0).contiguous()
            qq = torch.from_numpy(pa.decode_storage(qs[r0:r1], w.dtype)).permute(1, 0, 2).contiguous()
            pos = torch.arange(L - n, L)
            mask = torch.arange(L)[None, :] <= pos[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                                   scale=float(np.float32(w.scale)))
            assert np.allclose(out[r0:r1], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def pin_brute_force(fn):
    w, q_start, qs = _case([6, 9], [4, 9], hq=2, hkv=1, D=2, B=2, seed=11)
    out = _run(fn, w, q_start, qs)
    k = pa.decode_storage(raw_numpy(w.k_cache), w.dtype)
    v = pa.decode_storage(raw_numpy(w.v_cache), w.dtype)
    sc = float(np.float32(w.scale))
    for s in range(2):
        L = int(w.context_lens[s])
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        for t in range(r1 - r0):
            p = L - (r1 - r0) + t
            for h in range(2):
                qv = pa.decode_storage(qs[r0 + t, h], w.dtype)
                xs, vs = [], []
                for i in range(p + 1):
                    blk, off = int(w.block_tables[s, i // w.block_size]), i % w.block_size
                    xs.append(sc * sum(qv[d] * k[blk, off, 0, d] for d in range(2)))
                    vs.append(v[blk, off, 0])
                m = max(xs)
                e = [np.exp(x - m) for x in xs]
                want = sum(ei * vi for ei, vi in zip(e, vs)) / sum(e)
                assert np.allclose(out[r0 + t, h], want, rtol=0, atol=1e-13)


def pin_needle_is_causal(fn):
    w, q_start, qs = _case([24], [24], hq=2, hkv=2, D=8, B=4, seed=21)
    j = 10
    kc = raw_numpy(w.k_cache).copy()
    vc = raw_numpy(w.v_cache).copy()
    blk, off = int(w.block_tables[0, j // 4]), j % 4
    qf = qs.astype(np.float64)
    kc[blk, off] = 0
    kc[blk, off, :, 0] = 4096.0                      # key j dominates every score where it is visible
    qs2 = qs.copy()
    qs2[:, :, 0] = np.abs(qf[:, :, 0]) + 1.0
    a = fn(qs2, kc, vc, w.block_tables, w.context_lens, q_start, w.scale, w.dtype, 4)
    vc2 = vc.copy()
    vc2[blk, off] += 7.0                             # change only V_j
    b = fn(qs2, kc, vc2, w.block_tables, w.context_lens, q_start, w.scale, w.dtype, 4)
    assert np.array_equal(a[:j], b[:j]), "rows before the needle must not see it"
    vj = pa.decode_storage(vc2[blk, off], w.dtype)
    for t in range(j, 24):
        assert np.allclose(b[t], vj, rtol=0, atol=1e-9)


def pin_last_row_is_decode(fn):
    w, q_start, qs = _case([13, 30, 8], [5, 30, 1], hq=4, hkv=2, D=16, B=4, seed=31)
    out = _run(fn, w, q_start, qs)
    last = q_start[1:] - 1
    dec = pa.oracle_decode(qs[last], raw_numpy(w.k_cache), raw_numpy(w.v_cache), w.block_tables,
                           w.context_lens, w.scale, w.dtype, w.block_size)
    assert np.allclose(out[last], dec, rtol=0, atol=1e-13)


PINS = [pin_sdpa, pin_brute_force, pin_needle_is_causal, pin_last_row_is_decode]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_prefill_oracle_meets_pin(pin):
    pin(pf.oracle_prefill)


def _planted(positions):
    def fn(q, kc, vc, tables, lens, q_start, scale, dtype, B):
        saved = pf.chunk_positions
        pf.chunk_positions = positions
        try:
            return pf.oracle_prefill(q, kc, vc, tables, lens, q_start, scale, dtype, B)
        finally:
            pf.chunk_positions = saved
    return fn


PLANTED = {
    "positions-from-zero": lambda n, L: np.arange(0, n, dtype=np.int64),
    "one-too-few-keys": lambda n, L: np.arange(L - n, L, dtype=np.int64) - 1,
    "one-too-many-keys": lambda n, L: np.minimum(np.arange(L - n, L, dtype=np.int64) + 1, L - 1),
    "not-causal": lambda n, L: np.full(n, L - 1, dtype=np.int64),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_prefill_mistake_is_caught(name):
    fn = _planted(PLANTED[name])
    caught = []
    for pin in PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, name
