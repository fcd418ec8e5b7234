"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin is a plain function that raises AssertionError when the oracle is
wrong.  The last test plants mistakes in the oracle (on the CPU, by patching
one of its functions) and checks that the pins catch every one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
from workloads import make_small, make_workload, permute_pool, raw_numpy, identity_tables

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_ranges(name):
    B = None
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "block_size":
                B = int(parts[1])
            else:
                rows.append(tuple(int(x) for x in parts))
    return B, rows


def _read_kv(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                d[k] = float(v)
    return d


def _run(w, lens=None, seqs=None, return_weights=False):
    lens = w.context_lens if lens is None else lens
    return pa.oracle_decode(raw_numpy(w.q), raw_numpy(w.k_cache), raw_numpy(w.v_cache), w.block_tables,
                            lens, w.scale, w.dtype, w.block_size, seqs=seqs, return_weights=return_weights)


# --------------------------------------------------------------------------- pins

def pin_worked_examples():
    """P1/P2: the two address-translation examples printed on the pages."""
    for fname in ("address_translation_block17_block4.txt", "address_translation_block7_1_12.txt"):
        B, rows = _read_ranges(fname)
        table = [phys for (_, _, phys) in rows]
        for first, last, phys in rows:
            for i in range(first, last + 1):
                slot = pa.slot_of(table, i, B)
                assert slot // B == phys, (fname, i, slot)
                assert slot % B == i - first, (fname, i, slot)
    # the token after the first block of the first example opens block 4 at offset 0
    assert pa.oracle_slot_mapping(np.array([[17, 4]]), [16], 16).tolist() == [64]


def pin_permutation_invariance():
    """P3: relabelling physical blocks changes nothing (bitwise: same fp64 op order)."""
    for k in (2, 3, 4):
        w = make_small(k)
        perm = np.random.default_rng(11 + k).permutation(w.num_blocks)
        a = _run(w)
        b = _run(permute_pool(w, perm))
        assert np.array_equal(a, b), k


def pin_identity_equals_contiguous():
    """P4: with an identity table the pool, read in order, is each sequence's
    contiguous cache, and paged attention equals torch's scaled-dot-product
    attention on it (fp64 on the CPU; torch widens the stored bits itself)."""
    for k in (1, 2, 3, 5):
        w = identity_tables(make_small(k))
        S, MB, B = w.num_seqs, w.max_blocks_per_seq, w.block_size
        out = _run(w)
        kc = w.k_cache.to(torch.float64).reshape(S, MB * B, w.kv_heads, w.head_dim)
        vc = w.v_cache.to(torch.float64).reshape(S, MB * B, w.kv_heads, w.head_dim)
        for s in range(S):
            L = int(w.context_lens[s])
            K = kc[s, :L].permute(1, 0, 2).repeat_interleave(w.group, dim=0).unsqueeze(0)
            V = vc[s, :L].permute(1, 0, 2).repeat_interleave(w.group, dim=0).unsqueeze(0)
            q = w.q[s].to(torch.float64).unsqueeze(0).unsqueeze(2)
            ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=w.scale)
            ref = ref[0, :, 0, :].numpy()
            assert np.max(np.abs(out[s] - ref)) <= 1e-12, (k, s)


def pin_cow_siblings():
    """P5: (i) siblings that alias the prompt blocks give the same output as
    siblings holding private copies of them; (ii) siblings with the same q and
    no private tail give identical outputs."""
    w = make_small(4)
    n_prompts, n_sib, prompt_len = w.meta["prompts"]
    pb = w.meta["prompt_blocks"]
    # private copies: every sibling but the first of each prompt gets new blocks
    extra = []
    tables = w.block_tables.astype(np.int64).copy()
    nxt = w.num_blocks
    for s in range(w.num_seqs):
        if s % n_sib == 0:
            continue
        for b in range(pb):
            extra.append(int(tables[s, b]))
            tables[s, b] = nxt
            nxt += 1
    idx = torch.tensor(extra, dtype=torch.long)
    kc = torch.cat([w.k_cache, w.k_cache.index_select(0, idx)])
    vc = torch.cat([w.v_cache, w.v_cache.index_select(0, idx)])
    a = _run(w)
    b = pa.oracle_decode(raw_numpy(w.q), raw_numpy(kc), raw_numpy(vc), tables, w.context_lens, w.scale,
                         w.dtype, w.block_size)
    assert np.array_equal(a, b)
    w2 = make_small(4, shared_q=True, zero_tails=True)
    o2 = _run(w2)
    for j in range(n_prompts):
        for k in range(1, n_sib):
            assert np.array_equal(o2[j * n_sib], o2[j * n_sib + k])
    # and distinct prompts really differ
    assert not np.array_equal(o2[0], o2[n_sib])


def pin_weights_sum_to_one():
    """P6: softmax weights of every (sequence, head) sum to 1."""
    for k in (1, 3, 5):
        w = make_small(k)
        _, ws = _run(w, return_weights=True)
        for key, wt in ws.items():
            assert abs(wt.sum() - 1.0) <= 1e-12, key
            assert np.all(wt >= 0)


def pin_single_token_returns_v0():
    """P7: a context of one token returns that token's V row exactly."""
    for k in (1, 2, 3):
        w = make_small(k)
        lens = np.ones(w.num_seqs, dtype=np.int32)
        out = _run(w, lens=lens)
        v = w.v_cache.to(torch.float64).numpy()
        for s in range(w.num_seqs):
            p = int(w.block_tables[s, 0])
            for h in range(w.q_heads):
                assert np.array_equal(out[s, h], v[p, 0, h // w.group]), (k, s, h)


def _brute(qf, kpool, vpool, table, L, B, scale, G):
    """Independent scalar reference: nested Python loops and math.exp."""
    Hq, D = len(qf), len(qf[0])
    res = []
    for h in range(Hq):
        g = h // G
        xs = []
        for i in range(L):
            blk = table[i // B]
            off = i - (i // B) * B
            xs.append(scale * sum(qf[h][d] * kpool[blk][off][g][d] for d in range(D)))
        m = max(xs)
        es = [math.exp(x - m) for x in xs]
        z = sum(es)
        row = []
        for d in range(D):
            acc = 0.0
            for i in range(L):
                blk = table[i // B]
                off = i - (i // B) * B
                acc += es[i] / z * vpool[blk][off][g][d]
            row.append(acc)
        res.append(row)
    return res


def pin_brute_force():
    """P8: every B in {1,2,4}, L in 1..9, D in {1,2}, G in {1,2}, random tables."""
    rng = np.random.default_rng(4242)
    for B in (1, 2, 4):
        for D in (1, 2):
            for G in (1, 2):
                Hkv = 2
                Hq = Hkv * G
                for L in range(1, 10):
                    nb = -(-L // B)
                    NB = nb + 3
                    table = rng.permutation(NB)[:nb]
                    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
                    kp = rng.standard_normal((NB, B, Hkv, D)).astype(np.float32)
                    vp = rng.standard_normal((NB, B, Hkv, D)).astype(np.float32)
                    scale = float(np.float32(0.7))
                    out = pa.oracle_decode(q, kp, vp, table[None, :], [L], scale, "f32", B)
                    ref = _brute(q[0].astype(float).tolist(), kp.astype(float).tolist(),
                                 vp.astype(float).tolist(), table.tolist(), L, B, scale, G)
                    assert np.max(np.abs(out[0] - np.array(ref))) <= 1e-13, (B, D, G, L)


def _needle_inputs(w, s, n):
    """K = 0 except K_n[g, 0] = 16 for every kv head; q[:, 0] = 16, rest 0."""
    q = np.zeros_like(raw_numpy(w.q))
    k = np.zeros_like(raw_numpy(w.k_cache))
    one6 = np.float32(16.0)
    if w.dtype == "bf16":
        one6 = np.uint16(0x4180)  # 16.0 in bf16
    q[:, :, 0] = one6
    slot = pa.slot_of(w.block_tables[s], n, w.block_size)
    k.reshape(-1, w.kv_heads, w.head_dim)[slot, :, 0] = one6
    return q, k


def pin_needle():
    """P9: scores 256 at position n and 0 elsewhere; e^-256 vanishes, so the
    output is V_n (closed form)."""
    for kcfg in (1, 2, 5):
        w = make_small(kcfg)
        v64 = pa.decode_storage(raw_numpy(w.v_cache), w.dtype)
        for s in range(w.num_seqs):
            L = int(w.context_lens[s])
            for n in sorted({0, L // 2, L - 1}):
                q, k = _needle_inputs(w, s, n)
                out = pa.oracle_decode(q, k, raw_numpy(w.v_cache), w.block_tables, w.context_lens, 1.0,
                                       w.dtype, w.block_size, seqs=[s])
                slot = pa.slot_of(w.block_tables[s], n, w.block_size)
                vn = v64.reshape(-1, w.kv_heads, w.head_dim)[slot]
                for h in range(w.q_heads):
                    assert np.max(np.abs(out[s, h] - vn[h // w.group])) <= 1e-100, (kcfg, s, n, h)


def position_sum_inputs(w):
    """q = 0 (uniform weights); V_i[g, 0] = i mod 256, V_i[g, 1] = i div 256,
    written at each logical position's slot; every other V element 0."""
    q = np.zeros_like(raw_numpy(w.q))
    v = np.zeros_like(raw_numpy(w.v_cache))
    flat = v.reshape(-1, w.kv_heads, w.head_dim)
    for s in range(w.num_seqs):
        for i in range(int(w.context_lens[s])):
            slot = pa.slot_of(w.block_tables[s], i, w.block_size)
            a, b = float(i % 256), float(i // 256)
            if w.dtype == "bf16":
                a = np.array([a], np.float32).view(np.uint32)[0] >> 16
                b = np.array([b], np.float32).view(np.uint32)[0] >> 16
            flat[slot, :, 0] = a
            flat[slot, :, 1] = b
    return q, v


def pin_position_sum():
    """P10: uniform weights make the output the mean of the V rows; the means
    of i mod 256 and i div 256 over 0..L-1 have closed forms."""
    for kcfg in (1, 2, 3, 5):
        w = make_small(kcfg)
        q, v = position_sum_inputs(w)
        out = pa.oracle_decode(q, raw_numpy(w.k_cache), v, w.block_tables, w.context_lens, w.scale,
                               w.dtype, w.block_size)
        for s in range(w.num_seqs):
            L = int(w.context_lens[s])
            full, rem = divmod(L, 256)
            mod_sum = full * (255 * 256 // 2) + rem * (rem - 1) // 2
            div_sum = 256 * (full * (full - 1) // 2) + full * rem
            assert np.allclose(out[s, :, 0], mod_sum / L, rtol=1e-13, atol=0), (kcfg, s)
            assert np.allclose(out[s, :, 1], div_sum / L, rtol=1e-13, atol=1e-15), (kcfg, s)
            assert np.all(out[s, :, 2:] == 0)


def pin_gqa_equals_repeated_mha():
    """P11: grouped heads give what full multi-head attention gives with every
    kv head repeated G times in place."""
    for kcfg in (3, 5):
        w = make_small(kcfg)
        G = w.group
        assert G > 1
        a = _run(w)
        kr = w.k_cache.repeat_interleave(G, dim=2).contiguous()
        vr = w.v_cache.repeat_interleave(G, dim=2).contiguous()
        b = pa.oracle_decode(raw_numpy(w.q), raw_numpy(kr), raw_numpy(vr), w.block_tables, w.context_lens,
                             w.scale, w.dtype, w.block_size)
        assert np.array_equal(a, b)


def pin_fragmentation_bound():
    """P12: only a sequence's last block is partly empty; the page's numbers."""
    g = _read_kv("fragmentation_bound.txt")
    B = int(g["block_size"])
    L = int(g["avg_context"])
    blocks = -(-L // B)
    idle = blocks * B - L
    assert idle <= g["max_idle_slots"] and idle / L <= g["max_waste_fraction"]
    assert (blocks, idle) == (32, 12)
    for k in (1, 2, 3, 4, 5):
        w = make_small(k)
        for s in range(w.num_seqs):
            L = int(w.context_lens[s])
            owned = -(-(L + 1) // w.block_size)
            assert owned * w.block_size - (L + 1) <= w.block_size - 1
            # the table covers the append position
            assert owned <= w.max_blocks_per_seq


def pin_append():
    """P13: the new rows land at the oracle's slots bit for bit, every other
    byte of both pools is unchanged, shared prompt blocks are untouched, and a
    length that is a multiple of B writes offset 0 of the next table entry."""
    for k in (1, 2, 4):
        w = make_small(k)
        kc, vc = raw_numpy(w.k_cache), raw_numpy(w.v_cache)
        kn, vn = raw_numpy(w.k_new), raw_numpy(w.v_new)
        k2, v2 = pa.oracle_append(kc, vc, w.block_tables, w.context_lens, kn, vn, w.block_size)
        B = w.block_size
        slots = pa.oracle_slot_mapping(w.block_tables, w.context_lens, B)
        assert len(set(slots.tolist())) == len(slots)
        kf, vf = k2.reshape(-1, w.kv_heads, w.head_dim), v2.reshape(-1, w.kv_heads, w.head_dim)
        for s, slot in enumerate(slots):
            assert np.array_equal(kf[slot].view(np.uint8), kn[s].view(np.uint8))
            assert np.array_equal(vf[slot].view(np.uint8), vn[s].view(np.uint8))
            L = int(w.context_lens[s])
            assert slot == int(w.block_tables[s, L // B]) * B + L % B
            if L % B == 0:
                assert slot % B == 0 and slot // B == int(w.block_tables[s, L // B])
        mask = np.ones(kf.shape[0], dtype=bool)
        mask[slots] = False
        assert np.array_equal(kf[mask].view(np.uint8), kc.reshape(kf.shape)[mask].view(np.uint8))
        assert np.array_equal(vf[mask].view(np.uint8), vc.reshape(vf.shape)[mask].view(np.uint8))
        if "prompts" in w.meta:
            shared = np.unique(w.block_tables[:, :w.meta["prompt_blocks"]])
            assert np.array_equal(k2[shared].view(np.uint8), kc[shared].view(np.uint8))
    # decode after append attends to the new token at position L
    w = make_small(2)
    k2, v2 = pa.oracle_append(raw_numpy(w.k_cache), raw_numpy(w.v_cache), w.block_tables, w.context_lens,
                              raw_numpy(w.k_new), raw_numpy(w.v_new), w.block_size)
    out = pa.oracle_decode(raw_numpy(w.q), k2, v2, w.block_tables, w.context_lens + 1, w.scale, w.dtype,
                           w.block_size, seqs=[0])
    L = int(w.context_lens[0])
    kk = pa.decode_storage(pa.gather_context(k2, w.block_tables[0], L + 1, w.block_size), w.dtype)
    assert np.array_equal(kk[L], pa.decode_storage(raw_numpy(w.k_new)[0], w.dtype))
    assert np.all(np.isfinite(out[0]))


PINS = [pin_worked_examples, pin_permutation_invariance, pin_identity_equals_contiguous, pin_cow_siblings,
        pin_weights_sum_to_one, pin_single_token_returns_v0, pin_brute_force, pin_needle, pin_position_sum,
        pin_gqa_equals_repeated_mha, pin_fragmentation_bound, pin_append]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ------------------------------------------------------------ planted mistakes

def _mut_slot_unit(table_row, i, B):
    return int(table_row[i // B]) + i % B


def _mut_slot_reversed(table_row, i, B):
    return int(table_row[i // B]) * B + (B - 1 - i % B)


def _mut_head_mod(h, group, kv_heads):
    return h % kv_heads


_orig_gather = pa.gather_context
_orig_softmax = pa.softmax_attention
_orig_decode = pa.decode_storage


def _mut_drop_last(cache, row, L, B):
    return _orig_gather(cache, row, max(L - 1, 0), B) if L > 1 else _orig_gather(cache, row, L, B)[:0]


def _mut_extra_token(cache, row, L, B):
    rows = _orig_gather(cache, row, L, B)
    return np.concatenate([rows, rows[:1]])


def _mut_no_scale(q, k, v, scale):
    return _orig_softmax(q, k, v, 1.0)


def _mut_swap_kv(q, k, v, scale):
    return _orig_softmax(q, v, k, scale)


def _mut_sign(q, k, v, scale):
    x = scale * (k @ q)
    e = np.exp(np.min(x) - x)
    w = e / e.sum()
    return w @ v, w


def _mut_bf16_shift(raw, dtype):
    if dtype == "bf16":
        return (raw.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return _orig_decode(raw, dtype)


def _mut_f32_round(raw, dtype):
    if dtype == "f32":
        return raw.astype(np.float16).astype(np.float64)
    return _orig_decode(raw, dtype)


MUTANTS = {
    "slot_unit": ("slot_of", _mut_slot_unit),
    "slot_reversed_offset": ("slot_of", _mut_slot_reversed),
    "head_mod": ("kv_head_of", _mut_head_mod),
    "drop_last_token": ("gather_context", _mut_drop_last),
    "extra_token": ("gather_context", _mut_extra_token),
    "no_scale": ("softmax_attention", _mut_no_scale),
    "swap_kv": ("softmax_attention", _mut_swap_kv),
    "sign_flip": ("softmax_attention", _mut_sign),
    "bf16_shift": ("decode_storage", _mut_bf16_shift),
    "f32_rounding": ("decode_storage", _mut_f32_round),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(pa, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion or a crash both mean the pin noticed
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
