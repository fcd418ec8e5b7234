"""GPU parity of the fused append + decode step (paged_attn_decode_append):
each sequence's new K/V row lands in slot T[L / B] * B + L % B, bit for bit
against the oracle's own slot computation, and the decode over the L + 1
tokens matches the fp64 oracle on the appended pools within the stated
tolerance.  It must also equal, bitwise, the two-launch path
(paged_kv_append_at, then paged_attn_decode of L + 1), which runs the same
plan over the same lengths.
"""
import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
from workloads import make_small, make_workload, raw_numpy
from gpu_common import assert_parity, gpu_decode, oracle_out, say, to_gpu
from test_gpu_parity import _FULL, full

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_357_amd as pk
    pk.load_library()
    return pk


def fused(pk, w, d, lens=None, P=0, max_len=None):
    lens = w.context_lens if lens is None else np.asarray(lens, dtype=np.int32)
    lens_t = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to(d.q.device)
    max_len = int(lens.max()) + 1 if max_len is None else int(max_len)
    out = pk.decode_append(d.q, d.k, d.v, d.kn, d.vn, d.tables, lens_t, w.scale, max_len, P)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def pools_equal(d, k2, v2):
    return (np.array_equal(raw_numpy(d.k.cpu()).view(np.uint8), k2.view(np.uint8))
            and np.array_equal(raw_numpy(d.v.cpu()).view(np.uint8), v2.view(np.uint8)))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("P", [0, 16, 64, 512])
def test_small_fused_step_matches_oracle(pk, k, P):
    w = make_small(k)
    lens1 = w.context_lens + 1
    dt = pk.DTYPE_BF16 if w.dtype == "bf16" else pk.DTYPE_F32
    plan = pk.plan(w.num_seqs, w.q_heads, w.kv_heads, w.head_dim, w.block_size, int(lens1.max()), dt, P)
    say(f"fused small config {k} partition {P} S={w.num_seqs} max L+1={int(lens1.max())} plan={plan}")
    d = to_gpu(w)
    out = fused(pk, w, d, P=P)
    k2, v2 = pa.oracle_append(raw_numpy(w.k_cache), raw_numpy(w.v_cache), w.block_tables, w.context_lens,
                              raw_numpy(w.k_new), raw_numpy(w.v_new), w.block_size)
    assert pools_equal(d, k2, v2), "pools differ from the oracle's append"
    ref = oracle_out(w, lens=lens1, k_cache=k2, v_cache=v2)
    assert_parity(out, ref, w, what=f"fused append + decode(L+1) P={P}")
    # the two-launch path on fresh pools: same plan, same lengths, same bits
    d2 = to_gpu(w)
    pk.append_at(d2.k, d2.v, d2.kn, d2.vn, d2.tables, d2.lens)
    out2 = gpu_decode(pk, w, d2, lens=lens1, partition_size=P, max_len=int(lens1.max()))
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), "fused and two-launch outputs differ"


# (q heads, kv heads, head_dim, block, dtype): vector core, matrix core with
# one wave per kv head, matrix core with four lockstep waves, fp32.
SHAPES = [(4, 4, 128, 16, "bf16"), (8, 2, 128, 16, "bf16"), (16, 4, 128, 32, "bf16"), (8, 2, 64, 16, "f32")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
@pytest.mark.parametrize("P", [0, 64])
def test_fused_edge_cases(pk, shape, P):
    """L = 0 attends only the new token (its V row exactly); an invalid
    length, a length whose L + 1 exceeds the bound, and a bad table entry at
    the append block give NaN rows and write nothing; a length that is a
    multiple of B lands at offset 0 of its next block; the other rows match
    the oracle.  The lengths put one sequence past 512 so P = 0 runs the
    balanced schedule."""
    Hq, Hkv, D, B, dtype = shape
    base = np.array([600, 1, 40, 300, 70, 1000, 17, 5], dtype=np.int64)
    w = make_workload("fused-edges", base, Hq, Hkv, D, B, dtype, 358901)
    G = Hq // Hkv
    maxL = int(base.max()) + 1
    lens = base.copy()
    lens[0] = 0
    lens[1] = -3
    lens[2] = maxL            # L + 1 beyond the bound
    lens[4] = (base[4] // B) * B  # a multiple of B: offset 0 of the block after its last full one
    tables = w.block_tables.copy()
    tables[3, lens[3] // B] = w.num_blocks + 5  # the append block's entry outside the pool
    d = to_gpu(w)
    d.tables = torch.from_numpy(np.ascontiguousarray(tables)).cuda()
    say(f"fused edges {shape} P={P}")
    out = fused(pk, w, d, lens=lens, P=P, max_len=maxL)
    keep = lens.copy()
    keep[[1, 2, 3]] = -1
    k2, v2 = pa.oracle_append(raw_numpy(w.k_cache), raw_numpy(w.v_cache), w.block_tables, keep,
                              raw_numpy(w.k_new), raw_numpy(w.v_new), B)
    assert pools_equal(d, k2, v2), "pools differ from the oracle's append"
    vn = w.v_new.float().numpy()
    for h in range(Hq):
        assert np.array_equal(out[0, h], vn[0, h // G]), "L = 0 must return the new V row"
    for s in (1, 2, 3):
        assert np.all(np.isnan(out[s])), s
    rest = [0, 4, 5, 6, 7]
    ref = oracle_out(w, lens=keep + 1, seqs=rest, k_cache=k2, v_cache=v2)
    assert_parity(out, ref, w, seqs=rest, what=f"fused edge rows P={P}")


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_full_fused_step(pk, k):
    """The benchmark's step at full size (its launch configuration: automatic
    plan, bound max(L) + 1): slot rows bit for bit, every other row and every
    shared prompt block untouched, outputs bitwise equal to the two-launch
    path and within tolerance of the oracle on sampled sequences."""
    w, d = full(k)
    B = w.block_size
    lens1 = w.context_lens + 1
    dt = pk.DTYPE_BF16 if w.dtype == "bf16" else pk.DTYPE_F32
    say(f"fused full config {k}: S={w.num_seqs} plan="
        f"{pk.plan(w.num_seqs, w.q_heads, w.kv_heads, w.head_dim, B, int(lens1.max()), dt)}")
    k0, v0 = d.k.clone(), d.v.clone()
    out = fused(pk, w, d)
    slots = pa.oracle_slot_mapping(w.block_tables, w.context_lens, B)
    ib = torch.int16 if w.dtype == "bf16" else torch.int32
    idx = torch.from_numpy(slots).cuda()
    mask = torch.ones(w.num_blocks * B, dtype=torch.bool, device="cuda")
    mask[idx] = False
    for pool, before, new in ((d.k, k0, d.kn), (d.v, v0, d.vn)):
        flat = pool.view(w.num_blocks * B, -1).view(ib)
        assert torch.equal(flat.index_select(0, idx), new.reshape(len(slots), -1).view(ib))
        assert torch.equal(flat[mask], before.view(w.num_blocks * B, -1).view(ib)[mask])
    if k == 4:
        shared = torch.from_numpy(np.unique(w.block_tables[:, :w.meta["prompt_blocks"]]).astype(np.int64))
        assert torch.equal(d.k.index_select(0, shared.cuda()).cpu(), w.k_cache.index_select(0, shared))
    # two-launch path on the original pools
    pk.append_at(k0, v0, d.kn, d.vn, d.tables, d.lens)
    out2 = gpu_decode(pk, w, d, lens=lens1, k=k0, v=v0)
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), "fused and two-launch outputs differ"
    del k0, v0
    seqs = list(range(8)) if k <= 3 else ([0, 1, 2, 3, 17, 130, 257, 511] if k == 4 else [0, 5])
    k2, v2 = raw_numpy(d.k.cpu()), raw_numpy(d.v.cpu())
    ref = oracle_out(w, lens=lens1, seqs=seqs, k_cache=k2, v_cache=v2)
    assert_parity(out, ref, w, seqs=seqs, what="fused append + decode(L+1)")
    _FULL.pop(k, None)  # the pools now differ from the generator's
