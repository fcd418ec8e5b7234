"""GPU parity of the balanced schedule against the fp64 oracle.

With automatic partitioning and a longest sequence beyond 512 tokens, the
decode cuts the chunks of all (sequence, kv head) segments into equal shares
of the resident waves; share boundaries fall inside segments, and the pieces
are merged by a second kernel (one wave per query-head row, or four waves per
row when segments are cut into many pieces).  These cases pin both merge
kernels, shares that hold many short segments, segments split over hundreds
of waves, and the special rows (empty, invalid, bad block ids) inside a
balanced batch.  Tolerances as in the other parity tests.
"""
import numpy as np
import pytest
import torch

from workloads import make_workload
from gpu_common import TOL, assert_parity, gpu_decode, oracle_out, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_357_amd as pk
    pk.load_library()
    return pk


def _dt(pk, w):
    return pk.DTYPE_BF16 if w.dtype == "bf16" else pk.DTYPE_F32


def _assert_balanced(pk, w, max_len=None):
    max_len = w.max_context_len if max_len is None else max_len
    P, W = pk.plan(w.num_seqs, w.q_heads, w.kv_heads, w.head_dim, w.block_size, max_len, _dt(pk, w))
    assert P == 0, "expected the balanced schedule"
    assert W in (1024, 2048, 3072, 4096)  # one share per resident wave: 1..4 per SIMD of 256 CUs
    return W


def _mixed_lengths(n, seed, hi=900):
    rng = np.random.default_rng(seed)
    lens = np.clip(np.rint(rng.lognormal(np.log(60.0), 1.0, size=n)), 1, hi).astype(np.int64)
    lens[0] = hi  # the longest sequence exceeds one partition
    return lens


@pytest.mark.parametrize("dtype,hq,hkv,D,B", [("bf16", 2, 2, 128, 16), ("bf16", 8, 2, 128, 32),
                                              ("f32", 2, 2, 64, 16), ("bf16", 4, 2, 64, 16),
                                              ("f32", 4, 2, 64, 32)])
def test_many_short_segments_narrow_merge(pk, dtype, hq, hkv, D, B):
    """Hundreds of short sequences: shares hold many whole segments plus a
    piece at each end; few pieces per segment select the one-wave merge."""
    lens = _mixed_lengths(700, 11 + hq + D)
    w = make_workload(f"short-{dtype}-{hq}-{hkv}-{D}-{B}", lens, hq, hkv, D, B, dtype, 5150 + D + hq)
    W = _assert_balanced(pk, w)
    assert W < 8 * w.num_seqs * w.kv_heads  # one-wave merge
    say(f"{w.name}: S={w.num_seqs} sum L={int(lens.sum())} workers={W}")
    out = gpu_decode(pk, w, to_gpu(w))
    assert_parity(out, oracle_out(w), w, what="balanced, narrow merge")


@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 8, 1), ("bf16", 2, 2), ("f32", 1, 1)])
def test_one_long_sequence_over_all_workers(pk, dtype, hq, hkv):
    """A single sequence: every worker holds a piece of the same segments,
    hundreds of pieces per row go through the four-wave merge."""
    L = 12000 if dtype == "bf16" else 6000
    w = make_workload(f"one-long-{dtype}-{hq}-{hkv}", [L], hq, hkv, 128 if dtype == "bf16" else 64, 16, dtype,
                      6160 + hq)
    _assert_balanced(pk, w)
    out = gpu_decode(pk, w, to_gpu(w))
    assert_parity(out, oracle_out(w), w, what="balanced, one sequence")


def test_special_rows_inside_a_balanced_batch(pk):
    w = make_workload("special-balanced", _mixed_lengths(64, 3, hi=2000), 8, 2, 128, 16, "bf16", 6170)
    _assert_balanced(pk, w)
    d = to_gpu(w)
    lens = w.context_lens.copy()
    maxL = int(lens.max())
    lens[1] = 0
    lens[2] = 1
    lens[3] = -5
    lens[4] = maxL + 3
    out = gpu_decode(pk, w, d, lens=lens, max_len=maxL)
    assert np.all(out[1] == 0)
    v = w.v_cache.float().numpy()
    p0 = int(w.block_tables[2, 0])
    for h in range(w.q_heads):
        assert np.array_equal(out[2, h], v[p0, 0, h // w.group])
    assert np.all(np.isnan(out[3])) and np.all(np.isnan(out[4]))
    ok = [s for s in range(w.num_seqs) if s not in (1, 2, 3, 4)]
    ref = oracle_out(w, lens=np.where(lens < 0, 0, np.minimum(lens, maxL)), seqs=ok)
    assert_parity(out, ref, w, seqs=ok, what="rows next to special ones")
    # a block id outside the pool is never read and turns its sequence's rows into NaN
    t = w.block_tables.copy()
    t[0, 3] = w.num_blocks + 7
    d.tables = torch.from_numpy(t).cuda()
    out = gpu_decode(pk, w, d)
    assert np.all(np.isnan(out[0]))
    ok = list(range(1, w.num_seqs))
    assert_parity(out, oracle_out(w, seqs=ok), w, seqs=ok, what="rows next to a bad table")


def test_all_rows_empty_or_invalid(pk):
    w = make_workload("empty-balanced", [700, 5, 40], 4, 4, 128, 16, "bf16", 6180)
    d = to_gpu(w)
    for lens in ([0, 0, 0], [0, -1, 0], [800, 0, 900]):
        out = gpu_decode(pk, w, d, lens=np.array(lens, np.int32), max_len=700)
        for s, L in enumerate(lens):
            if L == 0:
                assert np.all(out[s] == 0)
            else:
                assert np.all(np.isnan(out[s]))


def test_stages_equal_whole_call_balanced(pk):
    w = make_workload("stages-balanced", _mixed_lengths(40, 9, hi=3000), 16, 4, 128, 16, "bf16", 6190)
    d = to_gpu(w)
    call = pk.DecodeCall(d.q, d.k, d.v, d.tables, d.lens, w.scale, w.max_context_len)
    assert call.plan[0] == 0
    a = call.run().clone()
    call.out.fill_(float("nan"))
    call.partitions()
    call.reduce()
    torch.cuda.synchronize()
    assert torch.equal(a, call.out)
    again = call.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, again), "not deterministic"


def test_balanced_and_partitioned_agree(pk):
    """The two schedules group tokens differently; both are within the
    tolerance of the oracle and of each other."""
    w = make_workload("both-schedules", _mixed_lengths(96, 21, hi=2500), 32, 8, 128, 32, "bf16", 6200)
    d = to_gpu(w)
    a = gpu_decode(pk, w, d)             # balanced
    b = gpu_decode(pk, w, d, partition_size=512)
    ref = oracle_out(w)
    assert_parity(a, ref, w, what="balanced")
    assert_parity(b, ref, w, what="partitioned")
    assert float(np.max(np.abs(a.astype(np.float64) - b))) <= 2 * TOL[w.dtype]


def _queue_workload(case):
    rng = np.random.default_rng(358777 if case.startswith("g16") else (358781 if case.startswith("g4") else 358778))
    if case.startswith("g16"):
        lens = rng.integers(1, 41, size=2048)
        lens[17] = 700
        return make_workload("queue-g16", lens, 64, 4, 128, 16, "bf16", 358779), 17
    if case.startswith("g4"):  # matrix-core kernel, four lockstep waves per worker
        lens = rng.integers(1, 25, size=2048)
        lens[900] = 600
        return make_workload("queue-g4", lens, 64, 16, 128, 16, "bf16", 358782), 900
    lens = rng.integers(1, 25, size=2048)
    lens[1000] = 600
    return make_workload("queue-g1", lens, 16, 16, 128, 16, "bf16", 358780), 1000


@pytest.mark.parametrize("case", ["g16-three-records", "g1-many-segments"])
def test_piece_queue_flushes_mid_stream(pk, case):
    """Each wave keeps its finished pieces in an LDS queue and writes them out
    at its end, or when the queue is full.  Group 16 at head_dim 128 takes
    8 KiB a record, three per wave, against about 8 pieces per wave (2048
    sequences x 4 kv heads); 2048 short sequences with 16 kv heads give each
    wave about 32 pieces.  Every row is compared with the partitioned
    schedule, and a sample with the oracle."""
    w, long_seq = _queue_workload(case)
    _assert_balanced(pk, w)
    d = to_gpu(w)
    say(f"{case}: S={w.num_seqs} G={w.group} sum L={int(w.context_lens.sum())}")
    out = gpu_decode(pk, w, d)
    part = gpu_decode(pk, w, d, partition_size=512)
    e = float(np.max(np.abs(out.astype(np.float64) - part)))
    say(f"{case}: max|balanced - partitioned| = {e:.3e}")
    assert np.all(np.isfinite(out)) and e <= TOL[w.dtype]
    seqs = sorted(set(range(0, w.num_seqs, max(1, w.num_seqs // 40))) | {long_seq, w.num_seqs - 1})
    ref = oracle_out(w, seqs=seqs)
    assert_parity(out, ref, w, seqs=seqs, what="queued pieces")


@pytest.mark.parametrize("case", ["g1-many-segments", "g4-many-segments"])
def test_fused_append_rows_beyond_the_row_store(pk, case):
    """The fused append keeps about 18-21 new rows per wave in LDS; 2048
    short sequences with 16 kv heads end about 32 segments per wave (vector
    core, and matrix core with four lockstep heads per worker), so the rest
    are written to the pool before their segments are read.  Pools and
    outputs must equal the two-launch path (append_at, then the decode of
    L + 1) bit for bit, and a sample must match the oracle."""
    import oracle.paged_attention as pa
    from workloads import raw_numpy
    w, long_seq = _queue_workload(case)
    lens1 = w.context_lens + 1
    dt = _dt(pk, w)
    assert pk.plan(w.num_seqs, w.q_heads, w.kv_heads, w.head_dim, w.block_size, int(lens1.max()), dt)[0] == 0
    d = to_gpu(w)
    out = pk.decode_append(d.q, d.k, d.v, d.kn, d.vn, d.tables, d.lens, w.scale, int(lens1.max()))
    torch.cuda.synchronize()
    d2 = to_gpu(w)
    pk.append_at(d2.k, d2.v, d2.kn, d2.vn, d2.tables, d2.lens)
    out2 = gpu_decode(pk, w, d2, lens=lens1, max_len=int(lens1.max()))
    assert torch.equal(d.k, d2.k) and torch.equal(d.v, d2.v), "pools differ from the two-launch path"
    out = out.cpu().numpy()
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), "outputs differ from the two-launch path"
    k2, v2 = raw_numpy(d.k.cpu()), raw_numpy(d.v.cpu())
    seqs = sorted(set(range(0, w.num_seqs, 50)) | {long_seq, w.num_seqs - 1})
    ref = oracle_out(w, lens=lens1, seqs=seqs, k_cache=k2, v_cache=v2)
    assert_parity(out, ref, w, seqs=seqs, what="fused rows beyond the row store")
