"""The no-allocation decode entry point (paged_attn_decode_noalloc) against
the workspace form (paged_attn_decode), through the C ABI: both run the same
plan and kernels, so the outputs must be bitwise equal, and both within the
stated tolerance of the oracle.  Two calls in a row share the one scratch
array of the GPU; the second, smaller one must not see the first one's
leftovers."""
from dataclasses import replace
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from workloads import make_small, make_workload
from gpu_common import assert_parity, gpu_decode, oracle_out, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_357_amd as pk
    pk.load_library()
    return pk


def _noalloc(pk, w, d, partition_size=0, lens=None):
    lens = w.context_lens if lens is None else np.asarray(lens, dtype=np.int32)
    lens_t = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to(d.q.device)
    out = torch.full((w.num_seqs, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device=d.q.device)
    pk.decode_noalloc(d.q, d.k, d.v, d.tables, lens_t, w.scale, int(lens.max()), out, partition_size)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _cases():
    # balanced schedule (a sequence beyond 512 tokens): vector-ALU and matrix-core kernels
    big_valu = make_workload("noalloc-valu", [1400, 37, 900, 1], 8, 8, 128, 16, "bf16", 361001)
    big_mfma = make_workload("noalloc-mfma", [2100, 700, 1, 1500, 64], 32, 4, 128, 32, "bf16", 361002)
    return [("balanced vector-ALU", big_valu, 0), ("balanced matrix-core", big_mfma, 0),
            ("partitioned", make_small(5), 256), ("single partition", make_small(1), 0)]


@pytest.mark.parametrize("i", range(4))
def test_noalloc_equals_workspace_call_twice(pk, i):
    label, w, P = _cases()[i]
    say(f"no-alloc {label}: {w.name} S={w.num_seqs} max L={w.max_context_len} P={P}")
    d = to_gpu(w)
    ref = gpu_decode(pk, w, d, partition_size=P)
    first = _noalloc(pk, w, d, P)
    assert np.array_equal(first.view(np.uint32), ref.view(np.uint32)), label
    assert_parity(first, oracle_out(w), w, what=f"no-alloc {label}")
    # second call, smaller input: the first sequences with shorter lengths
    n = max(1, w.num_seqs - 1)
    lens2 = np.maximum(w.context_lens[:n] // 2, 1).astype(np.int32)
    sub = replace(w, context_lens=lens2, block_tables=w.block_tables[:n].copy(), q=w.q[:n].contiguous())
    d2 = SimpleNamespace(q=d.q[:n].contiguous(), k=d.k, v=d.v, tables=d.tables[:n].contiguous())
    ref2 = gpu_decode(pk, sub, d2, partition_size=P)
    second = _noalloc(pk, sub, d2, P)
    assert np.array_equal(second.view(np.uint32), ref2.view(np.uint32)), label
    assert_parity(second, oracle_out(sub), sub, what=f"no-alloc {label}, second call")
