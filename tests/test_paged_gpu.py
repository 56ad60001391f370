"""Paged (block-table) KV views on the GPU.

Every paged call is held to the CPU oracle directly: selections bit-exact, outputs
within 1e-5 (fp32 KV) / 2e-3 (bf16), for LoD decode and prefill, two-tier, the
sparsity ablation, three-tier INT4, the dense baselines and the build (assignments and
summaries).  The view only changes addressing, so each call must also give bit for bit
what the same call gives on a strided copy of the cache.

The paged cache scatters each sequence's blocks over a shared pool in a seeded random
order, as a serving engine's block allocator leaves them."""
import numpy as np
import pytest
import torch

from hierarchical_kv_approximation_amd import lod
from oracle import oracle as orc

from lodcase import (TOL, Case, compare_index, configs, decode_and_compare, paged_copy,
                     prefill_and_compare, sample_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _paged_case(g, o, B, T, seed, bs):
    """A case whose index is built THROUGH the block table (the strided cache is kept
    only for the bit-equality checks)."""
    case = Case(g, o, B, T, seed=seed)
    Kp, Vp, table = paged_copy(case.Kd, case.Vd, bs, seed=seed + 1)
    lod.build_chunk(g, case.index, Kp, Vp, 0, T // 256, block_table=table)
    torch.cuda.synchronize()
    return case, (Kp, Vp, table)


@pytest.mark.parametrize("dtype,hq,hkv,bs,TP", [
    (torch.bfloat16, 16, 2, 16, 2),
    (torch.bfloat16, 16, 2, 128, 0),    # two-tier
    (torch.bfloat16, 64, 8, 1, 2),      # one position per block
    (torch.float32, 4, 2, 32, 2),       # fp32 caches (VALU kernels)
])
def test_paged_lod_against_oracle(dtype, hq, hkv, bs, TP):
    bf = dtype == torch.bfloat16
    g, o = configs(dtype, hq, hkv, G=8, TP=TP, W=512 if bf else 256, S=4 if bf else 1)
    B, T = 2, 4096
    case, view = _paged_case(g, o, B, T, 71, bs)
    keys = [(b, h) for b in range(B) for h in range(hkv)]
    st, oidx = case.oracle_index(keys)
    for b, h in keys:  # assignments, layout and summaries built through the table
        compare_index(case.index, oidx[(b, h)], b, h, case.nchunks)
    decode_and_compare(case, (st, oidx), [T, 2345], case.queries(seed=73), view=view)
    Q = case.queries(seed=74, n_rows=512)
    prefill_and_compare(case, Q, T - 512, sample_rows(B, 512, hq, 80, 75), view=view)


def test_paged_dense_baselines_against_oracle():
    g, o = configs(torch.bfloat16, 16, 2, G=8)
    B, T = 2, 4096
    case, (Kp, Vp, table) = _paged_case(g, o, B, T, 76, 16)
    q = case.queries(seed=77)
    seq = [T, 1999]
    sl = torch.tensor(seq, dtype=torch.int32, device="cuda")
    dec = lod.dense_decode(g, Kp, Vp, q.cuda(), sl, T, block_table=table).cpu().numpy()
    Q = case.queries(seed=78, n_rows=300)
    pre = lod.dense_prefill(g, Kp, Vp, Q.cuda(), T - 300, block_table=table).cpu().numpy()
    qf, Qf = q.float().numpy(), Q.float().numpy()
    st = {kv: case.stream(*kv) for kv in [(b, h) for b in range(B) for h in range(2)]}
    worst = 0.0
    for b in range(B):
        for h in (0, 7, 8, 15):
            ref, _ = orc.dense(o, *st[(b, h // 8)], qf[b, h], seq[b] - 1)
            worst = max(worst, float(np.max(np.abs(dec[b, h] - ref))))
    rows = sample_rows(B, 300, 16, 40, 79)
    ref = orc.dense_rows(o, st, Qf, T - 300, rows)
    worst = max([worst] + [float(np.max(np.abs(pre[r] - ref[r]))) for r in rows])
    assert worst <= TOL[torch.bfloat16], worst


@pytest.mark.parametrize("TP", [2, 0])
def test_paged_sparsity_ablation_against_oracle(TP):
    g, o = configs(torch.bfloat16, 16, 2, G=8, TP=TP, drop=True)
    B, T = 2, 4096
    case, view = _paged_case(g, o, B, T, 80, 16)
    orc_ = case.oracle_index([(b, h) for b in range(B) for h in range(2)])
    decode_and_compare(case, orc_, [T, 3001], case.queries(seed=81), view=view)
    Q = case.queries(seed=82, n_rows=256)
    prefill_and_compare(case, Q, T - 256, sample_rows(B, 256, 16, 60, 83), view=view)


def test_paged_int4_pages_against_oracle():
    """INT4 pages read no cache rows in the open step; the window and sinks still come
    through the block table."""
    g = lod.Config(n_q_heads=16, n_kv_heads=2, groups=8, dtype=torch.bfloat16, int4_pages=True)
    o = orc.Config(d=128, groups=8, bf16=True, int4_pages=True)
    B, T = 2, 4096
    case, view = _paged_case(g, o, B, T, 84, 16)
    orc_ = case.oracle_index([(b, h) for b in range(B) for h in range(2)])
    decode_and_compare(case, orc_, [T, 3333], case.queries(seed=85), view=view)
    Q = case.queries(seed=86, n_rows=256)
    prefill_and_compare(case, Q, T - 256, sample_rows(B, 256, 16, 60, 87), view=view)


@pytest.mark.parametrize("dtype,hq,hkv,bs", [
    (torch.bfloat16, 16, 2, 16),
    (torch.bfloat16, 64, 8, 1),
    (torch.float32, 4, 2, 32),
])
def test_paged_view_equals_strided_bit_for_bit(dtype, hq, hkv, bs):
    bf = dtype == torch.bfloat16
    g, o = configs(dtype, hq, hkv, G=8, W=512 if bf else 256, S=4 if bf else 1)
    B, T = 2, 4096
    case = Case(g, o, B, T, seed=88)
    case.build_gpu()
    Kp, Vp, table = paged_copy(case.Kd, case.Vd, bs, seed=89)
    idx = lod.LodIndex.allocate(g, B, T, device="cuda")
    lod.build_chunk(g, idx, Kp, Vp, 0, T // 256, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(idx.mem, case.index.mem)
    q = case.queries(seed=90).cuda()
    sl = torch.tensor([T, 2345], dtype=torch.int32, device="cuda")
    a = lod.attend_decode(g, case.index, case.Kd, case.Vd, q, sl, T, want_selection=True)
    b = lod.attend_decode(g, idx, Kp, Vp, q, sl, T, want_selection=True, block_table=table)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(lod.dense_decode(g, case.Kd, case.Vd, q, sl, T),
                       lod.dense_decode(g, Kp, Vp, q, sl, T, block_table=table))
    Q = case.queries(seed=91, n_rows=512).cuda()
    a = lod.attend_prefill(g, case.index, case.Kd, case.Vd, Q, T - 512, want_selection=True)
    b = lod.attend_prefill(g, idx, Kp, Vp, Q, T - 512, want_selection=True, block_table=table)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(lod.dense_prefill(g, case.Kd, case.Vd, Q, T - 512),
                       lod.dense_prefill(g, Kp, Vp, Q, T - 512, block_table=table))
