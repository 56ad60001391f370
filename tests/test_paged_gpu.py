"""Paged (block-table) KV views on the GPU: every call gives bit for bit what the same
call gives on a strided copy of the cache (the view changes addressing only), and the
strided path itself is held to the oracle by the other parity tests.

The paged cache scatters each sequence's blocks over a shared pool in a seeded random
order, as a serving engine's block allocator leaves them."""
import numpy as np
import pytest
import torch

from hierarchical_kv_approximation_amd import lod

from lodcase import Case, configs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _paged(K, V, bs, seed, spare=7):
    """[B][T][Hkv][d] -> pool [nblk][bs][Hkv][d] (blocks in random order, a few unused)
    and block_table [B][T/bs]."""
    B, T = K.shape[0], K.shape[1]
    nb = T // bs
    nblk = B * nb + spare
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(nblk)[: B * nb].astype(np.int32))
    table = perm.view(B, nb).to(K.device)
    Kp = torch.zeros(nblk, bs, *K.shape[2:], dtype=K.dtype, device=K.device)
    Vp = torch.zeros_like(Kp)
    Kp[table.view(-1).long()] = K.reshape(B * nb, bs, *K.shape[2:])
    Vp[table.view(-1).long()] = V.reshape(B * nb, bs, *V.shape[2:])
    return Kp, Vp, table.contiguous()


@pytest.mark.parametrize("dtype,hq,hkv,bs", [
    (torch.bfloat16, 16, 2, 16),
    (torch.bfloat16, 16, 2, 128),
    (torch.bfloat16, 64, 8, 1),
    (torch.float32, 4, 2, 32),
])
def test_paged_view_equals_strided(dtype, hq, hkv, bs):
    g, o = configs(dtype, hq, hkv, G=8, W=512 if dtype == torch.bfloat16 else 256,
                   S=4 if dtype == torch.bfloat16 else 1)
    B, T = 2, 4096
    case = Case(g, o, B, T, seed=71)
    case.build_gpu()
    Kp, Vp, table = _paged(case.Kd, case.Vd, bs, seed=72)

    # build: the index built through the table is byte-identical
    idx = lod.LodIndex.allocate(g, B, T, device="cuda")
    lod.build_chunk(g, idx, Kp, Vp, 0, T // 256, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(idx.mem, case.index.mem)

    # decode (LoD and dense) at ragged lengths
    q = case.queries(seed=73).cuda()
    sl = torch.tensor([T, 2345], dtype=torch.int32, device="cuda")
    a = lod.attend_decode(g, case.index, case.Kd, case.Vd, q, sl, T, want_selection=True)
    b = lod.attend_decode(g, idx, Kp, Vp, q, sl, T, want_selection=True, block_table=table)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(lod.dense_decode(g, case.Kd, case.Vd, q, sl, T),
                       lod.dense_decode(g, Kp, Vp, q, sl, T, block_table=table))

    # prefill (LoD and dense) over the last 512 rows
    Q = case.queries(seed=74, n_rows=512).cuda()
    a = lod.attend_prefill(g, case.index, case.Kd, case.Vd, Q, T - 512, want_selection=True)
    b = lod.attend_prefill(g, idx, Kp, Vp, Q, T - 512, want_selection=True, block_table=table)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(lod.dense_prefill(g, case.Kd, case.Vd, Q, T - 512),
                       lod.dense_prefill(g, Kp, Vp, Q, T - 512, block_table=table))


def test_paged_view_with_sparsity_ablation():
    g, o = configs(torch.bfloat16, 16, 2, G=8, drop=True)
    B, T = 2, 4096
    case = Case(g, o, B, T, seed=75)
    case.build_gpu()
    Kp, Vp, table = _paged(case.Kd, case.Vd, 16, seed=76)
    q = case.queries(seed=77).cuda()
    sl = torch.tensor([T, 3001], dtype=torch.int32, device="cuda")
    assert torch.equal(lod.attend_decode(g, case.index, case.Kd, case.Vd, q, sl, T),
                       lod.attend_decode(g, case.index, Kp, Vp, q, sl, T, block_table=table))


def test_paged_view_with_int4_pages():
    """INT4 pages read no cache rows in the open step; the window and sinks still come
    through the block table: paged and strided agree bit for bit."""
    g = lod.Config(n_q_heads=16, n_kv_heads=2, groups=8, dtype=torch.bfloat16, int4_pages=True)
    from oracle import oracle as orc
    o = orc.Config(d=128, groups=8, bf16=True, int4_pages=True)
    B, T = 2, 4096
    case = Case(g, o, B, T, seed=78)
    case.build_gpu()
    Kp, Vp, table = _paged(case.Kd, case.Vd, 16, seed=79)
    idx = lod.LodIndex.allocate(g, B, T, device="cuda")
    lod.build_chunk(g, idx, Kp, Vp, 0, T // 256, block_table=table)
    q = case.queries(seed=80).cuda()
    sl = torch.tensor([T, 3333], dtype=torch.int32, device="cuda")
    Q = case.queries(seed=81, n_rows=256).cuda()
    torch.cuda.synchronize()
    assert torch.equal(idx.mem, case.index.mem)
    assert torch.equal(lod.attend_decode(g, case.index, case.Kd, case.Vd, q, sl, T),
                       lod.attend_decode(g, idx, Kp, Vp, q, sl, T, block_table=table))
    assert torch.equal(lod.attend_prefill(g, case.index, case.Kd, case.Vd, Q, T - 256),
                       lod.attend_prefill(g, idx, Kp, Vp, Q, T - 256, block_table=table))
