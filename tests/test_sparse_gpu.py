"""GPU parity of the sparsity ablation (coarse remainder dropped, selection unchanged)
against the CPU oracle, for decode and prefill, bf16 and fp32 caches.

Bar: group and page selections bit-exact; outputs within 1e-5 (fp32 KV) / 2e-3 (bf16)."""
import numpy as np
import pytest
import torch

from hierarchical_kv_approximation_amd import lod
from oracle import oracle as orc

from lodcase import TOL, Case, configs
from lodcase import decode_and_compare as _decode_and_compare
from lodcase import prefill_and_compare as _prefill_and_compare
from lodcase import sample_rows as _sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,hq,hkv,G,TG,TP,seq", [
    (torch.bfloat16, 16, 2, 8, 8, 2, [8192, 5000]),    # three-tier selection, exact keys only
    (torch.bfloat16, 16, 2, 8, 8, 0, [8192, 777]),     # opened groups fully exact
    (torch.bfloat16, 16, 2, 4, 16, 0, [8192, 6000]),   # larger groups, larger token budget
    (torch.float32, 1, 1, 4, 8, 2, [4096, 3000]),      # fp32: slices with add-back path
    (torch.float32, 4, 2, 8, 8, 0, [4096, 2049]),
])
def test_sparse_decode_parity(dtype, hq, hkv, G, TG, TP, seq):
    g, o = configs(dtype, hq, hkv, G=G, TG=TG, TP=TP, W=512 if dtype == torch.bfloat16 else 256,
                   S=4 if dtype == torch.bfloat16 else 1, drop=True)
    case = Case(g, o, 2, max(seq), seed=61)
    case.build_gpu()
    orc_ = case.oracle_index([(b, h) for b in range(2) for h in range(hkv)])
    _decode_and_compare(case, orc_, seq, case.queries(seed=62))


def test_sparse_decode_differs_from_lod_only_by_the_remainder():
    """Same index, same queries: LoD and the ablation open the same groups and pages."""
    g, o = configs(torch.bfloat16, 16, 2, G=8)
    gs, _ = configs(torch.bfloat16, 16, 2, G=8, drop=True)
    case = Case(g, o, 2, 8192, seed=63)
    case.build_gpu()
    q = case.queries(seed=64).cuda()
    sl = torch.tensor([8192, 4321], dtype=torch.int32, device="cuda")
    out_l, sg_l, sp_l = lod.attend_decode(g, case.index, case.Kd, case.Vd, q, sl, 8192, want_selection=True)
    out_s, sg_s, sp_s = lod.attend_decode(gs, case.index, case.Kd, case.Vd, q, sl, 8192, want_selection=True)
    torch.cuda.synchronize()
    assert torch.equal(sg_l, sg_s) and torch.equal(sp_l, sp_s)
    assert float((out_l - out_s).abs().max()) > 1e-3


@pytest.mark.parametrize("dtype,hq,hkv,q_start,nq,G,TG,TP", [
    (torch.bfloat16, 64, 8, 2048, 600, 8, 8, 2),
    (torch.bfloat16, 16, 2, 1536, 512, 8, 8, 0),
    (torch.bfloat16, 16, 2, 1280, 400, 4, 16, 0),
    (torch.float32, 4, 4, 1024, 300, 4, 8, 2),
])
def test_sparse_prefill_parity(dtype, hq, hkv, q_start, nq, G, TG, TP):
    g, o = configs(dtype, hq, hkv, G=G, TG=TG, TP=TP, drop=True)
    T = q_start + nq
    case = Case(g, o, 2, ((T + 255) // 256) * 256, seed=65)
    case.build_gpu()
    Q = case.queries(seed=66, n_rows=nq)
    _prefill_and_compare(case, Q, q_start, _sample_rows(2, nq, hq, 100, 67))
