"""GPU parity of prefill (LoD and the dense causal baseline) against the CPU oracle."""
import numpy as np
import pytest
import torch

from hierarchical_kv_approximation_amd import lod
from oracle import oracle as orc

from lodcase import TOL, Case, configs
from lodcase import prefill_and_compare as _prefill_and_compare
from lodcase import sample_rows as _sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,hq,hkv,q_start,nq", [
    (torch.bfloat16, 64, 8, 512, 700),
    (torch.bfloat16, 16, 4, 0, 333),
    (torch.bfloat16, 8, 8, 256, 129),
    (torch.float32, 4, 4, 256, 100),
])
def test_dense_prefill_parity(dtype, hq, hkv, q_start, nq):
    g, o = configs(dtype, hq, hkv, G=8)
    T = q_start + nq
    case = Case(g, o, 2, ((T + 255) // 256) * 256, seed=31)
    Q = case.queries(seed=32, n_rows=nq)
    out = lod.dense_prefill(g, case.Kd, case.Vd, Q.cuda(), q_start).cpu().numpy()
    rows = _sample_rows(2, nq, hq, 60, 33)
    st = {kv: case.stream(*kv) for kv in {(b, h // (hq // hkv)) for b, _, h in rows}}
    ref = orc.dense_rows(o, st, Q.float().numpy(), q_start, rows)
    worst = max(float(np.max(np.abs(out[b, i, h] - ref[(b, i, h)]))) for b, i, h in rows)
    assert worst <= TOL[dtype], worst


@pytest.mark.parametrize("dtype,hq,hkv,q_start,nq,G,TG,TP", [
    (torch.bfloat16, 64, 8, 2048, 2600, 8, 8, 2),   # two row batches, ragged last query chunk
    (torch.bfloat16, 16, 4, 0, 700, 8, 8, 2),       # rows with no summarised chunk
    (torch.bfloat16, 8, 8, 1024, 333, 8, 8, 2),     # one head per KV head
    (torch.bfloat16, 8, 4, 768, 300, 8, 8, 2),      # two heads per KV head
    (torch.bfloat16, 16, 2, 1536, 512, 8, 8, 0),    # two-tier: opened groups fully exact
    (torch.bfloat16, 16, 2, 1536, 512, 8, 8, 1),
    (torch.bfloat16, 16, 2, 1536, 512, 8, 8, 3),
    (torch.bfloat16, 16, 2, 1280, 400, 4, 4, 2),
    (torch.bfloat16, 16, 2, 1280, 400, 16, 16, 2),
    (torch.bfloat16, 64, 8, 2048, 2100, 16, 16, 2),  # 16 opened groups in a 2048-row batch: the
                                                     # block-at-a-time sweep with 8-entry lane
                                                     # lists, 64-column select with 16-entry networks
    (torch.float32, 4, 4, 1024, 300, 4, 8, 2),      # fp32 caches: row-by-row path
])
def test_lod_prefill_parity(dtype, hq, hkv, q_start, nq, G, TG, TP):
    g, o = configs(dtype, hq, hkv, G=G, TG=TG, TP=TP)
    T = q_start + nq
    case = Case(g, o, 2, ((T + 255) // 256) * 256, seed=41)
    case.build_gpu()
    Q = case.queries(seed=42, n_rows=nq)
    rows = _sample_rows(2, nq, hq, 120, 43)
    _prefill_and_compare(case, Q, q_start, rows)


@pytest.mark.parametrize("G,TG,TP,kind", [
    (2, 4, 2, "matched"),     # groups of about 128 keys: runs of more than 64 rows, summaries
    (2, 2, 1, "diffuse"),     # one opened page of eight: mostly summary terms
    (16, 16, 2, "diffuse"),   # small groups, many distinct ones: more than 4 runs per workgroup
])
def test_lod_prefill_group_kernel_paths(G, TG, TP, kind):
    """The opened pages' MFMA kernel on its rarer paths: groups whose members and page
    summaries need several key tiles, pairs that leave most pages of a group unopened,
    and workgroups whose pairs span many groups (meta rows loaded beyond the first
    four runs)."""
    g, o = configs(torch.bfloat16, 16, 2, G=G, TG=TG, TP=TP)
    case = Case(g, o, 1, 4096, seed=56)
    case.build_gpu()
    Q = case.queries(seed=57, n_rows=768, kind=kind)
    _prefill_and_compare(case, Q, 3328, _sample_rows(1, 768, 16, 100, 58))


def test_lod_prefill_diffuse_queries():
    g, o = configs(torch.bfloat16, 16, 2, G=8)
    case = Case(g, o, 1, 4096, seed=44)
    case.build_gpu()
    Q = case.queries(seed=45, n_rows=1024, kind="diffuse")
    _prefill_and_compare(case, Q, 3072, _sample_rows(1, 1024, 16, 100, 46))


@pytest.mark.parametrize("TG", [16, 8])
def test_lod_prefill_ties_take_the_exhaustive_path(TG):
    """Four centres shared by every chunk and zero variance: dozens of groups tie at the
    top score, more than a split's candidate list keeps, so selection falls back to
    ranking every group canonically (for both instantiations of the selection, up to 8 and
    up to 16 opened groups).  Zero variance also makes LoD equal dense attention."""
    g, o = configs(torch.bfloat16, 16, 2, G=8, TG=TG)
    case = Case(g, o, 1, 12288, seed=47, zero_variance=True, n_centres=4)
    case.build_gpu()
    Q = case.queries(seed=48, n_rows=512)
    _prefill_and_compare(case, Q, 11776, _sample_rows(1, 512, 16, 60, 49), check_dense=True)


def test_lod_prefill_32k_chunked_equals_one_shot():
    """32K-token prefill, 64/8 heads: one call over every row equals the chunked flow
    (build the chunk that leaves the window, then attend the next 256-row query chunk);
    sampled rows match the oracle.  Selections are identical; outputs agree to fp32
    rounding, since small calls split each tile's key list over several workgroups and
    so sum the softmax in a different order."""
    g, o = configs(torch.bfloat16, 64, 8, G=8)
    T = 32768
    case = Case(g, o, 1, T, seed=50)
    case.build_gpu()
    Q = case.queries(seed=51, n_rows=T)
    rows = _sample_rows(1, T, 64, 150, 52)
    _, one = _prefill_and_compare(case, Q, 0, rows)

    fresh = lod.LodIndex.allocate(g, 1, T, device="cuda")
    Qd = Q.cuda()
    out = torch.empty(1, T, 64, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(lod.prefill_ws_bytes(g, 1, 256, T), dtype=torch.uint8, device="cuda")
    nwin = g.window // 256
    for k in range(T // 256):
        if k - nwin >= 0:
            lod.build_chunk(g, fresh, case.Kd, case.Vd, k - nwin, 1)
        lod.attend_prefill(g, fresh, case.Kd, case.Vd, Qd[:, 256 * k: 256 * (k + 1)], 256 * k, ws=ws,
                           out=out[:, 256 * k: 256 * (k + 1)])
    torch.cuda.synchronize()
    assert float(np.max(np.abs(out.cpu().numpy() - one))) <= 1e-5


def test_lod_prefill_128k_chunked_sampled():
    """The full-size chunked prefill: 131072 tokens, GQA 64/8, bf16, 256-row query
    chunks, the chunk leaving the window built before each call (the benchmark's flow
    and launch configuration).  Sampled rows of three KV heads -- the first rows, rows
    just past a window boundary, rows across the sequence and the last row -- match the
    oracle: selections bit-exact (from a second pass that also returns them, whose
    outputs equal the first pass bit for bit), outputs within 2e-3."""
    g, o = configs(torch.bfloat16, 64, 8, G=8)
    T, C = 131072, 256
    case = Case(g, o, 1, T, seed=53, gen_device="cuda")
    Q = case.queries(seed=54, n_rows=T)
    nwin = g.window // C
    ws = torch.empty(lod.prefill_ws_bytes(g, 1, C, T), dtype=torch.uint8, device="cuda")
    out = torch.empty(1, T, 64, 128, dtype=torch.float32, device="cuda")
    sg = torch.empty(1, T, 64, 8, dtype=torch.int32, device="cuda")
    sp = torch.empty(1, T, 64, 8, 2, dtype=torch.int32, device="cuda")
    for k in range(T // C):
        if k - nwin >= 0:
            lod.build_chunk(g, case.index, case.Kd, case.Vd, k - nwin, 1)
        lod.attend_prefill(g, case.index, case.Kd, case.Vd, Q[:, C * k: C * (k + 1)], C * k, ws=ws,
                           out=out[:, C * k: C * (k + 1)])
    torch.cuda.synchronize()
    first = out.clone()
    for k in range(T // C):
        o2, s2, p2 = lod.attend_prefill(g, case.index, case.Kd, case.Vd, Q[:, C * k: C * (k + 1)], C * k,
                                        want_selection=True, ws=ws)
        out[:, C * k: C * (k + 1)] = o2
        sg[:, C * k: C * (k + 1)] = s2
        sp[:, C * k: C * (k + 1)] = p2
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    rng = np.random.default_rng(55)
    pos = sorted({0, 1, 511, 512, 767, 768, 1023, 65535, 65536, T - 257, T - 256, T - 1,
                  *rng.integers(0, T, 24).tolist()})
    rows = [(0, p, kvh * 8 + int(rng.integers(0, 8))) for p in pos for kvh in (0, 3, 7)]
    st, oidx = case.oracle_index([(0, 0), (0, 3), (0, 7)])
    pr = torch.tensor([p for _, p, _ in rows], device="cuda")
    hr = torch.tensor([h for _, _, h in rows], device="cuda")
    Qs = Q[0, pr, hr].float().cpu().numpy()
    got, gsg, gsp = (x[0, pr, hr].cpu().numpy() for x in (out, sg, sp))
    worst = 0.0
    for i, (_, p, h) in enumerate(rows):
        r = orc.attend(o, oidx[(0, h // 8)], *st[(0, h // 8)], Qs[i], p)
        assert np.array_equal(gsg[i], r["sel_groups"]), (p, h, gsg[i], r["sel_groups"])
        assert np.array_equal(gsp[i], r["sel_pages"]), (p, h)
        worst = max(worst, float(np.max(np.abs(got[i] - r["out"]))))
    assert worst <= TOL[torch.bfloat16], worst
