"""lod_attend_decode_noalloc: lod_attend_decode with the library's fixed device workspace,
for callers that cannot allocate.  Called through the C ABI twice in a row -- the second
call smaller, so it runs over the first call's leftovers -- and each time equal bit for
bit to lod_attend_decode with a caller workspace (the same kernels); requests above the
fixed size are refused before anything is enqueued."""
import pytest
import torch

from hierarchical_kv_approximation_amd import lod

from lodcase import Case, configs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(case, seq, qseed):
    g = case.gcfg
    q = case.queries(seed=qseed).cuda()
    sl = torch.tensor(seq, dtype=torch.int32, device="cuda")
    T = max(seq)
    assert lod.decode_ws_bytes(g, case.B, T) <= lod.NOALLOC_WS_BYTES
    ref = lod.attend_decode(g, case.index, case.Kd, case.Vd, q, sl, T, want_selection=True)
    got = lod.attend_decode_noalloc(g, case.index, case.Kd, case.Vd, q, sl, T, want_selection=True)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_noalloc_decode_equals_workspace_decode_twice_second_smaller():
    g, o = configs(torch.bfloat16, 64, 8, G=8)
    big = Case(g, o, 4, 32768, seed=111, gen_device="cuda")
    big.build_gpu()
    _both(big, [32768, 30001, 9000, 513], 112)
    g2, o2 = configs(torch.bfloat16, 16, 2, G=8, TP=0)
    small = Case(g2, o2, 2, 4096, seed=113, gen_device="cuda")
    small.build_gpu()
    _both(small, [4096, 1234], 114)
    g3, o3 = configs(torch.float32, 1, 1, G=4, W=256, S=1)
    f32 = Case(g3, o3, 1, 2048, seed=115, gen_device="cuda")
    f32.build_gpu()
    _both(f32, [2048], 116)


def test_noalloc_decode_refuses_requests_above_the_fixed_size():
    """Batch 64 at 128K needs more than the fixed workspace: refused with
    LOD_ERR_WORKSPACE before anything is enqueued (the index descriptor claims the
    size such a call needs; the refusal comes before any of it is read)."""
    g, o = configs(torch.bfloat16, 64, 8, G=8)
    case = Case(g, o, 1, 1024, seed=117, gen_device="cuda")
    B, T = 64, 131072  # lod_decode_ws_bytes > LOD_NOALLOC_WS_BYTES
    assert lod.decode_ws_bytes(g, B, T) > lod.NOALLOC_WS_BYTES
    q = torch.zeros(B, 64, 128, dtype=torch.bfloat16, device="cuda")
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.full((B, 64, 128), 7.0, device="cuda")
    idx = lod.Index(case.index.mem.data_ptr(), 1 << 40, B, T // 256)
    kv = lod.kv_view(case.Kd, case.Vd)
    rc = lod.lib().lod_attend_decode_noalloc(g.params(), idx, kv, lod._ptr(q), lod._ptr(sl), B, T, lod._ptr(out),
                                             None, None, lod._stream())
    assert rc == lod.LOD_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
