"""Three-tier INT4 on the GPU against the CPU oracle: the build's 4-bit codes and scales
bit for bit, decode and prefill selections bit for bit and outputs within 2e-3, and the
compressed storage is self-sufficient: once a chunk is built, its clustered rows are
never read from the cache again (they can be overwritten without changing any output).

Bar: codes, scales and selections bit-exact; outputs within 2e-3 max-abs (bf16 KV)."""
import numpy as np
import pytest
import torch

from hierarchical_kv_approximation_amd import lod
from oracle import oracle as orc

from lodcase import TOL, Case
from lodcase import decode_and_compare as _decode_and_compare
from lodcase import prefill_and_compare as _prefill_and_compare
from lodcase import sample_rows as _sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cfgs(Hq, Hkv, G=8, TG=8, TP=2, drop=False):
    g = lod.Config(n_q_heads=Hq, n_kv_heads=Hkv, groups=G, top_groups=TG, top_pages=TP, window=512,
                   n_sink=4, dtype=torch.bfloat16, drop_remainder=drop, int4_pages=True)
    o = orc.Config(d=128, groups=G, top_groups=TG, top_pages=TP, window=512, n_sink=4, bf16=True,
                   drop_remainder=drop, int4_pages=True)
    return g, o


def _unpack(codes):
    """[..., 64] uint8 -> [..., 128] int8 (element 2j in the low nibble of byte j)."""
    c = codes.astype(np.int16)
    lo, hi = c & 0xF, c >> 4
    out = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], 2 * codes.shape[-1])
    return ((out ^ 8) - 8).astype(np.int8)


def test_int4_build_codes_bit_exact():
    g, o = _cfgs(8, 2)
    case = Case(g, o, 2, 4096, seed=91, sigma=0.6)
    case.build_gpu()
    arr = case.index.arrays()
    st, oidx = case.oracle_index([(b, h) for b in range(2) for h in range(2)])
    n = case.nchunks
    for (b, h), idx in oidx.items():
        assert np.array_equal(_unpack(arr["q4k"][b, h, :n].cpu().numpy()), idx["qk"])
        assert np.array_equal(_unpack(arr["q4v"][b, h, :n].cpu().numpy()), idx["qv"])
        assert np.array_equal(arr["q4ks"][b, h, :n].cpu().numpy(), idx["qks"])
        assert np.array_equal(arr["q4vs"][b, h, :n].cpu().numpy(), idx["qvs"])


@pytest.mark.parametrize("hq,hkv,G,TG,TP,drop", [
    (16, 2, 8, 8, 2, False),
    (16, 2, 8, 8, 0, False),    # two-tier selection, every page of an opened group decoded
    (64, 8, 4, 16, 2, False),
    (16, 2, 8, 8, 2, True),     # with the sparsity ablation
])
def test_int4_decode_parity(hq, hkv, G, TG, TP, drop):
    g, o = _cfgs(hq, hkv, G, TG, TP, drop)
    case = Case(g, o, 2, 8192, seed=92)
    case.build_gpu()
    orc_ = case.oracle_index([(b, h) for b in range(2) for h in range(hkv)])
    _decode_and_compare(case, orc_, [8192, 4567], case.queries(seed=93))


@pytest.mark.parametrize("hq,hkv,q_start,nq,TP", [
    (64, 8, 2048, 600, 2),
    (16, 2, 1536, 512, 0),
])
def test_int4_prefill_parity(hq, hkv, q_start, nq, TP):
    g, o = _cfgs(hq, hkv, TP=TP)
    T = q_start + nq
    case = Case(g, o, 2, ((T + 255) // 256) * 256, seed=94)
    case.build_gpu()
    Q = case.queries(seed=95, n_rows=nq)
    _prefill_and_compare(case, Q, q_start, _sample_rows(2, nq, hq, 100, 96))


def test_int4_built_rows_are_never_read_from_the_cache():
    """Overwrite every clustered row of the built chunks with NaN: decode and prefill
    outputs do not change (sinks and the window are still read from the cache)."""
    g, o = _cfgs(16, 2)
    T = 8192
    case = Case(g, o, 2, T, seed=97)
    case.build_gpu()
    q = case.queries(seed=98).cuda()
    Q = case.queries(seed=99, n_rows=512).cuda()
    sl = torch.tensor([T, T - 700], dtype=torch.int32, device="cuda")
    dec = lod.attend_decode(g, case.index, case.Kd, case.Vd, q, sl, T)
    pre = lod.attend_prefill(g, case.index, case.Kd, case.Vd, Q, T - 512)
    # rows of the chunks that every query above sees summarised: those before the block
    # window of the earliest query (position T - 701)
    p_min = min(T - 701, T - 512)
    nb = p_min // 256 - g.window // 256 + 1
    Kn, Vn = case.Kd.clone(), case.Vd.clone()
    Kn[:, g.n_sink: nb * 256] = float("nan")
    Vn[:, g.n_sink: nb * 256] = float("nan")
    dec2 = lod.attend_decode(g, case.index, Kn, Vn, q, sl, T)
    pre2 = lod.attend_prefill(g, case.index, Kn, Vn, Q, T - 512)
    torch.cuda.synchronize()
    assert torch.equal(dec, dec2)
    assert torch.equal(pre, pre2)
