"""GPU parity of video LoD ("Level of Detail Attention", section "Video LoD") against
the CPU oracle, through the C ABI.

Bar: block summaries bit-exact (bf16 mean keys and values, fp32 mean queries), the
opened blocks of every query block bit-exact, outputs within 2e-3 (bf16 inputs).
Sizes span several key tiles of 64 blocks with a ragged tail, ragged grids whose far
blocks are clipped, GQA, batches, the ablation, c above the block count, and the
full-size workload on sampled (head, query block) pairs."""
import numpy as np
import pytest
import torch

from hierarchical_kv_approximation_amd import lod, synth
from oracle import video as vo

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cfgs(F, H, W, Hq, Hkv, c, block=(4, 4, 4), drop=False):
    g = lod.VideoConfig(frames=F, height=H, width=W, n_q_heads=Hq, n_kv_heads=Hkv, block=block, top_blocks=c,
                        drop_remainder=drop)
    o = vo.VideoConfig(d=128, frames=F, height=H, width=W, block=block, top_blocks=c, bf16=True,
                       drop_remainder=drop)
    return g, o


def _run(g, Q, K, V):
    Qd, Kd, Vd = Q.cuda(), K.cuda(), V.cuda()
    ws = torch.empty(lod.video_ws_bytes(g, Q.shape[0]), dtype=torch.uint8, device="cuda")
    out, sel = lod.attend_video(g, Kd, Vd, Qd, want_selection=True, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy(), {k: v.cpu() for k, v in lod.video_arrays(g, ws, Q.shape[0]).items()}


def _np(*ts):
    return [t.float().numpy() for t in ts]


@pytest.mark.parametrize("F,H,W,Hq,Hkv,B,block", [
    (8, 8, 12, 4, 2, 2, (4, 4, 4)),
    (5, 6, 7, 2, 1, 1, (4, 4, 4)),      # clipped blocks on every far face
    (3, 9, 10, 2, 2, 1, (2, 4, 8)),
])
def test_video_summaries_are_bit_exact(F, H, W, Hq, Hkv, B, block):
    g, o = _cfgs(F, H, W, Hq, Hkv, 4, block)
    print(f"video summaries grid={F}x{H}x{W} heads={Hq}/{Hkv} B={B} block={block}", flush=True)
    Q, K, V = synth.video_qkv(B, F, H, W, Hq, Hkv, seed=101)
    _, _, arr = _run(g, Q, K, V)
    r = vo.forward(o, *_np(Q, K, V), pairs=[])
    assert np.array_equal(arr["kbar"].float().numpy(), r["kbar"])
    assert np.array_equal(arr["vbar"].float().numpy(), r["vbar"])
    assert np.array_equal(arr["qbar"].numpy().view(np.uint32), r["qbar"].view(np.uint32))
    assert np.allclose(arr["lnn"].numpy(), np.log(r["count"]), rtol=2e-7, atol=0)


@pytest.mark.parametrize("F,H,W,Hq,Hkv,B,c,block,kind", [
    (8, 32, 36, 2, 1, 1, 16, (4, 4, 4), "matched"),   # 144 blocks: 3 coarse tiles, ragged tail
    (8, 32, 36, 4, 2, 2, 5, (4, 4, 4), "diffuse"),
    (5, 6, 7, 2, 2, 1, 3, (4, 4, 4), "matched"),      # clipped blocks, c above half the blocks
    (4, 16, 16, 2, 1, 1, 64, (4, 4, 4), "matched"),   # c above the block count: all open
    (3, 9, 10, 2, 1, 1, 7, (2, 4, 8), "diffuse"),
    (6, 12, 12, 2, 1, 1, 16, (1, 4, 4), "matched"),   # 16-token blocks
])
def test_video_lod_parity(F, H, W, Hq, Hkv, B, c, block, kind):
    g, o = _cfgs(F, H, W, Hq, Hkv, c, block)
    print(f"video parity grid={F}x{H}x{W} heads={Hq}/{Hkv} B={B} c={c} block={block} {kind}", flush=True)
    Q, K, V = synth.video_qkv(B, F, H, W, Hq, Hkv, seed=103, kind=kind)
    out, sel, _ = _run(g, Q, K, V)
    r = vo.forward(o, *_np(Q, K, V))
    assert np.array_equal(sel, r["sel"])
    err = np.abs(out - r["out"]).max()
    assert err <= TOL, err


def test_video_ablation_parity_and_same_choice():
    F, H, W = 8, 32, 36
    g, o = _cfgs(F, H, W, 2, 1, 16, drop=True)
    gl, _ = _cfgs(F, H, W, 2, 1, 16)
    Q, K, V = synth.video_qkv(1, F, H, W, 2, 1, seed=107, kind="diffuse")  # coarse mass matters
    out, sel, _ = _run(g, Q, K, V)
    out_l, sel_l, _ = _run(gl, Q, K, V)
    r = vo.forward(o, *_np(Q, K, V))
    assert np.array_equal(sel, r["sel"]) and np.array_equal(sel, sel_l)
    assert np.abs(out - r["out"]).max() <= TOL
    assert np.abs(out - out_l).max() > 1e-3


def test_video_open_everything_equals_dense():
    """With c at least the block count, LoD is the dense bidirectional softmax."""
    F, H, W = 4, 16, 16  # 16 blocks
    g, o = _cfgs(F, H, W, 2, 1, 16)
    Q, K, V = synth.video_qkv(1, F, H, W, 2, 1, seed=109, kind="diffuse")
    out, _, _ = _run(g, Q, K, V)
    dense = lod.dense_video(g, K.cuda(), V.cuda(), Q.cuda())
    torch.cuda.synchronize()
    assert np.abs(out - dense.cpu().numpy()).max() <= TOL


@pytest.mark.parametrize("F,H,W,Hq,Hkv", [(5, 6, 7, 2, 1), (8, 16, 20, 4, 2)])
def test_video_dense_parity(F, H, W, Hq, Hkv):
    g, o = _cfgs(F, H, W, Hq, Hkv, 16)
    Q, K, V = synth.video_qkv(1, F, H, W, Hq, Hkv, seed=113)
    dense = lod.dense_video(g, K.cuda(), V.cuda(), Q.cuda())
    torch.cuda.synchronize()
    nb = o.n_blocks
    pairs = [(0, h, j) for h in range(Hq) for j in sorted({0, nb // 3, nb - 1})]
    r = vo.forward(o, *_np(Q, K, V), pairs=pairs, dense=True)
    ok = ~np.isnan(r["dense"])
    assert np.abs(dense.cpu().numpy()[ok] - r["dense"][ok]).max() <= TOL


def test_video_zero_variance_blocks_match_dense():
    """Keys identical inside every block: the coarse terms lose nothing."""
    F, H, W = 8, 16, 16
    g, _ = _cfgs(F, H, W, 2, 1, 2)
    Q, K, V = synth.video_qkv(1, F, H, W, 2, 1, seed=127, kind="diffuse", zero_variance_block=(4, 4, 4))
    out, _, _ = _run(g, Q, K, V)
    dense = lod.dense_video(g, K.cuda(), V.cuda(), Q.cuda())
    torch.cuda.synchronize()
    assert np.abs(out - dense.cpu().numpy()).max() <= TOL


def test_video_full_size_sampled():
    """The benchmark workload (20 x 48 x 80 grid, 40 query and KV heads, c = 16) on
    sampled (head, query block) pairs, in the launch configuration the benchmark times."""
    F, H, W, Hh = 20, 48, 80, 40
    g, o = _cfgs(F, H, W, Hh, Hh, 16)
    print(f"video full size grid={F}x{H}x{W} heads={Hh}", flush=True)
    Q, K, V = synth.video_qkv(1, F, H, W, Hh, Hh, seed=131, device="cuda")
    out, sel, _ = _run(g, Q, K, V)
    nb = o.n_blocks
    for h in (0, 17, 39):
        Qh, Kh, Vh = _np(Q[:, :, h:h + 1].cpu(), K[:, :, h:h + 1].cpu(), V[:, :, h:h + 1].cpu())
        blocks = [0, 311, 777, nb - 1]
        r = vo.forward(o, Qh, Kh, Vh, pairs=[(0, 0, j) for j in blocks])
        for j in blocks:
            assert np.array_equal(sel[0, h, j], r["sel"][0, 0, j]), (h, j)
            tok = vo.members(o, j)
            assert np.abs(out[0, tok, h] - r["out"][0, tok, 0]).max() <= TOL, (h, j)


@pytest.mark.parametrize("nby,nbx", [(40, 50), (50, 80), (80, 100)])
def test_video_large_grids_sampled(nby, nbx):
    """2000, 4000 and 8000 blocks: the choice is made with 4, 2 and 1 query blocks per
    select workgroup (the score buffer bounds it); sampled pairs against the oracle."""
    F, H, W = 4, 4 * nby, 4 * nbx
    g, o = _cfgs(F, H, W, 1, 1, 16)
    print(f"video large grid={F}x{H}x{W}", flush=True)
    Q, K, V = synth.video_qkv(1, F, H, W, 1, 1, seed=137, device="cuda")
    out, sel, _ = _run(g, Q, K, V)
    nb = o.n_blocks
    blocks = [0, nb // 2 + 1, nb - 1]
    r = vo.forward(o, *_np(Q.cpu(), K.cpu(), V.cpu()), pairs=[(0, 0, j) for j in blocks])
    for j in blocks:
        assert np.array_equal(sel[0, 0, j], r["sel"][0, 0, j]), j
        tok = vo.members(o, j)
        assert np.abs(out[0, tok, 0] - r["out"][0, tok, 0]).max() <= TOL, j


def test_video_select_fallback_when_winners_crowd_one_lane():
    """8192 blocks: every block whose id is a multiple of 64 (one lane's entries in the
    select wave) has identical keys along the queries' direction, so more than 128 keys
    tie at the top and the selection takes its fallback path; ties go to the lower ids."""
    F, H, W = 4, 256, 512
    g, o = _cfgs(F, H, W, 1, 1, 16)
    T = F * H * W
    gen = torch.Generator().manual_seed(139)
    u = torch.randn(128, generator=gen)
    t = torch.arange(T)
    f, y, x = t // (H * W), (t // W) % H, t % W
    blk = ((f // 4) * (H // 4) + y // 4) * (W // 4) + x // 4
    K = 0.1 * torch.randn(1, T, 1, 128, generator=gen)
    K[0, blk % 64 == 0, 0] = u
    Q = (u + 0.05 * torch.randn(1, T, 1, 128, generator=gen)).to(torch.bfloat16)
    K = K.to(torch.bfloat16)
    V = torch.randn(1, T, 1, 128, generator=gen).to(torch.bfloat16)
    out, sel, _ = _run(g, Q, K, V)
    nb = o.n_blocks
    blocks = [0, 4097, nb - 1]
    r = vo.forward(o, *_np(Q, K, V), pairs=[(0, 0, j) for j in blocks])
    for j in blocks:
        assert list(sel[0, 0, j]) == list(range(0, 1024, 64)), j
        assert np.array_equal(sel[0, 0, j], r["sel"][0, 0, j]), j
        tok = vo.members(o, j)
        assert np.abs(out[0, tok, 0] - r["out"][0, tok, 0]).max() <= TOL, j
