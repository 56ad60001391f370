"""Pins of the video LoD oracle to facts fixed by the method and by mathematics.

The method: "Level of Detail Attention" (featherless.ai blog), section "Video LoD"
(4x4x4 blocks of queries and keys/values, c = 16), with the tiers of "How It Works".
No test re-types the oracle's formulas: they use index arithmetic written another way,
numpy fp64 means and dots, a textbook dense softmax, an explicit expansion of the
coarse terms into repeated keys, Jensen's inequality and brute-force sorting.
"""
import math

import numpy as np
import pytest
import torch

from hierarchical_kv_approximation_amd import synth
from oracle import video as vo

GRIDS = [(8, 8, 8), (5, 6, 7), (4, 4, 12), (1, 3, 2)]


def _qkv(F, H, W, d, seed, Hq=1, Hkv=1, kind="matched", round_bf16=True, **kw):
    Q, K, V = synth.video_qkv(1, F, H, W, Hq, Hkv, d, seed=seed, kind=kind, region=(4, 4, 4),
                              dtype=torch.bfloat16 if round_bf16 else torch.float32, **kw)
    return Q.float().numpy(), K.float().numpy(), V.float().numpy()


def _softmax(lam, val):
    lam = np.asarray(lam, np.float64)
    w = np.exp(lam - lam.max())
    return (w[:, None] * np.asarray(val, np.float64)).sum(0) / w.sum()


# --------------------------------------------------------------------------- geometry

@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("block", [(4, 4, 4), (2, 4, 8), (1, 1, 1)])
def test_blocks_partition_the_grid(grid, block):
    """Every token lies in exactly one block: the one its coordinates divided by the
    block extents name, block ids in raster order of block coordinates."""
    F, H, W = grid
    cfg = vo.VideoConfig(d=4, frames=F, height=H, width=W, block=block)
    nby, nbx = -(-H // block[1]), -(-W // block[2])
    assert cfg.n_blocks == -(-F // block[0]) * nby * nbx
    t = np.arange(F * H * W)
    f, y, x = t // (H * W), (t // W) % H, t % W
    expect = ((f // block[0]) * nby + y // block[1]) * nbx + x // block[2]
    seen = np.full(F * H * W, -1)
    for b in range(cfg.n_blocks):
        m = vo.members(cfg, b)
        assert np.all(np.diff(m) > 0), "members ascend"
        assert np.all(seen[m] == -1), "no token in two blocks"
        seen[m] = b
    assert np.array_equal(seen, expect)


# --------------------------------------------------------------------------- summaries

@pytest.mark.parametrize("grid", GRIDS[:3])
def test_block_means_are_the_members_means(grid):
    """kbar, vbar are the members' means (fp64 numpy) rounded once to bf16; the mean
    query stays fp32; counts are the clipped block volumes."""
    F, H, W = grid
    cfg = vo.VideoConfig(d=32, frames=F, height=H, width=W, bf16=True)
    Q, K, V = _qkv(F, H, W, 32, seed=3)
    for X, rnd in ((K[0, :, 0], True), (V[0, :, 0], True), (Q[0, :, 0], False)):
        mean, cnt = vo.summaries(cfg, X, rnd)
        for b in range(cfg.n_blocks):
            m = vo.members(cfg, b)
            assert cnt[b] == len(m)
            ref = X[m].astype(np.float64).mean(0)
            # fp32 summation of <= 64 terms, then (for bf16) one rounding: half a bf16 ulp
            tol = (np.abs(ref) * (2.0 ** -8 if rnd else 0.0) + 64 * 2.0 ** -24 * np.abs(X[m]).max(0)
                   + 1e-30)
            assert np.all(np.abs(mean[b] - ref) <= tol)
            if rnd:
                assert np.array_equal(mean[b], torch.from_numpy(mean[b]).to(torch.bfloat16).float().numpy())


def test_means_of_identical_bf16_rows_are_exact():
    """A block whose keys are all one bf16 vector has that vector as its mean."""
    cfg = vo.VideoConfig(d=16, frames=4, height=8, width=8, bf16=True)
    Q, K, V = _qkv(4, 8, 8, 16, seed=5, zero_variance_block=(4, 4, 4))
    mean, _ = vo.summaries(cfg, K[0, :, 0], True)
    for b in range(cfg.n_blocks):
        m = vo.members(cfg, b)
        assert np.all(K[0, m, 0] == K[0, m[0], 0])
        assert np.array_equal(mean[b], K[0, m[0], 0])


# --------------------------------------------------------------------------- selection

@pytest.mark.parametrize("c", [1, 3, 5, 40])
def test_selection_is_the_top_c_of_a_full_sort(c):
    """The opened blocks are the first c of a full sort by (score desc, id asc); with
    fewer blocks than c every block opens and the rest is -1.  Scores agree with fp64
    dots within the fp32 chain's error bound."""
    cfg = vo.VideoConfig(d=64, frames=8, height=8, width=12, top_blocks=c, bf16=True)
    Q, K, V = _qkv(8, 8, 12, 64, seed=7)
    kbar, _ = vo.summaries(cfg, K[0, :, 0], True)
    qbar, _ = vo.summaries(cfg, Q[0, :, 0], False)
    nb = cfg.n_blocks
    for j in range(nb):
        sel, sc = vo.select(cfg, qbar[j], kbar)
        exact = kbar.astype(np.float64) @ qbar[j].astype(np.float64)
        bound = 64 * 2.0 ** -24 * (np.abs(kbar).astype(np.float64) @ np.abs(qbar[j]).astype(np.float64))
        assert np.all(np.abs(sc - exact) <= bound + 1e-30)
        order = np.lexsort((np.arange(nb), -sc.astype(np.float64)))
        k = min(c, nb)
        assert np.array_equal(sel[:k], np.sort(order[:k]))
        assert np.all(sel[k:] == -1)


def test_equal_scores_open_the_lower_block_id():
    """Ties between scores go to the lower block id."""
    cfg = vo.VideoConfig(d=8, frames=4, height=4, width=16, top_blocks=2)
    kbar = np.zeros((cfg.n_blocks, 8), np.float32)
    kbar[:, 0] = 1.0  # every block scores the same
    kbar[3, 0] = 2.0  # except block 3
    sel, _ = vo.select(cfg, np.ones(8, np.float32), kbar)
    assert list(sel) == [0, 3]


# --------------------------------------------------------------------------- attention

@pytest.mark.parametrize("grid", GRIDS[:3])
def test_opening_every_block_is_dense_attention(grid):
    """With c at least the number of blocks nothing stays coarse: the output is the
    textbook bidirectional softmax over all keys."""
    F, H, W = grid
    cfg = vo.VideoConfig(d=16, frames=F, height=H, width=W, top_blocks=1000)
    Q, K, V = _qkv(F, H, W, 16, seed=11, round_bf16=False)
    r = vo.forward(cfg, Q, K, V)
    sc = 1.0 / math.sqrt(16)
    for t in range(0, F * H * W, 7):
        ref = _softmax(sc * (K[0, :, 0].astype(np.float64) @ Q[0, t, 0].astype(np.float64)), V[0, :, 0])
        assert np.max(np.abs(r["out"][0, t, 0] - ref)) < 1e-12


def test_lod_equals_dense_over_exact_keys_plus_repeated_means():
    """The expanded-dense identity: LoD output equals a plain softmax over the exact keys
    of the opened blocks plus n copies of every unopened block's (mean key, mean value)."""
    F, H, W, d = 5, 6, 7, 16
    cfg = vo.VideoConfig(d=d, frames=F, height=H, width=W, top_blocks=3, bf16=True)
    Q, K, V = _qkv(F, H, W, d, seed=13)
    r = vo.forward(cfg, Q, K, V)
    sc = 1.0 / math.sqrt(d)
    for j in range(cfg.n_blocks):
        sel = [b for b in r["sel"][0, 0, j] if b >= 0]
        keys, vals = [], []
        for b in range(cfg.n_blocks):
            m = vo.members(cfg, b)
            if b in sel:
                keys += list(K[0, m, 0]); vals += list(V[0, m, 0])
            else:
                keys += [r["kbar"][0, 0, b]] * len(m); vals += [r["vbar"][0, 0, b]] * len(m)
        keys = np.array(keys, np.float64)
        for t in vo.members(cfg, j):
            ref = _softmax(sc * (keys @ Q[0, t, 0].astype(np.float64)), vals)
            assert np.max(np.abs(r["out"][0, t, 0] - ref)) < 1e-12


def test_zero_variance_blocks_give_dense_attention():
    """Blocks whose keys are identical lose nothing by being summarised: the output
    equals dense attention (up to the fp32 rounding of the mean values)."""
    F, H, W, d = 8, 8, 8, 32
    cfg = vo.VideoConfig(d=d, frames=F, height=H, width=W, top_blocks=2, bf16=False)
    Q, K, V = _qkv(F, H, W, d, seed=17, round_bf16=False, kind="diffuse", zero_variance_block=(4, 4, 4))
    r = vo.forward(cfg, Q, K, V, dense=True)
    assert np.max(np.abs(r["out"] - r["dense"])) < 1e-6
    # and it is not the trivial case: most of the mass is coarse
    assert np.mean([np.mean(r["coarse_mass"][k] / (r["coarse_mass"][k] + r["exact_mass"][k]))
                    for k in r["coarse_mass"]]) > 0.3


def test_coarse_mass_never_exceeds_the_exact_mass_it_replaces():
    """Jensen: for every block, n exp(q.kbar) <= sum over members of exp(q.k_i) when kbar
    is the exact mean (fp32 storage), so the coarse remainder is conservative."""
    F, H, W, d = 8, 8, 8, 32
    cfg = vo.VideoConfig(d=d, frames=F, height=H, width=W, bf16=False)
    Q, K, V = _qkv(F, H, W, d, seed=19, round_bf16=False)
    kbar, cnt = vo.summaries(cfg, K[0, :, 0], False)
    sc = 1.0 / math.sqrt(d)
    q = Q[0, ::37, 0].astype(np.float64)
    for b in range(cfg.n_blocks):
        m = vo.members(cfg, b)
        coarse = cnt[b] * np.exp(sc * (q @ kbar[b].astype(np.float64)))
        exact = np.exp(sc * (q @ K[0, m, 0].astype(np.float64).T)).sum(1)
        assert np.all(coarse <= exact * (1 + 1e-6))


def test_dropping_the_remainder_is_softmax_over_the_opened_blocks():
    """The sparsity ablation keeps the same choice and only the opened blocks' keys."""
    F, H, W, d = 5, 6, 7, 16
    base = vo.VideoConfig(d=d, frames=F, height=H, width=W, top_blocks=2, bf16=True)
    drop = vo.VideoConfig(d=d, frames=F, height=H, width=W, top_blocks=2, bf16=True, drop_remainder=True)
    Q, K, V = _qkv(F, H, W, d, seed=23)
    r0, r1 = vo.forward(base, Q, K, V), vo.forward(drop, Q, K, V)
    assert np.array_equal(r0["sel"], r1["sel"])
    sc = 1.0 / math.sqrt(d)
    for j in range(base.n_blocks):
        m = np.concatenate([vo.members(base, b) for b in r1["sel"][0, 0, j] if b >= 0])
        for t in vo.members(base, j):
            ref = _softmax(sc * (K[0, m, 0].astype(np.float64) @ Q[0, t, 0].astype(np.float64)), V[0, m, 0])
            assert np.max(np.abs(r1["out"][0, t, 0] - ref)) < 1e-12


def test_query_heads_use_their_kv_head_and_choose_independently():
    """With GQA, query head h reads KV head h // g; each head makes its own choice."""
    F, H, W, d = 4, 8, 8, 16
    cfg = vo.VideoConfig(d=d, frames=F, height=H, width=W, top_blocks=1, bf16=True)
    Q, K, V = _qkv(F, H, W, d, seed=29, Hq=4, Hkv=2, kind="diffuse")
    r = vo.forward(cfg, Q, K, V)
    for h in range(4):
        one = vo.forward(cfg, Q[:, :, h:h + 1], K[:, :, h // 2:h // 2 + 1], V[:, :, h // 2:h // 2 + 1])
        assert np.array_equal(one["sel"][0, 0], r["sel"][0, h])
        assert np.array_equal(one["out"][0, :, 0], r["out"][0, :, h])
    assert not np.array_equal(r["sel"][0, 0], r["sel"][0, 1])


def test_hand_worked_example():
    """tests/golden/video_worked_example.json: a 1x2x4 grid with 1x2x2 blocks, d = 2, c = 1,
    worked by hand from the definitions (block means, a tied score going to the lower
    block id, LoD and dense outputs in closed form)."""
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "video_worked_example.json")))
    gr = fx["grid"]
    cfg = vo.VideoConfig(d=gr["d"], frames=gr["frames"], height=gr["height"], width=gr["width"],
                         block=tuple(gr["block"]), top_blocks=gr["top_blocks"], scale=gr["scale"], bf16=False)
    K = np.array(fx["K"], np.float32)[None, :, None, :]
    V = np.array(fx["V"], np.float32)[None, :, None, :]
    Q = np.array(fx["Q"], np.float32)[None, :, None, :]
    r = vo.forward(cfg, Q, K, V, dense=True)
    ex = fx["expected"]
    assert np.array_equal(r["kbar"][0, 0], np.array(ex["kbar"], np.float32))
    assert np.array_equal(r["vbar"][0, 0], np.array(ex["vbar"], np.float32))
    assert np.array_equal(r["qbar"][0, 0], np.array(ex["qbar"], np.float32))
    assert list(r["count"]) == ex["count"]
    assert r["sel"][0, 0].tolist() == ex["sel"]
    for t in (0, 1, 4, 5):
        assert np.allclose(r["out"][0, t, 0], ex["lod_block0_query"]["value"], rtol=0, atol=1e-12)
        assert np.allclose(r["dense"][0, t, 0], ex["dense_block0_query"]["value"], rtol=0, atol=1e-12)
    for t in (2, 3, 6, 7):
        assert np.allclose(r["out"][0, t, 0], ex["lod_block1_query"]["value"], rtol=0, atol=1e-12)
        assert np.allclose(r["dense"][0, t, 0], ex["dense_block1_query"]["value"], rtol=0, atol=1e-12)
