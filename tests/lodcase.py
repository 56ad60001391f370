"""Shared helpers of the GPU parity tests: build one case on both sides and compare.

Inputs come from the seeded generator only; the oracle sees the very same arrays as
the GPU (bf16 values converted exactly to fp32).  Every GPU call can go through a
strided view of the cache or through a paged (block-table) copy of it; either way the
result is held to the oracle."""
from __future__ import annotations

import numpy as np
import torch

from hierarchical_kv_approximation_amd import lod, synth
from oracle import oracle as orc

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def configs(dtype, Hq, Hkv, G, TG=8, TP=2, W=512, S=4, iters=10, drop=False):
    gcfg = lod.Config(n_q_heads=Hq, n_kv_heads=Hkv, groups=G, top_groups=TG, top_pages=TP,
                      window=W, n_sink=S, kmeans_iters=iters, dtype=dtype, drop_remainder=drop)
    ocfg = orc.Config(d=128, groups=G, top_groups=TG, top_pages=TP, window=W, n_sink=S, iters=iters,
                      bf16=(dtype == torch.bfloat16), drop_remainder=drop)
    return gcfg, ocfg


class Case:
    """Inputs on host and device, GPU index built by k-means (or injected assignments)."""

    def __init__(self, gcfg, ocfg, B, T, seed=0, sigma=0.3, zero_variance=False, device="cuda",
                 gen_device="cpu", n_centres=32):
        self.gcfg, self.ocfg, self.B, self.T = gcfg, ocfg, B, T
        Hkv = gcfg.n_kv_heads
        K, V, cen, _ = synth.clustered_kv(B, T, Hkv, 128, seed=seed, sigma=sigma, dtype=gcfg.dtype,
                                          zero_variance=zero_variance, device=gen_device,
                                          n_centres=n_centres)
        self.cen = cen
        self.Kd, self.Vd = K.to(device), V.to(device)
        self.K, self.V = K, V  # generator-side copies (host or device)
        self.nchunks = T // 256
        self.index = lod.LodIndex.allocate(gcfg, B, T, device=device)
        self._streams = {}

    def build_gpu(self, n_chunks=None, assign_in=None):
        n = self.nchunks if n_chunks is None else n_chunks
        a = lod.build_chunk(self.gcfg, self.index, self.Kd, self.Vd, 0, n, assign_in=assign_in,
                            want_assign=True)
        torch.cuda.synchronize()
        return a

    def stream(self, b, h):
        if (b, h) not in self._streams:
            self._streams[(b, h)] = (self.K[b, :, h, :].float().cpu().numpy().copy(),
                                     self.V[b, :, h, :].float().cpu().numpy().copy())
        return self._streams[(b, h)]

    def oracle_index(self, keys, n_chunks=None, assign_in=None):
        n = self.nchunks if n_chunks is None else n_chunks
        st = {k: self.stream(*k) for k in keys}
        ain = None
        if assign_in is not None:
            ain = assign_in.cpu().numpy()
        return st, orc.build_all(self.ocfg, st, n, assign_in=ain)

    def queries(self, seed=1, kind="matched", n_rows=None):
        return synth.queries(self.B, self.gcfg.n_q_heads, self.cen, seed=seed, kind=kind,
                             n_rows=n_rows, dtype=self.gcfg.dtype)


def gpu_pages(index: lod.LodIndex, b, h, n_chunks):
    """Per-chunk page lists from the GPU index: (counts [n][PS], members [n][PS][16])."""
    a = index.arrays()
    G, PS = index.cfg.groups, index.cfg.page_slots
    meta = a["meta"][b, h, :n_chunks].cpu().numpy().astype(np.int64)
    gpg, pst, perm = meta[:, : G + 1], meta[:, G + 1: G + 1 + PS + 1], meta[:, G + 1 + PS + 1:]
    counts = pst[:, 1:] - pst[:, :-1]
    mem = -np.ones((n_chunks, PS, 16), np.int64)
    for c in range(n_chunks):
        for sl in range(PS):
            for k in range(counts[c, sl]):
                mem[c, sl, k] = c * 256 + perm[c, pst[c, sl] + k]
    return gpg, counts, mem


def compare_index(index: lod.LodIndex, oidx: dict, b, h, n_chunks):
    """Bit-exact comparison of one stream's summaries and layout with the oracle's."""
    a = index.arrays()
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    assert np.array_equal(a["assign"][b, h, :n_chunks].cpu().numpy().astype(np.int32), oidx["assign"]), \
        "k-means assignments differ"
    gpg, counts, mem = gpu_pages(index, b, h, n_chunks)
    G = index.cfg.groups
    gpage = a["gpage"][b, h, :n_chunks].cpu().numpy().astype(np.int64)
    assert np.array_equal(gpage & 0xffff, gpg[:, :G]) and np.array_equal(gpage >> 16, np.diff(gpg, axis=1)), \
        "group page ranges differ from the meta rows" 
    gcount = np.array([[counts[c, gpg[c, j]:gpg[c, j + 1]].sum() for j in range(G)]
                       for c in range(n_chunks)], dtype=np.int64).reshape(n_chunks, G)
    assert np.array_equal(gcount, oidx["gcount"])
    assert np.array_equal(counts, oidx["pcount"])
    assert np.array_equal(mem, oidx["pmem"])
    for name in ("gk", "gv", "pk", "pv"):
        g = f(a[name][b, h, :n_chunks])
        assert np.array_equal(g.view(np.uint32), oidx[name].view(np.uint32)), f"{name} differs"
    gln = a["gln"][b, h, :n_chunks].cpu().numpy()
    assert np.array_equal(np.isfinite(gln), oidx["gcount"] > 0)
    ok = oidx["gcount"] > 0
    assert np.allclose(gln[ok], np.log(oidx["gcount"][ok]), rtol=0, atol=1e-6)


def paged_copy(K, V, bs, seed, spare=7):
    """[B][T][Hkv][d] -> (pool [nblk][bs][Hkv][d] of K, of V, block_table [B][T/bs]):
    each sequence's blocks scattered over a shared pool in a seeded random order, a few
    blocks unused, as a serving engine's block allocator leaves them."""
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


def _view(case, view):
    """(K, V, block_table) the GPU calls read: the strided cache, or a paged copy."""
    return (case.Kd, case.Vd, None) if view is None else view


def decode_and_compare(case, keys_oidx, seq, q, check_heads=None, view=None):
    """GPU decode at seq_lens=seq vs the oracle on every (b, h) (or check_heads):
    selections bit-exact, outputs within tolerance.  Returns the worst error."""
    g, o = case.gcfg, case.ocfg
    st, oidx = keys_oidx
    K, V, table = _view(case, view)
    dev = case.Kd.device
    sl = torch.tensor(seq, dtype=torch.int32, device=dev)
    out, sg, sp = lod.attend_decode(g, case.index, K, V, q.to(dev), sl, max(seq), want_selection=True,
                                    block_table=table)
    torch.cuda.synchronize()
    out, sg, sp = out.cpu().numpy(), sg.cpu().numpy(), sp.cpu().numpy()
    qf = q.float().cpu().numpy()
    hpg = g.n_q_heads // g.n_kv_heads
    heads = check_heads or [(b, h) for b in range(case.B) for h in range(g.n_q_heads)]
    worst = 0.0
    for b, h in heads:
        kv = (b, h // hpg)
        r = orc.attend(o, oidx[kv], *st[kv], qf[b, h], seq[b] - 1)
        assert np.array_equal(sg[b, h], r["sel_groups"]), (b, h, sg[b, h], r["sel_groups"])
        assert np.array_equal(sp[b, h], r["sel_pages"]), (b, h)
        worst = max(worst, float(np.max(np.abs(out[b, h] - r["out"]))))
    assert worst <= TOL[g.dtype], worst
    return worst


def sample_rows(B, nq, Hq, n, seed):
    """n seeded (b, row, head) triples plus the four corners."""
    rng = np.random.default_rng(seed)
    rows = {(b, i, h) for b, i, h in zip(rng.integers(0, B, n), rng.integers(0, nq, n), rng.integers(0, Hq, n))}
    rows |= {(0, 0, 0), (B - 1, nq - 1, Hq - 1), (0, nq - 1, 0), (B - 1, 0, Hq - 1)}
    return sorted(rows)


def prefill_and_compare(case, Q, q_start, rows, check_dense=False, view=None):
    """GPU LoD prefill of every row of Q vs the oracle on the sampled rows: selection
    bit-exact, outputs within tolerance.  Returns (worst error, GPU outputs)."""
    g, o = case.gcfg, case.ocfg
    K, V, table = _view(case, view)
    out, sg, sp = lod.attend_prefill(g, case.index, K, V, Q.cuda(), q_start, want_selection=True,
                                     block_table=table)
    # without the selection outputs the kernels only certify which groups and pages open
    # (no rank order): the same groups and pages open, so the outputs agree bit for bit
    out_plain = lod.attend_prefill(g, case.index, K, V, Q.cuda(), q_start, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(out, out_plain), float((out - out_plain).abs().max())
    out, sg, sp = out.cpu().numpy(), sg.cpu().numpy(), sp.cpu().numpy()
    hpg = g.n_q_heads // g.n_kv_heads
    st, oidx = case.oracle_index(sorted({(b, h // hpg) for b, _, h in rows}))
    ref = orc.prefill_rows(o, st, oidx, Q.float().numpy(), q_start, rows)
    worst = 0.0
    for (b, i, h), r in ref.items():
        assert np.array_equal(sg[b, i, h], r["sel_groups"]), ((b, i, h), sg[b, i, h], r["sel_groups"])
        assert np.array_equal(sp[b, i, h], r["sel_pages"]), ((b, i, h), sp[b, i, h], r["sel_pages"])
        worst = max(worst, float(np.max(np.abs(out[b, i, h] - r["out"]))))
    assert worst <= TOL[g.dtype], worst
    if check_dense:
        dref = orc.dense_rows(o, st, Q.float().numpy(), q_start, rows)
        dworst = max(float(np.max(np.abs(out[r] - dref[r]))) for r in rows)
        assert dworst <= TOL[g.dtype], dworst
    return worst, out
