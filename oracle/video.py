"""Python face of the video LoD oracle (``video_oracle.c``, built into liblod_oracle.so).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU baseline
call it; the GPU library never does, and nothing here imports the GPU package.

Method: "Level of Detail Attention" (featherless.ai blog), section "Video LoD" --
queries and keys/values in 4x4x4 blocks of a video token grid, LoD at c = 16 opened
blocks.  The readings for what the section leaves open are in the header of
``video_oracle.c``.  Arrays follow the GPU layout: Q [B][T][Hq][d], K, V [B][T][Hkv][d]
with T = frames * height * width tokens in raster order.
"""
from __future__ import annotations

import ctypes
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import oracle as _orc


class _VParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("frames", ctypes.c_int32), ("height", ctypes.c_int32),
                ("width", ctypes.c_int32), ("bf", ctypes.c_int32), ("bh", ctypes.c_int32),
                ("bw", ctypes.c_int32), ("top_blocks", ctypes.c_int32),
                ("bf16_store", ctypes.c_int32), ("drop_remainder", ctypes.c_int32),
                ("scale", ctypes.c_double)]


_vlib = None


def _L():
    global _vlib
    if _vlib is None:
        lib = _orc._L()
        P = ctypes.POINTER
        f32p, i32p, f64p, pp = P(ctypes.c_float), P(ctypes.c_int32), P(ctypes.c_double), P(_VParams)
        lib.orc_video_blocks.restype = ctypes.c_int32
        lib.orc_video_blocks.argtypes = [pp]
        lib.orc_video_members.restype = ctypes.c_int32
        lib.orc_video_members.argtypes = [pp, ctypes.c_int32, i32p]
        lib.orc_video_summaries.restype = ctypes.c_int32
        lib.orc_video_summaries.argtypes = [pp, f32p, ctypes.c_int32, f32p, i32p]
        lib.orc_video_select.restype = ctypes.c_int32
        lib.orc_video_select.argtypes = [pp, f32p, f32p, i32p, f32p]
        lib.orc_video_attend.restype = ctypes.c_int32
        lib.orc_video_attend.argtypes = [pp, f32p, f32p, f32p, f32p, f32p, i32p, i32p, ctypes.c_int32,
                                         f64p, f64p, f64p]
        lib.orc_video_dense.restype = ctypes.c_int32
        lib.orc_video_dense.argtypes = [pp, f32p, f32p, f32p, ctypes.c_int32, f64p]
        _vlib = lib
    return _vlib


def _p(a, ct):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ct))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc < 0:
        raise RuntimeError(f"{what} failed with status {rc}")
    return rc


@dataclass(frozen=True)
class VideoConfig:
    """Grid, block shape and LoD parameters of video attention (4x4x4 blocks, c = 16)."""
    d: int = 128
    frames: int = 8
    height: int = 8
    width: int = 8
    block: tuple = (4, 4, 4)
    top_blocks: int = 16
    bf16: bool = False
    scale: float | None = None
    drop_remainder: bool = False

    def params(self) -> _VParams:
        sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)
        return _VParams(self.d, self.frames, self.height, self.width, *self.block, self.top_blocks,
                        1 if self.bf16 else 0, 1 if self.drop_remainder else 0, sc)

    @property
    def n_tokens(self) -> int:
        return self.frames * self.height * self.width

    @property
    def n_blocks(self) -> int:
        return _check(_L().orc_video_blocks(ctypes.byref(self.params())), "orc_video_blocks")

    @property
    def block_size(self) -> int:
        return self.block[0] * self.block[1] * self.block[2]


def members(cfg: VideoConfig, blk: int) -> np.ndarray:
    """Tokens of block blk, ascending."""
    tok = np.empty(cfg.block_size, np.int32)
    n = _check(_L().orc_video_members(ctypes.byref(cfg.params()), blk, _p(tok, ctypes.c_int32)),
               "orc_video_members")
    return tok[:n].copy()


def summaries(cfg: VideoConfig, X, round_bf16: bool):
    """Per-block canonical means of X [T][d]: (mean [nb][d] float32, count [nb] int32)."""
    X = _f32(X)
    nb = cfg.n_blocks
    mean = np.empty((nb, cfg.d), np.float32)
    cnt = np.empty(nb, np.int32)
    _check(_L().orc_video_summaries(ctypes.byref(cfg.params()), _p(X, ctypes.c_float), 1 if round_bf16 else 0,
                                    _p(mean, ctypes.c_float), _p(cnt, ctypes.c_int32)), "orc_video_summaries")
    return mean, cnt


def select(cfg: VideoConfig, qbar_row, kbar):
    """Opened blocks of one query block (ascending, -1 padding) and every score."""
    qbar_row, kbar = _f32(qbar_row), _f32(kbar)
    sel = np.empty(cfg.top_blocks, np.int32)
    sc = np.empty(kbar.shape[0], np.float32)
    _check(_L().orc_video_select(ctypes.byref(cfg.params()), _p(qbar_row, ctypes.c_float),
                                 _p(kbar, ctypes.c_float), _p(sel, ctypes.c_int32), _p(sc, ctypes.c_float)),
           "orc_video_select")
    return sel, sc


def attend_block(cfg: VideoConfig, Qh, Kh, Vh, kbar, vbar, count, sel_row, qblk: int):
    """LoD output of the queries of block qblk for one (query head, KV head) pair:
    (out [n][d] float64, exact mass [n], coarse mass [n]) in member order."""
    n = len(members(cfg, qblk))
    out = np.empty((n, cfg.d), np.float64)
    me = np.empty(n, np.float64)
    mc = np.empty(n, np.float64)
    sel_row = np.ascontiguousarray(sel_row, np.int32)
    _check(_L().orc_video_attend(ctypes.byref(cfg.params()), _p(Qh, ctypes.c_float), _p(Kh, ctypes.c_float),
                                 _p(Vh, ctypes.c_float), _p(kbar, ctypes.c_float), _p(vbar, ctypes.c_float),
                                 _p(count, ctypes.c_int32), _p(sel_row, ctypes.c_int32), qblk,
                                 _p(out, ctypes.c_double), _p(me, ctypes.c_double), _p(mc, ctypes.c_double)),
           "orc_video_attend")
    return out, me, mc


def dense_block(cfg: VideoConfig, Qh, Kh, Vh, qblk: int):
    """Dense bidirectional output of the queries of block qblk (float64, member order)."""
    n = len(members(cfg, qblk))
    out = np.empty((n, cfg.d), np.float64)
    _check(_L().orc_video_dense(ctypes.byref(cfg.params()), _p(Qh, ctypes.c_float), _p(Kh, ctypes.c_float),
                                _p(Vh, ctypes.c_float), qblk, _p(out, ctypes.c_double)), "orc_video_dense")
    return out


def forward(cfg: VideoConfig, Q, K, V, *, pairs=None, threads=None, dense: bool = False):
    """Video LoD attention over Q [B][T][Hq][d], K, V [B][T][Hkv][d].

    pairs: optional list of (b, h, qblk) to evaluate (default: every query block of
    every head).  Returns a dict with
      out    [B][T][Hq][d] float64 (NaN where not evaluated),
      sel    [B][Hq][nb][c] int32 (-2 where not evaluated),
      kbar, vbar [B][Hkv][nb][d] float32, qbar [B][Hq][nb][d] float32, count [nb],
      exact_mass, coarse_mass  {(b, h, qblk): [n]},
      dense  [B][T][Hq][d] float64 of the same pairs when dense=True.
    Summaries cover every block; the selection and outputs only the given pairs."""
    Q, K, V = np.asarray(Q), np.asarray(K), np.asarray(V)
    B, T, Hq, d = Q.shape
    Hkv = K.shape[2]
    assert T == cfg.n_tokens and d == cfg.d and Hq % Hkv == 0
    g = Hq // Hkv
    nb = cfg.n_blocks
    th = threads or os.cpu_count() or 1
    Ks = {(b, h): _f32(K[b, :, h, :]) for b in range(B) for h in range(Hkv)}
    Vs = {(b, h): _f32(V[b, :, h, :]) for b in range(B) for h in range(Hkv)}
    Qs = {(b, h): _f32(Q[b, :, h, :]) for b in range(B) for h in range(Hq)}
    kbar = np.empty((B, Hkv, nb, d), np.float32)
    vbar = np.empty((B, Hkv, nb, d), np.float32)
    qbar = np.empty((B, Hq, nb, d), np.float32)
    count = None
    for (b, h) in Ks:
        kbar[b, h], count = summaries(cfg, Ks[(b, h)], cfg.bf16)
        vbar[b, h], _ = summaries(cfg, Vs[(b, h)], cfg.bf16)
    for (b, h) in Qs:
        qbar[b, h], _ = summaries(cfg, Qs[(b, h)], False)
    if pairs is None:
        pairs = [(b, h, j) for b in range(B) for h in range(Hq) for j in range(nb)]
    out = np.full((B, T, Hq, d), np.nan)
    dout = np.full((B, T, Hq, d), np.nan) if dense else None
    sel = np.full((B, Hq, nb, cfg.top_blocks), -2, np.int32)
    em, cm = {}, {}

    def one(pr):
        b, h, j = pr
        kv = (b, h // g)
        s, _ = select(cfg, qbar[b, h, j], kbar[b, h // g])
        o, me, mc = attend_block(cfg, Qs[(b, h)], Ks[kv], Vs[kv], kbar[kv[0], kv[1]], vbar[kv[0], kv[1]],
                                 count, s, j)
        do = dense_block(cfg, Qs[(b, h)], Ks[kv], Vs[kv], j) if dense else None
        return pr, s, o, me, mc, do

    with ThreadPoolExecutor(th) as ex:
        for (b, h, j), s, o, me, mc, do in ex.map(one, pairs):
            tok = members(cfg, j)
            sel[b, h, j] = s
            out[b, tok, h] = o
            if dense:
                dout[b, tok, h] = do
            em[(b, h, j)], cm[(b, h, j)] = me, mc
    return {"out": out, "sel": sel, "kbar": kbar, "vbar": vbar, "qbar": qbar, "count": count,
            "exact_mass": em, "coarse_mass": cm, "dense": dout}
