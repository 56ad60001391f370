"""Python face of the LoD attention oracle (``lod_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline call it; the GPU library never does.  It imports nothing from the GPU
package and the GPU package imports nothing from here.

Everything is numpy on the host.  Arrays that the method treats as one
(sequence, KV head) stream are passed to C as contiguous ``float32 [T][d]``.
The method follows "Level of Detail Attention" (featherless.ai blog), section
"How It Works"; the readings for what the post leaves open are in the header of
``lod_oracle.c``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lod_oracle.c")
_SRC_VIDEO = os.path.join(_HERE, "video_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblod_oracle.so")

ORC_OK = 0
ORC_ERR_ARG = -1
ORC_ERR_DOUBLE_COUNT = -2
ORC_ERR_NOT_BUILT = -3


def build_library(force: bool = True) -> str:
    """Compile the oracle with gcc: no fast-math, no fp contraction."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", _LIB_PATH + ".tmp", _SRC, _SRC_VIDEO, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("chunk", ctypes.c_int32), ("page", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("top_groups", ctypes.c_int32),
                ("top_pages", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("bf16_store", ctypes.c_int32), ("scale", ctypes.c_double),
                ("drop_remainder", ctypes.c_int32), ("int4_pages", ctypes.c_int32)]


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_library(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        f32p, i32p, f64p = P(ctypes.c_float), P(ctypes.c_int32), P(ctypes.c_double)
        pp = P(_Params)
        lib.orc_round_bf16.restype = ctypes.c_float
        lib.orc_round_bf16.argtypes = [ctypes.c_float]
        lib.orc_canonical_dot.restype = ctypes.c_float
        lib.orc_canonical_dot.argtypes = [f32p, f32p, ctypes.c_int32]
        lib.orc_kmeans.restype = ctypes.c_int32
        lib.orc_kmeans.argtypes = [f32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, i32p, f64p]
        lib.orc_page_slots.restype = ctypes.c_int32
        lib.orc_page_slots.argtypes = [pp]
        lib.orc_built_chunks.restype = ctypes.c_int32
        lib.orc_built_chunks.argtypes = [pp, ctypes.c_int32]
        lib.orc_build.restype = ctypes.c_int32
        lib.orc_build.argtypes = [pp, f32p, f32p, ctypes.c_int32, i32p, i32p, i32p, f32p, f32p,
                                  i32p, i32p, i32p, f32p, f32p]
        lib.orc_attend.restype = ctypes.c_int32
        i8p = P(ctypes.c_int8)
        lib.orc_attend.argtypes = [pp, f32p, ctypes.c_int32, ctypes.c_int32, i32p, f32p, f32p,
                                   i32p, i32p, i32p, f32p, f32p, f32p, f32p, i8p, i8p, f32p, f32p,
                                   f64p, i32p, i32p, f64p, i32p]
        lib.orc_encode_int4.restype = ctypes.c_int32
        lib.orc_encode_int4.argtypes = [pp, f32p, f32p, ctypes.c_int32, i32p, f32p, f32p, i8p, i8p,
                                        f32p, f32p]
        lib.orc_dense.restype = ctypes.c_int32
        lib.orc_dense.argtypes = [pp, f32p, ctypes.c_int32, f32p, f32p, f64p, f64p]
        _lib = lib
    return _lib


def _p(a, ct):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ct))


@dataclass(frozen=True)
class Config:
    """LoD parameters (chunk 256, pages of 16, top 8 groups, top 2 pages by default)."""
    d: int = 128
    chunk: int = 256
    page: int = 16
    groups: int = 8
    top_groups: int = 8
    top_pages: int = 2
    window: int = 512
    n_sink: int = 4
    iters: int = 10
    bf16: bool = False
    scale: float | None = None
    drop_remainder: bool = False  # sparsity ablation: exact keys only, no coarse terms
    int4_pages: bool = False      # three-tier INT4: opened pages decoded from 4-bit codes

    def params(self) -> _Params:
        sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)
        return _Params(self.d, self.chunk, self.page, self.groups, self.top_groups,
                       self.top_pages, self.window, self.n_sink, self.iters,
                       1 if self.bf16 else 0, sc, 1 if self.drop_remainder else 0,
                       1 if self.int4_pages else 0)

    @property
    def page_slots(self) -> int:
        return self.chunk // self.page + self.groups

    def built_chunks(self, p: int) -> int:
        return max(0, p // self.chunk - self.window // self.chunk + 1)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def round_bf16(x) -> np.ndarray:
    x = _f32(x)
    f = _L().orc_round_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.float32).reshape(x.shape)


def canonical_dot(a, b) -> np.float32:
    a, b = _f32(a), _f32(b)
    assert a.shape == b.shape and a.ndim == 1
    return np.float32(_L().orc_canonical_dot(_p(a, ctypes.c_float), _p(b, ctypes.c_float),
                                             a.shape[0]))


def kmeans(x, groups: int, iters: int):
    """Returns (assign[m] int32, objective[iters] float64)."""
    x = _f32(x)
    m, d = x.shape
    a = np.empty(m, np.int32)
    obj = np.empty(iters, np.float64)
    rc = _L().orc_kmeans(_p(x, ctypes.c_float), m, d, groups, iters, _p(a, ctypes.c_int32),
                         _p(obj, ctypes.c_double))
    if rc != ORC_OK:
        raise RuntimeError(f"orc_kmeans failed: {rc}")
    return a, obj


def build_stream(cfg: Config, K, V, n_chunks: int, assign_in=None) -> dict:
    """Multi-resolution view of chunks [0, n_chunks) of one stream K, V [T][d]."""
    K, V = _f32(K), _f32(V)
    C, G, PS, P, d = cfg.chunk, cfg.groups, cfg.page_slots, cfg.page, cfg.d
    assert K.shape[1] == d and K.shape[0] >= n_chunks * C
    idx = {
        "assign": np.empty((n_chunks, C), np.int32),
        "gcount": np.empty((n_chunks, G), np.int32),
        "gk": np.empty((n_chunks, G, d), np.float32),
        "gv": np.empty((n_chunks, G, d), np.float32),
        "pgroup": np.empty((n_chunks, PS), np.int32),
        "pcount": np.empty((n_chunks, PS), np.int32),
        "pmem": np.empty((n_chunks, PS, P), np.int32),
        "pk": np.empty((n_chunks, PS, d), np.float32),
        "pv": np.empty((n_chunks, PS, d), np.float32),
    }
    ain = None if assign_in is None else np.ascontiguousarray(assign_in, dtype=np.int32)
    prm = cfg.params()
    i32, f32 = ctypes.c_int32, ctypes.c_float
    rc = _L().orc_build(ctypes.byref(prm), _p(K, f32), _p(V, f32), n_chunks, _p(ain, i32),
                        _p(idx["assign"], i32), _p(idx["gcount"], i32), _p(idx["gk"], f32),
                        _p(idx["gv"], f32), _p(idx["pgroup"], i32), _p(idx["pcount"], i32),
                        _p(idx["pmem"], i32), _p(idx["pk"], f32), _p(idx["pv"], f32))
    if rc != ORC_OK:
        raise RuntimeError(f"orc_build failed: {rc}")
    idx["n_chunks"] = n_chunks
    if cfg.int4_pages:
        idx["qk"] = np.empty((n_chunks, C, d), np.int8)
        idx["qv"] = np.empty((n_chunks, C, d), np.int8)
        idx["qks"] = np.empty((n_chunks, C), np.float32)
        idx["qvs"] = np.empty((n_chunks, C), np.float32)
        i8 = ctypes.c_int8
        rc = _L().orc_encode_int4(ctypes.byref(prm), _p(K, f32), _p(V, f32), n_chunks, _p(idx["assign"], i32),
                                  _p(idx["gk"], f32), _p(idx["gv"], f32), _p(idx["qk"], i8), _p(idx["qv"], i8),
                                  _p(idx["qks"], f32), _p(idx["qvs"], f32))
        if rc != ORC_OK:
            raise RuntimeError(f"orc_encode_int4 failed: {rc}")
    return idx


def attend(cfg: Config, idx: dict, K, V, q, p: int):
    """LoD attention of one query at position p.

    Returns dict(out=float64[d], sel_groups, sel_pages, log_mass, n_terms)."""
    K, V, q = _f32(K), _f32(V), _f32(q)
    TG, TPW = cfg.top_groups, max(cfg.top_pages, 1)
    out = np.empty(cfg.d, np.float64)
    sg = np.empty(TG, np.int32)
    sp = np.empty(TG * TPW, np.int32)
    lm = np.zeros(1, np.float64)
    nt = np.zeros(3, np.int32)
    prm = cfg.params()
    i32, f32, f64, i8 = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_int8
    if cfg.int4_pages and "qk" not in idx:
        raise ValueError("the index was built without INT4 codes")
    rc = _L().orc_attend(ctypes.byref(prm), _p(q, f32), p, idx["n_chunks"], _p(idx["gcount"], i32),
                         _p(idx["gk"], f32), _p(idx["gv"], f32), _p(idx["pgroup"], i32),
                         _p(idx["pcount"], i32), _p(idx["pmem"], i32), _p(idx["pk"], f32),
                         _p(idx["pv"], f32), _p(K, f32), _p(V, f32), _p(idx.get("qk"), i8),
                         _p(idx.get("qv"), i8), _p(idx.get("qks"), f32), _p(idx.get("qvs"), f32),
                         _p(out, f64), _p(sg, i32), _p(sp, i32), _p(lm, f64), _p(nt, i32))
    if rc != ORC_OK:
        raise RuntimeError(f"orc_attend failed: {rc}")
    return {"out": out, "sel_groups": sg, "sel_pages": sp.reshape(TG, TPW),
            "log_mass": float(lm[0]), "n_terms": nt}


def dense(cfg: Config, K, V, q, p: int):
    """Dense causal softmax attention over rows [0, p]; returns (out float64[d], log_mass)."""
    K, V, q = _f32(K), _f32(V), _f32(q)
    out = np.empty(cfg.d, np.float64)
    lm = np.zeros(1, np.float64)
    prm = cfg.params()
    rc = _L().orc_dense(ctypes.byref(prm), _p(q, ctypes.c_float), p, _p(K, ctypes.c_float),
                        _p(V, ctypes.c_float), _p(out, ctypes.c_double), _p(lm, ctypes.c_double))
    if rc != ORC_OK:
        raise RuntimeError(f"orc_dense failed: {rc}")
    return out, float(lm[0])


# ---------------------------------------------------------------------------
# batched helpers over [B][T][Hkv][d] caches (threads over independent streams)
# ---------------------------------------------------------------------------

def _threads(threads):
    return threads or os.cpu_count() or 1


def streams(K, V):
    """Split [B][T][Hkv][d] caches into contiguous per-(b, kvh) streams."""
    K, V = np.asarray(K), np.asarray(V)
    B, T, Hkv, d = K.shape
    return {(b, h): (_f32(K[b, :, h, :]), _f32(V[b, :, h, :])) for b in range(B) for h in range(Hkv)}


def build_all(cfg: Config, st: dict, n_chunks, assign_in=None, threads=None) -> dict:
    """Build every stream.  n_chunks: int or {b: int}; assign_in: [B][Hkv][n][C] or None."""
    def one(key):
        b, h = key
        n = n_chunks[b] if isinstance(n_chunks, dict) else n_chunks
        ain = None if assign_in is None else np.asarray(assign_in)[b, h, :n]
        return key, build_stream(cfg, st[key][0], st[key][1], n, ain)
    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, list(st.keys())))


def decode(cfg: Config, st: dict, index: dict, Q, seq_lens, threads=None):
    """LoD decode for Q [B][Hq][d] at positions seq_lens[b]-1.

    Returns (out float32 [B][Hq][d], out64, sel_groups [B][Hq][TG], sel_pages [B][Hq][TG][TPW])."""
    Q = _f32(Q)
    B, Hq, d = Q.shape
    Hkv = len({k[1] for k in st})
    g = Hq // Hkv
    TG, TPW = cfg.top_groups, max(cfg.top_pages, 1)
    out = np.empty((B, Hq, d), np.float64)
    sg = np.empty((B, Hq, TG), np.int32)
    sp = np.empty((B, Hq, TG, TPW), np.int32)

    def one(bh):
        b, h = bh
        kv = (b, h // g)
        r = attend(cfg, index[kv], st[kv][0], st[kv][1], Q[b, h], int(seq_lens[b]) - 1)
        out[b, h], sg[b, h], sp[b, h] = r["out"], r["sel_groups"], r["sel_pages"]

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(one, [(b, h) for b in range(B) for h in range(Hq)]))
    return out.astype(np.float32), out, sg, sp


def prefill_rows(cfg: Config, st: dict, index: dict, Q, q_start: int, rows=None, threads=None):
    """LoD attention for prefill rows.  Q [B][n_q][Hq][d] holds rows q_start .. q_start+n_q-1.

    rows: optional list of (b, i, h) to evaluate (i is the row within Q); default all.
    Returns dict {(b, i, h): attend-result}."""
    Q = _f32(Q)
    B, nq, Hq, d = Q.shape
    Hkv = len({k[1] for k in st})
    g = Hq // Hkv
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(nq) for h in range(Hq)]

    def one(r):
        b, i, h = r
        kv = (b, h // g)
        return r, attend(cfg, index[kv], st[kv][0], st[kv][1], Q[b, i, h], q_start + i)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, rows))


def dense_rows(cfg: Config, st: dict, Q, q_start: int, rows, threads=None):
    """Dense causal attention for the (b, i, h) rows of Q [B][n_q][Hq][d]."""
    Q = _f32(Q)
    Hq = Q.shape[2]
    Hkv = len({k[1] for k in st})
    g = Hq // Hkv

    def one(r):
        b, i, h = r
        kv = (b, h // g)
        return r, dense(cfg, st[kv][0], st[kv][1], Q[b, i, h], q_start + i)[0]

    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, rows))
