"""ctypes binding of the LoD HIP library (liblod.so).

Argument marshalling only: every step of the method runs in the library's kernels.
torch provides device memory and the current HIP stream, nothing else.  The library
must be built (``__graft_entry__.build()`` or ``python -m
hierarchical_kv_approximation_amd._build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from dataclasses import dataclass, field

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblod.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "lod.h")

LOD_OK, LOD_ERR_ARG, LOD_ERR_UNSUPPORTED, LOD_ERR_WORKSPACE, LOD_ERR_HIP = 0, -1, -2, -3, -4
LOD_F32, LOD_BF16 = 0, 1


class Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "head_dim", "n_q_heads", "n_kv_heads", "chunk_size", "page_size", "groups_per_chunk",
        "top_groups", "top_pages", "window", "n_sink", "kmeans_iters", "kv_dtype")] + \
        [("scale", ctypes.c_float), ("drop_remainder", ctypes.c_int32), ("int4_pages", ctypes.c_int32)]


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_t", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32)]


class Index(ctypes.Structure):
    _fields_ = [("mem", ctypes.c_void_p), ("bytes", ctypes.c_size_t), ("batch", ctypes.c_int32),
                ("max_chunks", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("gk", "gv", "gln", "gkn", "gpage", "pk", "pv", "pln", "meta", "assign", "q4k", "q4v",
                 "q4ks", "q4vs", "total")] + \
        [("page_slots", ctypes.c_int32), ("meta_stride", ctypes.c_int32)]


class VideoParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "head_dim", "n_q_heads", "n_kv_heads", "frames", "height", "width", "block_f", "block_h",
        "block_w", "top_blocks", "kv_dtype", "drop_remainder")] + [("scale", ctypes.c_float)]


class VideoLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("kbar", "vbar", "lnn", "qbar", "sel", "total")] + \
        [("n_blocks", ctypes.c_int32)]


class LodError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {lib().lod_status_string(status).decode()}")
        self.status = status


_lib = None


def lib():
    """Load liblod.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m hierarchical_kv_approximation_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        P, vp, i32, i64, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pp = P(Params)
        L.lod_status_string.restype = ctypes.c_char_p
        L.lod_status_string.argtypes = [ctypes.c_int]
        L.lod_index_bytes.argtypes = [pp, i32, i32, P(sz)]
        L.lod_index_layout.argtypes = [pp, i32, i32, P(Layout)]
        L.lod_build_chunk.argtypes = [pp, P(Index), KV, i32, i32, i32, vp, vp, vp]
        L.lod_decode_ws_bytes.argtypes = [pp, i32, i32, P(sz)]
        L.lod_attend_decode.argtypes = [pp, P(Index), KV, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.lod_attend_decode_noalloc.argtypes = [pp, P(Index), KV, vp, vp, i32, i32, vp, vp, vp, vp]
        L.lod_prefill_ws_bytes.argtypes = [pp, i32, i32, i32, P(sz)]
        L.lod_attend_prefill.argtypes = [pp, P(Index), KV, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.lod_dense_decode_ws_bytes.argtypes = [pp, i32, i32, P(sz)]
        L.lod_dense_decode.argtypes = [pp, KV, vp, vp, i32, i32, vp, vp, sz, vp]
        L.lod_dense_prefill.argtypes = [pp, KV, vp, i32, i32, i32, vp, vp]
        L.lod_trace_events.argtypes = [P(vp), i32]
        vpp = P(VideoParams)
        L.lod_video_layout.argtypes = [vpp, i32, P(VideoLayout)]
        L.lod_video_ws_bytes.argtypes = [vpp, i32, P(sz)]
        L.lod_video_attend.argtypes = [vpp, KV, vp, i32, vp, vp, vp, sz, vp]
        L.lod_video_dense.argtypes = [vpp, KV, vp, i32, vp, vp]
        for fn in ("lod_index_bytes", "lod_index_layout", "lod_build_chunk", "lod_decode_ws_bytes",
                   "lod_attend_decode", "lod_attend_decode_noalloc", "lod_prefill_ws_bytes", "lod_attend_prefill",
                   "lod_dense_decode_ws_bytes", "lod_dense_decode", "lod_dense_prefill",
                   "lod_trace_events", "lod_video_layout", "lod_video_ws_bytes", "lod_video_attend",
                   "lod_video_dense"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/lod.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(lod_\w+)\s*\(", text, re.M)))


def _check(fn, status):
    if status != LOD_OK:
        raise LodError(fn, status)


@dataclass
class Config:
    """LoD parameters (chunk 256, pages of 16, top 8 groups / top 2 pages by default)."""
    n_q_heads: int = 64
    n_kv_heads: int = 8
    groups: int = 8
    top_groups: int = 8
    top_pages: int = 2
    window: int = 512
    n_sink: int = 4
    kmeans_iters: int = 10
    dtype: torch.dtype = torch.bfloat16
    head_dim: int = 128
    chunk_size: int = 256
    page_size: int = 16
    scale: float | None = None
    drop_remainder: bool = False  # sparsity ablation: the same selection, exact keys only
    int4_pages: bool = False      # three-tier INT4: opened pages decoded from 4-bit codes

    def params(self) -> Params:
        sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)
        dt = {torch.float32: LOD_F32, torch.bfloat16: LOD_BF16}.get(self.dtype, 99)
        return Params(self.head_dim, self.n_q_heads, self.n_kv_heads, self.chunk_size,
                      self.page_size, self.groups, self.top_groups, self.top_pages, self.window,
                      self.n_sink, self.kmeans_iters, dt, sc, 1 if self.drop_remainder else 0,
                      1 if self.int4_pages else 0)

    @property
    def page_slots(self) -> int:
        return self.chunk_size // self.page_size + self.groups


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def kv_view(K: torch.Tensor, V: torch.Tensor, block_table: torch.Tensor | None = None) -> KV:
    """The library's KV view.  Strided: K, V are [B][T][Hkv][d] (any strides, last dim
    contiguous).  Paged: K, V are [num_blocks][block_size][Hkv][d] caches and block_table
    [B][max_blocks] (device int32) names the block of every block_size positions."""
    assert K.shape == V.shape and K.stride() == V.stride() and K.dtype == V.dtype
    assert K.stride(3) == 1
    if block_table is None:
        return KV(K.data_ptr(), V.data_ptr(), K.stride(0), K.stride(1), K.stride(2), None, 0, 0)
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.dim() == 2
    return KV(K.data_ptr(), V.data_ptr(), K.stride(0), K.stride(1), K.stride(2), block_table.data_ptr(),
              K.shape[1], block_table.shape[1])


def _batch(K, block_table):
    return K.shape[0] if block_table is None else block_table.shape[0]


@dataclass
class LodIndex:
    """Caller-owned multi-resolution view (a device byte tensor)."""
    cfg: Config
    batch: int
    max_chunks: int
    mem: torch.Tensor = field(repr=False)

    @classmethod
    def allocate(cls, cfg: Config, batch: int, max_tokens: int, device="cuda"):
        n = ctypes.c_size_t()
        _check("lod_index_bytes", lib().lod_index_bytes(ctypes.byref(cfg.params()), batch, max_tokens,
                                                        ctypes.byref(n)))
        mem = torch.zeros(n.value, dtype=torch.uint8, device=device)
        return cls(cfg, batch, max_tokens // cfg.chunk_size, mem)

    def c(self) -> Index:
        return Index(self.mem.data_ptr(), self.mem.numel(), self.batch, self.max_chunks)

    def layout(self) -> Layout:
        L = Layout()
        _check("lod_index_layout", lib().lod_index_layout(ctypes.byref(self.cfg.params()), self.batch,
                                                          self.max_chunks, ctypes.byref(L)))
        return L

    def arrays(self) -> dict:
        """Typed views of the index arrays (for inspection and tests)."""
        L, cfg = self.layout(), self.cfg
        U = self.batch * cfg.n_kv_heads
        NC, G, PS, d = self.max_chunks, cfg.groups, L.page_slots, cfg.head_dim
        es = 2 if cfg.dtype == torch.bfloat16 else 4

        def view(off, count, dt, shape):
            nbytes = count * torch.tensor([], dtype=dt).element_size()
            return self.mem[off:off + nbytes].view(dt).view(*shape)

        return {
            "gk": view(L.gk, U * NC * G * d, cfg.dtype, (self.batch, cfg.n_kv_heads, NC, G, d)),
            "gv": view(L.gv, U * NC * G * d, cfg.dtype, (self.batch, cfg.n_kv_heads, NC, G, d)),
            "gln": view(L.gln, U * NC * G, torch.float32, (self.batch, cfg.n_kv_heads, NC, G)),
            "gkn": view(L.gkn, U * NC * G, torch.float32, (self.batch, cfg.n_kv_heads, NC, G)),
            "gpage": view(L.gpage, U * NC * G, torch.int32, (self.batch, cfg.n_kv_heads, NC, G)),
            "pk": view(L.pk, U * NC * PS * d, cfg.dtype, (self.batch, cfg.n_kv_heads, NC, PS, d)),
            "pv": view(L.pv, U * NC * PS * d, cfg.dtype, (self.batch, cfg.n_kv_heads, NC, PS, d)),
            "pln": view(L.pln, U * NC * PS, torch.float32, (self.batch, cfg.n_kv_heads, NC, PS)),
            "meta": view(L.meta, U * NC * L.meta_stride, torch.int16,
                         (self.batch, cfg.n_kv_heads, NC, L.meta_stride)),
            "assign": view(L.assign, U * NC * cfg.chunk_size, torch.int8,
                           (self.batch, cfg.n_kv_heads, NC, cfg.chunk_size)),
            **({"q4k": view(L.q4k, U * NC * cfg.chunk_size * d // 2, torch.uint8,
                            (self.batch, cfg.n_kv_heads, NC, cfg.chunk_size, d // 2)),
                "q4v": view(L.q4v, U * NC * cfg.chunk_size * d // 2, torch.uint8,
                            (self.batch, cfg.n_kv_heads, NC, cfg.chunk_size, d // 2)),
                "q4ks": view(L.q4ks, U * NC * cfg.chunk_size, torch.float32,
                             (self.batch, cfg.n_kv_heads, NC, cfg.chunk_size)),
                "q4vs": view(L.q4vs, U * NC * cfg.chunk_size, torch.float32,
                             (self.batch, cfg.n_kv_heads, NC, cfg.chunk_size))} if cfg.int4_pages else {}),
        } if es else None


def build_chunk(cfg: Config, index: LodIndex, K, V, chunk_begin: int, n_chunks: int,
                assign_in: torch.Tensor | None = None, want_assign: bool = False,
                block_table: torch.Tensor | None = None):
    """lod_build_chunk over chunks [chunk_begin, chunk_begin + n_chunks) of every sequence."""
    B = _batch(K, block_table)
    aout = None
    if want_assign:
        aout = torch.empty(B, cfg.n_kv_heads, n_chunks, cfg.chunk_size, dtype=torch.int32, device=K.device)
    if assign_in is not None:
        assign_in = assign_in.to(device=K.device, dtype=torch.int32).contiguous()
    idx = index.c()
    _check("lod_build_chunk", lib().lod_build_chunk(ctypes.byref(cfg.params()), ctypes.byref(idx),
                                                    kv_view(K, V, block_table), B, chunk_begin, n_chunks,
                                                    _ptr(assign_in), _ptr(aout), _stream()))
    return aout


def decode_ws_bytes(cfg: Config, batch: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check("lod_decode_ws_bytes", lib().lod_decode_ws_bytes(ctypes.byref(cfg.params()), batch,
                                                            max_seq_len, ctypes.byref(n)))
    return n.value


def attend_decode(cfg: Config, index: LodIndex, K, V, q, seq_lens: torch.Tensor, max_seq_len: int,
                  want_selection: bool = False, ws: torch.Tensor | None = None,
                  out: torch.Tensor | None = None, block_table: torch.Tensor | None = None):
    """lod_attend_decode; q [B][Hq][d]; seq_lens device int32 [B].  Returns out (fp32) or
    (out, sel_groups, sel_pages)."""
    B = q.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty(B, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=dev)
    sg = sp = None
    if want_selection:
        sg = torch.empty(B, cfg.n_q_heads, cfg.top_groups, dtype=torch.int32, device=dev)
        sp = torch.empty(B, cfg.n_q_heads, cfg.top_groups, max(cfg.top_pages, 1), dtype=torch.int32,
                         device=dev)
    if ws is None:
        ws = torch.empty(decode_ws_bytes(cfg, B, max_seq_len), dtype=torch.uint8, device=dev)
    idx = index.c()
    _check("lod_attend_decode", lib().lod_attend_decode(
        ctypes.byref(cfg.params()), ctypes.byref(idx), kv_view(K, V, block_table), _ptr(q), _ptr(seq_lens), B,
        max_seq_len, _ptr(out), _ptr(sg), _ptr(sp), _ptr(ws), ws.numel(), _stream()))
    return (out, sg, sp) if want_selection else out


NOALLOC_WS_BYTES = 32 << 20  # LOD_NOALLOC_WS_BYTES of include/lod.h


def attend_decode_noalloc(cfg: Config, index: LodIndex, K, V, q, seq_lens: torch.Tensor, max_seq_len: int,
                          want_selection: bool = False, out: torch.Tensor | None = None,
                          sel: tuple | None = None, block_table: torch.Tensor | None = None):
    """lod_attend_decode_noalloc: lod_attend_decode with the library's fixed device
    workspace.  Pass `out` (and `sel` = (sel_groups, sel_pages)) to allocate nothing here
    either.  Returns out or (out, sel_groups, sel_pages)."""
    B = q.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty(B, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=dev)
    sg = sp = None
    if sel is not None:
        sg, sp = sel
    elif want_selection:
        sg = torch.empty(B, cfg.n_q_heads, cfg.top_groups, dtype=torch.int32, device=dev)
        sp = torch.empty(B, cfg.n_q_heads, cfg.top_groups, max(cfg.top_pages, 1), dtype=torch.int32,
                         device=dev)
    idx = index.c()
    _check("lod_attend_decode_noalloc", lib().lod_attend_decode_noalloc(
        ctypes.byref(cfg.params()), ctypes.byref(idx), kv_view(K, V, block_table), _ptr(q), _ptr(seq_lens), B,
        max_seq_len, _ptr(out), _ptr(sg), _ptr(sp), _stream()))
    return (out, sg, sp) if (want_selection or sel is not None) else out


def prefill_ws_bytes(cfg: Config, batch: int, n_q: int, max_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check("lod_prefill_ws_bytes", lib().lod_prefill_ws_bytes(ctypes.byref(cfg.params()), batch, n_q,
                                                              max_tokens, ctypes.byref(n)))
    return n.value


def attend_prefill(cfg: Config, index: LodIndex, K, V, q, q_start: int, want_selection: bool = False,
                   ws: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   block_table: torch.Tensor | None = None):
    """lod_attend_prefill; q [B][n_q][Hq][d] holds rows q_start .. q_start+n_q-1."""
    B, nq = q.shape[0], q.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty(B, nq, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=dev)
    sg = sp = None
    if want_selection:
        sg = torch.empty(B, nq, cfg.n_q_heads, cfg.top_groups, dtype=torch.int32, device=dev)
        sp = torch.empty(B, nq, cfg.n_q_heads, cfg.top_groups, max(cfg.top_pages, 1),
                         dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(max(1, prefill_ws_bytes(cfg, B, nq, q_start + nq)), dtype=torch.uint8, device=dev)
    idx = index.c()
    _check("lod_attend_prefill", lib().lod_attend_prefill(
        ctypes.byref(cfg.params()), ctypes.byref(idx), kv_view(K, V, block_table), _ptr(q), q_start, nq, B,
        _ptr(out), _ptr(sg), _ptr(sp), _ptr(ws), ws.numel(), _stream()))
    return (out, sg, sp) if want_selection else out


def dense_decode_ws_bytes(cfg: Config, batch: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check("lod_dense_decode_ws_bytes", lib().lod_dense_decode_ws_bytes(
        ctypes.byref(cfg.params()), batch, max_seq_len, ctypes.byref(n)))
    return n.value


def dense_decode(cfg: Config, K, V, q, seq_lens: torch.Tensor, max_seq_len: int,
                 ws: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 block_table: torch.Tensor | None = None):
    B = q.shape[0]
    if out is None:
        out = torch.empty(B, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(dense_decode_ws_bytes(cfg, B, max_seq_len), dtype=torch.uint8, device=q.device)
    _check("lod_dense_decode", lib().lod_dense_decode(
        ctypes.byref(cfg.params()), kv_view(K, V, block_table), _ptr(q), _ptr(seq_lens), B, max_seq_len,
        _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def dense_prefill(cfg: Config, K, V, q, q_start: int, out: torch.Tensor | None = None,
                  block_table: torch.Tensor | None = None):
    B, nq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty(B, nq, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
    _check("lod_dense_prefill", lib().lod_dense_prefill(
        ctypes.byref(cfg.params()), kv_view(K, V, block_table), _ptr(q), q_start, nq, B, _ptr(out), _stream()))
    return out


def trace_events(events):
    """Set (list of raw hipEvent_t handles) or clear (None) the library's trace events."""
    if events is None:
        _check("lod_trace_events", lib().lod_trace_events(None, 0))
        return None
    arr = (ctypes.c_void_p * len(events))(*events)
    _check("lod_trace_events", lib().lod_trace_events(arr, len(events)))
    return arr  # caller keeps it alive while tracing


# ---------------------------------------------------------------------------- video LoD

@dataclass
class VideoConfig:
    """Video LoD: a frames x height x width token grid cut into 4x4x4 blocks, each query
    block opening its top c = 16 key blocks."""
    frames: int = 8
    height: int = 8
    width: int = 8
    n_q_heads: int = 8
    n_kv_heads: int = 8
    block: tuple = (4, 4, 4)
    top_blocks: int = 16
    dtype: torch.dtype = torch.bfloat16
    head_dim: int = 128
    scale: float | None = None
    drop_remainder: bool = False

    def params(self) -> VideoParams:
        sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)
        dt = {torch.float32: LOD_F32, torch.bfloat16: LOD_BF16}.get(self.dtype, 99)
        return VideoParams(self.head_dim, self.n_q_heads, self.n_kv_heads, self.frames, self.height,
                           self.width, *self.block, self.top_blocks, dt, 1 if self.drop_remainder else 0, sc)

    @property
    def n_tokens(self) -> int:
        return self.frames * self.height * self.width


def video_layout(cfg: VideoConfig, batch: int) -> VideoLayout:
    L = VideoLayout()
    _check("lod_video_layout", lib().lod_video_layout(ctypes.byref(cfg.params()), batch, ctypes.byref(L)))
    return L


def video_ws_bytes(cfg: VideoConfig, batch: int) -> int:
    n = ctypes.c_size_t()
    _check("lod_video_ws_bytes", lib().lod_video_ws_bytes(ctypes.byref(cfg.params()), batch, ctypes.byref(n)))
    return n.value


def video_arrays(cfg: VideoConfig, ws: torch.Tensor, batch: int) -> dict:
    """Views of the summaries and choice that lod_video_attend left in `ws`."""
    L = video_layout(cfg, batch)
    nb, d = L.n_blocks, cfg.head_dim

    def view(off, n, dt):
        es = torch.tensor([], dtype=dt).element_size()
        return ws[off:off + n * es].view(dt)
    return {
        "kbar": view(L.kbar, batch * cfg.n_kv_heads * nb * d, torch.bfloat16).view(batch, cfg.n_kv_heads, nb, d),
        "vbar": view(L.vbar, batch * cfg.n_kv_heads * nb * d, torch.bfloat16).view(batch, cfg.n_kv_heads, nb, d),
        "lnn": view(L.lnn, nb, torch.float32),
        "qbar": view(L.qbar, batch * cfg.n_q_heads * nb * d, torch.float32).view(batch, cfg.n_q_heads, nb, d),
        "sel": view(L.sel, batch * cfg.n_q_heads * nb * cfg.top_blocks, torch.int32).view(
            batch, cfg.n_q_heads, nb, cfg.top_blocks),
    }


def _video_shapes(cfg: VideoConfig, K, V, q):
    B, T = q.shape[0], cfg.n_tokens
    assert q.is_contiguous() and tuple(q.shape) == (B, T, cfg.n_q_heads, cfg.head_dim)
    assert K.shape[0] == B and tuple(K.shape[1:]) == (T, cfg.n_kv_heads, cfg.head_dim)
    assert q.dtype == K.dtype == V.dtype
    return B


def attend_video(cfg: VideoConfig, K, V, q, want_selection: bool = False, ws: torch.Tensor | None = None,
                 out: torch.Tensor | None = None):
    """Video LoD attention.  q [B][T][Hq][d], K, V [B][T][Hkv][d] (bf16, T = frames*height*
    width in raster order).  Returns (out [B][T][Hq][d] fp32, sel [B][Hq][NB][c] or None)."""
    B = _video_shapes(cfg, K, V, q)
    if out is None:
        out = torch.empty(B, cfg.n_tokens, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(video_ws_bytes(cfg, B), dtype=torch.uint8, device=q.device)
    sel = None
    if want_selection:
        nb = video_layout(cfg, B).n_blocks
        sel = torch.empty(B, cfg.n_q_heads, nb, cfg.top_blocks, dtype=torch.int32, device=q.device)
    _check("lod_video_attend", lib().lod_video_attend(
        ctypes.byref(cfg.params()), kv_view(K, V), _ptr(q), B, _ptr(out), _ptr(sel), _ptr(ws), ws.numel(),
        _stream()))
    return out, sel


def dense_video(cfg: VideoConfig, K, V, q, out: torch.Tensor | None = None):
    """Dense bidirectional attention over the whole grid (the baseline), same layout."""
    B = _video_shapes(cfg, K, V, q)
    if out is None:
        out = torch.empty(B, cfg.n_tokens, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
    _check("lod_video_dense", lib().lod_video_dense(
        ctypes.byref(cfg.params()), kv_view(K, V), _ptr(q), B, _ptr(out), _stream()))
    return out
