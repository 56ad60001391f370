"""The C ABI on the host: the library loads, exports what include/lod.h declares, sizes
its buffers consistently, and rejects bad arguments before enqueuing anything.  No call
here reaches a kernel launch, so this runs without a GPU."""
import ctypes

import pytest
import torch

from hierarchical_kv_approximation_amd import lod

FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def _p(cfg):
    return ctypes.byref(cfg.params())


def test_library_exports_every_declared_function():
    names = lod.header_functions()
    assert {"lod_build_chunk", "lod_attend_decode", "lod_attend_prefill"} <= set(names)
    L = lod.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = lod.lib()
    for code in (0, -1, -2, -3, -4, 7):
        assert L.lod_status_string(code)


@pytest.mark.parametrize("int4", [False, True])
def test_index_layout_is_aligned_and_disjoint(int4):
    cfg = lod.Config(int4_pages=int4)
    L = lod.Layout()
    assert lod.lib().lod_index_layout(_p(cfg), 4, 128, ctypes.byref(L)) == 0
    U, NC, G, PS, d = 4 * 8, 128, 8, 16 + 8, 128
    sizes = {"gk": U * NC * G * d * 2, "gv": U * NC * G * d * 2, "gln": U * NC * G * 4,
             "gkn": U * NC * G * 4, "gpage": U * NC * G * 4,
             "pk": U * NC * PS * d * 2, "pv": U * NC * PS * d * 2, "pln": U * NC * PS * 4,
             "meta": U * NC * L.meta_stride * 2, "assign": U * NC * 256}
    if int4:
        sizes.update({"q4k": U * NC * 256 * d // 2, "q4v": U * NC * 256 * d // 2,
                      "q4ks": U * NC * 256 * 4, "q4vs": U * NC * 256 * 4})
    spans = sorted((getattr(L, k), getattr(L, k) + v) for k, v in sizes.items())
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert all(getattr(L, k) % 256 == 0 for k in sizes)
    assert spans[-1][1] <= L.total
    assert L.page_slots == PS and L.meta_stride >= (G + 1) + (PS + 1) + 256
    n = ctypes.c_size_t()
    assert lod.lib().lod_index_bytes(_p(cfg), 4, 128 * 256, ctypes.byref(n)) == 0
    assert n.value == L.total


def test_workspace_sizes_grow_with_context():
    cfg = lod.Config()
    a = lod.decode_ws_bytes(cfg, 8, 32768)
    b = lod.decode_ws_bytes(cfg, 8, 131072)
    assert 0 < a <= b
    assert lod.dense_decode_ws_bytes(cfg, 1, 131072) > 0
    assert lod.prefill_ws_bytes(cfg, 1, 256, 32768) > 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, lod.LOD_ERR_UNSUPPORTED),
    ("chunk_size", 128, lod.LOD_ERR_UNSUPPORTED),
    ("page_size", 8, lod.LOD_ERR_UNSUPPORTED),
    ("groups", 17, lod.LOD_ERR_UNSUPPORTED),
    ("groups", 0, lod.LOD_ERR_ARG),
    ("top_groups", 0, lod.LOD_ERR_ARG),
    ("top_pages", -1, lod.LOD_ERR_ARG),
    ("window", 300, lod.LOD_ERR_ARG),
    ("n_sink", 256, lod.LOD_ERR_ARG),
    ("kmeans_iters", 0, lod.LOD_ERR_ARG),
    ("n_q_heads", 12, lod.LOD_ERR_ARG),
    ("n_q_heads", 48, lod.LOD_ERR_UNSUPPORTED),
    ("dtype", torch.float16, lod.LOD_ERR_UNSUPPORTED),
    ("scale", 0.0, lod.LOD_ERR_ARG),
])
def test_bad_params_rejected_by_every_entry_point(field, value, status):
    cfg = lod.Config(**{field: value})
    L = lod.lib()
    idx = lod.Index(FAKE.value, 1 << 40, 1, 512)
    kv = lod.KV(FAKE.value, FAKE.value, 0, 1024, 128)
    n = ctypes.c_size_t()
    assert L.lod_index_bytes(_p(cfg), 1, 4096, ctypes.byref(n)) == status
    assert L.lod_decode_ws_bytes(_p(cfg), 1, 4096, ctypes.byref(n)) == status
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(idx), kv, 1, 0, 1, None, None, None) == status
    assert L.lod_attend_decode(_p(cfg), ctypes.byref(idx), kv, FAKE, FAKE, 1, 4096, FAKE, None, None,
                               FAKE, 1 << 40, None) == status
    assert L.lod_attend_decode_noalloc(_p(cfg), ctypes.byref(idx), kv, FAKE, FAKE, 1, 4096, FAKE, None, None,
                                       None) == status
    assert L.lod_attend_prefill(_p(cfg), ctypes.byref(idx), kv, FAKE, 0, 256, 1, FAKE, None, None,
                                FAKE, 1 << 40, None) == status
    assert L.lod_dense_decode(_p(cfg), kv, FAKE, FAKE, 1, 4096, FAKE, FAKE, 1 << 40, None) == status
    assert L.lod_dense_prefill(_p(cfg), kv, FAKE, 0, 256, 1, FAKE, None) == status


def test_int4_flag_values():
    """int4_pages is 0 or 1, and INT4 pages need bf16 caches."""
    L = lod.lib()
    n = ctypes.c_size_t()
    p = lod.Config().params()
    p.int4_pages = 2
    assert L.lod_index_bytes(ctypes.byref(p), 1, 4096, ctypes.byref(n)) == lod.LOD_ERR_ARG
    p = lod.Config(dtype=torch.float32, int4_pages=True).params()
    assert L.lod_index_bytes(ctypes.byref(p), 1, 4096, ctypes.byref(n)) == lod.LOD_ERR_UNSUPPORTED
    p = lod.Config(int4_pages=True).params()
    assert L.lod_index_bytes(ctypes.byref(p), 1, 4096, ctypes.byref(n)) == lod.LOD_OK


def test_bad_buffers_rejected():
    cfg = lod.Config(n_q_heads=8, n_kv_heads=1)
    L = lod.lib()
    n = ctypes.c_size_t()
    assert L.lod_index_bytes(_p(cfg), 1, 8192, ctypes.byref(n)) == 0
    good = lod.Index(FAKE.value, n.value, 1, 32)
    kv = lod.KV(FAKE.value, FAKE.value, 0, 1024, 128)
    E = lod.LOD_ERR_ARG
    # null index memory, batch mismatch, chunk range beyond capacity
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(lod.Index(None, n.value, 1, 32)), kv, 1, 0, 1, None, None, None) == E
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(good), kv, 2, 0, 1, None, None, None) == E
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(good), kv, 1, 30, 3, None, None, None) == E
    # index buffer smaller than its layout
    small = lod.Index(FAKE.value, n.value - 1, 1, 32)
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(small), kv, 1, 0, 1, None, None, None) == lod.LOD_ERR_WORKSPACE
    # strides that break 16-byte rows, null cache
    bad_kv = lod.KV(FAKE.value, FAKE.value, 0, 1027, 128)
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(good), bad_kv, 1, 0, 1, None, None, None) == E
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(good), lod.KV(None, FAKE.value, 0, 1024, 128), 1, 0, 1, None, None, None) == E
    # decode: contexts that need chunks the index cannot hold; workspace too small / missing
    assert L.lod_attend_decode(_p(cfg), ctypes.byref(good), kv, FAKE, FAKE, 1, 9000 + 512, FAKE,
                               None, None, FAKE, 1 << 40, None) == E
    assert L.lod_attend_decode(_p(cfg), ctypes.byref(good), kv, FAKE, FAKE, 1, 8192, FAKE, None, None,
                               FAKE, 16, None) == lod.LOD_ERR_WORKSPACE
    assert L.lod_attend_decode(_p(cfg), ctypes.byref(good), kv, FAKE, FAKE, 1, 8192, FAKE, None, None,
                               None, 1 << 40, None) == lod.LOD_ERR_WORKSPACE
    assert L.lod_attend_decode(_p(cfg), ctypes.byref(good), kv, FAKE, None, 1, 8192, FAKE, None, None,
                               FAKE, 1 << 40, None) == E
    # the fixed-workspace decode: the same argument checks, then its size limit
    assert L.lod_attend_decode_noalloc(_p(cfg), ctypes.byref(good), kv, FAKE, FAKE, 1, 9000 + 512, FAKE,
                                       None, None, None) == E
    assert L.lod_attend_decode_noalloc(_p(cfg), ctypes.byref(lod.Index(FAKE.value, n.value, 2, 32)), kv, FAKE,
                                       FAKE, 1, 8192, FAKE, None, None, None) == E
    big = lod.Config(n_q_heads=64, n_kv_heads=8)
    nb = ctypes.c_size_t()
    assert L.lod_index_bytes(_p(big), 64, 131072, ctypes.byref(nb)) == 0
    assert lod.decode_ws_bytes(big, 64, 131072) > lod.NOALLOC_WS_BYTES
    assert L.lod_attend_decode_noalloc(_p(big), ctypes.byref(lod.Index(FAKE.value, nb.value, 64, 512)), kv, FAKE,
                                       FAKE, 64, 131072, FAKE, None, None, None) == lod.LOD_ERR_WORKSPACE
    # prefill: q_start not on a chunk boundary
    assert L.lod_attend_prefill(_p(cfg), ctypes.byref(good), kv, FAKE, 100, 256, 1, FAKE, None, None,
                                FAKE, 1 << 40, None) == E
    assert L.lod_dense_decode(_p(cfg), kv, FAKE, FAKE, 1, 8192, FAKE, FAKE, 8, None) == lod.LOD_ERR_WORKSPACE


def test_paged_view_checks():
    """A block-table view needs a power-of-two block size and table rows that cover every
    position the call reads; anything else is rejected before launch."""
    cfg = lod.Config(n_q_heads=8, n_kv_heads=1)
    L = lod.lib()
    n = ctypes.c_size_t()
    assert L.lod_index_bytes(_p(cfg), 1, 8192, ctypes.byref(n)) == 0
    idx = lod.Index(FAKE.value, n.value, 1, 32)
    E = lod.LOD_ERR_ARG

    def paged(bs, maxb):
        return lod.KV(FAKE.value, FAKE.value, bs * 1024, 1024, 128, FAKE.value, bs, maxb)

    for bad in (paged(24, 4096), paged(0, 4096), paged(1 << 17, 1)):
        assert L.lod_build_chunk(_p(cfg), ctypes.byref(idx), bad, 1, 0, 1, None, None, None) == E
    # chunks 0..3 read 1024 positions: 63 blocks of 16 are too few
    assert L.lod_build_chunk(_p(cfg), ctypes.byref(idx), paged(16, 63), 1, 0, 4, None, None, None) == E
    # decode reads positions up to max_seq_len - 1, prefill up to q_start + n_q - 1
    assert L.lod_attend_decode(_p(cfg), ctypes.byref(idx), paged(16, 511), FAKE, FAKE, 1, 8192, FAKE,
                               None, None, FAKE, 1 << 40, None) == E
    assert L.lod_attend_prefill(_p(cfg), ctypes.byref(idx), paged(32, 39), FAKE, 1024, 256, 1, FAKE, None,
                                None, FAKE, 1 << 40, None) == E
    assert L.lod_dense_decode(_p(cfg), paged(16, 100), FAKE, FAKE, 1, 8192, FAKE, FAKE, 1 << 40, None) == E
    assert L.lod_dense_prefill(_p(cfg), paged(64, 3), FAKE, 0, 256, 1, FAKE, None) == E


def test_product_path_refuses_to_run_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(lod, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(lod, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        lod.lib()


def test_misaligned_q_or_out_rejected():
    """Queries and outputs are read and written 16 bytes at a time: both must be 16-byte
    aligned, else every entry point returns LOD_ERR_ARG before enqueuing anything."""
    cfg = lod.Config(n_q_heads=8, n_kv_heads=1)
    L = lod.lib()
    n = ctypes.c_size_t()
    assert L.lod_index_bytes(_p(cfg), 1, 8192, ctypes.byref(n)) == 0
    idx = lod.Index(FAKE.value, n.value, 1, 32)
    kv = lod.KV(FAKE.value, FAKE.value, 0, 1024, 128)
    odd = ctypes.c_void_p(0x10004)
    E = lod.LOD_ERR_ARG
    for qq, oo in ((odd, FAKE), (FAKE, odd)):
        assert L.lod_attend_decode(_p(cfg), ctypes.byref(idx), kv, qq, FAKE, 1, 8192, oo, None, None,
                                   FAKE, 1 << 40, None) == E
        assert L.lod_attend_prefill(_p(cfg), ctypes.byref(idx), kv, qq, 0, 256, 1, oo, None, None,
                                    FAKE, 1 << 40, None) == E
        assert L.lod_dense_decode(_p(cfg), kv, qq, FAKE, 1, 8192, oo, FAKE, 1 << 40, None) == E
        assert L.lod_dense_prefill(_p(cfg), kv, qq, 0, 256, 1, oo, None) == E
