"""The video LoD C ABI on the host: exported, sized consistently, and rejecting bad
arguments before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes

import pytest
import torch

from hierarchical_kv_approximation_amd import lod

FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def _p(cfg):
    return ctypes.byref(cfg.params())


def _kv():
    return lod.KV(FAKE.value, FAKE.value, 0, 8 * 128, 128, None, 0, 0)


def test_video_entry_points_are_exported():
    names = set(lod.header_functions())
    for fn in ("lod_video_layout", "lod_video_ws_bytes", "lod_video_attend", "lod_video_dense"):
        assert fn in names
        assert hasattr(lod.lib(), fn)


@pytest.mark.parametrize("batch", [1, 3])
def test_video_layout_is_aligned_disjoint_and_sized(batch):
    cfg = lod.VideoConfig(frames=21, height=45, width=80, n_q_heads=16, n_kv_heads=4, top_blocks=16)
    L = lod.video_layout(cfg, batch)
    nb = 6 * 12 * 20  # clipped 4x4x4 blocks of a 21 x 45 x 80 grid
    assert L.n_blocks == nb
    d = 128
    arrays = [(L.kbar, batch * 4 * nb * d * 2), (L.vbar, batch * 4 * nb * d * 2), (L.lnn, nb * 4),
              (L.qbar, batch * 16 * nb * d * 4), (L.sel, batch * 16 * nb * 16 * 4)]
    end = 0
    for off, n in arrays:
        assert off % 256 == 0 and off >= end
        end = off + n
    assert L.total >= end
    assert lod.video_ws_bytes(cfg, batch) == L.total


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, lod.LOD_ERR_UNSUPPORTED),
    ("dtype", torch.float32, lod.LOD_ERR_UNSUPPORTED),
    ("dtype", torch.float16, lod.LOD_ERR_ARG),
    ("block", (4, 4, 8), lod.LOD_ERR_UNSUPPORTED),
    ("block", (0, 4, 4), lod.LOD_ERR_ARG),
    ("top_blocks", 0, lod.LOD_ERR_ARG),
    ("top_blocks", 65, lod.LOD_ERR_UNSUPPORTED),
    ("n_q_heads", 12, lod.LOD_ERR_ARG),
    ("frames", 0, lod.LOD_ERR_ARG),
    ("frames", 16000, lod.LOD_ERR_UNSUPPORTED),  # 4000 * 2 * 2 = 16000 blocks > 13312
    ("scale", 0.0, lod.LOD_ERR_ARG),
    ("drop_remainder", 2, lod.LOD_ERR_ARG),
])
def test_bad_video_params_rejected_by_every_entry_point(field, value, status):
    if field == "drop_remainder":
        p = lod.VideoConfig().params()
        p.drop_remainder = value
        pp = ctypes.byref(p)
    else:
        pp = _p(lod.VideoConfig(**{field: value}))
    L = lod.lib()
    n = ctypes.c_size_t()
    lay = lod.VideoLayout()
    assert L.lod_video_layout(pp, 1, ctypes.byref(lay)) == status
    assert L.lod_video_ws_bytes(pp, 1, ctypes.byref(n)) == status
    assert L.lod_video_attend(pp, _kv(), FAKE, 1, FAKE, None, FAKE, 1 << 40, None) == status
    assert L.lod_video_dense(pp, _kv(), FAKE, 1, FAKE, None) == status


def test_bad_video_buffers_rejected():
    cfg = lod.VideoConfig()
    L = lod.lib()
    E = lod.LOD_ERR_ARG
    need = lod.video_ws_bytes(cfg, 1)
    # batch, null q / out / cache, strides that break 16-byte rows, misaligned pointers
    assert L.lod_video_attend(_p(cfg), _kv(), FAKE, 0, FAKE, None, FAKE, need, None) == E
    assert L.lod_video_attend(_p(cfg), _kv(), None, 1, FAKE, None, FAKE, need, None) == E
    assert L.lod_video_attend(_p(cfg), _kv(), FAKE, 1, None, None, FAKE, need, None) == E
    assert L.lod_video_attend(_p(cfg), lod.KV(None, FAKE.value, 0, 1024, 128, None, 0, 0), FAKE, 1, FAKE, None,
                              FAKE, need, None) == E
    assert L.lod_video_attend(_p(cfg), lod.KV(FAKE.value, FAKE.value, 0, 1027, 128, None, 0, 0), FAKE, 1, FAKE,
                              None, FAKE, need, None) == E
    assert L.lod_video_attend(_p(cfg), _kv(), ctypes.c_void_p(0x10008), 1, FAKE, None, FAKE, need, None) == E
    assert L.lod_video_dense(_p(cfg), _kv(), FAKE, 1, ctypes.c_void_p(0x10004), None) == E
    # workspace too small or missing
    assert L.lod_video_attend(_p(cfg), _kv(), FAKE, 1, FAKE, None, FAKE, need - 1, None) == lod.LOD_ERR_WORKSPACE
    assert L.lod_video_attend(_p(cfg), _kv(), FAKE, 1, FAKE, None, None, need, None) == lod.LOD_ERR_WORKSPACE
    # a paged view is not supported for video grids
    paged = lod.KV(FAKE.value, FAKE.value, 0, 1024, 128, FAKE.value, 16, 64)
    assert L.lod_video_attend(_p(cfg), paged, FAKE, 1, FAKE, None, FAKE, need, None) == lod.LOD_ERR_UNSUPPORTED
    assert L.lod_video_dense(_p(cfg), paged, FAKE, 1, FAKE, None) == lod.LOD_ERR_UNSUPPORTED
