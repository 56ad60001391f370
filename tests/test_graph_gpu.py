"""The entry points under HIP graph capture: the library enqueues kernels only, all on the
caller's stream (no memsets, copies, allocations, host syncs or streams of its own).  Each
graph is replayed three times with the program's own eager work and synchronizations
between the replays, and every replay must give bit for bit what the eager call gave:
no kernel's result depends on the order in which its workgroups run or take list slots."""
import pytest
import torch

from hierarchical_kv_approximation_amd import lod, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, outs, refs):
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        junk = torch.randn(1 << 20, device="cuda") * rep  # the program's own eager work
        junk.sum().item()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {rep} differs from the eager call"


def test_decode_and_prefill_graph_replays_equal_eager():
    dev = torch.device("cuda")
    B, T = 2, 8192
    cfg = lod.Config(n_q_heads=16, n_kv_heads=2, groups=8, top_groups=8, top_pages=2, window=512, n_sink=4)
    K, V, cen, _ = synth.clustered_kv(B, T, 2, 128, seed=71, device=dev)
    index = lod.LodIndex.allocate(cfg, B, T, device=dev)
    lod.build_chunk(cfg, index, K, V, 0, T // 256 - 1)
    torch.cuda.synchronize()
    # decode
    q = synth.queries(B, 16, cen, seed=72)
    seq = torch.tensor([T, 5000], dtype=torch.int32, device=dev)
    ws = torch.empty(lod.decode_ws_bytes(cfg, B, T), dtype=torch.uint8, device=dev)
    out = torch.empty(B, 16, 128, dtype=torch.float32, device=dev)
    ref = lod.attend_decode(cfg, index, K, V, q, seq, T, ws=ws, out=out).clone()
    g = _capture(lambda: lod.attend_decode(cfg, index, K, V, q, seq, T, ws=ws, out=out))
    _replays_match(g, [out], [ref])
    # bf16 prefill of two 2048-row batches
    nq, q0 = 4096, 4096
    qp = synth.queries(B, 16, cen, seed=73, n_rows=nq)
    wsp = torch.empty(lod.prefill_ws_bytes(cfg, B, nq, q0 + nq), dtype=torch.uint8, device=dev)
    outp = torch.empty(B, nq, 16, 128, dtype=torch.float32, device=dev)
    refp = lod.attend_prefill(cfg, index, K, V, qp, q0, ws=wsp, out=outp).clone()
    gp = _capture(lambda: lod.attend_prefill(cfg, index, K, V, qp, q0, ws=wsp, out=outp))
    _replays_match(gp, [outp], [refp])


def test_video_graph_replays_equal_eager():
    dev = torch.device("cuda")
    cfg = lod.VideoConfig(frames=8, height=32, width=36, n_q_heads=4, n_kv_heads=2, top_blocks=16)
    Q, K, V = synth.video_qkv(1, 8, 32, 36, 4, 2, seed=74, device=dev)
    ws = torch.empty(lod.video_ws_bytes(cfg, 1), dtype=torch.uint8, device=dev)
    out = torch.empty(1, cfg.n_tokens, 4, 128, dtype=torch.float32, device=dev)
    nb = lod.video_layout(cfg, 1).n_blocks
    sel = torch.empty(1, 4, nb, 16, dtype=torch.int32, device=dev)

    def call():
        rc = lod.lib().lod_video_attend(cfg.params(), lod.kv_view(K, V), lod._ptr(Q), 1, lod._ptr(out),
                                        lod._ptr(sel), lod._ptr(ws), ws.numel(), lod._stream())
        assert rc == lod.LOD_OK
    call()
    torch.cuda.synchronize()
    ref, refs = out.clone(), sel.clone()
    g = _capture(call)
    _replays_match(g, [out, sel], [ref, refs])
