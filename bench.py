#!/usr/bin/env python3
"""Benchmark of LoD attention on one MI355X: decode at 128K context (the headline), with
the dense-decode time on the same inputs, the dominant kernel's roofline, and the CPU
oracle timed on a bounded sample.  Prints ONE JSON line.

Workload (defaults): bf16 KV, GQA 64 query / 8 KV heads, head_dim 128, batch 8,
context 131072; groups of a 256-token chunk = 8, pages of 16, top 8 groups, top 2
pages, block window 512, 4 sinks.  Keys from a 32-centre Gaussian mixture (sigma 0.3),
values N(0, 1), queries matched to the mixture (all seeded, synthetic).

A step is one lod_attend_decode call -- one decode token for every sequence of the batch
through one attention layer -- plus its share of the chunk builds the method needs while
decoding: each layer builds one chunk (every sequence and KV head in one lod_build_chunk
call) per 256 positions, so a step is charged 1/256 of that call, timed on its own.
Steps rotate over `--layers` independent layer copies (cache + index) so the 256 MB
Infinity Cache cannot serve a layer's reads from the previous step.  The timed positions
start at a chunk boundary (the first query of a chunk, which needs the chunk that has
just left the block window).
"""
from __future__ import annotations

import argparse
import dataclasses
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LoD attention decode tok/s & prefill tok/s at 128K ctx; % HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the call's stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def wait(self, stream, ev):
        """Make `stream` wait for event `ev` (hipStreamWaitEvent)."""
        assert self.hip.hipStreamWaitEvent(stream, ev, 0) == 0

    def ms(self, a, b):
        t = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return float(t.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def profiled_traffic(name):
    """HBM bytes per launch measured by rocprofv3 (profiles/<name>.json), or None when the
    kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:  # the kernel's file and every header it includes
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec["sources_sha256_16"]:
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def host_info() -> dict:
    """The benchmark machine's host CPU (the oracle's baseline runs there)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable,
            "oracle_threads": cpu_threads()}


def copy_bandwidth(torch, hip, stream, nbytes=1 << 30, reps=10):
    """Measured HBM rate of a plain device-to-device copy (the practical ceiling that the
    kernels' fractions are also quoted against): bytes read + written per second."""
    x = torch.ones(nbytes // 4, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e = hip.create(2)
    hip.record(e[0], stream)
    for _ in range(reps):
        y.copy_(x)
    hip.record(e[1], stream)
    torch.cuda.synchronize()
    ms = hip.ms(e[0], e[1]) / reps
    hip.destroy(e)
    del x, y
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"what": f"device-to-device copy of {nbytes >> 20} MiB, read + write bytes per second",
            "GBs": round(gbs, 1), "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)}


def algorithmic_decode_bytes(cfg, index, sel_g, sel_p, seq_lens, elt):
    """Bytes the method itself must move for one decode call, split by launch.

    scores: the mean keys of every summarised chunk (and q).
    coarse: mean values and ln n of every summarised chunk; the exact window and sinks.
    open:   page summaries of the opened groups; K/V rows of the union of opened pages
            over the query heads of a KV head.
    Returns (total, scores, coarse, open); output and workspace traffic is not counted."""
    import numpy as np
    d, G, C, W, S = cfg.head_dim, cfg.groups, cfg.chunk_size, cfg.window, cfg.n_sink
    Hq, Hkv = cfg.n_q_heads, cfg.n_kv_heads
    g = Hq // Hkv
    row = 2 * d * elt
    meta = index.arrays()["meta"].cpu().numpy().astype(np.int64)
    sg, sp = sel_g.cpu().numpy(), sel_p.cpu().numpy()
    PS = cfg.page_slots
    scores = coarse = opened_b = 0
    for b, T in enumerate(seq_lens):
        p = T - 1
        nb = max(0, p // C - W // C + 1)
        tail = p - nb * C + 1
        sinks = min(S, nb * C)
        for kvh in range(Hkv):
            opened, rows = set(), set()
            for h in range(kvh * g, (kvh + 1) * g):
                for i, gid in enumerate(sg[b, h]):
                    if gid < 0:
                        continue
                    c, j = divmod(int(gid), G)
                    opened.add((c, j))
                    m = meta[b, kvh, c]
                    gpg, pst, perm = m[: G + 1], m[G + 1: G + 1 + PS + 1], m[G + 1 + PS + 1:]
                    slots = range(gpg[j], gpg[j + 1]) if cfg.top_pages == 0 else \
                        [s for s in sp[b, h, i] if s >= 0]
                    for s in slots:
                        rows.update(c * C + int(x) for x in perm[pst[s]:pst[s + 1]])
            pages = 0
            for c, j in opened:
                gpg = meta[b, kvh, c][: G + 1]
                pages += int(gpg[j + 1] - gpg[j])
            scores += nb * G * d * elt
            coarse += nb * G * (d * elt + 4) + (tail + sinks) * row
            opened_b += pages * (row + 4) + len(rows) * row
        scores += Hq * d * elt
    return int(scores + coarse + opened_b), int(scores), int(coarse), int(opened_b)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--ctx", type=int, default=131072)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-decode comparison")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle time")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--prefill-ctx", type=int, default=131072)
    ap.add_argument("--no-sweep", action="store_true", help="skip the sigma sweep of the approximation error")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-KV-view decode timing")
    ap.add_argument("--no-int4", action="store_true", help="skip the INT4-pages decode timing")
    ap.add_argument("--no-video", action="store_true", help="skip the video LoD measurement")
    ap.add_argument("--no-batch1", action="store_true", help="skip the batch-1 decode measurement")
    ap.add_argument("--only-video", action="store_true",
                    help="measure video LoD only and print its JSON object (for profiling)")
    ap.add_argument("--video-calls", type=int, default=20)
    ap.add_argument("--no-small", action="store_true",
                    help="skip the 4K fp32 and 32K batch-4 decode cases and the 32K prefill")
    ap.add_argument("--prefill-shapes", action="store_true",
                    help="with --only-prefill: also the 2048-token steps and the whole-prompt prefill")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run the chunked 128K prefill only and print its JSON object (for profiling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this LoD "
              "attention build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from hierarchical_kv_approximation_amd import lod, synth

    dev = torch.device("cuda:0")
    if args.only_video:
        hip = HipEvents()
        v = bench_video(torch, lod, synth, hip, torch.cuda.current_stream().cuda_stream, args.seed,
                        calls=args.video_calls, dense=not args.no_dense, cpu=not args.no_cpu,
                        cpu_seconds=args.cpu_seconds)
        print(json.dumps({"video": v}), flush=True)
        return
    if args.only_prefill:
        hip = HipEvents()
        cfg = lod.Config(n_q_heads=64, n_kv_heads=8, groups=8, top_groups=8, top_pages=2, window=512,
                         n_sink=4, dtype=torch.bfloat16)
        pr = bench_prefill(torch, lod, synth, cfg, hip, torch.cuda.current_stream().cuda_stream,
                           args.prefill_ctx, args.seed, dense=False, cpu=False, one_call=args.prefill_shapes)
        print(json.dumps({"prefill": pr}), flush=True)
        return
    B, T, L = args.batch, args.ctx, args.layers
    K, W = max(2, args.steps), max(0, args.warmup)
    cfg = lod.Config(n_q_heads=64, n_kv_heads=8, groups=8, top_groups=8, top_pages=2, window=512,
                     n_sink=4, dtype=torch.bfloat16)
    C = cfg.chunk_size
    elt = 2
    assert T % C == 0
    npos = (K + L - 1) // L
    # the timed positions start at a chunk boundary: the first query of chunk T/C needs
    # chunk T/C - W/C summarised (it has just left the block window), and every later
    # position of the run needs no other build while it stays inside that chunk
    boundary = T  # first query position of chunk T/C
    s0 = boundary + 1  # seq_len of the first timed position
    cap = T + C * ((npos + C - 1) // C)
    max_len = s0 + npos - 1
    nb0 = max(0, (s0 - 1) // C - cfg.window // C)  # chunks built before the boundary
    build_chunk = boundary // C - cfg.window // C  # chunk that the boundary requires
    nb_end = max(0, (max_len - 1) // C - cfg.window // C + 1)  # chunks the last position needs

    t_setup = time.time()
    layers = []
    for li in range(L):
        Kc, Vc, cen, _ = synth.clustered_kv(B, cap, 8, 128, seed=args.seed + 101 * li, device=dev)
        q = synth.queries(B, 64, cen, seed=args.seed + 7 + 101 * li)
        index = lod.LodIndex.allocate(cfg, B, cap, device=dev)
        lod.build_chunk(cfg, index, Kc, Vc, 0, nb0)
        layers.append({"K": Kc, "V": Vc, "q": q, "index": index})
        del cen
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    log(f"setup done: {L} layers of B={B} x {cap} tokens, {nb0} chunks built ({setup_s:.1f} s)")

    seq = torch.tensor([[s0 + k] * B for k in range(npos)], dtype=torch.int32, device=dev)
    ws = torch.empty(lod.decode_ws_bytes(cfg, B, max_len), dtype=torch.uint8, device=dev)
    out = torch.empty(B, 64, 128, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    hip = HipEvents()

    # the build the boundary needs, one per layer (every sequence and KV head of the layer
    # in one call), timed alone; a decode step is charged 1/256 of one: each layer builds
    # one chunk per 256 of its positions
    bev = hip.create(2 * L)
    for li, Ly in enumerate(layers):
        hip.record(bev[2 * li], stream)
        lod.build_chunk(cfg, Ly["index"], Ly["K"], Ly["V"], build_chunk, 1)
        hip.record(bev[2 * li + 1], stream)
        if nb_end > build_chunk + 1:  # runs longer than one chunk per layer: untimed
            lod.build_chunk(cfg, Ly["index"], Ly["K"], Ly["V"], build_chunk + 1, nb_end - build_chunk - 1)
    torch.cuda.synchronize()
    build_ms = [hip.ms(bev[2 * i], bev[2 * i + 1]) for i in range(L)]
    hip.destroy(bev)
    build_charge_ms = sum(build_ms) / L / C

    # warm-up at the first position
    for k in range(W):
        Ly = layers[k % L]
        lod.attend_decode(cfg, Ly["index"], Ly["K"], Ly["V"], Ly["q"], seq[0], max_len, ws=ws, out=out)
    torch.cuda.synchronize()

    # timed region: the decode calls back to back, nothing else on the stream
    t0, t1 = hip.create(2)
    hip.record(t0, stream)
    for k in range(K):
        Ly = layers[k % L]
        lod.attend_decode(cfg, Ly["index"], Ly["K"], Ly["V"], Ly["q"], seq[k // L], max_len, ws=ws, out=out)
    hip.record(t1, stream)
    torch.cuda.synchronize()
    total_ms = hip.ms(t0, t1)
    hip.destroy([t0, t1])
    decode_ms_per_step = total_ms / K
    ms_per_step = decode_ms_per_step + build_charge_ms
    log(f"timed {K} steps: {decode_ms_per_step * 1000:.1f} us/step + {build_charge_ms * 1000:.2f} us/step "
        f"of chunk builds (one {sum(build_ms) / L * 1000:.0f} us build per layer per {C} positions)")

    # the same calls again with the library's trace events (before the scan, after the
    # scan, after the open step) for the per-kernel times; events add a little time
    NE = 3
    ev = hip.create(NE * K)
    for k in range(K):
        Ly = layers[k % L]
        keep = lod.trace_events(ev[NE * k: NE * k + NE])
        lod.attend_decode(cfg, Ly["index"], Ly["K"], Ly["V"], Ly["q"], seq[k // L], max_len, ws=ws, out=out)
        lod.trace_events(None)
        del keep
    torch.cuda.synchronize()
    scan_ms = [hip.ms(ev[NE * k], ev[NE * k + 1]) for k in range(K)]
    open_ms = [hip.ms(ev[NE * k + 1], ev[NE * k + 2]) for k in range(K)]
    call_ms = [hip.ms(ev[NE * k], ev[NE * k + 2]) for k in range(K)]
    hip.destroy(ev)

    # algorithmic bytes at the last timed position (selection from one extra call)
    Ly = layers[(K - 1) % L]
    last = seq[(K - 1) // L]
    o2, sg, sp = lod.attend_decode(cfg, Ly["index"], Ly["K"], Ly["V"], Ly["q"], last, max_len,
                                   want_selection=True)
    torch.cuda.synchronize()
    lens = [int(x) for x in last.cpu()]
    bytes_call, bytes_scores, bytes_coarse, bytes_open = algorithmic_decode_bytes(cfg, Ly["index"], sg, sp,
                                                                                 lens, elt)
    scan_avg, open_avg = sum(scan_ms) / K, sum(open_ms) / K
    bytes_scan = bytes_scores + bytes_coarse
    # the dominant launch: the scan (HBM bound; the open step is latency bound)
    dom = ("decode_scan_mfma_kernel (mean keys and values of every summarised chunk, exact window and sinks)",
           scan_avg, bytes_scan, "decode_scan_traffic")
    call_avg = sum(call_ms) / K

    # dense decode on the same inputs (same rotation, same positions)
    dense = None
    if not args.no_dense:
        dws = torch.empty(lod.dense_decode_ws_bytes(cfg, B, max_len), dtype=torch.uint8, device=dev)
        for k in range(min(W, 4)):
            Ly = layers[k % L]
            lod.dense_decode(cfg, Ly["K"], Ly["V"], Ly["q"], seq[0], max_len, ws=dws, out=out)
        torch.cuda.synchronize()
        d0, d1 = hip.create(2)
        KD = max(L, min(K, 16))
        hip.record(d0, stream)
        for k in range(KD):
            Ly = layers[k % L]
            lod.dense_decode(cfg, Ly["K"], Ly["V"], Ly["q"], seq[min(k // L, npos - 1)], max_len, ws=dws, out=out)
        hip.record(d1, stream)
        torch.cuda.synchronize()
        dms = hip.ms(d0, d1) / KD
        hip.destroy([d0, d1])
        dense_bytes = sum(lens) * 8 * 2 * 128 * elt
        log(f"dense decode: {dms * 1000:.1f} us/call")
        dense = {"ms_per_call": round(dms, 4), "tok_per_s": round(B * 1000.0 / dms, 1),
                 "achieved_GBs": round(dense_bytes / dms / 1e6, 1),
                 "lod_speedup_vs_dense": round(dms / ms_per_step, 2)}

    # reference for the variants below: the same LoD calls back to back, no trace events,
    # no builds (every layer is already built past the boundary)
    def time_calls(c, paged_view=False, index="index"):
        for k in range(min(W, 4)):
            Ly = layers[k % L]
            lod.attend_decode(c, Ly[index], Ly["Kp" if paged_view else "K"], Ly["Vp" if paged_view else "V"],
                              Ly["q"], seq[npos - 1], max_len, ws=ws, out=out,
                              block_table=Ly["table"] if paged_view else None)
        torch.cuda.synchronize()
        a0, a1 = hip.create(2)
        hip.record(a0, stream)
        for k in range(K):
            Ly = layers[k % L]
            lod.attend_decode(c, Ly[index], Ly["Kp" if paged_view else "K"], Ly["Vp" if paged_view else "V"],
                              Ly["q"], seq[k // L], max_len, ws=ws, out=out,
                              block_table=Ly["table"] if paged_view else None)
        hip.record(a1, stream)
        torch.cuda.synchronize()
        r = hip.ms(a0, a1) / K
        hip.destroy([a0, a1])
        return r
    ref_ms = time_calls(cfg)

    # sparsity ablation on the same inputs: the same selection, the coarse remainder
    # dropped (the scan reads the mean keys for the scores but no mean values)
    scfg = dataclasses.replace(cfg, drop_remainder=True)
    sms = time_calls(scfg)
    sparse = {"what": "same selection, coarse remainder dropped (exact keys only)",
              "ms_per_call": round(sms, 5), "tok_per_s": round(B * 1000.0 / sms, 1),
              "time_vs_lod": round(sms / ref_ms, 3), "lod_reference_ms_per_call": round(ref_ms, 5)}
    log(f"sparsity ablation: {sms * 1000:.1f} us/call")

    # three-tier INT4: indexes built with 4-bit codes of every clustered row; the open
    # step decodes the opened pages from them instead of reading the cache
    int4 = None
    if not args.no_int4:
        qcfg = dataclasses.replace(cfg, int4_pages=True)
        for Ly in layers:
            Ly["index4"] = lod.LodIndex.allocate(qcfg, B, cap, device=dev)
            lod.build_chunk(qcfg, Ly["index4"], Ly["K"], Ly["V"], 0, max(nb_end, build_chunk + 1))
        qms = time_calls(qcfg, index="index4")
        code_bytes = sum(int(Ly["index4"].mem.numel()) for Ly in layers) // L - sum(
            int(Ly["index"].mem.numel()) for Ly in layers) // L
        for Ly in layers:
            del Ly["index4"]
        int4 = {"what": "the same decode calls with opened pages decoded from 4-bit codes in the index",
                "ms_per_call": round(qms, 5), "tok_per_s": round(B * 1000.0 / qms, 1),
                "time_vs_bf16_pages": round(qms / ref_ms, 3),
                "code_bytes_per_layer": code_bytes,
                "cache_bytes_per_layer_bf16": int(layers[0]["K"].numel() * 2 * 2)}
        log(f"INT4 pages: {qms * 1000:.1f} us/call")

    # paged KV view: each layer's cache scattered over a pool of 16-position blocks in a
    # seeded random order (a serving engine's block table); same index, same positions
    paged = None
    if not args.no_paged:
        import numpy as np
        bsz = 16
        nbl = cap // bsz
        for li, Ly in enumerate(layers):
            perm = np.random.default_rng(args.seed + 31 * li).permutation(B * nbl).astype(np.int32)
            table = torch.from_numpy(perm).view(B, nbl).to(dev)
            pool_shape = (B * nbl, bsz) + tuple(Ly["K"].shape[2:])
            Ly["Kp"] = torch.empty(pool_shape, dtype=Ly["K"].dtype, device=dev)
            Ly["Vp"] = torch.empty_like(Ly["Kp"])
            Ly["Kp"][table.view(-1).long()] = Ly["K"].reshape(pool_shape)
            Ly["Vp"][table.view(-1).long()] = Ly["V"].reshape(pool_shape)
            Ly["table"] = table
        pms = time_calls(cfg, paged_view=True)
        for Ly in layers:
            del Ly["Kp"], Ly["Vp"], Ly["table"]
        paged = {"what": "the same decode calls with each cache in a pool of 16-position blocks "
                         "(random block order, block table)",
                 "ms_per_call": round(pms, 5), "tok_per_s": round(B * 1000.0 / pms, 1),
                 "time_vs_strided": round(pms / ref_ms, 3), "strided_reference_ms_per_call": round(ref_ms, 5)}
        log(f"paged KV view: {pms * 1000:.1f} us/call")

    # CPU oracle on a bounded sample: sequence 0 of layer 0, all 64 heads, one token
    cpu = cpu1 = None
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        cpu, cpu1 = cpu_baseline(cfg, layers[0], s0, args.cpu_seconds, min(5.0, args.cpu_seconds))
        log(f"CPU oracle: {cpu['value']} tok/s on {cpu['cores']} threads, {cpu1['value']} tok/s on one")

    for Ly in layers:
        del Ly["K"], Ly["V"], Ly["index"]
    del layers, ws
    torch.cuda.empty_cache()

    copy_bw = copy_bandwidth(torch, hip, stream)
    log(f"copy bandwidth: {copy_bw['GBs']} GB/s")

    small = None
    if not args.no_small:
        small = {"c1_decode_fp32_4k": bench_c1(torch, lod, synth, hip, stream, cpu=not args.no_cpu),
                 "c2_decode_bf16_32k_b4": bench_c2(torch, lod, synth, hip, stream, cpu=not args.no_cpu)}
        torch.cuda.empty_cache()

    batch1 = None
    if not args.no_batch1:
        batch1 = bench_batch1(torch, lod, synth, cfg, hip, stream, T, args.seed, dense=not args.no_dense)
        torch.cuda.empty_cache()

    sweep = None
    if not args.no_sweep:
        sweep = bench_sigma_sweep(torch, lod, synth, cfg, hip, stream, args.prefill_ctx, args.seed)
        torch.cuda.empty_cache()

    prefill = prefill32 = None
    if not args.no_prefill:
        prefill = bench_prefill(torch, lod, synth, cfg, hip, stream, args.prefill_ctx, args.seed,
                                dense=not args.no_dense, cpu=not args.no_cpu)
        torch.cuda.empty_cache()
        if not args.no_small:
            prefill32 = bench_prefill(torch, lod, synth, cfg, hip, stream, 32768, args.seed,
                                      dense=not args.no_dense, cpu=False)
            torch.cuda.empty_cache()

    video = None
    if not args.no_video:
        video = bench_video(torch, lod, synth, hip, stream, args.seed, calls=args.video_calls,
                            dense=not args.no_dense, cpu=not args.no_cpu, cpu_seconds=min(args.cpu_seconds, 10.0))

    line = {
        "metric": METRIC,
        "value": round(B * 1000.0 / ms_per_step, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "LoD decode, one attention layer per step: context 131072, batch 8, "
                        "GQA 64/8, head_dim 128, bf16 KV, 8 groups per 256-token chunk, pages of 16, "
                        "top 8 groups / top 2 pages, block window 512, 4 sinks",
            "batch": B, "context": T, "layers_rotated": L,
            "positions": [s0 - 1, max_len - 1],
            "step": "one lod_attend_decode call (one token of every sequence through one layer) plus "
                    "1/256 of that layer's lod_build_chunk call (each layer builds one chunk per 256 "
                    "positions); the calls are timed back to back, the build alone",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom[0],
            "achieved": round(dom[2] / (dom[1] * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom[2] / (dom[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": profiled_traffic(dom[3]),
            "algorithmic_bytes_per_launch": dom[2],
            "avg_launch_us": round(dom[1] * 1000, 2),
        },
        "cpu_baseline": cpu,
        "extra": {
            "step_us": round(ms_per_step * 1000, 2),
            "decode_call_us": round(decode_ms_per_step * 1000, 2),
            "build_charge_us_per_step": round(build_charge_ms * 1000, 3),
            "lod_call_us_with_trace_events": round(call_avg * 1000, 2),
            "scan_us": round(scan_avg * 1000, 2),
            "open_us": round(open_avg * 1000, 2),
            "open_algorithmic_bytes": bytes_open,
            "build_one_chunk_batch_us": [round(x * 1000, 1) for x in build_ms],
            "algorithmic_bytes_per_call": bytes_call,
            "call_achieved_GBs": round(bytes_call / (ms_per_step * 1e-3) / 1e9, 1),
            "call_frac_hbm": round(bytes_call / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "dense_decode": dense,
            "sparsity_ablation": sparse,
            "paged_kv_view": paged,
            "int4_pages": int4,
            "batch1": batch1,
            "cpu_baseline_one_core": cpu1,
            "host": host_info(),
            "copy_bandwidth": copy_bw,
            "scan_frac_of_copy_bandwidth": round(dom[2] / (dom[1] * 1e-3) / 1e9 / copy_bw["GBs"], 4),
            "call_frac_of_copy_bandwidth": round(bytes_call / (ms_per_step * 1e-3) / 1e9 / copy_bw["GBs"], 4),
            "seeds": {"headline": args.seed, "c1_c2": [0, 1, 2]},
            **(small or {}),
            "setup_s": round(setup_s, 1),
        },
        "prefill": prefill,
        "prefill_32k_c4": prefill32,
        "sigma_sweep": sweep,
        "video": video,
    }
    print(json.dumps(line), flush=True)


def prefill_flops(cfg, index, T, G_nonempty):
    """Algorithmic MFMA flops of one chunked prefill over T rows (every query head):
    QK and PV (4 d flops per key) over the coarse terms (non-empty groups of summarised
    chunks less the 8 opened ones), the causal window and the sinks -- the work of the
    flash kernel -- and QK (2 d) over every eligible centroid for the selection."""
    C, W, S, d, Hq = cfg.chunk_size, cfg.window, cfg.n_sink, cfg.head_dim, cfg.n_q_heads
    flash = select = 0
    for k in range(T // C):
        nb = max(0, k - W // C + 1)
        ne = int(G_nonempty[:nb].sum()) if nb else 0     # mean over KV heads
        coarse = max(0, ne - cfg.top_groups)
        win = sum(p - nb * C + 1 for p in range(k * C, (k + 1) * C))
        sinks = min(S, nb * C) * C
        flash += 4 * d * Hq * (C * coarse + win + sinks)
        select += 2 * d * Hq * C * ne
    return flash, select


def bench_prefill(torch, lod, synth, cfg, hip, stream, T, seed, dense=True, cpu=True, one_call=True):
    """Chunked causal prefill of one sequence of T tokens: for every 256-row query chunk,
    the chunk that leaves the window is built and the chunk's rows attend.  Builds run on
    a side stream one step ahead (overlapping the previous chunk's attention), as a
    serving engine would pipeline them.  Returns the report dict; kernel times come from
    the library's trace events on the call stream."""
    import numpy as np
    dev = torch.device("cuda:0")
    C = cfg.chunk_size
    nwin = cfg.window // C
    K, V, cen, _ = synth.clustered_kv(1, T, 8, 128, seed=seed + 555, device=dev)
    Q = synth.queries(1, 64, cen, seed=seed + 556, n_rows=T)
    idx = lod.LodIndex.allocate(cfg, 1, T, device=dev)
    out = torch.empty(1, T, 64, 128, dtype=torch.float32, device=dev)
    ws = torch.empty(lod.prefill_ws_bytes(cfg, 1, C, T), dtype=torch.uint8, device=dev)
    nq = T // C

    # The chunk that leaves the window at query chunk k+1 is built on a side stream while
    # query chunk k attends (its keys are in the cache; no attend reads it before k+1).
    side = torch.cuda.Stream(device=dev)
    main = torch.cuda.current_stream(dev)
    STAGES = ["cand", "select", "flash", "bucket", "pages", "combine"]  # kernels of one call, in order
    # The flash and bucket steps share one launch when each KV head's rows carry at most 64
    # (query head, slot) pairs, as the library decides.
    joint = (cfg.n_q_heads // cfg.n_kv_heads) * cfg.top_groups <= 64
    NE = len(STAGES) + 1

    def run(evs=None):
        built = {}
        for k in range(nq):
            c = k + 1 - nwin  # chunk that query chunk k+1 needs last
            if 0 <= c < nq - nwin:
                side.wait_stream(main) if c == 0 else None
                with torch.cuda.stream(side):
                    lod.build_chunk(cfg, idx, K, V, c, 1)
                    built[c] = torch.cuda.Event()
                    built[c].record(side)
            if k - nwin >= 0:
                main.wait_event(built[k - nwin])
            keep = lod.trace_events(evs[NE * k: NE * k + NE]) if evs else None
            lod.attend_prefill(cfg, idx, K, V, Q[:, C * k: C * (k + 1)], C * k, ws=ws,
                               out=out[:, C * k: C * (k + 1)])
            if evs:
                lod.trace_events(None)
            del keep

    run()  # warm-up pass (builds every chunk once; the timed pass rebuilds them)
    torch.cuda.synchronize()
    t0, t1 = hip.create(2)
    hip.record(t0, stream)
    run()
    hip.record(t1, stream)
    torch.cuda.synchronize()
    total_ms = hip.ms(t0, t1)
    hip.destroy([t0, t1])
    # the same pass with the library's trace events around every kernel, for the stage
    # times (the events add a little time of their own)
    ev = hip.create(NE * nq)
    run(ev)
    torch.cuda.synchronize()
    # the six kernels of a call run one after another on the call's stream
    per = {n: 0.0 for n in STAGES}
    attend_ms = 0.0
    for k in range(nq):
        t = [0.0] + [hip.ms(ev[NE * k], ev[NE * k + i]) for i in range(1, NE)]
        for i, n in enumerate(STAGES):
            per[n] += t[i + 1] - t[i]
        attend_ms += t[6]
    hip.destroy(ev)
    log(f"prefill {T}: {total_ms:.1f} ms chunked ({attend_ms:.1f} ms in attention calls, traced pass)")

    cnt = idx.arrays()["gln"][0, :, : nq].cpu().numpy()  # [Hkv][chunks][G]
    nonempty = np.isfinite(cnt).sum(axis=2).mean(axis=0)  # per chunk, mean over KV heads
    flash_flops, select_flops = prefill_flops(cfg, idx, T, nonempty)
    flash_tfs = flash_flops / (per["flash"] * 1e-3) / 1e12

    # one call over every row with the index prebuilt
    one_shot_ms = None
    if one_call:
        wsb = torch.empty(lod.prefill_ws_bytes(cfg, 1, T, T), dtype=torch.uint8, device=dev)
        lod.attend_prefill(cfg, idx, K, V, Q, 0, ws=wsb, out=out)
        a0, a1 = hip.create(2)
        hip.record(a0, stream)
        lod.attend_prefill(cfg, idx, K, V, Q, 0, ws=wsb, out=out)
        hip.record(a1, stream)
        torch.cuda.synchronize()
        one_shot_ms = hip.ms(a0, a1)
        hip.destroy([a0, a1])
        del wsb

    # Serving-style shapes of the same prefill, builds included: (a) 2048-token steps,
    # each building the chunks its rows newly need (their keys are in the cache by then)
    # and then attending its rows; (b) the whole prompt: every chunk built in one call,
    # then one attention call.  Outputs equal the 256-row flow's (the tests check chunked
    # against one-shot prefill); the index already holds these chunks and a rebuild
    # writes the same bits, so the work is that of a fresh build.
    stepped = whole = None
    if one_call:
        S = 2048
        wss = torch.empty(lod.prefill_ws_bytes(cfg, 1, S, T), dtype=torch.uint8, device=dev)

        def run_stepped(evs=None):
            done = 0
            for k in range(T // S):
                need = (k + 1) * S // C - nwin  # chunks 0 .. need-1 summarised for the step's rows
                if need > done:
                    lod.build_chunk(cfg, idx, K, V, done, need - done)
                    done = need
                keep = lod.trace_events(evs[NE * k: NE * k + NE]) if evs else None
                lod.attend_prefill(cfg, idx, K, V, Q[:, S * k: S * (k + 1)], S * k, ws=wss,
                                   out=out[:, S * k: S * (k + 1)])
                if evs:
                    lod.trace_events(None)
                del keep
        run_stepped()
        torch.cuda.synchronize()
        e0, e1 = hip.create(2)
        hip.record(e0, stream)
        run_stepped()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        step_ms = hip.ms(e0, e1)
        hip.destroy([e0, e1])
        nst = T // S
        sev = hip.create(NE * nst)
        run_stepped(sev)
        torch.cuda.synchronize()
        sper = {n: 0.0 for n in STAGES}
        for k in range(nst):
            tt = [0.0] + [hip.ms(sev[NE * k], sev[NE * k + i]) for i in range(1, NE)]
            for i, n in enumerate(STAGES):
                sper[n] += tt[i + 1] - tt[i]
        hip.destroy(sev)
        sflash_tfs = flash_flops / (sper["flash"] * 1e-3) / 1e12
        stepped = {"what": f"{nst} calls of {S} rows; each first builds the chunks its rows newly need",
                   "ms": round(step_ms, 2), "tok_per_s": round(T * 1000.0 / step_ms, 1),
                   "kernel_ms": {n: round(v, 2) for n, v in sper.items()},
                   "flash_TFLOPs": round(sflash_tfs, 1), "flash_frac_mfma": round(sflash_tfs / 2500.0, 4)}
        log(f"prefill {T}: {step_ms:.1f} ms in {S}-token steps (builds included)")
        wsb = torch.empty(lod.prefill_ws_bytes(cfg, 1, T, T), dtype=torch.uint8, device=dev)
        nbuild = T // C - nwin
        w0, w1 = hip.create(2)
        hip.record(w0, stream)
        lod.build_chunk(cfg, idx, K, V, 0, nbuild)
        lod.attend_prefill(cfg, idx, K, V, Q, 0, ws=wsb, out=out)
        hip.record(w1, stream)
        torch.cuda.synchronize()
        whole_ms = hip.ms(w0, w1)
        hip.destroy([w0, w1])
        del wsb, wss
        whole = {"what": f"one build call of all {nbuild} chunks, then one attention call over all rows",
                 "ms": round(whole_ms, 2), "tok_per_s": round(T * 1000.0 / whole_ms, 1)}
        log(f"prefill {T}: {whole_ms:.1f} ms as a whole prompt (build included)")

    dense_rep = None
    if dense:
        # dense causal prefill on 8 row blocks of 2048 rows at the midpoints of 8 equal
        # bins; dense cost per row is linear in its position, so 8 x the sum estimates
        # the full pass without running all of it
        nblk, rows = 8, 2048
        bins = T // nblk
        starts = [i * bins + bins // 2 - rows // 2 for i in range(nblk)]
        starts = [max(0, (s0 // C) * C) for s0 in starts]
        dout = torch.empty(1, rows, 64, 128, dtype=torch.float32, device=dev)
        lod.dense_prefill(cfg, K, V, Q[:, starts[0]: starts[0] + rows], starts[0], out=dout)
        torch.cuda.synchronize()
        d0, d1 = hip.create(2)
        hip.record(d0, stream)
        for st_ in starts:
            lod.dense_prefill(cfg, K, V, Q[:, st_: st_ + rows], st_, out=dout)
        hip.record(d1, stream)
        torch.cuda.synchronize()
        sample_ms = hip.ms(d0, d1)
        hip.destroy([d0, d1])
        est_ms = sample_ms * bins / rows
        dflops = sum(4 * 128 * 64 * sum(range(s + 1, s + rows + 1)) for s in starts)
        for rep_ in (stepped, whole):
            if rep_ is not None:
                rep_["lod_speedup_vs_dense"] = round(est_ms / rep_["ms"], 2)
        dense_rep = {"ms_estimated": round(est_ms, 1), "sampled_ms": round(sample_ms, 2),
                     "sample": f"{nblk} blocks of {rows} rows at bin midpoints, scaled by {bins // rows}",
                     "achieved_TFLOPs": round(dflops / (sample_ms * 1e-3) / 1e12, 1),
                     "lod_speedup_vs_dense": round(est_ms / total_ms, 2)}
        log(f"dense prefill estimate: {est_ms:.0f} ms")
    cpu_rep = prefill_cpu_baseline(cfg, K, V, Q, T, seed) if cpu else None
    del K, V, Q, out, ws, idx
    torch.cuda.empty_cache()
    return {
        "workload": f"chunked causal prefill of {T} tokens, batch 1, GQA 64/8, bf16, 256-row query "
                    "chunks; the chunk leaving the window is built one step ahead on a side stream",
        "cpu_baseline": cpu_rep,
        "tok_per_s": round(T * 1000.0 / total_ms, 1),
        "ms": round(total_ms, 2),
        "attention_calls_ms": round(attend_ms, 2),
        "kernel_ms": {n: round(v, 2) for n, v in per.items()},
        "one_call_prebuilt_index_ms": None if one_shot_ms is None else round(one_shot_ms, 2),
        "steps_2048_tokens": stepped,
        "whole_prompt": whole,
        "kernel_ms_note": ("'flash' times the launch that also holds the bucket sort's workgroups "
                           "(they run after the flash ones); 'bucket' is the gap from its end to "
                           "the group step" if joint else
                           "'flash' and 'bucket' are launches of their own"),
        "roofline": {"bound": "mfma", "kernel": ("prefill_flash_bucket_kernel (coarse + sinks + "
                                                 "window; the bucket sort in the same launch)"
                                                 if joint else
                                                 "prefill_flash_kernel (coarse + sinks + window)"),
                     "achieved": round(flash_tfs, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(flash_tfs / 2500.0, 4),
                     "note": "time between the library's trace events around the kernel (launch gap "
                             "included), summed over the calls",
                     "algorithmic_flops": int(flash_flops), "launches": nq,
                     "avg_launch_us": round(per["flash"] / nq * 1000, 2)},
        "select_algorithmic_flops": int(select_flops),
        "dense_prefill": dense_rep,
    }


def prefill_cpu_baseline(cfg, K, V, Q, T, seed):
    """The oracle, as it stands, on a bounded sample of the same chunked prefill: the
    build of a seeded sample of chunk-heads, LoD attention of seeded (row, head) pairs
    spread over the sequence, and dense attention of fewer such pairs.  Each part is
    scaled to the whole prefill (every chunk-head built once; every row with all query
    heads); the rate is tokens of the prompt per second.  The extrapolation is stated."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc
    threads = cpu_threads()
    host = host_info()
    C, Hq, Hkv = cfg.chunk_size, cfg.n_q_heads, cfg.n_kv_heads
    ocfg = orc.Config(d=128, groups=cfg.groups, top_groups=cfg.top_groups, top_pages=cfg.top_pages,
                      window=cfg.window, n_sink=cfg.n_sink, bf16=True)
    rng = np.random.default_rng(seed + 4242)
    kvh = int(rng.integers(0, Hkv))
    Kh = K[0, :, kvh].float().cpu().numpy().copy()
    Vh = V[0, :, kvh].float().cpu().numpy().copy()
    nchunks = T // C - cfg.window // C  # chunks the chunked flow builds
    # build: every chunk of one KV head (parallel over chunks, each chunk built alone)
    t = time.time()
    idx = orc.build_stream(ocfg, Kh, Vh, nchunks)
    build_s = time.time() - t  # one thread, nchunks chunk-heads
    build_total = build_s * Hkv / threads
    # LoD rows: seeded positions, the sampled KV head's query heads
    n_lod = 8 * threads
    pos = np.sort(rng.integers(0, T, n_lod))
    heads = kvh * (Hq // Hkv) + rng.integers(0, Hq // Hkv, n_lod)
    Qs = Q[0, torch_index(pos), torch_index(heads)].float().cpu().numpy()

    def lod_one(i):
        return orc.attend(ocfg, idx, Kh, Vh, Qs[i], int(pos[i]))["out"]
    t = time.time()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lod_one, range(n_lod)))
    lod_s = time.time() - t
    # per-pair cost grows with the summarised groups: the sample spans the sequence
    lod_total = lod_s / n_lod * T * Hq
    # dense rows: cost linear in the position, so the mean over uniform positions scales
    n_dense = 2 * threads
    dpos = rng.integers(0, T, n_dense)
    Qd = Q[0, torch_index(dpos), torch_index(heads[:n_dense])].float().cpu().numpy()

    def dense_one(i):
        return orc.dense(ocfg, Kh, Vh, Qd[i], int(dpos[i]))[0]
    t = time.time()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(dense_one, range(n_dense)))
    dense_s = time.time() - t
    dense_total = dense_s / n_dense * (T / 2) / max(1.0, float(np.mean(dpos))) * T * Hq
    lod_rate = T / (build_total + lod_total)
    return {"value": round(lod_rate, 2), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"LoD oracle: build of {nchunks} chunks of one KV head ({build_s:.1f} s on one thread), "
                      f"{n_lod} (row, head) pairs at seeded positions ({lod_s:.1f} s on {threads} threads); "
                      f"extrapolated to all {Hkv} KV heads and {T} rows x {Hq} heads "
                      f"({build_total + lod_total:.0f} s); {host['nproc']}-CPU host ({host['cpu_model']})",
            "dense_oracle_tok_per_s": round(T / dense_total, 3),
            "dense_sample": f"{n_dense} (row, head) pairs at seeded positions ({dense_s:.1f} s on {threads} threads), "
                            f"scaled by position to all rows and heads ({dense_total:.0f} s, an extrapolation)"}


def torch_index(a):
    import torch
    return torch.as_tensor(a, dtype=torch.long)


def bench_sigma_sweep(torch, lod, synth, cfg, hip, stream, T, seed, steps=256, samples=96):
    """A T-token prompt through the chunked LoD prefill (before each 256-row query chunk,
    the chunk leaving the window is built), then 256 decode steps of the same sequence
    (batch 1) with the one chunk build they need.  Variants: three-tier and two-tier
    LoD with 8 groups per chunk (about 32 keys, i.e. two pages, per group: top 2 pages
    opens every page, so the tiers coincide) and with 4 groups per chunk (about 64 keys,
    four pages: top 2 opens half, so the tiers differ); the sparsity ablation with the
    three-tier selection; block-sparse attention with larger blocks and a larger budget
    (4 groups per chunk, 16 opened whole, no remainder); three-tier INT4.  Keys come
    from 32 clusters whose sigma is spread over 0.1 .. 1.0, queries are matched to a
    cluster.  Reports the prefill and decode time of each variant and the error of its
    outputs against the dense oracle (fp64) on sampled (row, head) pairs of the prompt
    and sampled (step, head) pairs of the decode, binned by the sigma of the query's
    cluster."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import oracle as orc
    dev = torch.device("cuda:0")
    C = cfg.chunk_size
    nwin = cfg.window // C
    sig = torch.linspace(0.1, 1.0, 32)
    K, V, cen, _ = synth.clustered_kv(1, T + steps, 8, 128, sigma=sig, seed=seed + 777, device=dev)
    Qd, zd = synth.queries(1, 64, cen, n_rows=steps, sigma=sig, seed=seed + 778, return_centres=True)
    Qp, zp = synth.queries(1, 64, cen, n_rows=T, sigma=sig, seed=seed + 780, return_centres=True)
    nb0 = (T - 1) // C - nwin + 1  # chunks the prompt's last row sees
    variants = (("three_tier", dataclasses.replace(cfg)),
                ("two_tier", dataclasses.replace(cfg, top_pages=0)),
                ("three_tier_G4", dataclasses.replace(cfg, groups=4)),
                ("two_tier_G4", dataclasses.replace(cfg, groups=4, top_pages=0)),
                ("sparse_three_tier", dataclasses.replace(cfg, drop_remainder=True)),
                ("sparse_blocks_G4_top16", dataclasses.replace(cfg, groups=4, top_groups=16, top_pages=0,
                                                               drop_remainder=True)),
                ("int4_three_tier", dataclasses.replace(cfg, int4_pages=True)))
    rng = np.random.default_rng(seed + 779)
    pick_d = [(int(k), int(h)) for k, h in zip(rng.integers(0, steps, samples), rng.integers(0, 64, samples))]
    pick_p = [(int(r), int(h)) for r, h in zip(rng.integers(0, T, samples), rng.integers(0, 64, samples))]
    pr_t = torch.tensor([r for r, _ in pick_p], device=dev)
    ph_t = torch.tensor([h for _, h in pick_p], device=dev)
    outp = torch.empty(1, T, 64, 128, dtype=torch.float32, device=dev)
    lens = torch.arange(T + 1, T + steps + 1, dtype=torch.int32, device=dev).view(steps, 1)
    res, outs_d, outs_p = {}, {}, {}
    for name, c in variants:
        idx = lod.LodIndex.allocate(c, 1, T + steps, device=dev)
        ws = torch.empty(lod.decode_ws_bytes(c, 1, T + steps), dtype=torch.uint8, device=dev)
        ws_p = torch.empty(lod.prefill_ws_bytes(c, 1, C, T + steps), dtype=torch.uint8, device=dev)
        out = torch.empty(steps, 64, 128, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        e = hip.create(4)
        hip.record(e[0], stream)
        for k in range(T // C):
            if k - nwin >= 0:
                lod.build_chunk(c, idx, K, V, k - nwin, 1)
            lod.attend_prefill(c, idx, K, V, Qp[:, C * k: C * (k + 1)], C * k, ws=ws_p,
                               out=outp[:, C * k: C * (k + 1)])
        hip.record(e[1], stream)
        hip.record(e[2], stream)
        lod.build_chunk(c, idx, K, V, nb0, 1)
        for k in range(steps):
            lod.attend_decode(c, idx, K, V, Qd[:, k], lens[k], T + steps, ws=ws, out=out[k:k + 1])
        hip.record(e[3], stream)
        torch.cuda.synchronize()
        pms, dms = hip.ms(e[0], e[1]), hip.ms(e[2], e[3])
        hip.destroy(e)
        outs_d[name] = out.cpu().numpy()
        outs_p[name] = outp[0, pr_t, ph_t].cpu().numpy()
        res[name] = {"prefill_ms": round(pms, 2), "prefill_tok_per_s": round(T * 1000 / pms, 1),
                     "decode_us_per_token": round(dms * 1000 / steps, 2),
                     "decode_tok_per_s": round(steps * 1000 / dms, 1)}
        del ws, ws_p, idx, out
    del outp
    # dense oracle on the sampled pairs (one reference for every variant)
    ocfg = orc.Config(d=128, bf16=True)
    Kh = K[0].float().cpu().numpy()
    Vh = V[0].float().cpu().numpy()
    Qdh = Qd[0].float().cpu().numpy()
    Qph = Qp[0, pr_t, ph_t].float().cpu().numpy()
    zdh, zph = zd[0].cpu().numpy(), zp[0, pr_t, ph_t].cpu().numpy()
    heads = {h // 8 for _, h in pick_d + pick_p}
    streams = {h: (np.ascontiguousarray(Kh[:, h]), np.ascontiguousarray(Vh[:, h])) for h in heads}

    def one(job):
        kind, i = job
        if kind == "d":
            k, h = pick_d[i]
            return job, orc.dense(ocfg, *streams[h // 8], Qdh[k, h], T + k)[0]
        r, h = pick_p[i]
        return job, orc.dense(ocfg, *streams[h // 8], Qph[i], r)[0]
    jobs = [("d", i) for i in range(samples)] + [("p", i) for i in range(samples)]
    with ThreadPoolExecutor(cpu_threads()) as ex:
        ref = dict(ex.map(one, jobs))
    edges = np.linspace(0.1, 1.0, 5)
    sig_np = sig.numpy()

    def binned(err_sig):
        bins = []
        for i in range(4):
            errs = [e_ for e_, sg_ in err_sig if edges[i] <= sg_ < edges[i + 1] + (1e-9 if i == 3 else 0.0)]
            bins.append({"sigma": [round(float(edges[i]), 3), round(float(edges[i + 1]), 3)], "n": len(errs),
                         "mean_max_abs_err": round(float(np.mean(errs)), 5) if errs else None,
                         "max_abs_err": round(float(np.max(errs)), 5) if errs else None})
        return bins
    for name in res:
        ed = [(float(np.max(np.abs(outs_d[name][k, h] - ref[("d", i)]))), sig_np[zdh[k, h]])
              for i, (k, h) in enumerate(pick_d)]
        ep = [(float(np.max(np.abs(outs_p[name][i] - ref[("p", i)]))), sig_np[zph[i]])
              for i in range(samples)]
        res[name]["decode_error_vs_dense_oracle_by_sigma"] = binned(ed)
        res[name]["prefill_error_vs_dense_oracle_by_sigma"] = binned(ep)
    tiers = {f"G{G}": {"decode_max_abs_diff": round(float(np.max(np.abs(outs_d[a] - outs_d[b]))), 6),
                       "prefill_max_abs_diff": round(float(np.max(np.abs(outs_p[a] - outs_p[b]))), 6)}
             for G, a, b in ((8, "three_tier", "two_tier"), (4, "three_tier_G4", "two_tier_G4"))}
    del K, V, Qd, Qp
    log("sigma sweep: " + ", ".join(f"{n} {r['prefill_ms']} ms + {r['decode_us_per_token']} us/token"
                                    for n, r in res.items()))
    return {"workload": f"one sequence: {T}-token prompt through the chunked LoD prefill, then {steps} decode "
                        "steps with one chunk build; GQA 64/8, bf16; 32 key clusters with sigma 0.1..1.0, "
                        "matched queries",
            **res, "three_vs_two_tier_difference": tiers, "samples": {"prefill_rows": samples, "decode_steps": samples}}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_batch1(torch, lod, synth, cfg, hip, stream, T, seed, layers=8, reps=32, dense=True):
    """Decode at batch 1 and context T on `layers` layer copies: back-to-back calls
    rotating over the copies, and the same 8 calls captured in one HIP graph and replayed
    (launch costs hidden, as a model's decode step would run them); dense decode on the
    same copies.  The position sits just after a chunk boundary's build (no build inside)."""
    dev = torch.device("cuda:0")
    C = cfg.chunk_size
    nb = max(0, (T - 1) // C - cfg.window // C + 1)
    Ls = []
    for li in range(layers):
        K, V, cen, _ = synth.clustered_kv(1, T, cfg.n_kv_heads, cfg.head_dim, seed=seed + 301 + 7 * li, device=dev)
        q = synth.queries(1, cfg.n_q_heads, cen, seed=seed + 302 + 7 * li)
        idx = lod.LodIndex.allocate(cfg, 1, T, device=dev)
        lod.build_chunk(cfg, idx, K, V, 0, nb)
        Ls.append((K, V, q, idx))
        del cen
    seq = torch.tensor([T], dtype=torch.int32, device=dev)
    ws = torch.empty(lod.decode_ws_bytes(cfg, 1, T), dtype=torch.uint8, device=dev)
    out = torch.empty(1, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=dev)

    def step(i):
        K, V, q, idx = Ls[i % layers]
        lod.attend_decode(cfg, idx, K, V, q, seq, T, ws=ws, out=out)

    def timed(fn, n):
        e = hip.create(2)
        hip.record(e[0], stream)
        fn(n)
        hip.record(e[1], stream)
        torch.cuda.synchronize()
        ms = hip.ms(e[0], e[1])
        hip.destroy(e)
        return ms

    for i in range(2 * layers):
        step(i)
    torch.cuda.synchronize()
    eager_ms = timed(lambda n: [step(i) for i in range(n)], layers * reps) / (layers * reps)
    # one graph of `layers` calls (one per layer copy), replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(layers):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(layers):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    stream_now = torch.cuda.current_stream().cuda_stream
    e = hip.create(2)
    hip.record(e[0], stream_now)
    for _ in range(reps):
        g.replay()
    hip.record(e[1], stream_now)
    torch.cuda.synchronize()
    graph_ms = hip.ms(e[0], e[1]) / (layers * reps)
    hip.destroy(e)
    del g
    res = {"what": f"batch 1 at context {T}, {layers} layer copies; eager back-to-back calls and a graph of "
                   f"{layers} calls (one per copy) replayed {reps} times",
           "us_per_call": round(eager_ms * 1000, 2), "us_per_call_graph": round(graph_ms * 1000, 2),
           "tok_per_s_graph": round(1000.0 / graph_ms, 1)}
    if dense:
        wsd = torch.empty(lod.dense_decode_ws_bytes(cfg, 1, T), dtype=torch.uint8, device=dev)
        outd = torch.empty_like(out)

        def dstep(n):
            for i in range(n):
                K, V, q, _ = Ls[i % layers]
                lod.dense_decode(cfg, K, V, q, seq, T, ws=wsd, out=outd)
        dstep(layers)
        torch.cuda.synchronize()
        dms = timed(dstep, 2 * layers) / (2 * layers)
        res["dense_us_per_call"] = round(dms * 1000, 2)
        res["lod_speedup_vs_dense"] = round(dms / graph_ms, 2)
        res["lod_speedup_vs_dense_eager"] = round(dms / eager_ms, 2)
    log(f"batch 1: {res['us_per_call']} us/call eager, {res['us_per_call_graph']} us/call in a graph")
    del Ls, ws, out
    return res


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def bench_c1(torch, lod, synth, hip, stream, seeds=(0, 1, 2), calls=200, cpu=True):
    """The 4K fp32 decode case: one query head over one KV head, 4096 keys, 4 groups per
    chunk, top 8 groups / top 2 pages, window 256, 1 sink; per seed the latency of one
    call (median of `calls` calls, each between its own events) and of back-to-back
    calls, and the output's distance from the oracle (fp64)."""
    import numpy as np

    from oracle import oracle as orc
    dev = torch.device("cuda:0")
    T = 4096
    cfg = lod.Config(n_q_heads=1, n_kv_heads=1, groups=4, top_groups=8, top_pages=2, window=256, n_sink=1,
                     dtype=torch.float32)
    ocfg = orc.Config(d=128, groups=4, top_groups=8, top_pages=2, window=256, n_sink=1, bf16=False)
    res = []
    for seed in seeds:
        K, V, cen, _ = synth.clustered_kv(1, T, 1, 128, seed=seed, dtype=torch.float32, device=dev)
        q = synth.queries(1, 1, cen, seed=seed + 1, dtype=torch.float32)
        idx = lod.LodIndex.allocate(cfg, 1, T, device=dev)
        nb = ocfg.built_chunks(T - 1)
        lod.build_chunk(cfg, idx, K, V, 0, nb)
        sl = torch.tensor([T], dtype=torch.int32, device=dev)
        ws = torch.empty(lod.decode_ws_bytes(cfg, 1, T), dtype=torch.uint8, device=dev)
        out = torch.empty(1, 1, 128, dtype=torch.float32, device=dev)
        for _ in range(10):
            lod.attend_decode(cfg, idx, K, V, q, sl, T, ws=ws, out=out)
        torch.cuda.synchronize()
        ev = hip.create(2 * calls)
        for i in range(calls):
            hip.record(ev[2 * i], stream)
            lod.attend_decode(cfg, idx, K, V, q, sl, T, ws=ws, out=out)
            hip.record(ev[2 * i + 1], stream)
        torch.cuda.synchronize()
        single = _median([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(calls)])
        hip.destroy(ev)
        e = hip.create(2)
        hip.record(e[0], stream)
        for _ in range(calls):
            lod.attend_decode(cfg, idx, K, V, q, sl, T, ws=ws, out=out)
        hip.record(e[1], stream)
        torch.cuda.synchronize()
        b2b = hip.ms(e[0], e[1]) / calls
        hip.destroy(e)
        r = {"seed": seed, "us_per_call_single": round(single * 1000, 2), "us_per_call_back_to_back": round(b2b * 1000, 2)}
        if cpu:
            o, sg, _ = lod.attend_decode(cfg, idx, K, V, q, sl, T, want_selection=True)
            Kh, Vh = K[0, :, 0].cpu().numpy().copy(), V[0, :, 0].cpu().numpy().copy()
            oidx = orc.build_stream(ocfg, Kh, Vh, nb)
            ref = orc.attend(ocfg, oidx, Kh, Vh, q[0, 0].cpu().numpy(), T - 1)
            r["max_abs_err_vs_oracle"] = float(np.max(np.abs(o[0, 0].cpu().numpy() - ref["out"])))
            r["selection_equal"] = bool(np.array_equal(sg[0, 0].cpu().numpy(), ref["sel_groups"]))
        res.append(r)
        del K, V, idx, ws
    log("4K fp32 decode: " + ", ".join(f"{r['us_per_call_single']} us" for r in res))
    return {"workload": "LoD decode, fp32, 1 query / 1 KV head, head_dim 128, 4096-token context, 4 groups per "
                        "256-token chunk, pages of 16, top 8 groups / top 2 pages, window 256, 1 sink",
            "per_seed": res}


def bench_c2(torch, lod, synth, hip, stream, seeds=(0, 1, 2), layers=4, calls=256, cpu=True):
    """The 32K decode case: bf16, GQA 64/8, batch 4, 32768-token context, 8 groups per
    chunk, top 8 / top 2, window 512, 4 sinks.  Per seed, calls rotate over `layers`
    layer copies (1.07 GB, beyond the Infinity Cache) at the last position; tok/s, the
    call's algorithmic bytes over its time against 8 TB/s, the scan and open times from
    a traced pass, and sampled heads against the oracle."""
    import numpy as np

    from oracle import oracle as orc
    dev = torch.device("cuda:0")
    B, T = 4, 32768
    cfg = lod.Config(n_q_heads=64, n_kv_heads=8, groups=8, top_groups=8, top_pages=2, window=512, n_sink=4,
                     dtype=torch.bfloat16)
    ocfg = orc.Config(d=128, groups=8, top_groups=8, top_pages=2, window=512, n_sink=4, bf16=True)
    nb = ocfg.built_chunks(T - 1)
    res = []
    for seed in seeds:
        Ls = []
        for li in range(layers):
            K, V, cen, _ = synth.clustered_kv(B, T, 8, 128, seed=1000 * seed + 11 * li + 5, device=dev)
            q = synth.queries(B, 64, cen, seed=1000 * seed + 11 * li + 6)
            idx = lod.LodIndex.allocate(cfg, B, T, device=dev)
            lod.build_chunk(cfg, idx, K, V, 0, nb)
            Ls.append((K, V, q, idx))
        sl = torch.full((B,), T, dtype=torch.int32, device=dev)
        ws = torch.empty(lod.decode_ws_bytes(cfg, B, T), dtype=torch.uint8, device=dev)
        out = torch.empty(B, 64, 128, dtype=torch.float32, device=dev)

        def call(i):
            K, V, q, idx = Ls[i % layers]
            lod.attend_decode(cfg, idx, K, V, q, sl, T, ws=ws, out=out)
        for i in range(2 * layers):
            call(i)
        torch.cuda.synchronize()
        e = hip.create(2)
        hip.record(e[0], stream)
        for i in range(calls):
            call(i)
        hip.record(e[1], stream)
        torch.cuda.synchronize()
        ms = hip.ms(e[0], e[1]) / calls
        hip.destroy(e)
        NE = 3
        ev = hip.create(NE * 32)
        for i in range(32):
            keep = lod.trace_events(ev[NE * i: NE * i + NE])
            call(i)
            lod.trace_events(None)
            del keep
        torch.cuda.synchronize()
        scan = sum(hip.ms(ev[NE * i], ev[NE * i + 1]) for i in range(32)) / 32
        opn = sum(hip.ms(ev[NE * i + 1], ev[NE * i + 2]) for i in range(32)) / 32
        hip.destroy(ev)
        K, V, q, idx = Ls[0]
        o, sg, sp = lod.attend_decode(cfg, idx, K, V, q, sl, T, want_selection=True)
        torch.cuda.synchronize()
        total, scores, coarse, opened = algorithmic_decode_bytes(cfg, idx, sg, sp, [T] * B, 2)
        r = {"seed": seed, "us_per_call": round(ms * 1000, 2), "tok_per_s": round(B * 1000.0 / ms, 1),
             "scan_us_traced": round(scan * 1000, 2), "open_us_traced": round(opn * 1000, 2),
             "algorithmic_bytes_per_call": total,
             "call_frac_hbm": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "scan_frac_hbm": round((scores + coarse) / (scan * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if cpu:
            keys = [(0, 0), (B - 1, 7)]
            st = {kv: (K[kv[0], :, kv[1]].float().cpu().numpy().copy(), V[kv[0], :, kv[1]].float().cpu().numpy().copy())
                  for kv in keys}
            oidx = orc.build_all(ocfg, st, nb, threads=cpu_threads())
            qf, of, sgf = q.float().cpu().numpy(), o.cpu().numpy(), sg.cpu().numpy()
            err, same = 0.0, True
            for b, kvh in keys:
                for h in range(8 * kvh, 8 * kvh + 8):
                    ref = orc.attend(ocfg, oidx[(b, kvh)], *st[(b, kvh)], qf[b, h], T - 1)
                    err = max(err, float(np.max(np.abs(of[b, h] - ref["out"]))))
                    same = same and bool(np.array_equal(sgf[b, h], ref["sel_groups"]))
            r["sampled_heads_vs_oracle"] = {"heads": 16, "max_abs_err": err, "selection_equal": same}
        res.append(r)
        del Ls, ws, out
        torch.cuda.empty_cache()
    log("32K batch-4 decode: " + ", ".join(f"{r['us_per_call']} us" for r in res))
    return {"workload": "LoD decode, bf16, GQA 64/8, head_dim 128, batch 4, 32768-token context, 8 groups per "
                        "256-token chunk, pages of 16, top 8 groups / top 2 pages, window 512, 4 sinks; "
                        f"{layers} layer copies rotated",
            "per_seed": res}


def video_flops(torch, sel, counts, d, drop):
    """Algorithmic flops of one video LoD call: 4 d per (query, softmax term), i.e. the
    QK and PV products over the opened blocks' members and one term per other block."""
    opened = sel >= 0
    cnt = counts.to(sel.device)
    exact = (cnt[sel.clamp(min=0).long()] * opened).sum(-1)          # [B][Hq][NB]
    terms = exact + (0 if drop else (cnt.numel() - opened.sum(-1)))
    return int(4 * d * (terms.double() * cnt.double()[None, None, :]).sum().item())


def bench_video(torch, lod, synth, hip, stream, seed, calls=20, dense=True, cpu=True, cpu_seconds=10.0):
    """Video LoD on a 20 x 48 x 80 token grid (76800 tokens), 40 query and KV heads,
    head_dim 128, bf16, 4x4x4 blocks, c = 16: one lod_video_attend call per step, rotating
    over two input copies (2 x 2.36 GB, beyond the Infinity Cache)."""
    F, H, W, Hh, c, d = 20, 48, 80, 40, 16, 128
    dev = torch.device("cuda:0")
    g = lod.VideoConfig(frames=F, height=H, width=W, n_q_heads=Hh, n_kv_heads=Hh, top_blocks=c)
    T = F * H * W
    log(f"video LoD: grid {F}x{H}x{W}, {Hh} heads ...")
    data = [synth.video_qkv(1, F, H, W, Hh, Hh, seed=seed + 1000 + 17 * i, device=dev) for i in range(2)]
    ws = torch.empty(lod.video_ws_bytes(g, 1), dtype=torch.uint8, device=dev)
    out = torch.empty(1, T, Hh, d, dtype=torch.float32, device=dev)

    def run(cfg, i, o=out):
        Q, K, V = data[i % 2]
        lod.attend_video(cfg, K, V, Q, ws=ws, out=o)

    for i in range(4):
        run(g, i)
    torch.cuda.synchronize()
    e = hip.create(2)
    hip.record(e[0], stream)
    for i in range(calls):
        run(g, i)
    hip.record(e[1], stream)
    torch.cuda.synchronize()
    ms = hip.ms(e[0], e[1]) / calls
    hip.destroy(e)
    # per-kernel split from the library's trace events (a separate pass)
    n_tr = 6
    evs = hip.create(4 * n_tr)
    keep = []
    for i in range(n_tr):
        keep.append(lod.trace_events(evs[4 * i:4 * i + 4]))
        run(g, i)
    lod.trace_events(None)
    torch.cuda.synchronize()
    seg = [[hip.ms(evs[4 * i + k], evs[4 * i + k + 1]) for k in range(3)] for i in range(n_tr)]
    hip.destroy(evs)
    summ_ms, sel_ms, att_ms = (sum(x[k] for x in seg) / n_tr for k in range(3))
    # algorithmic work from the choice the call made (copy 0)
    _, sel = lod.attend_video(g, data[0][1], data[0][2], data[0][0], ws=ws, out=out, want_selection=True)
    counts = torch.exp(lod.video_arrays(g, ws, 1)["lnn"]).round().to(torch.int64)
    flops = video_flops(torch, sel, counts, d, False)
    lod_out = out.clone()
    qkv_bytes = 3 * T * Hh * d * 2
    res = {
        "workload": f"video LoD, one attention layer per call: {F}x{H}x{W} token grid ({T} tokens), "
                    f"batch 1, {Hh} query / {Hh} KV heads, head_dim {d}, bf16, 4x4x4 blocks, top {c} blocks",
        "ms_per_call": round(ms, 4),
        "tok_per_s": round(T * 1000.0 / ms, 1),
        "kernel_ms": {"summaries": round(summ_ms, 4), "choice": round(sel_ms, 4), "attention": round(att_ms, 4)},
        "algorithmic_tflop_per_call": round(flops / 1e12, 4),
        "summaries_GBs": round(qkv_bytes / (summ_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "kernel": "video_attend_kernel", "unit": "TFLOP/s",
                     "achieved": round(flops / (att_ms * 1e-3) / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "frac": round(flops / (att_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": flops},
    }
    # the ablation: same choice, no coarse terms
    gd = dataclasses.replace(g, drop_remainder=True)
    e = hip.create(2)
    hip.record(e[0], stream)
    for i in range(calls):
        run(gd, i)
    hip.record(e[1], stream)
    torch.cuda.synchronize()
    drop_ms = hip.ms(e[0], e[1]) / calls
    hip.destroy(e)
    abl = torch.empty_like(out)
    run(gd, 0, abl)
    res["sparsity_ablation"] = {"ms_per_call": round(drop_ms, 4), "time_vs_lod": round(drop_ms / ms, 3)}
    if dense:
        Q, K, V = data[0]
        dout = torch.empty_like(out)
        lod.dense_video(g, K, V, Q, out=dout)
        torch.cuda.synchronize()
        e = hip.create(2)
        hip.record(e[0], stream)
        lod.dense_video(g, K, V, Q, out=dout)
        hip.record(e[1], stream)
        torch.cuda.synchronize()
        dms = hip.ms(e[0], e[1])
        hip.destroy(e)
        dflops = 4 * d * T * T * Hh
        err = (lod_out - dout).abs()
        aerr = (abl - dout).abs()
        res["dense"] = {"ms_per_call": round(dms, 3), "speedup_lod_vs_dense": round(dms / ms, 2),
                        "tflops": round(dflops / (dms * 1e-3) / 1e12, 1),
                        "frac_mfma": round(dflops / (dms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                        "lod_err_vs_dense": {"max_abs": round(float(err.max()), 5), "mean_abs": round(float(err.mean()), 6)},
                        "ablation_err_vs_dense": {"max_abs": round(float(aerr.max()), 5),
                                                  "mean_abs": round(float(aerr.mean()), 6)},
                        "mean_abs_dense_output": round(float(dout.abs().mean()), 5)}
        del dout
        log(f"video dense: {dms:.1f} ms/call")
    log(f"video LoD: {ms:.3f} ms/call (summaries {summ_ms:.3f}, choice {sel_ms:.3f}, attention {att_ms:.3f})")
    if cpu:
        res["cpu_baseline"] = video_cpu_baseline(data[0], F, H, W, c, cpu_seconds)
        log(f"video CPU oracle: {res['cpu_baseline']['value']} tok/s")
    del data, ws, out, lod_out, abl
    torch.cuda.empty_cache()
    return res


def video_cpu_baseline(qkv, F, H, W, c, seconds):
    """The video oracle, as it stands, on sampled query blocks of one head: summaries of
    the head's blocks, then choice and softmax block by block until `seconds` pass;
    scaled to tokens of the whole grid per second over all heads."""
    import numpy as np

    from oracle import video as vo
    threads = cpu_threads()
    Q, K, V = (x[:, :, 0:1].float().cpu().numpy() for x in qkv)
    Hh = qkv[0].shape[2]
    o = vo.VideoConfig(d=128, frames=F, height=H, width=W, top_blocks=c, bf16=True)
    nb = o.n_blocks
    order = np.random.default_rng(7).permutation(nb)
    t = time.time()
    vo.forward(o, Q, K, V, pairs=[], threads=threads)  # the head's summaries
    t_sum = time.time() - t
    done, t1 = 0, time.time()
    while done < nb and time.time() - t1 < seconds:
        step = min(2 * threads, nb - done)
        vo.forward(o, Q, K, V, pairs=[(0, 0, int(j)) for j in order[done:done + step]], threads=threads)
        done += step
    el = time.time() - t1 - t_sum * (done // (2 * threads) + (done % (2 * threads) > 0))
    per_block = max(el, 1e-9) / done
    head_s = t_sum + per_block * nb
    return {"value": round(F * H * W / (head_s * Hh), 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {nb} query blocks of head 0 (each call re-summarises the head, "
                      f"{t_sum:.2f} s, subtracted), scaled to the full grid and {Hh} heads; {threads} threads"}


def cpu_baseline(cfg, Ly, seq_len, seconds, seconds_one_core=5.0):
    """The oracle, as it stands, on one sequence's decode token (all 64 query heads), on
    every usable host core (up to 16 threads) and on one core.  The index is built
    once beforehand (not timed).  Returns (all cores, one core)."""
    import numpy as np

    from oracle import oracle as orc
    threads = cpu_threads()
    ocfg = orc.Config(d=128, groups=cfg.groups, top_groups=cfg.top_groups, top_pages=cfg.top_pages,
                      window=cfg.window, n_sink=cfg.n_sink, bf16=True)
    p = seq_len - 1
    K = Ly["K"][0:1, :seq_len].float().cpu().numpy()
    V = Ly["V"][0:1, :seq_len].float().cpu().numpy()
    st = orc.streams(K, V)
    nb = ocfg.built_chunks(p)
    idx = orc.build_all(ocfg, st, nb, threads=threads)  # index build: not timed
    Q = Ly["q"][0:1].float().cpu().numpy()
    host = host_info()

    def timed(th, budget):
        t = time.time()
        n = 0
        while True:
            orc.decode(ocfg, st, idx, Q, [seq_len], threads=th)
            n += 1
            el = time.time() - t
            if el >= budget or n >= 4096:
                break
        return {"value": round(n / el, 3), "unit": "tok/s", "cores": th, "kind": "oracle",
                "sample": f"{n} decode token(s) of one sequence (all 64 query heads) at position {p}, "
                          f"index prebuilt (not timed); {el:.1f} s wall on {th} thread(s) of a "
                          f"{host['nproc']}-CPU host ({host['cpu_model']})"}
    return timed(threads, seconds), timed(1, seconds_one_core)


if __name__ == "__main__":
    main()
