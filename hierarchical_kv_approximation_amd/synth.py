"""Seeded synthetic inputs for LoD attention: clustered keys, Gaussian values, queries.

This module holds input generation only -- none of the method's arithmetic -- and
serves both the GPU path and the CPU oracle, which always receive the very same
arrays.  Shapes follow the KV cache layout of the library: K, V are
[B][T][H_kv][d] and decode queries are [B][H_q][d].

Keys: for every (sequence, KV head) there are ``n_centres`` centres drawn from
N(0, I_d); each position picks a centre uniformly and adds sigma_z * N(0, I_d)
noise.  ``sigma`` is a float or a per-centre tensor (a sweep).  Values are N(0, I_d)
independent of the keys.  Queries are "matched" (a centre of the KV head's
mixture plus the same noise, so attention is peaked) or "diffuse" (N(0, I_d)).
The zero-variance variant fills every 256-token chunk with four distinct centres
in four contiguous runs of 64 positions, with centres rounded to bfloat16 so that
means of repeated keys are exact in fp32.
"""
from __future__ import annotations

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def clustered_kv(B: int, T: int, Hkv: int, d: int = 128, *, n_centres: int = 32,
                 sigma=0.3, seed: int = 0, dtype=torch.bfloat16, device="cpu",
                 zero_variance: bool = False, chunk: int = 256):
    """Returns (K, V, centres, z) with K, V [B][T][Hkv][d] in ``dtype``.

    centres [B][Hkv][n_centres][d] fp32; z [B][T][Hkv] int64 centre of each key."""
    gen = _gen(seed, device)
    centres = torch.randn(B, Hkv, n_centres, d, generator=gen, device=device)
    if zero_variance:
        centres = centres.to(torch.bfloat16).float()
        nchunk = (T + chunk - 1) // chunk
        base = torch.randint(0, n_centres, (B, nchunk, Hkv), generator=gen, device=device)
        run = (torch.arange(T, device=device) % chunk) // (chunk // 4)
        step = max(1, n_centres // 4)
        z = (base[:, torch.arange(T, device=device) // chunk, :] + run[None, :, None] * step) % n_centres
    else:
        z = torch.randint(0, n_centres, (B, T, Hkv), generator=gen, device=device)
    if isinstance(sigma, torch.Tensor):
        sig = sigma.to(device=device, dtype=torch.float32)
    else:
        sig = torch.full((n_centres,), float(sigma), device=device)
    K = torch.empty(B, T, Hkv, d, dtype=dtype, device=device)
    V = torch.empty(B, T, Hkv, d, dtype=dtype, device=device)
    hidx = torch.arange(Hkv, device=device)
    for b in range(B):  # one sequence at a time bounds the fp32 temporaries
        mu = centres[b][hidx[None, :], z[b]]  # [T][Hkv][d]
        if zero_variance:
            kb = mu
        else:
            eps = torch.randn(T, Hkv, d, generator=gen, device=device)
            kb = mu + sig[z[b]][..., None] * eps
        K[b] = kb.to(dtype)
        V[b] = torch.randn(T, Hkv, d, generator=gen, device=device).to(dtype)
    return K, V, centres, z


def queries(B: int, Hq: int, centres: torch.Tensor, *, n_rows: int | None = None,
            sigma=0.3, kind: str = "matched", seed: int = 1, dtype=torch.bfloat16,
            return_centres: bool = False):
    """Queries drawn against the key mixture of each query head's KV head.

    Returns [B][Hq][d] (decode) or, with n_rows, [B][n_rows][Hq][d] (prefill); with
    return_centres also the centre index of every matched query (same shape without
    d; -1 for diffuse queries)."""
    device = centres.device
    Bc, Hkv, nc, d = centres.shape
    assert Bc == B and Hq % Hkv == 0
    g = Hq // Hkv
    gen = _gen(seed, device)
    rows = 1 if n_rows is None else n_rows
    z = torch.full((B, rows, Hq), -1, dtype=torch.int64, device=device)
    if kind == "diffuse":
        q = torch.randn(B, rows, Hq, d, generator=gen, device=device)
    elif kind == "matched":
        z = torch.randint(0, nc, (B, rows, Hq), generator=gen, device=device)
        kvh = (torch.arange(Hq, device=device) // g)[None, None, :].expand(B, rows, Hq)
        bb = torch.arange(B, device=device)[:, None, None].expand(B, rows, Hq)
        mu = centres[bb, kvh, z]
        if isinstance(sigma, torch.Tensor):
            sig = sigma.to(device=device, dtype=torch.float32)[z][..., None]
        else:
            sig = float(sigma)
        q = mu + sig * torch.randn(B, rows, Hq, d, generator=gen, device=device)
    else:
        raise ValueError(f"unknown query kind {kind!r}")
    q = q.to(dtype)
    if n_rows is None:
        q, z = q[:, 0], z[:, 0]
    return (q, z) if return_centres else q


def video_qkv(B: int, frames: int, height: int, width: int, Hq: int, Hkv: int, d: int = 128, *,
              region=(8, 8, 8), n_centres: int = 32, sigma: float = 0.3, seed: int = 0,
              kind: str = "matched", dtype=torch.bfloat16, device="cpu", zero_variance_block=None):
    """Video tokens on a frames x height x width grid (raster order, T tokens).

    Returns (Q [B][T][Hq][d], K, V [B][T][Hkv][d]) in ``dtype``.  The grid is tiled by
    ``region`` boxes (clipped at the edges); every box of every (sequence, KV head)
    draws one of ``n_centres`` N(0, I_d) centres, and its keys are that centre plus
    sigma * N(0, I_d): nearby tokens look alike, as in video.  "matched" queries are
    the centre of their own box plus the same noise; "diffuse" queries are N(0, I_d).
    Values are N(0, I_d).  With ``zero_variance_block`` = (bf, bh, bw) every such
    block's keys are one centre rounded to bfloat16 with no noise."""
    gen = _gen(seed, device)
    T = frames * height * width
    g = Hq // Hkv
    assert Hq % Hkv == 0
    f = torch.arange(frames, device=device)[:, None, None]
    y = torch.arange(height, device=device)[None, :, None]
    x = torch.arange(width, device=device)[None, None, :]
    box = region if zero_variance_block is None else zero_variance_block
    ny, nx = -(-height // box[1]), -(-width // box[2])
    rid = ((f // box[0]) * ny + y // box[1]) * nx + x // box[2]
    rid = rid.reshape(T)
    nreg = int(rid.max()) + 1
    centres = torch.randn(B, Hkv, n_centres, d, generator=gen, device=device)
    if zero_variance_block is not None:
        centres = centres.to(torch.bfloat16).float()
    z = torch.randint(0, n_centres, (B, Hkv, nreg), generator=gen, device=device)
    K = torch.empty(B, T, Hkv, d, dtype=dtype, device=device)
    V = torch.empty(B, T, Hkv, d, dtype=dtype, device=device)
    Q = torch.empty(B, T, Hq, d, dtype=dtype, device=device)
    for b in range(B):
        for h in range(Hkv):
            mu = centres[b, h][z[b, h][rid]]  # [T][d]
            if zero_variance_block is None:
                K[b, :, h] = (mu + sigma * torch.randn(T, d, generator=gen, device=device)).to(dtype)
            else:
                K[b, :, h] = mu.to(dtype)
            V[b, :, h] = torch.randn(T, d, generator=gen, device=device).to(dtype)
            for j in range(g):
                if kind == "matched":
                    q = mu + sigma * torch.randn(T, d, generator=gen, device=device)
                elif kind == "diffuse":
                    q = torch.randn(T, d, generator=gen, device=device)
                else:
                    raise ValueError(f"unknown query kind {kind!r}")
                Q[b, :, h * g + j] = q.to(dtype)
    return Q, K, V
