// lod_video.hip -- video LoD attention ("Level of Detail Attention", section "Video
// LoD") and its dense bidirectional baseline, on MFMA.
//
// Tokens of an F x H x W grid (raster order) are cut into blocks (4x4x4), clipped at
// the far edges.  A block keeps its mean key and value, as a group does in "How It
// Works", and the queries of a block share one choice of opened key blocks, made with
// their mean query.  Three kernels:
//   summary  per (sequence, head, block): mean key and value (KV heads, rounded to
//            bf16) or mean query (query heads, kept fp32): fp32 sums in member order,
//            correctly rounded divide;
//   select   per (sequence, query head, up to 4 query blocks, one per wave): the fp32
//            fma chain of each mean query against every mean key, then the top c by
//            (score desc, id asc), stored in ascending id order;
//   attend   per (sequence, query head, query block): one online softmax over the
//            members of the opened blocks and, for every other block, one term with
//            bias ln n (the coarse remainder); the dense mode walks every key.
// The attend kernel keeps keys as MFMA rows and the block's 64 query slots as MFMA
// columns (S^T = K Q^T, one 16-column block per wave), so a lane holds one column of P
// and the PV product O^T = V^T P^T takes P straight from registers; V is staged
// transposed in LDS and P enters the PV product as bf16 hi + lo parts.
#include <math.h>

#include "lod_mfma.h"

namespace lodi {

constexpr int kVideoSlots = 64;          // member slots of a block (volume <= 64)
constexpr int kVideoMaxBlocks = 15360;   // blocks of a grid, at most
constexpr int kVideoMaxTop = 64;         // opened blocks per query block, at most
constexpr int kVideoScoreLds = 61440;    // bytes of select scores per workgroup, at most
constexpr uint32_t kTakenBits = 0x7fffffffu;  // marks a chosen score (a NaN no chain makes)

struct VideoArgs {
    const bf16_t* k;
    const bf16_t* v;
    int64_t sb, st, sh;         // strided KV view (elements)
    const bf16_t* q;            // [B][T][Hq][d]
    int F, H, W;                // grid
    int bf, bh, bw, bsz;        // block extents and volume
    int nby, nbx, NB, T;        // blocks along rows and columns, block count, tokens
    int Hq, Hkv, c, drop;
    float scale;
    bf16_t* kbar;               // workspace [B][Hkv][NB][d]
    bf16_t* vbar;
    float* lnn;                 // [NB]
    float* qbar;                // [B][Hq][NB][d]
    int32_t* sel;               // [B][Hq][NB][c]
    int32_t* sel_out;           // nullable copy of sel
    float* out;                 // [B][T][Hq][d]
};

// Token of member slot m of block blk, or -1 when the slot lies outside the grid.
__device__ __forceinline__ int video_token(const VideoArgs& A, int blk, int m) {
    if (m >= A.bsz) return -1;
    const int bfi = blk / (A.nby * A.nbx), byi = (blk / A.nbx) % A.nby, bxi = blk % A.nbx;
    const int i = m / (A.bh * A.bw), j = (m / A.bw) % A.bh, k = m % A.bw;
    const int f = bfi * A.bf + i, y = byi * A.bh + j, x = bxi * A.bw + k;
    return (f < A.F && y < A.H && x < A.W) ? (f * A.H + y) * A.W + x : -1;
}

// ---------------------------------------------------------------------------- summary

// grid (NB, Hkv + Hq, B).  y < Hkv: mean key and value of KV head y; else the mean
// query of query head y - Hkv.  Rows are staged with 16-byte loads, then thread
// (tensor, column) sums its column over the members in slot order, which is ascending
// token order.
__global__ __launch_bounds__(kThreads) void video_summary_kernel(VideoArgs A) {
    __shared__ alignas(16) bf16_t rows[2][kVideoSlots][kD];
    __shared__ int tok[kVideoSlots];
    const int blk = blockIdx.x, hh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const bool isq = hh >= A.Hkv;
    if (tid < kVideoSlots) tok[tid] = video_token(A, blk, tid);
    __syncthreads();
    const int ntens = isq ? 1 : 2;
    for (int i = tid; i < ntens * kVideoSlots * (kD / 8); i += kThreads) {
        const int tsr = i / (kVideoSlots * (kD / 8)), m = (i / (kD / 8)) % kVideoSlots, ch = i % (kD / 8);
        const int t = tok[m];
        if (t < 0) continue;
        const bf16_t* src = isq ? A.q + (((int64_t)b * A.T + t) * A.Hq + (hh - A.Hkv)) * kD
                                : (tsr ? A.v : A.k) + (int64_t)b * A.sb + (int64_t)t * A.st + (int64_t)hh * A.sh;
        *reinterpret_cast<uint4*>(&rows[tsr][m][8 * ch]) = *reinterpret_cast<const uint4*>(src + 8 * ch);
    }
    __syncthreads();
    const int tsr = tid / kD, col = tid % kD;
    if (tsr >= ntens) return;
    float s = 0.0f;
    int n = 0;
    for (int m = 0; m < A.bsz; ++m) {
        if (tok[m] < 0) continue;
        s = s + bf16_bits_to_f32(rows[tsr][m][col]);
        ++n;
    }
    const float mean = s / (float)n;  // every block holds its slot 0
    if (isq) {
        A.qbar[(((int64_t)b * A.Hq + (hh - A.Hkv)) * A.NB + blk) * kD + col] = mean;
    } else {
        bf16_t* dst = tsr ? A.vbar : A.kbar;
        dst[(((int64_t)b * A.Hkv + hh) * A.NB + blk) * kD + col] = f32_to_bf16_rne(mean);
        if (b == 0 && hh == 0 && tid == 0) A.lnn[blk] = logf((float)n);
    }
}

// ---------------------------------------------------------------------------- select

// grid (ceil(NB / QPW), Hq, B), dynamic LDS QPW * NB floats.  Query blocks
// QPW*x .. QPW*x + QPW-1; wave w < QPW ranks the scores of query block QPW*x + w.
template <int QPW>
__global__ __launch_bounds__(kThreads) void video_select_kernel(VideoArgs A) {
    extern __shared__ float sc[];  // [QPW][NB]
    __shared__ alignas(16) float qs[QPW][kD];
    __shared__ int win[4][kVideoMaxTop];
    const int hq = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int qb0 = blockIdx.x * QPW;
    const int kvh = hq / (A.Hq / A.Hkv);
    for (int i = tid; i < QPW * kD; i += kThreads) {
        const int qi = i / kD, t = i % kD;
        const int qb = min(qb0 + qi, A.NB - 1);
        qs[qi][t] = A.qbar[(((int64_t)b * A.Hq + hq) * A.NB + qb) * kD + t];
    }
    __syncthreads();
    // scores: one mean key per thread and pass, QPW chains over it in index order
    const bf16_t* kb = A.kbar + ((int64_t)b * A.Hkv + kvh) * A.NB * kD;
    for (int j = tid; j < A.NB; j += kThreads) {
        const uint4* row = reinterpret_cast<const uint4*>(kb + (int64_t)j * kD);
        float acc[QPW];
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) acc[qi] = 0.0f;
#pragma unroll 4
        for (int c8 = 0; c8 < kD / 8; ++c8) {
            const uint4 u = row[c8];
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kf = bf16_bits_to_f32((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu);
#pragma unroll
                for (int qi = 0; qi < QPW; ++qi) acc[qi] = __builtin_fmaf(qs[qi][8 * c8 + e], kf, acc[qi]);
            }
        }
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) sc[qi * A.NB + j] = acc[qi];
    }
    __syncthreads();
    if (w >= QPW) return;
    const int qb = qb0 + w;
    if (qb >= A.NB) return;
    float* s = sc + w * A.NB;
    const int k = min(A.c, A.NB);
    // each lane keeps the best key of its entries j = l, l + 64, ...; the wave takes the
    // best of all lanes k times, and the owner of each winner marks it and rescans
    auto best_of = [&]() {
        uint64_t bk = 0;
        for (int j = l; j < A.NB; j += 64) {
            const float x = s[j];
            if (__float_as_uint(x) == kTakenBits) continue;
            const uint64_t key = rank_key(x, (uint32_t)j);
            bk = key > bk ? key : bk;
        }
        return bk;
    };
    uint64_t mine = best_of();
    int wsel = -1;
    for (int r = 0; r < k; ++r) {
        const uint64_t top = wave_max_u64(mine);
        const int j = (int)key_id(top);
        if (l == r) wsel = j;
        if ((j & 63) == l) {
            s[j] = __uint_as_float(kTakenBits);
            mine = best_of();
        }
    }
    win[w][l] = wsel;
    wave_sync_lds();
    if (l < A.c) {
        const int64_t o = (((int64_t)b * A.Hq + hq) * A.NB + qb) * A.c;
        int pos = l, val = -1;
        if (l < k) {
            pos = 0;
            for (int i = 0; i < k; ++i) pos += win[w][i] < wsel;
            val = wsel;
        }
        A.sel[o + pos] = val;
        if (A.sel_out) A.sel_out[o + pos] = val;
    }
}

// ---------------------------------------------------------------------------- attend

struct VideoSmem {
    alignas(16) bf16_t kt[kFlashKeys][kD];      // key tile, 16-byte chunks XOR-swizzled
    alignas(16) bf16_t vT[kD][kFlashKeys + 4];  // value tile, transposed
    float bias[kFlashKeys];
    int sel[kVideoMaxTop];
    uint32_t opened[kVideoMaxBlocks / 32];      // bitmap of the opened key blocks
};

struct VideoState {
    f32x4_t O[8];  // O^T, one 16 x 16 tile per d block
    float m, l;
};

// One tile of 64 key slots: rows krow(r), vrow(r) (always readable addresses), bias
// bias_of(r) (-inf: no key).  Column = this lane's query slot (16 w + l % 16).
template <typename KRow, typename VRow, typename Bias>
__device__ __forceinline__ void video_tile(VideoSmem& s, VideoState& F, const bf16x8_t* qf, KRow krow, VRow vrow,
                                           Bias bias_of, float scale) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    for (int i = w; i < kFlashKeys / 4; i += 4) {
        const int row = 4 * i + (l >> 4);
        const int cp = l & 15, c = cp ^ (row & 15);
        __builtin_amdgcn_global_load_lds(krow(row) + 8 * c, &s.kt[4 * i][0], 16, 0, 0);
    }
    uint4 vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i, key = idx & 63, ch = idx >> 6;
        vv[i] = *reinterpret_cast<const uint4*>(vrow(key) + 8 * ch);
    }
    if (tid < kFlashKeys) s.bias[tid] = bias_of(tid);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i, key = idx & 63, ch = idx >> 6;
        const uint32_t u[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s.vT[8 * ch + 2 * e][key] = (bf16_t)(u[e] & 0xffffu);
            s.vT[8 * ch + 2 * e + 1][key] = (bf16_t)(u[e] >> 16);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // S^T = K Q^T: 4 key blocks of 16 for this wave's 16 columns
    f32x4_t S[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        S[kb] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int row = 16 * kb + (l & 15);
            const int chunk = (4 * kk + (l >> 4)) ^ (row & 15);
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&s.kt[row][8 * chunk]);
            S[kb] = mfma16(a, qf[kk], S[kb]);
        }
    }
    // logits and the online softmax (a column's 64 keys live in lanes l, l^16, l^32, l^48)
    float P[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float b = s.bias[16 * kb + 4 * (l >> 4) + r];
            const float lam = b != -INFINITY ? __builtin_fmaf(scale, S[kb][r], b) : -INFINITY;
            P[kb][r] = lam;
            mt = fmaxf(mt, lam);
        }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(F.m, mt);
    const float a = F.m == -INFINITY ? 0.0f : softmax_exp(F.m - mn);
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float lam = P[kb][r];
            const float p = lam == -INFINITY ? 0.0f : softmax_exp(lam - mn);
            P[kb][r] = p;
            ls += p;
        }
    F.l = __builtin_fmaf(F.l, a, ls);
    F.m = mn;
#pragma unroll
    for (int db = 0; db < 8; ++db) F.O[db] *= a;
    // O^T += V^T P^T over two 32-key steps; P as bf16 hi + lo
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        bf16x8_t ph, pl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __bf16 h, lo;
            split_bf16(P[2 * st + j / 4][j % 4], h, lo);
            ph[j] = h;
            pl[j] = lo;
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const bf16_t* vr = &s.vT[16 * db + (l & 15)][32 * st + 4 * (l >> 4)];
            const uint2 lo4 = *reinterpret_cast<const uint2*>(vr);
            const uint2 hi4 = *reinterpret_cast<const uint2*>(vr + 16);
            const u32x4_t raw = {lo4.x, lo4.y, hi4.x, hi4.y};  // keys 8 (l/16) .. +7 of the step
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, raw);
            F.O[db] = mfma16(av, ph, F.O[db]);
            F.O[db] = mfma16(av, pl, F.O[db]);
        }
    }
    __syncthreads();
}

// grid (NB, Hq, B): the 64 query slots of query block blockIdx.x of query head
// blockIdx.y.  LoD: the opened blocks' members, then the mean keys of the other blocks
// with bias ln n.  DENSE: every key of the grid in tiles of 64 consecutive tokens.
template <bool DENSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void video_attend_kernel(VideoArgs A) {
    __shared__ VideoSmem s;
    const int qb = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int kvh = hq / (A.Hq / A.Hkv);
    const int qt = video_token(A, qb, 16 * w + (l & 15));
    bf16x8_t qf[4];
    {
        const bf16_t* qr = A.q + (((int64_t)b * A.T + (qt < 0 ? 0 : qt)) * A.Hq + hq) * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[kk] = qt < 0 ? zero_bf16x8() : *reinterpret_cast<const bf16x8_t*>(qr + 32 * kk + 8 * (l >> 4));
    }
    VideoState F;
    F.m = -INFINITY;
    F.l = 0.0f;
#pragma unroll
    for (int db = 0; db < 8; ++db) F.O[db] = {0.0f, 0.0f, 0.0f, 0.0f};
    const bf16_t* kc = A.k + (int64_t)b * A.sb + (int64_t)kvh * A.sh;
    const bf16_t* vc = A.v + (int64_t)b * A.sb + (int64_t)kvh * A.sh;

    if (DENSE) {
        for (int k0 = 0; k0 < A.T; k0 += kFlashKeys) {
            const int nk = min(kFlashKeys, A.T - k0);
            video_tile(
                s, F, qf, [&](int r) { return kc + (int64_t)(k0 + min(r, nk - 1)) * A.st; },
                [&](int r) { return vc + (int64_t)(k0 + min(r, nk - 1)) * A.st; },
                [&](int r) { return r < nk ? 0.0f : -INFINITY; }, A.scale);
        }
    } else {
        const int32_t* selr = A.sel + (((int64_t)b * A.Hq + hq) * A.NB + qb) * A.c;
        for (int i = tid; i < (A.NB + 31) / 32; i += kThreads) s.opened[i] = 0;
        __syncthreads();
        if (tid < A.c) {
            const int j = selr[tid];
            s.sel[tid] = j;
            if (j >= 0) atomicOr(&s.opened[j >> 5], 1u << (j & 31));
        }
        __syncthreads();
        // exact: the members of each opened block (ascending ids, -1 padding last)
        for (int u = 0; u < A.c; ++u) {
            const int j = s.sel[u];
            if (j < 0) break;
            const int t0 = video_token(A, j, 0);  // slot 0 always lies in the grid
            auto tok = [&](int r) {
                const int t = video_token(A, j, r);
                return t < 0 ? t0 : t;
            };
            video_tile(
                s, F, qf, [&](int r) { return kc + (int64_t)tok(r) * A.st; },
                [&](int r) { return vc + (int64_t)tok(r) * A.st; },
                [&](int r) { return video_token(A, j, r) < 0 ? -INFINITY : 0.0f; }, A.scale);
        }
        // coarse: every other block's mean key and value with bias ln n
        if (!A.drop) {
            const bf16_t* kb = A.kbar + ((int64_t)b * A.Hkv + kvh) * A.NB * kD;
            const bf16_t* vb = A.vbar + ((int64_t)b * A.Hkv + kvh) * A.NB * kD;
            for (int j0 = 0; j0 < A.NB; j0 += kFlashKeys) {
                video_tile(
                    s, F, qf, [&](int r) { return kb + (int64_t)min(j0 + r, A.NB - 1) * kD; },
                    [&](int r) { return vb + (int64_t)min(j0 + r, A.NB - 1) * kD; },
                    [&](int r) {
                        const int j = j0 + r;
                        return (j < A.NB && !((s.opened[j >> 5] >> (j & 31)) & 1u)) ? A.lnn[j] : -INFINITY;
                    },
                    A.scale);
            }
        }
    }
    // column total (the 4 lanes of a column hold partial sums), then write
    float lt = F.l;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (qt < 0) return;
    float* dst = A.out + (((int64_t)b * A.T + qt) * A.Hq + hq) * kD;
    const float inv = 1.0f / lt;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        const f32x4_t o = F.O[db];
        *reinterpret_cast<float4*>(dst + 16 * db + 4 * (l >> 4)) =
            make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
}

// ---------------------------------------------------------------------------- host side

static int check_video_params(const lod_video_params* p) {
    if (!p) return LOD_ERR_ARG;
    if (p->head_dim <= 0 || p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->n_q_heads % p->n_kv_heads != 0)
        return LOD_ERR_ARG;
    if (p->frames <= 0 || p->height <= 0 || p->width <= 0 || p->block_f <= 0 || p->block_h <= 0 ||
        p->block_w <= 0 || p->top_blocks <= 0)
        return LOD_ERR_ARG;
    if ((int64_t)p->frames * p->height * p->width > INT32_MAX) return LOD_ERR_ARG;
    if (!(p->scale > 0.0f) || !isfinite(p->scale)) return LOD_ERR_ARG;
    if (p->drop_remainder != 0 && p->drop_remainder != 1) return LOD_ERR_ARG;
    if (p->kv_dtype != LOD_F32 && p->kv_dtype != LOD_BF16) return LOD_ERR_ARG;
    if (p->head_dim != kD || p->kv_dtype != LOD_BF16) return LOD_ERR_UNSUPPORTED;
    if ((int64_t)p->block_f * p->block_h * p->block_w > kVideoSlots || p->top_blocks > kVideoMaxTop)
        return LOD_ERR_UNSUPPORTED;
    const int64_t nb = ceil_div(p->frames, p->block_f) * ceil_div(p->height, p->block_h) *
                       ceil_div(p->width, p->block_w);
    if (nb > kVideoMaxBlocks) return LOD_ERR_UNSUPPORTED;
    return LOD_OK;
}

static lod_video_layout_t video_layout(const lod_video_params* p, int32_t batch) {
    lod_video_layout_t L{};
    const size_t nb = (size_t)(ceil_div(p->frames, p->block_f) * ceil_div(p->height, p->block_h) *
                               ceil_div(p->width, p->block_w));
    const size_t B = (size_t)batch, d = (size_t)p->head_dim;
    size_t o = 0;
    L.kbar = o; o = align256(o + B * p->n_kv_heads * nb * d * 2);
    L.vbar = o; o = align256(o + B * p->n_kv_heads * nb * d * 2);
    L.lnn = o;  o = align256(o + nb * 4);
    L.qbar = o; o = align256(o + B * p->n_q_heads * nb * d * 4);
    L.sel = o;  o = align256(o + B * p->n_q_heads * nb * p->top_blocks * 4);
    L.total = o;
    L.n_blocks = (int32_t)nb;
    return L;
}

static int check_video_view(const lod_kv& kv, const void* q, const float* out) {
    if (!kv.k || !kv.v || !q || !out) return LOD_ERR_ARG;
    if (kv.block_table) return LOD_ERR_UNSUPPORTED;
    if (kv.stride_t <= 0 || kv.stride_h < 0 || kv.stride_b < 0) return LOD_ERR_ARG;
    if ((kv.stride_t | kv.stride_h | kv.stride_b) % 8 != 0) return LOD_ERR_ARG;
    if (((uintptr_t)kv.k | (uintptr_t)kv.v | (uintptr_t)q | (uintptr_t)out) % 16 != 0) return LOD_ERR_ARG;
    return LOD_OK;
}

static VideoArgs video_args(const lod_video_params* p, const lod_kv& kv, const void* q, float* out) {
    VideoArgs A{};
    A.k = static_cast<const bf16_t*>(kv.k);
    A.v = static_cast<const bf16_t*>(kv.v);
    A.sb = kv.stride_b; A.st = kv.stride_t; A.sh = kv.stride_h;
    A.q = static_cast<const bf16_t*>(q);
    A.F = p->frames; A.H = p->height; A.W = p->width;
    A.bf = p->block_f; A.bh = p->block_h; A.bw = p->block_w;
    A.bsz = p->block_f * p->block_h * p->block_w;
    A.nby = (int)ceil_div(p->height, p->block_h);
    A.nbx = (int)ceil_div(p->width, p->block_w);
    A.NB = (int)ceil_div(p->frames, p->block_f) * A.nby * A.nbx;
    A.T = p->frames * p->height * p->width;
    A.Hq = p->n_q_heads; A.Hkv = p->n_kv_heads;
    A.c = p->top_blocks;
    A.drop = p->drop_remainder;
    A.scale = p->scale;
    A.out = out;
    return A;
}

template <int QPW>
static void launch_video_select(const VideoArgs& A, int batch, hipStream_t st) {
    hipLaunchKernelGGL((video_select_kernel<QPW>), dim3((unsigned)ceil_div(A.NB, QPW), A.Hq, batch), dim3(kThreads),
                       (size_t)QPW * A.NB * sizeof(float), st, A);
}

}  // namespace lodi

using namespace lodi;

extern "C" int lod_video_layout(const lod_video_params* params, int32_t batch, lod_video_layout_t* layout) {
    const int rc = check_video_params(params);
    if (rc != LOD_OK) return rc;
    if (batch <= 0 || !layout) return LOD_ERR_ARG;
    *layout = video_layout(params, batch);
    return LOD_OK;
}

extern "C" int lod_video_ws_bytes(const lod_video_params* params, int32_t batch, size_t* bytes) {
    lod_video_layout_t L;
    const int rc = lod_video_layout(params, batch, &L);
    if (rc != LOD_OK) return rc;
    if (!bytes) return LOD_ERR_ARG;
    *bytes = L.total;
    return LOD_OK;
}

extern "C" int lod_video_attend(const lod_video_params* params, lod_kv kv, const void* q, int32_t batch,
                                float* out, int32_t* sel_blocks, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_video_params(params);
    if (rc != LOD_OK) return rc;
    if (batch <= 0) return LOD_ERR_ARG;
    rc = check_video_view(kv, q, out);
    if (rc != LOD_OK) return rc;
    const lod_video_layout_t L = video_layout(params, batch);
    if (!ws || ws_bytes < L.total) return LOD_ERR_WORKSPACE;
    if ((uintptr_t)ws % 16 != 0) return LOD_ERR_ARG;
    VideoArgs A = video_args(params, kv, q, out);
    char* base = static_cast<char*>(ws);
    A.kbar = reinterpret_cast<bf16_t*>(base + L.kbar);
    A.vbar = reinterpret_cast<bf16_t*>(base + L.vbar);
    A.lnn = reinterpret_cast<float*>(base + L.lnn);
    A.qbar = reinterpret_cast<float*>(base + L.qbar);
    A.sel = reinterpret_cast<int32_t*>(base + L.sel);
    A.sel_out = sel_blocks;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(video_summary_kernel, dim3(A.NB, A.Hkv + A.Hq, batch), dim3(kThreads), 0, st, A);
    // as many query blocks per select workgroup as the score buffer allows
    if ((size_t)4 * A.NB * sizeof(float) <= (size_t)kVideoScoreLds) launch_video_select<4>(A, batch, st);
    else if ((size_t)2 * A.NB * sizeof(float) <= (size_t)kVideoScoreLds) launch_video_select<2>(A, batch, st);
    else launch_video_select<1>(A, batch, st);
    hipLaunchKernelGGL((video_attend_kernel<false>), dim3(A.NB, A.Hq, batch), dim3(kThreads), 0, st, A);
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}

extern "C" int lod_video_dense(const lod_video_params* params, lod_kv kv, const void* q, int32_t batch, float* out,
                               void* stream) {
    int rc = check_video_params(params);
    if (rc != LOD_OK) return rc;
    if (batch <= 0) return LOD_ERR_ARG;
    rc = check_video_view(kv, q, out);
    if (rc != LOD_OK) return rc;
    VideoArgs A = video_args(params, kv, q, out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL((video_attend_kernel<true>), dim3(A.NB, A.Hq, batch), dim3(kThreads), 0, st, A);
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}
