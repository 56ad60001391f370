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
constexpr int kVideoMaxBlocks = 13312;   // blocks of a grid, at most
constexpr int kVideoMaxTop = 64;         // opened blocks per query block, at most
constexpr int kVideoScoreLds = 53248;    // bytes of select scores per workgroup (with the static arrays, under 64 KB)
constexpr int kVideoCand = 128;          // top-c candidates a select wave ranks exactly
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

// grid (ceil(Hkv / 8) + ceil(Hq / 16), NB, B).  Thread (tensor slot tt = tid / 16,
// column group cg = tid % 16) owns columns 8 cg .. 8 cg + 7 of one tensor of block
// blockIdx.y: a unit x < ceil(Hkv / 8) covers the keys (even tt) and values (odd tt) of
// KV heads 8 x + tt / 2; a later unit the queries of 16 query heads.  The thread reads
// the block's rows 16 at a time with 16-byte loads and adds each column in member
// order, which is ascending token order.
__global__ __launch_bounds__(kThreads) void video_summary_kernel(VideoArgs A) {
    __shared__ int tok[kVideoSlots];
    const int u = blockIdx.x, blk = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int cg = tid & 15, tt = tid >> 4;
    const int nku = (A.Hkv + 7) / 8;
    const bool isq = u >= nku;
    const int head = isq ? 16 * (u - nku) + tt : 8 * u + (tt >> 1);
    const bool valid = head < (isq ? A.Hq : A.Hkv);
    const bf16_t* base = isq ? A.q + ((int64_t)b * A.T * A.Hq + head) * kD + 8 * cg
                             : ((tt & 1) ? A.v : A.k) + (int64_t)b * A.sb + (int64_t)head * A.sh + 8 * cg;
    const int64_t ts = isq ? (int64_t)A.Hq * kD : A.st;  // elements between tokens
    if (tid < kVideoSlots) tok[tid] = video_token(A, blk, tid);
    __syncthreads();
    if (!valid) return;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    int n = 0;
    for (int rb = 0; rb < A.bsz; rb += 16) {
        uint4 x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = rb + i < kVideoSlots ? tok[rb + i] : -1;
            x[i] = t >= 0 ? *reinterpret_cast<const uint4*>(base + (int64_t)t * ts) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (rb + i >= kVideoSlots || tok[rb + i] < 0) continue;
            const uint32_t wd[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = acc[e] + bf16_bits_to_f32((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            ++n;
        }
    }
    float mean[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mean[e] = acc[e] / (float)n;  // every block holds its slot 0
    if (isq) {
        float* dst = A.qbar + (((int64_t)b * A.Hq + head) * A.NB + blk) * kD + 8 * cg;
        *reinterpret_cast<float4*>(dst) = make_float4(mean[0], mean[1], mean[2], mean[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(mean[4], mean[5], mean[6], mean[7]);
    } else {
        bf16_t* dst = ((tt & 1) ? A.vbar : A.kbar) + (((int64_t)b * A.Hkv + head) * A.NB + blk) * kD + 8 * cg;
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pk[e] = (uint32_t)f32_to_bf16_rne(mean[2 * e]) | ((uint32_t)f32_to_bf16_rne(mean[2 * e + 1]) << 16);
        *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        if (b == 0 && u == 0 && tid == 0) A.lnn[blk] = logf((float)n);
    }
}

// ---------------------------------------------------------------------------- select

// grid (ceil(NB / QPW), Hq, B), dynamic LDS QPW * NB floats.  Query blocks
// QPW*x .. QPW*x + QPW-1 share every mean key the workgroup loads.
template <int QPW>
__global__ __launch_bounds__(kThreads) void video_select_kernel(VideoArgs A) {
    extern __shared__ float sc[];  // [QPW][NB]
    __shared__ alignas(16) float qs[QPW][kD];
    __shared__ int win[4][kVideoMaxTop];
    __shared__ uint64_t ckey[4][kVideoCand];
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
    // Wave w ranks query blocks QPW*x + w, + w + 4, ...  The k-th largest of the 64 lane
    // maxima (lane l holds entries l, l + 64, ...) is at most the k-th largest key, so
    // every winner is among the keys at or above it; those candidates are compacted and
    // ranked exactly.  More than kVideoCand candidates (the best keys crowd into a few
    // lanes) fall back to k rounds of a wave-wide maximum with rescans.
    const int k = min(A.c, A.NB);
    for (int qq = w; qq < QPW; qq += 4) {
        const int qb = qb0 + qq;
        if (qb >= A.NB) break;
        float* s = sc + qq * A.NB;
        const int64_t o = (((int64_t)b * A.Hq + hq) * A.NB + qb) * A.c;
        uint64_t lm = 0;
        for (int j = l; j < A.NB; j += 64) {
            const uint64_t key = rank_key(s[j], (uint32_t)j);
            lm = key > lm ? key : lm;
        }
        // k rounds over the lane maxima (keys are distinct, so one lane leaves per round);
        // at least k lanes hold entries, so tau is a real key
        uint64_t cur = lm, tau = 0;
        for (int r = 0; r < k; ++r) {
            tau = wave_max_u64(cur);
            if (cur == tau) cur = 0;
        }
        int ncand = 0;
        for (int j0 = 0; j0 < A.NB; j0 += 64) {
            const int j = j0 + l;
            const uint64_t key = j < A.NB ? rank_key(s[j], (uint32_t)j) : 0;
            const bool in = key >= tau;
            const uint64_t bal = __ballot(in);
            const int pos = ncand + __popcll(bal & ((1ull << l) - 1ull));
            if (in && pos < kVideoCand) ckey[w][pos] = key;
            ncand += __popcll(bal);
        }
        wave_sync_lds();
        if (ncand <= kVideoCand) {
            // rank of each candidate among all candidates; winners store their id by rank
            for (int i = l; i < ncand; i += 64) {
                const uint64_t mine = ckey[w][i];
                int rank = 0;
                for (int j = 0; j < ncand; ++j) rank += ckey[w][j] > mine;
                if (rank < k) win[w][rank] = (int)key_id(mine);
            }
        } else {
            uint64_t best = 0;
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
            best = best_of();
            int wsel = -1;
            for (int r = 0; r < k; ++r) {
                const uint64_t top = wave_max_u64(best);
                const int j = (int)key_id(top);
                if (l == r) wsel = j;
                if ((j & 63) == l) {
                    s[j] = __uint_as_float(kTakenBits);
                    best = best_of();
                }
            }
            if (l < k) win[w][l] = wsel;
        }
        wave_sync_lds();
        // the k winners in ascending id order, -1 padding up to c
        if (l < A.c) {
            int pos = l, val = -1;
            if (l < k) {
                val = win[w][l];
                pos = 0;
                for (int i = 0; i < k; ++i) pos += win[w][i] < val;
            }
            A.sel[o + pos] = val;
            if (A.sel_out) A.sel_out[o + pos] = val;
        }
        wave_sync_lds();  // win[w] and ckey[w] are rewritten by the next query block
    }
}

// ---------------------------------------------------------------------------- attend

// A workgroup takes two neighbouring query blocks (raster order) of one query head;
// wave w serves query block w / 2, columns 32 (w % 2) .. +31 (two 16-column MFMA
// blocks).  Its key tiles are the union of the two blocks' opened blocks, then the mean
// keys of all blocks; a wave skips the exact tiles its own block did not open, and the
// coarse tiles mask its own opened blocks.  K and V tiles are double buffered and
// loaded straight into LDS; both are row-major with 16-byte chunks XOR-swizzled (K by
// row & 15, V by 2 (row & 7)), and V^T operands come from transposing LDS reads.
constexpr int kVideoPair = 2;  // query blocks per attend workgroup
constexpr float kLog2e = 1.4426950408889634f;

struct VideoSmem {
    alignas(16) bf16_t kt[2][kFlashKeys][kD];  // key tiles (double buffer)
    alignas(16) bf16_t vt[2][kFlashKeys][kD];  // value tiles (double buffer)
    float bias[2][kVideoPair][kFlashKeys];     // [buffer][query block of the pair][key slot]
    int tl[kVideoPair * kVideoMaxTop];         // exact tiles: block ids, ascending
    int tmask[kVideoPair * kVideoMaxTop];      // bit q: query block q of the pair opened it
    int sl[kVideoPair][kVideoMaxTop];          // each block's opened list
    uint32_t opened[kVideoPair][kVideoMaxBlocks / 32];
    int tdesc[kVideoPair * kVideoMaxTop][2];   // exact tiles: block origin token, clipped extents
    int nex;
};

__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return 2 * (row & 7); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 4 bf16 of a V^T operand: this lane gets V[key0 + r][d0 + lane % 16] for r = 0..3,
// where the 16 lanes of its group read (row key0 + i / 4, elements d0 + 4 (i % 4) ..).
__device__ __forceinline__ s16x4_t vt_read(const bf16_t (*vt)[kD], int key0, int d0, int i) {
    const int row = key0 + (i >> 2);
    const int e = d0 + 4 * (i & 3);
    const int chunk = (e >> 3) ^ swz_v(row);
    const bf16_t* p = &vt[row][8 * chunk + (e & 7)];
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
}

template <bool DENSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void video_attend_kernel(VideoArgs A) {
    __shared__ VideoSmem s;
    const int pair = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
    const int kvh = hq / (A.Hq / A.Hkv);
    const int qb0 = kVideoPair * pair;
    const int nqb = min(kVideoPair, A.NB - qb0);
    const int qi = w >> 1;  // query block of this wave within the pair
    const bool on = qi < nqb;
    const int qb = qb0 + min(qi, nqb - 1);

    // member slots of the tile rows this thread loads (rows 4 (w + 4 ii) + g) and of its
    // bias entry (row l): token offset from the block origin and (frame, row, column)
    // offsets; a slot beyond the block volume gets offsets no block reaches
    int soff[5], si[5], sj[5], sk[5];
#pragma unroll
    for (int ii = 0; ii < 5; ++ii) {
        const int m = ii < 4 ? 4 * (w + 4 * ii) + g : l;
        const int i = m / (A.bh * A.bw), j = (m / A.bw) % A.bh, k = m % A.bw;
        soff[ii] = (i * A.H + j) * A.W + k;
        si[ii] = m < A.bsz ? i : 1 << 20;
        sj[ii] = j;
        sk[ii] = k;
    }
    // Q^T operands of this lane's two columns
    bf16x8_t qf[2][4];
    int qt[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        qt[cb] = on ? video_token(A, qb, 32 * (w & 1) + 16 * cb + li) : -1;
        const bf16_t* qr = A.q + (((int64_t)b * A.T + (qt[cb] < 0 ? 0 : qt[cb])) * A.Hq + hq) * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[cb][kk] = qt[cb] < 0 ? zero_bf16x8() : *reinterpret_cast<const bf16x8_t*>(qr + 32 * kk + 8 * g);
    }
    f32x4_t O[2][8];
    float m_run[2], l_run[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) O[cb][db] = {0.0f, 0.0f, 0.0f, 0.0f};
    }
    const bf16_t* kc = A.k + (int64_t)b * A.sb + (int64_t)kvh * A.sh;
    const bf16_t* vc = A.v + (int64_t)b * A.sb + (int64_t)kvh * A.sh;
    const bf16_t* kbr = A.kbar + ((int64_t)b * A.Hkv + kvh) * A.NB * kD;
    const bf16_t* vbr = A.vbar + ((int64_t)b * A.Hkv + kvh) * A.NB * kD;
    const float sc2 = A.scale * kLog2e;  // logits in log2 units: exp2 weights

    int nex = 0;
    if (!DENSE) {
        for (int i = tid; i < kVideoPair * (kVideoMaxBlocks / 32); i += kThreads) (&s.opened[0][0])[i] = 0;
        __syncthreads();
        if (tid < kVideoPair * A.c) {
            const int q = tid / A.c, u = tid % A.c;
            const int j = q < nqb ? A.sel[(((int64_t)b * A.Hq + hq) * A.NB + qb0 + q) * A.c + u] : -1;
            s.sl[q][u] = j;
            if (j >= 0) atomicOr(&s.opened[q][j >> 5], 1u << (j & 31));
        }
        __syncthreads();
        if (tid == 0) {  // merge the two ascending lists (-1 padding last)
            int ia = 0, ib = 0, n = 0;
            const int* sa = s.sl[0];
            const int* sb2 = s.sl[1];
            auto len = [&](const int* x) {
                int c = 0;
                while (c < A.c && x[c] >= 0) ++c;
                return c;
            };
            const int na = len(sa), nb = nqb > 1 ? len(sb2) : 0;
            while (ia < na || ib < nb) {
                int x, mk;
                if (ib >= nb || (ia < na && sa[ia] < sb2[ib])) { x = sa[ia++]; mk = 1; }
                else if (ia >= na || sb2[ib] < sa[ia]) { x = sb2[ib++]; mk = 2; }
                else { x = sa[ia]; ++ia; ++ib; mk = 3; }
                s.tl[n] = x;
                s.tmask[n] = mk;
                ++n;
            }
            s.nex = n;
        }
        __syncthreads();
        nex = s.nex;
        if (tid < nex) {  // origin token and clipped extents of each opened block
            const int j = s.tl[tid];
            const int bfi = j / (A.nby * A.nbx), byi = (j / A.nbx) % A.nby, bxi = j % A.nbx;
            s.tdesc[tid][0] = ((bfi * A.bf) * A.H + byi * A.bh) * A.W + bxi * A.bw;
            s.tdesc[tid][1] = min(A.bf, A.F - bfi * A.bf) | (min(A.bh, A.H - byi * A.bh) << 8) |
                              (min(A.bw, A.W - bxi * A.bw) << 16);
        }
        __syncthreads();
    }
    const int ntc = DENSE || A.drop ? 0 : (A.NB + kFlashKeys - 1) / kFlashKeys;
    const int nt = DENSE ? (A.T + kFlashKeys - 1) / kFlashKeys : nex + ntc;

    // Load tile t into buffer `buf`: K and V rows straight to LDS, and the two bias rows.
    auto issue = [&](int t, int buf) {
        const int kind = DENSE ? 0 : (t < nex ? 1 : 2);  // 0 dense run, 1 opened block, 2 coarse
        const bf16_t* kbase = kind == 2 ? kbr : kc;
        const bf16_t* vbase = kind == 2 ? vbr : vc;
        const int64_t stride = kind == 2 ? (int64_t)kD : A.st;
        int origin = 0, lf = 0, lh = 0, lw = 0, first = 0, nk = 0;
        if (kind == 1) {
            origin = s.tdesc[t][0];
            const int ext = s.tdesc[t][1];
            lf = ext & 255;
            lh = (ext >> 8) & 255;
            lw = ext >> 16;
        } else {
            first = kind == 0 ? t * kFlashKeys : (t - nex) * kFlashKeys;
            nk = min(kFlashKeys, (kind == 0 ? A.T : A.NB) - first);
        }
        // slot ii of this thread -> row index (token or block) and whether it holds a key
        auto row_of = [&](int ii, int r, bool& ok) -> int {
            if (kind == 1) {
                ok = si[ii] < lf && sj[ii] < lh && sk[ii] < lw;
                return origin + (ok ? soff[ii] : 0);
            }
            ok = r < nk;
            return first + (ok ? r : nk - 1);
        };
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = w + 4 * ii;
            const int row = 4 * i + g;
            bool ok;
            const int64_t off = (int64_t)row_of(ii, row, ok) * stride;
            __builtin_amdgcn_global_load_lds(kbase + off + 8 * (li ^ swz_k(row)), &s.kt[buf][4 * i][0], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vbase + off + 8 * (li ^ swz_v(row)), &s.vt[buf][4 * i][0], 16, 0, 0);
        }
        if (tid < kVideoPair * kFlashKeys) {
            const int q = tid >> 6, r = l;
            bool ok;
            const int x = row_of(4, r, ok);
            float bv = -INFINITY;  // in log2 units, like the scaled logits
            if (kind == 0) bv = ok ? 0.0f : -INFINITY;
            else if (kind == 1) bv = ok && ((s.tmask[t] >> q) & 1) ? 0.0f : -INFINITY;
            else if (ok && !((s.opened[q][x >> 5] >> (x & 31)) & 1u)) bv = A.lnn[x] * kLog2e;
            s.bias[buf][q][r] = bv;
        }
    };

    if (nt > 0) issue(0, 0);
    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 < nt) issue(t + 1, buf ^ 1);
        const bool use = on && (DENSE || t >= nex || ((s.tmask[t] >> qi) & 1));
        if (!use) continue;
        // S^T = K Q^T: 4 key blocks x 2 column blocks
        f32x4_t S[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            S[kb][0] = {0.0f, 0.0f, 0.0f, 0.0f};
            S[kb][1] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int row = 16 * kb + li;
                const int chunk = (4 * kk + g) ^ swz_k(row);
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&s.kt[buf][row][8 * chunk]);
                S[kb][0] = mfma16(a, qf[0][kk], S[kb][0]);
                S[kb][1] = mfma16(a, qf[1][kk], S[kb][1]);
            }
        }
        // logits in log2 units and the online softmax (a column's 64 keys live in lanes
        // l, l^16, l^32, l^48).  A masked key has bias -inf, so its logit is -inf and its
        // weight exp2(-inf) = 0.  The first tile a wave computes always holds a key of its
        // own (an opened block's slot 0, or a dense run), so the running maximum is finite
        // from then on and no difference below is -inf - (-inf).
        const float* bias = s.bias[buf][qi];
        float P[4][2][4];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float lam = __builtin_fmaf(sc2, S[kb][cb][r], bias[16 * kb + 4 * g + r]);
                    P[kb][cb][r] = lam;
                    mt = fmaxf(mt, lam);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float mn = fmaxf(m_run[cb], mt);
            const float a = __builtin_amdgcn_exp2f(m_run[cb] - mn);  // 0 on the first tile
            float ls = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(P[kb][cb][r] - mn);
                    P[kb][cb][r] = p;
                    ls += p;
                }
            l_run[cb] = __builtin_fmaf(l_run[cb], a, ls);
            m_run[cb] = mn;
            if (__any(a != 1.0f)) {  // the maximum moved for some column of the wave
#pragma unroll
                for (int db = 0; db < 8; ++db) O[cb][db] *= a;
            }
        }
        // O^T += V^T P^T over two 32-key steps.  MFMA k index e of lane group g is key
        // 32 st + 16 (e / 4) + 4 g + e % 4 on both operands; P as bf16 hi + lo.
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bf16x8_t ph[2], pl[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int j = 0; j < 8; j += 2) {  // two at a time: one packed conversion each
                    const f32x2_t x = {P[2 * st + j / 4][cb][j % 4], P[2 * st + j / 4][cb][j % 4 + 1]};
                    const bf16x2_t h = __builtin_convertvector(x, bf16x2_t);
                    const f32x2_t r = x - __builtin_convertvector(h, f32x2_t);
                    const bf16x2_t lo = __builtin_convertvector(r, bf16x2_t);
                    ph[cb][j] = h[0];
                    ph[cb][j + 1] = h[1];
                    pl[cb][j] = lo[0];
                    pl[cb][j + 1] = lo[1];
                }
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const s16x4_t v0 = vt_read(s.vt[buf], 32 * st + 4 * g, 16 * db, li);
                const s16x4_t v1 = vt_read(s.vt[buf], 32 * st + 16 + 4 * g, 16 * db, li);
                const s16x4_t both[2] = {v0, v1};
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, both);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    O[cb][db] = mfma16(av, ph[cb], O[cb][db]);
                    O[cb][db] = mfma16(av, pl[cb], O[cb][db]);
                }
            }
        }
    }
    // column totals (the 4 lanes of a column hold partial sums), then write
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        float lt = l_run[cb];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        if (qt[cb] < 0) continue;
        float* dst = A.out + (((int64_t)b * A.T + qt[cb]) * A.Hq + hq) * kD;
        const float inv = 1.0f / lt;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const f32x4_t o = O[cb][db];
            *reinterpret_cast<float4*>(dst + 16 * db + 4 * g) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
        }
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
    trace_point(0, st);
    hipLaunchKernelGGL(video_summary_kernel, dim3((A.Hkv + 7) / 8 + (A.Hq + 15) / 16, A.NB, batch), dim3(kThreads), 0,
                       st, A);
    trace_point(1, st);
    // as many query blocks per select workgroup as the score buffer allows
    if ((size_t)8 * A.NB * sizeof(float) <= (size_t)kVideoScoreLds) launch_video_select<8>(A, batch, st);
    else if ((size_t)4 * A.NB * sizeof(float) <= (size_t)kVideoScoreLds) launch_video_select<4>(A, batch, st);
    else if ((size_t)2 * A.NB * sizeof(float) <= (size_t)kVideoScoreLds) launch_video_select<2>(A, batch, st);
    else launch_video_select<1>(A, batch, st);
    trace_point(2, st);
    hipLaunchKernelGGL((video_attend_kernel<false>), dim3((unsigned)ceil_div(A.NB, kVideoPair), A.Hq, batch),
                       dim3(kThreads), 0, st, A);
    trace_point(3, st);
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
    hipLaunchKernelGGL((video_attend_kernel<true>), dim3((unsigned)ceil_div(A.NB, kVideoPair), A.Hq, batch),
                       dim3(kThreads), 0, st, A);
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}
