// lod_decode.hip -- LoD decode (subsystems b, c, d) and the dense decode baseline.
//
// "Queries start by scoring themselves against the low resolution centroids. We take
// the top eight ... score the query against those page summaries ... take the top two
// pages ... apply exact attention to these, as well as the most recent block sliding
// window ... and one or more sink tokens.  We combine the exactly attended KV pairs
// with a coarse remainder in a single softmax" ("Level of Detail Attention",
// How It Works).
//
// Three launches per call, all on the caller's stream:
//  1. scan    grid (slices + window tiles, KV heads, batch).  A slice workgroup streams
//             a contiguous run of group summaries (mean keys, then mean values) of one
//             (sequence, KV head) through LDS for all g query heads of that KV head.
//             Ranking scores are the canonical fp32 fma chain (one lane per (group,
//             head), query in registers).  Each head's local top-k groups become
//             candidates and are left out of the slice's coarse softmax partial; every
//             other non-empty group adds exp(scale*r + ln n) * vbar.  Every global top-k
//             group is in its slice's local top-k, so one pass over the summaries
//             suffices.  Window workgroups do exact tiles of the block window and the
//             sinks.
//  2. open    grid (top_groups, query heads, batch).  Merges the candidates into the
//             global top-k, scores the pages of opened group i, opens the top pages,
//             attends their rows exactly, adds unopened pages as coarse terms, and adds
//             back the coarse terms of candidates that lost the global ranking.
//  3. combine grid (query heads, batch).  Log-sum-exp merge of every partial state.
// Partial states are (o[d] = sum w v, m, l) relative to their own max m.
#include "lod_device.h"

namespace lodi {

constexpr int kKS = kD + 4;  // padded LDS row (floats)

struct DecodeArgs {
    const void* k;
    const void* v;
    int64_t sb, st, sh;
    const char* index;
    lod_index_layout_t L;
    int max_chunks;
    const void* q;
    const int32_t* seq_lens;
    int max_seq_len;
    float* out;
    int32_t* sel_groups;
    int32_t* sel_pages;
    float* part;
    uint64_t* cand;
    int Hq, Hkv, G, TG, TP, W, n_sink;
    float scale;
    int slice, nslice, nwin, nslot;
    // query rows: with seq_lens, row r is sequence r at position seq_lens[r]-1 (decode);
    // without, row r is sequence seq0 + r / rows_per_seq at position pos0 + r % rows_per_seq
    int seq0, rows_per_seq, pos0;
};

__device__ __forceinline__ void row_info(const DecodeArgs& A, int row, int& seq, int& p);

__device__ __forceinline__ int query_pos(const int32_t* seq_lens, int b, int max_seq_len) {
    int s = seq_lens[b];
    s = s < 1 ? 1 : (s > max_seq_len ? max_seq_len : s);
    return s - 1;
}
__device__ __forceinline__ int nbuilt(int p, int W) {
    int nb = p / kChunk - W / kChunk + 1;
    return nb < 0 ? 0 : nb;
}
__device__ __forceinline__ void row_info(const DecodeArgs& A, int row, int& seq, int& p) {
    if (A.seq_lens) {
        seq = row;
        p = query_pos(A.seq_lens, row, A.max_seq_len);
    } else {
        seq = A.seq0 + row / A.rows_per_seq;
        p = A.pos0 + row % A.rows_per_seq;
    }
}

// Stage n rows (row stride in elements) into an fp32 LDS tile.
template <typename T>
__device__ __forceinline__ void stage_rows(float (*dst)[kKS], const T* base, int64_t stride, int n) {
    constexpr int P16 = Elt<T>::kPer16;
    constexpr int CPR = kD / P16;
    for (int c = threadIdx.x; c < n * CPR; c += kThreads) {
        const int r = c / CPR, col = c % CPR;
        const uint4 u = *reinterpret_cast<const uint4*>(base + (int64_t)r * stride + col * P16);
        float f[P16];
        Elt<T>::unpack(u, f);
#pragma unroll
        for (int e = 0; e < P16; e += 4)
            *reinterpret_cast<float4*>(&dst[r][col * P16 + e]) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
    }
}

// Reduction over the kThreads/HG threads of one head (max or sum), result in all of them.
template <int HG, bool MAX>
__device__ __forceinline__ float head_allreduce(float v, float* red) {
    constexpr int TPH = kThreads / HG;
    constexpr int W = TPH < 64 ? TPH : 64;
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) {
        const float o = __shfl_xor(v, m, 64);
        v = MAX ? fmaxf(v, o) : v + o;
    }
    if constexpr (TPH > 64) {
        constexpr int WPH = TPH / 64;
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        __syncthreads();
        if (lane == 0) red[wave] = v;
        __syncthreads();
        const int h = threadIdx.x / TPH;
        float r = red[h * WPH];
#pragma unroll
        for (int i = 1; i < WPH; ++i) r = MAX ? fmaxf(r, red[h * WPH + i]) : r + red[h * WPH + i];
        v = r;
    }
    return v;
}

// Canonical ranking chains: lam_h[r] = fma chain of q_h . k_r over t = 0..d-1.
template <int HG>
__device__ __forceinline__ void score_tile(const float (*tk)[kKS], int n, const float* qr,
                                           float* lam_h, int li) {
    constexpr int TPH = kThreads / HG;
    for (int r0 = li; r0 < n; r0 += 2 * TPH) {
        const int r1 = r0 + TPH;
        const bool has1 = r1 < n;
        const float* k0 = tk[r0];
        const float* k1 = tk[has1 ? r1 : r0];
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int t = 0; t < kD; t += 4) {
            const float4 x0 = *reinterpret_cast<const float4*>(k0 + t);
            const float4 x1 = *reinterpret_cast<const float4*>(k1 + t);
            a0 = __builtin_fmaf(qr[t], x0.x, a0);
            a1 = __builtin_fmaf(qr[t], x1.x, a1);
            a0 = __builtin_fmaf(qr[t + 1], x0.y, a0);
            a1 = __builtin_fmaf(qr[t + 1], x1.y, a1);
            a0 = __builtin_fmaf(qr[t + 2], x0.z, a0);
            a1 = __builtin_fmaf(qr[t + 2], x1.z, a1);
            a0 = __builtin_fmaf(qr[t + 3], x0.w, a0);
            a1 = __builtin_fmaf(qr[t + 3], x1.w, a1);
        }
        lam_h[r0] = a0;
        if (has1) lam_h[r1] = a1;
    }
}

template <int HG>
struct ScanSmem {
    float tk[kTile][kKS];
    float tv[kTile][kKS];
    float lam[HG][4 * kTile];
    float red[kThreads / 64];
    uint64_t ckey[HG][kMaxTG];
};

// Thread roles inside a head (TPH = 256/HG threads): scoring rows li, li+TPH, ...;
// PV: dims 4*db..4*db+3 over rows rp, rp+RP, ... (RP = TPH/32 row phases).
template <int HG>
struct Roles {
    static constexpr int TPH = kThreads / HG;
    static constexpr int RP = TPH / 32;
    int h, li, db, rp;
    __device__ Roles() {
        h = threadIdx.x / TPH;
        li = threadIdx.x % TPH;
        db = li % 32;
        rp = li / 32;
    }
};

template <typename T>
__device__ __forceinline__ void load_q(float* qr, const void* q, int64_t row) {
    const T* qp = reinterpret_cast<const T*>(q) + row * kD;
#pragma unroll
    for (int t = 0; t < kD; ++t) qr[t] = Elt<T>::to_f32(qp[t]);
}

// Finish a workgroup's partial state: sum PV row phases and write (o, m, l).
template <int HG>
__device__ void write_partial(ScanSmem<HG>& s, const Roles<HG>& R, float* o, float m, float l,
                              float* dst_head0, int64_t head_stride, bool normalise = false) {
    constexpr int RP = Roles<HG>::RP;
    float* scratch = &s.tk[0][0];
    if constexpr (RP > 1) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) scratch[(R.h * RP + R.rp) * kD + 4 * R.db + e] = o[e];
        __syncthreads();
        if (R.rp == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a = scratch[(R.h * RP) * kD + 4 * R.db + e];
                for (int k = 1; k < RP; ++k) a += scratch[(R.h * RP + k) * kD + 4 * R.db + e];
                o[e] = a;
            }
        }
    }
    if (R.rp == 0) {
        float* dst = dst_head0 + (int64_t)R.h * head_stride;
        if (normalise) {
            const float inv = 1.0f / l;
            *reinterpret_cast<float4*>(dst + 4 * R.db) =
                make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
        } else {
            *reinterpret_cast<float4*>(dst + 4 * R.db) = make_float4(o[0], o[1], o[2], o[3]);
            if (R.db == 0) { dst[kD] = m; dst[kD + 1] = l; }
        }
    }
}

// Exact rows [r0, r1) of one (sequence, KV head) with online softmax across tiles.
template <typename T, int HG>
__device__ void exact_rows(ScanSmem<HG>& s, const Roles<HG>& R, const float* qr, const T* kb,
                           const T* vb, int64_t st, int r0, int r1, float scale, float& m_run,
                           float& l_run, float* o) {
    constexpr int TPH = Roles<HG>::TPH, RP = Roles<HG>::RP;
    for (int base = r0; base < r1; base += kTile) {
        const int n = min(kTile, r1 - base);
        stage_rows<T>(s.tk, kb + (int64_t)base * st, st, n);
        stage_rows<T>(s.tv, vb + (int64_t)base * st, st, n);
        __syncthreads();
        score_tile<HG>(s.tk, n, qr, s.lam[R.h], R.li);
        float mx = -INFINITY;
        for (int r = R.li; r < n; r += TPH) {
            const float lv = scale * s.lam[R.h][r];
            s.lam[R.h][r] = lv;
            mx = fmaxf(mx, lv);
        }
        mx = head_allreduce<HG, true>(mx, s.red);
        const float m_new = fmaxf(m_run, mx);
        float ls = 0.0f;
        for (int r = R.li; r < n; r += TPH) {
            const float w = softmax_exp(s.lam[R.h][r] - m_new);
            s.lam[R.h][r] = w;
            ls += w;
        }
        ls = head_allreduce<HG, false>(ls, s.red);
        const float alpha = m_run == -INFINITY ? 0.0f : softmax_exp(m_run - m_new);
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] *= alpha;
        __syncthreads();
        for (int r = R.rp; r < n; r += RP) {
            const float w = s.lam[R.h][r];
            const float4 vv = *reinterpret_cast<const float4*>(&s.tv[r][4 * R.db]);
            o[0] = __builtin_fmaf(w, vv.x, o[0]);
            o[1] = __builtin_fmaf(w, vv.y, o[1]);
            o[2] = __builtin_fmaf(w, vv.z, o[2]);
            o[3] = __builtin_fmaf(w, vv.w, o[3]);
        }
        __syncthreads();
    }
}

template <typename T, int HG>
__global__ __launch_bounds__(kThreads) void decode_scan_kernel(DecodeArgs A) {
    __shared__ ScanSmem<HG> s;
    const Roles<HG> R;
    constexpr int TPH = Roles<HG>::TPH, RP = Roles<HG>::RP;
    const int kvh = blockIdx.y, b = blockIdx.z;  // b: query row
    int seq, p;
    row_info(A, b, seq, p);
    const int nb = nbuilt(p, A.W);
    const int ng = nb * A.G;
    const int64_t unit = (int64_t)seq * A.Hkv + kvh;
    const int hq0 = kvh * HG;
    float* part0 = A.part + ((int64_t)(b * A.Hq + hq0) * A.nslot + blockIdx.x) * kPartStride;
    const int64_t head_stride = (int64_t)A.nslot * kPartStride;

    float qr[kD];
    load_q<T>(qr, A.q, (int64_t)b * A.Hq + hq0 + R.h);
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    if ((int)blockIdx.x < A.nslice) {
        // ---------------- slice of group summaries
        const int g0 = blockIdx.x * A.slice;
        const int cnt = min(A.slice, ng - g0);
        uint64_t* cand = A.cand + ((int64_t)(b * A.Hq + hq0) * A.nslice + blockIdx.x) * A.TG;
        const int64_t cand_head_stride = (int64_t)A.nslice * A.TG;
        if (cnt <= 0) {
            for (int e = threadIdx.x; e < HG * A.TG; e += kThreads)
                cand[(e / A.TG) * cand_head_stride + e % A.TG] = 0;
            write_partial<HG>(s, R, o, m_run, l_run, part0, head_stride);
            return;
        }
        const T* gk = reinterpret_cast<const T*>(A.index + A.L.gk) + (unit * A.max_chunks * A.G + g0) * kD;
        const T* gv = reinterpret_cast<const T*>(A.index + A.L.gv) + (unit * A.max_chunks * A.G + g0) * kD;
        const float* gln = reinterpret_cast<const float*>(A.index + A.L.gln) + unit * A.max_chunks * A.G + g0;
        // 1. ranking scores of every group of the slice, all heads
        for (int base = 0; base < cnt; base += kTile) {
            const int n = min(kTile, cnt - base);
            stage_rows<T>(s.tk, gk + (int64_t)base * kD, kD, n);
            __syncthreads();
            score_tile<HG>(s.tk, n, qr, s.lam[R.h] + base, R.li);
            __syncthreads();
        }
        // 2. local top-k per head (one wave per head); candidates leave the coarse sum
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        for (int h = wave; h < HG; h += kThreads / 64) {
            uint64_t kk[4];
            float lnn[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = lane + 64 * k;
                lnn[k] = r < cnt ? gln[r] : -INFINITY;
                kk[k] = (r < cnt && lnn[k] != -INFINITY) ? rank_key(s.lam[h][r], (uint32_t)(g0 + r)) : 0;
            }
            int taken = 0;
            int round = 0;
            for (; round < A.TG; ++round) {
                uint64_t best = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (!(taken >> k & 1) && kk[k] > best) best = kk[k];
                const uint64_t wb = wave_max_u64(best);
                if (wb == 0) break;
                if (lane == 0) s.ckey[h][round] = wb;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (kk[k] == wb) taken |= 1 << k;
            }
            if (lane == 0)
                for (int k = round; k < A.TG; ++k) s.ckey[h][k] = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = lane + 64 * k;
                if (r < cnt)
                    s.lam[h][r] = ((taken >> k & 1) || lnn[k] == -INFINITY)
                                      ? -INFINITY
                                      : A.scale * s.lam[h][r] + lnn[k];
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < HG * A.TG; e += kThreads)
            cand[(e / A.TG) * cand_head_stride + e % A.TG] = s.ckey[e / A.TG][e % A.TG];
        // 3. coarse softmax partial over the remaining groups
        float mx = -INFINITY;
        for (int r = R.li; r < cnt; r += TPH) mx = fmaxf(mx, s.lam[R.h][r]);
        mx = head_allreduce<HG, true>(mx, s.red);
        float ls = 0.0f;
        for (int r = R.li; r < cnt; r += TPH) {
            const float lv = s.lam[R.h][r];
            const float w = (lv == -INFINITY) ? 0.0f : softmax_exp(lv - mx);
            s.lam[R.h][r] = w;
            ls += w;
        }
        ls = head_allreduce<HG, false>(ls, s.red);
        m_run = mx;
        l_run = ls;
        __syncthreads();
        for (int base = 0; base < cnt; base += kTile) {
            const int n = min(kTile, cnt - base);
            stage_rows<T>(s.tv, gv + (int64_t)base * kD, kD, n);
            __syncthreads();
            for (int r = R.rp; r < n; r += RP) {
                const float w = s.lam[R.h][base + r];
                const float4 vv = *reinterpret_cast<const float4*>(&s.tv[r][4 * R.db]);
                o[0] = __builtin_fmaf(w, vv.x, o[0]);
                o[1] = __builtin_fmaf(w, vv.y, o[1]);
                o[2] = __builtin_fmaf(w, vv.z, o[2]);
                o[3] = __builtin_fmaf(w, vv.w, o[3]);
            }
            __syncthreads();
        }
        write_partial<HG>(s, R, o, m_run, l_run, part0, head_stride);
        return;
    }

    // ---------------- sinks (window block 0) and window tiles
    const int w = blockIdx.x - A.nslice;
    int r0, r1;
    if (w == 0) {
        r0 = 0;
        r1 = min(A.n_sink, nb * kChunk);  // with nb == 0 the window already covers them
        r1 = min(r1, p + 1);
    } else {
        r0 = nb * kChunk + (w - 1) * kTile;
        r1 = min(r0 + kTile, p + 1);
    }
    if (r1 > r0) {
        const T* kb = reinterpret_cast<const T*>(A.k) + seq * A.sb + kvh * A.sh;
        const T* vb = reinterpret_cast<const T*>(A.v) + seq * A.sb + kvh * A.sh;
        exact_rows<T, HG>(s, R, qr, kb, vb, A.st, r0, r1, A.scale, m_run, l_run, o);
    }
    write_partial<HG>(s, R, o, m_run, l_run, part0, head_stride);
}

// ---------------------------------------------------------------------------- open

constexpr int kBatch = 64;  // items per online-softmax batch in the open kernel

template <typename T>
struct OpenSmem {
    float qs[kD];
    uint64_t sel[kMaxTG];
    int nsel;
    int npg, ps0, c, nex;
    float pr[kPage];
    int prank[kPage];  // rank of each page of the group (-1: not opened)
    int pst[kPage + 1];
    int ipos[kChunk];  // exact positions of opened pages
    int bpos[kBatch];  // batch items: position (exact) or -1 (coarse)
    float blam[kBatch];
    float bw[kBatch];
    const T* bv[kBatch];
    int bn;
    float ored[16][kD];
};

// 8 consecutive elements of a row starting at element 8*l16, as fp32.
template <typename T>
__device__ __forceinline__ void load8(const T* row, int l16, float* f);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* row, int l16, float* f) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + 8 * l16);
    Elt<bf16_t>::unpack(u, f);
}
template <>
__device__ __forceinline__ void load8<float>(const float* row, int l16, float* f) {
    const uint4 u0 = *reinterpret_cast<const uint4*>(row + 8 * l16);
    const uint4 u1 = *reinterpret_cast<const uint4*>(row + 8 * l16 + 4);
    Elt<float>::unpack(u0, f);
    Elt<float>::unpack(u1, f + 4);
}

// Online-softmax step over the current batch (s.bn items in s.bpos / s.blam / s.bv).
template <typename T>
__device__ void open_batch(OpenSmem<T>& s, const float* q8, const T* kb, const T* vb, int64_t st,
                           float scale, float& m_run, float& l_run, float* o8) {
    const int sg = threadIdx.x >> 4, l16 = threadIdx.x & 15;
    const int n = s.bn;
    for (int it = sg; it < n; it += 16) {
        const int pos = s.bpos[it];
        if (pos >= 0) {
            float kf[8];
            load8<T>(kb + (int64_t)pos * st, l16, kf);
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = __builtin_fmaf(q8[e], kf[e], a);
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) a += __shfl_xor(a, m, 64);
            if (l16 == 0) s.blam[it] = scale * a;
        }
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int it = 0; it < n; ++it) mx = fmaxf(mx, s.blam[it]);
    const float m_new = fmaxf(m_run, mx);
    if (threadIdx.x < n) s.bw[threadIdx.x] = softmax_exp(s.blam[threadIdx.x] - m_new);
    __syncthreads();
    float ls = 0.0f;
    for (int it = 0; it < n; ++it) ls += s.bw[it];
    const float alpha = m_run == -INFINITY ? 0.0f : softmax_exp(m_run - m_new);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] *= alpha;
    for (int it = sg; it < n; it += 16) {
        const int pos = s.bpos[it];
        const T* vr = pos >= 0 ? vb + (int64_t)pos * st : s.bv[it];
        float vf[8];
        load8<T>(vr, l16, vf);
        const float w = s.bw[it];
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = __builtin_fmaf(w, vf[e], o8[e]);
    }
    __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(kThreads) void decode_open_kernel(DecodeArgs A) {
    __shared__ OpenSmem<T> s;
    const int i = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int HG = A.Hq / A.Hkv;
    const int kvh = hq / HG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = tid & 15;
    int seq, p;
    row_info(A, b, seq, p);  // b: query row
    const int nb = nbuilt(p, A.W);
    const int ng = nb * A.G;
    const int64_t unit = (int64_t)seq * A.Hkv + kvh;
    const int PS = A.L.page_slots;
    const int TPW = A.TP > 0 ? A.TP : 1;
    const T* qp = reinterpret_cast<const T*>(A.q) + ((int64_t)b * A.Hq + hq) * kD;
    if (tid < kD) s.qs[tid] = Elt<T>::to_f32(qp[tid]);
    float q8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q8[e] = Elt<T>::to_f32(qp[8 * l16 + e]);

    // 1. global top-k over the slices' candidates (wave 0): per-lane sorted top-16,
    //    then k rounds of a wave-wide max.
    const int nsl_used = ng > 0 ? (ng + A.slice - 1) / A.slice : 0;
    const int ncand = nsl_used * A.TG;
    const uint64_t* cand = A.cand + (int64_t)(b * A.Hq + hq) * A.nslice * A.TG;
    if (wave == 0) {
        uint64_t lst[kMaxTG];
#pragma unroll
        for (int k = 0; k < kMaxTG; ++k) lst[k] = 0;
        for (int k = lane; k < ncand; k += 64) {
            uint64_t x = cand[k];
#pragma unroll
            for (int e = 0; e < kMaxTG; ++e) {
                const uint64_t hi = lst[e] > x ? lst[e] : x;
                const uint64_t lo = lst[e] > x ? x : lst[e];
                lst[e] = hi;
                x = lo;
            }
        }
        int round = 0;
        for (; round < A.TG; ++round) {
            const uint64_t wb = wave_max_u64(lst[0]);
            if (wb == 0) break;
            if (lane == 0) s.sel[round] = wb;
            if (lst[0] == wb) {
#pragma unroll
                for (int e = 0; e < kMaxTG - 1; ++e) lst[e] = lst[e + 1];
                lst[kMaxTG - 1] = 0;
            }
        }
        if (lane == 0) s.nsel = round;
    }
    __syncthreads();
    const int nsel = s.nsel;
    const uint64_t kth = nsel == A.TG ? s.sel[A.TG - 1] : 0;
    const bool have = i < nsel;
    const uint32_t gid = have ? key_id(s.sel[i]) : 0;
    if (A.sel_groups && tid == 0) A.sel_groups[((int64_t)b * A.Hq + hq) * A.TG + i] = have ? (int)gid : -1;

    const T* kb = reinterpret_cast<const T*>(A.k) + seq * A.sb + kvh * A.sh;
    const T* vb = reinterpret_cast<const T*>(A.v) + seq * A.sb + kvh * A.sh;
    float o8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // 2. opened group i: page ranking, exact rows of opened pages, unopened pages coarse
    if (have) {
        const int c = gid / A.G, j = gid % A.G;
        const int16_t* meta = reinterpret_cast<const int16_t*>(A.index + A.L.meta) +
                              (unit * A.max_chunks + c) * A.L.meta_stride;
        const int16_t* gpg = meta;
        const int16_t* pst = meta + (A.G + 1);
        const int16_t* perm = meta + (A.G + 1) + (PS + 1);
        if (tid == 0) {
            s.ps0 = gpg[j];
            s.npg = gpg[j + 1] - gpg[j];
            s.c = c;
        }
        __syncthreads();
        const int npg = s.npg, ps0 = s.ps0;
        if (tid <= npg) s.pst[tid] = pst[ps0 + tid];
        const T* pk = reinterpret_cast<const T*>(A.index + A.L.pk) + (unit * A.max_chunks + c) * PS * kD;
        const T* pv = reinterpret_cast<const T*>(A.index + A.L.pv) + (unit * A.max_chunks + c) * PS * kD;
        const float* pln = reinterpret_cast<const float*>(A.index + A.L.pln) + (unit * A.max_chunks + c) * PS;
        if (wave == 0) {
            float r = 0.0f;
            if (A.TP > 0 && lane < npg) {
                const T* row = pk + (int64_t)(ps0 + lane) * kD;
                for (int t = 0; t < kD; t += Elt<T>::kPer16) {
                    float f[Elt<T>::kPer16];
                    Elt<T>::unpack(*reinterpret_cast<const uint4*>(row + t), f);
#pragma unroll
                    for (int e = 0; e < Elt<T>::kPer16; ++e) r = __builtin_fmaf(s.qs[t + e], f[e], r);
                }
            }
            if (lane < kPage) s.prank[lane] = (A.TP == 0 && lane < npg) ? 0 : -1;
            if (lane < npg) s.pr[lane] = r;
            if (A.TP > 0) {
                uint64_t key = lane < npg ? rank_key(r, (uint32_t)lane) : 0;
                const int nopen = npg < A.TP ? npg : A.TP;
                for (int k = 0; k < nopen; ++k) {
                    const uint64_t wb = wave_max_u64(key);
                    if (key == wb) { s.prank[lane] = k; key = 0; }
                }
            }
        }
        __syncthreads();
        if (A.sel_pages && tid < TPW) {
            int slot = -1;
            if (A.TP > 0)
                for (int e = 0; e < npg; ++e)
                    if (s.prank[e] == tid) slot = ps0 + e;
            A.sel_pages[(((int64_t)b * A.Hq + hq) * A.TG + i) * TPW + tid] = slot;
        }
        // exact positions of the opened pages (in page order)
        if (tid == 0) {
            int n = 0;
            for (int e = 0; e < npg; ++e) {
                if (s.prank[e] < 0) continue;
                for (int qq = s.pst[e]; qq < s.pst[e + 1]; ++qq) s.ipos[n++] = c * kChunk + perm[qq];
            }
            s.nex = n;
        }
        __syncthreads();
        const int nex = s.nex;
        for (int base = 0; base < nex; base += kBatch) {
            const int n = min(kBatch, nex - base);
            if (tid < n) s.bpos[tid] = s.ipos[base + tid];
            if (tid == 0) s.bn = n;
            __syncthreads();
            open_batch<T>(s, q8, kb, vb, A.st, A.scale, m_run, l_run, o8);
        }
        // unopened pages of the opened group: coarse terms
        if (tid == 0) {
            int n = 0;
            for (int e = 0; e < npg; ++e) {
                if (s.prank[e] >= 0) continue;
                s.bpos[n] = -1;
                s.blam[n] = A.scale * s.pr[e] + pln[ps0 + e];
                s.bv[n] = pv + (int64_t)(ps0 + e) * kD;
                ++n;
            }
            s.bn = n;
        }
        __syncthreads();
        if (s.bn > 0) open_batch<T>(s, q8, kb, vb, A.st, A.scale, m_run, l_run, o8);
    } else {
        if (A.sel_pages && tid < TPW)
            A.sel_pages[(((int64_t)b * A.Hq + hq) * A.TG + i) * TPW + tid] = -1;
    }

    // 3. add back the coarse terms of candidates that lost the global ranking
    if (kth != 0) {
        const T* gv = reinterpret_cast<const T*>(A.index + A.L.gv) + unit * A.max_chunks * A.G * kD;
        const float* gln = reinterpret_cast<const float*>(A.index + A.L.gln) + unit * A.max_chunks * A.G;
        for (int base = i; base < ncand; base += A.TG * kBatch) {
            // candidates base, base+TG, ... (up to kBatch of them) -> compact the losers
            __syncthreads();
            if (tid == 0) s.bn = 0;
            __syncthreads();
            if (tid < kBatch) {
                const int k = base + tid * A.TG;
                const uint64_t key = k < ncand ? cand[k] : 0;
                if (key != 0 && key < kth) {
                    const int slot = atomicAdd(&s.bn, 1);
                    const uint32_t g = key_id(key);
                    s.bpos[slot] = -1;
                    s.blam[slot] = A.scale * key_score(key) + gln[g];
                    s.bv[slot] = gv + (int64_t)g * kD;
                }
            }
            __syncthreads();
            if (s.bn > 0) {
                // canonical order of terms inside the batch does not matter for the
                // result beyond rounding; sort nothing, but make it deterministic:
                if (tid == 0) {
                    // insertion sort by group id (small batches)
                    const int n = s.bn;
                    for (int x = 1; x < n; ++x) {
                        const float lv = s.blam[x];
                        const T* vv = s.bv[x];
                        int y = x - 1;
                        while (y >= 0 && s.bv[y] > vv) {
                            s.blam[y + 1] = s.blam[y];
                            s.bv[y + 1] = s.bv[y];
                            --y;
                        }
                        s.blam[y + 1] = lv;
                        s.bv[y + 1] = vv;
                    }
                }
                __syncthreads();
                open_batch<T>(s, q8, kb, vb, A.st, A.scale, m_run, l_run, o8);
            }
        }
    }

    // 4. partial state of slot nslice + nwin + i
    const int sg = tid >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) s.ored[sg][8 * l16 + e] = o8[e];
    __syncthreads();
    float* dst = A.part + ((int64_t)(b * A.Hq + hq) * A.nslot + A.nslice + A.nwin + i) * kPartStride;
    if (tid < kD) {
        float a = 0.0f;
        for (int k = 0; k < 16; ++k) a += s.ored[k][tid];
        dst[tid] = a;
    }
    if (tid == 0) { dst[kD] = m_run; dst[kD + 1] = l_run; }
}

// ---------------------------------------------------------------------------- combine

__global__ __launch_bounds__(kD) void combine_kernel(const float* part, int nslot, float* out,
                                                     int Hq) {
    const int hq = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const float* ph = part + (int64_t)(b * Hq + hq) * nslot * kPartStride;
    float M = -INFINITY;
    for (int k = 0; k < nslot; ++k) M = fmaxf(M, ph[(int64_t)k * kPartStride + kD]);
    float L = 0.0f, O = 0.0f;
    for (int k = 0; k < nslot; ++k) {
        const float m = ph[(int64_t)k * kPartStride + kD];
        if (m == -INFINITY) continue;
        const float e = softmax_exp(m - M);
        L = __builtin_fmaf(ph[(int64_t)k * kPartStride + kD + 1], e, L);
        O = __builtin_fmaf(ph[(int64_t)k * kPartStride + t], e, O);
    }
    out[((int64_t)b * Hq + hq) * kD + t] = O / L;
}

// ---------------------------------------------------------------------------- dense decode

struct DenseArgs {
    const void* k;
    const void* v;
    int64_t sb, st, sh;
    const void* q;
    const int32_t* seq_lens;
    int max_seq_len;
    float* part;
    float* out;  // non-null: nsplit == 1 and rows write normalised outputs here
    int Hq, Hkv, rows_per_wg, nsplit;
    float scale;
    int seq0, rows_per_seq, pos0;  // row mapping when seq_lens is null (as DecodeArgs)
};

template <typename T, int HG>
__global__ __launch_bounds__(kThreads) void dense_decode_kernel(DenseArgs A) {
    __shared__ ScanSmem<HG> s;
    const Roles<HG> R;
    const int kvh = blockIdx.y, b = blockIdx.z;  // b: query row
    int seq, p;
    if (A.seq_lens) {
        seq = b;
        p = query_pos(A.seq_lens, b, A.max_seq_len);
    } else {
        seq = A.seq0 + b / A.rows_per_seq;
        p = A.pos0 + b % A.rows_per_seq;
    }
    const int hq0 = kvh * HG;
    float qr[kD];
    load_q<T>(qr, A.q, (int64_t)b * A.Hq + hq0 + R.h);
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;
    const int r0 = blockIdx.x * A.rows_per_wg;
    const int r1 = min(r0 + A.rows_per_wg, p + 1);
    if (r1 > r0) {
        const T* kb = reinterpret_cast<const T*>(A.k) + seq * A.sb + kvh * A.sh;
        const T* vb = reinterpret_cast<const T*>(A.v) + seq * A.sb + kvh * A.sh;
        exact_rows<T, HG>(s, R, qr, kb, vb, A.st, r0, r1, A.scale, m_run, l_run, o);
    }
    if (A.out) {  // one split per row: write the normalised output directly
        write_partial<HG>(s, R, o, m_run, l_run, A.out + ((int64_t)b * A.Hq + hq0) * kD, kD, true);
        return;
    }
    float* part0 = A.part + ((int64_t)(b * A.Hq + hq0) * A.nsplit + blockIdx.x) * kPartStride;
    write_partial<HG>(s, R, o, m_run, l_run, part0, (int64_t)A.nsplit * kPartStride);
}

// ---------------------------------------------------------------------------- host side

static int check_kv(const lod_params* p, const lod_kv& kv) {
    if (!kv.k || !kv.v || kv.stride_t <= 0 || kv.stride_h < 0 || kv.stride_b < 0) return LOD_ERR_ARG;
    const int per16 = p->kv_dtype == LOD_BF16 ? 8 : 4;
    if ((kv.stride_t | kv.stride_h | kv.stride_b) % per16 != 0) return LOD_ERR_ARG;
    return LOD_OK;
}

template <typename T, int HG>
static int launch_decode(const DecodeArgs& A, int rows, hipStream_t st) {
    if (A.nslice + A.nwin > 0)
        hipLaunchKernelGGL((decode_scan_kernel<T, HG>), dim3(A.nslice + A.nwin, A.Hkv, rows),
                           dim3(kThreads), 0, st, A);
    hipLaunchKernelGGL((decode_open_kernel<T>), dim3(A.TG, A.Hq, rows), dim3(kThreads), 0, st, A);
    hipLaunchKernelGGL(combine_kernel, dim3(A.Hq, rows), dim3(kD), 0, st, (const float*)A.part,
                       A.nslot, A.out, A.Hq);
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}

template <typename T, int HG>
static int launch_dense(const DenseArgs& A, float* out, int rows, hipStream_t st) {
    hipLaunchKernelGGL((dense_decode_kernel<T, HG>), dim3(A.nsplit, A.Hkv, rows), dim3(kThreads), 0,
                       st, A);
    if (!A.out)
        hipLaunchKernelGGL(combine_kernel, dim3(A.Hq, rows), dim3(kD), 0, st, (const float*)A.part,
                           A.nsplit, out, A.Hq);
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}


static int dispatch_decode(const lod_params* params, const DecodeArgs& A, int rows, hipStream_t st) {
    const int g = A.Hq / A.Hkv;
    if (params->kv_dtype == LOD_BF16) {
        switch (g) {
            case 1: return launch_decode<bf16_t, 1>(A, rows, st);
            case 2: return launch_decode<bf16_t, 2>(A, rows, st);
            case 4: return launch_decode<bf16_t, 4>(A, rows, st);
            default: return launch_decode<bf16_t, 8>(A, rows, st);
        }
    }
    switch (g) {
        case 1: return launch_decode<float, 1>(A, rows, st);
        case 2: return launch_decode<float, 2>(A, rows, st);
        case 4: return launch_decode<float, 4>(A, rows, st);
        default: return launch_decode<float, 8>(A, rows, st);
    }
}

static int dispatch_dense(const lod_params* params, const DenseArgs& A, float* out, int rows,
                          hipStream_t st) {
    const int g = A.Hq / A.Hkv;
    if (params->kv_dtype == LOD_BF16) {
        switch (g) {
            case 1: return launch_dense<bf16_t, 1>(A, out, rows, st);
            case 2: return launch_dense<bf16_t, 2>(A, out, rows, st);
            case 4: return launch_dense<bf16_t, 4>(A, out, rows, st);
            default: return launch_dense<bf16_t, 8>(A, out, rows, st);
        }
    }
    switch (g) {
        case 1: return launch_dense<float, 1>(A, out, rows, st);
        case 2: return launch_dense<float, 2>(A, out, rows, st);
        case 4: return launch_dense<float, 4>(A, out, rows, st);
        default: return launch_dense<float, 8>(A, out, rows, st);
    }
}

static void fill_decode_args(DecodeArgs& A, const lod_params* params, const lod_index* index,
                             const lod_index_layout_t& L, const lod_kv& kv, const DecodePlan& P,
                             void* ws) {
    A.k = kv.k; A.v = kv.v; A.sb = kv.stride_b; A.st = kv.stride_t; A.sh = kv.stride_h;
    A.index = reinterpret_cast<const char*>(index->mem);
    A.L = L;
    A.max_chunks = index->max_chunks;
    A.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + P.off_part);
    A.cand = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + P.off_cand);
    A.Hq = params->n_q_heads; A.Hkv = params->n_kv_heads; A.G = params->groups_per_chunk;
    A.TG = params->top_groups; A.TP = params->top_pages; A.W = params->window;
    A.n_sink = params->n_sink; A.scale = params->scale;
    A.slice = P.slice; A.nslice = P.nslice; A.nwin = P.nwin; A.nslot = P.nslot;
    A.seq0 = 0; A.rows_per_seq = 1; A.pos0 = 0;
}

// Prefill rows are processed in groups of this many rows per launch.
constexpr int kPrefillRows = 256;

}  // namespace lodi

using namespace lodi;

extern "C" int lod_attend_decode(const lod_params* params, const lod_index* index, lod_kv kv,
                                 const void* q, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_seq_len, float* out, int32_t* sel_groups,
                                 int32_t* sel_pages, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!index || !index->mem || !q || !seq_lens || !out || batch <= 0 || max_seq_len <= 0)
        return LOD_ERR_ARG;
    if ((rc = check_kv(params, kv)) != LOD_OK) return rc;
    if (batch != index->batch) return LOD_ERR_ARG;
    if (built_chunks(params, (int64_t)max_seq_len - 1) > index->max_chunks) return LOD_ERR_ARG;
    const lod_index_layout_t L = make_layout(params, index->batch, index->max_chunks);
    if (index->bytes < L.total) return LOD_ERR_WORKSPACE;
    const DecodePlan P = plan_decode(params, batch, max_seq_len);
    if (!ws || ws_bytes < P.bytes) return LOD_ERR_WORKSPACE;
    DecodeArgs A;
    fill_decode_args(A, params, index, L, kv, P, ws);
    A.q = q; A.seq_lens = seq_lens; A.max_seq_len = max_seq_len;
    A.out = out; A.sel_groups = sel_groups; A.sel_pages = sel_pages;
    return dispatch_decode(params, A, batch, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int lod_prefill_ws_bytes(const lod_params* params, int32_t batch, int32_t n_q,
                                    int32_t max_tokens, size_t* bytes) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!bytes || batch <= 0 || n_q <= 0 || max_tokens <= 0) return LOD_ERR_ARG;
    *bytes = plan_decode(params, n_q < kPrefillRows ? n_q : kPrefillRows, max_tokens).bytes;
    return LOD_OK;
}

extern "C" int lod_attend_prefill(const lod_params* params, const lod_index* index, lod_kv kv,
                                  const void* q, int32_t q_start, int32_t n_q, int32_t batch,
                                  float* out, int32_t* sel_groups, int32_t* sel_pages, void* ws,
                                  size_t ws_bytes, void* stream) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!index || !index->mem || !q || !out || batch <= 0 || n_q <= 0 || q_start < 0) return LOD_ERR_ARG;
    if (q_start % params->chunk_size != 0) return LOD_ERR_ARG;
    if ((rc = check_kv(params, kv)) != LOD_OK) return rc;
    if (batch != index->batch) return LOD_ERR_ARG;
    const int64_t end = (int64_t)q_start + n_q;
    if (end > INT32_MAX || built_chunks(params, end - 1) > index->max_chunks) return LOD_ERR_ARG;
    const lod_index_layout_t L = make_layout(params, index->batch, index->max_chunks);
    if (index->bytes < L.total) return LOD_ERR_WORKSPACE;
    const int rows_max = n_q < kPrefillRows ? n_q : kPrefillRows;
    const DecodePlan P = plan_decode(params, rows_max, (int32_t)end);
    if (!ws || ws_bytes < P.bytes) return LOD_ERR_WORKSPACE;
    DecodeArgs A;
    fill_decode_args(A, params, index, L, kv, P, ws);
    A.seq_lens = nullptr;
    A.max_seq_len = (int32_t)end;
    const int Hq = params->n_q_heads, TG = params->top_groups;
    const int TPW = params->top_pages > 0 ? params->top_pages : 1;
    const size_t eb = params->kv_dtype == LOD_BF16 ? 2 : 4;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (int b = 0; b < batch; ++b) {
        for (int r0 = 0; r0 < n_q; r0 += kPrefillRows) {
            const int rows = (n_q - r0) < kPrefillRows ? (n_q - r0) : kPrefillRows;
            const int64_t row0 = (int64_t)b * n_q + r0;
            A.q = reinterpret_cast<const char*>(q) + row0 * Hq * kD * eb;
            A.out = out + row0 * Hq * kD;
            A.sel_groups = sel_groups ? sel_groups + row0 * Hq * TG : nullptr;
            A.sel_pages = sel_pages ? sel_pages + row0 * Hq * TG * TPW : nullptr;
            A.seq0 = b;
            A.rows_per_seq = rows;
            A.pos0 = q_start + r0;
            if ((rc = dispatch_decode(params, A, rows, st)) != LOD_OK) return rc;
        }
    }
    return LOD_OK;
}

extern "C" int lod_dense_decode(const lod_params* params, lod_kv kv, const void* q,
                                const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                float* out, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!q || !seq_lens || !out || batch <= 0 || max_seq_len <= 0) return LOD_ERR_ARG;
    if ((rc = check_kv(params, kv)) != LOD_OK) return rc;
    const DensePlan P = plan_dense(params, batch, max_seq_len);
    if (!ws || ws_bytes < P.bytes) return LOD_ERR_WORKSPACE;
    DenseArgs A;
    A.k = kv.k; A.v = kv.v; A.sb = kv.stride_b; A.st = kv.stride_t; A.sh = kv.stride_h;
    A.q = q; A.seq_lens = seq_lens; A.max_seq_len = max_seq_len;
    A.part = reinterpret_cast<float*>(ws);
    A.out = nullptr;
    A.Hq = params->n_q_heads; A.Hkv = params->n_kv_heads;
    A.rows_per_wg = P.rows_per_wg; A.nsplit = P.nsplit; A.scale = params->scale;
    A.seq0 = 0; A.rows_per_seq = 1; A.pos0 = 0;
    return dispatch_dense(params, A, out, batch, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int lod_dense_prefill(const lod_params* params, lod_kv kv, const void* q, int32_t q_start,
                                 int32_t n_q, int32_t batch, float* out, void* stream) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!q || !out || batch <= 0 || n_q <= 0 || q_start < 0) return LOD_ERR_ARG;
    if ((rc = check_kv(params, kv)) != LOD_OK) return rc;
    const int64_t end = (int64_t)q_start + n_q;
    if (end > INT32_MAX) return LOD_ERR_ARG;
    DenseArgs A;
    A.k = kv.k; A.v = kv.v; A.sb = kv.stride_b; A.st = kv.stride_t; A.sh = kv.stride_h;
    A.seq_lens = nullptr; A.max_seq_len = (int32_t)end;
    A.part = nullptr;
    A.Hq = params->n_q_heads; A.Hkv = params->n_kv_heads;
    A.rows_per_wg = (int)end; A.nsplit = 1; A.scale = params->scale;
    const size_t eb = params->kv_dtype == LOD_BF16 ? 2 : 4;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (int b = 0; b < batch; ++b) {
        const int64_t row0 = (int64_t)b * n_q;
        A.q = reinterpret_cast<const char*>(q) + row0 * A.Hq * kD * eb;
        A.out = out + row0 * A.Hq * kD;
        A.seq0 = b; A.rows_per_seq = n_q; A.pos0 = q_start;
        if ((rc = dispatch_dense(params, A, A.out, n_q, st)) != LOD_OK) return rc;
    }
    return LOD_OK;
}
