// lod_decode.hip -- LoD decode (subsystems b, c, d) and the dense decode baseline.
//
// A query first ranks the group centroids and opens the best groups, then ranks the
// page summaries inside those groups and opens the best pages; the keys of opened pages,
// the recent block window and the sink tokens are attended exactly, and everything else
// enters the same softmax as count-weighted means ("Level of Detail Attention", How It
// Works).
//
// bf16 caches: two launches per call, on the caller's stream.
//  1. scan    grid (KV heads, batch, scan workgroups per unit).  A unit is a (sequence,
//             KV head); its workgroups stream equal runs of its 64-row tiles (the group
//             summaries of every summarised chunk, then the sinks and the block window)
//             through LDS for all query heads of the KV head: MFMA scores (written out
//             for the selection), online softmax over every group (coarse, logit
//             scale*S + ln n) and exact row, MFMA value sums, one partial state each.
//  2. open    grid (query heads, batch).  Exact top groups from the stored scores and
//             their error bounds (only candidates near the cut run the canonical chain),
//             top pages, the opened pages' rows exactly and the unopened pages' means,
//             then the merge of the scan's partials, from which the opened groups' coarse
//             terms are subtracted with the very logits the scan used.
// fp32 caches (VALU): slice workgroups with canonical chains keep each slice's local top
// groups out of their coarse partial and an open step adds back those that lose the
// global ranking; the dense baseline and row-by-row prefill reuse these kernels.
// Partial states are (o[d] = sum w v, m, l) relative to their own max m.
#include <mutex>

#include "lod_device.h"
#include "lod_mfma.h"

namespace lodi {

constexpr int kKS = kD + 4;  // padded LDS row (floats)

struct DecodeArgs {
    const void* k;
    const void* v;
    int64_t sb, st, sh;
    const int32_t* btab;  // paged view: block table [batch][maxb], else null
    int bshift, maxb;
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
    float* score;      // bf16: MFMA ranking scores [rows][Hq][score_stride]
    int score_stride;
    int Hq, Hkv, G, TG, TP, W, n_sink;
    float scale;
    int drop;  // 1: no coarse remainder (sparsity ablation)
    int q4;    // 1: opened pages decoded from the index's 4-bit codes (three-tier INT4)
    int slice, nslice, nwin, nslot;
    // query rows: with seq_lens, row r is sequence r at position seq_lens[r]-1 (decode);
    // without, row r is sequence seq0 + r / rows_per_seq at position pos0 + r % rows_per_seq
    int seq0, rows_per_seq, pos0;
};

__device__ __forceinline__ void row_info(const DecodeArgs& A, int row, int& seq, int& p);

struct DenseArgs {
    const void* k;
    const void* v;
    int64_t sb, st, sh;
    const int32_t* btab;  // paged view: block table [batch][maxb], else null
    int bshift, maxb;
    const void* q;
    const int32_t* seq_lens;
    int max_seq_len;
    float* part;
    float* out;  // non-null: nsplit == 1 and rows write normalised outputs here
    int Hq, Hkv, rows_per_wg, nsplit;
    float scale;
    int seq0, rows_per_seq, pos0;  // row mapping when seq_lens is null (as DecodeArgs)
};

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

// Stage n rows (row r at row(r)) into an fp32 LDS tile.
template <typename T, typename RowPtr>
__device__ __forceinline__ void stage_rows_at(float (*dst)[kKS], RowPtr row, int n) {
    constexpr int P16 = Elt<T>::kPer16;
    constexpr int CPR = kD / P16;
    for (int c = threadIdx.x; c < n * CPR; c += kThreads) {
        const int r = c / CPR, col = c % CPR;
        const uint4 u = *reinterpret_cast<const uint4*>(row(r) + col * P16);
        float f[P16];
        Elt<T>::unpack(u, f);
#pragma unroll
        for (int e = 0; e < P16; e += 4)
            *reinterpret_cast<float4*>(&dst[r][col * P16 + e]) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
    }
}
// Stage n rows of a strided array (row stride in elements).
template <typename T>
__device__ __forceinline__ void stage_rows(float (*dst)[kKS], const T* base, int64_t stride, int n) {
    stage_rows_at<T>(dst, [&](int r) { return base + (int64_t)r * stride; }, n);
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
// Row x of K / V: krow(x), vrow(x) (cache positions).
template <typename T, int HG, typename KRow, typename VRow>
__device__ void exact_rows(ScanSmem<HG>& s, const Roles<HG>& R, const float* qr, KRow krow, VRow vrow,
                           int r0, int r1, float scale, float& m_run, float& l_run, float* o) {
    constexpr int TPH = Roles<HG>::TPH, RP = Roles<HG>::RP;
    for (int base = r0; base < r1; base += kTile) {
        const int n = min(kTile, r1 - base);
        stage_rows_at<T>(s.tk, [&](int r) { return krow(base + r); }, n);
        stage_rows_at<T>(s.tv, [&](int r) { return vrow(base + r); }, n);
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
        // 3. coarse softmax partial over the remaining groups (none without the remainder)
        if (A.drop) {
            write_partial<HG>(s, R, o, m_run, l_run, part0, head_stride);
            return;
        }
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
        const T* kh = reinterpret_cast<const T*>(A.k) + kvh * A.sh;
        const T* vh = reinterpret_cast<const T*>(A.v) + kvh * A.sh;
        exact_rows<T, HG>(s, R, qr, [&](int x) { return kh + kv_row_rt(A, seq, x); },
                          [&](int x) { return vh + kv_row_rt(A, seq, x); }, r0, r1, A.scale, m_run, l_run, o);
    }
    write_partial<HG>(s, R, o, m_run, l_run, part0, head_stride);
}

// ---------------------------------------------------------------------------- open + combine

// Wave-local ordering of LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kOpenBatch = 4;   // items per subgroup whose loads are issued together
constexpr int kOpenCand = 128;  // canonical re-scoring candidates kept per head
constexpr int kPartLds = kScanMaxSlots;  // scan partial states per head copied to LDS (bf16 path)
constexpr int kPartLdsFloats = (kPartLds * (kPartStride / 4) + 63) / 64 * 64 * 4;
constexpr int kMetaMax = 320;   // int16 entries of one chunk's meta row (>= meta_stride)
constexpr int kMetaRows = 2 * kMaxTG;  // meta rows in LDS: candidates prefetched when this few
constexpr int kSpecPages = 16 * kMetaRows;  // candidate pages scored ahead (at most 16 per group)
constexpr int kGPW = kMaxTG / 4;             // opened groups per wave (at most)
constexpr int kItemsPerWave = kGPW * kChunk; // exact rows of a wave's groups (two-tier bound)

template <typename T>
struct OpenSmem {
    alignas(16) int16_t meta[kMetaRows][kMetaMax];  // meta rows: prefetched candidates' or opened groups'
    float qs[kD];
    uint64_t sel[kMaxTG];
    int nsel;
    int ex[4][kItemsPerWave];  // per wave: exact positions of the opened pages
    int nex[4];
    int cp[4][kGPW * kPage];   // per wave: unopened pages as (group slot k << 8 | page e)
    float cl[4][kGPW * kPage]; // and their logits
    int ncp[4];
    float sm[16], sl[16];      // subgroup states
    float so[16][kD];
    float scan_m, scan_l;      // merged state of the scan workgroups' partials
    float scan_o[kD];
    // selection from MFMA scores (bf16 path)
    alignas(16) float wl[4][4];  // per wave: its largest lower bounds (at most 4)
    int ncand;
    int32_t cg[kOpenCand];     // candidates: group id, canonical score, MFMA score, ln n,
    float cs[kOpenCand];       // page range (first slot | count << 16), first entry in pr
    float cS[kOpenCand];
    int32_t cP[kOpenCand], cpo[kOpenCand + 1];
    float pr[kSpecPages];      // canonical scores and ln n of the candidates' pages (when
    float pl[kSpecPages];      // scored ahead of the group ranking: pscore_ready)
    int pscore_ready;
    int mrow[kMaxTG];          // meta row (in s.meta) of opened group i
    int meta_ready;            // meta rows were prefetched (bf16 path)
    uint64_t red[4];
    float sub_S[kMaxTG];       // opened groups' MFMA scores in the scan
    float sub_lam[kMaxTG];     // and their coarse logits there (subtracted)
    alignas(16) float plds[kPartLdsFloats];  // the scan partial states (bf16 path), when they fit
};

// Merge of the scan workgroups' partial states of one head by waves 2-3 (one dimension
// per thread; loads issued 16 slots at a time) into s.scan_*.
template <typename T>
__device__ __forceinline__ void open_merge_scan(OpenSmem<T>& s, const float* part, int nscan) {
    const int tid = threadIdx.x;
    if (tid < 2 * 64) return;
    const int d = tid - 128;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int k0 = 0; k0 < nscan; k0 += 16) {
        float mm[16], ll[16], oo[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int k = k0 + x;
            mm[x] = -INFINITY;
            if (k < nscan) {
                const float* pp = part + (int64_t)k * kPartStride;
                mm[x] = pp[kD];
                ll[x] = pp[kD + 1];
                oo[x] = pp[d];
            }
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            if (mm[x] == -INFINITY) continue;
            const float mn = fmaxf(M, mm[x]);
            const float a = softmax_exp(M - mn), e = softmax_exp(mm[x] - mn);
            L = __builtin_fmaf(ll[x], e, L * a);
            O = __builtin_fmaf(oo[x], e, O * a);
            M = mn;
        }
    }
    s.scan_o[d] = O;
    if (d == 0) { s.scan_m = M; s.scan_l = L; }
}

// Pages of the opened groups s.sel[0..nsel) and the exact attention over them.  Wave w
// handles opened groups w, w+4, ...: all of its groups' meta rows, then all of their
// page rankings (one lane per (group, page), 16-lane segmented top-k), then the item
// lists, so the dependent global round trips are few.  Every 16-lane subgroup then
// streams items with its loads batched into its online-softmax state st.
// Block update of a 16-lane online softmax with up to OB terms (logit lam[x], -inf: none;
// value: 8 elements of this lane packed in vp[x]): one rescale to the new maximum, then
// the weighted values.
template <typename T, int OB, int U>
__device__ __forceinline__ void open_block_add(Online& st, const float* lam, const u32x4_t (*vp)[U]) {
    constexpr int P16 = Elt<T>::kPer16;
    float mb = -INFINITY;
#pragma unroll
    for (int x = 0; x < OB; ++x) mb = fmaxf(mb, lam[x]);
    if (mb == -INFINITY) return;
    const float mn = fmaxf(st.m, mb);
    const float a = softmax_exp(st.m - mn);  // st.m = -inf -> 0
    st.l *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[e] *= a;
#pragma unroll
    for (int x = 0; x < OB; ++x) {
        if (lam[x] == -INFINITY) continue;  // no term (its value registers may repeat a row)
        const float w = softmax_exp(lam[x] - mn);
        float vf[8];
#pragma unroll
        for (int u = 0; u < U; ++u) Elt<T>::unpack(vp[x][u], vf + u * P16);
        st.l += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[e] = __builtin_fmaf(w, vf[e], st.o[e]);
    }
    st.m = mn;
}

// DROP: no coarse remainder, so unopened pages add no terms (a run-time flag on the fp32
// path, DROP_RT; a compile-time one on the bf16 path).
// Q4 (bf16 only): the opened pages' rows are decoded from the index's 4-bit codes
// (fma(scale, code, group mean)) instead of read from the cache.
template <typename T, int OB, bool PAGED, bool DROP_RT = true, bool DROP = false, bool Q4 = false>
__device__ void open_pages(const DecodeArgs& A, OpenSmem<T>& s, int nsel, int seq, int kvh, int64_t head,
                           const float* q8, Online& st) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, sgw = lane >> 4;
    const int64_t unit = (int64_t)seq * A.Hkv + kvh;
    const int PS = A.L.page_slots;
    const int TPW = A.TP > 0 ? A.TP : 1;
    // head kvh of sequence seq; the row of a position adds kv_pos
    const T* kh = reinterpret_cast<const T*>(A.k) + kvh * A.sh + kv_seq<PAGED>(A, seq);
    const T* vh = reinterpret_cast<const T*>(A.v) + kvh * A.sh + kv_seq<PAGED>(A, seq);
    const T* pk_u = reinterpret_cast<const T*>(A.index + A.L.pk) + unit * A.max_chunks * PS * kD;
    const T* pv_u = reinterpret_cast<const T*>(A.index + A.L.pv) + unit * A.max_chunks * PS * kD;
    const float* pln_u = reinterpret_cast<const float*>(A.index + A.L.pln) + unit * A.max_chunks * PS;
    const int16_t* meta_u = reinterpret_cast<const int16_t*>(A.index + A.L.meta) + unit * A.max_chunks * A.L.meta_stride;

    // meta rows of this wave's groups (all loads in flight together), unless prefetched
    const int ngw = (A.TG - wave + 3) / 4;  // group slots of this wave (k: group i = wave + 4k)
    const int ms16 = A.L.meta_stride / 8;   // 16-byte pieces per meta row
    // meta row of opened group i: rows of meta_stride entries in the flat LDS buffer
    int16_t* const mflat = &s.meta[0][0];
    auto mrowp = [&](int i) { return mflat + s.mrow[i] * A.L.meta_stride; };
    if (!s.meta_ready) {
        for (int x = lane; x < ngw * ms16; x += 64) {
            const int k = x / ms16, e = x % ms16, i = wave + 4 * k;
            if (i < nsel) {
                const int c = key_id(s.sel[i]) / A.G;
                *reinterpret_cast<uint4*>(mrowp(i) + e * 8) =
                    *reinterpret_cast<const uint4*>(meta_u + (int64_t)c * A.L.meta_stride + e * 8);
            }
        }
        wave_sync();
    }
    // page ranking: lane (k = lane/16, e = lane%16) scores page e of group i = wave+4k
    {
        const int k = lane >> 4, e = lane & 15, i = wave + 4 * k;
        int c = 0, j = 0, ps0 = 0, npg = 0;
        if (k < ngw && i < nsel) {
            const uint32_t gid = key_id(s.sel[i]);
            c = gid / A.G;
            j = gid % A.G;
            ps0 = mrowp(i)[j];
            npg = mrowp(i)[j + 1] - ps0;
        }
        float r = 0.0f;
        if (s.pscore_ready) {
            // scored ahead: candidate mrow[i], page e (item 16 * mrow[i] + e)
            if (e < npg) r = s.pr[16 * s.mrow[i] + e];
        } else if (A.TP > 0 && e < npg) {
            const T* row = pk_u + ((int64_t)c * PS + ps0 + e) * kD;
            constexpr int P16 = Elt<T>::kPer16;
            uint4 u[kD / P16];
#pragma unroll
            for (int x = 0; x < kD / P16; ++x) u[x] = *reinterpret_cast<const uint4*>(row + x * P16);
#pragma unroll
            for (int x = 0; x < kD / P16; ++x) {
                float f[P16];
                Elt<T>::unpack(u[x], f);
#pragma unroll
                for (int t = 0; t < P16; ++t) r = __builtin_fmaf(s.qs[x * P16 + t], f[t], r);
            }
        }
        const float lnp = e < npg ? (s.pscore_ready ? s.pl[16 * s.mrow[i] + e] : pln_u[(int64_t)c * PS + ps0 + e])
                                  : -INFINITY;
        int rank = (A.TP == 0 && e < npg) ? 0 : -1;
        if (A.TP > 0) {
            uint64_t key = e < npg ? rank_key(r, (uint32_t)e) : 0;
            const int nopen = npg < A.TP ? npg : A.TP;  // uniform within the 16-lane segment
            for (int t = 0; t < A.TP; ++t) {          // uniform trip count for the row reductions
                const uint64_t m = row16_max_u64(key);
                if (t < nopen && key == m && m != 0) { rank = t; key = 0; }
            }
        }
        // sel_pages: lane t of the segment writes the slot of rank t
        if (A.sel_pages) {
            const int seg0 = lane & ~15;
            int slot_of_rank = -1;
            for (int x = 0; x < 16; ++x) {
                const int rk = __shfl(rank, seg0 + x, 64);
                if (A.TP > 0 && rk == e) slot_of_rank = ps0 + x;
            }
            if (k < ngw && i < A.TG && e < TPW)
                A.sel_pages[(head * A.TG + i) * TPW + e] = i < nsel ? slot_of_rank : -1;
        }
        // item lists: unopened pages (coarse) and exact rows of opened pages
        const bool coarse = e < npg && rank < 0;
        const uint64_t cm = __ballot(coarse);
        if (coarse) {
            const int at = __popcll(cm & ((1ull << lane) - 1ull));
            s.cp[wave][at] = (k << 8) | e;
            s.cl[wave][at] = A.scale * r + lnp;
        }
        if (lane == 0) s.ncp[wave] = __popcll(cm);
        // exact rows: page e of group slot k contributes pst[e+1]-pst[e] rows
        const int16_t* pst = mrowp(i < kMaxTG ? i : 0) + (A.G + 1);
        const int16_t* perm = pst + (PS + 1);
        const int cnt = (e < npg && rank >= 0) ? pst[ps0 + e + 1] - pst[ps0 + e] : 0;
        int off = wave_incl_scan_i32(cnt);  // inclusive prefix over the wave's lanes
        const int total = __builtin_amdgcn_readlane(off, 63);
        off -= cnt;
        const int p0 = (e < npg && rank >= 0) ? pst[ps0 + e] : 0;
#pragma unroll
        for (int x = 0; x < kPage; ++x)  // a page holds at most kPage rows
            if (x < cnt) s.ex[wave][off + x] = (c * kChunk + perm[p0 + x]) | (Q4 ? k << 24 : 0);
        if (lane == 0) s.nex[wave] = total;
    }
    wave_sync();

    // exact rows of the wave's groups, then its coarse pages (subgroup sgw takes sgw, sgw+4, ...)
    const int nex = s.nex[wave];
    constexpr int P16 = Elt<T>::kPer16, U = 8 / P16;  // 16-byte pieces per 8 elements
    if constexpr (Q4) {
        // entries: position | group slot << 24; the slots' mean rows stay in registers
        const int64_t qrow0 = unit * A.max_chunks * kChunk;
        const uint8_t* q4k = reinterpret_cast<const uint8_t*>(A.index + A.L.q4k) + qrow0 * (kD / 2);
        const uint8_t* q4v = reinterpret_cast<const uint8_t*>(A.index + A.L.q4v) + qrow0 * (kD / 2);
        const float* q4ks = reinterpret_cast<const float*>(A.index + A.L.q4ks) + qrow0;
        const float* q4vs = reinterpret_cast<const float*>(A.index + A.L.q4vs) + qrow0;
        const bf16_t* gk_u = reinterpret_cast<const bf16_t*>(A.index + A.L.gk) + unit * A.max_chunks * A.G * kD;
        const bf16_t* gv_u = reinterpret_cast<const bf16_t*>(A.index + A.L.gv) + unit * A.max_chunks * A.G * kD;
        u32x4_t mk[kGPW], mv[kGPW];
#pragma unroll
        for (int k = 0; k < kGPW; ++k) {
            const int i = wave + 4 * k;
            const int64_t g = (k < ngw && i < nsel) ? (int64_t)key_id(s.sel[i]) : 0;
            mk[k] = *reinterpret_cast<const u32x4_t*>(gk_u + g * kD + 8 * l16);
            mv[k] = *reinterpret_cast<const u32x4_t*>(gv_u + g * kD + 8 * l16);
        }
        auto pick = [&](const u32x4_t* m, int k) {
            return k == 0 ? m[0] : (k == 1 ? m[1] : (k == 2 ? m[2] : m[3]));
        };
        auto decode8 = [&](uint32_t code, float sc, const u32x4_t& mean, float* f) {
            float mf[8];
            Elt<bf16_t>::unpack(mean, mf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int q = (int)((code >> (4 * e)) & 0xfu);
                f[e] = __builtin_fmaf(sc, (float)((q ^ 8) - 8), mf[e]);
            }
        };
        for (int base = 0; base < nex; base += 4 * OB) {
            uint32_t kc[OB], vc[OB];
            float ks[OB], vs[OB];
            int slot[OB];
#pragma unroll
            for (int x = 0; x < OB; ++x) {
                const int it = base + sgw + 4 * x;
                const int ent = it < nex ? s.ex[wave][it] : 0;
                const int64_t pos = ent & 0xffffff;
                slot[x] = ent >> 24;
                kc[x] = *reinterpret_cast<const uint32_t*>(q4k + pos * (kD / 2) + 4 * l16);
                vc[x] = *reinterpret_cast<const uint32_t*>(q4v + pos * (kD / 2) + 4 * l16);
                ks[x] = q4ks[pos];
                vs[x] = q4vs[pos];
            }
            float lam[OB];
#pragma unroll
            for (int x = 0; x < OB; ++x) {
                float kf[8];
                decode8(kc[x], ks[x], pick(mk, slot[x]), kf);
                float a = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) a = __builtin_fmaf(q8[e], kf[e], a);
                lam[x] = row16_sum_f32(a);
            }
            float mb = -INFINITY;
#pragma unroll
            for (int x = 0; x < OB; ++x) {
                lam[x] = base + sgw + 4 * x < nex ? A.scale * lam[x] : -INFINITY;
                mb = fmaxf(mb, lam[x]);
            }
            if (mb == -INFINITY) continue;
            const float mn = fmaxf(st.m, mb);
            const float a = softmax_exp(st.m - mn);
            st.l *= a;
#pragma unroll
            for (int e = 0; e < 8; ++e) st.o[e] *= a;
#pragma unroll
            for (int x = 0; x < OB; ++x) {
                if (lam[x] == -INFINITY) continue;
                const float w = softmax_exp(lam[x] - mn);
                float vf[8];
                decode8(vc[x], vs[x], pick(mv, slot[x]), vf);
                st.l += w;
#pragma unroll
                for (int e = 0; e < 8; ++e) st.o[e] = __builtin_fmaf(w, vf[e], st.o[e]);
            }
            st.m = mn;
        }
    } else {
        for (int base = 0; base < nex; base += 4 * OB) {
            // every item's row position first, then every row load: items past nex repeat
            // the last row (masked below), so no load sits behind a branch of its own,
            // where each item's LDS read was waited for before its loads were issued
            int ent[OB];
#pragma unroll
            for (int x = 0; x < OB; ++x) ent[x] = s.ex[wave][min(base + sgw + 4 * x, nex - 1)];
            u32x4_t kp[OB][U], vp[OB][U];  // rows kept packed until used
#pragma unroll
            for (int x = 0; x < OB; ++x) {
                const int64_t ro = kv_pos<PAGED>(A, seq, ent[x]);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    kp[x][u] = *reinterpret_cast<const u32x4_t*>(kh + ro + 8 * l16 + u * P16);
                    vp[x][u] = *reinterpret_cast<const u32x4_t*>(vh + ro + 8 * l16 + u * P16);
                }
            }
            // keeps the value loads here, in flight beside the key loads (the compiler
            // would otherwise sink them to their use, after the dot products)
            asm volatile("" ::: "memory");
            // block update of the subgroup's online softmax: dot products and their
            // reductions side by side, one rescale, then the weighted values
            float lam[OB];
#pragma unroll
            for (int x = 0; x < OB; ++x) {
                float kf[8];
#pragma unroll
                for (int u = 0; u < U; ++u) Elt<T>::unpack(kp[x][u], kf + u * P16);
                float a = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) a = __builtin_fmaf(q8[e], kf[e], a);
                lam[x] = a;
            }
#pragma unroll
            for (int x = 0; x < OB; ++x) lam[x] = row16_sum_f32(lam[x]);
#pragma unroll
            for (int x = 0; x < OB; ++x) lam[x] = base + sgw + 4 * x < nex ? A.scale * lam[x] : -INFINITY;
            open_block_add<T, OB, U>(st, lam, vp);
        }
    }
    const int ncp = (DROP || (DROP_RT && A.drop)) ? 0 : s.ncp[wave];  // unopened pages: coarse terms
    for (int base = 0; base < ncp; base += 4 * OB) {
        // as for the exact rows: the items' LDS entries first (past ncp: the last item,
        // masked), then every page row load
        int cpe[OB];
        float lam[OB];
#pragma unroll
        for (int x = 0; x < OB; ++x) {
            const int it = min(base + sgw + 4 * x, ncp - 1);
            cpe[x] = s.cp[wave][it];
            lam[x] = base + sgw + 4 * x < ncp ? s.cl[wave][it] : -INFINITY;
        }
        const T* rows[OB];
#pragma unroll
        for (int x = 0; x < OB; ++x) {
            const int k = cpe[x] >> 8, e = cpe[x] & 255, i = wave + 4 * k;
            const uint32_t gid = key_id(s.sel[i]);
            const int c = gid / A.G, ps0 = mrowp(i)[gid % A.G];
            rows[x] = pv_u + ((int64_t)c * PS + ps0 + e) * kD + 8 * l16;
        }
        u32x4_t vp[OB][U];
#pragma unroll
        for (int x = 0; x < OB; ++x)
#pragma unroll
            for (int u = 0; u < U; ++u) vp[x][u] = *reinterpret_cast<const u32x4_t*>(rows[x] + u * P16);
        asm volatile("" ::: "memory");  // the loads stay issued together, ahead of their use
        open_block_add<T, OB, U>(st, lam, vp);
    }
}

// Write the 16 subgroup states to LDS (before a barrier).
template <typename T>
__device__ __forceinline__ void open_stash(OpenSmem<T>& s, const Online& st) {
    const int tid = threadIdx.x, l16 = tid & 15, sg = tid >> 4;
    if (l16 == 0) { s.sm[sg] = st.m; s.sl[sg] = st.l; }
#pragma unroll
    for (int e = 0; e < 8; ++e) s.so[sg][8 * l16 + e] = st.o[e];
}

// One workgroup per (query row, query head) (fp32 path): the slices' local top-k
// candidates are merged into the global top-k, the opened groups are attended through
// their pages, losing candidates are added back as coarse terms, and the state is
// merged with the scan workgroups' partial states into the final output.
template <typename T, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_open_kernel(DecodeArgs A) {
    __shared__ OpenSmem<T> s;
    const int hq = blockIdx.x, b = blockIdx.y;
    const int HG = A.Hq / A.Hkv;
    const int kvh = hq / HG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, sgw = lane >> 4;
    int seq, p;
    row_info(A, b, seq, p);
    const int nb = nbuilt(p, A.W);
    const int ng = nb * A.G;
    const int64_t unit = (int64_t)seq * A.Hkv + kvh;
    const int64_t head = (int64_t)b * A.Hq + hq;
    const T* qp = reinterpret_cast<const T*>(A.q) + head * kD;
    if (tid < kD) s.qs[tid] = Elt<T>::to_f32(qp[tid]);
    float q8[8];
    load8<T>(qp, l16, q8);
    open_merge_scan(s, A.part + head * A.nslot * kPartStride, A.nslice + A.nwin);

    // 1. global top-k over the slices' candidates (wave 0)
    const int nsl_used = ng > 0 ? (ng + A.slice - 1) / A.slice : 0;
    const int ncand = nsl_used * A.TG;
    const uint64_t* cand = A.cand + head * A.nslice * A.TG;
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
    if (tid < kMaxTG) s.mrow[tid] = tid;
    if (tid == 0) { s.meta_ready = 0; s.pscore_ready = 0; }
    __syncthreads();
    const int nsel = s.nsel;
    const uint64_t kth = nsel == A.TG ? s.sel[A.TG - 1] : 0;
    if (A.sel_groups && tid < A.TG) A.sel_groups[head * A.TG + tid] = tid < nsel ? (int)key_id(s.sel[tid]) : -1;

    Online st;
    st.init();
    open_pages<T, kOpenBatch, PAGED>(A, s, nsel, seq, kvh, head, q8, st);

    // add back the coarse terms of candidates that lost the global ranking
    if (kth != 0 && !A.drop) {
        const T* gv = reinterpret_cast<const T*>(A.index + A.L.gv) + unit * A.max_chunks * A.G * kD;
        const float* gln = reinterpret_cast<const float*>(A.index + A.L.gln) + unit * A.max_chunks * A.G;
        constexpr int AB = 2 * kOpenBatch;
        for (int k0 = wave * 4 + sgw; k0 < ncand; k0 += 16 * AB) {
            float vf[AB][8], lam[AB];
#pragma unroll
            for (int x = 0; x < AB; ++x) {
                const int k = k0 + 16 * x;
                lam[x] = -INFINITY;
                if (k < ncand) {
                    const uint64_t key = cand[k];
                    if (key != 0 && key < kth) {
                        const uint32_t g = key_id(key);
                        lam[x] = A.scale * key_score(key) + gln[g];
                        load8<T>(gv + (int64_t)g * kD, l16, vf[x]);
                    }
                }
            }
#pragma unroll
            for (int x = 0; x < AB; ++x)
                if (lam[x] != -INFINITY) st.add(lam[x], vf[x]);
        }
    }

    // merge the 16 subgroup states with the merged scan state, normalise
    open_stash(s, st);
    __syncthreads();
    if (tid < kD) {
        float M = s.scan_m;
        for (int k = 0; k < 16; ++k) M = fmaxf(M, s.sm[k]);
        float L = 0.0f, O = 0.0f;
        if (s.scan_m != -INFINITY) {
            const float e = softmax_exp(s.scan_m - M);
            L = s.scan_l * e;
            O = s.scan_o[tid] * e;
        }
        for (int k = 0; k < 16; ++k) {
            if (s.sm[k] == -INFINITY) continue;
            const float e = softmax_exp(s.sm[k] - M);
            L = __builtin_fmaf(s.sl[k], e, L);
            O = __builtin_fmaf(s.so[k][tid], e, O);
        }
        A.out[head * kD + tid] = O / L;
    }
}

// ---------------------------------------------------------------------------- MFMA scan (bf16)
//
// Ranking scores and logits of a 16-row block come from v_mfma_f32_16x16x32_bf16 with
// the g query heads as the rows of A (padded to 16) and 16 key rows as the columns of
// B; every lane loads its 16-byte operand slices straight from HBM, so each key byte is
// read once and shared by all heads.  bf16 x bf16 products are exact in fp32, so an
// MFMA score S differs from the exact dot product, and so does the canonical fp32 fma
// chain r, by at most gamma_128 * sum|q_t k_t| <= gamma_128 * |q| |kbar|; hence
// |S - r| <= E = kErrC * |q| |kbar| with kErrC = 8 * 128 * 2^-24 (four times the
// two-sided bound).  A slice's exact local top-k by r is therefore inside
// {g : S_g + E_g >= T}, T being the k-th largest S_g - E_g, and only those candidates
// are re-scored with the canonical chain.  Selection stays bit-exact; logits of the
// coarse terms use S.

constexpr int kMRows = 128;     // rows per chunk of the MFMA kernels

template <int HG>
struct MSmem {
    union {
        alignas(16) bf16_t vl[kMRows][kD];  // value rows of the tile, loaded straight into LDS
        float ored[8 / ((HG + 3) / 4)][4 * ((HG + 3) / 4)][kD];  // PV row-phase sums (after the last PV)
    } u;
    float sc[HG][kMRows];             // MFMA scores of the tile
    alignas(16) float wT[kMRows][8];  // softmax weights, [row][head] (heads >= HG: 0)
    float lnn[kMRows];                // ln n of the tile's groups
    float mrun[HG], lrun[HG], alpha[HG];
};

// MFMA A operand of the g query heads of this KV head (rows >= g are zero).
template <int HG>
__device__ __forceinline__ void mfma_load_q(const bf16_t* q0, bf16x8_t* qa) {
    const int l = threadIdx.x & 63;
    const int h = l & 15;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        if (h < HG) {
            qa[kk] = *reinterpret_cast<const bf16x8_t*>(q0 + h * kD + 32 * kk + 8 * (l >> 4));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qa[kk][e] = (__bf16)0.0f;
        }
    }
}

// Issue global->LDS loads of value rows r < n (n <= kMRows) into s.vl; completion is
// awaited by mfma_wait_lds.  One instruction moves 4 rows (64 lanes x 16 bytes).
template <int HG, typename RowPtr>
__device__ __forceinline__ void mfma_issue_v(MSmem<HG>& s, RowPtr vrow, int n) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    for (int i = w; 4 * i < n; i += 4) {
        int r = 4 * i + (l >> 4);
        r = r < n ? r : n - 1;
        __builtin_amdgcn_global_load_lds(vrow(r) + 8 * (l & 15), &s.u.vl[4 * i][0], 16, 0, 0);
    }
}
__device__ __forceinline__ void mfma_wait_lds() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// S[h][r] for rows r < n (n <= kMRows) whose key rows are krow(r).
template <int HG, typename RowPtr>
__device__ __forceinline__ void mfma_scores(float (*sc)[kMRows], const bf16x8_t* qa, RowPtr krow, int n) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int nblk = (n + 15) >> 4;
    constexpr int NB = kMRows / 64;
    bf16x8_t kb[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int blk = w + 4 * i;
        if (blk < nblk) {
            int rr = blk * 16 + (l & 15);
            rr = rr < n ? rr : n - 1;
            const bf16_t* row = krow(rr);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kb[i][kk] = *reinterpret_cast<const bf16x8_t*>(row + 32 * kk + 8 * (l >> 4));
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int blk = w + 4 * i;
        if (blk < nblk) {
            f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], kb[i][kk], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * (l >> 4) + r;
                if (h < HG) sc[h][blk * 16 + (l & 15)] = acc[r];
            }
        }
    }
}

// PV over rows r < n with weights s.wT[r][.] and value rows s.vl[r]: thread (head quad
// hq, row phase rp, dims 4*db..4*db+3) accumulates o[i][e] for heads 4*hq+i.
template <int HG>
__device__ __forceinline__ void mfma_pv(MSmem<HG>& s, int n, float (*o)[4]) {
    constexpr int HQ = (HG + 3) / 4, RPH = 8 / HQ;
    const int tid = threadIdx.x;
    const int hq = tid / (32 * RPH), rp = (tid / 32) % RPH, db = tid & 31;
    for (int r = rp; r < n; r += RPH) {
        const uint2 u = *reinterpret_cast<const uint2*>(&s.u.vl[r][4 * db]);
        const float4 w4 = *reinterpret_cast<const float4*>(&s.wT[r][4 * hq]);
        const float v[4] = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                            __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
        const float w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[i][e] = __builtin_fmaf(w[i], v[e], o[i][e]);
    }
}

// Sum the row phases of o and write the partial state (o, m, l) of every head.
template <int HG>
__device__ void mfma_write_partial(MSmem<HG>& s, float (*o)[4], float* dst_head0, int64_t head_stride,
                                   bool normalise = false) {
    constexpr int HQ = (HG + 3) / 4, RPH = 8 / HQ;
    const int tid = threadIdx.x;
    const int hq = tid / (32 * RPH), rp = (tid / 32) % RPH, db = tid & 31;
    __syncthreads();  // s.u is reused
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) s.u.ored[rp][4 * hq + i][4 * db + e] = o[i][e];
    __syncthreads();
    for (int x = tid; x < HG * kD; x += kThreads) {
        const int h = x / kD, d = x % kD;
        float a = s.u.ored[0][h][d];
        for (int k = 1; k < RPH; ++k) a += s.u.ored[k][h][d];
        dst_head0[(int64_t)h * head_stride + d] = normalise ? a / s.lrun[h] : a;
    }
    if (!normalise && tid < HG) {
        dst_head0[(int64_t)tid * head_stride + kD] = s.mrun[tid];
        dst_head0[(int64_t)tid * head_stride + kD + 1] = s.lrun[tid];
    }
}

// Exact rows (window, sinks, dense): online softmax over chunks of up to 256 rows.
// Row r of the list is position pos(r) = r < ns ? r : base + (r - ns).
template <int HG, typename RowOff>
__device__ void mfma_exact_rows(MSmem<HG>& s, const bf16x8_t* qa, const bf16_t* kb, const bf16_t* vb,
                                RowOff roff, int ns, int base, int nrows, float scale, float (*o)[4]) {
    constexpr int HQ = (HG + 3) / 4, RPH = 8 / HQ;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int hq = tid / (32 * RPH);
    for (int c0 = 0; c0 < nrows; c0 += kMRows) {
        const int n = min(kMRows, nrows - c0);
        auto pos = [&](int r) { const int x = c0 + r; return x < ns ? x : base + (x - ns); };
        auto krow = [&](int r) { return kb + roff(pos(r)); };
        auto vrow = [&](int r) { return vb + roff(pos(r)); };
        mfma_issue_v<HG>(s, vrow, n);
        mfma_scores<HG>(s.sc, qa, krow, n);
        __syncthreads();
        for (int h = w; h < HG; h += 4) {
            float lam[kMRows / 64], mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < kMRows / 64; ++k) {
                const int r = l + 64 * k;
                lam[k] = r < n ? scale * s.sc[h][r] : -INFINITY;
                mx = fmaxf(mx, lam[k]);
            }
            mx = wave_max_f32(mx, 64);
            const float mold = s.mrun[h];
            const float mn = fmaxf(mold, mx);
            float ls = 0.0f;
#pragma unroll
            for (int k = 0; k < kMRows / 64; ++k) {
                const int r = l + 64 * k;
                const float wgt = lam[k] == -INFINITY ? 0.0f : softmax_exp(lam[k] - mn);
                if (r < n) s.wT[r][h] = wgt;
                ls += wgt;
            }
            ls = wave_sum_f32(ls, 64);
            if (l == 0) {
                const float a = mold == -INFINITY ? 0.0f : softmax_exp(mold - mn);
                s.alpha[h] = a;
                s.lrun[h] = s.lrun[h] * a + ls;
                s.mrun[h] = mn;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = (4 * hq + i < HG) ? s.alpha[4 * hq + i] : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[i][e] *= a;
        }
        mfma_wait_lds();
        mfma_pv<HG>(s, n, o);
        __syncthreads();
    }
}

template <int HG>
__device__ __forceinline__ void mfma_init(MSmem<HG>& s, float (*o)[4]) {
    const int tid = threadIdx.x;
    if (tid < HG) { s.mrun[tid] = -INFINITY; s.lrun[tid] = 0.0f; s.alpha[tid] = 0.0f; }
    for (int x = tid; x < kMRows * 8; x += kThreads) (&s.wT[0][0])[x] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[i][e] = 0.0f;
}

// ---------------------------------------------------------------------------- scan (bf16)

// The scan of a (sequence, KV head) unit walks one list of 64-row tiles: the group
// summaries of every summarised chunk (coarse rows, logit scale * S + ln n), then the
// exact rows of the sinks and the block window (logit scale * S).  The unit's
// workgroups take equal runs of that list.  A tile's key and value rows are read with
// flat 16-byte loads (consecutive lanes, consecutive bytes) into registers one tile
// ahead, then written to LDS: keys row-major with their 16-byte chunks XOR-swizzled by
// row, values transposed (dimension-major) in 8-row blocks XOR-swizzled by dimension, so
// that both MFMA operand reads are 16-byte and spread over the banks.  Scores S = q K^T
// and the value sums O^T = V^T P^T run on MFMA; P enters as bf16 hi + lo.
constexpr int kSTile = kScanTile;                      // rows per scan tile
constexpr int kSPieces = kSTile * kD / 8 / kThreads;   // 16-byte pieces per thread and row kind
constexpr int kSWStride = kSTile + 8;                  // bf16 per head row of the weights
static_assert(kSPieces == 4, "the scan stage packs four rows per thread");

template <int HG>
struct MScanSmem {
    alignas(16) bf16_t kl[kSTile][kD];   // key rows (swizzled chunks)
    alignas(16) bf16_t vt[kD][kSTile];   // value columns: vt[d][8 * (b ^ (d / 8 % 8)) + j] = V[8b + j][d]
    alignas(16) bf16_t wh[16][kSWStride];  // softmax weights [head][row], bf16 hi (heads >= HG: 0)
    alignas(16) bf16_t wl[16][kSWStride];  // and lo parts
    float bias[kSTile];                  // ln n of a coarse tile's groups, 0 for exact rows
    alignas(16) float sc[HG][kSTile];    // MFMA scores of the tile
    float mrun[HG], lrun[HG], alpha[16];
};

// Rows of one unit: coarse tiles first, then the exact rows (list index x is position x
// for the sinks, w0 + x - ns after them).
struct ScanSrc {
    const bf16_t* gk;
    const bf16_t* gv;
    const float* gln;
    int ng;
    const bf16_t* kb;  // head kvh of sequence seq; row of position x: kb + kv_pos(*this, seq, x)
    const bf16_t* vb;
    int64_t sb, st;
    const int32_t* btab;
    int bshift, maxb, seq;
    int ns, w0, nex;
};

// Tile t of a unit's list: coarse tiles (group summaries) first, then exact tiles (sinks
// and window rows); up to kSTile rows of one kind, starting at row r0 of its list.  (A
// split by 16-row blocks, balancing bytes across a unit's workgroups, was slower: the
// partial tiles add iterations, and an iteration's latency, not its bytes, sets the pace
// of a workgroup.)
struct ScanTile {
    int coarse, r0, n;
};

__device__ __forceinline__ ScanTile scan_tile(int t, int ntc, int ng, int nex) {
    ScanTile T;
    T.coarse = t < ntc;
    T.r0 = (T.coarse ? t : t - ntc) * kSTile;
    T.n = min(kSTile, (T.coarse ? ng : nex) - T.r0);
    return T;
}

// One tile in registers: thread tid holds the 16-byte chunk c = tid % 16 of rows
// 4g .. 4g+3, g = tid / 16, of its key and value rows (rows past the tile repeat its last
// row), and the bias of row tid.  Four rows per thread let the value transpose go to LDS
// as 8-byte words (four rows of one dimension).
struct ScanRegs {
    u32x4_t k[kSPieces], v[kSPieces];
    float bias;
};

// DROP (no coarse remainder): coarse tiles only give scores, so their values are not read.
template <bool DROP, bool PAGED>
__device__ __forceinline__ void scan_fetch(ScanRegs& R, const ScanSrc& S, const ScanTile& T) {
    const int tid = threadIdx.x, c = tid & 15, g = tid >> 4;
    if (T.coarse) {
        const int r0 = T.r0, n = T.n;
#pragma unroll
        for (int i = 0; i < kSPieces; ++i) {
            const int row = min(4 * g + i, n - 1);
            const int64_t off = (int64_t)(r0 + row) * kD + 8 * c;
            // read once per call: non-temporal, so that these rows do not push out of
            // the caches what the open step reads next (meta rows, norms, opened pages)
            R.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(S.gk + off));
            if (!DROP) R.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(S.gv + off));
        }
        R.bias = tid < kSTile ? S.gln[r0 + min(tid, n - 1)] : 0.0f;
    } else {
        const int x0 = T.r0, n = T.n;
#pragma unroll
        for (int i = 0; i < kSPieces; ++i) {
            const int x = x0 + min(4 * g + i, n - 1);
            const int pos = x < S.ns ? x : S.w0 + (x - S.ns);
            const int64_t off = kv_pos<PAGED>(S, S.seq, pos) + 8 * c;
            R.k[i] = *reinterpret_cast<const u32x4_t*>(S.kb + off);
            R.v[i] = *reinterpret_cast<const u32x4_t*>(S.vb + off);
        }
        R.bias = 0.0f;
    }
}

// Keys row-major with 16-byte chunks swizzled by row; values transposed, one 8-byte
// write per dimension holding rows 4g .. 4g+3 (packed from the four row registers).
template <int HG>
__device__ __forceinline__ void scan_stage(MScanSmem<HG>& s, const ScanRegs& R) {
    const int tid = threadIdx.x, c = tid & 15, g = tid >> 4;
#pragma unroll
    for (int i = 0; i < kSPieces; ++i) {
        const int row = 4 * g + i;
        *reinterpret_cast<u32x4_t*>(&s.kl[row][8 * (c ^ (row & 15))]) = R.k[i];
    }
    // rows 4g .. 4g+3 sit at column positions 8 * ((g / 2) ^ (d / 8 % 8)) + 4 * (g % 2) + i
    const int pos = 8 * ((g >> 1) ^ (c & 7)) + 4 * (g & 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t a0 = R.v[0][m], a1 = R.v[1][m], a2 = R.v[2][m], a3 = R.v[3][m];
        uint2 lo, hi;  // dimension 8c + 2m (low halves) and 8c + 2m + 1 (high halves)
        lo.x = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
        lo.y = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
        hi.x = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
        hi.y = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
        *reinterpret_cast<uint2*>(&s.vt[8 * c + 2 * m][pos]) = lo;
        *reinterpret_cast<uint2*>(&s.vt[8 * c + 2 * m + 1][pos]) = hi;
    }
    if (tid < kSTile) s.bias[tid] = R.bias;
}

// MFMA scores of the staged tile into s.sc: wave w takes rows 16w .. 16w+15 (query heads
// are the A rows, rows >= HG zero).
template <int HG>
__device__ __forceinline__ void scan_scores(MScanSmem<HG>& s, const bf16x8_t* qa) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int row = 16 * w + (l & 15);
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int chunk = (4 * kk + (l >> 4)) ^ (row & 15);
        const bf16x8_t kbv = *reinterpret_cast<const bf16x8_t*>(&s.kl[row][8 * chunk]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], kbv, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * (l >> 4) + r;
        if (h < HG) s.sc[h][row] = acc[r];
    }
}

// O^T += V^T P^T over the staged tile: wave w takes dims 32w .. 32w+31 (two 16-row MFMA
// blocks); lane l holds o[mb][i] = O^T[32w + 16mb + 4(l/16) + i][head l%16].
template <int HG>
__device__ __forceinline__ void scan_pv(const MScanSmem<HG>& s, f32x4_t* o) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int kb = 0; kb < kSTile / 32; ++kb) {
        const int rb = 4 * kb + (l >> 4);  // 8-row block of this lane's operand
        const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&s.wh[l & 15][8 * rb]);
        const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&s.wl[l & 15][8 * rb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int d = 32 * w + 16 * mb + (l & 15);
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&s.vt[d][8 * (rb ^ ((d >> 3) & 7))]);
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, o[mb], 0, 0, 0);
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, o[mb], 0, 0, 0);
        }
    }
}

// Decode launch 1 (bf16): workgroup x of a (sequence, KV head) unit scans tiles
// [x * nt / nslice, (x + 1) * nt / nslice) of the unit's tile list: MFMA scores (written
// out for the selection on coarse tiles), online softmax and PV, then its partial state.
template <int HG, bool DROP, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void decode_scan_mfma_kernel(DecodeArgs A) {
    __shared__ MScanSmem<HG> s;
    const int kvh = blockIdx.x, b = blockIdx.y, slice = blockIdx.z;  // b: query row
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    int seq, p;
    row_info(A, b, seq, p);
    const int nb = nbuilt(p, A.W);
    const int64_t unit = (int64_t)seq * A.Hkv + kvh;
    const int64_t gbase = unit * A.max_chunks * A.G;
    ScanSrc S;
    S.gk = reinterpret_cast<const bf16_t*>(A.index + A.L.gk) + gbase * kD;
    S.gv = reinterpret_cast<const bf16_t*>(A.index + A.L.gv) + gbase * kD;
    S.gln = reinterpret_cast<const float*>(A.index + A.L.gln) + gbase;
    S.ng = nb * A.G;
    S.kb = reinterpret_cast<const bf16_t*>(A.k) + kvh * A.sh + kv_seq<PAGED>(A, seq);
    S.vb = reinterpret_cast<const bf16_t*>(A.v) + kvh * A.sh + kv_seq<PAGED>(A, seq);
    S.sb = A.sb; S.st = A.st; S.btab = A.btab; S.bshift = A.bshift; S.maxb = A.maxb; S.seq = seq;
    S.ns = min(A.n_sink, nb * kChunk);
    S.w0 = nb * kChunk;
    S.nex = S.ns + (p + 1 - S.w0);
    const int ntc = (S.ng + kSTile - 1) / kSTile;
    const int nt = ntc + (S.nex + kSTile - 1) / kSTile;
    // The slice is the slowest grid dimension, so on a CU the workgroups of lower slices
    // are the older ones, and the oldest waves issue first: the youngest workgroups of a
    // CU run last, much of the time alone.  So the older slices take the larger shares
    // (one tile more when the tiles do not divide evenly) and the end of the list (the
    // window's exact tiles, read from the cache with a stride, are the slowest), and the
    // youngest the first coarse tiles.
    const int tq = nt / A.nslice, tr = nt % A.nslice;
    const int t1 = nt - (slice * tq + min(slice, tr));
    const int t0 = t1 - (tq + (slice < tr ? 1 : 0));
    const int hq0 = kvh * HG;
    float* part0 = A.part + ((int64_t)(b * A.Hq + hq0) * A.nslot + slice) * kPartStride;
    const int64_t head_stride = (int64_t)A.nslot * kPartStride;
    float* sdst = A.score + ((int64_t)b * A.Hq + hq0) * A.score_stride;
    const bf16_t* q0 = reinterpret_cast<const bf16_t*>(A.q) + ((int64_t)b * A.Hq + hq0) * kD;

    if (tid < HG) { s.mrun[tid] = -INFINITY; s.lrun[tid] = 0.0f; }
    if (tid < 16) s.alpha[tid] = 0.0f;
    // weight rows of the heads past HG stay zero
    for (int x = tid; x < 16 * kSWStride; x += kThreads) {
        (&s.wh[0][0])[x] = 0;
        (&s.wl[0][0])[x] = 0;
    }
    f32x4_t o[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    bf16x8_t qa[4];
    mfma_load_q<HG>(q0, qa);
    ScanRegs R;
    if (t0 < t1) scan_fetch<DROP, PAGED>(R, S, scan_tile(t0, ntc, S.ng, S.nex));

    for (int t = t0; t < t1; ++t) {
        const ScanTile cur = scan_tile(t, ntc, S.ng, S.nex);
        const bool coarse = cur.coarse;
        const int r0 = cur.r0, n = cur.n;
        scan_stage(s, R);  // the last tile's PV is done (barrier at the end of the loop)
        if (t + 1 < t1) scan_fetch<DROP, PAGED>(R, S, scan_tile(t + 1, ntc, S.ng, S.nex));  // in flight
        __syncthreads();
        scan_scores<HG>(s, qa);
        __syncthreads();
        // coarse tiles: the scores go out for the selection, one float4 per head and four
        // groups, -inf for an empty group (only the last tile of the unit's groups is
        // partial; its last float4 may pass the end: those rows lie inside score_stride
        // and are never read)
        if (coarse && tid < 16 * HG && 4 * (tid & 15) < n) {
            const int h = tid >> 4, j = tid & 15;
            float4 v = *reinterpret_cast<const float4*>(&s.sc[h][4 * j]);
            if (s.bias[4 * j] == -INFINITY) v.x = -INFINITY;
            if (s.bias[4 * j + 1] == -INFINITY) v.y = -INFINITY;
            if (s.bias[4 * j + 2] == -INFINITY) v.z = -INFINITY;
            if (s.bias[4 * j + 3] == -INFINITY) v.w = -INFINITY;
            *reinterpret_cast<float4*>(sdst + (int64_t)h * A.score_stride + r0 + 4 * j) = v;
        }
        // without the remainder a coarse tile only yields scores
        const bool accumulate = !(DROP && coarse);
        for (int h = w; h < (accumulate ? HG : 0); h += 4) {
            // coarse: the same expression the open kernel uses for the groups it subtracts
            const float bb = s.bias[l];
            const float lam = (l < n && bb != -INFINITY) ? A.scale * s.sc[h][l] + bb : -INFINITY;
            const float mx = wave_max_f32(lam, 64);
            const float mold = s.mrun[h];
            const float mn = fmaxf(mold, mx);
            const float wgt = lam == -INFINITY ? 0.0f : softmax_exp(lam - mn);
            __bf16 hi, lo;
            split_bf16(wgt, hi, lo);
            s.wh[h][l] = __builtin_bit_cast(bf16_t, hi);
            s.wl[h][l] = __builtin_bit_cast(bf16_t, lo);
            const float ls = wave_sum_f32(wgt, 64);
            if (l == 0) {
                const float a = mold == -INFINITY ? 0.0f : softmax_exp(mold - mn);
                s.alpha[h] = a;
                s.lrun[h] = s.lrun[h] * a + ls;
                s.mrun[h] = mn;
            }
        }
        __syncthreads();
        if (accumulate) {
            const float a = s.alpha[l & 15];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[mb][i] *= a;
            scan_pv<HG>(s, o);
        }
        __syncthreads();
    }

    // partial state (o, m, l) of every head
    const int h = l & 15;
    if (h < HG) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part0[(int64_t)h * head_stride + 32 * w + 16 * mb + 4 * (l >> 4) + i] = o[mb][i];
    }
    if (tid < HG) {
        part0[(int64_t)tid * head_stride + kD] = s.mrun[tid];
        part0[(int64_t)tid * head_stride + kD + 1] = s.lrun[tid];
    }
}

// ---------------------------------------------------------------------------- open (bf16)

// Opened groups from the stored MFMA scores S of every group of the head.  With
// E_g = kErrC |q| |kbar_g| bounding |S_g - r_g| (r: canonical chain), the exact top-k by
// r lies in {g : S_g + E_g >= T}, T being the k-th largest S_g - E_g; those candidates
// are re-scored canonically and ranked exactly (score desc, id asc).  Columns with more
// candidates than kOpenCand (massive ties) rank every group canonically.
// Head mapping: consecutive workgroups take different KV heads, so the query heads of
// one KV head share an XCD and its L2 (workgroups are dealt to the 8 XCDs round robin).
// The scan included the opened groups in its coarse sums; their terms, with the very
// same logits, are subtracted in the final merge.  The subtracted mass never exceeds
// the scan's, and the exact terms of the opened pages carry at least the same order of
// mass, so fp32 cancellation stays near 1e-6 of the output scale.
template <bool DROP, bool PAGED, bool Q4>
__device__ void decode_open_role(const DecodeArgs& A, OpenSmem<bf16_t>& s, int b, int hq) {
    const int HG = A.Hq / A.Hkv;
    const int kvh = hq / HG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15;
    int seq, p;
    row_info(A, b, seq, p);
    const int nb = nbuilt(p, A.W);
    const int ng = nb * A.G;
    const int TG = A.TG;
    const int64_t unit = (int64_t)seq * A.Hkv + kvh;
    const int64_t head = (int64_t)b * A.Hq + hq;
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.q) + head * kD;
    const float* S = A.score + head * A.score_stride;
    const float* gkn = reinterpret_cast<const float*>(A.index + A.L.gkn) + unit * A.max_chunks * A.G;
    const float* gln = reinterpret_cast<const float*>(A.index + A.L.gln) + unit * A.max_chunks * A.G;
    const int32_t* gpage = reinterpret_cast<const int32_t*>(A.index + A.L.gpage) + unit * A.max_chunks * A.G;
    const bf16_t* gk = reinterpret_cast<const bf16_t*>(A.index + A.L.gk) + unit * A.max_chunks * A.G * kD;
    const bf16_t* gv = reinterpret_cast<const bf16_t*>(A.index + A.L.gv) + unit * A.max_chunks * A.G * kD;
    const int16_t* meta_u = reinterpret_cast<const int16_t*>(A.index + A.L.meta) + unit * A.max_chunks * A.L.meta_stride;
    const bf16_t* pk_u = reinterpret_cast<const bf16_t*>(A.index + A.L.pk) + unit * A.max_chunks * A.L.page_slots * kD;
    const float* pln_u = reinterpret_cast<const float*>(A.index + A.L.pln) + unit * A.max_chunks * A.L.page_slots;

    // loads of the first round trip, issued together: q, the scores, the bounds' inputs
    float q8[8];
    load8<bf16_t>(qp, l16, q8);
    const float qv = tid < kD ? bf16_bits_to_f32(qp[tid]) : 0.0f;
    constexpr int SPT = 16;  // groups per thread per round
    // the scan stored -inf as the score of an empty group: only non-empty ones compete
    float sv[SPT], kn[SPT];
    int32_t gp[SPT];
    auto load_scores = [&](int g0) {
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int g = g0 + tid + kThreads * u;
            sv[u] = -INFINITY;
            if (g < ng) { sv[u] = S[g]; kn[u] = gkn[g]; gp[u] = gpage[g]; }
        }
    };
    if (ng > 0) load_scores(0);
    // scan partial states: straight into LDS (awaited before the final merge), else
    // merged from global memory by waves 2-3
    const int nscan = A.nslice + A.nwin;
    const float* part = A.part + head * A.nslot * kPartStride;
    const bool part_in_lds = nscan <= kPartLds;
    if (part_in_lds) {
        const int npiece = nscan * (kPartStride / 4);  // 16-byte pieces
        for (int i = wave; 64 * i < npiece; i += 4) {
            const int pc = min(64 * i + lane, npiece - 1);
            __builtin_amdgcn_global_load_lds(part + 4 * pc, &s.plds[256 * i], 16, 0, 0);
        }
    }
    if (tid < kD) s.qs[tid] = qv;
    // |q| (16 lanes, 8 values each), rounded up
    float qn = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) qn = __builtin_fmaf(q8[e], q8[e], qn);
    qn = sqrtf(row16_sum_f32(qn)) * 1.0001f;
    const float eq = kErrC * qn;
    if (!part_in_lds) open_merge_scan(s, part, nscan);

    // 1a. every thread: the largest lower bound S - E among its groups.  The k-th
    //     largest of these per-thread maxima is a lower bound of the k-th largest over
    //     all groups, so it is a valid threshold.
    float mx = -INFINITY;
    for (int g0 = 0; g0 < ng; g0 += SPT * kThreads) {
        if (g0 > 0) load_scores(g0);
#pragma unroll
        for (int u = 0; u < SPT; ++u)
            if (sv[u] != -INFINITY) mx = fmaxf(mx, sv[u] - eq * kn[u]);
    }
    // 1b. each wave: its R largest maxima (with multiplicity), R = min(TG, 4).  Any TG of
    //     them are maxima of distinct threads, so the TG-th largest of the 4R values is
    //     again a lower bound of the TG-th largest over all groups.
    const int R = TG < 4 ? TG : 4;
    {
        int taken = 0;
        for (int round = 0; round < R && taken < R; ++round) {
            const float m = wave_max_f32(mx, 64);
            if (m == -INFINITY) break;
            const bool mine = mx == m;
            const int c = __popcll(__ballot(mine));
            if (lane == 0)
                for (int x = 0; x < c && taken + x < R; ++x) s.wl[wave][taken + x] = m;
            taken += c;
            if (mine) mx = -INFINITY;
        }
        if (lane == 0)
            for (int x = taken < R ? taken : R; x < 4; ++x) s.wl[wave][x] = -INFINITY;
    }
    if (tid == 0) { s.ncand = 0; s.meta_ready = 0; s.pscore_ready = 0; }
    __syncthreads();
    // 1c. every thread: T = the TG-th largest of the 16 list entries (sorting network;
    //     -inf when fewer than TG are finite)
    float T;
    {
        float v[16];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            const float4 f = *reinterpret_cast<const float4*>(&s.wl[w4][0]);
            v[4 * w4] = f.x; v[4 * w4 + 1] = f.y; v[4 * w4 + 2] = f.z; v[4 * w4 + 3] = f.w;
        }
        // bitonic sort, descending
#pragma unroll
        for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
            for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int x = i ^ j;
                    if (x > i) {
                        const bool desc = (i & k) == 0;
                        const float hi = fmaxf(v[i], v[x]), lo = fminf(v[i], v[x]);
                        v[i] = desc ? hi : lo;
                        v[x] = desc ? lo : hi;
                    }
                }
        T = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (e == TG - 1) T = v[e];
    }
    // 1d. candidates: S + E >= T (a single block of groups is still in registers).  They
    //     are few, so each takes its slot with an LDS atomic; the order of the slots does
    //     not matter (ranking compares keys).
    for (int g0 = 0; g0 < ng; g0 += SPT * kThreads) {
        if (ng > SPT * kThreads) load_scores(g0);
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            if (sv[u] != -INFINITY && sv[u] + eq * kn[u] >= T) {
                const int at = atomicAdd(&s.ncand, 1);
                if (at < kOpenCand) {
                    s.cg[at] = g0 + tid + kThreads * u;
                    s.cS[at] = sv[u];
                    s.cP[at] = gp[u];
                }
            }
        }
    }
    __syncthreads();
    const int ncand = s.ncand;
    if (ncand <= kOpenCand) {
        // the opened groups are among the candidates: with at most kMetaRows of them,
        // their meta rows go to LDS now (row x: candidate x), overlapping the canonical
        // re-scoring; otherwise the page step loads the opened groups' rows (row i: the
        // group of rank i)
        const bool prefetch = ncand <= kMetaRows;
        if (prefetch) {
            const int ms16 = A.L.meta_stride / 8;
            const int npiece = ncand * ms16;
            int16_t* mflat = &s.meta[0][0];
            for (int i = wave; 64 * i < npiece; i += 4) {
                // piece pc (row x, 16-byte piece e) lands at mflat + 8 * pc: candidate x's
                // row starts at x * meta_stride entries, as the page step addresses it
                const int pc = min(64 * i + lane, npiece - 1);
                const int x = pc / ms16, e = pc % ms16;
                __builtin_amdgcn_global_load_lds(meta_u + (int64_t)(s.cg[x] / A.G) * A.L.meta_stride + 8 * e,
                                                 mflat + 512 * i, 16, 0, 0);
            }
            // canonical scores of every candidate's pages, ahead of the group ranking (the
            // page step then only ranks them): item f = (candidate f / 16, page f % 16) on
            // the threads of waves 1-3; the group chains below run on wave 0
            if (tid >= 64) {
                for (int f = tid - 64; f < ncand * 16; f += kThreads - 64) {
                    const int x = f >> 4, e = f & 15;
                    const int cp = s.cP[x], npg = cp >> 16;
                    if (e < npg) {
                        const int64_t slot = (int64_t)(s.cg[x] / A.G) * A.L.page_slots + (cp & 0xffff) + e;
                        const bf16_t* row = pk_u + slot * kD;
                        uint4 u[16];
#pragma unroll
                        for (int c = 0; c < 16; ++c) u[c] = *reinterpret_cast<const uint4*>(row + 8 * c);
                        const float lnp = pln_u[slot];
                        float acc = 0.0f;
#pragma unroll
                        for (int c = 0; c < 16; ++c) {
                            float fv[8];
                            Elt<bf16_t>::unpack(u[c], fv);
#pragma unroll
                            for (int t = 0; t < 8; ++t) acc = __builtin_fmaf(s.qs[8 * c + t], fv[t], acc);
                        }
                        s.pr[f] = acc;
                        s.pl[f] = lnp;
                    }
                }
            }
        }
        for (int x = tid; x < ncand; x += kThreads) {
            const bf16_t* row = gk + (int64_t)s.cg[x] * kD;
            uint4 u[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) u[c] = *reinterpret_cast<const uint4*>(row + 8 * c);
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                float f[8];
                Elt<bf16_t>::unpack(u[c], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(s.qs[8 * c + e], f[e], acc);
            }
            s.cs[x] = acc;
        }
        __syncthreads();
        for (int x = tid; x < ncand; x += kThreads) {
            const uint64_t key = rank_key(s.cs[x], (uint32_t)s.cg[x]);
            int rank = 0;
            for (int y = 0; y < ncand; ++y) rank += rank_key(s.cs[y], (uint32_t)s.cg[y]) > key;
            if (rank < TG) {
                s.sel[rank] = key;
                s.mrow[rank] = prefetch ? x : rank;
                s.sub_S[rank] = s.cS[x];
            }
        }
        if (tid == 0) {
            s.nsel = ncand < TG ? ncand : TG;
            s.meta_ready = prefetch;
            s.pscore_ready = prefetch;
        }
    } else {
        // exhaustive: canonical score of every non-empty group, workgroup-wide top-TG
        uint64_t top[kMaxTG];
#pragma unroll
        for (int e = 0; e < kMaxTG; ++e) top[e] = 0;
        for (int g = tid; g < ng; g += kThreads) {
            if (gln[g] == -INFINITY) continue;
            const bf16_t* row = gk + (int64_t)g * kD;
            float acc = 0.0f;
            for (int c = 0; c < 16; ++c) {
                float f[8];
                Elt<bf16_t>::unpack(*reinterpret_cast<const uint4*>(row + 8 * c), f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(s.qs[8 * c + e], f[e], acc);
            }
            uint64_t x = rank_key(acc, (uint32_t)g);
#pragma unroll
            for (int e = 0; e < kMaxTG; ++e) {
                const uint64_t hi = top[e] > x ? top[e] : x, lo = top[e] > x ? x : top[e];
                top[e] = hi;
                x = lo;
            }
        }
        int k = 0;
        for (int round = 0; round < TG; ++round) {
            const uint64_t wm = wave_max_u64(top[0]);
            if (lane == 0) s.red[wave] = wm;
            __syncthreads();
            uint64_t m = s.red[0];
            for (int x = 1; x < 4; ++x) m = s.red[x] > m ? s.red[x] : m;
            __syncthreads();
            if (m == 0) break;
            if (tid == 0) s.sel[round] = m;
            if (top[0] == m) {
#pragma unroll
                for (int e = 0; e < kMaxTG - 1; ++e) top[e] = top[e + 1];
                top[kMaxTG - 1] = 0;
            }
            ++k;
        }
        if (tid == 0) s.nsel = k;
        if (tid < kMaxTG) s.mrow[tid] = tid;
        __syncthreads();
        if (tid < k) {
            const uint32_t g = key_id(s.sel[tid]);
            s.sub_S[tid] = S[g];
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // prefetched meta rows (global -> LDS) of this wave
    __syncthreads();
    const int nsel = s.nsel;
    if (A.sel_groups && tid < TG) A.sel_groups[head * TG + tid] = tid < nsel ? (int)key_id(s.sel[tid]) : -1;
    // the opened groups' mean values and ln n (loads in flight during the page work)
    // (raw bits: converted where used, so nothing waits for them before then)
    uint32_t vsub[kMaxTG];
    if (tid < kD) {
#pragma unroll
        for (int i = 0; i < kMaxTG; ++i)
            vsub[i] = (i < nsel && !DROP) ? gv[(int64_t)key_id(s.sel[i]) * kD + tid] : 0u;
    }
    const float lsub = (tid < nsel && !DROP) ? gln[key_id(s.sel[tid < kMaxTG ? tid : 0])] : 0.0f;

    Online st;
    st.init();
    open_pages<bf16_t, 2 * kOpenBatch, PAGED, false, DROP, Q4>(A, s, nsel, seq, kvh, head, q8, st);
    open_stash(s, st);
    // the opened groups' coarse logits in the scan, by the scan's own arithmetic
    if (tid < nsel) s.sub_lam[tid] = A.scale * s.sub_S[tid] + lsub;
    if (part_in_lds) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // out = scan state - opened groups' coarse terms (the very logits the scan used) +
    // the exact terms of the opened groups.  Thread tid < kD takes dimension tid; the
    // scan state comes from the partials in LDS (maximum first, then the sums), or from
    // the merge of waves 2-3.
    if (tid < kD) {
        float SM, SL, SO;
        if (part_in_lds) {
            SM = -INFINITY;
            for (int k = 0; k < nscan; ++k) SM = fmaxf(SM, s.plds[k * kPartStride + kD]);
            SL = 0.0f;
            SO = 0.0f;
            if (SM != -INFINITY) {
#pragma unroll 4
                for (int k = 0; k < nscan; ++k) {
                    const float* pp = &s.plds[k * kPartStride];
                    const float e = pp[kD] == -INFINITY ? 0.0f : softmax_exp(pp[kD] - SM);
                    SL = __builtin_fmaf(pp[kD + 1], e, SL);
                    SO = __builtin_fmaf(pp[tid], e, SO);
                }
            }
        } else {
            SM = s.scan_m;
            SL = s.scan_l;
            SO = s.scan_o[tid];
        }
        float M = SM;
#pragma unroll
        for (int k = 0; k < 16; ++k) M = fmaxf(M, s.sm[k]);
        float L = 0.0f, O = 0.0f;
        if (SM != -INFINITY) {
            const float e = softmax_exp(SM - M);
            L = SL * e;
            O = SO * e;
#pragma unroll
            for (int i = 0; i < kMaxTG; ++i) {
                if (i >= nsel || DROP) break;  // no remainder: nothing was summed
                const float w = softmax_exp(s.sub_lam[i] - M);
                L -= w;
                O = __builtin_fmaf(-w, bf16_bits_to_f32(vsub[i]), O);
            }
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float e = s.sm[k] == -INFINITY ? 0.0f : softmax_exp(s.sm[k] - M);
            L = __builtin_fmaf(s.sl[k], e, L);
            O = __builtin_fmaf(s.so[k][tid], e, O);
        }
        A.out[head * kD + tid] = O / L;
    }
}

// Decode launch 2 (bf16): one workgroup per (sequence, query head) runs the open step and
// the final merge.  Consecutive workgroups take different KV heads, so the query heads
// of one KV head share an XCD (workgroups are dealt to the 8 XCDs round robin).
template <bool DROP, bool PAGED, bool Q4>
__global__ __launch_bounds__(kThreads) void decode_open_mfma_kernel(DecodeArgs A) {
    __shared__ OpenSmem<bf16_t> s;
    const int j = blockIdx.x;
    decode_open_role<DROP, PAGED, Q4>(A, s, blockIdx.y, (j % A.Hkv) * (A.Hq / A.Hkv) + j / A.Hkv);
}


// Dense decode (bf16): split workgroups over rows, MFMA scores, online softmax.
template <int HG, bool PAGED>
__global__ __launch_bounds__(kThreads) void dense_decode_mfma_kernel(DenseArgs A) {
    __shared__ MSmem<HG> s;
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
    const bf16_t* q0 = reinterpret_cast<const bf16_t*>(A.q) + ((int64_t)b * A.Hq + hq0) * kD;
    float o[4][4];
    mfma_init<HG>(s, o);
    bf16x8_t qa[4];
    mfma_load_q<HG>(q0, qa);
    __syncthreads();
    const int r0 = blockIdx.x * A.rows_per_wg;
    const int r1 = min(r0 + A.rows_per_wg, p + 1);
    if (r1 > r0) {
        const bf16_t* kh = reinterpret_cast<const bf16_t*>(A.k) + kvh * A.sh + kv_seq<PAGED>(A, seq);
        const bf16_t* vh = reinterpret_cast<const bf16_t*>(A.v) + kvh * A.sh + kv_seq<PAGED>(A, seq);
        mfma_exact_rows<HG>(s, qa, kh, vh, [&](int x) { return kv_pos<PAGED>(A, seq, x); }, 0, r0, r1 - r0,
                            A.scale, o);
    }
    if (A.out) {
        mfma_write_partial<HG>(s, o, A.out + ((int64_t)b * A.Hq + hq0) * kD, kD, true);
        return;
    }
    float* part0 = A.part + ((int64_t)(b * A.Hq + hq0) * A.nsplit + blockIdx.x) * kPartStride;
    mfma_write_partial<HG>(s, o, part0, (int64_t)A.nsplit * kPartStride);
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
        const T* kh = reinterpret_cast<const T*>(A.k) + kvh * A.sh;
        const T* vh = reinterpret_cast<const T*>(A.v) + kvh * A.sh;
        exact_rows<T, HG>(s, R, qr, [&](int x) { return kh + kv_row_rt(A, seq, x); },
                          [&](int x) { return vh + kv_row_rt(A, seq, x); }, r0, r1, A.scale, m_run, l_run, o);
    }
    if (A.out) {  // one split per row: write the normalised output directly
        write_partial<HG>(s, R, o, m_run, l_run, A.out + ((int64_t)b * A.Hq + hq0) * kD, kD, true);
        return;
    }
    float* part0 = A.part + ((int64_t)(b * A.Hq + hq0) * A.nsplit + blockIdx.x) * kPartStride;
    write_partial<HG>(s, R, o, m_run, l_run, part0, (int64_t)A.nsplit * kPartStride);
}

// ---------------------------------------------------------------------------- host side


template <typename T, int HG, bool PAGED>
static void launch_decode_view(const DecodeArgs& A, int rows, hipStream_t st) {
    trace_point(0, st);
    if constexpr (sizeof(T) == 2) {
        if (A.nslice + A.nwin > 0) {
            // KV head fastest, then the row, then the slice: a unit's workgroups share
            // an XCD (workgroups go to the 8 XCDs round robin), the one the open step's
            // workgroups of that KV head use, and slices of one unit reach a CU at
            // different times, so no unit as a whole starts last
            const dim3 sg(A.Hkv, rows, A.nslice + A.nwin);
            if (A.drop)
                hipLaunchKernelGGL((decode_scan_mfma_kernel<HG, true, PAGED>), sg, dim3(kThreads), 0, st, A);
            else
                hipLaunchKernelGGL((decode_scan_mfma_kernel<HG, false, PAGED>), sg, dim3(kThreads), 0, st, A);
        }
        trace_point(1, st);
        // with INT4 pages the open step reads no cache rows, so the view does not matter
        const dim3 og(A.Hq, rows);
        if (A.q4 && A.drop)
            hipLaunchKernelGGL((decode_open_mfma_kernel<true, false, true>), og, dim3(kThreads), 0, st, A);
        else if (A.q4)
            hipLaunchKernelGGL((decode_open_mfma_kernel<false, false, true>), og, dim3(kThreads), 0, st, A);
        else if (A.drop)
            hipLaunchKernelGGL((decode_open_mfma_kernel<true, PAGED, false>), og, dim3(kThreads), 0, st, A);
        else
            hipLaunchKernelGGL((decode_open_mfma_kernel<false, PAGED, false>), og, dim3(kThreads), 0, st, A);
        trace_point(2, st);
    } else {
        if (A.nslice + A.nwin > 0)
            hipLaunchKernelGGL((decode_scan_kernel<T, HG>), dim3(A.nslice + A.nwin, A.Hkv, rows),
                               dim3(kThreads), 0, st, A);
        trace_point(1, st);
        hipLaunchKernelGGL((decode_open_kernel<T, PAGED>), dim3(A.Hq, rows), dim3(kThreads), 0, st, A);
        trace_point(2, st);
    }
}

template <typename T, int HG>
static int launch_decode(const DecodeArgs& A, int rows, hipStream_t st) {
    if (A.btab)
        launch_decode_view<T, HG, true>(A, rows, st);
    else
        launch_decode_view<T, HG, false>(A, rows, st);
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}

template <typename T, int HG>
static int launch_dense(const DenseArgs& A, float* out, int rows, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        if (A.btab)
            hipLaunchKernelGGL((dense_decode_mfma_kernel<HG, true>), dim3(A.nsplit, A.Hkv, rows), dim3(kThreads), 0,
                               st, A);
        else
            hipLaunchKernelGGL((dense_decode_mfma_kernel<HG, false>), dim3(A.nsplit, A.Hkv, rows), dim3(kThreads), 0,
                               st, A);
    } else {
        hipLaunchKernelGGL((dense_decode_kernel<T, HG>), dim3(A.nsplit, A.Hkv, rows), dim3(kThreads), 0,
                           st, A);
    }
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
    A.k = kv.k; A.v = kv.v;
    set_kv_map(A, kv);
    A.index = reinterpret_cast<const char*>(index->mem);
    A.L = L;
    A.max_chunks = index->max_chunks;
    A.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + P.off_part);
    A.cand = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + P.off_cand);
    A.score = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + P.off_score);
    A.score_stride = P.score_stride;
    A.Hq = params->n_q_heads; A.Hkv = params->n_kv_heads; A.G = params->groups_per_chunk;
    A.TG = params->top_groups; A.TP = params->top_pages; A.W = params->window;
    A.n_sink = params->n_sink; A.scale = params->scale; A.drop = params->drop_remainder;
    A.q4 = params->int4_pages;
    A.slice = P.slice; A.nslice = P.nslice; A.nwin = P.nwin; A.nslot = P.nslot;
    A.seq0 = 0; A.rows_per_seq = 1; A.pos0 = 0;
}

// Prefill rows are processed in groups of this many rows per launch.
constexpr int kPrefillRows = 256;

}  // namespace lodi

using namespace lodi;

namespace lodi {
// Every check of a decode call except its workspace (host only, nothing enqueued).
static int check_decode_args(const lod_params* params, const lod_index* index, const lod_kv& kv,
                             const void* q, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                             const float* out) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!index || !index->mem || !q || !seq_lens || !out || batch <= 0 || max_seq_len <= 0)
        return LOD_ERR_ARG;
    if (!aligned16(q) || !aligned16(out)) return LOD_ERR_ARG;
    if ((rc = check_kv_view(params, kv, max_seq_len)) != LOD_OK) return rc;
    if (batch != index->batch) return LOD_ERR_ARG;
    if (built_chunks(params, (int64_t)max_seq_len - 1) > index->max_chunks) return LOD_ERR_ARG;
    if (index->bytes < make_layout(params, index->batch, index->max_chunks).total) return LOD_ERR_WORKSPACE;
    return LOD_OK;
}
}  // namespace lodi

extern "C" int lod_attend_decode(const lod_params* params, const lod_index* index, lod_kv kv,
                                 const void* q, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_seq_len, float* out, int32_t* sel_groups,
                                 int32_t* sel_pages, void* ws, size_t ws_bytes, void* stream) {
    const int rc = check_decode_args(params, index, kv, q, seq_lens, batch, max_seq_len, out);
    if (rc != LOD_OK) return rc;
    const lod_index_layout_t L = make_layout(params, index->batch, index->max_chunks);
    const DecodePlan P = plan_decode(params, batch, max_seq_len);
    if (!ws || ws_bytes < P.bytes) return LOD_ERR_WORKSPACE;
    DecodeArgs A;
    fill_decode_args(A, params, index, L, kv, P, ws);
    A.q = q; A.seq_lens = seq_lens; A.max_seq_len = max_seq_len;
    A.out = out; A.sel_groups = sel_groups; A.sel_pages = sel_pages;
    return dispatch_decode(params, A, batch, reinterpret_cast<hipStream_t>(stream));
}

// Workspace of lod_attend_decode_noalloc: a fixed device array, one copy per device
// (loaded with the library's code object and held until the process ends).  In host code
// the symbol is only a stand-in: its device address for the current device comes from
// hipGetSymbolAddress, taken once per device and kept in noalloc_ws[].
static __device__ __align__(256) unsigned char scratch[LOD_NOALLOC_WS_BYTES];

namespace lodi {
constexpr int kNoallocDevices = 64;
static std::mutex noalloc_mu;
static void* noalloc_ws[kNoallocDevices];

// Device address of `scratch` on the current device (looked up on first use).
static int noalloc_workspace(void** ws) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LOD_ERR_HIP;
    if (dev >= kNoallocDevices) return LOD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_ws[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LOD_ERR_HIP;
        noalloc_ws[dev] = p;
    }
    *ws = noalloc_ws[dev];
    return LOD_OK;
}
}  // namespace lodi

extern "C" int lod_attend_decode_noalloc(const lod_params* params, const lod_index* index, lod_kv kv,
                                         const void* q, const int32_t* seq_lens, int32_t batch,
                                         int32_t max_seq_len, float* out, int32_t* sel_groups,
                                         int32_t* sel_pages, void* stream) {
    int rc = check_decode_args(params, index, kv, q, seq_lens, batch, max_seq_len, out);
    if (rc != LOD_OK) return rc;
    if (plan_decode(params, batch, max_seq_len).bytes > (size_t)LOD_NOALLOC_WS_BYTES) return LOD_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((rc = noalloc_workspace(&ws)) != LOD_OK) return rc;
    return lod_attend_decode(params, index, kv, q, seq_lens, batch, max_seq_len, out, sel_groups, sel_pages,
                             ws, (size_t)LOD_NOALLOC_WS_BYTES, stream);
}

// Row-by-row prefill (fp32 caches): each group of up to kPrefillRows rows runs as that
// many decode queries.  Arguments are validated by the caller.
int lodi::prefill_rows_ws_bytes(const lod_params* params, int32_t n_q, int32_t max_tokens, size_t* bytes) {
    *bytes = plan_decode(params, n_q < kPrefillRows ? n_q : kPrefillRows, max_tokens).bytes;
    return LOD_OK;
}

int lodi::prefill_rows(const lod_params* params, const lod_index* index, lod_kv kv, const void* q,
                       int32_t q_start, int32_t n_q, int32_t batch, float* out, int32_t* sel_groups,
                       int32_t* sel_pages, void* ws, size_t ws_bytes, void* stream) {
    int rc = LOD_OK;
    const int64_t end = (int64_t)q_start + n_q;
    const lod_index_layout_t L = make_layout(params, index->batch, index->max_chunks);
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
    if (!aligned16(q) || !aligned16(out)) return LOD_ERR_ARG;
    if ((rc = check_kv_view(params, kv, max_seq_len)) != LOD_OK) return rc;
    const DensePlan P = plan_dense(params, batch, max_seq_len);
    if (!ws || ws_bytes < P.bytes) return LOD_ERR_WORKSPACE;
    DenseArgs A;
    A.k = kv.k; A.v = kv.v;
    set_kv_map(A, kv);
    A.q = q; A.seq_lens = seq_lens; A.max_seq_len = max_seq_len;
    A.part = reinterpret_cast<float*>(ws);
    A.out = nullptr;
    A.Hq = params->n_q_heads; A.Hkv = params->n_kv_heads;
    A.rows_per_wg = P.rows_per_wg; A.nsplit = P.nsplit; A.scale = params->scale;
    A.seq0 = 0; A.rows_per_seq = 1; A.pos0 = 0;
    return dispatch_dense(params, A, out, batch, reinterpret_cast<hipStream_t>(stream));
}

// Dense causal prefill of fp32 caches: one workgroup per (row, KV head) on the VALU.
int lodi::dense_prefill_valu(const lod_params* params, lod_kv kv, const void* q, int32_t q_start,
                             int32_t n_q, int32_t batch, float* out, void* stream) {
    int rc = LOD_OK;
    const int64_t end = (int64_t)q_start + n_q;
    DenseArgs A;
    A.k = kv.k; A.v = kv.v;
    set_kv_map(A, kv);
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
