// lod_build.hip -- subsystem (a): per-chunk clustering, page split and summaries.
//
// After every 256-token chunk the keys are clustered into groups, each group is cut
// into pages of 16 keys, and every group and page keeps its mean key and mean value
// ("Level of Detail Attention", How It Works).
//
// One workgroup (256 threads, 4 waves) per (chunk, KV head, sequence).  The chunk's
// non-sink keys sit in LDS in their storage type.
//
// Assignment (argmin over centroids of the squared distance, an fp32 fma chain over
// the dimensions in index order, ties to the lowest group):
//   bf16 keys: the distances |x|^2 + |mu|^2 - 2 x.mu come from MFMA (centroids split
//     into bf16 hi + lo parts) together with a bound on their distance from the
//     canonical chain.  A point whose nearest centroid is certain under that bound is
//     assigned directly; the others (rare, plus exact ties) run the canonical chains,
//     one 16-lane subgroup per point.  The result is the canonical argmin.
//   fp32 keys: every thread runs the canonical chains of its own key.
// Update: members are sorted by group with wave ballots (position order inside a
// group) and thread (group, dimension) sums just its group's members in position
// order, so the means are bit-reproducible.
#include "lod_mfma.h"

namespace lodi {

struct BuildArgs {
    const void* k;
    const void* v;
    int64_t sb, st, sh;
    const int32_t* btab;  // paged view: block table [batch][maxb], else null
    int bshift, maxb;
    char* index;  // lod_index.mem
    lod_index_layout_t L;
    int max_chunks;
    int chunk_begin, n_chunks;
    int n_kv_heads, G, n_sink, iters;
    int int4;  // three-tier INT4: store 4-bit codes of every clustered row
    const int32_t* assign_in;
    int32_t* assign_out;
};

constexpr int kMuStride = kD + 4;  // centroid row stride: rows start 4 banks apart

// Bound on |D_mfma - D_canonical| / (|x|^2 + |mu|^2) for the squared distance D of a
// bf16 key x and an fp32 centroid mu (u = 2^-24):
//   |x.(mu - hi - lo)| <= 2^-16 |x||mu|; MFMA accumulation of the 256 exact products
//   <= gamma_256 (1 + 2^-8) |x||mu|; |x|^2 and |mu|^2 each within gamma_128 of
//   themselves; the final add and subtract within 2u (|x|^2 + |mu|^2 + 2|x.mu|); the
//   canonical chain is within (gamma_128 + 3u) D of the exact D, and
//   D <= 2 (|x|^2 + |mu|^2).  With 2|x||mu| <= |x|^2 + |mu|^2 the total is below
//   5.5e-5; the constant is 2.44e-4.
constexpr float kDistErrC = 32.0f * 128.0f / 16777216.0f;

template <typename T, int GMAX>
struct BuildSmem {
    alignas(16) T x[kChunk][kD];  // bf16: 16-byte chunks XOR-swizzled by row
    alignas(16) float mu[GMAX][kMuStride];
    alignas(16) bf16_t muh[GMAX][kD];  // bf16 hi / lo parts of mu (bf16 keys)
    alignas(16) bf16_t mul[GMAX][kD];
    float mun[GMAX][2];      // |mu_j|^2 over dimensions 0..63 and 64..127
    float xn[kChunk];        // |x_i|^2 (bf16 keys)
    int32_t a[kChunk];       // group of member i
    int32_t unc[kChunk];     // members whose nearest centroid is not certain
    int32_t nunc;
    int32_t chg[2];            // an assignment changed in the pass (by pass parity)
    int32_t gchg[2][GMAX];     // group j gained or lost a member in the pass
    int32_t cnt[GMAX];
    int32_t goff[GMAX + 1];  // first perm entry of each group
    int32_t gpg[GMAX + 1];   // first page slot of each group
    int32_t pst[kChunk / kPage + GMAX + 1];
    int32_t perm[kChunk];    // member indices ordered by (group, position)
    int32_t wcnt[kThreads / 64][GMAX];
};

// Column of element (i, t) in the LDS key/value tile.
template <typename T>
__device__ __forceinline__ int xcol(int i, int t) {
    if constexpr (sizeof(T) == 2)
        return (((t >> 3) ^ (i & 15)) << 3) | (t & 7);
    else
        return t;
}
template <typename T, int GMAX>
__device__ __forceinline__ float xat(const BuildSmem<T, GMAX>& s, int i, int t) {
    return Elt<T>::to_f32(s.x[i][xcol<T>(i, t)]);
}

// Load the chunk's members (positions >= n_sink) of K or V into LDS.
template <typename T, int GMAX>
__device__ void load_members(BuildSmem<T, GMAX>& s, const BuildArgs& A, const T* base, int b, int t0, int first_off,
                             int m) {
    constexpr int P16 = Elt<T>::kPer16;
    constexpr int CPR = kD / P16;  // 16-byte chunks per row
    for (int c = threadIdx.x; c < m * CPR; c += kThreads) {
        const int i = c / CPR, col = c % CPR;
        const T* src = base + kv_row_rt(A, b, t0 + first_off + i) + col * P16;
        *reinterpret_cast<uint4*>(&s.x[i][xcol<T>(i, col * P16)]) = *reinterpret_cast<const uint4*>(src);
    }
}

// Members grouped by assignment: cnt[j], goff[j] (exclusive prefix) and perm, which
// lists every group's members in position order; gpg[j] (first page slot of group j)
// and pst (first perm entry of every page slot, PS + 1 entries).  Ranks come from wave
// ballots.
template <typename T, int GMAX>
__device__ void sort_members(BuildSmem<T, GMAX>& s, int m, int G, int PS, int next = 0) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ai = tid < m ? s.a[tid] : -1;
    int rank = 0;
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
        if (j < G) {
            const uint64_t mk = __ballot(ai == j);
            if (ai == j) rank = __popcll(mk & ((1ull << lane) - 1ull));
            if (lane == 0) s.wcnt[wv][j] = __popcll(mk);
        }
    }
    // flags of the next pass (their last reader finished before this pass began)
    if (tid < GMAX) s.gchg[next][tid] = 0;
    if (tid == 0) { s.chg[next] = 0; s.nunc = 0; }
    __syncthreads();
    if (ai >= 0) {
        int off = 0;
#pragma unroll
        for (int j = 0; j < GMAX; ++j)
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w)
                if (j < ai || (j == ai && w < wv)) off += s.wcnt[w][j];
        s.perm[off + rank] = tid;
    }
    if (tid <= G) {
        // counts, member offsets, page slots (pages of 16 in member order) and page starts
        int c[GMAX];
#pragma unroll
        for (int j = 0; j < GMAX; ++j) {
            c[j] = 0;
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w) c[j] += j < G ? s.wcnt[w][j] : 0;
        }
        int off = 0, pg = 0, n = 0;
#pragma unroll
        for (int j = 0; j < GMAX; ++j) {
            if (j < tid) { off += c[j]; pg += (c[j] + kPage - 1) / kPage; }
            if (j == tid) n = c[j];
        }
        s.goff[tid] = off;
        s.gpg[tid] = pg;
        if (tid < G) {
            s.cnt[tid] = n;
            for (int q = 0; q * kPage < n; ++q) s.pst[pg + q] = off + q * kPage;
        } else {
            for (int q = pg; q <= PS; ++q) s.pst[q] = off;
        }
    }
    __syncthreads();
}

// Group means over the sorted members into s.mu: thread (j, t) with t = tid % 128 and
// j = tid / 128 + 2k sums its group's members in position order (fp32, plain adds),
// then divides by the count.  j is uniform in a wave.  only: if non-null, groups with
// only[j] == 0 keep their row (their member set did not change).  keep_empty: leave an
// empty group's row untouched (a Lloyd update), else write 0.  split: also store the
// bf16 hi/lo parts and the squared norm halves used by the MFMA assignment.
template <typename T, int GMAX>
__device__ void group_means(BuildSmem<T, GMAX>& s, int G, bool keep_empty, bool split = false,
                            const int32_t* only = nullptr) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int t = tid & (kD - 1);
    for (int j = tid >> 7; j < G; j += 2) {
        if (only && !only[j]) continue;  // uniform in the wave
        const int b0 = s.goff[j], n = s.cnt[j];
        float acc = 0.0f;
        int q = 0;
        for (; q + 8 <= n; q += 8) {
            int idx[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) idx[u] = s.perm[b0 + q + u];
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = xat(s, idx[u], t);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc = acc + x[u];
        }
        for (; q < n; ++q) acc = acc + xat(s, s.perm[b0 + q], t);
        float mu = s.mu[j][t];
        if (n > 0) mu = acc / (float)n;
        else if (!keep_empty) mu = 0.0f;
        s.mu[j][t] = mu;
        if constexpr (sizeof(T) == 2) {
            if (split) {
                const bf16_t h = f32_to_bf16_rne(mu);
                s.muh[j][t] = h;
                s.mul[j][t] = f32_to_bf16_rne(mu - bf16_bits_to_f32(h));
                const float sq = wave_sum_f32(mu * mu, 64);
                if (lane == 0) s.mun[j][(tid >> 6) & 1] = sq;
            }
        }
    }
}

// Canonical squared distance of member i to centroid j (fma chain in index order).
template <typename T, int GMAX>
__device__ __forceinline__ float canonical_dist(const BuildSmem<T, GMAX>& s, int i, int j) {
    float acc = 0.0f;
#pragma unroll 4
    for (int t = 0; t < kD; t += 4) {
        const float4 mu = *reinterpret_cast<const float4*>(&s.mu[j][t]);
        const float d0 = xat(s, i, t) - mu.x, d1 = xat(s, i, t + 1) - mu.y;
        const float d2 = xat(s, i, t + 2) - mu.z, d3 = xat(s, i, t + 3) - mu.w;
        acc = __builtin_fmaf(d0, d0, acc);
        acc = __builtin_fmaf(d1, d1, acc);
        acc = __builtin_fmaf(d2, d2, acc);
        acc = __builtin_fmaf(d3, d3, acc);
    }
    return acc;
}

// Assignment of bf16 keys on MFMA with a certified argmin.  Wave w handles members
// 64w .. 64w+63 as four blocks of 16; D^T = M X^T puts the centroids on MFMA rows, so
// lane l holds groups 4(l/16)+r of member l%16 of the block.  A member is assigned
// when exactly one group's lower bound reaches the smallest upper bound; otherwise it
// is queued for the canonical chains.
template <int GMAX>
__device__ void assign_mfma(BuildSmem<bf16_t, GMAX>& s, int m, int G, int pass) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int row = l & 15;  // A-operand centroid row of this lane
    bf16x8_t ahi[4], alo[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        if (row < GMAX) {
            ahi[kk] = *reinterpret_cast<const bf16x8_t*>(&s.muh[row][32 * kk + 8 * (l >> 4)]);
            alo[kk] = *reinterpret_cast<const bf16x8_t*>(&s.mul[row][32 * kk + 8 * (l >> 4)]);
        } else {
            ahi[kk] = zero_bf16x8();
            alo[kk] = zero_bf16x8();
        }
    }
    float mun[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = 4 * (l >> 4) + r;
        mun[r] = j < GMAX ? s.mun[j < GMAX ? j : 0][0] + s.mun[j < GMAX ? j : 0][1] : 0.0f;
    }

#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
        const int p = 64 * w + 16 * pb + (l & 15);  // member of this lane's column
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8_t b =
                *reinterpret_cast<const bf16x8_t*>(&s.x[p][((4 * kk + (l >> 4)) ^ (p & 15)) << 3]);
            acc = mfma16(ahi[kk], b, acc);
            acc = mfma16(alo[kk], b, acc);
        }
        const float xn = s.xn[p];
        float lb[4];
        float minub = INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 4 * (l >> 4) + r;
            const float nrm = xn + mun[r];
            const float dd = nrm - 2.0f * acc[r];
            const float e = kDistErrC * nrm;
            lb[r] = j < G ? dd - e : INFINITY;
            minub = fminf(minub, j < G ? dd + e : INFINITY);
        }
        minub = fminf(minub, __shfl_xor(minub, 16, 64));
        minub = fminf(minub, __shfl_xor(minub, 32, 64));
        // candidates: (count << 8) | (group + 1 of a lane with exactly one), summed
        int nc = 0, jc = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (lb[r] <= minub) { ++nc; jc = 4 * (l >> 4) + r + 1; }
        int pk = (nc << 8) | (nc == 1 ? jc : 0);
        pk += __shfl_xor(pk, 16, 64);
        pk += __shfl_xor(pk, 32, 64);
        if ((l >> 4) == 0 && p < m) {
            if ((pk >> 8) == 1) {
                const int j = (pk & 255) - 1, old = s.a[p];
                if (j != old) {
                    s.a[p] = j;
                    s.chg[pass] = 1;
                    s.gchg[pass][j] = 1;
                    if (old >= 0) s.gchg[pass][old] = 1;
                }
            } else {
                s.unc[atomicAdd(&s.nunc, 1)] = p;
            }
        }
    }
}

// Canonical assignment of the queued members: one 16-lane subgroup per member, lane q
// runs the chain of centroid q; argmin with ties to the lowest q.
template <int GMAX>
__device__ void assign_uncertain(BuildSmem<bf16_t, GMAX>& s, int G, int pass) {
    const int tid = threadIdx.x, q = tid & 15;
    const int n = s.nunc;
    for (int u0 = 0; u0 < n; u0 += kThreads / 16) {
        const int u = u0 + (tid >> 4);
        const bool live = u < n;  // uniform per subgroup
        const int i = live ? s.unc[u] : 0;
        float d = (live && q < G && q < GMAX) ? canonical_dist(s, i, q < GMAX ? q : 0) : INFINITY;
        int j = q;
#pragma unroll
        for (int sh = 1; sh < 16; sh <<= 1) {
            const float od = __shfl_xor(d, sh, 64);
            const int oj = __shfl_xor(j, sh, 64);
            if (od < d || (od == d && oj < j)) { d = od; j = oj; }
        }
        if (live && q == 0) {
            const int old = s.a[i];
            if (j != old) {
                s.a[i] = j;
                s.chg[pass] = 1;
                s.gchg[pass][j] = 1;
                if (old >= 0) s.gchg[pass][old] = 1;
            }
        }
    }
}

// Assignment step of fp32 keys: member i (one thread) -> argmin_j of the fma chain of
// (x - mu_j)^2; every thread runs the GMAX chains (centroids j >= G are zero and never
// chosen), reading the centroids as LDS broadcasts.
template <int GMAX>
__device__ void assign_valu(BuildSmem<float, GMAX>& s, const float* xr, int m, int G) {
    const int i = threadIdx.x;
    float acc[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int t = 0; t < kD; t += 4) {
#pragma unroll
        for (int j = 0; j < GMAX; ++j) {
            const float4 mu = *reinterpret_cast<const float4*>(&s.mu[j][t]);
            const float d0 = xr[t] - mu.x, d1 = xr[t + 1] - mu.y;
            const float d2 = xr[t + 2] - mu.z, d3 = xr[t + 3] - mu.w;
            acc[j] = __builtin_fmaf(d0, d0, acc[j]);
            acc[j] = __builtin_fmaf(d1, d1, acc[j]);
            acc[j] = __builtin_fmaf(d2, d2, acc[j]);
            acc[j] = __builtin_fmaf(d3, d3, acc[j]);
        }
    }
    if (i < m) {
        int best = 0;
        float bd = acc[0];
#pragma unroll
        for (int j = 1; j < GMAX; ++j)
            if (j < G && acc[j] < bd) { bd = acc[j]; best = j; }
        s.a[i] = best;
    }
}

// Page means, and optionally group means, in one pass over the sorted members: thread
// (j, t) with t = tid % 128 and j = tid / 128 + 2k walks group j's members in position
// order, one page (16 members) at a time, keeping two fp32 sums: the page's (stored at
// every page end) and, with groups, the group's (into s.mu at the end; 0 when empty).
// Page slots past the chunk's last page are stored as 0.
// Both are plain sequential sums, the same as summing each set on its own.
template <typename T, int GMAX>
__device__ void summaries(BuildSmem<T, GMAX>& s, int G, int PS, T* pdst, bool groups) {
    const int tid = threadIdx.x;
    const int t = tid & (kD - 1);
    for (int sl = s.gpg[G] + (tid >> 7); sl < PS; sl += 2) store_elt(&pdst[(int64_t)sl * kD + t], 0.0f);
    for (int j = tid >> 7; j < G; j += 2) {
        const int b0 = s.goff[j], n = s.cnt[j], pg0 = s.gpg[j];
        float gacc = 0.0f;
        for (int q0 = 0; q0 < n; q0 += kPage) {
            const int np = min(kPage, n - q0);
            int idx[kPage];
#pragma unroll
            for (int u = 0; u < kPage; ++u) idx[u] = u < np ? s.perm[b0 + q0 + u] : 0;
            float x[kPage];
#pragma unroll
            for (int u = 0; u < kPage; ++u) x[u] = xat(s, idx[u], t);
            float pacc = 0.0f;
#pragma unroll
            for (int u = 0; u < kPage; ++u)
                if (u < np) {
                    pacc = pacc + x[u];
                    gacc = gacc + x[u];
                }
            store_elt(&pdst[(int64_t)(pg0 + q0 / kPage) * kD + t], pacc / (float)np);
        }
        if (groups) s.mu[j][t] = n > 0 ? gacc / (float)n : 0.0f;
    }
}

// Three-tier INT4 codes of the chunk's rows (bf16 keys or values in s.x, their group
// means in s.mu): member i (thread i) stores the residual from its group's stored mean
// (the mean rounded to bf16) as 128 4-bit codes at chunk-local position first_off + i,
// with scale max|r| / 7 and codes rint(r / scale) clamped to [-8, 7] (0 when the scale
// is 0); element 2j sits in the low nibble of byte j.  Sink positions get zero codes
// and scale.  This follows the page's note that centroid groups let clustered rows be
// stored at INT4 and decoded only for opened pages (section "Additional Benefits").
template <int GMAX>
__device__ void encode_rows_int4(const BuildSmem<bf16_t, GMAX>& s, int m, int first_off, uint8_t* q4,
                                 float* q4s) {
    const int tid = threadIdx.x;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    if (tid < first_off) {
#pragma unroll
        for (int u = 0; u < kD / 32; ++u) reinterpret_cast<uint4*>(q4 + (int64_t)tid * (kD / 2))[u] = zero;
        q4s[tid] = 0.0f;
    }
    if (tid >= m) return;
    const int i = tid, j = s.a[i];
    // residual of elements 8c .. 8c+7 (LDS reads; recomputed in the second pass)
    auto resid8 = [&](int c, float* r) {
        float f[8];
        Elt<bf16_t>::unpack(*reinterpret_cast<const uint4*>(&s.x[i][8 * (c ^ (i & 15))]), f);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            r[e] = f[e] - Elt<bf16_t>::to_f32(Elt<bf16_t>::store_round(s.mu[j][8 * c + e]));
    };
    float mx = 0.0f;
    for (int c = 0; c < kD / 8; ++c) {
        float r[8];
        resid8(c, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(r[e]));
    }
    const float sc = mx / 7.0f;
    uint32_t* dst = reinterpret_cast<uint32_t*>(q4 + (int64_t)(first_off + i) * (kD / 2));
    for (int c = 0; c < kD / 8; ++c) {
        float r[8];
        resid8(c, r);
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q = sc == 0.0f ? 0.0f : fminf(fmaxf(rintf(r[e] / sc), -8.0f), 7.0f);
            v |= ((uint32_t)(int)q & 0xfu) << (4 * e);
        }
        dst[c] = v;
    }
    q4s[first_off + i] = sc;
}

template <typename T, int GMAX>
__global__ __launch_bounds__(kThreads) void build_chunk_kernel(BuildArgs A) {
    __shared__ BuildSmem<T, GMAX> s;
    const int c = A.chunk_begin + blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int G = A.G;
    const int tid = threadIdx.x;
    const int first_off = (c == 0) ? A.n_sink : 0;  // sinks are never clustered
    const int m = kChunk - first_off;
    const int PS = A.L.page_slots;
    const int64_t unit = (int64_t)b * A.n_kv_heads + h;

    // head h of the cache; rows through kv_row_rt (positions c * kChunk + ...)
    const T* kbase = reinterpret_cast<const T*>(A.k) + h * A.sh;
    const T* vbase = reinterpret_cast<const T*>(A.v) + h * A.sh;
    const int t0 = c * kChunk;

    load_members(s, A, kbase, b, t0, first_off, m);
    if (tid == 0) s.nunc = 0;
    __syncthreads();

    if (A.assign_in) {
        const int32_t* ain = A.assign_in + ((unit * A.n_chunks) + blockIdx.x) * (int64_t)kChunk;
        if (tid < m) {
            int g = ain[first_off + tid];
            s.a[tid] = g < 0 ? 0 : (g >= G ? G - 1 : g);
        }
        __syncthreads();
        sort_members(s, m, G, PS);
        group_means(s, G, false);
        __syncthreads();
    } else {
        // seeds: mu_j = x[floor(j*m/G)]; unused centroid rows are zero
        for (int e = tid; e < GMAX * kD; e += kThreads) {
            const int j = e / kD, t = e % kD;
            const float mu = j < G ? xat(s, (j * m) / G, t) : 0.0f;
            s.mu[j][t] = mu;
            if constexpr (sizeof(T) == 2) {
                const bf16_t h = f32_to_bf16_rne(mu);
                s.muh[j][t] = h;
                s.mul[j][t] = f32_to_bf16_rne(mu - bf16_bits_to_f32(h));
                const float sq = wave_sum_f32(mu * mu, 64);  // e / 64 is uniform per wave
                if ((tid & 63) == 0) s.mun[j][(e >> 6) & 1] = sq;
            }
        }
        if constexpr (sizeof(T) == 2) {
            // |x_i|^2 for the distance bound (any summation order will do)
            float ss = 0.0f;
            const int i = tid < m ? tid : 0;
            uint4 u[kD / 8];
#pragma unroll
            for (int c = 0; c < kD / 8; ++c) u[c] = *reinterpret_cast<const uint4*>(&s.x[i][8 * c]);
#pragma unroll
            for (int c = 0; c < kD / 8; ++c) {
                float f[8];
                Elt<bf16_t>::unpack(u[c], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
            }
            s.xn[tid] = ss;
            s.a[tid] = -1;
            if (tid < GMAX) { s.gchg[0][tid] = 0; s.gchg[1][tid] = 0; }
            if (tid < 2) s.chg[tid] = 0;
            __syncthreads();
            // Lloyd passes; a pass that changes no assignment reached a fixed point, and
            // every later pass would repeat it, so the loop stops there.
            for (int it = 0; it < A.iters; ++it) {
                const int pass = it & 1;
                assign_mfma(s, m, G, pass);
                __syncthreads();
                if (s.nunc > 0) {  // uniform: read after the barrier
                    assign_uncertain(s, G, pass);
                    __syncthreads();
                }
                if (!s.chg[pass]) break;  // uniform
                sort_members(s, m, G, PS, pass ^ 1);
                group_means(s, G, true, true, s.gchg[pass]);
                __syncthreads();
            }
        } else {
            float xr[kD];
            {
                const int i = tid < m ? tid : 0;
#pragma unroll
                for (int t = 0; t < kD; ++t) xr[t] = xat(s, i, t);
            }
            __syncthreads();
            for (int it = 0; it < A.iters; ++it) {
                assign_valu(s, xr, m, G);
                __syncthreads();
                sort_members(s, m, G, PS);
                group_means(s, G, true);
                __syncthreads();
            }
        }
    }
    // s.mu holds the means of the final assignment (stored as 0 for empty groups).

    // Outputs: assignments, meta, group key means, ln n.
    const size_t gbase = (size_t)unit * A.max_chunks * G + (size_t)c * G;
    const size_t pbase = (size_t)unit * A.max_chunks * PS + (size_t)c * PS;
    T* gk = reinterpret_cast<T*>(A.index + A.L.gk) + gbase * kD;
    T* gv = reinterpret_cast<T*>(A.index + A.L.gv) + gbase * kD;
    float* gln = reinterpret_cast<float*>(A.index + A.L.gln) + gbase;
    float* gkn = reinterpret_cast<float*>(A.index + A.L.gkn) + gbase;
    int32_t* gpage = reinterpret_cast<int32_t*>(A.index + A.L.gpage) + gbase;
    T* pk = reinterpret_cast<T*>(A.index + A.L.pk) + pbase * kD;
    T* pv = reinterpret_cast<T*>(A.index + A.L.pv) + pbase * kD;
    float* pln = reinterpret_cast<float*>(A.index + A.L.pln) + pbase;
    int16_t* meta = reinterpret_cast<int16_t*>(A.index + A.L.meta) +
                    ((size_t)unit * A.max_chunks + c) * A.L.meta_stride;
    int8_t* asg = reinterpret_cast<int8_t*>(A.index + A.L.assign) +
                  ((size_t)unit * A.max_chunks + c) * kChunk;
    {
        const int off = tid;  // chunk-local position
        const int g = off < first_off ? -1 : s.a[off - first_off];
        asg[off] = (int8_t)g;
        if (A.assign_out) A.assign_out[((unit * A.n_chunks) + blockIdx.x) * (int64_t)kChunk + off] = g;
        meta[(G + 1) + (PS + 1) + off] = off < m ? (int16_t)(s.perm[off] + first_off) : (int16_t)-1;
        if (off <= G) meta[off] = (int16_t)s.gpg[off];
        if (off <= PS) meta[(G + 1) + off] = (int16_t)s.pst[off];
    }
    for (int e = tid; e < G * kD; e += kThreads) {
        const int j = e / kD, t = e % kD;
        store_elt(&gk[e], s.cnt[j] > 0 ? s.mu[j][t] : 0.0f);
    }
    if (tid < G) {
        gln[tid] = s.cnt[tid] > 0 ? logf((float)s.cnt[tid]) : -INFINITY;
        gpage[tid] = s.gpg[tid] | ((s.gpg[tid + 1] - s.gpg[tid]) << 16);
    }
    // Norm bound of every stored mean key (the storage-rounded value), rounded up
    // generously; it only widens the error bound that MFMA ranking scores are checked
    // against.
    {
        // 16 lanes per group, 8 dimensions each, then a 16-lane sum
        const int j = tid >> 4, q = tid & 15;
        float ss = 0.0f;
        if (j < G && s.cnt[j] > 0)
#pragma unroll
            for (int t = 8 * q; t < 8 * q + 8; ++t) {
                const float x = Elt<T>::to_f32(Elt<T>::store_round(s.mu[j][t]));
                ss = __builtin_fmaf(x, x, ss);
            }
        ss = wave_sum_f32(ss, 16);
        if (j < G && q == 0) gkn[j] = sqrtf(ss) * 1.0001f + 1e-30f;
    }
    // Values of the chunk: loads issued now, written to LDS once the keys are done.
    constexpr int P16 = Elt<T>::kPer16;
    constexpr int CPR = kD / P16;
    constexpr int VPT = kChunk * CPR / kThreads;  // 16-byte pieces per thread
    uint4 vreg[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int cidx = tid + kThreads * k, i = cidx / CPR, col = cidx % CPR;
        vreg[k] = i < m ? *reinterpret_cast<const uint4*>(vbase + kv_row_rt(A, b, t0 + first_off + i) + col * P16)
                        : make_uint4(0, 0, 0, 0);
    }
    // Page means of keys (group means of keys are already in s.mu).
    summaries(s, G, PS, pk, false);
    const int64_t qrow = ((int64_t)unit * A.max_chunks + c) * kChunk;  // first code row of the chunk
    if constexpr (sizeof(T) == 2) {
        if (A.int4)
            encode_rows_int4(s, m, first_off, reinterpret_cast<uint8_t*>(A.index + A.L.q4k) + qrow * (kD / 2),
                             reinterpret_cast<float*>(A.index + A.L.q4ks) + qrow);
    }
    if (tid < PS) {
        const int n = s.pst[tid + 1] - s.pst[tid];
        pln[tid] = n > 0 ? logf((float)n) : -INFINITY;
    }
    __syncthreads();

    // Values: same means over the same members (group means into s.mu, now free).
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int cidx = tid + kThreads * k, i = cidx / CPR, col = cidx % CPR;
        if (i < m) *reinterpret_cast<uint4*>(&s.x[i][xcol<T>(i, col * P16)]) = vreg[k];
    }
    __syncthreads();
    summaries(s, G, PS, pv, true);
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
        if (A.int4)
            encode_rows_int4(s, m, first_off, reinterpret_cast<uint8_t*>(A.index + A.L.q4v) + qrow * (kD / 2),
                             reinterpret_cast<float*>(A.index + A.L.q4vs) + qrow);
    }
    for (int e = tid; e < G * kD; e += kThreads) {
        const int j = e / kD, t = e % kD;
        store_elt(&gv[e], s.cnt[j] > 0 ? s.mu[j][t] : 0.0f);
    }
}

template <typename T, int GMAX>
static int launch_build(const BuildArgs& A, int batch, hipStream_t st) {
    dim3 grid(A.n_chunks, A.n_kv_heads, batch);
    hipLaunchKernelGGL((build_chunk_kernel<T, GMAX>), grid, dim3(kThreads), 0, st, A);
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}

}  // namespace lodi

using namespace lodi;

extern "C" int lod_build_chunk(const lod_params* params, const lod_index* index, lod_kv kv,
                               int32_t batch, int32_t chunk_begin, int32_t n_chunks,
                               const int32_t* assign_in, int32_t* assign_out, void* stream) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!index || !index->mem || !kv.k || !kv.v || batch <= 0 || chunk_begin < 0 || n_chunks < 0)
        return LOD_ERR_ARG;
    if (batch != index->batch || chunk_begin + (int64_t)n_chunks > index->max_chunks)
        return LOD_ERR_ARG;
    if ((rc = check_kv_view(params, kv, (chunk_begin + (int64_t)n_chunks) * params->chunk_size)) != LOD_OK)
        return rc;
    lod_index_layout_t L = make_layout(params, index->batch, index->max_chunks);
    if (index->bytes < L.total) return LOD_ERR_WORKSPACE;
    if (n_chunks == 0) return LOD_OK;
    BuildArgs A;
    A.k = kv.k; A.v = kv.v;
    set_kv_map(A, kv);
    A.index = reinterpret_cast<char*>(index->mem);
    A.L = L;
    A.max_chunks = index->max_chunks;
    A.chunk_begin = chunk_begin; A.n_chunks = n_chunks;
    A.n_kv_heads = params->n_kv_heads; A.G = params->groups_per_chunk;
    A.n_sink = params->n_sink; A.iters = params->kmeans_iters;
    A.int4 = params->int4_pages;
    A.assign_in = assign_in; A.assign_out = assign_out;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int G = A.G;
    if (params->kv_dtype == LOD_BF16) {
        if (G <= 4) return launch_build<bf16_t, 4>(A, batch, st);
        if (G <= 8) return launch_build<bf16_t, 8>(A, batch, st);
        return launch_build<bf16_t, 16>(A, batch, st);
    }
    if (G <= 4) return launch_build<float, 4>(A, batch, st);
    if (G <= 8) return launch_build<float, 8>(A, batch, st);
    return launch_build<float, 16>(A, batch, st);
}
