// lod_build.hip -- subsystem (a): per-chunk clustering, page split and summaries.
//
// "After every chunk of 256 tokens, similar keys are grouped into centroid clusters.
// Within each cluster, keys are divided into pages of 16 keys each" and each level
// keeps an average key and value ("Level of Detail Attention", How It Works).
//
// One workgroup (256 threads, 4 waves) per (chunk, KV head, sequence).  The chunk's
// non-sink keys sit in LDS in their storage type; during the assignment step every
// thread keeps its own key in fp32 registers and reads the centroids as LDS
// broadcasts, so the G squared-distance fma chains run in index order exactly as the
// definition states.  The update step gives one thread per (group, dimension), which
// sums the members in position order, so the means are bit-reproducible.
#include "lod_device.h"

namespace lodi {

struct BuildArgs {
    const void* k;
    const void* v;
    int64_t sb, st, sh;
    char* index;  // lod_index.mem
    lod_index_layout_t L;
    int max_chunks;
    int chunk_begin, n_chunks;
    int n_kv_heads, G, n_sink, iters;
    const int32_t* assign_in;
    int32_t* assign_out;
};

// LDS budget: keys (or values) of one chunk in storage type + centroids + bookkeeping.
template <typename T, int GMAX>
struct BuildSmem {
    T x[kChunk][kD];
    float mu[GMAX][kD];
    int32_t a[kChunk];       // group of member i
    int32_t cnt[GMAX];
    int32_t goff[GMAX + 1];  // first perm entry of each group
    int32_t gpg[GMAX + 1];   // first page slot of each group
    int32_t pst[kChunk / kPage + GMAX + 1];
    int32_t perm[kChunk];    // member indices ordered by (group, position)
    int32_t wcnt[kThreads / 64][GMAX];
};

// One Lloyd update: mu_j = fp32 mean of members with a_i == j, in member order.
// Thread (j, t) pairs: t = tid % 128, j = tid / 128 + 2k.
template <typename T, int GMAX>
__device__ void group_means(BuildSmem<T, GMAX>& s, int m, int G, bool write_mu, float* out_sum,
                            int* out_cnt) {
    const int tid = threadIdx.x;
    const int t = tid & (kD - 1);
    const int j0 = tid >> 7;
    constexpr int JP = (GMAX + 1) / 2;
    float sum[JP];
    int cnt[JP];
#pragma unroll
    for (int k = 0; k < JP; ++k) { sum[k] = 0.0f; cnt[k] = 0; }
    // members in position order; LDS loads are issued eight at a time
    int i = 0;
    for (; i + 8 <= m; i += 8) {
        int ai[8];
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            ai[u] = s.a[i + u];
            x[u] = Elt<T>::to_f32(s.x[i + u][t]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int k = 0; k < JP; ++k)
                if (ai[u] == j0 + 2 * k) { sum[k] = sum[k] + x[u]; cnt[k] += 1; }
    }
    for (; i < m; ++i) {
        const int ai = s.a[i];
        const float x = Elt<T>::to_f32(s.x[i][t]);
#pragma unroll
        for (int k = 0; k < JP; ++k)
            if (ai == j0 + 2 * k) { sum[k] = sum[k] + x; cnt[k] += 1; }
    }
#pragma unroll
    for (int k = 0; k < JP; ++k) {
        const int j = j0 + 2 * k;
        if (j < G) {
            if (write_mu && cnt[k] > 0) s.mu[j][t] = sum[k] / (float)cnt[k];
            if (out_sum) out_sum[j * kD + t] = cnt[k] > 0 ? sum[k] / (float)cnt[k] : 0.0f;
            if (out_cnt && t == 0) out_cnt[j] = cnt[k];
        }
    }
}

// Assignment step: member i (one thread) -> argmin_j of the fma chain of (x - mu_j)^2.
template <typename T, int GMAX>
__device__ void assign_step(BuildSmem<T, GMAX>& s, const float* xr, int m, int G) {
    const int i = threadIdx.x;
    float acc[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int t = 0; t < kD; t += 4) {
#pragma unroll
        for (int j = 0; j < GMAX; ++j) {
            if (j < G) {
                const float4 mu = *reinterpret_cast<const float4*>(&s.mu[j][t]);
                float d0 = xr[t] - mu.x, d1 = xr[t + 1] - mu.y;
                float d2 = xr[t + 2] - mu.z, d3 = xr[t + 3] - mu.w;
                acc[j] = __builtin_fmaf(d0, d0, acc[j]);
                acc[j] = __builtin_fmaf(d1, d1, acc[j]);
                acc[j] = __builtin_fmaf(d2, d2, acc[j]);
                acc[j] = __builtin_fmaf(d3, d3, acc[j]);
            }
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

// Mean over the members of page slot e / kD at dimension e % kD (position order;
// the member indices are fetched before the values so the LDS loads overlap).
template <typename T, int GMAX>
__device__ __forceinline__ float page_mean(BuildSmem<T, GMAX>& s, int e) {
    const int sl = e / kD, t = e % kD;
    const int b0 = s.pst[sl], n = s.pst[sl + 1] - b0;
    int idx[kPage];
#pragma unroll
    for (int q = 0; q < kPage; ++q) idx[q] = q < n ? s.perm[b0 + q] : 0;
    float x[kPage];
#pragma unroll
    for (int q = 0; q < kPage; ++q) x[q] = Elt<T>::to_f32(s.x[idx[q]][t]);
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < kPage; ++q)
        if (q < n) acc = acc + x[q];
    return n > 0 ? acc / (float)n : 0.0f;
}

// Load the chunk's members (positions >= n_sink) of K or V into LDS.
template <typename T, int GMAX>
__device__ void load_members(BuildSmem<T, GMAX>& s, const T* base, int64_t st, int first_off,
                             int m) {
    constexpr int P16 = Elt<T>::kPer16;
    constexpr int CPR = kD / P16;  // 16-byte chunks per row
    for (int c = threadIdx.x; c < m * CPR; c += kThreads) {
        const int i = c / CPR, col = c % CPR;
        const T* src = base + (int64_t)(first_off + i) * st + col * P16;
        *reinterpret_cast<uint4*>(&s.x[i][col * P16]) = *reinterpret_cast<const uint4*>(src);
    }
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

    const T* kbase = reinterpret_cast<const T*>(A.k) + b * A.sb + h * A.sh + (int64_t)c * kChunk * A.st;
    const T* vbase = reinterpret_cast<const T*>(A.v) + b * A.sb + h * A.sh + (int64_t)c * kChunk * A.st;

    load_members(s, kbase, A.st, first_off, m);
    __syncthreads();

    if (A.assign_in) {
        const int32_t* ain = A.assign_in + ((unit * A.n_chunks) + blockIdx.x) * (int64_t)kChunk;
        if (tid < m) {
            int g = ain[first_off + tid];
            s.a[tid] = g < 0 ? 0 : (g >= G ? G - 1 : g);
        }
        __syncthreads();
    } else {
        // seeds: mu_j = x[floor(j*m/G)]
        for (int e = tid; e < G * kD; e += kThreads) {
            const int j = e / kD, t = e % kD;
            s.mu[j][t] = Elt<T>::to_f32(s.x[(j * m) / G][t]);
        }
        // this thread's own key in fp32 registers
        float xr[kD];
        {
            const int i = tid < m ? tid : 0;
#pragma unroll
            for (int t = 0; t < kD; ++t) xr[t] = Elt<T>::to_f32(s.x[i][t]);
        }
        __syncthreads();
        for (int it = 0; it < A.iters; ++it) {
            assign_step(s, xr, m, G);
            __syncthreads();
            group_means(s, m, G, true, nullptr, nullptr);
            __syncthreads();
        }
    }

    // Final means of keys (the centroids of the last update, recomputed the same way).
    float* gmean = &s.mu[0][0];  // reuse: group means of keys, then of values
    group_means(s, m, G, false, gmean, s.cnt);
    __syncthreads();

    // Layout: group offsets, page slots, ranks -> perm, page starts.
    if (tid == 0) {
        int o = 0, pg = 0;
        for (int j = 0; j < G; ++j) {
            s.goff[j] = o;
            s.gpg[j] = pg;
            for (int q = 0; q * kPage < s.cnt[j]; ++q) s.pst[pg + q] = o + q * kPage;
            o += s.cnt[j];
            pg += (s.cnt[j] + kPage - 1) / kPage;
        }
        s.goff[G] = o;
        s.gpg[G] = pg;
        for (int q = pg; q <= PS; ++q) s.pst[q] = o;
    }
    __syncthreads();
    {
        // rank of member tid among the earlier members of its group: ballot prefix
        // counts inside the wave plus the counts of earlier waves
        const int ai = tid < m ? s.a[tid] : -1;
        const int lane = tid & 63, wv = tid >> 6;
        int rank = 0;
        for (int j = 0; j < G; ++j) {
            const uint64_t mk = __ballot(ai == j);
            if (ai == j) rank = __popcll(mk & ((1ull << lane) - 1ull));
            if (lane == 0) s.wcnt[wv][j] = __popcll(mk);
        }
        __syncthreads();
        if (ai >= 0) {
            for (int w = 0; w < wv; ++w) rank += s.wcnt[w][ai];
            s.perm[s.goff[ai] + rank] = tid;
        }
    }
    __syncthreads();

    // Outputs: assignments, meta, group key means, ln n.
    const size_t gbase = (size_t)unit * A.max_chunks * G + (size_t)c * G;
    const size_t pbase = (size_t)unit * A.max_chunks * PS + (size_t)c * PS;
    T* gk = reinterpret_cast<T*>(A.index + A.L.gk) + gbase * kD;
    T* gv = reinterpret_cast<T*>(A.index + A.L.gv) + gbase * kD;
    float* gln = reinterpret_cast<float*>(A.index + A.L.gln) + gbase;
    float* gkn = reinterpret_cast<float*>(A.index + A.L.gkn) + gbase;
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
        const int j = e / kD;
        store_elt(&gk[e], s.cnt[j] > 0 ? gmean[e] : 0.0f);
    }
    if (tid < G) gln[tid] = s.cnt[tid] > 0 ? logf((float)s.cnt[tid]) : -INFINITY;
    // Norm bound of every stored mean key (the storage-rounded value), rounded up
    // generously; it only widens the error bound that MFMA ranking scores are checked
    // against.
    if (tid < G) {
        float ss = 0.0f;
        if (s.cnt[tid] > 0)
            for (int t = 0; t < kD; ++t) {
                const float x = Elt<T>::to_f32(Elt<T>::store_round(gmean[tid * kD + t]));
                ss = __builtin_fmaf(x, x, ss);
            }
        gkn[tid] = sqrtf(ss) * 1.0001f + 1e-30f;
    }
    // Page means of keys: thread (slot, t) sums <= 16 members in position order.
    for (int e = tid; e < PS * kD; e += kThreads) store_elt(&pk[e], page_mean(s, e));
    if (tid < PS) {
        const int n = s.pst[tid + 1] - s.pst[tid];
        pln[tid] = n > 0 ? logf((float)n) : -INFINITY;
    }
    __syncthreads();

    // Values: same means over the same members.
    load_members(s, vbase, A.st, first_off, m);
    __syncthreads();
    group_means(s, m, G, false, gmean, nullptr);
    for (int e = tid; e < PS * kD; e += kThreads) store_elt(&pv[e], page_mean(s, e));
    __syncthreads();
    for (int e = tid; e < G * kD; e += kThreads) {
        const int j = e / kD;
        store_elt(&gv[e], s.cnt[j] > 0 ? gmean[e] : 0.0f);
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
    if (kv.stride_t <= 0 || kv.stride_h < 0 || kv.stride_b < 0) return LOD_ERR_ARG;
    const int per16 = params->kv_dtype == LOD_BF16 ? 8 : 4;
    if ((kv.stride_t | kv.stride_h | kv.stride_b) % per16 != 0) return LOD_ERR_ARG;
    lod_index_layout_t L = make_layout(params, index->batch, index->max_chunks);
    if (index->bytes < L.total) return LOD_ERR_WORKSPACE;
    if (n_chunks == 0) return LOD_OK;
    BuildArgs A;
    A.k = kv.k; A.v = kv.v; A.sb = kv.stride_b; A.st = kv.stride_t; A.sh = kv.stride_h;
    A.index = reinterpret_cast<char*>(index->mem);
    A.L = L;
    A.max_chunks = index->max_chunks;
    A.chunk_begin = chunk_begin; A.n_chunks = n_chunks;
    A.n_kv_heads = params->n_kv_heads; A.G = params->groups_per_chunk;
    A.n_sink = params->n_sink; A.iters = params->kmeans_iters;
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
