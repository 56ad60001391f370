/*
 * lod_oracle.c -- plain, slow CPU oracle for Level-of-Detail (LoD) attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the GPU library; the two only see the same seeded inputs.
 *
 * Source of the method: the blog post "Level of Detail Attention: allocating
 * resolution instead of sparsity" (featherless.ai), section "How It Works":
 *   - every 256-token chunk of keys is clustered into centroid groups, and each
 *     group is cut into pages of 16 keys, each with an average key and value;
 *   - a query scores the group centroids, opens the best eight groups, scores the
 *     page summaries inside them and opens the best two pages per group;
 *   - exact attention covers the opened pages, the recent block window and the
 *     sink tokens; every unopened group and every unopened page of an opened group
 *     enters the same softmax as its mean key/value repeated by its key count.
 * Where the post is silent, the readings below are used (each is also listed in
 * the design notes of the repository):
 *   clustering  = Lloyd's k-means on the chunk's non-sink keys, squared L2,
 *                 seeds mu_j = x[floor(j*m/G)], ties to the lowest group,
 *                 an empty group keeps its centroid and ends with n = 0;
 *   summaries   = fp32 sum in position order, correctly rounded divide by n,
 *                 round-to-nearest-even to the storage type;
 *   ranking     = unscaled fp32 fma chain over the head dimension in index
 *                 order, ties to the lower group / page id;
 *   window      = block granular: a query at p sees chunks floor(p/C)-W/C+1 ..
 *                 floor(p/C) exactly (its own causally);
 *   coarse term = logit scale*q.kbar + ln n with value vbar (n identical copies).
 * All softmax arithmetic is fp64.
 *
 * Sparsity ablation (drop_remainder = 1): the same selection, but the softmax holds
 * only the exact keys.  This is the token-removing alternative that the post's "The
 * Main Idea" section contrasts LoD with, and the attention of "Coarse Semantic Blocks
 * for Efficient Training-Free Sparse Attention" (readsearch.ai listing, abstract): a
 * query scores the centroids of key blocks and attends to the original keys of the
 * blocks it selects (with top_pages = 0, every key of an opened group).
 *
 * Three-tier INT4 (int4_pages = 1), from the post's "Additional Benefits" section:
 * because a group holds similar keys, the clustered rows are stored compressed as
 * 4-bit codes, and only the pages a query opens are decoded.  Reading: every clustered
 * key (value) row is stored as its residual from its group's stored mean key (value),
 * with one scale per row, s = max_t |r_t| / 7, and codes rint(r_t / s) clamped to
 * [-8, 7] (all 0 when s = 0); a decoded element is fma(s, code, mean).  Members of
 * opened pages enter the softmax decoded; sinks and the window stay exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_DOUBLE_COUNT (-2)
#define ORC_ERR_NOT_BUILT (-3)
#define ORC_ERR_NOMEM (-4)

typedef struct {
    int32_t d;          /* head dimension */
    int32_t chunk;      /* C: tokens per chunk (256) */
    int32_t page;       /* P: keys per page (16) */
    int32_t groups;     /* G: centroid groups per chunk */
    int32_t top_groups; /* groups opened per query (8) */
    int32_t top_pages;  /* pages opened per opened group (2); 0 = two-tier */
    int32_t window;     /* W: exact block window, a multiple of C */
    int32_t n_sink;     /* s: leading positions that are always exact */
    int32_t iters;      /* k-means rounds (10) */
    int32_t bf16_store; /* 1: summaries are rounded to bfloat16 */
    double scale;       /* softmax scale, 1/sqrt(d) */
    int32_t drop_remainder; /* 1: no coarse terms (sparsity ablation) */
    int32_t int4_pages;     /* 1: opened pages decoded from 4-bit codes (three-tier INT4) */
} orc_params;

/* Page slots per chunk: at most C/P full pages plus one partial page per group. */
int32_t orc_page_slots(const orc_params* P) { return P->chunk / P->page + P->groups; }

/* Round-to-nearest-even of an fp32 value to bfloat16, returned as fp32. */
float orc_round_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) {
        if (u & 0x007fffffu) u |= 0x00400000u; /* keep NaN a NaN */
        u &= 0xffff0000u;
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);
        u &= 0xffff0000u;
    }
    memcpy(&x, &u, 4);
    return x;
}

/* Ranking score: acc = fma(a_t, b_t, acc) for t = 0..d-1, fp32, from acc = 0. */
float orc_canonical_dot(const float* a, const float* b, int32_t d) {
    float acc = 0.0f;
    for (int32_t t = 0; t < d; ++t) acc = fmaf(a[t], b[t], acc);
    return acc;
}

/* k-means distance: acc = fma(x_t - mu_t, x_t - mu_t, acc), fp32, index order. */
static float kdist(const float* x, const float* mu, int32_t d) {
    float acc = 0.0f;
    for (int32_t t = 0; t < d; ++t) {
        float df = x[t] - mu[t];
        acc = fmaf(df, df, acc);
    }
    return acc;
}

static double dot64(const float* a, const float* b, int32_t d) {
    double acc = 0.0;
    for (int32_t t = 0; t < d; ++t) acc += (double)a[t] * (double)b[t];
    return acc;
}

/*
 * Lloyd's k-means on m points x[m][d] with G groups and `iters` rounds of
 * (assign, update).  assign[i] receives the assignment of the last round.
 * objective (nullable, `iters` entries) receives, for each round, the fp64 sum of
 * squared distances of the points to the centroids they were assigned to in that
 * round (the centroids of the previous round) -- the quantity Lloyd's iteration
 * never increases.
 */
int32_t orc_kmeans(const float* x, int32_t m, int32_t d, int32_t G, int32_t iters,
                   int32_t* assign, double* objective) {
    if (!x || !assign || m < 1 || d < 1 || G < 1 || iters < 1) return ORC_ERR_ARG;
    float* mu = (float*)malloc(sizeof(float) * (size_t)G * d);
    float* sum = (float*)malloc(sizeof(float) * (size_t)d);
    if (!mu || !sum) { free(mu); free(sum); return ORC_ERR_NOMEM; }
    for (int32_t j = 0; j < G; ++j) {
        int64_t seed = ((int64_t)j * m) / G;
        memcpy(mu + (size_t)j * d, x + (size_t)seed * d, sizeof(float) * (size_t)d);
    }
    for (int32_t it = 0; it < iters; ++it) {
        /* assignment step: nearest centroid, ties to the lowest index */
        for (int32_t i = 0; i < m; ++i) {
            const float* xi = x + (size_t)i * d;
            int32_t best = 0;
            float bestd = kdist(xi, mu, d);
            for (int32_t j = 1; j < G; ++j) {
                float dj = kdist(xi, mu + (size_t)j * d, d);
                if (dj < bestd) { bestd = dj; best = j; }
            }
            assign[i] = best;
        }
        if (objective) {
            double obj = 0.0;
            for (int32_t i = 0; i < m; ++i) {
                const float* xi = x + (size_t)i * d;
                const float* mj = mu + (size_t)assign[i] * d;
                for (int32_t t = 0; t < d; ++t) {
                    double df = (double)xi[t] - (double)mj[t];
                    obj += df * df;
                }
            }
            objective[it] = obj;
        }
        /* update step: fp32 mean of the members in position order; empty keeps */
        for (int32_t j = 0; j < G; ++j) {
            int32_t cnt = 0;
            for (int32_t t = 0; t < d; ++t) sum[t] = 0.0f;
            for (int32_t i = 0; i < m; ++i) {
                if (assign[i] != j) continue;
                const float* xi = x + (size_t)i * d;
                for (int32_t t = 0; t < d; ++t) sum[t] = sum[t] + xi[t];
                ++cnt;
            }
            if (cnt > 0)
                for (int32_t t = 0; t < d; ++t) mu[(size_t)j * d + t] = sum[t] / (float)cnt;
        }
    }
    free(mu);
    free(sum);
    return ORC_OK;
}

/* Mean of rows[idx[0..n)] of a [*][d] array: fp32 sum in the given order,
 * correctly rounded divide, then the storage rounding. */
static void canonical_mean(const float* rows, const int32_t* idx, int32_t n, int32_t d,
                           int32_t bf16, float* out) {
    for (int32_t t = 0; t < d; ++t) {
        float s = 0.0f;
        for (int32_t k = 0; k < n; ++k) s = s + rows[(size_t)idx[k] * d + t];
        float mval = s / (float)n;
        out[t] = bf16 ? orc_round_bf16(mval) : mval;
    }
}

/*
 * Build the multi-resolution view of chunks [0, n_chunks) of one (sequence, KV
 * head) stream.  K, V: [T][d] fp32 with T >= n_chunks*C.
 * assign_in (nullable) [n_chunks][C]: chunk-local group of every position, -1 for
 * sinks; when given, k-means is skipped.
 * Outputs (all [n_chunks][...]):
 *   assign [C]        group of each chunk-local position, -1 for sinks
 *   gcount [G], gk [G][d], gv [G][d]       group count and mean key / value
 *   pgroup [PS], pcount [PS], pmem [PS][P]  page's group, key count, absolute
 *                                           member positions (-1 padding)
 *   pk [PS][d], pv [PS][d]                   page mean key / value
 * PS = C/P + G.  A group's pages are consecutive slots in group order; inside a
 * group, members are in ascending position and pages are runs of P of them.
 */
int32_t orc_build(const orc_params* P, const float* K, const float* V, int32_t n_chunks,
                  const int32_t* assign_in, int32_t* assign, int32_t* gcount, float* gk,
                  float* gv, int32_t* pgroup, int32_t* pcount, int32_t* pmem, float* pk,
                  float* pv) {
    if (!P || !K || !V || n_chunks < 0) return ORC_ERR_ARG;
    const int32_t C = P->chunk, Pg = P->page, G = P->groups, d = P->d, s = P->n_sink;
    const int32_t PS = orc_page_slots(P);
    if (C < 1 || Pg < 1 || G < 1 || d < 1 || s < 0 || s >= C) return ORC_ERR_ARG;
    float* xs = (float*)malloc(sizeof(float) * (size_t)C * d);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    int32_t* mem = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    if (!xs || !pos || !a || !mem) {
        free(xs); free(pos); free(a); free(mem);
        return ORC_ERR_NOMEM;
    }
    int32_t rc = ORC_OK;
    for (int32_t c = 0; c < n_chunks && rc == ORC_OK; ++c) {
        const int32_t start = c * C;
        int32_t m = 0;
        for (int32_t off = 0; off < C; ++off) {
            int32_t p = start + off;
            if (p < s) continue; /* sinks are never clustered */
            pos[m] = p;
            memcpy(xs + (size_t)m * d, K + (size_t)p * d, sizeof(float) * (size_t)d);
            ++m;
        }
        if (assign_in) {
            for (int32_t i = 0; i < m; ++i) {
                int32_t g = assign_in[(size_t)c * C + (pos[i] - start)];
                if (g < 0 || g >= G) { rc = ORC_ERR_ARG; break; }
                a[i] = g;
            }
            if (rc != ORC_OK) break;
        } else {
            rc = orc_kmeans(xs, m, d, G, P->iters, a, NULL);
            if (rc != ORC_OK) break;
        }
        int32_t* asg = assign + (size_t)c * C;
        for (int32_t off = 0; off < C; ++off) asg[off] = -1;
        for (int32_t i = 0; i < m; ++i) asg[pos[i] - start] = a[i];

        int32_t* pgc = pgroup + (size_t)c * PS;
        int32_t* pcc = pcount + (size_t)c * PS;
        int32_t* pmc = pmem + (size_t)c * PS * Pg;
        for (int32_t q = 0; q < PS; ++q) { pgc[q] = -1; pcc[q] = 0; }
        for (int32_t k = 0; k < PS * Pg; ++k) pmc[k] = -1;
        memset(pk + (size_t)c * PS * d, 0, sizeof(float) * (size_t)PS * d);
        memset(pv + (size_t)c * PS * d, 0, sizeof(float) * (size_t)PS * d);

        int32_t slot = 0;
        for (int32_t j = 0; j < G; ++j) {
            int32_t n = 0;
            for (int32_t i = 0; i < m; ++i)
                if (a[i] == j) mem[n++] = pos[i]; /* ascending position */
            gcount[(size_t)c * G + j] = n;
            float* gkj = gk + ((size_t)c * G + j) * d;
            float* gvj = gv + ((size_t)c * G + j) * d;
            if (n == 0) {
                for (int32_t t = 0; t < d; ++t) { gkj[t] = 0.0f; gvj[t] = 0.0f; }
                continue;
            }
            canonical_mean(K, mem, n, d, P->bf16_store, gkj);
            canonical_mean(V, mem, n, d, P->bf16_store, gvj);
            for (int32_t b0 = 0; b0 < n; b0 += Pg) {
                int32_t np = (n - b0 < Pg) ? (n - b0) : Pg;
                if (slot >= PS) { rc = ORC_ERR_ARG; break; }
                pgc[slot] = j;
                pcc[slot] = np;
                for (int32_t k = 0; k < np; ++k) pmc[(size_t)slot * Pg + k] = mem[b0 + k];
                canonical_mean(K, mem + b0, np, d, P->bf16_store, pk + ((size_t)c * PS + slot) * d);
                canonical_mean(V, mem + b0, np, d, P->bf16_store, pv + ((size_t)c * PS + slot) * d);
                ++slot;
            }
            if (rc != ORC_OK) break;
        }
    }
    free(xs); free(pos); free(a); free(mem);
    return rc;
}

/* 4-bit code of one row: residual from the group mean, scale max|r|/7, rint, clamp. */
static void encode_row(const float* x, const float* mean, int32_t d, int8_t* code, float* scale) {
    float mx = 0.0f;
    for (int32_t t = 0; t < d; ++t) {
        const float r = x[t] - mean[t];
        const float a = r < 0.0f ? -r : r;
        if (a > mx) mx = a;
    }
    const float s = mx / 7.0f;
    *scale = s;
    for (int32_t t = 0; t < d; ++t) {
        if (s == 0.0f) { code[t] = 0; continue; }
        float c = rintf((x[t] - mean[t]) / s);
        if (c < -8.0f) c = -8.0f;
        if (c > 7.0f) c = 7.0f;
        code[t] = (int8_t)c;
    }
}

/*
 * Three-tier INT4 storage of chunks [0, n_chunks) built by orc_build: for every
 * chunk-local position with a group, codes [C][d] and a scale [C] for K and V (the
 * residual from the group's stored mean key / value); sinks get zero codes and scale.
 */
int32_t orc_encode_int4(const orc_params* P, const float* K, const float* V, int32_t n_chunks,
                        const int32_t* assign, const float* gk, const float* gv, int8_t* qk,
                        int8_t* qv, float* qks, float* qvs) {
    if (!P || !K || !V || !assign || !gk || !gv || !qk || !qv || !qks || !qvs || n_chunks < 0)
        return ORC_ERR_ARG;
    const int32_t C = P->chunk, G = P->groups, d = P->d;
    for (int32_t c = 0; c < n_chunks; ++c)
        for (int32_t off = 0; off < C; ++off) {
            const size_t row = (size_t)c * C + off;
            const int32_t j = assign[row];
            if (j < 0) {
                memset(qk + row * d, 0, (size_t)d);
                memset(qv + row * d, 0, (size_t)d);
                qks[row] = 0.0f;
                qvs[row] = 0.0f;
                continue;
            }
            if (j >= G) return ORC_ERR_ARG;
            const size_t p = (size_t)c * C + off;
            encode_row(K + p * d, gk + ((size_t)c * G + j) * d, d, qk + row * d, qks + row);
            encode_row(V + p * d, gv + ((size_t)c * G + j) * d, d, qv + row * d, qvs + row);
        }
    return ORC_OK;
}

/* Number of chunks summarised for a query at position p (block-granular window). */
int32_t orc_built_chunks(const orc_params* P, int32_t p) {
    int32_t nb = p / P->chunk - P->window / P->chunk + 1;
    return nb < 0 ? 0 : nb;
}

typedef struct {
    float r;
    int32_t id;
} ranked;

/* score descending, then id ascending (-0 and +0 compare equal) */
static int rank_cmp(const void* pa, const void* pb) {
    const ranked* a = (const ranked*)pa;
    const ranked* b = (const ranked*)pb;
    if (a->r > b->r) return -1;
    if (a->r < b->r) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

/*
 * LoD attention of one query q[d] at position p over one KV stream.
 * The index arrays are those of orc_build (at least n_b(p) chunks).
 * out[d]        fp64 output (normalised)
 * sel_groups    [top_groups] opened group ids (c*G + j), descending rank, -1 pad
 * sel_pages     [top_groups][max(top_pages,1)] opened chunk-local page slots,
 *               descending rank; -1 pad (and all -1 in two-tier mode)
 * log_mass      log of the softmax denominator over all terms (nullable)
 * n_terms       [0] exact keys, [1] coarse group terms, [2] coarse page terms (nullable)
 */
int32_t orc_attend(const orc_params* P, const float* q, int32_t p, int32_t n_chunks,
                   const int32_t* gcount, const float* gk, const float* gv,
                   const int32_t* pgroup, const int32_t* pcount, const int32_t* pmem,
                   const float* pk, const float* pv, const float* K, const float* V,
                   const int8_t* qk, const int8_t* qv, const float* qks, const float* qvs,
                   double* out, int32_t* sel_groups, int32_t* sel_pages, double* log_mass,
                   int32_t* n_terms) {
    if (!P || !q || !K || !V || !out || p < 0) return ORC_ERR_ARG;
    if (P->int4_pages && (!qk || !qv || !qks || !qvs)) return ORC_ERR_ARG;
    const int32_t C = P->chunk, Pg = P->page, G = P->groups, d = P->d, s = P->n_sink;
    const int32_t PS = orc_page_slots(P);
    const int32_t TG = P->top_groups, TP = P->top_pages;
    const int32_t TPW = TP > 0 ? TP : 1;
    const int32_t nb = orc_built_chunks(P, p);
    if (nb > n_chunks) return ORC_ERR_NOT_BUILT;

    const int32_t ng = nb * G;
    ranked* el = (ranked*)malloc(sizeof(ranked) * (size_t)(ng > 0 ? ng : 1));
    uint8_t* opened = (uint8_t*)calloc((size_t)(ng > 0 ? ng : 1), 1);
    uint8_t* exact = (uint8_t*)calloc((size_t)p + 1, 1);
    int32_t* xgroup = (int32_t*)calloc((size_t)p + 1, sizeof(int32_t)); /* opened-page member: group + 1 */
    uint8_t* popen = (uint8_t*)calloc((size_t)(nb > 0 ? nb : 1) * PS, 1);
    double* lam = NULL;
    const float** vals = NULL;
    if (!el || !opened || !exact || !popen || !xgroup) {
        free(el); free(opened); free(exact); free(popen); free(xgroup);
        return ORC_ERR_NOMEM;
    }
    int32_t rc = ORC_OK;

    /* 1. rank the non-empty groups of the summarised chunks */
    int32_t ne = 0;
    for (int32_t g = 0; g < ng; ++g) {
        if (gcount[g] <= 0) continue;
        el[ne].r = orc_canonical_dot(q, gk + (size_t)g * d, d);
        el[ne].id = g;
        ++ne;
    }
    qsort(el, (size_t)ne, sizeof(ranked), rank_cmp);
    const int32_t nsel = ne < TG ? ne : TG;
    if (sel_groups)
        for (int32_t i = 0; i < TG; ++i) sel_groups[i] = i < nsel ? el[i].id : -1;
    if (sel_pages)
        for (int32_t i = 0; i < TG * TPW; ++i) sel_pages[i] = -1;

    /* 2. inside every opened group, rank its pages and open the best TP */
    for (int32_t i = 0; i < nsel; ++i) {
        const int32_t g = el[i].id, c = g / G, j = g % G;
        opened[g] = 1;
        ranked pr[64];
        int32_t np = 0;
        for (int32_t sl = 0; sl < PS; ++sl) {
            if (pgroup[(size_t)c * PS + sl] != j) continue;
            if (np >= 64) { rc = ORC_ERR_ARG; break; }
            pr[np].r = orc_canonical_dot(q, pk + ((size_t)c * PS + sl) * d, d);
            pr[np].id = sl;
            ++np;
        }
        if (rc != ORC_OK) break;
        qsort(pr, (size_t)np, sizeof(ranked), rank_cmp);
        const int32_t nopen = (TP == 0 || np <= TP) ? np : TP;
        for (int32_t k = 0; k < nopen; ++k) {
            popen[(size_t)c * PS + pr[k].id] = 1;
            if (sel_pages && TP > 0) sel_pages[i * TPW + k] = pr[k].id;
        }
    }

    /* 3. the exact set: sinks, block window, members of opened pages */
    if (rc == ORC_OK) {
        int32_t dup = 0;
        for (int32_t x = 0; x < s && x <= p; ++x) exact[x] = 1;
        for (int32_t x = nb * C; x <= p; ++x) { dup |= (x < s) ? 0 : exact[x]; exact[x] = 1; }
        for (int32_t c = 0; c < nb; ++c)
            for (int32_t sl = 0; sl < PS; ++sl) {
                if (!popen[(size_t)c * PS + sl]) continue;
                for (int32_t k = 0; k < pcount[(size_t)c * PS + sl]; ++k) {
                    int32_t x = pmem[((size_t)c * PS + sl) * Pg + k];
                    if (x < 0 || x > p) { rc = ORC_ERR_ARG; break; }
                    dup |= exact[x];
                    exact[x] = 1;
                    xgroup[x] = c * G + pgroup[(size_t)c * PS + sl] + 1;
                }
            }
        if (dup && rc == ORC_OK) rc = ORC_ERR_DOUBLE_COUNT;
    }

    /* 4. gather all terms (logit, value row) and take one fp64 softmax */
    /* decoded rows of opened-page members (three-tier INT4) */
    float* dec = NULL;
    int32_t ndec = 0;
    if (rc == ORC_OK && P->int4_pages) {
        for (int32_t x = 0; x <= p; ++x) ndec += xgroup[x] != 0;
        dec = (float*)malloc(sizeof(float) * (size_t)(ndec > 0 ? ndec : 1) * 2 * d);
        if (!dec) rc = ORC_ERR_NOMEM;
    }
    if (rc == ORC_OK) {
        const int32_t maxt = (p + 1) + ng + nb * PS;
        lam = (double*)malloc(sizeof(double) * (size_t)maxt);
        vals = (const float**)malloc(sizeof(float*) * (size_t)maxt);
        if (!lam || !vals) rc = ORC_ERR_NOMEM;
    }
    if (rc == ORC_OK) {
        int32_t nt = 0, n_ex = 0, n_cg = 0, n_cp = 0, k4 = 0;
        for (int32_t x = 0; x <= p; ++x) {
            if (!exact[x]) continue;
            const float* kx = K + (size_t)x * d;
            const float* vx = V + (size_t)x * d;
            if (P->int4_pages && xgroup[x]) {
                const int32_t g = xgroup[x] - 1;
                float* kd = dec + (size_t)k4 * 2 * d;
                float* vd = kd + d;
                for (int32_t t = 0; t < d; ++t) {
                    kd[t] = fmaf(qks[x], (float)qk[(size_t)x * d + t], gk[(size_t)g * d + t]);
                    vd[t] = fmaf(qvs[x], (float)qv[(size_t)x * d + t], gv[(size_t)g * d + t]);
                }
                kx = kd;
                vx = vd;
                ++k4;
            }
            lam[nt] = P->scale * dot64(q, kx, d);
            vals[nt++] = vx;
            ++n_ex;
        }
        for (int32_t g = 0; g < ng && !P->drop_remainder; ++g) {
            if (gcount[g] <= 0) continue;
            if (!opened[g]) {
                lam[nt] = P->scale * dot64(q, gk + (size_t)g * d, d) + log((double)gcount[g]);
                vals[nt++] = gv + (size_t)g * d;
                ++n_cg;
            } else {
                const int32_t c = g / G, j = g % G;
                for (int32_t sl = 0; sl < PS; ++sl) {
                    if (pgroup[(size_t)c * PS + sl] != j || popen[(size_t)c * PS + sl]) continue;
                    lam[nt] = P->scale * dot64(q, pk + ((size_t)c * PS + sl) * d, d) +
                              log((double)pcount[(size_t)c * PS + sl]);
                    vals[nt++] = pv + ((size_t)c * PS + sl) * d;
                    ++n_cp;
                }
            }
        }
        double M = -INFINITY;
        for (int32_t k = 0; k < nt; ++k) if (lam[k] > M) M = lam[k];
        double Z = 0.0;
        for (int32_t t = 0; t < d; ++t) out[t] = 0.0;
        for (int32_t k = 0; k < nt; ++k) {
            double w = exp(lam[k] - M);
            Z += w;
            for (int32_t t = 0; t < d; ++t) out[t] += w * (double)vals[k][t];
        }
        for (int32_t t = 0; t < d; ++t) out[t] /= Z;
        if (log_mass) *log_mass = M + log(Z);
        if (n_terms) { n_terms[0] = n_ex; n_terms[1] = n_cg; n_terms[2] = n_cp; }
    }
    free(el); free(opened); free(exact); free(popen); free(xgroup); free(dec); free(lam); free(vals);
    return rc;
}

/* Dense causal softmax attention of q at position p over K, V rows [0, p]. */
int32_t orc_dense(const orc_params* P, const float* q, int32_t p, const float* K,
                  const float* V, double* out, double* log_mass) {
    if (!P || !q || !K || !V || !out || p < 0) return ORC_ERR_ARG;
    const int32_t d = P->d;
    double* lam = (double*)malloc(sizeof(double) * ((size_t)p + 1));
    if (!lam) return ORC_ERR_NOMEM;
    double M = -INFINITY;
    for (int32_t x = 0; x <= p; ++x) {
        lam[x] = P->scale * dot64(q, K + (size_t)x * d, d);
        if (lam[x] > M) M = lam[x];
    }
    double Z = 0.0;
    for (int32_t t = 0; t < d; ++t) out[t] = 0.0;
    for (int32_t x = 0; x <= p; ++x) {
        double w = exp(lam[x] - M);
        Z += w;
        for (int32_t t = 0; t < d; ++t) out[t] += w * (double)V[(size_t)x * d + t];
    }
    for (int32_t t = 0; t < d; ++t) out[t] /= Z;
    if (log_mass) *log_mass = M + log(Z);
    free(lam);
    return ORC_OK;
}
