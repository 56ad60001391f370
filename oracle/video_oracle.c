/*
 * video_oracle.c -- plain, slow CPU oracle for video LoD attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this code (it is part of liblod_oracle.so).  It shares no
 * code, header, table or helper with the GPU library.
 *
 * Source: the blog post "Level of Detail Attention: allocating resolution instead
 * of sparsity" (featherless.ai), section "Video LoD": LoD carried over to video,
 * where tokens are local in space and time, so queries and keys/values are handled
 * in 4x4x4 blocks, and the comparison runs LoD at c = 16.  The section states
 * nothing more, so the rest is read from the text method ("How It Works"):
 *   grid       tokens sit on an F x H x W grid in raster order, t = (f*H + y)*W + x;
 *              attention is bidirectional: every query sees every key (no causal
 *              mask, no window, no sinks);
 *   blocks     the grid is cut into bf x bh x bw blocks (4x4x4), clipped at the far
 *              edges; block ids run in raster order of the block coordinates and a
 *              block's members in ascending token order.  A block is the unit that
 *              is summarised and opened, as a group is in the text method: locality
 *              in space and time stands in for the clustering;
 *   summaries  per block the canonical mean key and value (fp32 sum in member
 *              order, correctly rounded divide by n, then the storage rounding) and
 *              its count n;
 *   selection  the queries of a block share one choice, made with the block's mean
 *              query (the same canonical mean, kept in fp32): it scores every key
 *              block with the unscaled fp32 fma chain over the head dimension in
 *              index order, and the top c blocks by (score desc, id asc) open;
 *   softmax    every query of the block takes exact logits scale*q.k over the
 *              members of the opened blocks, and for each unopened block one term
 *              scale*q.kbar + ln n with value vbar (the block's mean key and value
 *              repeated n times), all in one fp64 softmax;
 *   ablation   drop_remainder = 1 keeps the same choice but only the exact keys.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define VORC_OK 0
#define VORC_ERR_ARG (-1)
#define VORC_ERR_NOMEM (-4)

typedef struct {
    int32_t d;                      /* head dimension */
    int32_t frames, height, width;  /* token grid F x H x W */
    int32_t bf, bh, bw;             /* block extents along frames, rows, columns */
    int32_t top_blocks;             /* c: key blocks opened per query block */
    int32_t bf16_store;             /* 1: mean keys and values are rounded to bfloat16 */
    int32_t drop_remainder;         /* 1: no coarse terms (sparsity ablation) */
    double scale;                   /* softmax scale, 1/sqrt(d) */
} orc_video_params;

/* Round-to-nearest-even of an fp32 value to bfloat16, returned as fp32 (a copy of
 * the usual bit recipe, kept local so this file stands alone). */
static float vround_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) {
        if (u & 0x007fffffu) u |= 0x00400000u;
        u &= 0xffff0000u;
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);
        u &= 0xffff0000u;
    }
    memcpy(&x, &u, 4);
    return x;
}

static int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }

static int valid_params(const orc_video_params* P) {
    return P && P->d >= 1 && P->frames >= 1 && P->height >= 1 && P->width >= 1 && P->bf >= 1 &&
           P->bh >= 1 && P->bw >= 1 && P->top_blocks >= 1;
}

/* Number of blocks of the grid (or VORC_ERR_ARG). */
int32_t orc_video_blocks(const orc_video_params* P) {
    if (!valid_params(P)) return VORC_ERR_ARG;
    return cdiv(P->frames, P->bf) * cdiv(P->height, P->bh) * cdiv(P->width, P->bw);
}

/* Tokens of block blk in ascending order into tok[] (room for bf*bh*bw); returns the
 * count, or VORC_ERR_ARG. */
int32_t orc_video_members(const orc_video_params* P, int32_t blk, int32_t* tok) {
    const int32_t nb = orc_video_blocks(P);
    if (nb < 0 || blk < 0 || blk >= nb || !tok) return VORC_ERR_ARG;
    const int32_t nby = cdiv(P->height, P->bh), nbx = cdiv(P->width, P->bw);
    const int32_t bfi = blk / (nby * nbx), byi = (blk / nbx) % nby, bxi = blk % nbx;
    int32_t n = 0;
    for (int32_t i = 0; i < P->bf; ++i) {
        const int32_t f = bfi * P->bf + i;
        if (f >= P->frames) break;
        for (int32_t j = 0; j < P->bh; ++j) {
            const int32_t y = byi * P->bh + j;
            if (y >= P->height) break;
            for (int32_t k = 0; k < P->bw; ++k) {
                const int32_t x = bxi * P->bw + k;
                if (x >= P->width) break;
                tok[n++] = (f * P->height + y) * P->width + x;
            }
        }
    }
    return n;
}

/*
 * Per-block canonical means of X [T][d] (T = F*H*W): mean [nb][d] and count [nb].
 * round_bf16 = 1 rounds each mean to bfloat16 (stored keys and values of a bf16
 * cache); 0 keeps the fp32 mean (the block's mean query).
 */
int32_t orc_video_summaries(const orc_video_params* P, const float* X, int32_t round_bf16,
                            float* mean, int32_t* count) {
    const int32_t nb = orc_video_blocks(P);
    if (nb < 0 || !X || !mean || !count) return VORC_ERR_ARG;
    const int32_t d = P->d;
    int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)P->bf * P->bh * P->bw);
    if (!tok) return VORC_ERR_NOMEM;
    for (int32_t b = 0; b < nb; ++b) {
        const int32_t n = orc_video_members(P, b, tok);
        count[b] = n;
        for (int32_t t = 0; t < d; ++t) {
            float s = 0.0f;
            for (int32_t i = 0; i < n; ++i) s = s + X[(size_t)tok[i] * d + t];
            const float m = s / (float)n;
            mean[(size_t)b * d + t] = round_bf16 ? vround_bf16(m) : m;
        }
    }
    free(tok);
    return VORC_OK;
}

typedef struct {
    float score;
    int32_t id;
} vrank;

/* score descending, then id ascending */
static int vrank_cmp(const void* pa, const void* pb) {
    const vrank* a = (const vrank*)pa;
    const vrank* b = (const vrank*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

static int int_cmp(const void* pa, const void* pb) {
    const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/*
 * Choice of one query block.  qbar [d]: its mean query; kbar [nb][d]: the stored mean
 * keys.  sel [c] receives the opened block ids in ascending order, -1 padding when
 * nb < c.  scores (nullable, [nb]) receives every ranking score.
 */
int32_t orc_video_select(const orc_video_params* P, const float* qbar, const float* kbar,
                         int32_t* sel, float* scores) {
    const int32_t nb = orc_video_blocks(P);
    if (nb < 0 || !qbar || !kbar || !sel) return VORC_ERR_ARG;
    const int32_t d = P->d, c = P->top_blocks;
    vrank* r = (vrank*)malloc(sizeof(vrank) * (size_t)nb);
    if (!r) return VORC_ERR_NOMEM;
    for (int32_t b = 0; b < nb; ++b) {
        float acc = 0.0f;
        for (int32_t t = 0; t < d; ++t) acc = fmaf(qbar[t], kbar[(size_t)b * d + t], acc);
        r[b].score = acc;
        r[b].id = b;
        if (scores) scores[b] = acc;
    }
    qsort(r, (size_t)nb, sizeof(vrank), vrank_cmp);
    const int32_t k = nb < c ? nb : c;
    for (int32_t i = 0; i < k; ++i) sel[i] = r[i].id;
    qsort(sel, (size_t)k, sizeof(int32_t), int_cmp);
    for (int32_t i = k; i < c; ++i) sel[i] = -1;
    free(r);
    return VORC_OK;
}

static double vdot64(const float* a, const float* b, int32_t d) {
    double acc = 0.0;
    for (int32_t t = 0; t < d; ++t) acc += (double)a[t] * (double)b[t];
    return acc;
}

/*
 * LoD attention of the queries of block qblk.  Q [T][d] (this query head), K, V
 * [T][d] (its KV head), kbar, vbar [nb][d] and count [nb] from orc_video_summaries,
 * sel [c] from orc_video_select for qblk.  out [n][d] (n = members of qblk, in
 * ascending token order) receives the fp64 output.  exact_mass / coarse_mass
 * (nullable, [n]) receive, relative to each query's own maximum logit, the softmax
 * mass of the exact and of the coarse terms.
 */
int32_t orc_video_attend(const orc_video_params* P, const float* Q, const float* K, const float* V,
                         const float* kbar, const float* vbar, const int32_t* count, const int32_t* sel,
                         int32_t qblk, double* out, double* exact_mass, double* coarse_mass) {
    const int32_t nb = orc_video_blocks(P);
    if (nb < 0 || !Q || !K || !V || !kbar || !vbar || !count || !sel || !out || qblk < 0 || qblk >= nb)
        return VORC_ERR_ARG;
    const int32_t d = P->d, c = P->top_blocks, bsz = P->bf * P->bh * P->bw;
    int32_t* qtok = (int32_t*)malloc(sizeof(int32_t) * (size_t)bsz);
    int32_t* ktok = (int32_t*)malloc(sizeof(int32_t) * (size_t)bsz);
    char* opened = (char*)calloc((size_t)nb, 1);
    /* the term list of one query: exact keys, then coarse blocks */
    const size_t cap = (size_t)c * bsz + (size_t)nb;
    double* lam = (double*)malloc(sizeof(double) * cap);
    const float** val = (const float**)malloc(sizeof(float*) * cap);
    char* is_coarse = (char*)malloc(cap);
    int32_t* opened_tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)c * bsz);
    if (!qtok || !ktok || !opened || !lam || !val || !is_coarse || !opened_tok) {
        free(qtok); free(ktok); free(opened); free(lam); free(val); free(is_coarse); free(opened_tok);
        return VORC_ERR_NOMEM;
    }
    /* the opened blocks' members (each block at most once) */
    int32_t n_open = 0;
    for (int32_t i = 0; i < c; ++i) {
        const int32_t b = sel[i];
        if (b < 0) continue;
        if (b >= nb || opened[b]) {
            free(qtok); free(ktok); free(opened); free(lam); free(val); free(is_coarse); free(opened_tok);
            return VORC_ERR_ARG;
        }
        opened[b] = 1;
        const int32_t n = orc_video_members(P, b, ktok);
        for (int32_t j = 0; j < n; ++j) opened_tok[n_open++] = ktok[j];
    }
    const int32_t nq = orc_video_members(P, qblk, qtok);
    for (int32_t qi = 0; qi < nq; ++qi) {
        const float* q = Q + (size_t)qtok[qi] * d;
        size_t nt = 0;
        for (int32_t j = 0; j < n_open; ++j) {
            const int32_t t = opened_tok[j];
            lam[nt] = P->scale * vdot64(q, K + (size_t)t * d, d);
            val[nt] = V + (size_t)t * d;
            is_coarse[nt++] = 0;
        }
        if (!P->drop_remainder) {
            for (int32_t b = 0; b < nb; ++b) {
                if (opened[b]) continue;
                lam[nt] = P->scale * vdot64(q, kbar + (size_t)b * d, d) + log((double)count[b]);
                val[nt] = vbar + (size_t)b * d;
                is_coarse[nt++] = 1;
            }
        }
        double M = -INFINITY;
        for (size_t i = 0; i < nt; ++i) M = lam[i] > M ? lam[i] : M;
        double L = 0.0, me = 0.0, mc = 0.0;
        double* o = out + (size_t)qi * d;
        for (int32_t t = 0; t < d; ++t) o[t] = 0.0;
        for (size_t i = 0; i < nt; ++i) {
            const double w = exp(lam[i] - M);
            L += w;
            if (is_coarse[i]) mc += w; else me += w;
            for (int32_t t = 0; t < d; ++t) o[t] += w * (double)val[i][t];
        }
        for (int32_t t = 0; t < d; ++t) o[t] /= L;
        if (exact_mass) exact_mass[qi] = me;
        if (coarse_mass) coarse_mass[qi] = mc;
    }
    free(qtok); free(ktok); free(opened); free(lam); free(val); free(is_coarse); free(opened_tok);
    return VORC_OK;
}

/* Dense bidirectional attention of the queries of block qblk over all T keys (fp64),
 * out [n][d] in the block's member order. */
int32_t orc_video_dense(const orc_video_params* P, const float* Q, const float* K, const float* V,
                        int32_t qblk, double* out) {
    const int32_t nb = orc_video_blocks(P);
    if (nb < 0 || !Q || !K || !V || !out || qblk < 0 || qblk >= nb) return VORC_ERR_ARG;
    const int32_t d = P->d;
    const int64_t T = (int64_t)P->frames * P->height * P->width;
    int32_t* qtok = (int32_t*)malloc(sizeof(int32_t) * (size_t)P->bf * P->bh * P->bw);
    double* lam = (double*)malloc(sizeof(double) * (size_t)T);
    if (!qtok || !lam) { free(qtok); free(lam); return VORC_ERR_NOMEM; }
    const int32_t nq = orc_video_members(P, qblk, qtok);
    for (int32_t qi = 0; qi < nq; ++qi) {
        const float* q = Q + (size_t)qtok[qi] * d;
        double M = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            lam[t] = P->scale * vdot64(q, K + (size_t)t * d, d);
            M = lam[t] > M ? lam[t] : M;
        }
        double L = 0.0;
        double* o = out + (size_t)qi * d;
        for (int32_t t = 0; t < d; ++t) o[t] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double w = exp(lam[t] - M);
            L += w;
            for (int32_t e = 0; e < d; ++e) o[e] += w * (double)V[(size_t)t * d + e];
        }
        for (int32_t e = 0; e < d; ++e) o[e] /= L;
    }
    free(qtok); free(lam);
    return VORC_OK;
}
