/*
 * lod.h -- C ABI of the Level-of-Detail (LoD) attention library for AMD MI355X (gfx950).
 *
 * The method is the one described in "Level of Detail Attention: allocating
 * resolution instead of sparsity" (featherless.ai blog), section "How It Works":
 *   - after every chunk of 256 tokens the chunk's keys are clustered into centroid
 *     groups; each group is cut into pages of 16 keys; every group and page keeps a
 *     mean key, a mean value and its key count;
 *   - a query scores the group centroids and opens the top groups (8), scores the page
 *     summaries inside them and opens the top pages (2) of each opened group;
 *   - one softmax covers the exact keys (opened pages, the recent block window, the
 *     sink tokens) and a coarse remainder in which every unopened group and every
 *     unopened page of an opened group enters as its mean key/value repeated by its
 *     key count, i.e. with logit scale*q.kbar + ln(n) and value vbar.
 * Readings for what the post leaves open (k-means details, rounding, tie-breaks,
 * window granularity) are stated at each call below.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *     buffer; the library never allocates device memory and keeps no state apart from
 *     the optional trace events of lod_trace_events (and the fixed workspace of
 *     lod_attend_decode_noalloc).  It creates no stream or event.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue kernels
 *     on that stream (no memset, copy or host synchronisation), so they can be captured
 *     in a HIP graph; they return before the GPU finishes.  Device faults surface at the
 *     caller's next synchronisation of that stream.
 *   - Arguments are validated on the host before anything is enqueued: a bad argument
 *     returns LOD_ERR_ARG (or LOD_ERR_UNSUPPORTED / LOD_ERR_WORKSPACE) and enqueues
 *     nothing.  A failed launch returns LOD_ERR_HIP.  No exception crosses the ABI.
 *   - Calls are reentrant.  Calls that share output, index or workspace buffers must
 *     be ordered by the caller (same stream or events).
 *   - KV cache: element (b, t, h, i) of K is at k[b*stride_b + t*stride_t + h*stride_h + i]
 *     (strides in elements, last dimension contiguous, 16-byte aligned rows), or found
 *     through a block table (lod_kv below).
 *     Queries have the cache's element type; outputs are fp32.  q and out are 16-byte
 *     aligned (LOD_ERR_ARG otherwise).
 */
#ifndef LOD_H
#define LOD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    LOD_OK = 0,
    LOD_ERR_ARG = -1,         /* null pointer, inconsistent sizes, out-of-range value */
    LOD_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim != 128) */
    LOD_ERR_WORKSPACE = -3,   /* workspace or index buffer smaller than required */
    LOD_ERR_HIP = -4          /* a HIP launch or runtime call failed */
};

/* Element types of K, V and q. */
enum { LOD_F32 = 0, LOD_BF16 = 1 };

/*
 * LoD parameters.  Supported: head_dim 128; chunk_size 256; page_size 16;
 * 1 <= groups_per_chunk <= 16; 1 <= top_groups <= 16; 0 <= top_pages <= 16
 * (0 = two-tier: every page of an opened group is exact); window a positive multiple
 * of chunk_size; 0 <= n_sink < chunk_size; kmeans_iters >= 1;
 * n_q_heads = g * n_kv_heads with g in {1, 2, 4, 8}; drop_remainder 0 or 1; int4_pages 0
 * or 1 (1 needs kv_dtype LOD_BF16).
 *
 * int4_pages = 1 follows the post's "Additional Benefits" section (centroids keep
 * similar keys together, so the cache compresses to INT4, and in three-tier mode only
 * the selected pages are decompressed).  Reading: every clustered key (value) row is
 * stored as its residual r from its group's stored mean key (value), one fp32 scale per
 * row s = max_t |r_t| / 7, and codes rint(r_t / s) clamped to [-8, 7] (0 when s = 0);
 * a decoded element is fma(s, code, mean).  Members of opened pages enter the softmax
 * decoded; sinks and the block window are read from the cache.  Once a chunk is built,
 * its clustered rows are never read from the cache again.
 *
 * drop_remainder = 1 is the token-removing alternative that the post's "The Main Idea"
 * section contrasts LoD with: groups and pages are selected exactly as in LoD, but the
 * softmax holds only the exact keys (opened pages, block window, sinks).  With
 * top_pages = 0 it is block-sparse attention in the manner of "Coarse Semantic Blocks
 * for Efficient Training-Free Sparse Attention" (abstract): a query scores block
 * centroids and attends to the original keys of the blocks it selects.
 */
typedef struct {
    int32_t head_dim;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t chunk_size;       /* C: tokens per clustered chunk (256) */
    int32_t page_size;        /* P: keys per page (16) */
    int32_t groups_per_chunk; /* G: k-means groups per chunk */
    int32_t top_groups;       /* groups a query opens (8) */
    int32_t top_pages;        /* pages opened per opened group (2); 0 = two-tier */
    int32_t window;           /* W: exact block window in tokens */
    int32_t n_sink;           /* s: leading positions that are always exact */
    int32_t kmeans_iters;     /* Lloyd rounds per chunk (10) */
    int32_t kv_dtype;         /* LOD_F32 or LOD_BF16 */
    float scale;              /* softmax scale, normally 1/sqrt(head_dim) */
    int32_t drop_remainder;   /* 0: LoD (coarse remainder in the softmax); 1: sparsity
                                 ablation: the same selection, exact keys only */
    int32_t int4_pages;       /* 0: exact rows of opened pages from the KV cache; 1: three-
                                 tier INT4: the build stores every clustered row as 4-bit
                                 codes in the index and opened pages are decoded from them
                                 (bf16 caches only) */
} lod_params;

/*
 * View of the caller's KV cache.
 *   Strided (block_table == NULL): element (b, t, h, i) of K is at
 *     k[b*stride_b + t*stride_t + h*stride_h + i].
 *   Paged (block_table != NULL), the block-table layout of a vLLM-style serving engine:
 *     position t of sequence b lives in cache block blk = block_table[b*max_blocks +
 *     t/block_size], and element (b, t, h, i) of K is at
 *     k[blk*stride_b + (t % block_size)*stride_t + h*stride_h + i]
 *     (stride_b is then the stride between blocks).  block_size is a power of two in
 *     [1, 65536]; max_blocks must cover every position a call reads (checked on the
 *     host); the block ids themselves are device data and are not checked: each must
 *     name a block inside the caller's K and V buffers.
 * The paged view is a boundary change only: every call computes the same results as
 * with a strided copy of the same cache.
 */
typedef struct {
    const void* k;
    const void* v;
    int64_t stride_b, stride_t, stride_h;
    const int32_t* block_table; /* DEVICE [batch][max_blocks] int32, or NULL (strided) */
    int32_t block_size;         /* positions per cache block (paged view) */
    int32_t max_blocks;         /* row length of block_table (paged view) */
} lod_kv;

/* The multi-resolution view: one caller-allocated device buffer of `bytes` bytes,
 * sized by lod_index_bytes for (batch, max_chunks).  Its layout is given by
 * lod_index_layout; it holds absolute positions and summaries only, so it can be
 * copied as plain memory. */
typedef struct {
    void* mem;
    size_t bytes;
    int32_t batch;
    int32_t max_chunks;
} lod_index;

/*
 * Byte offsets of the arrays inside lod_index.mem (U = batch * n_kv_heads units,
 * NC = max_chunks, G = groups_per_chunk, PS = page_slots = C/P + G, d = head_dim,
 * E = element size of kv_dtype).  Every array is 256-byte aligned.
 *   gk, gv   [U][NC*G][d]  E     group mean key / value (storage-rounded)
 *   gln      [U][NC*G]     f32   ln(key count), -inf for an empty group
 *   gkn      [U][NC*G]     f32   upper bound of the Euclidean norm of the stored mean key
 *   gpage    [U][NC*G]     i32   first page slot of the group | its page count << 16
 *   pk, pv   [U][NC*PS][d] E     page mean key / value
 *   pln      [U][NC*PS]    f32   ln(key count), -inf for an unused page slot
 *   meta     [U][NC][meta_stride] int16: gpg[G+1] first page slot of each group,
 *            pst[PS+1] first perm entry of each page slot, perm[C] chunk-local offsets
 *            of the clustered keys ordered by (group, position)
 *   assign   [U][NC][C]    int8  group of every chunk-local position, -1 for sinks
 *   q4k, q4v [U][NC][C][d/2] uint8 (int4_pages only, else empty) 4-bit codes of every
 *            chunk-local row, two's complement, element 2j in the low nibble of byte j
 *   q4ks, q4vs [U][NC][C]  f32   their scales (0 for sinks)
 */
typedef struct {
    size_t gk, gv, gln, gkn, gpage, pk, pv, pln, meta, assign, q4k, q4v, q4ks, q4vs, total;
    int32_t page_slots;
    int32_t meta_stride; /* int16 entries per chunk in `meta` */
} lod_index_layout_t;

/* Human-readable name of a status code (static storage). */
const char* lod_status_string(int status);

/* Host-only: bytes of an index that holds max_tokens/chunk_size chunks per sequence. */
int lod_index_bytes(const lod_params* params, int32_t batch, int32_t max_tokens, size_t* bytes);

/* Host-only: array offsets for (batch, max_chunks); see lod_index_layout_t. */
int lod_index_layout(const lod_params* params, int32_t batch, int32_t max_chunks,
                     lod_index_layout_t* layout);

/*
 * Build chunks [chunk_begin, chunk_begin + n_chunks) of every sequence and KV head:
 * the step of "How It Works" in which each completed 256-token chunk has its keys
 * clustered into centroid groups and every group cut into pages of 16 keys.
 * Clustering: Lloyd's k-means on the chunk's non-sink keys (positions >= n_sink) in
 * fp32, seeds mu_j = x[floor(j*m/G)] for m members, kmeans_iters rounds of (assign to
 * the nearest centroid by the fp32 fma chain of squared differences in index order,
 * ties to the lower group; update to the fp32 mean in position order, correctly
 * rounded divide; an empty group keeps its centroid).  Sinks are never clustered.
 * Summaries: the same fp32 means of keys and values of each group and of each page
 * (runs of page_size members in position order inside a group), rounded to nearest
 * even to kv_dtype.  Chunks are independent, so one call over many chunks equals
 * one call per chunk.
 *   kv          the cache; K and V rows of the chunks must be written
 *   assign_in   nullable [batch][n_kv_heads][n_chunks][chunk_size] int32: groups to use
 *               instead of k-means (sinks: -1); values outside [0, G) for a non-sink
 *               position are clamped to that range on the device
 *   assign_out  nullable, same shape: the groups used
 * Errors: LOD_ERR_ARG if the range exceeds index->max_chunks or batch != index->batch.
 */
int lod_build_chunk(const lod_params* params, const lod_index* index, lod_kv kv, int32_t batch,
                    int32_t chunk_begin, int32_t n_chunks, const int32_t* assign_in,
                    int32_t* assign_out, void* stream);

/* Host-only: workspace bytes for lod_attend_decode at (batch, max_seq_len). */
int lod_decode_ws_bytes(const lod_params* params, int32_t batch, int32_t max_seq_len,
                        size_t* bytes);

/*
 * LoD decode: one query token per sequence (How It Works, all three paragraphs).
 * Sequence b's query sits at position p = seq_lens[b] - 1 and its own K/V row is
 * already in the cache.  Chunks c < n_b = max(0, p/C - W/C + 1) are summarised; the
 * block window [n_b*C, p] and the sinks [0, min(n_sink, p+1)) are exact.  Groups are
 * ranked by the unscaled fp32 fma chain q.kbar in index order, ties to the lower group
 * id c*G + j; pages of an opened group likewise, ties to the lower page slot.
 *   q           [batch][n_q_heads][head_dim], kv_dtype
 *   seq_lens    DEVICE [batch] int32; values are clamped to [1, max_seq_len]
 *   max_seq_len host bound on seq_lens (sizes the launch; chunks 0..n_b(max_seq_len-1)-1
 *               must be built for every sequence that reaches it)
 *   out         [batch][n_q_heads][head_dim] fp32
 *   sel_groups  nullable [batch][n_q_heads][top_groups] int32: opened group ids in rank
 *               order, -1 padding
 *   sel_pages   nullable [batch][n_q_heads][top_groups][max(top_pages,1)] int32: opened
 *               chunk-local page slots in rank order, -1 padding (all -1 in two-tier)
 *   ws          workspace of at least lod_decode_ws_bytes bytes (contents not kept)
 */
int lod_attend_decode(const lod_params* params, const lod_index* index, lod_kv kv,
                      const void* q, const int32_t* seq_lens, int32_t batch,
                      int32_t max_seq_len, float* out, int32_t* sel_groups,
                      int32_t* sel_pages, void* ws, size_t ws_bytes, void* stream);

/*
 * lod_attend_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments and results are those of lod_attend_decode; the
 * workspace is a fixed device array of LOD_NOALLOC_WS_BYTES bytes inside the library,
 * one per device, loaded with the library's code and kept until the process ends.
 *   - The call allocates nothing and calls no allocating routine.  The array's address
 *     on the current device is looked up once per device (hipGetSymbolAddress) on the
 *     first call there; `stream` must belong to the current device.
 *   - Arguments are checked as by lod_attend_decode; then LOD_ERR_WORKSPACE when
 *     lod_decode_ws_bytes(params, batch, max_seq_len) exceeds LOD_NOALLOC_WS_BYTES
 *     (32 MiB: e.g. batch 16 at 128K context, or batch 8 at 256K, with 64/8 heads);
 *     nothing is enqueued then.
 *   - Every call on one device shares that device's array and leaves its last contents
 *     there (no kernel reads workspace it has not written in the same call).  Calls that
 *     may overlap on one device race on it: order them (one stream, or events).
 */
#define LOD_NOALLOC_WS_BYTES (32u << 20)
int lod_attend_decode_noalloc(const lod_params* params, const lod_index* index, lod_kv kv,
                              const void* q, const int32_t* seq_lens, int32_t batch,
                              int32_t max_seq_len, float* out, int32_t* sel_groups,
                              int32_t* sel_pages, void* stream);

/* Host-only: workspace bytes for lod_attend_prefill. */
int lod_prefill_ws_bytes(const lod_params* params, int32_t batch, int32_t n_q,
                         int32_t max_tokens, size_t* bytes);

/*
 * LoD prefill (causal): rows q_start .. q_start+n_q-1 of every sequence, each row p
 * computed exactly as lod_attend_decode computes a query at p (same selection, same
 * terms).  K/V rows [0, q_start+n_q) must be in the cache and chunks
 * 0 .. n_b(q_start+n_q-1)-1 built.  q_start must be a multiple of chunk_size.
 *   q           [batch][n_q][n_q_heads][head_dim], kv_dtype
 *   out         [batch][n_q][n_q_heads][head_dim] fp32
 *   sel_groups  nullable [batch][n_q][n_q_heads][top_groups]
 *   sel_pages   nullable [batch][n_q][n_q_heads][top_groups][max(top_pages,1)]
 * Limit (bf16 caches): the rows of one call may see at most 16384 summarised groups per
 * KV head (512K tokens at 8 groups per chunk, 256K at 16): LOD_ERR_UNSUPPORTED beyond
 * that, before anything is enqueued.  fp32 caches have no such limit.
 */
int lod_attend_prefill(const lod_params* params, const lod_index* index, lod_kv kv,
                       const void* q, int32_t q_start, int32_t n_q, int32_t batch, float* out,
                       int32_t* sel_groups, int32_t* sel_pages, void* ws, size_t ws_bytes,
                       void* stream);

/* Host-only: workspace bytes for lod_dense_decode. */
int lod_dense_decode_ws_bytes(const lod_params* params, int32_t batch, int32_t max_seq_len,
                              size_t* bytes);

/*
 * Dense causal softmax attention of one query per sequence over rows [0, seq_lens[b]-1]
 * (no LoD): the baseline the method is measured against.  Same q/out/seq_lens layout
 * as lod_attend_decode; uses only params' head counts, head_dim, kv_dtype and scale.
 */
int lod_dense_decode(const lod_params* params, lod_kv kv, const void* q,
                     const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float* out,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Dense causal prefill: rows q_start .. q_start+n_q-1, row p attends to [0, p].
 * Same q/out layout as lod_attend_prefill.  No workspace.
 */
int lod_dense_prefill(const lod_params* params, lod_kv kv, const void* q, int32_t q_start,
                      int32_t n_q, int32_t batch, float* out, void* stream);

/*
 * Video LoD ("Level of Detail Attention", section "Video LoD"): the method carried over
 * to video, whose tokens are local in space and time, with queries and keys/values
 * handled in 4x4x4 blocks of the token grid and c = 16.  The section names only the
 * block shape and c; the rest follows the text method ("How It Works") read this way:
 *   - tokens sit on a frames x height x width grid, token t = (f*height + y)*width + x;
 *     attention is bidirectional (every query sees every key; no window, no sinks);
 *   - the grid is cut into block_f x block_h x block_w blocks, clipped at the far
 *     edges; block ids run in raster order of the block coordinates, a block's members
 *     in ascending token order.  A block plays the part of a group: it keeps its mean
 *     key and value (fp32 sums in member order, correctly rounded divide, rounded to
 *     nearest even to bf16) and ln(n) of its token count n;
 *   - the queries of a block share one choice: their mean query (the same fp32 mean,
 *     not rounded) scores every key block with the unscaled fp32 fma chain over the
 *     head dimension in index order, and the top_blocks best (score descending, then
 *     lower block id) open;
 *   - each query's softmax holds scale*q.k for every member of the opened blocks and,
 *     for every other block, one term scale*q.kbar + ln(n) with value vbar (its mean
 *     key and value repeated n times); drop_remainder = 1 leaves those terms out.
 * Supported: head_dim 128, kv_dtype LOD_BF16, block volume <= 64, 1 <= top_blocks <= 64,
 * at most 13312 blocks, n_q_heads a multiple of n_kv_heads (query head h reads KV head
 * h / (n_q_heads / n_kv_heads)); anything else valid returns LOD_ERR_UNSUPPORTED.
 */
typedef struct {
    int32_t head_dim;
    int32_t n_q_heads, n_kv_heads;
    int32_t frames, height, width;        /* token grid */
    int32_t block_f, block_h, block_w;    /* block extents along frames, rows, columns */
    int32_t top_blocks;                   /* c: key blocks each query block opens */
    int32_t kv_dtype;                     /* element type of q, K and V (LOD_BF16) */
    int32_t drop_remainder;               /* 0 or 1 (sparsity ablation) */
    float scale;                          /* softmax scale, usually 1/sqrt(head_dim) */
} lod_video_params;

/*
 * Byte offsets of the arrays in the workspace of lod_video_attend (NB blocks, d =
 * head_dim, B = batch); every array is 256-byte aligned.  They hold the last call's
 * summaries and choice, so tests can read them back:
 *   kbar, vbar  [B][n_kv_heads][NB][d] bf16   block mean key / value
 *   lnn         [NB]                   f32    ln(token count) of each block
 *   qbar        [B][n_q_heads][NB][d]  f32    block mean query
 *   sel         [B][n_q_heads][NB][top_blocks] int32  opened key blocks of each query
 *               block, ascending, -1 padding when NB < top_blocks
 */
typedef struct {
    size_t kbar, vbar, lnn, qbar, sel, total;
    int32_t n_blocks;
} lod_video_layout_t;

/* Host-only: workspace layout of lod_video_attend for `batch` sequences. */
int lod_video_layout(const lod_video_params* params, int32_t batch, lod_video_layout_t* layout);

/* Host-only: workspace bytes of lod_video_attend (layout.total). */
int lod_video_ws_bytes(const lod_video_params* params, int32_t batch, size_t* bytes);

/*
 * Video LoD attention of every token of `batch` token grids: summaries, choice and
 * softmax as described above, in one call.
 *   kv          strided view of K and V (block_table must be NULL: LOD_ERR_UNSUPPORTED
 *               otherwise); position t of the view is token t of the grid
 *   q           [batch][T][n_q_heads][head_dim] bf16, T = frames*height*width,
 *               16-byte aligned
 *   out         [batch][T][n_q_heads][head_dim] fp32
 *   sel_blocks  nullable [batch][n_q_heads][NB][top_blocks] int32: a copy of `sel`
 *   ws          workspace of at least lod_video_ws_bytes bytes, 16-byte aligned;
 *               LOD_ERR_WORKSPACE when smaller
 */
int lod_video_attend(const lod_video_params* params, lod_kv kv, const void* q, int32_t batch,
                     float* out, int32_t* sel_blocks, void* ws, size_t ws_bytes, void* stream);

/*
 * Dense bidirectional softmax attention of every token over all T keys: the baseline
 * video LoD is measured against.  Same q, kv and out layout as lod_video_attend; uses
 * the grid, head counts, head_dim, kv_dtype and scale of params.  No workspace.
 */
int lod_video_dense(const lod_video_params* params, lod_kv kv, const void* q, int32_t batch,
                    float* out, void* stream);

/*
 * Instrumentation (profiling only; results are unchanged).  While `events` is non-null,
 * every later lod_attend_decode / lod_attend_prefill / lod_video_attend call made from the
 * same host thread
 * records events[0] on its stream before its first kernel and events[1 + k] after its
 * k-th kernel (decode: k = 0 scan, 1 open-and-combine; bf16 prefill: k = 0 candidate
 * sweep, 1 select, 2 flash, 3 bucket, 4 pages, 5 combine, recorded again for every batch
 * of rows, so the last batch's times remain; lod_video_attend: k = 0 summaries, 1 choice,
 * 2 attention).  `events` points to n_events
 * hipEvent_t handles created by the caller, who reads them with hipEventElapsedTime;
 * kernels beyond n_events - 1 record nothing.  Pass NULL to stop.  Not for captured graphs.
 */
int lod_trace_events(void* const* events, int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* LOD_H */
