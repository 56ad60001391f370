// lod_internal.h -- layout, launch planning and argument checks shared by the host
// entry points of the LoD library.  Pure host C++ (no HIP types), so it also builds
// for CPU-only checks.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "lod.h"

namespace lodi {

constexpr int kD = 128;        // supported head dimension
constexpr int kChunk = 256;    // supported chunk size
constexpr int kPage = 16;      // supported page size
constexpr int kMaxG = 16;      // groups per chunk
constexpr int kMaxTG = 16;     // opened groups per query
constexpr int kThreads = 256;  // threads per workgroup of every kernel
constexpr int kTile = 64;      // rows per LDS tile in the decode kernels
constexpr int kPartStride = kD + 4;  // floats per partial softmax state: o[d], m, l, pad
constexpr int kScanTile = 64;        // rows per tile of the bf16 decode scan
constexpr int kScanMaxSlots = 40;    // bf16 decode scan workgroups per (sequence, KV head), at most
constexpr int kCUs = 256;            // compute units of the gfx950 part that launch shapes are sized for

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validate the parameter block (host).  Returns LOD_OK or an error status.
int check_params(const lod_params* p);

inline int elt_bytes(const lod_params* p) { return p->kv_dtype == LOD_BF16 ? 2 : 4; }
inline int page_slots(const lod_params* p) { return p->chunk_size / p->page_size + p->groups_per_chunk; }
inline int meta_stride(const lod_params* p) {
    int n = (p->groups_per_chunk + 1) + (page_slots(p) + 1) + p->chunk_size;
    return (n + 31) & ~31;  // 64-byte multiple of int16 entries
}
// Chunks summarised for a query at position pos (block-granular window).
inline int built_chunks(const lod_params* p, int64_t pos) {
    int64_t nb = pos / p->chunk_size - p->window / p->chunk_size + 1;
    return nb < 0 ? 0 : (int)nb;
}

lod_index_layout_t make_layout(const lod_params* p, int32_t batch, int32_t max_chunks);

// Decode launch plan, a pure function of (params, batch, max_seq_len).
struct DecodePlan {
    int slice;      // fp32: groups per slice workgroup (multiple of kTile); bf16: kScanTile
    int nslice;     // fp32: slice workgroups per (sequence, KV head); bf16: scan workgroups
    int nwin;       // fp32: window workgroups per (sequence, KV head); bf16: 0
    int nslot;      // partial softmax states per (sequence, query head)
    int score_stride;  // bf16: stored MFMA scores per (sequence, query head)
    size_t off_part, off_cand, off_score, bytes;
};
DecodePlan plan_decode(const lod_params* p, int32_t batch, int32_t max_seq_len);

struct DensePlan {
    int rows_per_wg;  // rows of one split workgroup (multiple of kTile)
    int nsplit;
    size_t bytes;
};
DensePlan plan_dense(const lod_params* p, int32_t batch, int32_t max_seq_len);

// Checks of a KV view shared by the entry points (host): strides, alignment, and for a
// paged view the block size and that the table rows cover `positions` positions.
int check_kv_view(const lod_params* p, const lod_kv& kv, int64_t positions);
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline int log2_exact(int32_t x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}
// Copy a KV view into a kernel argument block (fields sb, st, sh, btab, bshift, maxb).
template <typename Args>
inline void set_kv_map(Args& A, const lod_kv& kv) {
    A.sb = kv.stride_b; A.st = kv.stride_t; A.sh = kv.stride_h;
    A.btab = kv.block_table;
    A.bshift = kv.block_table ? log2_exact(kv.block_size) : 0;
    A.maxb = kv.block_table ? kv.max_blocks : 0;
}
// LoD prefill row by row through the decode kernels (fp32 caches).
int prefill_rows_ws_bytes(const lod_params* params, int32_t n_q, int32_t max_tokens, size_t* bytes);
int prefill_rows(const lod_params* params, const lod_index* index, lod_kv kv, const void* q,
                 int32_t q_start, int32_t n_q, int32_t batch, float* out, int32_t* sel_groups,
                 int32_t* sel_pages, void* ws, size_t ws_bytes, void* stream);
// Dense causal prefill of fp32 caches (VALU path).
int dense_prefill_valu(const lod_params* params, lod_kv kv, const void* q, int32_t q_start,
                       int32_t n_q, int32_t batch, float* out, void* stream);

// Events set by lod_trace_events for the calling host thread (null when off).
void* const* trace_events(int* n);
// Record trace event k on st when events are set and k is in range.
void trace_point(int k, hipStream_t st);


}  // namespace lodi
