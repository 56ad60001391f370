// lod_host.cpp -- host-only parts of the LoD C ABI: status strings, argument checks,
// index layout and workspace sizing.  Nothing here touches the GPU.
#include <math.h>

#include "lod_internal.h"

namespace lodi {

int check_params(const lod_params* p) {
    if (!p) return LOD_ERR_ARG;
    if (p->head_dim <= 0 || p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->chunk_size <= 0 ||
        p->page_size <= 0 || p->groups_per_chunk <= 0 || p->top_groups <= 0 ||
        p->top_pages < 0 || p->window <= 0 || p->n_sink < 0 || p->kmeans_iters <= 0)
        return LOD_ERR_ARG;
    if (p->n_q_heads % p->n_kv_heads != 0) return LOD_ERR_ARG;
    if (p->window % p->chunk_size != 0) return LOD_ERR_ARG;
    if (p->n_sink >= p->chunk_size) return LOD_ERR_ARG;
    if (!(p->scale > 0.0f) || !isfinite(p->scale)) return LOD_ERR_ARG;
    if (p->drop_remainder != 0 && p->drop_remainder != 1) return LOD_ERR_ARG;
    if (p->int4_pages != 0 && p->int4_pages != 1) return LOD_ERR_ARG;
    if (p->kv_dtype != LOD_F32 && p->kv_dtype != LOD_BF16) return LOD_ERR_UNSUPPORTED;
    if (p->int4_pages && p->kv_dtype != LOD_BF16) return LOD_ERR_UNSUPPORTED;
    if (p->head_dim != kD || p->chunk_size != kChunk || p->page_size != kPage)
        return LOD_ERR_UNSUPPORTED;
    if (p->groups_per_chunk > kMaxG || p->top_groups > kMaxTG || p->top_pages > kPage)
        return LOD_ERR_UNSUPPORTED;
    const int g = p->n_q_heads / p->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return LOD_ERR_UNSUPPORTED;
    return LOD_OK;
}

int check_kv_view(const lod_params* p, const lod_kv& kv, int64_t positions) {
    if (!kv.k || !kv.v || kv.stride_t <= 0 || kv.stride_h < 0 || kv.stride_b < 0) return LOD_ERR_ARG;
    const int per16 = p->kv_dtype == LOD_BF16 ? 8 : 4;
    if ((kv.stride_t | kv.stride_h | kv.stride_b) % per16 != 0) return LOD_ERR_ARG;
    if (kv.block_table) {
        const int32_t bs = kv.block_size;
        if (bs < 1 || bs > 65536 || (bs & (bs - 1)) != 0) return LOD_ERR_ARG;
        if (kv.max_blocks <= 0 || (int64_t)kv.max_blocks * bs < positions) return LOD_ERR_ARG;
    }
    return LOD_OK;
}

lod_index_layout_t make_layout(const lod_params* p, int32_t batch, int32_t max_chunks) {
    lod_index_layout_t L{};
    const size_t U = (size_t)batch * p->n_kv_heads;
    const size_t NC = (size_t)max_chunks;
    const size_t G = p->groups_per_chunk, PS = page_slots(p), d = p->head_dim;
    const size_t E = elt_bytes(p);
    size_t o = 0;
    L.gk = o;     o = align256(o + U * NC * G * d * E);
    L.gv = o;     o = align256(o + U * NC * G * d * E);
    L.gln = o;    o = align256(o + U * NC * G * 4);
    L.gkn = o;    o = align256(o + U * NC * G * 4);
    L.gpage = o;  o = align256(o + U * NC * G * 4);
    L.pk = o;     o = align256(o + U * NC * PS * d * E);
    L.pv = o;     o = align256(o + U * NC * PS * d * E);
    L.pln = o;    o = align256(o + U * NC * PS * 4);
    L.meta = o;   o = align256(o + U * NC * meta_stride(p) * 2);
    L.assign = o; o = align256(o + U * NC * p->chunk_size);
    const size_t Q = p->int4_pages ? U * NC * p->chunk_size : 0;  // rows with 4-bit codes
    L.q4k = o;    o = align256(o + Q * d / 2);
    L.q4v = o;    o = align256(o + Q * d / 2);
    L.q4ks = o;   o = align256(o + Q * 4);
    L.q4vs = o;   o = align256(o + Q * 4);
    L.total = o;
    L.page_slots = (int32_t)PS;
    L.meta_stride = meta_stride(p);
    return L;
}

DecodePlan plan_decode(const lod_params* p, int32_t batch, int32_t max_seq_len) {
    DecodePlan P{};
    const int nb = built_chunks(p, (int64_t)max_seq_len - 1);
    const int64_t ng = (int64_t)nb * p->groups_per_chunk;
    const int64_t units = (int64_t)batch * p->n_kv_heads;
    if (p->kv_dtype == LOD_BF16) {
        // MFMA path: the scan workgroups of a unit share its list of 64-row tiles (group
        // summaries, then sinks and window).  About 1024 workgroups (four per CU) over the
        // batch, no more than the unit has tiles, at most kScanMaxSlots per unit.
        const int64_t ntiles = ceil_div(ng, kScanTile) + ceil_div((int64_t)p->n_sink + p->window, kScanTile);
        int64_t per = ceil_div(1024, units);
        if (per > ntiles) per = ntiles;
        if (per > kScanMaxSlots) per = kScanMaxSlots;
        if (per < 1) per = 1;
        P.slice = kScanTile;
        P.nslice = (int)per;
        P.nwin = 0;
    } else {
        // VALU path: about 512 slice workgroups of up to 256 groups, then a sinks
        // workgroup and 64-row window tiles
        int64_t want = ceil_div(512, units);
        int64_t slice = ceil_div(ng > 0 ? ng : 1, want);
        slice = ceil_div(slice, kTile) * kTile;
        if (slice < kTile) slice = kTile;
        if (slice > 4 * kTile) slice = 4 * kTile;
        P.slice = (int)slice;
        P.nwin = 1 + (int)ceil_div(p->window, kTile);
    }
    if (p->kv_dtype != LOD_BF16) P.nslice = ng > 0 ? (int)ceil_div(ng, P.slice) : 0;
    P.nslot = P.nslice + P.nwin;
    const size_t heads = (size_t)batch * p->n_q_heads;
    P.off_part = 0;
    P.off_cand = align256(heads * P.nslot * kPartStride * sizeof(float));
    P.off_score = align256(P.off_cand + heads * (size_t)(P.nslice > 0 ? P.nslice : 1) *
                                            p->top_groups * sizeof(uint64_t));
    // bf16: MFMA ranking score of every group for every query head
    P.score_stride = (int)(ng > 0 ? ceil_div(ng, 64) * 64 : 64);
    P.bytes = align256(P.off_score + (p->kv_dtype == LOD_BF16 ? heads * (size_t)P.score_stride * 4 : 0));
    return P;
}

DensePlan plan_dense(const lod_params* p, int32_t batch, int32_t max_seq_len) {
    DensePlan P{};
    const int64_t units = (int64_t)batch * p->n_kv_heads;
    // About 1024 workgroups, at least 4 tiles each so partials stay a small fraction.
    int64_t want = ceil_div(1024, units);
    int64_t rows = ceil_div(max_seq_len, want);
    rows = ceil_div(rows, kTile) * kTile;
    if (rows < 4 * kTile) rows = 4 * kTile;
    P.rows_per_wg = (int)rows;
    P.nsplit = (int)ceil_div(max_seq_len, rows);
    P.bytes = align256((size_t)batch * p->n_q_heads * P.nsplit * kPartStride * sizeof(float));
    return P;
}

static thread_local void* const* g_trace = nullptr;
static thread_local int g_ntrace = 0;

void* const* trace_events(int* n) {
    *n = g_ntrace;
    return g_trace;
}

void trace_point(int k, hipStream_t st) {
    if (g_trace && k < g_ntrace) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(g_trace[k]), st);
}

}  // namespace lodi

using namespace lodi;

extern "C" {

const char* lod_status_string(int status) {
    switch (status) {
        case LOD_OK: return "LOD_OK";
        case LOD_ERR_ARG: return "LOD_ERR_ARG: invalid argument";
        case LOD_ERR_UNSUPPORTED: return "LOD_ERR_UNSUPPORTED: parameters not supported";
        case LOD_ERR_WORKSPACE: return "LOD_ERR_WORKSPACE: buffer too small";
        case LOD_ERR_HIP: return "LOD_ERR_HIP: HIP runtime or launch failure";
        default: return "unknown status";
    }
}

int lod_trace_events(void* const* events, int32_t n_events) {
    if (events && n_events <= 0) return LOD_ERR_ARG;
    g_trace = events;
    g_ntrace = events ? n_events : 0;
    return LOD_OK;
}

int lod_index_layout(const lod_params* params, int32_t batch, int32_t max_chunks,
                     lod_index_layout_t* layout) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!layout || batch <= 0 || max_chunks < 0) return LOD_ERR_ARG;
    *layout = make_layout(params, batch, max_chunks);
    return LOD_OK;
}

int lod_index_bytes(const lod_params* params, int32_t batch, int32_t max_tokens, size_t* bytes) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!bytes || batch <= 0 || max_tokens < 0) return LOD_ERR_ARG;
    *bytes = make_layout(params, batch, max_tokens / params->chunk_size).total;
    return LOD_OK;
}

int lod_decode_ws_bytes(const lod_params* params, int32_t batch, int32_t max_seq_len,
                        size_t* bytes) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!bytes || batch <= 0 || max_seq_len <= 0) return LOD_ERR_ARG;
    *bytes = plan_decode(params, batch, max_seq_len).bytes;
    return LOD_OK;
}

int lod_dense_decode_ws_bytes(const lod_params* params, int32_t batch, int32_t max_seq_len,
                              size_t* bytes) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!bytes || batch <= 0 || max_seq_len <= 0) return LOD_ERR_ARG;
    *bytes = plan_dense(params, batch, max_seq_len).bytes;
    return LOD_OK;
}

}  // extern "C"
