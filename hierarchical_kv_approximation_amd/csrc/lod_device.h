// lod_device.h -- device helpers shared by the LoD kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lod_internal.h"

namespace lodi {

typedef uint16_t bf16_t;  // bfloat16 bits
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16 raw bytes

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bfloat16 bits (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) {
        if (u & 0x007fffffu) u |= 0x00400000u;
        return (bf16_t)(u >> 16);
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
    static constexpr int kPer16 = 4;  // elements per 16-byte load
    __device__ static __forceinline__ float to_f32(float x) { return x; }
    __device__ static __forceinline__ float store_round(float x) { return x; }
    // Unpack one 16-byte chunk into kPer16 floats.
    __device__ static __forceinline__ void unpack(const uint4& u, float* o) {
        o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
        o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
    }
    __device__ static __forceinline__ void unpack(const u32x4_t& u, float* o) {
        o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
        o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
    }
};
template <> struct Elt<bf16_t> {
    static constexpr int kPer16 = 8;
    __device__ static __forceinline__ float to_f32(bf16_t x) { return bf16_bits_to_f32(x); }
    __device__ static __forceinline__ bf16_t store_round(float x) { return f32_to_bf16_rne(x); }
    __device__ static __forceinline__ void unpack(const uint4& u, float* o) {
        o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
        o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
        o[4] = __uint_as_float(u.z << 16); o[5] = __uint_as_float(u.z & 0xffff0000u);
        o[6] = __uint_as_float(u.w << 16); o[7] = __uint_as_float(u.w & 0xffff0000u);
    }
    __device__ static __forceinline__ void unpack(const u32x4_t& u, float* o) {
        o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
        o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
        o[4] = __uint_as_float(u.z << 16); o[5] = __uint_as_float(u.z & 0xffff0000u);
        o[6] = __uint_as_float(u.w << 16); o[7] = __uint_as_float(u.w & 0xffff0000u);
    }
};

// Storage conversion of an fp32 mean to the element type.
__device__ __forceinline__ void store_elt(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_elt(bf16_t* p, float x) { *p = f32_to_bf16_rne(x); }

// Ranking key: larger key = higher score, then lower id.  -0 and +0 rank equal.
__device__ __forceinline__ uint64_t rank_key(float r, uint32_t id) {
    uint32_t u = __float_as_uint(r == 0.0f ? 0.0f : r);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xffffffffu - (uint32_t)k; }
// Insert x into the descending list t[0..N), which keeps the N largest values seen (with
// multiplicity).  The new t[e] is the median of the old t[e-1], t[e] and x (x clamped
// into [t[e], t[e-1]]), so every entry is one independent med3 of old values; the head
// is med3(t[0], x, +inf), the larger of the two (no NaN reaches these lists).  x and the
// +inf pass through empty asm: otherwise the compiler turns the head back into a max
// with NaN quieting, and branches on x = -inf (an invalid element) to a copy of the list.
// pinf: +inf, formed by the caller through empty asm (once, outside its loops).
template <int N>
__device__ __forceinline__ void insert_desc(float (&t)[N], float x, float pinf) {
    asm volatile("" : "+v"(x));
    float prev = t[0];
    t[0] = __builtin_amdgcn_fmed3f(prev, x, pinf);
#pragma unroll
    for (int e = 1; e < N; ++e) {
        const float cur = t[e];
        t[e] = __builtin_amdgcn_fmed3f(prev, cur, x);
        prev = cur;
    }
}
template <int N>
__device__ __forceinline__ void insert_desc(float (&t)[N], float x) {
    float pinf = INFINITY;
    asm volatile("" : "+v"(pinf));
    insert_desc(t, x, pinf);
}
__device__ __forceinline__ float key_score(uint64_t k) {
    uint32_t u = (uint32_t)(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}

// Full-wavefront reductions of the ROCm device library (DPP based).  Every lane of the
// wave must execute them; the result is returned to every lane.
extern "C" __device__ __attribute__((const)) unsigned long long __ockl_wfred_max_u64(unsigned long long);
extern "C" __device__ __attribute__((const)) float __ockl_wfred_max_f32(float);
extern "C" __device__ __attribute__((const)) float __ockl_wfred_add_f32(float);

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) { return __ockl_wfred_max_u64(v); }
// width: reduce over aligned groups of `width` lanes (64 = the whole wave).
__device__ __forceinline__ float wave_max_f32(float v, int width) {
    if (width == 64) return __ockl_wfred_max_f32(v);
    for (int m = width >> 1; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_sum_f32(float v, int width) {
    if (width == 64) return __ockl_wfred_add_f32(v);
    for (int m = width >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Reductions over each aligned group of 16 lanes (a DPP row): rotations by 8, 4, 2 and 1
// lanes within the row.  Each step pairs lanes symmetrically, so every lane of the row
// ends with the same bits.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float row16_sum_f32(float v) {
    v += __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));  // row_ror:8
    v += __uint_as_float(dpp_u32<0x124>(__float_as_uint(v)));  // row_ror:4
    v += __uint_as_float(dpp_u32<0x122>(__float_as_uint(v)));  // row_ror:2
    v += __uint_as_float(dpp_u32<0x121>(__float_as_uint(v)));  // row_ror:1
    return v;
}
__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
#define LODI_ROW_MAX_STEP(CTRL)                                                              \
    {                                                                                     \
        const uint64_t o = ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) |         \
                           dpp_u32<CTRL>((uint32_t)v);                                    \
        v = o > v ? o : v;                                                                \
    }
    LODI_ROW_MAX_STEP(0x128)
    LODI_ROW_MAX_STEP(0x124)
    LODI_ROW_MAX_STEP(0x122)
    LODI_ROW_MAX_STEP(0x121)
#undef LODI_ROW_MAX_STEP
    return v;
}

// Inclusive prefix sum over the 64 lanes: a zero-filled shift scan inside each 16-lane
// row (DPP row_shr 1, 2, 4, 8), then the totals of the lower rows (read from lanes 15,
// 31, 47).  Every lane of the wave must execute it.
template <int CTRL>
__device__ __forceinline__ int dpp_shr_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
    v += dpp_shr_i32<0x111>(v);
    v += dpp_shr_i32<0x112>(v);
    v += dpp_shr_i32<0x114>(v);
    v += dpp_shr_i32<0x118>(v);
    const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
              t2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (int)(__lane_id() >> 4);
    return v + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
}

// Element offset of KV row (sequence b, position t) for head 0, for any argument block
// with fields sb, st (strides), btab (block table or null), bshift (log2 block size) and
// maxb (block-table row length), split as kv_seq(b) + kv_pos(b, t).  PAGED: position t
// sits in block btab[b][t >> bshift] at row t & (block size - 1), and kv_seq is 0;
// strided: sequence b starts at b * sb (kv_seq, loop invariant) and t adds t * st.
template <bool PAGED, typename Args>
__device__ __forceinline__ int64_t kv_seq(const Args& A, int b) {
    if constexpr (PAGED) return 0;
    else return (int64_t)b * A.sb;
}
template <bool PAGED, typename Args>
__device__ __forceinline__ int64_t kv_pos(const Args& A, int b, int t) {
    if constexpr (PAGED) {
        const int64_t blk = A.btab[(int64_t)b * A.maxb + (t >> A.bshift)];
        return blk * A.sb + (int64_t)(t & ((1 << A.bshift) - 1)) * A.st;
    } else {
        return (int64_t)t * A.st;
    }
}
template <bool PAGED, typename Args>
__device__ __forceinline__ int64_t kv_row(const Args& A, int b, int t) {
    return kv_seq<PAGED>(A, b) + kv_pos<PAGED>(A, b, t);
}
// The same with the view chosen at run time (kernels off the hot path).
template <typename Args>
__device__ __forceinline__ int64_t kv_row_rt(const Args& A, int b, int t) {
    return A.btab ? kv_row<true>(A, b, t) : kv_row<false>(A, b, t);
}

// Workgroup barrier over LDS traffic only: each wave waits for its own LDS operations
// (lgkmcnt 0), not for its vector memory operations, so loads of a later tile (also
// global -> LDS loads, whose completion the caller awaits with an explicit vmcnt wait
// before the barrier) stay in flight.  __syncthreads would wait for all of them.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Order this wave's earlier LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// exp(x) for x <= 0 (softmax weights); exp(-inf) = 0.
__device__ __forceinline__ float softmax_exp(float x) { return __expf(x); }

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

// Online-softmax state of one 16-lane subgroup: lane holds o for dims 8*l16 .. 8*l16+7.
struct Online {
    float m, l, o[8];
    __device__ void init() {
        m = -INFINITY;
        l = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.0f;
    }
    __device__ __forceinline__ void add(float lam, const float* v) {
        if (lam == -INFINITY) return;
        const float mn = fmaxf(m, lam);
        const float a = softmax_exp(m - mn);  // m = -inf -> 0
        const float w = softmax_exp(lam - mn);
        l = __builtin_fmaf(l, a, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(w, v[e], o[e] * a);
        m = mn;
    }
};

// Bound on |S - r| / (|q| |kbar|) between an MFMA dot product S of bf16 vectors (exact
// products, fp32 accumulation in any order) and the canonical fp32 fma chain r: each is
// within gamma_128 * sum|q_t k_t| <= gamma_128 |q| |kbar| of the exact value
// (gamma_n = n u / (1 - n u), u = 2^-24), so |S - r| <= 2 gamma_128 |q| |kbar|; the
// constant is four times that.
constexpr float kErrC = 8.0f * 128.0f / 16777216.0f;

}  // namespace lodi
