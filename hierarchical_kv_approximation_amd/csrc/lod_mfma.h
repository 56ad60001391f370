// lod_mfma.h -- MFMA operand types and small helpers shared by the MFMA kernels.
//
// v_mfma_f32_16x16x32_bf16 lane layout on gfx950 (checked on the device):
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B (32 x 16): lane l holds B[8 * (l / 16) + j][l % 16]
//   D (16 x 16): lane l holds D[4 * (l / 16) + r][l % 16], r = 0..3
#pragma once

#include "lod_device.h"

namespace lodi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
    bf16x8_t z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
    return z;
}

// fp32 -> bf16, round to nearest even (one hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

// Split x into bf16 hi + lo with x - hi - lo below 2^-16 |x| (for PV operands).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

constexpr int kFlashRowHeads = 128;  // query rows x heads per prefill workgroup
constexpr int kFlashKeys = 64;       // keys per LDS tile
constexpr int kFlashWaves = 8;       // waves of a prefill flash workgroup (one 16-column block each)
constexpr int kFlashThreads = 64 * kFlashWaves;

}  // namespace lodi
