// Device-side types and CDNA4 (gfx950) matrix-core helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace edda {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDModel = 1280;
constexpr int kHeads = 20;
constexpr int kHeadDim = 64;
constexpr int kQkvCols = 3 * kDModel;
constexpr int kWave = 64;

// v_mfma_f32_32x32x16_f16.  Lane l (g = l / 32) supplies A[l % 32][8g .. 8g+7] and
// B[8g .. 8g+7][l % 32]; it receives D[8i + 4g + j][l % 32] in element 4i + j.
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_f16.  Lane l (G = l / 16) supplies A[l % 16][8G .. 8G+7] and
// B[8G .. 8G+7][l % 16]; it receives D[4G + r][l % 16] in element r.
__device__ __forceinline__ f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even pack of two fp32 values into fp16x2 (v_cvt_pk_f16_f32).
__device__ __forceinline__ f16x2 pack_rne(float a, float b) {
  return __builtin_convertvector((f32x2){a, b}, f16x2);
}

__device__ __forceinline__ f16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
  f16x2 p0 = pack_rne(a0, a1), p1 = pack_rne(a2, a3), p2 = pack_rne(a4, a5), p3 = pack_rne(a6, a7);
  return (f16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ f16x8 load16(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ void store16(f16* p, f16x8 v) { *reinterpret_cast<f16x8*>(p) = v; }

// Eight int8 Q8_0 codes (little-endian bytes of q) as fp16 values (exact: |code| <= 127).
__device__ __forceinline__ f16x8 codes_to_f16(u32x2 q) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (f16)(float)(int8_t)(q[0] >> (8 * j));
    r[4 + j] = (f16)(float)(int8_t)(q[1] >> (8 * j));
  }
  return r;
}

// 2^x on the transcendental unit (v_exp_f32); x <= 0 here, tiny results flush to 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace edda
