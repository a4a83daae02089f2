// LayerNorm of one row by one wave, shared by the LayerNorm kernel and the block-row GEMM
// that normalises its own operand rows: y = (x - mean) / sqrt(var + 1e-5) * gamma + beta,
// var the biased variance, statistics in fp32 over values held in registers (two passes over
// the registers, one read of the row), one rounding to fp16.  (The fused decoder layer uses
// the same arithmetic.)  Each lane holds kGroups groups
// of 4 consecutive features (feature 4 (c * 64 + lane) + j), so a wave reads 512 contiguous
// bytes per group; both callers get bit-identical rows.
#pragma once

#include <math.h>

#include "device.hpp"

namespace edda {

constexpr float kLnEps = 1e-5f;

// Sum over the 64 lanes, in registers.  Within each 16-lane row a lane adds its partner's value
// with a symmetric partner relation (quad neighbours at distances 1 and 2, then mirrored lanes
// within 8 and 16: DPP), so every lane of a row holds the same row sum; the DPP row broadcasts
// then add row 0 into row 1 and row 2 into row 3 (from lane 15 of the row below), and rows 0-1
// into rows 2-3 (from lane 31), so lane 63 holds the total, which v_readlane hands to every
// lane.  (The gfx950 lane-swap builtins are avoided here: combined in one commutative operation,
// their two results have been compiled as if they were the same value.)
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float ln_dpp_add(float v) {
  const int p = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF, false);
  return v + __builtin_bit_cast(float, p);
}
__device__ __forceinline__ float ln_wave_sum(float v) {
  v = ln_dpp_add<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = ln_dpp_add<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = ln_dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = ln_dpp_add<0x140, 0xF>(v);  // row_mirror
  v = ln_dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = ln_dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// The row's values and its gamma / beta slices in registers (loaded together, so one memory
// round trip precedes the arithmetic).
template <int kGroups>
struct LnRow {
  f16x4 v[kGroups], g[kGroups], b[kGroups];
};

template <int kGroups>
__device__ __forceinline__ LnRow<kGroups> layer_norm_load(const f16* __restrict__ xr, const f16* __restrict__ gamma,
                                                          const f16* __restrict__ beta, int lane) {
  LnRow<kGroups> r;
#pragma unroll
  for (int c = 0; c < kGroups; ++c) {
    const int f = 4 * (c * kWave + lane);
    r.v[c] = *reinterpret_cast<const f16x4*>(xr + f);
    r.g[c] = *reinterpret_cast<const f16x4*>(gamma + f);
    r.b[c] = *reinterpret_cast<const f16x4*>(beta + f);
  }
  // Keep every load of the row here, ahead of the reductions (left to itself the scheduler
  // issues gamma and beta after them: a second memory round trip).
  __builtin_amdgcn_sched_barrier(0);
  return r;
}

// store(f, value) receives the normalised fp16 values of features f .. f + 3.
// The lane's sums run in four independent accumulators (one per position j of a group, added
// in group order, then combined as (s0 + s1) + (s2 + s3)): a 20-long chain of dependent adds
// would leave the wave waiting on the adder's latency.
template <int kGroups>
__device__ __forceinline__ float ln_stats(const LnRow<kGroups>& r, float& rstd) {
  constexpr int kFeatures = 256 * kGroups;
  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < kGroups; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] += (float)r.v[c][j];
  const float mean = ln_wave_sum((s[0] + s[1]) + (s[2] + s[3])) * (1.0f / kFeatures);
  float q[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < kGroups; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d = (float)r.v[c][j] - mean;
      q[j] += d * d;
    }
  rstd = 1.0f / sqrtf(ln_wave_sum((q[0] + q[1]) + (q[2] + q[3])) * (1.0f / kFeatures) + kLnEps);
  return mean;
}

template <int kGroups, typename Store>
__device__ __forceinline__ void ln_apply(const LnRow<kGroups>& r, float mean, float rstd, int lane, Store store) {
#pragma unroll
  for (int c = 0; c < kGroups; ++c) {
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = ((float)r.v[c][j] - mean) * rstd * (float)r.g[c][j] + (float)r.b[c][j];
    const f16x2 lo = pack_rne(o[0], o[1]), hi = pack_rne(o[2], o[3]);
    store(4 * (c * kWave + lane), (f16x4){lo[0], lo[1], hi[0], hi[1]});
  }
}

template <int kGroups, typename Store>
__device__ __forceinline__ void layer_norm_finish(const LnRow<kGroups>& r, int lane, Store store) {
  float rstd;
  const float mean = ln_stats<kGroups>(r, rstd);
  ln_apply<kGroups>(r, mean, rstd, lane, store);
}

// Two rows by one wave, their statistics interleaved (each row's arithmetic as above).
template <int kGroups, typename Store0, typename Store1>
__device__ __forceinline__ void layer_norm_finish2(const LnRow<kGroups>& r0, const LnRow<kGroups>& r1, int lane,
                                                   Store0 store0, Store1 store1) {
  float rstd0, rstd1;
  const float mean0 = ln_stats<kGroups>(r0, rstd0);
  const float mean1 = ln_stats<kGroups>(r1, rstd1);
  ln_apply<kGroups>(r0, mean0, rstd0, lane, store0);
  ln_apply<kGroups>(r1, mean1, rstd1, lane, store1);
}

template <int kGroups, typename Store>
__device__ __forceinline__ void layer_norm_row(const f16* __restrict__ xr, const f16* __restrict__ gamma,
                                               const f16* __restrict__ beta, int lane, Store store) {
  layer_norm_finish<kGroups>(layer_norm_load<kGroups>(xr, gamma, beta, lane), lane, store);
}

}  // namespace edda
