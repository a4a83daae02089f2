// Kernels 6 and 7: the decoder's block-sized GEMMs and the KV-cache append.
//
// Skinny GEMM (M <= 16 rows, the verification block): C[M, N] = act(A B^T + bias) +
// residual, as kernel 1, for the projections of the anchor plus drafted tokens.  The work is
// bound by streaming the weights (N x K fp16, read once), so operands go straight from
// global memory into registers, with no LDS staging and many workgroups in flight:
// workgroup j owns output columns 16j .. 16j+15 over the whole K; its 8 waves take the
// 32-deep K steps w, w+8, ... and each runs 16x16x32 MFMAs computing the transposed tile
// (weights as the A operand: lane l holds 8 consecutive k of weight row 16j + l % 16; the
// block rows as the B operand, rows past M clamped to M-1 and never stored).  The 8 partial
// tiles are summed in LDS; the epilogue adds the bias, applies the activation, adds the
// residual, rounds once to fp16, and each thread stores one element of a 16-column run.
//
// KV append: the block's K and V rows (columns 1280..2559 and 2560..3839 of its packed QKV
// rows) are copied into cache slots given per token, 16-byte chunks per thread.
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace edda {
namespace {

constexpr int kSkWaves = 8;
constexpr int kSkThreads = kSkWaves * kWave;
constexpr int kSkCols = 16;
constexpr int kSkUnroll = 4;

__device__ __forceinline__ float gelu_exact_sk(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}

template <int ACT, bool RES>
__global__ __launch_bounds__(kSkThreads) void skinny_gemm_kernel(const f16* __restrict__ A,
                                                                 const f16* __restrict__ Bt,
                                                                 const f16* __restrict__ bias,
                                                                 const f16* residual, int res_period, f16* C,
                                                                 int M, int N, int K) {
  __shared__ float red[kSkWaves][kSkCols][kSkCols + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kSkCols;
  const int steps = K / 32;
  const f16* wrow = Bt + (size_t)(n0 + r16) * K + 8 * g;
  const f16* xrow = A + (size_t)min(r16, M - 1) * K + 8 * g;
  f32x4 acc = {};
  int s = wave;
  // Groups of kSkUnroll steps: all loads of a group are issued before its MFMAs.
  for (; s + (kSkUnroll - 1) * kSkWaves < steps; s += kSkUnroll * kSkWaves) {
    f16x8 wf[kSkUnroll], xf[kSkUnroll];
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) {
      wf[u] = load16(wrow + 32 * (s + u * kSkWaves));
      xf[u] = load16(xrow + 32 * (s + u * kSkWaves));
    }
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) acc = mfma_16x16x32(wf[u], xf[u], acc);
  }
  for (; s < steps; s += kSkWaves) acc = mfma_16x16x32(load16(wrow + 32 * s), load16(xrow + 32 * s), acc);
  // acc[r] = C^T[n = 4 g + r][m = r16] partial over this wave's steps.
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * g + r][r16] = acc[r];
  __syncthreads();
  if (tid >= kSkCols * kSkCols) return;
  const int m = tid / kSkCols, n = tid % kSkCols;
  if (m >= M) return;
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < kSkWaves; ++w) v += red[w][n][m];
  if (bias) v += (float)bias[n0 + n];
  if constexpr (ACT == 1) v = gelu_exact_sk(v);
  if constexpr (RES) v += (float)residual[(size_t)(m % res_period) * N + n0 + n];
  C[(size_t)m * N + n0 + n] = (f16)v;
}

template <int ACT, bool RES>
hipError_t launch_sk(const void* A, const void* Bt, const void* bias, const void* residual, int res_period, void* C,
                     int M, int N, int K, hipStream_t stream) {
  hipLaunchKernelGGL((skinny_gemm_kernel<ACT, RES>), dim3(N / kSkCols), dim3(kSkThreads), 0, stream,
                     static_cast<const f16*>(A), static_cast<const f16*>(Bt), static_cast<const f16*>(bias),
                     static_cast<const f16*>(residual), res_period, static_cast<f16*>(C), M, N, K);
  return hipGetLastError();
}

// One workgroup per block token: 2 x 160 chunks of 16 bytes (K row, V row).
__global__ __launch_bounds__(256) void append_kv_kernel(const f16* __restrict__ qkv, Slots slots,
                                                        f16* __restrict__ k_cache, f16* __restrict__ v_cache) {
  const int t = blockIdx.x;
  const size_t dst = (size_t)slots.s[t] * kHeads * kHeadDim;
  const f16* src = qkv + (size_t)t * 3 * kHeads * kHeadDim;
  constexpr int kChunks = kHeads * kHeadDim / 8;  // 160 per row
  for (int c = threadIdx.x; c < 2 * kChunks; c += 256) {
    const bool is_v = c >= kChunks;
    const int cc = is_v ? c - kChunks : c;
    const f16x8 val = load16(src + (is_v ? 2 : 1) * kHeads * kHeadDim + 8 * cc);
    store16((is_v ? v_cache : k_cache) + dst + 8 * cc, val);
  }
}

}  // namespace

hipError_t launch_skinny_gemm(const void* A, const void* Bt, const void* bias, const void* residual, int res_period,
                              int act, void* C, int M, int N, int K, hipStream_t stream) {
  if (M < 1 || M > 16 || N % kSkCols || K % 32) return hipErrorInvalidValue;
  if (act == 1)
    return residual ? launch_sk<1, true>(A, Bt, bias, residual, res_period, C, M, N, K, stream)
                    : launch_sk<1, false>(A, Bt, bias, residual, res_period, C, M, N, K, stream);
  return residual ? launch_sk<0, true>(A, Bt, bias, residual, res_period, C, M, N, K, stream)
                  : launch_sk<0, false>(A, Bt, bias, residual, res_period, C, M, N, K, stream);
}

hipError_t launch_append_kv(const void* qkv, int n_q, const Slots& slots, void* k_cache, void* v_cache,
                            hipStream_t stream) {
  hipLaunchKernelGGL(append_kv_kernel, dim3(n_q), dim3(256), 0, stream, static_cast<const f16*>(qkv), slots,
                     static_cast<f16*>(k_cache), static_cast<f16*>(v_cache));
  return hipGetLastError();
}

}  // namespace edda
