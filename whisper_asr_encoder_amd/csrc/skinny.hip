// Kernel 6: the decoder's block-sized GEMMs (with the KV-cache append in a fused variant).
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
// Fused variants for the decoder layer: the operand rows normalised by LayerNorm inside the
// kernel (no separate LayerNorm launch), and the KV-cache append done by the QKV epilogue.

#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "layer_norm_row.hpp"

namespace edda {
namespace {

constexpr int kSkWaves = 8;
constexpr int kSkThreads = kSkWaves * kWave;
constexpr int kSkCols = 16;
constexpr int kSkUnroll = 4;
constexpr int kLnGroups = kDModel / 256;  // rows normalised in the kernel have 1280 features
constexpr int kALd = kDModel + 8;         // LDS row stride (halves): 16 rows hit 16 bank groups

__device__ __forceinline__ float gelu_exact_sk(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}

// LN: A's rows are LayerNorm inputs (K = 1280): every workgroup normalises the block rows
// into LDS (layer_norm_row, so the rows equal the LayerNorm kernel's bit for bit) while
// its first weight loads are in flight, and reads its operand rows from there.
// APPEND: C is a packed QKV block; its K and V columns are also stored into the caches'
// rows slots[m] (the KV-cache append, done by the epilogue).
struct SkinnyLn {
  const f16* gamma;
  const f16* beta;
};
struct SkinnyAppend {
  f16* k_cache;
  f16* v_cache;
  Slots slots;
};
// Split K (gridDim.y > 1): workgroup (j, sp) covers steps [sp * per, (sp + 1) * per) of
// column block j and stores its fp32 partial tile (agent-scope atomic stores, coherent across
// the XCDs' L2 caches without cache-wide operations); the last of the block's workgroups to
// count itself in on counters[j * kSplitCounterStride] sums the partials in split order (so the
// result does not depend on arrival order), applies the epilogue, and resets the counter.
struct SkinnySplit {
  uint32_t* counters;
  float* part;
};
struct SkinnyW {
  const void* w;       // fp16 [N][K], or int8 codes [N][K]
  const void* scales;  // null, or fp16 [K / 32][N]
};
constexpr int kSplitCounterStride = 16;  // uint32 words: one counter per 64 bytes

__device__ __forceinline__ void store_coherent_f32(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent_f32(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Q8: the weights are Q8_0 blocks: int8 codes [N][K] and fp16 scales [K / 32][N] (one per
// 32-deep block of a weight row, stored step-major so a lane's four output rows' scales of
// a step are 8 contiguous bytes).  A K step covers exactly one block, so the codes (exact
// in fp16) go through the MFMA on their own (accumulator 0) and the step's dot products are
// scaled in fp32: acc[r] += d[n][step] * sum_k q[n][k] x[m][k].
struct WFrag16 {
  f16x8 w;
};
struct WFragQ8 {
  u32x2 q;
  f16x4 d;
};

template <int ACT, bool RES, bool LN, bool APPEND, bool SPLIT, bool Q8>
__global__ __launch_bounds__(kSkThreads) void skinny_gemm_kernel(const f16* __restrict__ A,
                                                                 const void* __restrict__ Bt,
                                                                 const f16* __restrict__ wscale,
                                                                 const f16* __restrict__ bias,
                                                                 const f16* residual, int res_period, f16* C,
                                                                 int M, int N, int K, SkinnyLn ln,
                                                                 SkinnyAppend ap, SkinnySplit sk) {
  __shared__ int last_arrival;
  __shared__ float red[kSkWaves][kSkCols][kSkCols + 1];
  __shared__ __attribute__((aligned(16))) f16 a_lds[LN ? 16 * kALd : 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kSkCols;
  const int per = K / 32 / gridDim.y;  // steps of this workgroup's K range
  const int steps = (int)(blockIdx.y + 1) * per;
  using WFrag = std::conditional_t<Q8, WFragQ8, WFrag16>;
  // Weight row n0 + r16, 8 consecutive k of each step: 16 bytes (fp16) or 8 bytes (codes).
  const char* wrow = static_cast<const char*>(Bt) + (size_t)(n0 + r16) * K * (Q8 ? 1 : 2) + 8 * g * (Q8 ? 1 : 2);
  const f16* srow = Q8 ? wscale + n0 + 4 * g : nullptr;
  auto wload = [&](int st) -> WFrag {
    if constexpr (Q8) {
      return WFragQ8{*reinterpret_cast<const u32x2*>(wrow + 32 * st),
                     *reinterpret_cast<const f16x4*>(srow + (size_t)st * N)};
    } else {
      return WFrag16{*reinterpret_cast<const f16x8*>(wrow + 64 * st)};
    }
  };
  auto mma = [&](const WFrag& w, f16x8 x, f32x4 acc) -> f32x4 {
    if constexpr (Q8) {
      const f32x4 t = mfma_16x16x32(codes_to_f16(w.q), x, (f32x4){});
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fmaf((float)w.d[r], t[r], acc[r]);
      return acc;
    } else {
      return mfma_16x16x32(w.w, x, acc);
    }
  };
  const int arow = min(r16, M - 1);
  const f16* xrow = A + (size_t)arow * K + 8 * g;
  auto xload = [&](int st) -> f16x8 {
    if constexpr (LN) return *reinterpret_cast<const f16x8*>(&a_lds[arow * kALd + 32 * st + 8 * g]);
    else return load16(xrow + 32 * st);
  };
  f32x4 acc = {};
  int s = (int)blockIdx.y * per + wave;
  // Groups of kSkUnroll steps: all loads of a group are issued before its MFMAs.  The first
  // group's weights are requested before anything else.
  const bool group0 = s + (kSkUnroll - 1) * kSkWaves < steps;
  WFrag wf[kSkUnroll];
  f16x8 xf[kSkUnroll];
  if (group0) {
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) wf[u] = wload(s + u * kSkWaves);
  }
  if constexpr (LN) {
    // Rows wave and wave + 8 (M <= 16): both rows' loads are issued before either is used.
    const int r0 = wave, r1 = wave + kSkWaves;
    const LnRow<kLnGroups> row0 = layer_norm_load<kLnGroups>(A + (size_t)min(r0, M - 1) * kDModel, ln.gamma,
                                                             ln.beta, lane);
    const LnRow<kLnGroups> row1 = layer_norm_load<kLnGroups>(A + (size_t)min(r1, M - 1) * kDModel, ln.gamma,
                                                             ln.beta, lane);
    // Both rows' statistics interleaved; a row past M (clamped to row M - 1) is not stored.
    layer_norm_finish2<kLnGroups>(
        row0, row1, lane,
        [&](int f, f16x4 v) { if (r0 < M) *reinterpret_cast<f16x4*>(&a_lds[r0 * kALd + f]) = v; },
        [&](int f, f16x4 v) { if (r1 < M) *reinterpret_cast<f16x4*>(&a_lds[r1 * kALd + f]) = v; });
    __syncthreads();
  }
  if (group0) {
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) xf[u] = xload(s + u * kSkWaves);
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) acc = mma(wf[u], xf[u], acc);
    s += kSkUnroll * kSkWaves;
  }
  for (; s + (kSkUnroll - 1) * kSkWaves < steps; s += kSkUnroll * kSkWaves) {
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) {
      wf[u] = wload(s + u * kSkWaves);
      xf[u] = xload(s + u * kSkWaves);
    }
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) acc = mma(wf[u], xf[u], acc);
  }
  for (; s < steps; s += kSkWaves) acc = mma(wload(s), xload(s), acc);
  // acc[r] = C^T[n = 4 g + r][m = r16] partial over this wave's steps.
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * g + r][r16] = acc[r];
  __syncthreads();
  const int m = tid / kSkCols, n = tid % kSkCols;
  float v = 0.0f;
  if (tid < kSkCols * kSkCols) {
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) v += red[w][n][m];
  }
  if constexpr (SPLIT) {
    const int nsplit = gridDim.y;
    float* const part = sk.part + (size_t)blockIdx.x * nsplit * (kSkCols * kSkCols);
    if (tid < kSkCols * kSkCols) store_coherent_f32(part + blockIdx.y * (kSkCols * kSkCols) + tid, v);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial is acknowledged before the count
    __syncthreads();
    uint32_t* const counter = sk.counters + blockIdx.x * kSplitCounterStride;
    if (tid == 0)
      last_arrival = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)(nsplit - 1);
    __syncthreads();
    if (!last_arrival) return;
    if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid >= kSkCols * kSkCols || m >= M) return;
    v = 0.0f;
    for (int q = 0; q < nsplit; ++q) v += load_coherent_f32(part + q * (kSkCols * kSkCols) + tid);
  } else {
    if (tid >= kSkCols * kSkCols || m >= M) return;
  }
  if (bias) v += (float)bias[n0 + n];
  if constexpr (ACT == 1) v = gelu_exact_sk(v);
  if constexpr (RES) v += (float)residual[(size_t)(m % res_period) * N + n0 + n];
  const f16 out = (f16)v;
  C[(size_t)m * N + n0 + n] = out;
  if constexpr (APPEND) {
    const int col = n0 + n - kDModel;  // 0 .. 1279: K, 1280 .. 2559: V
    if (col >= 0) {
      const size_t row = (size_t)ap.slots.s[m] * kDModel;
      if (col < kDModel) ap.k_cache[row + col] = out;
      else ap.v_cache[row + col - kDModel] = out;
    }
  }
}

// W: fp16 weights (scales null) or Q8_0 codes with their scales.
template <int ACT, bool RES, bool LN, bool APPEND, bool SPLIT = false>
hipError_t launch_sk(const void* A, const SkinnyW& W, const void* bias, const void* residual, int res_period, void* C,
                     int M, int N, int K, SkinnyLn ln, const SkinnyAppend& ap, hipStream_t stream,
                     int nsplit = 1, SkinnySplit sk = {}) {
  const dim3 grid(N / kSkCols, nsplit);
  if (W.scales) {
    hipLaunchKernelGGL((skinny_gemm_kernel<ACT, RES, LN, APPEND, SPLIT, true>), grid, dim3(kSkThreads), 0, stream,
                       static_cast<const f16*>(A), W.w, static_cast<const f16*>(W.scales),
                       static_cast<const f16*>(bias), static_cast<const f16*>(residual), res_period,
                       static_cast<f16*>(C), M, N, K, ln, ap, sk);
  } else {
    hipLaunchKernelGGL((skinny_gemm_kernel<ACT, RES, LN, APPEND, SPLIT, false>), grid, dim3(kSkThreads), 0, stream,
                       static_cast<const f16*>(A), W.w, nullptr, static_cast<const f16*>(bias),
                       static_cast<const f16*>(residual), res_period, static_cast<f16*>(C), M, N, K, ln, ap, sk);
  }
  return hipGetLastError();
}

// Q8_0 quantizer: one thread per 32-value block of a weight row (see the Q8 comment above).
// Every decision is taken in fp32 as the format defines it: amax exact, d = amax / 127 and
// 1 / d correctly rounded, codes = round-half-away(x * (1 / d)), d stored as fp16 (RNE).
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const f16* __restrict__ w, int rows, int cols,
                                                            int8_t* __restrict__ codes, f16* __restrict__ scales) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const int blocks_per_row = cols / 32;
  if (t >= (long)rows * blocks_per_row) return;
  const int n = (int)(t / blocks_per_row), kb = (int)(t - (long)n * blocks_per_row);
  const f16* src = w + (size_t)n * cols + 32 * kb;
  f16x8 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = load16(src + 8 * i);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)v[i][j]));
  const float d = amax / 127.0f;
  const float inv = d != 0.0f ? 1.0f / d : 0.0f;
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t word[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = (int)roundf((float)v[i][j] * inv);
      word[j >> 2] |= (uint32_t)(uint8_t)(int8_t)c << (8 * (j & 3));
    }
    out[i >> 1][2 * (i & 1)] = word[0];
    out[i >> 1][2 * (i & 1) + 1] = word[1];
  }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + (size_t)n * cols + 32 * kb);
  dst[0] = out[0];
  dst[1] = out[1];
  scales[(size_t)kb * rows + n] = (f16)d;
}

}  // namespace

hipError_t launch_skinny_gemm(const void* A, const void* Bt, const void* bias, const void* residual, int res_period,
                              int act, void* C, int M, int N, int K, hipStream_t stream, const void* scales) {
  if (M < 1 || M > 16 || N % kSkCols || K % 32) return hipErrorInvalidValue;
  const SkinnyW W{Bt, scales};
  const SkinnyLn ln{};
  const SkinnyAppend ap{};
  if (act == 1)
    return residual ? launch_sk<1, true, false, false>(A, W, bias, residual, res_period, C, M, N, K, ln, ap, stream)
                    : launch_sk<1, false, false, false>(A, W, bias, residual, res_period, C, M, N, K, ln, ap, stream);
  return residual ? launch_sk<0, true, false, false>(A, W, bias, residual, res_period, C, M, N, K, ln, ap, stream)
                  : launch_sk<0, false, false, false>(A, W, bias, residual, res_period, C, M, N, K, ln, ap, stream);
}

// At most two K ranges per column block: measured on the decoder layer (32 layers, 16-token
// block; A/B in one process), 2 ranges 62.8 us per layer against 64.4 for 4 and 66.5 for 1 —
// the partials' round trip does not shrink with more ranges, the weight stream per range does.
int skinny_splits(int N, int K) {
  const int blocks = N / kSkCols, steps = K / 32;
  int s = 1;
  while (s < 2 && blocks * s * 2 <= 320 && steps % (2 * s) == 0 && steps / (2 * s) >= kSkWaves) s *= 2;
  return s;
}

size_t skinny_split_part_bytes(int N, int K) {
  const int s = skinny_splits(N, K);
  return s > 1 ? (size_t)(N / kSkCols) * s * kSkCols * kSkCols * sizeof(float) : 0;
}

hipError_t launch_skinny_gemm_split(const void* A, const void* Bt, const void* bias, const void* residual,
                                    int res_period, int act, void* C, int M, int N, int K, void* counters,
                                    void* part, hipStream_t stream, const void* scales) {
  if (M < 1 || M > 16 || N % kSkCols || K % 32 || act != 0) return hipErrorInvalidValue;
  const int ns = skinny_splits(N, K);
  if (ns == 1) return launch_skinny_gemm(A, Bt, bias, residual, res_period, act, C, M, N, K, stream, scales);
  if (!counters || !part) return hipErrorInvalidValue;
  const SkinnyW W{Bt, scales};
  const SkinnySplit sk{static_cast<uint32_t*>(counters), static_cast<float*>(part)};
  const SkinnyLn ln{};
  const SkinnyAppend ap{};
  return residual ? launch_sk<0, true, false, false, true>(A, W, bias, residual, res_period, C, M, N, K, ln, ap,
                                                           stream, ns, sk)
                  : launch_sk<0, false, false, false, true>(A, W, bias, residual, res_period, C, M, N, K, ln, ap,
                                                            stream, ns, sk);
}

hipError_t launch_skinny_ln_gemm(const void* A, const void* gamma, const void* beta, const void* Bt, const void* bias,
                                 int act, void* C, int M, int N, void* k_cache, void* v_cache, const Slots* slots,
                                 hipStream_t stream, const void* scales) {
  const int K = kDModel;
  if (M < 1 || M > 16 || N % kSkCols || !gamma || !beta) return hipErrorInvalidValue;
  const SkinnyW W{Bt, scales};
  const SkinnyLn ln{static_cast<const f16*>(gamma), static_cast<const f16*>(beta)};
  if (k_cache) {
    if (act != 0 || N != kQkvCols || !v_cache || !slots) return hipErrorInvalidValue;
    const SkinnyAppend ap{static_cast<f16*>(k_cache), static_cast<f16*>(v_cache), *slots};
    return launch_sk<0, false, true, true>(A, W, bias, nullptr, 1, C, M, N, K, ln, ap, stream);
  }
  const SkinnyAppend ap{};
  if (act == 1) return launch_sk<1, false, true, false>(A, W, bias, nullptr, 1, C, M, N, K, ln, ap, stream);
  return launch_sk<0, false, true, false>(A, W, bias, nullptr, 1, C, M, N, K, ln, ap, stream);
}

hipError_t launch_quantize_q8_0(const void* w, int rows, int cols, void* codes, void* scales, hipStream_t stream) {
  if (rows < 1 || cols < 32 || cols % 32) return hipErrorInvalidValue;
  const long blocks = ((long)rows * (cols / 32) + 255) / 256;
  if (blocks >= (1L << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const f16*>(w),
                     rows, cols, static_cast<int8_t*>(codes), static_cast<f16*>(scales));
  return hipGetLastError();
}

}  // namespace edda
