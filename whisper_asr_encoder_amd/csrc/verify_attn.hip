// Kernel 3: block-verification attention.  n_q <= 16 query tokens (anchor plus
// drafted tokens, or one token per beam) attend to a KV cache [n_kv, 20, 64]
// whose slot j holds position j, under per-query bitset mask rows (causal,
// token-tree ancestors, or none for cross-attention).
//
// The work is memory bound (each K/V byte is used by at most 16 queries) and small
// (a few MB per call), so the time is latency: the key sequence is split across
// many workgroups, one launch covers the call, and every load a wave needs is
// issued at kernel start.  A cache of at most 512 keys takes one workgroup per head: 4
// waves of up to three 32-key chunks (384 keys), else 8 waves of two; a longer one is split
// into 128-key ranges, one workgroup (split, head) each, 32 keys per wave.  Per wave and chunk, on
// 16x16x32 MFMAs: S^T = K Q^T (lane l holds 8 scores of query l % 16); masked softmax
// statistics over the wave's chunks via cross-lane max/sum (lane swaps between 16- and
// 32-lane halves); then O^T = V^T P^T, summed over the chunks, with P kept in
// registers as the B operand and V^T staged through wave-private LDS tiles.  The
// waves merge in LDS.  With more than one split, each workgroup writes fp32 partials
// (m, l, unnormalized o) to the workspace and counts itself in on a per-head arrival
// counter; the last to arrive merges every split of its head:
//   m = max_s m_s,  l = sum_s l_s 2^(m_s - m),  O = sum_s o_s 2^(m_s - m) / l,
// and sets the counter back to zero.  A query with no admitted key gets O = 0.
//
// Variants for the drafter's attention (llama.cpp DSpark diff): the head count is a runtime
// value (head_dim 64); the mask is explicit rows, none, or the causal block (query t of the
// block in the last n_q slots admits slots 0..n_kv-n_q+t) computed in the kernel; optional
// per-head sinks join the final normalization as one extra logit with a zero value:
//   M' = max(M, sink), L' = L 2^(M - M') + 2^(sink - M'), O = sum 2^(M - M') / L'.
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "../../include/edda.h"

namespace edda {
namespace {

constexpr int kVWaves = 4;
constexpr int kVThreads = kVWaves * kWave;
constexpr int kWaveKeys = 32;
constexpr int kSplitKeys = kVWaves * kWaveKeys;
constexpr int kMaxQ = 16;
constexpr int kVtLd = kWaveKeys + 4;  // V^T row stride (halves): 72 B, 8-byte aligned
// Per-head arrival counters at the workspace start, one per 256-byte line so that the
// heads' atomics do not queue on a shared line.
constexpr int kMaxHeads = 64;
constexpr int kCounterStride = 64;  // uint32 words
constexpr size_t kCounterBytes = (size_t)kMaxHeads * kCounterStride * sizeof(uint32_t);
static_assert(kCounterBytes == EDDA_VERIFY_COUNTER_BYTES, "counter region size in the public header");

// s_waitcnt immediate: vmcnt 0, expcnt and lgkmcnt at their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kMergeBatch = 16;  // splits whose partials the merging workgroup loads at once

// Two floats (8-byte aligned) as one agent-scope atomic access.
__device__ __forceinline__ void store_coherent(float* p, float a, float b) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, (f32x2){a, b}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 load_coherent(const float* p) {
  return __builtin_bit_cast(f32x2, __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }

// Max / sum over lanes {l, l ^ 16, l ^ 32, l ^ 48}.  The gfx950 lane swaps exchange
// odd and even 16-lane rows (permlane16) and the two 32-lane halves (permlane32)
// between two registers; with both operands x, the two results hold x of lane l and
// of lane l ^ 16 (resp. l ^ 32), in the same order in both lanes of a pair, so the
// combined value is bitwise equal across the four lanes.
__device__ __forceinline__ float quad_max(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = fmaxf(as_f32(p[0]), as_f32(p[1]));
  auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return fmaxf(as_f32(r[0]), as_f32(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = as_f32(p[0]) + as_f32(p[1]);
  auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}

// Fold a per-head sink (log2 units) into the running (M, L) and the accumulator scale.
__device__ __forceinline__ float apply_sink(float& M, float& L, float s2) {
  if (s2 == -INFINITY) return 1.0f;
  const float m2 = fmaxf(M, s2);
  const float a = M == -INFINITY ? 0.0f : exp2_fast(M - m2);
  L = L * a + exp2_fast(s2 - m2);
  M = m2;
  return a;
}

enum MaskMode { kMaskRows = 0, kMaskNone = 1, kMaskCausal = 2 };

// grid (n_splits, n_heads), 256 threads.  counters / part_ml / part_o are used only
// when n_splits > 1 (they are written by other workgroups, so not restrict).
// NW waves (4 or 8) of CPW 32-key chunks each.  A workgroup covers NW * 32 * CPW keys, wave w
// chunk c the 32 keys from (c NW + w) 32 on: one split of up to 512 keys (4 waves of up to 3
// chunks up to 384 keys, else 8 waves of 2 chunks), or 128-key splits of 4 waves of one chunk.
template <int kMode, int CPW, int NW>
__global__ __launch_bounds__(NW * kWave) void verify_kernel(
    const f16* __restrict__ q, int q_stride, int n_q, const f16* __restrict__ k, const f16* __restrict__ v,
    int n_kv, int n_heads, const uint32_t* __restrict__ mask, int mask_words, const float* __restrict__ sinks,
    f16* __restrict__ o, uint32_t* counters, float* part_ml, float* part_o) {
  __shared__ __attribute__((aligned(16))) f16 Vt[NW][CPW][kHeadDim * kVtLd];
  __shared__ float mw[NW][kMaxQ], lw[NW][kMaxQ];
  __shared__ __attribute__((aligned(16))) float ow[NW][kMaxQ][kHeadDim + 4];
  __shared__ int last_arrival;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, G = lane >> 4;
  const int split = blockIdx.x, head = blockIdx.y, n_splits = gridDim.x;
  const int wg_key0 = split * NW * kWaveKeys * CPW;
  auto chunk_key0 = [&](int c) { return wg_key0 + (c * NW + wave) * kWaveKeys; };  // multiple of 32
  const int kKvStride = n_heads * kHeadDim;
  const int last_key = n_kv - 1;
  const f16x8 z8 = {};

  // Every global load first, unconditionally (rows past the cache end are clamped to
  // its last row and masked out below; element offsets fit 32 bits for any valid n_kv).
  const bool q_ok = r16 < n_q;
  const int q_row = min(r16, n_q - 1);
  uint32_t bits[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int key0 = chunk_key0(c);
    bits[c] = 0xffffffffu;
    if constexpr (kMode == kMaskRows)
      bits[c] = mask[(uint32_t)(q_row * mask_words + min(key0 >> 5, mask_words - 1))];
    if constexpr (kMode == kMaskCausal) {
      const int last = n_kv - n_q + q_row - key0;  // highest admitted key, relative to key0
      bits[c] = last < 0 ? 0u : last >= 31 ? 0xffffffffu : (uint32_t)((2ull << last) - 1);
    }
  }
  f16x8 qf[2], kf[CPW][2][2], va[CPW][2], vb[CPW][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) qf[s] = load16(q + (uint32_t)(q_row * q_stride + head * kHeadDim + 32 * s + 8 * G));
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int key0 = chunk_key0(c);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = min(key0 + 16 * blk + r16, last_key);
      const uint32_t off = (uint32_t)(key * kKvStride + head * kHeadDim + 8 * G);
      kf[c][blk][0] = load16(k + off);
      kf[c][blk][1] = load16(k + (off + 32));
    }
    // V rows as two keys per 16-byte group, for the transposed LDS staging.
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int u = lane + kWave * r;
      const int kp = u >> 3, c8 = u & 7;
      const int key = key0 + 2 * kp;
      va[c][r] = load16(v + (uint32_t)(min(key, last_key) * kKvStride + head * kHeadDim + 8 * c8));
      vb[c][r] = load16(v + (uint32_t)(min(key + 1, last_key) * kKvStride + head * kHeadDim + 8 * c8));
    }
  }
  if (!q_ok) qf[0] = qf[1] = z8;

  // Stage this wave's V tiles transposed: Vt[d][key - key0]; key pairs share a 32-bit word.
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int u = lane + kWave * r;
      const int kp = u >> 3, c8 = u & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<f16x2*>(&Vt[wave][c][(8 * c8 + e) * kVtLd + 2 * kp]) = (f16x2){va[c][r][e], vb[c][r][e]};
    }

  // S^T for keys key0 + 16 blk + 4 G + r of each chunk, query r16; one softmax over the
  // wave's chunks.
  const float c_scale = kLog2e / 8.0f;
  float sc[CPW][8];
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    f32x4 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sacc[blk] = mfma_16x16x32(kf[c][blk][0], qf[0], (f32x4){});
      sacc[blk] = mfma_16x16x32(kf[c][blk][1], qf[1], sacc[blk]);
    }
    const uint32_t b = q_ok ? bits[c] : 0u;
    const int key0 = chunk_key0(c);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * blk + 4 * G + r;
        const bool ok = ((b >> kk) & 1u) && (key0 + kk < n_kv);
        const float sv = ok ? sacc[blk][r] * c_scale : -INFINITY;
        sc[c][4 * blk + r] = sv;
        m = fmaxf(m, sv);
      }
  }
  m = quad_max(m);
  float l = 0.0f;
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = (m == -INFINITY) ? 0.0f : exp2_fast(sc[c][i] - m);
      sc[c][i] = p;
      l += p;
    }
  l = quad_sum(l);

  __syncthreads();  // V^T tiles visible to every lane
  f16x8 pf[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
    pf[c] = pack8(sc[c][0], sc[c][1], sc[c][2], sc[c][3], sc[c][4], sc[c][5], sc[c][6], sc[c][7]);
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    f32x4 oa = {};
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const f16* row = &Vt[wave][c][(16 * dd + r16) * kVtLd];
      const f16x4 lo = *reinterpret_cast<const f16x4*>(row + 4 * G);
      const f16x4 hi = *reinterpret_cast<const f16x4*>(row + 16 + 4 * G);
      const f16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oa = mfma_16x16x32(vf, pf[c], oa);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) ow[wave][r16][16 * dd + 4 * G + r] = oa[r];
  }
  if (G == 0) {
    mw[wave][r16] = m;
    lw[wave][r16] = l;
  }
  __syncthreads();

  // Merge the NW waves: thread -> (query mq, dims d0 .. d0 + 3); with 8 waves the threads past
  // the 16th query read query 15's values and store nothing.
  const int mq_t = tid >> 4, mq = min(mq_t, kMaxQ - 1), d0 = (tid & 15) * 4;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w][mq]);
  float L = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = exp2_fast(mw[w][mq] - M);
      L += lw[w][mq] * wt;
      const f32x4 ov = *reinterpret_cast<const f32x4*>(&ow[w][mq][d0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += ov[j] * wt;
    }
  }
  const bool row_ok = mq_t < n_q;
  f16* out = o + ((size_t)mq * n_heads + head) * kHeadDim + d0;
  const float sink2 = sinks ? sinks[head] * kLog2e : -INFINITY;
  if (n_splits == 1) {
    if (!row_ok) return;
    const float a = apply_sink(M, L, sink2);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] *= a;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const f16x2 lo = pack_rne(acc[0] * inv, acc[1] * inv), hi = pack_rne(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<f16x4*>(out) = (f16x4){lo[0], lo[1], hi[0], hi[1]};
    return;
  }

  // Partials of this split, then the arrival count.  The partials and the counter are
  // accessed with agent-scope atomics, which the XCDs' separate L2 caches keep coherent
  // without whole-cache write-back or invalidation.  Each wave waits until its stores
  // are acknowledged before the workgroup barrier, so they are visible device-wide
  // before thread 0 counts the workgroup in; the last workgroup's loads are issued
  // after the count returned.
  // Slot (split s, query mq, head): (m, l) at part_ml[2 slot], o at part_o[64 slot + d0];
  // slot = (s n_q + mq) n_heads + head, all offsets below 2^31 for any valid call.
  const int slot0 = mq * n_heads + head, slot_step = n_q * n_heads;
  if (row_ok) {
    const int slot = split * slot_step + slot0;
    store_coherent(part_o + (uint32_t)(slot * kHeadDim + d0), acc[0], acc[1]);
    store_coherent(part_o + (uint32_t)(slot * kHeadDim + d0 + 2), acc[2], acc[3]);
    if (d0 == 0) store_coherent(part_ml + (uint32_t)(slot * 2), M, L);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid == 0)
    last_arrival = __hip_atomic_fetch_add(&counters[head * kCounterStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (uint32_t)(n_splits - 1);
  __syncthreads();
  if (!last_arrival) return;
  // Every split has arrived: reset the counter for the next call.
  if (tid == 0) __hip_atomic_store(&counters[head * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!row_ok) return;
  // Merge the splits kMergeBatch at a time: every load of a batch is issued before any
  // is used (indices past the last split are clamped and their weights dropped), and
  // the running (M, L, sum) is rescaled to each batch's maximum.
  M = -INFINITY;
  L = 0.0f;
  f32x4 sum = {};
  for (int s0 = 0; s0 < n_splits; s0 += kMergeBatch) {
    float pm[kMergeBatch], pl[kMergeBatch];
    f32x4 po[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int slot = min(s0 + i, n_splits - 1) * slot_step + slot0;
      const f32x2 ml = load_coherent(part_ml + (uint32_t)(slot * 2));
      const f32x2 o01 = load_coherent(part_o + (uint32_t)(slot * kHeadDim + d0));
      const f32x2 o23 = load_coherent(part_o + (uint32_t)(slot * kHeadDim + d0 + 2));
      pm[i] = ml[0];
      pl[i] = ml[1];
      po[i] = (f32x4){o01[0], o01[1], o23[0], o23[1]};
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (s0 + i < n_splits) mb = fmaxf(mb, pm[i]);
    if (mb == -INFINITY) continue;  // no admitted key so far
    const float a = M == -INFINITY ? 0.0f : exp2_fast(M - mb);
    L *= a;
#pragma unroll
    for (int j = 0; j < 4; ++j) sum[j] *= a;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      // 0 for a split with no admitted key (m = -inf) and for indices past the last split.
      const float wt = s0 + i < n_splits ? exp2_fast(pm[i] - mb) : 0.0f;
      L += pl[i] * wt;
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[j] += po[i][j] * wt;
    }
    M = mb;
  }
  const float a = apply_sink(M, L, sink2);
#pragma unroll
  for (int j = 0; j < 4; ++j) sum[j] *= a;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const f16x2 lo = pack_rne(sum[0] * inv, sum[1] * inv), hi = pack_rne(sum[2] * inv, sum[3] * inv);
  *reinterpret_cast<f16x4*>(out) = (f16x4){lo[0], lo[1], hi[0], hi[1]};
}

}  // namespace

namespace {
constexpr int kOneWorkgroupKeys = 4 * kSplitKeys;  // up to 512 keys: one workgroup per head

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_words(void* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

int verify_num_splits(int n_kv) { return n_kv <= kOneWorkgroupKeys ? 1 : (n_kv + kSplitKeys - 1) / kSplitKeys; }

size_t verify_workspace_bytes(int n_q, int n_kv, int n_heads) {
  const int s = verify_num_splits(n_kv);
  if (s <= 1) return 0;
  return kCounterBytes + (size_t)s * n_q * n_heads * (2 + kHeadDim) * sizeof(float);
}

hipError_t launch_verify(const void* q, int q_stride, int n_q, const void* k, const void* v, int n_kv, int n_heads,
                         int mask_mode, const uint32_t* mask, const float* sinks, void* o, void* workspace,
                         hipStream_t stream) {
  const int n_splits = verify_num_splits(n_kv);
  const int mask_words = (n_kv + 31) / 32;
  uint32_t* counters = nullptr;
  float* part_ml = nullptr;
  float* part_o = nullptr;
  if (n_splits > 1) {
    counters = static_cast<uint32_t*>(workspace);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    part_o = part_ml + (size_t)n_splits * n_q * n_heads * 2;
  }
  const dim3 grid(n_splits, n_heads);
  int threads = kVThreads;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, static_cast<const f16*>(q), q_stride, n_q,
                       static_cast<const f16*>(k), static_cast<const f16*>(v), n_kv, n_heads, mask, mask_words, sinks,
                       static_cast<f16*>(o), counters, part_ml, part_o);
    return hipGetLastError();
  };
  // One split: 4 waves of 1-3 chunks up to 384 keys, else 8 waves of 2 (measured: at 360
  // keys 4 waves of 3 chunks beat 8 of 2 by 7 %, at 448 keys 8 of 2 beat 4 of 4 by 12 %).
  auto by_chunks = [&](auto mode_c) {
    constexpr int M = decltype(mode_c)::value;
    if (n_splits == 1 && n_kv > 3 * kSplitKeys) {
      threads = 8 * kWave;
      return go(verify_kernel<M, 2, 8>);
    }
    if (n_splits == 1 && n_kv > 2 * kSplitKeys) return go(verify_kernel<M, 3, kVWaves>);
    if (n_splits == 1 && n_kv > kSplitKeys) return go(verify_kernel<M, 2, kVWaves>);
    return go(verify_kernel<M, 1, kVWaves>);
  };
  if (mask_mode == kMaskRows) return by_chunks(std::integral_constant<int, kMaskRows>());
  if (mask_mode == kMaskCausal) return by_chunks(std::integral_constant<int, kMaskCausal>());
  return by_chunks(std::integral_constant<int, kMaskNone>());
}

}  // namespace edda
