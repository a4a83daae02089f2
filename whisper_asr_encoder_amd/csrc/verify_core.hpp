// The block-verification attention of one (split, head) work unit, shared by the standalone
// verification kernel and the fused decoder layer.  n_q <= 16 query tokens attend to a KV
// cache [n_kv, n_heads, 64] whose slot j holds position j, under per-query bitset mask rows
// (causal, token-tree ancestors, or none for cross-attention).
//
// A unit covers NW waves x CPW 32-key chunks (wave w, chunk c: the 32 keys from
// (c NW + w) 32 on, after the unit's first key).  Per wave and chunk, on 16x16x32 MFMAs:
// S^T = K Q^T (lane l holds 8 scores of query l % 16); masked softmax statistics over the
// wave's chunks via cross-lane max/sum (lane swaps between 16- and 32-lane halves); then
// O^T = V^T P^T, summed over the chunks, with P kept in registers as the B operand and V^T
// staged through wave-private LDS tiles.  The waves merge in LDS.  With more than one split,
// each unit writes fp32 partials (m, l, unnormalized o) and counts itself in on a per-head
// arrival counter; the last to arrive merges every split of its head:
//   m = max_s m_s,  l = sum_s l_s 2^(m_s - m),  O = sum_s o_s 2^(m_s - m) / l,
// and sets the counter back to zero.  A query with no admitted key gets O = 0.
//
// Variants for the drafter's attention (llama.cpp DSpark diff): the head count is a runtime
// value (head_dim 64); the mask is explicit rows, none, or the causal block (query t of the
// block in the last n_q slots admits slots 0..n_kv-n_q+t) computed in the kernel; optional
// per-head sinks join the final normalization as one extra logit with a zero value:
//   M' = max(M, sink), L' = L 2^(M - M') + 2^(sink - M'), O = sum 2^(M - M') / L'.
#pragma once

#include <math.h>

#include "device.hpp"

namespace edda {
namespace vcore {

constexpr int kWaveKeys = 32;
constexpr int kMaxQ = 16;
constexpr int kVtLd = kWaveKeys + 4;  // V^T row stride (halves): 72 B, 8-byte aligned
// Per-head arrival counters, one per 256-byte line so that the heads' atomics do not queue
// on a shared line.
constexpr int kCounterStride = 64;  // uint32 words
// s_waitcnt immediate: vmcnt 0, expcnt and lgkmcnt at their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kMergeBatch = 16;  // default: splits whose partials the merging unit loads at once

enum MaskMode { kMaskRows = 0, kMaskNone = 1, kMaskCausal = 2 };

// Two floats (8-byte aligned) as one agent-scope atomic access: coherent across the XCDs'
// separate L2 caches without whole-cache write-back or invalidation.
__device__ __forceinline__ void store_coherent(float* p, float a, float b) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, (f32x2){a, b}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 load_coherent(const float* p) {
  return __builtin_bit_cast(f32x2, __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Four floats (16-byte aligned) read / written with the device-coherent cache policy (sc1)
// through a buffer access: at a float index from a wave-uniform base.  One 16-byte store per
// lane keeps a wave's 1 KB of partials in whole 64-byte lines (two 8-byte stores would each
// touch every line with half of its bytes, doubling the write requests).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ f32x4 load_coherent4(const float* base, uint32_t idx) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(coherent_rsrc(base), 4 * idx, 0, 16));
}
__device__ __forceinline__ void store_coherent4(float* base, uint32_t idx, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), coherent_rsrc(base), 4 * idx, 0, 16);
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

// LDS of one unit.
template <int CPW, int NW>
struct Smem {
  alignas(16) f16 Vt[NW][CPW][kHeadDim * kVtLd];
  float mw[NW][kMaxQ], lw[NW][kMaxQ];
  alignas(16) float ow[NW][kMaxQ][kHeadDim + 4];
  int last_arrival;
};

// One call's operands.  counters / part_ml / part_o are used only when n_splits > 1 (they
// are written by other workgroups, so not restrict).
struct Args {
  const f16* q;
  int q_stride;
  int n_q;
  const f16* k;
  const f16* v;
  int n_kv;
  int n_heads;
  const uint32_t* mask;
  int mask_words;
  const float* sinks;
  f16* o;
  uint32_t* counters;
  float* part_ml;
  float* part_o;
};

// Memory policy of the standalone kernel: every operand was written before the launch.
struct PlainIo {
  static constexpr bool kFreshRows = false;
  __device__ bool fresh(int) const { return false; }
  __device__ void wait() const {}
  __device__ static f16x8 load_q(const f16* base, uint32_t off) { return load16(base + off); }
  __device__ f16x8 fresh_k(int, int) const { return f16x8{}; }
  __device__ f16x8 fresh_v(int, int) const { return f16x8{}; }
  // O row-major: [n_q][n_heads][64].
  __device__ static void store_o(const Args& a, int mq, int head, int d0, f16x4 v) {
    *reinterpret_cast<f16x4*>(a.o + ((size_t)mq * a.n_heads + head) * kHeadDim + d0) = v;
  }
};

// The unit (split, head) of n_splits.  Io supplies the memory policy: wait() runs after the
// K/V loads of the rows that exist before the unit starts and before every other load; keys
// for which fresh(key) holds are loaded only after it, through fresh_k / fresh_v(key, column
// within the [n_heads * 64] row); Q through load_q(base, element offset); O's four values (query mq, head, dims d0 ..
// d0 + 3) stored through store_o(args, mq, head, d0, values).  Threads of a workgroup all call this (it has barriers); it
// returns per thread.  tid: the thread's index in the workgroup.  MB: splits whose partials
// the merging unit loads at once.
template <int kMode, int CPW, int NW, typename Io, int MB = kMergeBatch>
__device__ __forceinline__ void verify_unit(const Args& a, int split, int head, int n_splits, Smem<CPW, NW>& sm,
                                            const Io& io, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, G = lane >> 4;
  static_assert(NW * kWave >= kMaxQ * (kHeadDim / 4), "the merge gives each (query, 4 dims) a thread");
  const int wg_key0 = split * NW * kWaveKeys * CPW;
  auto chunk_key0 = [&](int c) { return wg_key0 + (c * NW + wave) * kWaveKeys; };  // multiple of 32
  const int kKvStride = a.n_heads * kHeadDim;
  const int n_kv = a.n_kv, n_q = a.n_q;
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
      bits[c] = a.mask[(uint32_t)(q_row * a.mask_words + min(key0 >> 5, a.mask_words - 1))];
    if constexpr (kMode == kMaskCausal) {
      const int last = n_kv - n_q + q_row - key0;  // highest admitted key, relative to key0
      bits[c] = last < 0 ? 0u : last >= 31 ? 0xffffffffu : (uint32_t)((2ull << last) - 1);
    }
  }
  f16x8 qf[2], kf[CPW][2][2], va[CPW][2], vb[CPW][2];
  auto k_off = [&](int c, int blk) {
    const int key = min(chunk_key0(c) + 16 * blk + r16, last_key);
    return (uint32_t)(key * kKvStride + head * kHeadDim + 8 * G);
  };
  // V rows as two keys per 16-byte group, for the transposed LDS staging.
  auto v_key = [&](int c, int r, int odd) {
    const int u = lane + kWave * r;
    return min(chunk_key0(c) + 2 * (u >> 3) + odd, last_key);
  };
  auto v_off = [&](int key, int r) {
    const int u = lane + kWave * r;
    return (uint32_t)(key * kKvStride + head * kHeadDim + 8 * (u & 7));
  };
  // With rows written in the launch (Io::kFreshRows): which of the lane's keys are such rows is
  // decided once, before the wait; keys past the cache end load nothing (zeros: their scores are
  // masked below and their P is exactly 0), rather than the clamped last row, which may itself
  // be one of the fresh rows.
  bool fk[CPW][2], fv[CPW][2][2];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint32_t off = k_off(c, blk);
      if constexpr (Io::kFreshRows) {
        const int key = chunk_key0(c) + 16 * blk + r16;
        const bool in = key < n_kv;
        fk[c][blk] = in && io.fresh(key);
        if (in && !fk[c][blk]) {
          kf[c][blk][0] = load16(a.k + off);
          kf[c][blk][1] = load16(a.k + (off + 32));
        } else {
          kf[c][blk][0] = kf[c][blk][1] = z8;
        }
      } else {
        kf[c][blk][0] = load16(a.k + off);
        kf[c][blk][1] = load16(a.k + (off + 32));
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k0 = v_key(c, r, 0), k1 = v_key(c, r, 1);
      if constexpr (Io::kFreshRows) {
        const int u = lane + kWave * r;
        const int key0 = chunk_key0(c) + 2 * (u >> 3);
        const bool in0 = key0 < n_kv, in1 = key0 + 1 < n_kv;
        fv[c][r][0] = in0 && io.fresh(key0);
        fv[c][r][1] = in1 && io.fresh(key0 + 1);
        va[c][r] = in0 && !fv[c][r][0] ? load16(a.v + v_off(k0, r)) : z8;
        vb[c][r] = in1 && !fv[c][r][1] ? load16(a.v + v_off(k1, r)) : z8;
      } else {
        va[c][r] = load16(a.v + v_off(k0, r));
        vb[c][r] = load16(a.v + v_off(k1, r));
      }
    }
  }
  io.wait();
  if constexpr (Io::kFreshRows) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        if (fk[c][blk]) {
          const int key = chunk_key0(c) + 16 * blk + r16;
          kf[c][blk][0] = io.fresh_k(key, head * kHeadDim + 8 * G);
          kf[c][blk][1] = io.fresh_k(key, head * kHeadDim + 8 * G + 32);
        }
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int key0 = chunk_key0(c) + 2 * ((lane + kWave * r) >> 3);
        const int col = head * kHeadDim + 8 * ((lane + kWave * r) & 7);
        if (fv[c][r][0]) va[c][r] = io.fresh_v(key0, col);
        if (fv[c][r][1]) vb[c][r] = io.fresh_v(key0 + 1, col);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
    qf[s] = io.load_q(a.q, (uint32_t)(q_row * a.q_stride + head * kHeadDim + 32 * s + 8 * G));
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
        *reinterpret_cast<f16x2*>(&sm.Vt[wave][c][(8 * c8 + e) * kVtLd + 2 * kp]) = (f16x2){va[c][r][e], vb[c][r][e]};
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
      const f16* row = &sm.Vt[wave][c][(16 * dd + r16) * kVtLd];
      const f16x4 lo = *reinterpret_cast<const f16x4*>(row + 4 * G);
      const f16x4 hi = *reinterpret_cast<const f16x4*>(row + 16 + 4 * G);
      const f16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oa = mfma_16x16x32(vf, pf[c], oa);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.ow[wave][r16][16 * dd + 4 * G + r] = oa[r];
  }
  if (G == 0) {
    sm.mw[wave][r16] = m;
    sm.lw[wave][r16] = l;
  }
  __syncthreads();

  // Merge the NW waves: thread -> (query mq, dims d0 .. d0 + 3); threads past the 16th query
  // (NW > 4) read query 15's values and store nothing.
  const int mq_t = tid >> 4, mq = min(mq_t, kMaxQ - 1), d0 = (tid & 15) * 4;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.mw[w][mq]);
  float L = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = exp2_fast(sm.mw[w][mq] - M);
      L += sm.lw[w][mq] * wt;
      const f32x4 ov = *reinterpret_cast<const f32x4*>(&sm.ow[w][mq][d0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += ov[j] * wt;
    }
  }
  const bool row_ok = mq_t < n_q;
  const float sink2 = a.sinks ? a.sinks[head] * kLog2e : -INFINITY;
  if (n_splits == 1) {
    if (!row_ok) return;
    const float s = apply_sink(M, L, sink2);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] *= s;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const f16x2 lo = pack_rne(acc[0] * inv, acc[1] * inv), hi = pack_rne(acc[2] * inv, acc[3] * inv);
    Io::store_o(a, mq, head, d0, (f16x4){lo[0], lo[1], hi[0], hi[1]});
    return;
  }

  // Partials of this split, then the arrival count.  The partials and the counter are
  // accessed with agent-scope atomics.  Each wave waits until its stores are acknowledged
  // before the workgroup barrier, so they are visible device-wide before thread 0 counts the
  // unit in; the last unit's loads are issued after the count returned.
  // Slot (split s, query mq, head): (m, l) at part_ml[2 slot], o at part_o[64 slot + d0];
  // slot = (s n_q + mq) n_heads + head, all offsets below 2^31 for any valid call.
  const int slot0 = mq * a.n_heads + head, slot_step = n_q * a.n_heads;
  if (row_ok) {
    const int slot = split * slot_step + slot0;
    store_coherent4(a.part_o, (uint32_t)(slot * kHeadDim + d0), (f32x4){acc[0], acc[1], acc[2], acc[3]});
    if (d0 == 0) store_coherent(a.part_ml + (uint32_t)(slot * 2), M, L);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  uint32_t* const counter = &a.counters[head * kCounterStride];
  if (tid == 0)
    sm.last_arrival =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(n_splits - 1);
  __syncthreads();
  if (!sm.last_arrival) return;
  // Every split has arrived: reset the counter for the next call.
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!row_ok) return;
  // Merge the splits MB at a time: every load of a batch is issued before any
  // is used (indices past the last split are clamped and their weights dropped), and
  // the running (M, L, sum) is rescaled to each batch's maximum.
  M = -INFINITY;
  L = 0.0f;
  f32x4 sum = {};
  for (int s0 = 0; s0 < n_splits; s0 += MB) {
    float pm[MB], pl[MB];
    f32x4 po[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int slot = min(s0 + i, n_splits - 1) * slot_step + slot0;
      const f32x2 ml = load_coherent(a.part_ml + (uint32_t)(slot * 2));
      po[i] = load_coherent4(a.part_o, (uint32_t)(slot * kHeadDim + d0));
      pm[i] = ml[0];
      pl[i] = ml[1];
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (s0 + i < n_splits) mb = fmaxf(mb, pm[i]);
    if (mb == -INFINITY) continue;  // no admitted key so far
    const float s = M == -INFINITY ? 0.0f : exp2_fast(M - mb);
    L *= s;
#pragma unroll
    for (int j = 0; j < 4; ++j) sum[j] *= s;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      // 0 for a split with no admitted key (m = -inf) and for indices past the last split.
      const float wt = s0 + i < n_splits ? exp2_fast(pm[i] - mb) : 0.0f;
      L += pl[i] * wt;
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[j] += po[i][j] * wt;
    }
    M = mb;
  }
  const float s = apply_sink(M, L, sink2);
#pragma unroll
  for (int j = 0; j < 4; ++j) sum[j] *= s;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const f16x2 lo = pack_rne(sum[0] * inv, sum[1] * inv), hi = pack_rne(sum[2] * inv, sum[3] * inv);
  Io::store_o(a, mq, head, d0, (f16x4){lo[0], lo[1], hi[0], hi[1]});
}

}  // namespace vcore
}  // namespace edda
