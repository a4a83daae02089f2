// Kernel 3: block-verification attention.  n_q <= 16 query tokens (anchor plus
// drafted tokens, or one token per beam) attend to a KV cache [n_kv, 20, 64]
// whose slot j holds position j, under per-query bitset mask rows (causal,
// token-tree ancestors, or none for cross-attention).
//
// The work is memory bound (each K/V byte is used by at most 16 queries), so
// the key sequence is split across workgroups: workgroup (split, head) covers
// kSplitKeys keys, each of its 4 waves 32 of them.  Per wave, on 16x16x32
// MFMAs: S^T = K Q^T (lane l holds 8 scores of query l % 16), masked online
// softmax statistics via cross-lane max/sum, then O^T = V^T P^T with P kept in
// registers as the B operand and V^T staged through a wave-private LDS tile.
// The 4 waves merge in LDS; with more than one split, fp32 partials
// (m, l, unnormalized o) go to the workspace and a second kernel merges them:
//   m = max_s m_s,  l = sum_s l_s 2^(m_s - m),  O = sum_s o_s 2^(m_s - m) / l.
// A query with no admitted key gets O = 0.
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace edda {
namespace {

constexpr int kVWaves = 4;
constexpr int kVThreads = kVWaves * kWave;
constexpr int kWaveKeys = 32;
constexpr int kSplitKeys = kVWaves * kWaveKeys;
constexpr int kMaxQ = 16;
constexpr int kVtLd = kWaveKeys + 4;  // V^T row stride (halves): 72 B, 8-byte aligned

__global__ __launch_bounds__(kVThreads) void verify_split_kernel(
    const f16* __restrict__ q, int n_q, const f16* __restrict__ k, const f16* __restrict__ v,
    int n_kv, const uint32_t* __restrict__ mask, int mask_words, f16* __restrict__ o,
    float* __restrict__ part_ml, float* __restrict__ part_o, int n_splits) {
  __shared__ __attribute__((aligned(16))) f16 Vt[kVWaves][kHeadDim * kVtLd];
  __shared__ float mw[kVWaves][kMaxQ], lw[kVWaves][kMaxQ];
  __shared__ float ow[kVWaves][kMaxQ][kHeadDim + 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, G = lane >> 4;
  const int split = blockIdx.x, head = blockIdx.y;
  const int key0 = split * kSplitKeys + wave * kWaveKeys;  // multiple of 32
  const size_t kv_stride = (size_t)kHeads * kHeadDim;
  const f16x8 z8 = {};

  // Q^T fragments: lane holds Q[r16][head][32 s + 8 G .. +7].
  const bool q_ok = r16 < n_q;
  f16x8 qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    qf[s] = q_ok ? load16(q + ((size_t)r16 * kHeads + head) * kHeadDim + 32 * s + 8 * G) : z8;

  // Stage this wave's V tile transposed: Vt[d][key - key0]; key pairs share a 32-bit word.
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int u = lane + kWave * r;
    const int kp = u >> 3, c = u & 7;
    const int key = key0 + 2 * kp;
    const f16x8 a = key < n_kv ? load16(v + key * kv_stride + head * kHeadDim + 8 * c) : z8;
    const f16x8 b = key + 1 < n_kv ? load16(v + (key + 1) * kv_stride + head * kHeadDim + 8 * c) : z8;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<f16x2*>(&Vt[wave][(8 * c + e) * kVtLd + 2 * kp]) = (f16x2){a[e], b[e]};
  }

  // S^T for keys key0 + 16 blk + 4 G + r, query r16.
  f32x4 sacc[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int key = key0 + 16 * blk + r16;
    const f16* kp = k + key * kv_stride + head * kHeadDim + 8 * G;
    const f16x8 k0 = key < n_kv ? load16(kp) : z8;
    const f16x8 k1 = key < n_kv ? load16(kp + 32) : z8;
    sacc[blk] = mfma_16x16x32(k0, qf[0], (f32x4){});
    sacc[blk] = mfma_16x16x32(k1, qf[1], sacc[blk]);
  }
  uint32_t bits = 0;
  if (q_ok && key0 < n_kv) bits = mask ? mask[(size_t)r16 * mask_words + (key0 >> 5)] : 0xffffffffu;
  const float c_scale = kLog2e / 8.0f;
  float sc[8];
  float m = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = 16 * blk + 4 * G + r;
      const bool ok = ((bits >> kk) & 1u) && (key0 + kk < n_kv);
      const float s = ok ? sacc[blk][r] * c_scale : -INFINITY;
      sc[4 * blk + r] = s;
      m = fmaxf(m, s);
    }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  float l = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = (m == -INFINITY) ? 0.0f : exp2_fast(sc[i] - m);
    sc[i] = p;
    l += p;
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  __syncthreads();  // V^T tiles visible to every lane
  const f16x8 pf = pack8(sc[0], sc[1], sc[2], sc[3], sc[4], sc[5], sc[6], sc[7]);
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    const f16* row = &Vt[wave][(16 * dd + r16) * kVtLd];
    const f16x4 lo = *reinterpret_cast<const f16x4*>(row + 4 * G);
    const f16x4 hi = *reinterpret_cast<const f16x4*>(row + 16 + 4 * G);
    const f16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const f32x4 oa = mfma_16x16x32(vf, pf, (f32x4){});
#pragma unroll
    for (int r = 0; r < 4; ++r) ow[wave][r16][16 * dd + 4 * G + r] = oa[r];
  }
  if (G == 0) {
    mw[wave][r16] = m;
    lw[wave][r16] = l;
  }
  __syncthreads();

  // Merge the 4 waves: thread -> (query, 4 consecutive dims).
  const int mq = tid >> 4, d0 = (tid & 15) * 4;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kVWaves; ++w) M = fmaxf(M, mw[w][mq]);
  float L = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) {
      const float wt = exp2_fast(mw[w][mq] - M);
      L += lw[w][mq] * wt;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += ow[w][mq][d0 + j] * wt;
    }
  }
  if (mq >= n_q) return;
  if (n_splits == 1) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const f16x2 lo = pack_rne(acc[0] * inv, acc[1] * inv), hi = pack_rne(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<f16x4*>(o + ((size_t)mq * kHeads + head) * kHeadDim + d0) =
        (f16x4){lo[0], lo[1], hi[0], hi[1]};
  } else {
    const size_t slot = ((size_t)split * n_q + mq) * kHeads + head;
    *reinterpret_cast<f32x4*>(part_o + slot * kHeadDim + d0) = (f32x4){acc[0], acc[1], acc[2], acc[3]};
    if (d0 == 0) *reinterpret_cast<f32x2*>(part_ml + slot * 2) = (f32x2){M, L};
  }
}

// grid (n_q, 20 heads), 64 threads: lane -> one output dimension.
__global__ __launch_bounds__(kWave) void verify_merge_kernel(const float* __restrict__ part_ml,
                                                             const float* __restrict__ part_o,
                                                             int n_splits, int n_q,
                                                             f16* __restrict__ o) {
  const int qi = blockIdx.x, head = blockIdx.y, d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s)
    M = fmaxf(M, part_ml[(((size_t)s * n_q + qi) * kHeads + head) * 2]);
  float L = 0.0f, acc = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const size_t slot = ((size_t)s * n_q + qi) * kHeads + head;
      const float wt = exp2_fast(part_ml[slot * 2] - M);
      L += part_ml[slot * 2 + 1] * wt;
      acc += part_o[slot * kHeadDim + d] * wt;
    }
  }
  o[((size_t)qi * kHeads + head) * kHeadDim + d] = (f16)(L > 0.0f ? acc / L : 0.0f);
}

}  // namespace

int verify_num_splits(int n_kv) { return (n_kv + kSplitKeys - 1) / kSplitKeys; }

size_t verify_workspace_bytes(int n_q, int n_kv) {
  const int s = verify_num_splits(n_kv);
  if (s <= 1) return 0;
  return (size_t)s * n_q * kHeads * (2 + kHeadDim) * sizeof(float);
}

hipError_t launch_verify(const void* q, int n_q, const void* k, const void* v, int n_kv,
                         const uint32_t* mask, void* o, void* workspace, hipStream_t stream) {
  const int n_splits = verify_num_splits(n_kv);
  float* part_ml = nullptr;
  float* part_o = nullptr;
  if (n_splits > 1) {
    part_ml = static_cast<float*>(workspace);
    part_o = part_ml + (size_t)n_splits * n_q * kHeads * 2;
  }
  const int mask_words = (n_kv + 31) / 32;
  hipLaunchKernelGGL(verify_split_kernel, dim3(n_splits, kHeads), dim3(kVThreads), 0, stream,
                     static_cast<const f16*>(q), n_q, static_cast<const f16*>(k),
                     static_cast<const f16*>(v), n_kv, mask, mask_words, static_cast<f16*>(o),
                     part_ml, part_o, n_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  hipLaunchKernelGGL(verify_merge_kernel, dim3(n_q, kHeads), dim3(kWave), 0, stream, part_ml, part_o,
                     n_splits, n_q, static_cast<f16*>(o));
  return hipGetLastError();
}

}  // namespace edda
