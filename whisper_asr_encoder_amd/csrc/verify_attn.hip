// Kernel 3: block-verification attention (the unit's arithmetic: verify_core.hpp).
//
// The work is memory bound (each K/V byte is used by at most 16 queries) and small
// (a few MB per call), so the time is latency: the key sequence is split across
// many workgroups, one launch covers the call, and every load a wave needs is
// issued at kernel start.  A cache of at most 512 keys takes one workgroup per head: 4
// waves of up to three 32-key chunks (384 keys), else 8 waves of two; a longer one is split
// into 128-key ranges, one workgroup (split, head) each, 32 keys per wave, merged in the same
// launch by the last workgroup of each head to arrive.
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "verify_core.hpp"
#include "../../include/edda.h"

namespace edda {
namespace {

using namespace vcore;

constexpr int kVWaves = 4;
constexpr int kVThreads = kVWaves * kWave;
constexpr int kChunk4 = kVWaves * kWaveKeys;  // keys of 4 waves x one 32-key chunk
// Caches longer than kOneWorkgroupKeys: splits of kSplitWaves waves x kSplitCpw chunks.
constexpr int kSplitWaves = 4, kSplitCpw = 1;
constexpr int kSplitKeys = kSplitWaves * kSplitCpw * kWaveKeys;
// Per-head arrival counters at the workspace start, one per 256-byte line.
constexpr int kMaxHeads = 64;
constexpr size_t kCounterBytes = (size_t)kMaxHeads * kCounterStride * sizeof(uint32_t);
static_assert(kCounterBytes == EDDA_VERIFY_COUNTER_BYTES, "counter region size in the public header");

// grid (n_splits, n_heads): one unit per workgroup (verify_core.hpp).
// NW waves (4 or 8) of CPW 32-key chunks each: one split of up to 512 keys (4 waves of up to
// 3 chunks up to 384 keys, else 8 waves of 2 chunks), or 128-key splits of 4 waves of one chunk.
template <int kMode, int CPW, int NW>
__global__ __launch_bounds__(NW * kWave) void verify_kernel(Args a) {
  __shared__ Smem<CPW, NW> sm;
  verify_unit<kMode, CPW, NW>(a, blockIdx.x, blockIdx.y, gridDim.x, sm, PlainIo{}, (int)threadIdx.x);
}

constexpr int kOneWorkgroupKeys = 4 * kChunk4;  // up to 512 keys: one workgroup per head

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
    // o partials first (16-byte aligned for the merge's 16-byte loads), then (m, l).
    part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    part_ml = part_o + (size_t)n_splits * n_q * n_heads * kHeadDim;
  }
  const dim3 grid(n_splits, n_heads);
  int threads = kVThreads;
  auto go = [&](auto kernel) {
    const Args a{static_cast<const f16*>(q), q_stride, n_q, static_cast<const f16*>(k), static_cast<const f16*>(v),
                 n_kv, n_heads, mask, mask_words, sinks, static_cast<f16*>(o), counters, part_ml, part_o};
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, a);
    return hipGetLastError();
  };
  // One split: 4 waves of 1-3 chunks up to 384 keys, else 8 waves of 2 (measured: at 360
  // keys 4 waves of 3 chunks beat 8 of 2 by 7 %, at 448 keys 8 of 2 beat 4 of 4 by 12 %).
  auto by_chunks = [&](auto mode_c) {
    constexpr int M = decltype(mode_c)::value;
    if (n_splits > 1) {
      threads = kSplitWaves * kWave;
      return go(verify_kernel<M, kSplitCpw, kSplitWaves>);
    }
    if (n_kv > 3 * kChunk4) {
      threads = 8 * kWave;
      return go(verify_kernel<M, 2, 8>);
    }
    if (n_kv > 2 * kChunk4) return go(verify_kernel<M, 3, kVWaves>);
    if (n_kv > kChunk4) return go(verify_kernel<M, 2, kVWaves>);
    return go(verify_kernel<M, 1, kVWaves>);
  };
  if (mask_mode == kMaskRows) return by_chunks(std::integral_constant<int, kMaskRows>());
  if (mask_mode == kMaskCausal) return by_chunks(std::integral_constant<int, kMaskCausal>());
  return by_chunks(std::integral_constant<int, kMaskNone>());
}

}  // namespace edda
