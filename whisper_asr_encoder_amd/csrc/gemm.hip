// Kernel 1: fp16 GEMM on gfx950 matrix cores with a fused epilogue, used for the packed
// QKV projection (N = 3840), the attention output projection (N = 1280), the MLP
// (N = 5120 with GELU, N = 1280 with the residual) and the convolutional stem.
//
// C[M, N] = act(A[M, K] * Bt[N, K]^T + bias[N]) + residual[m % period, N].  A
// (activations) and Bt (weights in output-feature-major "Linear" layout) are both
// K-contiguous, so a 16-byte LDS read yields one MFMA operand fragment with no
// transpose.  The MFMA computes C^T tiles (weights as the A operand); fp32
// accumulation, the epilogue in fp32 (act: none or the exact GELU x * Phi(x)), one
// round-to-nearest-even to fp16.
//
// Data movement (one workgroup per BM x BN tile, K step BK = 64): 4 compute waves
// issue the MFMAs and 4 producer waves (one of each per SIMD) the global -> LDS copies.
//  * global -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4) into a ring of
//    STAGES tiles.  A DMA instruction is accepted only as fast as the CU's address
//    unit drains (~16 clk per KB), and a wave waiting to issue one issues nothing
//    else, so the copies and the MFMAs overlap only when different waves issue them.
//    The producers fill all STAGES stages, then per tile k: wait for tile k (vmcnt),
//    join barrier k, and refill the stage of tile k-1 with tile k-1+STAGES (every
//    compute wave finished reading tile k-1 before joining barrier k).  (Joining
//    barrier 0 right after tile 0 measured slower: at kernel start every CU pulls its
//    first tiles at once, and the compute waves then wait at the next barriers.)  They leave
//    after the last barrier of the K loop, with no copy in flight.
//    A DMA instruction writes 1 KB = 8 rows of 128 bytes contiguously, so rows are
//    not padded; instead the eight 16-byte chunks of row r are XOR-permuted with
//    (r >> 1) & 7, which keeps the 16 rows of a fragment read on distinct banks.
//    The DMA is issued from inline asm and waited for with explicit vmcnt counts.
//  * LDS -> registers: the fragments of k16 step s+1 are read while the MFMAs of
//    step s run (one read slotted after each MFMA), double-buffered in VGPRs.
//  * epilogue: bias and residual values are loaded at kernel start in the accumulator
//    layout; the results (fp16) are staged through LDS and written back as full rows
//    with 16-byte stores, instead of 8-byte pieces of 32 rows.  Every residual element
//    a workgroup reads belongs to its own tile and is read before any store, so the
//    residual may be the output buffer itself.
// Workgroups are mapped to tiles XCD-aware: workgroup w runs on XCD w % 8, and each
// XCD gets one rectangular region of the output (the 8 regions chosen to minimise the
// A and B bytes the eight L2s fetch), so operands are fetched once per region.  Rows of A beyond M are fetched from row M-1
// (valid memory) and never stored.
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace edda {
namespace {

constexpr int kBK = 64;             // K elements per tile
constexpr int kRowBytes = kBK * 2;  // 128 bytes per tile row
constexpr int kKSteps = kBK / 16;   // 16-deep MFMA steps per tile
constexpr int kComputeWaves = 4;
constexpr int kProducerWaves = 4;
constexpr int kComputeThreads = kComputeWaves * kWave;
constexpr int kGemmThreads = (kComputeWaves + kProducerWaves) * kWave;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kCus = 256;
constexpr int kSc1 = 16;  // buffer-instruction cache policy bit: device-coherent (sc1)

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS DMA of 16 bytes per lane: lane i's bytes land at LDS byte address
// lds_addr + 16 i (lds_addr wave-uniform, passed in M0).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(g), "s"(lds_addr) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// Wait until at most n DMA instructions of this wave are outstanding, then join the
// workgroup barrier.  One asm statement with a memory clobber, so no LDS access
// moves across it.  No memory fence: a fence would drain every in-flight DMA.
template <int n>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(n) : "memory");
}

// Workgroup barrier with no memory wait (the producers wait for the copies); the
// memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

// f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<N, I + 1>(f);
  }
}

// Compiler-visible wait for every outstanding LDS read of this wave.
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Tile order, computed on the host.  Logical tile t (see the kernel) lies in region r
// when first[r] <= t < first[r+1]; inside region r, M-tile mlo[r] + u % height[r] and
// N-tile nlo[r] + u / height[r] with u = t - first[r], the quotient taken as
// (u * inv[r]) >> 32 with inv[r] = ceil(2^32 / height[r]) (up to 2^32 for height 1;
// exact for u, height < 2^16).
struct TileMap {
  int32_t first[kXcds + 1];
  int32_t mlo[kXcds], nlo[kXcds], height[kXcds];
  uint64_t inv[kXcds];
};

// Fused epilogue: bias [N] or null; residual [*, N] (row m reads row m % res_period) or
// null; act 0 = none, 1 = GELU (applied before the residual).
struct Epilogue {
  const f16* bias;
  const f16* residual;
  int res_period;
  int act;
};

__device__ __forceinline__ float gelu_exact(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// ACT (0 none, 1 GELU) and RES (residual present) are compile-time, so a kernel carries
// only the epilogue code it runs (the GELU is inlined per output element).
template <int BM, int BN, int WM, int WN, int STAGES, int ACT, bool RES>
__global__ __launch_bounds__(kGemmThreads) void gemm_bias_kernel(const f16* __restrict__ A,
                                                                 const f16* __restrict__ Bt,
                                                                 f16* C, int M, int N, int K,
                                                                 TileMap map, Epilogue ep) {
  static_assert(WM * WN == kComputeWaves, "wave grid must use the compute waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert((BM / 8) % kProducerWaves == 0 && (BN / 8) % kProducerWaves == 0,
                "DMA groups must split evenly");
  constexpr int AGW = BM / 8 / kProducerWaves, BGW = BN / 8 / kProducerWaves;
  constexpr int IPW = AGW + BGW;  // DMA instructions per producer wave per tile
  static_assert(IPW * (STAGES - 1) < 64, "vmcnt range");
  constexpr int kStageBytes = (BM + BN) * kRowBytes;
  constexpr int kCld = BN + 8;    // epilogue tile row stride (halves)
  static_assert(BM * kCld * 2 <= STAGES * kStageBytes, "epilogue tile must fit in the ring");
  static_assert(STAGES >= 2, "need at least two stages");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, g = lane >> 5;

  const int nwg = gridDim.x, wid = blockIdx.x;
  const int xcd = wid % kXcds, per = nwg / kXcds, rem = nwg % kXcds;
  // Logical tile index t: the workgroups of one XCD take a contiguous range of t.
  const int t = xcd * per + min(xcd, rem) + wid / kXcds;
  // t enumerates tiles region by region: the output is cut into reg_m x reg_n regions
  // (reg_m * reg_n = 8) of M-tile bands x N-tile bands, M-tile fastest inside a region,
  // so an XCD fetches only its band of A and of B.
  int r = 0;
#pragma unroll
  for (int i = 1; i < kXcds; ++i) r += t >= map.first[i];
  int first = map.first[0], mlo = map.mlo[0], nlo = map.nlo[0], height = map.height[0];
  uint64_t inv = map.inv[0];
#pragma unroll
  for (int i = 1; i < kXcds; ++i)
    if (r == i) first = map.first[i], mlo = map.mlo[i], nlo = map.nlo[i], height = map.height[i], inv = map.inv[i];
  const uint32_t u = (uint32_t)(t - first);
  const int q = (int)(((uint64_t)u * inv) >> 32);  // u < 2^16, inv <= 2^32: no overflow
  const int mi = mlo + (int)u - q * height;
  const int ni = nlo + q;
  const int m0 = mi * BM;
  const int n0 = ni * BN;
  const int nk = K / kBK;

  // DMA sources: lane i of an 8-row group fetches row group*8 + i/8, physical chunk i%8,
  // i.e. logical chunk (i%8) ^ swz(row).
  if (wave >= kComputeWaves) {
    // Producer wave pw: DMA groups pw * AGW .. of A and pw * BGW .. of B.  Lane i of an
    // 8-row group fetches row group*8 + i/8, physical chunk i%8, i.e. logical chunk
    // (i%8) ^ swz(row).
    const int pw = wave - kComputeWaves;
    const int dr = lane >> 3, dpc = lane & 7;
    const f16* a_src[AGW];
    const f16* b_src[BGW];
#pragma unroll
    for (int j = 0; j < AGW; ++j) {
      const int row = (pw * AGW + j) * 8 + dr;
      a_src[j] = A + (size_t)min(m0 + row, M - 1) * K + (dpc ^ swz(row)) * 8;
    }
#pragma unroll
    for (int j = 0; j < BGW; ++j) {
      const int row = (pw * BGW + j) * 8 + dr;
      b_src[j] = Bt + (size_t)(n0 + row) * K + (dpc ^ swz(row)) * 8;
    }
    const uint32_t smem_addr = __builtin_amdgcn_readfirstlane(lds_address(smem));
    auto issue = [&](int kt) {
      const uint32_t st = smem_addr + (kt % STAGES) * kStageBytes;
      const int k0 = kt * kBK;
#pragma unroll
      for (int j = 0; j < AGW; ++j) dma16(a_src[j] + k0, st + (pw * AGW + j) * 1024);
#pragma unroll
      for (int j = 0; j < BGW; ++j) dma16(b_src[j] + k0, st + BM * kRowBytes + (pw * BGW + j) * 1024);
    };
    // Wait until tile j has landed, with `after` (< STAGES) later tiles still allowed in
    // flight, then join barrier j.
    auto wait_tile = [&](int after) {
      static_for<STAGES>([&](auto c) {
        constexpr int n = decltype(c)::value;
        if (after == n) wait_vmcnt_barrier<IPW * n>();
      });
    };
#pragma unroll
    for (int p = 0; p < STAGES; ++p)
      if (p < nk) issue(p);
    wait_tile(min(STAGES, nk) - 1);  // barrier 0
    for (int j = 1; j < nk; ++j) {
      // Tiles issued so far: 0 .. min(j - 2 + STAGES, nk - 1).
      wait_tile(min(STAGES - 2, nk - 1 - j));  // barrier j
      if (j - 1 + STAGES < nk) issue(j - 1 + STAGES);
    }
    return;
  }

  // Fragment byte offsets inside a stage: row l32 (+ multiples of 32), chunk (2s+g) ^ swz(row).
  int frag_off[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) frag_off[s] = l32 * kRowBytes + (((2 * s + g) ^ swz(l32)) << 4);

  // Bias values of this lane's output columns, loaded now so the epilogue does not wait.
  // One uniform branch around each group of loads, so they are in flight together.
  f16x4 bias_v[FN][4];
  if (ep.bias) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bias_v[fn][i] = *reinterpret_cast<const f16x4*>(ep.bias + n0 + wn * WTN + 32 * fn + 8 * i + 4 * g);
  } else {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) bias_v[fn][i] = (f16x4){};
  }
  // Residual values of this lane's outputs (row m0 + wm*WTM + 32 fm + l32, 4 columns);
  // rows past M read row M-1 and are never stored.
  f16x4 res_v[FN][4][FM];
  if constexpr (RES) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = min(m0 + wm * WTM + 32 * fm + l32, M - 1) % ep.res_period;
      const f16* rrow = ep.residual + (size_t)m * N + n0 + wn * WTN + 4 * g;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) res_v[fn][i][fm] = *reinterpret_cast<const f16x4*>(rrow + 32 * fn + 8 * i);
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) res_v[fn][i][fm] = (f16x4){};
  }

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = (f32x16){};

  f16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](int kt, int s, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    const char* sa = smem + (kt % STAGES) * kStageBytes + wm * WTM * kRowBytes;
    const char* sb = smem + (kt % STAGES) * kStageBytes + BM * kRowBytes + wn * WTN * kRowBytes;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      fa[set][fm] = *reinterpret_cast<const f16x8*>(sa + fm * 32 * kRowBytes + frag_off[s]);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      fb[set][fn] = *reinterpret_cast<const f16x8*>(sb + fn * 32 * kRowBytes + frag_off[s]);
  };
  auto mfmas = [&](auto set_c) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_32x32x16(fb[set][fn], fa[set][fm], acc[fn][fm]);
  };
  // Slot one LDS read after each MFMA (then the remaining MFMAs).
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < FM + FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = FM + FN; i < FM * FN; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  static_assert(kKSteps == 4, "the step schedule below assumes four k16 steps per tile");

  // Steps 0..2 of tile kt: read step s+1 while the MFMAs of step s run.
  auto first_steps = [&](int kt) {
    __builtin_amdgcn_sched_barrier(0);
    read_frags(kt, 1, S1());
    mfmas(S0());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(kt, 2, S0());
    mfmas(S1());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(kt, 3, S1());
    mfmas(S0());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };

  plain_barrier();  // barrier 0: tile 0 has landed
  read_frags(0, 0, S0());
  for (int kt = 0; kt + 1 < nk; ++kt) {
    first_steps(kt);
    // Tile kt is fully read once its last fragments are in registers: barrier kt+1
    // publishes that (the producers then refill its stage) and, on the producers' side,
    // that tile kt+1 has landed; step 0 of tile kt+1 is read during the last MFMAs of
    // tile kt.
    wait_lds_reads();
    plain_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(kt + 1, 0, S0());
    mfmas(S1());
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  }
  first_steps(nk - 1);
  mfmas(S1());

  // Epilogue: bias, activation, residual, fp16; stage the tile in LDS, then coalesced
  // 16-byte row stores.
  // Only the compute waves are left (the producers ended after the K loop, which a
  // workgroup barrier no longer waits for).
  wait_lds_reads();
  __syncthreads();  // every compute wave is done reading the ring
  f16* cs = reinterpret_cast<f16*>(smem);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nl = wn * WTN + 32 * fn + 8 * i + 4 * g;  // tile-local column
      const f16x4 bb = bias_v[fn][i];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int ml = wm * WTM + 32 * fm + l32;
        const f16x4 rr = res_v[fn][i][fm];
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = acc[fn][fm][4 * i + j] + (float)bb[j];
          if constexpr (ACT == 1) v[j] = gelu_exact(v[j]);
          if constexpr (RES) v[j] += (float)rr[j];
        }
        const f16x2 lo = pack_rne(v[0], v[1]);
        const f16x2 hi = pack_rne(v[2], v[3]);
        *reinterpret_cast<f16x4*>(cs + ml * kCld + nl) = (f16x4){lo[0], lo[1], hi[0], hi[1]};
      }
    }
  }
  __syncthreads();
  // Row stores with the device-coherent policy (sc1): the lines are written through to
  // memory as the tile finishes, while other tiles still compute, instead of staying dirty in
  // the XCD's L2 until the write-back at the end of the kernel, which nothing overlaps.
  // Offsets are taken from the tile's origin (wave-uniform), so they stay small.
  constexpr int kChunksPerRow = BN / 8;
  constexpr int kChunks = BM * kChunksPerRow;
  const __amdgpu_buffer_rsrc_t c_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(C + (size_t)m0 * N + n0, (short)0, 0x7fffffff, 0x00020000);
#pragma unroll 4
  for (int c = tid; c < kChunks; c += kComputeThreads) {
    const int ml = c / kChunksPerRow, cc = c % kChunksPerRow;
    if (m0 + ml < M)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, load16(cs + ml * kCld + cc * 8)), c_rsrc,
                                             2 * (ml * N + cc * 8), 0, kSc1);
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int ACT, bool RES>
hipError_t launch_tile(const void* A, const void* Bt, void* C, int M, int N, int K, const Epilogue& ep,
                       hipStream_t stream) {
  const int mt = (M + BM - 1) / BM, nt = N / BN;
  // XCD regions: reg_m x reg_n = 8 minimising the operand bytes fetched into the eight L2s,
  // reg_n * |A| + reg_m * |B|  (proportional to reg_n * M + reg_m * N); bands must be non-empty.
  int reg_m = 1, reg_n = 1;
  long best = -1;
  for (int a = 1; a <= kXcds; a *= 2) {
    const int b = kXcds / a;
    if (a > mt || b > nt) continue;
    const long cost = (long)b * M + (long)a * N;
    if (best < 0 || cost < best) best = cost, reg_m = a, reg_n = b;
  }
  // Region r = i * reg_n + j covers M-tile band i and N-tile band j.  Regions beyond
  // reg_m * reg_n (fewer than 8 when a band would be empty) get empty ranges.
  TileMap map{};
  int acc = 0;
  for (int r = 0; r < kXcds; ++r) {
    map.first[r] = acc;
    if (r < reg_m * reg_n) {
      const int i = r / reg_n, j = r % reg_n;
      const int mlo = mt * i / reg_m, mhi = mt * (i + 1) / reg_m;
      const int nlo = nt * j / reg_n, nhi = nt * (j + 1) / reg_n;
      map.mlo[r] = mlo, map.nlo[r] = nlo, map.height[r] = mhi - mlo;
      map.inv[r] = (((uint64_t)1 << 32) + (mhi - mlo) - 1) / (uint64_t)(mhi - mlo);
      acc += (mhi - mlo) * (nhi - nlo);
    } else {
      map.mlo[r] = map.nlo[r] = 0, map.height[r] = 1, map.inv[r] = (uint64_t)1 << 32;
    }
  }
  map.first[kXcds] = acc;
  if ((long)mt * nt >= 65536) return hipErrorInvalidValue;  // the quotient trick needs u < 2^16
  dim3 grid(nt * mt);
  hipLaunchKernelGGL((gemm_bias_kernel<BM, BN, WM, WN, STAGES, ACT, RES>), grid, dim3(kGemmThreads), 0, stream,
                     static_cast<const f16*>(A), static_cast<const f16*>(Bt), static_cast<f16*>(C), M, N,
                     K, map, ep);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int STAGES>
struct Tile {
  template <int ACT, bool RES>
  static hipError_t run(const void* A, const void* Bt, void* C, int M, int N, int K, const Epilogue& ep,
                        hipStream_t stream) {
    if constexpr (BN == 256 && RES) {
      return hipErrorInvalidValue;  // never selected (see launch_gemm)
    } else {
      return launch_tile<BM, BN, WM, WN, STAGES, ACT, RES>(A, Bt, C, M, N, K, ep, stream);
    }
  }
};

}  // namespace

hipError_t launch_gemm(const void* A, const void* Bt, const void* bias, const void* residual, int res_period,
                       int act, void* C, int M, int N, int K, hipStream_t stream) {
  if (M <= 16 && K % 32 == 0 && N % 16 == 0)  // the decoder's block rows: weight streaming
    return launch_skinny_gemm(A, Bt, bias, residual, residual ? res_period : 1, act, C, M, N, K, stream);
  const Epilogue ep{static_cast<const f16*>(bias), static_cast<const f16*>(residual),
                    residual ? res_period : 1, act};
  auto with_epilogue = [&](auto tile) {
    using T = decltype(tile);
    if (act == 1)
      return residual ? T::template run<1, true>(A, Bt, C, M, N, K, ep, stream)
                      : T::template run<1, false>(A, Bt, C, M, N, K, ep, stream);
    return residual ? T::template run<0, true>(A, Bt, C, M, N, K, ep, stream)
                    : T::template run<0, false>(A, Bt, C, M, N, K, ep, stream);
  };
  // Tile width by a cost model of one launch: rounds of tiles over the CUs times the
  // cost of a K step, the larger of its copy time (operand bytes at ~38 B/clk per CU,
  // measured) and its MFMA time (4096 FLOP/clk per CU).  The 256-wide tile has no
  // register room for the residual values.
  const int bns[] = {256, 192, 128, 64};
  int best = 64;
  double best_cost = -1.0;
  for (int bn : bns) {
    if (N % bn || (bn == 256 && residual)) continue;
    const long tiles = (long)((M + 127) / 128) * (N / bn);
    const double step = fmax((128.0 + bn) * 128.0 / 38.0, 128.0 * bn * 128.0 / 4096.0);
    const double cost = (double)((tiles + kCus - 1) / kCus) * step;
    if (best_cost < 0 || cost < best_cost) best_cost = cost, best = bn;
  }
  // Ring depth per tile, measured: the stages in flight on one XCD's 30 CUs must leave its
  // 4 MB L2 room (128 x 192: 3 stages of 40 KB beat 4 by 2-9 %, 128 x 64: 4 of 24 KB beat 6
  // by 10-23 %, the deeper the K the more).
  switch (best) {
    case 256: return with_epilogue(Tile<128, 256, 2, 2, 3>());
    case 192: return with_epilogue(Tile<128, 192, 2, 2, 3>());
    case 128: return with_epilogue(Tile<128, 128, 2, 2, 3>());
    default: return with_epilogue(Tile<128, 64, 2, 2, 4>());
  }
}

hipError_t launch_gemm_bias(const void* A, const void* Bt, const void* bias, void* C, int M, int N,
                            int K, hipStream_t stream) {
  return launch_gemm(A, Bt, bias, nullptr, 1, 0, C, M, N, K, stream);
}

}  // namespace edda
