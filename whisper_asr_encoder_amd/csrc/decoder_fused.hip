// Kernel 8: the decoder's verification layer in one launch.
//
// The layer is eight dependent steps, each a few microseconds of latency-bound work on a
// 16-token block (LN1 + QKV + cache append, self-attention, output projection + residual,
// LN2 + cross query, cross-attention, cross output projection + residual, LN3 + fc1 + GELU,
// fc2 + residual).  Run as eight launches, every step pays a launch, a cold start and its
// weights' first round trip after the previous step ended.  Here one launch of persistent
// workgroups takes work items from a single atomic ticket counter, items numbered step by
// step; an item of step p first issues the loads that depend on nothing computed in this
// launch (its weight fragments into registers, the old K/V cache rows, the cross-attention
// K/V), then waits until every item of step p - 1 has set its done flag, then loads its
// activations and finishes.  Workgroups run ahead of the step being computed, so the next
// steps' weights stream in while the current step runs.
//
// Deadlock freedom without co-residency: tickets are handed out in increasing order and an
// item waits only for items of earlier steps, which hold lower tickets and so were all claimed
// by workgroups that are running and that themselves wait only on earlier steps.  The waits
// are bounded (a launch always ends).  Each item, once its stores are acknowledged, sets its
// own done flag (a store; atomics on one line serialise at the memory side, ~12 ns each, and
// polls of that line queue with them); an item's wait reads the flags of the step before.
// The last workgroup to leave clears the ticket, the exit count and the flags, which the
// launch leaves zero as it found them.
//
// Memory ordering across the XCDs' separate L2 caches: everything one step writes and a
// later step reads is stored with agent-scope atomic stores, which write through to the
// device's coherence point, and an item's stores are acknowledged (vmcnt 0) before its
// workgroup barrier and its done flag.  Every workspace buffer is written by one step and read
// only after that step's flags are all set, and no item reads it earlier in the launch; an L2
// cache therefore never holds a stale copy of it (the caches are invalidated at kernel start),
// and consumers read it with plain loads, which miss in their L2 and fetch from the coherence
// point.  The self-attention reads the appended K/V rows from the QKV block, not from the
// cache: with a cache that is only 16-byte aligned, a row's 128-byte line can hold the end of
// a neighbouring old row that another item loaded before its wait.  Loads issued before a wait
// (weights, old cache rows, cross-attention K/V, the layer input) touch nothing this launch
// writes.  Measured and dropped: an agent-scope acquire fence per item with plain loads after
// it (each fence invalidates the whole XCD's L2 under the other workgroups on it: the layer
// ran 55 % slower); release fences (their L2 write-back costs 4-14 us, hence the write-through
// stores); 8-byte device-coherent loads of the activations (2-3x slower than plain 16-byte
// loads).
//
// Work items (the block GEMMs as kernel 6: weights as the MFMA A operand, 8 waves over the
// 32-deep K steps, summed in LDS; a LayerNorm is computed once per item):
//   0  LN1 + QKV + K/V cache append, 64 columns          60 items, x from the layer input
//   1  self-attention, one item per head (<= 512 keys)   20
//   2  output projection + residual x, 32 columns        40
//   3  LN2 + cross query, 32 columns                     40
//   4  cross-attention, 512-key splits x 20 heads        20 * ceil(n_frames / 512)
//   5  cross output projection + residual x1, 32 cols    40
//   6  LN3 + fc1 + GELU, 64 columns                      80
//   7  fc2 (K = 5120) + residual x2, 16 columns          80
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "layer_norm_row.hpp"
#include "verify_core.hpp"

namespace edda {
namespace {

constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;
constexpr int kFCols = 16;
constexpr int kFLnGroups = kDModel / 256;
constexpr int kFALd = kDModel + 8;  // LDS row stride (halves) of the normalised rows
constexpr int kSteps = 8;
// Item sizes (fewer, larger items keep fewer workgroups waiting per step): the QKV GEMM 64
// columns (4 blocks) per item, the 1280-wide projections 32 (2 blocks), fc1 64, fc2 16 over
// the whole K = 5120; cross-attention splits of 512 keys (8 waves of two 32-key chunks).
constexpr int kQkvBlocks = 4, kProjBlocks = 2, kFc1Blocks = 4;
constexpr int kCrossCpw = 2;
constexpr int kCrossKeys = kCrossCpw * 8 * 32;
constexpr int kCrossMergeBatch = 4;  // 1500 frames: 3 splits
constexpr int kMaxStackLayers = kDecoderFusedMaxLayers;
constexpr int kCtlStride = 64;  // uint32 words: the two counters 256 bytes apart
constexpr int kSpinLimit = 1 << 20;  // polls (seconds) before a wait gives up
constexpr int kCoarseSleep = 127;    // s_sleep units of 64 clocks between polls
constexpr int kFineSleep = 8;
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ uint32_t ld32c(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64c(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st32c(void* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float gelu_exact_f(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// The wait of an item of step p: wave 0 reads done flags (64 per load instruction, at most
// kMaxPollLoads per lane) until all are set (bounded), then the workgroup proceeds.  First,
// rarely, those of step p - 2 (an item claimed well ahead of its turn), then more often those
// of step p - 1: every poll is a device-coherent load that competes with the weight and
// activation traffic (measured on the layer: polling every ~0.25 us beat both polling
// continuously and keeping two polls in flight; polling every ~0.5 us or more ran slower).
// Reads only: a flag line is never the target of atomics, which the memory side serialises.
constexpr int kMaxPollLoads = 4;  // flags of up to 256 items per step
template <int kSleep>
__device__ __forceinline__ void poll_flags(const uint32_t* flags, int begin, int end) {
  const int lane = threadIdx.x;
  for (int i = 0; i < kSpinLimit; ++i) {
    bool set = true;
#pragma unroll
    for (int k = 0; k < kMaxPollLoads; ++k) {
      // Unconditional loads (indices past the step clamped to its first flag, their values
      // ignored): one wait for all of them.
      const int j = begin + lane + kWave * k;
      set &= ld32c(&flags[j < end ? j : begin]) != 0u || j >= end;
    }
    if (__all(set)) return;
    __builtin_amdgcn_s_sleep(kSleep);
  }
}
struct StepWait {
  const uint32_t* flags;  // null: no wait (step 0)
  int coarse_begin, coarse_end;  // flag indices of step p - 2 (empty for p < 2)
  int begin, end;                // flag indices of step p - 1
  __device__ void operator()() const {
    if (flags && threadIdx.x < kWave) {
      if (coarse_end > coarse_begin) poll_flags<kCoarseSleep>(flags, coarse_begin, coarse_end);
      poll_flags<kFineSleep>(flags, begin, end);
    }
    __syncthreads();
  }
};

// Every thread's stores acknowledged, then the item's done flag.
__device__ __forceinline__ void publish(uint32_t* flag) {
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0) st32c(flag, 1u);
}

// The pointers of one layer.
struct LayerPtrs {
  // ln1_g, ln1_b, w_qkv, b_qkv, w_o, b_o, ln2_g, ln2_b, w_qc, b_qc, w_oc, b_oc, ln3_g, ln3_b,
  // w_fc1, b_fc1, w_fc2, b_fc2 (weights [out][in] fp16, or Q8_0 codes; biases may be null)
  const f16* w[18];
  const f16* scales[6];  // Q8_0 scales of the six matrices, or null
  f16* k_cache;
  f16* v_cache;
  const f16* cross_k;
  const f16* cross_v;
};

struct FusedArgs {
  const f16* x;  // input of the first layer
  f16* y;        // output of the last layer
  int n_q;
  Slots slots;
  int n_kv;
  const uint32_t* mask;
  int mask_words;
  int n_frames;
  int cross_splits;
  int n_layers;
  // Workspace rows of layer l at lws + l * lws_stride + off_*; off_y: a layer's output (the
  // next layer's input) except the last layer's, which goes to y.
  char* lws;
  size_t lws_stride;
  uint32_t off_qkv, off_o, off_x1, off_qc, off_h, off_x2, off_f, off_y;
  uint32_t* verify_counters;
  float* part_ml;
  float* part_o;
  uint32_t* ctl;  // ticket at ctl[0], exit count at ctl[kCtlStride]
  uint32_t* flags;  // one done flag per item of every layer
  int step_end[kSteps];  // running item totals of one layer
  LayerPtrs layer[kMaxStackLayers];
};

// The operands of one block GEMM: C[M, N] = act(A W^T + bias) + residual.
struct GemmOp {
  const void* w;       // fp16 [N][K], or Q8_0 int8 codes [N][K]
  const f16* scales;   // null, or the Q8_0 scales fp16 [K / 32][N]
  const f16* bias;
  const f16* a;  // [M][K] operand rows, or the LayerNorm's input rows
  const f16* gamma;
  const f16* beta;
  const f16* res;  // [M][N] or null
  f16* c;          // [M][N]
  int N, K;
  bool a_fresh;    // the LayerNorm rows were written in this launch (loaded after the wait)
  bool res_fresh;  // the residual was written in this launch (loaded after the wait)
  f16* k_cache;    // APPEND: the caches whose rows slots[m] receive the K and V columns
  f16* v_cache;
};

constexpr int kMaxBlocks = 4;  // column blocks of one GEMM item
struct GemmSmem {
  float red[kFWaves][kMaxBlocks * kFCols][kFCols + 1];
  alignas(16) f16 a_lds[16 * kFALd];
};

// Fragment order of a [16][K] operand consumed by the block GEMMs: for each 32-deep step s, the
// 64 lanes' 16-byte fragments in lane order (lane 16 g + r holds row r, k = 32 s + 8 g ..
// 8 g + 7), so a consumer's load instruction reads 1 KB contiguous (row-major rows give 16
// separate 64-byte pieces per instruction).  Element (m, k) sits at frag_index(m, k).
__device__ __forceinline__ uint32_t frag_index(int m, int k) {
  return (uint32_t)((((k >> 5) * 4 + ((k >> 3) & 3)) * 16 + m) * 8 + (k & 7));
}

// One block-GEMM item: NB column blocks of 16 (C[:, n0 .. n0 + 16 NB)) over the whole K = 256 NU
// (wave w takes the 32-deep steps w, w + 8, ...).  op.a_fresh / op.res_fresh: the LayerNorm
// rows / the residual were written in this launch and are loaded after the wait (the other
// operands a step reads after its wait always are).  A_FRAG / C_FRAG: A is read, C written, in
// fragment order (C_FRAG: no residual, no append).  Q8: the weights are Q8_0 codes and scales,
// each step's dot products scaled in fp32 as in kernel 6.  Per block the arithmetic is kernel
// 6's (same fragments, same summation order over steps and waves).
template <int NB, int NU, int ACT, bool LN, bool A_FRAG, bool APPEND, bool C_FRAG, bool Q8>
__device__ __forceinline__ void gemm_item(const FusedArgs& fa, const GemmOp& op, int item, const StepWait& wait,
                                          GemmSmem& sm, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int M = fa.n_q, K = op.K, N = op.N;
  const int n0 = item * NB * kFCols;
  // LayerNorm input rows: staged through LDS by all threads, 16-byte chunk t + 512 i of the
  // M x 1280 block each (a wave's load is 1 KB contiguous).  Rows that exist before the launch
  // are loaded ahead of the weights (a wave's loads return in order, so rows queued behind
  // 80 KB of weights would wait for them); gamma and beta (constants) before the wait.
  constexpr int kLnChunks = 16 * kDModel / 8, kLnPerThread = kLnChunks / kFThreads;
  static_assert(kLnChunks % kFThreads == 0, "LayerNorm chunks per thread");
  f16x8 raw[LN ? kLnPerThread : 1];
  f16x4 gam[LN ? kFLnGroups : 1], bet[LN ? kFLnGroups : 1];
  auto ln_chunk = [&](int i) { return (uint32_t)((tid + kFThreads * i) * 8); };  // element index
  if constexpr (LN) {
    if (!op.a_fresh) {
#pragma unroll
      for (int i = 0; i < kLnPerThread; ++i)
        if ((int)ln_chunk(i) < M * kDModel) raw[i] = load16(op.a + ln_chunk(i));
    }
  }
  if constexpr (LN) {
#pragma unroll
    for (int c = 0; c < kFLnGroups; ++c) {
      gam[c] = *reinterpret_cast<const f16x4*>(op.gamma + 4 * (c * kWave + lane));
      bet[c] = *reinterpret_cast<const f16x4*>(op.beta + 4 * (c * kWave + lane));
    }
  }
  // Weight fragments: row n0 + 16 b + r16, 8 consecutive k of each step.
  // Q8: 8 bytes of codes of the same row and k, and the scales of the lane's four output
  // columns n0 + 16 b + 4 g + r at the step.
  using WFrag = std::conditional_t<Q8, u32x2, f16x8>;
  WFrag wf[NB][NU];
  f16x4 wd[Q8 ? NB : 1][Q8 ? NU : 1];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int n = n0 + kFCols * b;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int st = wave + 8 * u;
      if constexpr (Q8) {
        const int8_t* crow = static_cast<const int8_t*>(op.w) + (size_t)(n + r16) * K + 8 * g;
        wf[b][u] = *reinterpret_cast<const u32x2*>(crow + 32 * st);
        wd[b][u] = *reinterpret_cast<const f16x4*>(op.scales + (size_t)st * N + n + 4 * g);
      } else {
        const f16* wrow = static_cast<const f16*>(op.w) + (size_t)(n + r16) * K + 8 * g;
        wf[b][u] = load16(wrow + 32 * st);
      }
    }
  }
  // Epilogue thread: block eb, row em, columns en, en + 1 of the block.
  const int eb = tid >> 7, em = (tid >> 3) & 15, en = 2 * (tid & 7);
  const int ecol = n0 + kFCols * eb + en;
  const bool epi = tid < NB * 128 && em < M;
  f16x2 bias2 = {};
  if (op.bias && epi) bias2 = *reinterpret_cast<const f16x2*>(op.bias + ecol);
  f16x2 res2 = {};
  if (op.res && !op.res_fresh && epi) res2 = *reinterpret_cast<const f16x2*>(op.res + (size_t)em * N + ecol);
  wait();

  const int arow = min(r16, M - 1);
  f16x8 xf[NU];
  if constexpr (LN) {
    if (op.a_fresh) {
#pragma unroll
      for (int i = 0; i < kLnPerThread; ++i)
        if ((int)ln_chunk(i) < M * kDModel) raw[i] = load16(op.a + ln_chunk(i));
    }
#pragma unroll
    for (int i = 0; i < kLnPerThread; ++i) {
      const int e = (int)ln_chunk(i), row = e / kDModel;
      if (e < M * kDModel) *reinterpret_cast<f16x8*>(&sm.a_lds[row * kFALd + e - row * kDModel]) = raw[i];
    }
    __syncthreads();
    // Rows wave and wave + 8, normalised in place (each row belongs to one wave); both rows'
    // statistics interleaved (a row past M is computed from whatever the buffer holds and not
    // stored).
    const int r0 = wave, r1 = wave + kFWaves;
    LnRow<kFLnGroups> row[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < kFLnGroups; ++c) {
        row[h].v[c] = *reinterpret_cast<const f16x4*>(&sm.a_lds[(wave + kFWaves * h) * kFALd + 4 * (c * kWave + lane)]);
        row[h].g[c] = gam[c];
        row[h].b[c] = bet[c];
      }
    layer_norm_finish2<kFLnGroups>(
        row[0], row[1], lane,
        [&](int f, f16x4 v) { if (r0 < M) *reinterpret_cast<f16x4*>(&sm.a_lds[r0 * kFALd + f]) = v; },
        [&](int f, f16x4 v) { if (r1 < M) *reinterpret_cast<f16x4*>(&sm.a_lds[r1 * kFALd + f]) = v; });
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NU; ++u)
      xf[u] = *reinterpret_cast<const f16x8*>(&sm.a_lds[arow * kFALd + 32 * (wave + 8 * u) + 8 * g]);
  } else {
    if constexpr (A_FRAG) {
#pragma unroll
      for (int u = 0; u < NU; ++u) xf[u] = load16(op.a + ((wave + 8 * u) * kWave + lane) * 8);
    } else {
      const uint32_t xrow = (uint32_t)(arow * K + 8 * g);
#pragma unroll
      for (int u = 0; u < NU; ++u)
        xf[u] = load16(op.a + xrow + 32 * (wave + 8 * u));
    }
  }
  if (op.res && op.res_fresh && epi) res2 = *reinterpret_cast<const f16x2*>(op.res + (size_t)em * N + ecol);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    f32x4 acc = {};
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if constexpr (Q8) {
        const f32x4 t = mfma_16x16x32(codes_to_f16(wf[b][u]), xf[u], (f32x4){});
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf((float)wd[b][u][r], t[r], acc[r]);
      } else {
        acc = mfma_16x16x32(wf[b][u], xf[u], acc);
      }
    }
    // acc[r] = C^T[n = 16 b + 4 g + r][m = r16] over this wave's steps.
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.red[wave][kFCols * b + 4 * g + r][r16] = acc[r];
  }
  __syncthreads();
  if (!epi) return;
  float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    v0 += sm.red[w][kFCols * eb + en][em];
    v1 += sm.red[w][kFCols * eb + en + 1][em];
  }
  v0 += (float)bias2[0];
  v1 += (float)bias2[1];
  if constexpr (ACT == 1) {
    v0 = gelu_exact_f(v0);
    v1 = gelu_exact_f(v1);
  }
  v0 += (float)res2[0];
  v1 += (float)res2[1];
  const uint32_t out = __builtin_bit_cast(uint32_t, pack_rne(v0, v1));
  if constexpr (C_FRAG) {
    static_assert(!APPEND, "the appended rows come from a row-major QKV block");
    st32c(op.c + frag_index(em, ecol), out);  // columns ecol, ecol + 1 are adjacent there too
    return;
  }
  st32c(op.c + (size_t)em * N + ecol, out);
  if constexpr (APPEND) {
    const int col = ecol - kDModel;  // 0 .. 1279: K, 1280 .. 2559: V (a pair never straddles)
    if (col >= 0) {
      const size_t row = (size_t)fa.slots.s[em] * kDModel;
      if (col < kDModel) st32c(op.k_cache + row + col, out);
      else st32c(op.v_cache + row + col - kDModel, out);
    }
  }
}

// Memory policies of the attention items (verify_core.hpp).
struct SelfIo {
  static constexpr bool kFreshRows = true;
  const int8_t* fresh_row;  // LDS: block row of each cache slot, -1 for a slot not in the block
  const f16* qkv;           // the block's packed QKV rows: its K and V are the appended rows
  StepWait w;
  __device__ bool fresh(int key) const { return fresh_row[key] >= 0; }
  __device__ void wait() const { w(); }
  __device__ static f16x8 load_q(const f16* base, uint32_t off) { return load16(base + off); }
  // The appended rows read from the QKV block (written once in the launch, read after its
  // flags) rather than from the cache, whose lines may also hold the end of an old row.
  __device__ f16x8 fresh_k(int key, int col) const { return load16(qkv + fresh_row[key] * kQkvCols + kDModel + col); }
  __device__ f16x8 fresh_v(int key, int col) const {
    return load16(qkv + fresh_row[key] * kQkvCols + 2 * kDModel + col);
  }
  __device__ static void store_o(const vcore::Args& a, int mq, int head, int d0, f16x4 v) {
    st64c(a.o + frag_index(mq, head * kHeadDim + d0), __builtin_bit_cast(uint64_t, v));
  }
};
struct CrossIo {
  static constexpr bool kFreshRows = false;
  StepWait w;
  __device__ bool fresh(int) const { return false; }
  __device__ void wait() const { w(); }
  __device__ static f16x8 load_q(const f16* base, uint32_t off) { return load16(base + off); }
  __device__ f16x8 fresh_k(int, int) const { return f16x8{}; }
  __device__ f16x8 fresh_v(int, int) const { return f16x8{}; }
  __device__ static void store_o(const vcore::Args& a, int mq, int head, int d0, f16x4 v) {
    st64c(a.o + frag_index(mq, head * kHeadDim + d0), __builtin_bit_cast(uint64_t, v));
  }
};

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
template <int CPW>
constexpr size_t kArenaBytes =
    cmax(cmax(sizeof(vcore::Smem<CPW, kFWaves>), sizeof(vcore::Smem<kCrossCpw, kFWaves>)), sizeof(GemmSmem));

// SELF_CPW: 32-key chunks per wave of the self-attention (1: n_kv <= 256, 2: <= 512).
// SELF_MODE: vcore::kMaskRows or kMaskNone.  Q8: Q8_0 projection weights.
template <int SELF_CPW, int SELF_MODE, bool Q8>
__global__ __launch_bounds__(kFThreads) void decoder_layer_kernel(FusedArgs fa) {
  __shared__ __attribute__((aligned(16))) unsigned char arena[kArenaBytes<SELF_CPW>];
  __shared__ int8_t fresh_row[2 * kFWaves * vcore::kWaveKeys];
  __shared__ int s_item;
  uint32_t* const ctl = fa.ctl;
  const int per_layer = fa.step_end[kSteps - 1];
  const int total = per_layer * fa.n_layers;
  if (threadIdx.x == 0) s_item = (int)__hip_atomic_fetch_add(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int item = s_item;
  while (item < total) {
    // The thread index laundered once per item: without this the compiler hoists every
    // step's lane-dependent offsets out of the loop and keeps them all live (spills).
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    // The next ticket is claimed now and used after this item: its round trip overlaps the
    // item.  (Holding two tickets keeps the order argument: the next item is of this step or
    // a later one, and this workgroup finishes the current item first.)
    uint32_t next = 0;
    if (tid == 0) next = __hip_atomic_fetch_add(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int layer = item / per_layer, in_layer = item - layer * per_layer;
    int p = 0;
    while (in_layer >= fa.step_end[p]) ++p;
    const int local = in_layer - (p ? fa.step_end[p - 1] : 0);
    // Steps are ordered across layers: global step layer * 8 + p waits for global steps - 1
    // (fine) and - 2 (coarse).
    auto flag_range = [&](int gstep, int& begin, int& end) {
      const int l = gstep / kSteps, q = gstep % kSteps;
      begin = l * per_layer + (q ? fa.step_end[q - 1] : 0);
      end = l * per_layer + fa.step_end[q];
    };
    const int gstep = layer * kSteps + p;
    StepWait wait{gstep >= 1 ? fa.flags : nullptr, 0, 0, 0, 0};
    if (gstep >= 2) flag_range(gstep - 2, wait.coarse_begin, wait.coarse_end);
    if (gstep >= 1) flag_range(gstep - 1, wait.begin, wait.end);
    const LayerPtrs& L = fa.layer[layer];
    char* const wsl = fa.lws + (size_t)layer * fa.lws_stride;
    f16* const qkv = reinterpret_cast<f16*>(wsl + fa.off_qkv);
    f16* const o = reinterpret_cast<f16*>(wsl + fa.off_o);
    f16* const x1 = reinterpret_cast<f16*>(wsl + fa.off_x1);
    f16* const qc = reinterpret_cast<f16*>(wsl + fa.off_qc);
    f16* const h = reinterpret_cast<f16*>(wsl + fa.off_h);
    f16* const x2 = reinterpret_cast<f16*>(wsl + fa.off_x2);
    f16* const f = reinterpret_cast<f16*>(wsl + fa.off_f);
    // The layer's input: the launch's input, or the previous layer's output (written in it).
    const bool x_fresh = layer > 0;
    const f16* const x =
        x_fresh ? reinterpret_cast<const f16*>(fa.lws + (size_t)(layer - 1) * fa.lws_stride + fa.off_y) : fa.x;
    f16* const y = layer == fa.n_layers - 1 ? fa.y : reinterpret_cast<f16*>(wsl + fa.off_y);
    GemmSmem& gs = *reinterpret_cast<GemmSmem*>(arena);
    switch (p) {
      case 0:
        gemm_item<kQkvBlocks, 5, 0, true, false, true, false, Q8>(
            fa, GemmOp{L.w[2], L.scales[0], L.w[3], x, L.w[0], L.w[1], nullptr, qkv, kQkvCols, kDModel, x_fresh, false,
                       L.k_cache, L.v_cache},
            local, wait, gs, tid);
        break;
      case 1: {
        fresh_row[tid] = -1;  // 512 threads, 512 slots
        __syncthreads();
        if (tid < fa.n_q) fresh_row[fa.slots.s[tid]] = (int8_t)tid;
        __syncthreads();
        const vcore::Args a{qkv, kQkvCols, fa.n_q, L.k_cache, L.v_cache, fa.n_kv, kHeads, fa.mask, fa.mask_words,
                            nullptr, o, fa.verify_counters, fa.part_ml, fa.part_o};
        vcore::verify_unit<SELF_MODE, SELF_CPW, kFWaves>(a, 0, local, 1,
                                                         *reinterpret_cast<vcore::Smem<SELF_CPW, kFWaves>*>(arena),
                                                         SelfIo{fresh_row, qkv, wait}, tid);
        break;
      }
      case 2:
        gemm_item<kProjBlocks, 5, 0, false, true, false, false, Q8>(
            fa, GemmOp{L.w[4], L.scales[1], L.w[5], o, nullptr, nullptr, x, x1, kDModel, kDModel, true, x_fresh},
            local, wait, gs, tid);
        break;
      case 3:
        gemm_item<kProjBlocks, 5, 0, true, false, false, false, Q8>(
            fa, GemmOp{L.w[8], L.scales[2], L.w[9], x1, L.w[6], L.w[7], nullptr, qc, kDModel, kDModel, true, false},
            local, wait, gs, tid);
        break;
      case 4: {
        const vcore::Args a{qc, kDModel, fa.n_q, L.cross_k, L.cross_v, fa.n_frames, kHeads, nullptr, 0,
                            nullptr, h, fa.verify_counters, fa.part_ml, fa.part_o};
        vcore::verify_unit<vcore::kMaskNone, kCrossCpw, kFWaves, CrossIo, kCrossMergeBatch>(
            a, local % fa.cross_splits, local / fa.cross_splits, fa.cross_splits,
            *reinterpret_cast<vcore::Smem<kCrossCpw, kFWaves>*>(arena), CrossIo{wait}, tid);
        break;
      }
      case 5:
        gemm_item<kProjBlocks, 5, 0, false, true, false, false, Q8>(
            fa, GemmOp{L.w[10], L.scales[3], L.w[11], h, nullptr, nullptr, x1, x2, kDModel, kDModel, true, true},
            local, wait, gs, tid);
        break;
      case 6:
        gemm_item<kFc1Blocks, 5, 1, true, false, false, true, Q8>(
            fa, GemmOp{L.w[14], L.scales[4], L.w[15], x2, L.w[12], L.w[13], nullptr, f, 4 * kDModel, kDModel, true,
                       false},
            local, wait, gs, tid);
        break;
      default:
        gemm_item<1, 20, 0, false, true, false, false, Q8>(
            fa, GemmOp{L.w[16], L.scales[5], L.w[17], f, nullptr, nullptr, x2, y, kDModel, 4 * kDModel, true, true},
            local, wait, gs, tid);
        break;
    }
    publish(&fa.flags[item]);
    if (tid == 0) s_item = (int)next;
    __syncthreads();
    item = s_item;
  }
  // The last workgroup to leave (every other one has left, so nothing else touches the
  // counters or flags in this launch) clears them for the next launch.
  __shared__ int s_last;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&ctl[kCtlStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  for (int i = threadIdx.x; i < total; i += kFThreads) st32c(&fa.flags[i], 0u);
  if (threadIdx.x == 0) {
    st32c(&ctl[0], 0u);
    st32c(&ctl[kCtlStride], 0u);
  }
}

}  // namespace

int decoder_fused_items(int n_frames) {
  const int cross_splits = (n_frames + kCrossKeys - 1) / kCrossKeys;
  // QKV, self-attention, the three projections, cross-attention, fc1, fc2
  return kQkvCols / (kQkvBlocks * kFCols) + kHeads + 3 * (kDModel / (kProjBlocks * kFCols)) + kHeads * cross_splits +
         4 * kDModel / (kFc1Blocks * kFCols) + kDModel / kFCols;
}

bool decoder_fused_supported(int n_q, int n_kv, int n_frames) {
  const int cross_splits = (n_frames + kCrossKeys - 1) / kCrossKeys;
  return n_q >= 1 && n_q <= 16 && n_kv >= 1 && n_kv <= 2 * kFWaves * vcore::kWaveKeys && n_frames >= 1 &&
         kHeads * cross_splits <= kMaxPollLoads * kWave && decoder_fused_items(n_frames) <= kDecoderFusedMaxItems;
}

hipError_t launch_decoder_layer_fused(const DecoderFusedParams& p, hipStream_t stream) {
  if (!decoder_fused_supported(p.n_q, p.n_kv, p.n_frames) || p.workgroups < 1 || p.n_layers < 1 ||
      p.n_layers > kMaxStackLayers)
    return hipErrorInvalidValue;
  FusedArgs fa{};
  fa.x = static_cast<const f16*>(p.x);
  fa.y = static_cast<f16*>(p.y);
  fa.n_q = p.n_q;
  fa.slots = p.slots;
  fa.n_kv = p.n_kv;
  fa.mask = p.mask;
  fa.mask_words = (p.n_kv + 31) / 32;
  fa.n_frames = p.n_frames;
  fa.cross_splits = (p.n_frames + kCrossKeys - 1) / kCrossKeys;
  fa.n_layers = p.n_layers;
  fa.lws = static_cast<char*>(p.lws);
  fa.lws_stride = p.lws_stride;
  fa.off_qkv = p.off_qkv, fa.off_o = p.off_o, fa.off_x1 = p.off_x1, fa.off_qc = p.off_qc;
  fa.off_h = p.off_h, fa.off_x2 = p.off_x2, fa.off_f = p.off_f, fa.off_y = p.off_y;
  fa.verify_counters = static_cast<uint32_t*>(p.verify_counters);
  fa.part_o = static_cast<float*>(p.part);  // o partials first (16-byte aligned), then (m, l)
  fa.part_ml = fa.part_o + (size_t)fa.cross_splits * p.n_q * kHeads * kHeadDim;
  fa.ctl = static_cast<uint32_t*>(p.ctl);
  fa.flags = static_cast<uint32_t*>(p.flags);
  const bool q8 = p.layer[0].scales[0] != nullptr;
  for (int l = 0; l < p.n_layers; ++l) {
    const DecoderFusedLayer& s = p.layer[l];
    if ((s.scales[0] != nullptr) != q8) return hipErrorInvalidValue;
    LayerPtrs& d = fa.layer[l];
    for (int i = 0; i < 18; ++i) d.w[i] = static_cast<const f16*>(s.w[i]);
    for (int i = 0; i < 6; ++i) d.scales[i] = static_cast<const f16*>(s.scales[i]);
    d.k_cache = static_cast<f16*>(s.k_cache);
    d.v_cache = static_cast<f16*>(s.v_cache);
    d.cross_k = static_cast<const f16*>(s.cross_k);
    d.cross_v = static_cast<const f16*>(s.cross_v);
  }
  const int counts[kSteps] = {kQkvCols / (kQkvBlocks * kFCols), kHeads, kDModel / (kProjBlocks * kFCols),
                              kDModel / (kProjBlocks * kFCols), kHeads * fa.cross_splits,
                              kDModel / (kProjBlocks * kFCols), 4 * kDModel / (kFc1Blocks * kFCols), kDModel / kFCols};
  int run = 0;
  for (int i = 0; i < kSteps; ++i) fa.step_end[i] = (run += counts[i]);
  if (run != decoder_fused_items(p.n_frames)) return hipErrorInvalidValue;
  const dim3 grid(p.workgroups), block(kFThreads);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, 0, stream, fa); };
  const bool rows = p.mask != nullptr;
  const bool one_chunk = p.n_kv <= kFWaves * vcore::kWaveKeys;
  if (q8) {
    if (one_chunk) rows ? go(decoder_layer_kernel<1, vcore::kMaskRows, true>) : go(decoder_layer_kernel<1, vcore::kMaskNone, true>);
    else rows ? go(decoder_layer_kernel<2, vcore::kMaskRows, true>) : go(decoder_layer_kernel<2, vcore::kMaskNone, true>);
  } else {
    if (one_chunk) rows ? go(decoder_layer_kernel<1, vcore::kMaskRows, false>) : go(decoder_layer_kernel<1, vcore::kMaskNone, false>);
    else rows ? go(decoder_layer_kernel<2, vcore::kMaskRows, false>) : go(decoder_layer_kernel<2, vcore::kMaskNone, false>);
  }
  return hipGetLastError();
}

size_t decoder_fused_part_bytes(int n_q, int n_frames) {
  const int cs = (n_frames + kCrossKeys - 1) / kCrossKeys;
  return cs > 1 ? (size_t)cs * n_q * kHeads * (2 + kHeadDim) * sizeof(float) : 0;
}

}  // namespace edda
