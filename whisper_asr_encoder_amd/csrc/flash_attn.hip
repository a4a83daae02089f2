// Kernel 2: flash attention for the encoder (fp16 Q/K/V, fp32 softmax statistics
// and accumulation); scores never leave registers.
//
// Work unit.  One workgroup per (window, chunk segment, 128 query rows, head).
// With chunk_len = c > 0 each chunk of a window is an independent segment whose
// rows admit keys [seg0, min(seg0 + c, valid)); with c = 0 the segment is the
// whole window and its key interval is [0, valid).  Masking is therefore one key
// interval per workgroup: only the tail of that interval is masked elementwise.
//
// Workgroup = 8 waves = 2 query groups (64 rows each) x 4 key quarters.  Keys are
// consumed in iterations of 128: quarter j takes keys [32 j, 32 j + 32) of each
// iteration, so each wave sees a quarter of the keys and the four partial results
// of a query group are merged through LDS at the end.  Two waves share every K/V
// tile (one per query group), and each wave runs two 32-row query blocks against
// each K/V fragment, halving LDS reads per MFMA.
//
// Per wave and 32-key tile, on 32x32x16 MFMAs:
//   S^T = K Q^T   K fragments from LDS, Q^T fragments resident in registers; lane l
//                 holds 16 scores of query l % 32 (per query block), so row
//                 statistics need per-lane work plus one exchange with lane l ^ 32.
//                 Q is held pre-scaled by log2(e)/8 and the MFMA accumulator starts
//                 at -m, so the MFMA itself yields the exponent S log2(e)/8 - m.
//   P = 2^(S log2(e)/8 - m)  with m a per-row reference: the row maximum of the
//                 wave's first tile.  Later tiles reuse it; when a tile's sum of P
//                 reaches 2^14 (a P value might approach the fp16 range) the tile
//                 is recomputed against the new maximum and the running sums are
//                 rescaled, so the result is exact softmax either way.
//   l += sum P    in fp32 adds (v_dot2 shares the matrix pipeline, so it would
//                 serialise against the other query group's MFMAs).
//   O^T += V^T P^T  fp16 P is already laid out as the B operand (the MFMA's k index
//                 is permuted identically on both operands); V^T fragments are read
//                 with ds_read_b64_tr_b16 from the row-major V tile.
// K and V tiles reach LDS by direct-to-LDS DMA (natural row layout, 16-byte chunks
// XOR-swizzled per row) through a 4-stage ring; the workgroup's Q rows arrive the same way
// once, ahead of the first tiles, instead of each wave loading its rows from memory (four
// waves share every query row, and the start of the kernel is bound by that first burst).
// A wave raises its issue priority for its MFMA phase, so its matrix instructions go out
// ahead of the partner wave's softmax arithmetic on the same SIMD.
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace edda {
namespace {

constexpr int kKT = 32;                 // keys per tile (one quarter of an iteration)
constexpr int kQuarters = 4;
constexpr int kQGroups = 2;
constexpr int kQW = 64;                 // query rows per wave
constexpr int kBMq = kQGroups * kQW;    // 128 query rows per workgroup
constexpr int kIterKeys = kQuarters * kKT;
constexpr int kWaves = kQGroups * kQuarters;
constexpr int kThreads = kWaves * kWave;
constexpr int kStages = 4;  // tile i is live for four barrier slots (see the schedule below)
constexpr int kRowB = kHeadDim * 2;     // 128 bytes per K/V row
constexpr int kTileB = kKT * kRowB;     // 4 KB
constexpr int kStageB = kQuarters * 2 * kTileB;  // K and V tiles of every quarter: 32 KB
constexpr int kXcds = 8;
constexpr int kMaxBatchPerLaunch = 256;
constexpr float kRedoSum = 16384.0f;    // per-tile sum of P that triggers a re-reference
constexpr int kOutLd = kHeadDim + 8;    // LDS row stride (halves) of the finished output block
constexpr int kSc1 = 16;                // buffer-instruction cache policy bit: device-coherent (sc1)
constexpr float kQScale = 0.18033688011112042f;  // log2(e) / sqrt(64)

struct ValidLens {
  int32_t v[kMaxBatchPerLaunch];
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(g), "s"(lds_addr) : "m0");
}
// Wait for this wave's DMA down to n outstanding instructions, then the workgroup
// barrier.  The scheduling barriers keep every instruction (arithmetic included) on its
// side, so the work of a barrier slot stays in that slot.
template <int n>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(n) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// 16-byte chunk swizzle of a 128-byte row: h = (row >> 1) & 7 rotated right by one bit.
// Rows 2m and 2m+1 fall in opposite bank halves, so K fragment reads (one row per lane)
// need h bijective over 8 rows; transposed V reads touch rows 4m..4m+3 at once, so rows
// 4m and 4m+2 must differ above bit 0 of the swizzle, which the rotation gives.
__device__ __forceinline__ int swz(int row) {
  const int h = (row >> 1) & 7;
  return ((h & 1) << 2) | (h >> 1);
}

// Byte offset of element (row, col) in a swizzled 128-byte-row tile.
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * kRowB + ((((col >> 3) ^ swz(row)) << 4) | ((col & 7) << 1));
}

// Transposed LDS read: with lane 4r+c of each 16-lane group addressing 4 consecutive
// fp16 of row r, lane i of the group receives column i of those 4 rows.
__device__ __forceinline__ f16x4 read_tr(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_void*)p);
  return __builtin_bit_cast(f16x4, v);
}

// q = u / h, r = u % h for 0 <= u < 2^24, from rcp = 1/h (fp32, host-rounded): u and
// u * rcp are within one unit of the quotient, which one correction step fixes.
__device__ __forceinline__ void divmod_rcp(int u, int h, float rcp, int& q, int& r) {
  q = (int)((float)u * rcp);
  r = u - q * h;
  if (r < 0) --q, r += h;
  if (r >= h) ++q, r -= h;
}

__global__ __launch_bounds__(kThreads) void flash_attn_kernel(
    const f16* __restrict__ qkv, f16* __restrict__ O, int seq_len, int seg_len_max, int n_segs,
    int tiles_per_seg, float rcp_segs, float rcp_tiles, int window0, int uniform_valid, ValidLens valid) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave / kQuarters, quarter = wave % kQuarters;
  const int l32 = lane & 31, g = lane >> 5;

  // XCD-aware decode: consecutive logical tiles (the query tiles of one head) share an XCD.
  const int nwg = gridDim.x, wid = blockIdx.x;
  const int xcd = wid % kXcds, per = nwg / kXcds, rem = nwg % kXcds;
  const int t = xcd * per + min(xcd, rem) + wid / kXcds;
  int t1, qt, seg, wloc;
  divmod_rcp(t, tiles_per_seg, rcp_tiles, t1, qt);
  const int t2 = t1 / kHeads, head = t1 - t2 * kHeads;
  divmod_rcp(t2, n_segs, rcp_segs, wloc, seg);
  const int window = window0 + wloc;

  const int seg0 = seg * seg_len_max;
  const int seg_end = min(seg0 + seg_len_max, seq_len);
  const int q_begin = seg0 + qt * kBMq;
  if (q_begin >= seg_end) return;  // uniform for the workgroup
  const int k_lo = seg0;
  const int k_hi = max(k_lo, min(seg0 + seg_len_max, uniform_valid >= 0 ? uniform_valid : (int)valid.v[wloc]));

  const size_t win_row0 = (size_t)window * seq_len;
  const f16* qkv_w = qkv + win_row0 * kQkvCols;
  const int wq0 = q_begin + qg * kQW;  // this wave's first query row
  const bool wave_rows = wq0 < seg_end;

  if (k_hi <= k_lo) {  // no admitted key: zero rows
    if (wave_rows) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int q = wq0 + 32 * qb + l32;
        if (q < seg_end) {
          f16* orow = O + (win_row0 + q) * kDModel + head * kHeadDim;
#pragma unroll
          for (int c = 0; c < 4; ++c) store16(orow + 8 * (2 * c + g), (f16x8){});
        }
      }
    }
    return;
  }

  f16x8 qf[2][4];  // Q^T fragments, read from LDS once Q has landed

  // DMA duties: wave (qg, quarter) loads quarter's K (qg 0) or V (qg 1) tile: 4 x 8 rows.
  const int n_iter = (k_hi - k_lo + kIterKeys - 1) / kIterKeys;
  const uint32_t smem_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
  const f16* dma_base = qkv_w + (qg == 0 ? kDModel : 2 * kDModel) + head * kHeadDim;
  const int drow = lane >> 3;  // row within an 8-row DMA group
  // One DMA instruction: rows 8j .. 8j+7 of this wave's share of tile it.
  auto issue_part = [&](int it, int j) {
    const uint32_t st = smem_addr + (it % kStages) * kStageB + quarter * 2 * kTileB + qg * kTileB;
    const int row = 8 * j + drow;
    const int key = min(k_lo + it * kIterKeys + quarter * kKT + row, k_hi - 1);  // past the interval: masked
    const int lc = (lane & 7) ^ swz(row);
    dma16(dma_base + (size_t)key * kQkvCols + 8 * lc, st + j * 1024);
  };
  auto issue = [&](int it) {
#pragma unroll
    for (int j = 0; j < kKT / 8; ++j) issue_part(it, j);
  };
  constexpr int IPW = kKT / 8;
  // The same copy for a tile wholly inside [k_lo, k_hi) (every tile but the last), which
  // needs no clamp: a wave-uniform 64-bit source base (tile, part j) plus a per-lane 32-bit
  // offset that depends only on the lane and the parity of j (the row swizzle), so the copy
  // costs no vector arithmetic.
  const uint64_t dma_sbase = (uint64_t)(uintptr_t)(dma_base + (size_t)(k_lo + quarter * kKT) * kQkvCols);
  uint32_t dma_voff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    dma_voff[par] = (uint32_t)(drow * kQkvCols * 2 + 16 * ((lane & 7) ^ swz(8 * par + drow)));
  auto issue_part_inside = [&](int it, int j) {
    const uint32_t st = smem_addr + (it % kStages) * kStageB + quarter * 2 * kTileB + qg * kTileB + j * 1024;
    const uint64_t src = dma_sbase + (uint64_t)(it * kIterKeys + 8 * j) * (kQkvCols * 2);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(dma_voff[j & 1]), "s"(src), "s"(st) : "m0");
  };

  // Per-lane LDS offsets.
  int kfrag_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kfrag_off[s] = tile_off(l32, 16 * s + 8 * g);
  int vtr_off[2][2][2];  // [db][sigma][half]
  {
    const int i = lane & 15, r = i >> 2, c = i & 3;
    const int d0 = 16 * ((lane >> 4) & 1) + 4 * c;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int h = 0; h < 2; ++h) vtr_off[db][sg][h] = tile_off(16 * sg + 8 * h + 4 * g + r, 32 * db + d0);
  }

  // Per query block: reference m in scaled units (-inf until a key is seen) and the
  // MFMA accumulator seed -m (0 while m is -inf).
  float mref[2] = {-INFINITY, -INFINITY};
  f32x16 cneg[2] = {(f32x16){}, (f32x16){}};
  float l_run[2] = {0.0f, 0.0f};
  f32x16 oacc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) oacc[a][b] = (f32x16){};
  f32x16 sacc[2];   // scores of the tile between its MFMA and softmax phases
  f16x8 pf[2][2];   // fp16 P of the tile between its softmax and PV phases

  auto k_tile = [&](int it) { return smem + (it % kStages) * kStageB + quarter * 2 * kTileB; };

  // One MFMA phase: S^T for tile qk_it (if >= 0; only the last tile can extend past k_hi,
  // so only it masks), then O^T += V^T P^T for tile pv_it (if >= 0).  Every LDS fragment
  // read of the phase is issued first, so the MFMAs wait for the LDS latency once, and the
  // scores come first so that they are complete before this wave's next softmax while the
  // PV products finish.  dma >= 0: also issue the four DMA instructions of tile dma, one
  // per MFMA pair, so the address unit never sees a burst.
  // inside: tile dma lies wholly inside [k_lo, k_hi) (the unclamped copy form).
  auto phase = [&](int pv_it, int qk_it, bool last, int dma, auto inside) {
    auto dma_part = [&](int j) {
      if constexpr (decltype(inside)::value) issue_part_inside(dma, j);
      else issue_part(dma, j);
    };
    __builtin_amdgcn_s_setprio(1);
    f16x8 vfr[2][2], kf[4];
    if (qk_it >= 0) {
      const char* ks = k_tile(qk_it);
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[s] = *reinterpret_cast<const f16x8*>(ks + kfrag_off[s]);
    }
    if (pv_it >= 0) {
      const char* vs = k_tile(pv_it) + kTileB;
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const f16x4 lo = read_tr(vs + vtr_off[db][sg][0]);
          const f16x4 hi = read_tr(vs + vtr_off[db][sg][1]);
          vfr[sg][db] = (f16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (qk_it >= 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sacc[qb] = mfma_32x32x16(kf[0], qf[qb][0], cneg[qb]);
#pragma unroll
        for (int s = 1; s < 4; ++s) {
          sacc[qb] = mfma_32x32x16(kf[s], qf[qb][s], sacc[qb]);
          if (pv_it < 0 && dma >= 0 && (s & 1)) dma_part(2 * qb + (s >> 1));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (pv_it >= 0) {
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) oacc[qb][db] = mfma_32x32x16(vfr[sg][db], pf[qb][sg], oacc[qb][db]);
          if (dma >= 0) dma_part(2 * sg + db);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (qk_it >= 0 && last) {
      // Admitted keys of this lane's tile rows: key index kt0 + 8(e>>2) + 4g + (e&3) < k_hi.
      const int lim = k_hi - (k_lo + qk_it * kIterKeys + quarter * kKT) - 4 * g;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (8 * (e >> 2) + (e & 3) >= lim) sacc[qb][e] = -INFINITY;
    }
  };
  // Row maximum of the current tile per query block (both lane halves agree).
  auto tile_max = [&](int qb) {
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, sacc[qb][e]);
    return fmaxf(m, __shfl_xor(m, 32));
  };
  float lt[2];
  auto probabilities = [&]() {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = exp2_fast(sacc[qb][e]);
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const float* q = p + 8 * sg;
        const f16x2 a = pack_rne(q[0], q[1]), b = pack_rne(q[2], q[3]);
        const f16x2 c = pack_rne(q[4], q[5]), d = pack_rne(q[6], q[7]);
        pf[qb][sg] = (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
      }
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = p[e] + p[e + 8];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] += t[e + 4];
      lt[qb] = (t[0] + t[2]) + (t[1] + t[3]);
    }
  };
  // Softmax of the tile in sacc.  The first tile of a wave sets the reference (a fully
  // masked first tile leaves it at -inf with P = 0; all later tiles are masked too).
  // Later tiles keep it unless their P sum shows scores well above it: then the tile is
  // redone against the new maximum and the running sums are rescaled.
  auto softmax = [&](bool first) {
    if (first) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        mref[qb] = tile_max(qb);
        const float off = mref[qb] == -INFINITY ? 0.0f : mref[qb];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sacc[qb][e] -= off;
          cneg[qb][e] = -off;
        }
      }
    }
    probabilities();
    if (!first && __builtin_amdgcn_ballot_w64(lt[0] >= kRedoSum || lt[1] >= kRedoSum) != 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float d = fmaxf(tile_max(qb), 0.0f);  // excess of this tile over the reference
        const float alpha = exp2_fast(-d);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
        mref[qb] += d;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sacc[qb][e] -= d;
          cneg[qb][e] = -mref[qb];
        }
      }
      probabilities();
    }
    l_run[0] += lt[0];
    l_run[1] += lt[1];
  };

  // Ping-pong schedule over barrier slots b = 0 .. 2 n_iter + 1 (slot b lies between
  // barrier b and the next one).  Query group 0 runs the MFMA phase of iteration i
  // (QK of tile i, PV of tile i-1) in slot 2i and the softmax of tile i in slot 2i+1;
  // query group 1 runs one slot later, so on every SIMD one wave of each group alternates
  // MFMA and VALU work against the other.  Only the even barriers are workgroup barriers
  // (both groups pass the same n_iter + 1 of them); an odd slot boundary is a scheduling
  // fence alone, since no LDS hazard crosses it: tile t's stage is read from slot 2t to
  // slot 2t+3 and reloaded with tile t+4 after barrier 2t+4, each wave spreading its share
  // of tile i+2 over its MFMA phase of iteration i (slot 2i or 2i+1) and waiting for tile i
  // before barrier 2i.  (A workgroup barrier at the odd boundaries too, forcing the two
  // groups to swap roles in step, measured 3 % slower.)  The first and last tiles are
  // peeled so the steady-state body has no conditions.  Q's DMA is issued before tile 0's,
  // so the wait for tile 0 at barrier 0 covers it too.
  auto even_barrier = [&](int j) {  // barrier 2j: tile j has landed in LDS
    if (j + 1 < n_iter) {
      wait_vmcnt_barrier<IPW>();
    } else {
      wait_vmcnt_barrier<0>();
    }
  };
  auto odd_barrier = [&]() { __builtin_amdgcn_sched_barrier(0); };  // slot boundary: no s_barrier
  const int nl = n_iter - 1;  // last tile
  // The workgroup's 128 query rows reach LDS by DMA into stage 3 (whose first tile, tile 3,
  // is copied after slot boundary 2, the second workgroup barrier; every wave reads its Q
  // fragments before that barrier), two instructions of 8 rows per wave, issued before the
  // first tiles.  Rows past the segment load its last
  // row (finite values whose outputs are never stored).
  char* const q_lds = smem + 3 * kStageB;
  {
    const uint32_t qst = smem_addr + 3 * kStageB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 16 * wave + 8 * j + drow;
      const int q = min(q_begin + row, seg_end - 1);
      const int lc = (lane & 7) ^ swz(row);
      dma16(qkv_w + (size_t)q * kQkvCols + head * kHeadDim + 8 * lc, qst + (16 * wave + 8 * j) * kRowB);
    }
  }
  issue(0);
  if (n_iter > 1) issue(1);
  // Q^T fragments from LDS once tile 0 (and Q, issued before it) has landed: lane holds
  // Q[wq0 + 32 qb + l32][16 s + 8 g .. +7] scaled by log2(e)/8, applied as q c_hi + q c_lo
  // with c_hi = fp16(c), so the product is rounded once.
  auto load_q = [&]() {
    const f16x8 chi = (f16x8)(f16)kQScale;
    const f16x8 clo = (f16x8)(f16)(kQScale - (float)(f16)kQScale);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int r = qg * kQW + 32 * qb + l32;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 v = *reinterpret_cast<const f16x8*>(q_lds + tile_off(r, 16 * s + 8 * g));
        qf[qb][s] = __builtin_elementwise_fma(v, chi, v * clo);
      }
    }
  };

  const int dma0 = n_iter > 2 ? 2 : -1;
  using In = std::integral_constant<bool, true>;
  using NoIn = std::integral_constant<bool, false>;
  if (qg == 0) {
    even_barrier(0);
    load_q();
    phase(-1, 0, nl == 0, dma0, NoIn());
    odd_barrier();
    softmax(true);
    int i = 1;
    for (; i + 3 < n_iter; ++i) {  // copies tile i + 2 <= n_iter - 2: inside the interval
      even_barrier(i);
      phase(i - 1, i, false, i + 2, In());
      odd_barrier();
      softmax(false);
    }
    if (i + 2 < n_iter) {  // copies the last tile
      even_barrier(i);
      phase(i - 1, i, false, i + 2, NoIn());
      odd_barrier();
      softmax(false);
      ++i;
    }
    if (i < nl) {
      even_barrier(i);
      phase(i - 1, i, false, -1, NoIn());
      odd_barrier();
      softmax(false);
    }
    if (nl > 0) {
      even_barrier(nl);
      phase(nl - 1, nl, true, -1, NoIn());
      odd_barrier();
      softmax(false);
    }
    even_barrier(n_iter);
    phase(nl, -1, false, -1, NoIn());
    odd_barrier();
  } else {
    even_barrier(0);
    load_q();
    odd_barrier();
    phase(-1, 0, nl == 0, dma0, NoIn());
    even_barrier(1);
    softmax(true);
    int i = 1;
    for (; i + 3 < n_iter; ++i) {
      odd_barrier();
      phase(i - 1, i, false, i + 2, In());
      even_barrier(i + 1);
      softmax(false);
    }
    if (i + 2 < n_iter) {
      odd_barrier();
      phase(i - 1, i, false, i + 2, NoIn());
      even_barrier(i + 1);
      softmax(false);
      ++i;
    }
    if (i < nl) {
      odd_barrier();
      phase(i - 1, i, false, -1, NoIn());
      even_barrier(i + 1);
      softmax(false);
    }
    if (nl > 0) {
      odd_barrier();
      phase(nl - 1, nl, true, -1, NoIn());
      even_barrier(nl + 1);
      softmax(false);
    }
    odd_barrier();
    phase(nl, -1, false, -1, NoIn());
  }

  // Merge the four key quarters of each query group in one LDS round (the ring is free:
  // every DMA completed before the last iteration's barrier).  Wave `quarter` of a group
  // finalises output block (qb, db) = (quarter / 2, quarter % 2): it receives the other
  // three waves' partial O^T of that block and their (m, l) of that query block.
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) l_run[qb] += __shfl_xor(l_run[qb], 32);
  f32x4* const xo = reinterpret_cast<f32x4*>(smem);          // [group][owner][3 sources][4][64]
  f32x4* const xml = xo + kQGroups * 4 * 3 * 4 * kWave;       // [group][source][64]: m0, l0, m1, l1
  auto oslot = [&](int owner, int src) {
    return xo + ((qg * 4 + owner) * 3 + (src > owner ? src - 1 : src)) * 4 * kWave;
  };
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    if (blk == quarter) continue;
    f32x4* sl = oslot(blk, quarter);
    const f32x16& o = oacc[blk >> 1][blk & 1];
#pragma unroll
    for (int c = 0; c < 4; ++c) sl[c * kWave + lane] = (f32x4){o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
  }
  xml[(qg * 4 + quarter) * kWave + lane] = (f32x4){mref[0], l_run[0], mref[1], l_run[1]};
  __syncthreads();
  // The finished fp16 block goes to LDS first (rows of kOutLd halves after the merge
  // buffers), so that the workgroup writes whole 128-byte rows below.
  f16* const ost = reinterpret_cast<f16*>(xml + kQGroups * 4 * kWave);
  static_assert((kQGroups * 4 * 3 * 4 + kQGroups * 4) * kWave * 16 + kBMq * kOutLd * 2 <= kStages * kStageB,
                "merge buffers and the output block must fit in the ring");
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    if (blk != quarter || !wave_rows) continue;
    const int qb = blk >> 1, db = blk & 1;
    f32x4 ml[4];
    float M = mref[qb];
#pragma unroll
    for (int src = 0; src < 4; ++src) {
      if (src == blk) continue;
      ml[src] = xml[(qg * 4 + src) * kWave + lane];
      M = fmaxf(M, ml[src][2 * qb]);
    }
    f32x16 o = oacc[qb][db];
    float l = 0.0f;
    if (M != -INFINITY) {  // some quarter saw a key of this row
      const float w = mref[qb] == -INFINITY ? 0.0f : exp2_fast(mref[qb] - M);
      l = l_run[qb] * w;
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] *= w;
#pragma unroll
      for (int src = 0; src < 4; ++src) {
        if (src == blk) continue;
        const float ms = ml[src][2 * qb];
        const float ws = ms == -INFINITY ? 0.0f : exp2_fast(ms - M);
        l += ml[src][2 * qb + 1] * ws;
        const f32x4* sl = oslot(blk, src);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 v = sl[c * kWave + lane];
#pragma unroll
          for (int k = 0; k < 4; ++k) o[4 * c + k] += v[k] * ws;
        }
      }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    f16* orow = ost + (qg * kQW + 32 * qb + l32) * kOutLd;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 lo = pack_rne(o[4 * i + 0] * inv, o[4 * i + 1] * inv);
      const f16x2 hi = pack_rne(o[4 * i + 2] * inv, o[4 * i + 3] * inv);
      *reinterpret_cast<f16x4*>(orow + 32 * db + 8 * i + 4 * g) = (f16x4){lo[0], lo[1], hi[0], hi[1]};
    }
  }
  __syncthreads();
  // Rows q_begin .. of this head's 64 columns: 8 lanes per 128-byte row, written through to
  // memory (sc1) as the GEMM's output rows are.  Offsets from the block's origin.
  const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      O + (win_row0 + q_begin) * kDModel + head * kHeadDim, (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
  for (int c = tid; c < kBMq * 8; c += kThreads) {
    const int r = c >> 3, cc = c & 7;
    if (q_begin + r < seg_end)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, *reinterpret_cast<const f16x8*>(ost + r * kOutLd + 8 * cc)), o_rsrc,
          2 * (r * kDModel + 8 * cc), 0, kSc1);
  }
}

}  // namespace

hipError_t launch_flash_attn(const void* qkv, void* O, int batch, int seq_len, int chunk_len,
                             const int32_t* valid_host, hipStream_t stream) {
  const int seg_len_max = chunk_len > 0 ? chunk_len : seq_len;
  const int n_segs = (seq_len + seg_len_max - 1) / seg_len_max;
  const int tiles_per_seg = (seg_len_max + kBMq - 1) / kBMq;
  for (int w0 = 0; w0 < batch; w0 += kMaxBatchPerLaunch) {
    const int nb = min(kMaxBatchPerLaunch, batch - w0);
    ValidLens vl;
    for (int b = 0; b < nb; ++b) vl.v[b] = valid_host ? valid_host[w0 + b] : seq_len;
    for (int b = nb; b < kMaxBatchPerLaunch; ++b) vl.v[b] = 0;
    int uniform = vl.v[0];
    for (int b = 1; b < nb; ++b)
      if (vl.v[b] != uniform) uniform = -1;
    const long nwg = (long)nb * n_segs * tiles_per_seg * kHeads;
    if (nwg >= (1L << 24)) return hipErrorInvalidValue;  // the decode's division range
    dim3 grid((unsigned)nwg);
    hipLaunchKernelGGL(flash_attn_kernel, grid, dim3(kThreads), 0, stream,
                       static_cast<const f16*>(qkv), static_cast<f16*>(O), seq_len, seg_len_max,
                       n_segs, tiles_per_seg, 1.0f / (float)n_segs, 1.0f / (float)tiles_per_seg, w0, uniform, vl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace edda
