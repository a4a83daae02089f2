// Kernel 2: flash attention for the encoder (fp16 Q/K/V, fp32 online softmax and
// accumulation); the score matrix never leaves registers.
//
// Work unit: one workgroup per (window, chunk segment, 32*NW query rows, head).
// With chunk_len = c > 0 every chunk of a window is an independent segment
// whose rows admit keys [seg0, min(seg0 + c, valid)); with c = 0 the segment is
// the whole window and the key interval is [0, valid).  Masking therefore
// reduces to one key interval per workgroup: the key loop visits only that
// interval, and only its last, partial 64-key tile masks elements.
//
// Per wave (32 query rows) and 64-key tile, on 32x32x16 MFMAs:
//   S^T = K Q^T  : K fragments from LDS, Q^T fragments resident in registers.
//                  Lane l then holds 32 scores of ONE query (l % 32), so row
//                  max / sum need only per-lane work plus one exchange with
//                  lane l ^ 32.
//   P   = 2^(S*log2e/8 - m)   (fp32, v_exp_f32), packed to fp16 with RNE.
//   O^T += V^T P^T : the fp16 P values are already laid out as the B operand
//                  (the MFMA's k index is permuted consistently on both
//                  operands); V^T fragments come from a transposed LDS copy.
// K/V tiles are double-buffered in LDS: the global loads of tile t+1 are in
// flight while tile t is computed.
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace edda {
namespace {

constexpr int kKeyTile = 64;
constexpr int kKld = kHeadDim + 8;   // K tile row stride (halves): 144 B, 16-byte aligned
constexpr int kVld = kKeyTile + 4;   // V^T tile row stride (halves): 136 B, 8-byte aligned
constexpr int kMaxBatchPerLaunch = 256;

struct ValidLens {
  int32_t v[kMaxBatchPerLaunch];
};

template <int NW>
__global__ __launch_bounds__(NW * kWave) void flash_attn_kernel(const f16* __restrict__ qkv,
                                                                f16* __restrict__ O, int seq_len,
                                                                int seg_len_max, int n_segs,
                                                                int tiles_per_seg, int window0,
                                                                ValidLens valid) {
  constexpr int NT = NW * kWave;
  constexpr int BM = 32 * NW;
  constexpr int KC = kKeyTile * 8 / NT;   // K 16-byte chunks per thread per tile
  constexpr int VP = kKeyTile / 2 * 8 / NT;  // V key-pair chunks per thread per tile
  static_assert(KC >= 1 && VP >= 1, "tile too small for the workgroup");

  __shared__ __attribute__((aligned(16))) f16 Ks[2][kKeyTile * kKld];
  __shared__ __attribute__((aligned(16))) f16 Vts[2][kHeadDim * kVld];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int head = blockIdx.y;

  int t = blockIdx.x;
  const int qt = t % tiles_per_seg;
  t /= tiles_per_seg;
  const int seg = t % n_segs;
  const int wloc = t / n_segs;
  const int window = window0 + wloc;

  const int seg0 = seg * seg_len_max;
  const int seg_len = min(seg_len_max, seq_len - seg0);
  const int q_begin = seg0 + qt * BM;
  if (q_begin >= seg0 + seg_len) return;  // whole workgroup beyond this segment's rows
  const int k_lo = seg0;
  const int k_hi = max(k_lo, min(seg0 + seg_len_max, (int)valid.v[wloc]));

  const size_t win_row0 = (size_t)window * seq_len;
  const int q_row = q_begin + 32 * wave + l32;  // this lane's query (window-local)
  const bool row_ok = q_row < seg0 + seg_len;
  const f16* qkv_w = qkv + win_row0 * kQkvCols;
  f16* out_row = O + (win_row0 + q_row) * kDModel + head * kHeadDim;

  if (k_hi <= k_lo) {  // no admitted key: O = 0 for every row of the segment
    if (row_ok) {
      const f16x8 z = {};
#pragma unroll
      for (int c = 0; c < kHeadDim / 8; c += 2) store16(out_row + 8 * (c + g), z);
    }
    return;
  }

  // Q^T fragments (B operand): lane holds Q[q_row][16 s + 8 g .. +7] for s = 0..3.
  f16x8 qf[4];
  {
    const f16x8 z = {};
    const f16* qp = qkv_w + (size_t)q_row * kQkvCols + head * kHeadDim + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = row_ok ? load16(qp + 16 * s) : z;
  }

  const f16* kbase = qkv_w + kDModel + head * kHeadDim;
  const f16* vbase = qkv_w + 2 * kDModel + head * kHeadDim;
  f16x8 rk[KC], rv0[VP], rv1[VP];
  const f16x8 z8 = {};

  auto gload = [&](int kt) {
#pragma unroll
    for (int r = 0; r < KC; ++r) {
      const int idx = tid + NT * r;
      const int key = kt + (idx >> 3), c = idx & 7;
      rk[r] = key < k_hi ? load16(kbase + (size_t)key * kQkvCols + 8 * c) : z8;
    }
#pragma unroll
    for (int r = 0; r < VP; ++r) {
      const int idx = tid + NT * r;
      const int key = kt + 2 * (idx >> 3), c = idx & 7;
      rv0[r] = key < k_hi ? load16(vbase + (size_t)key * kQkvCols + 8 * c) : z8;
      rv1[r] = key + 1 < k_hi ? load16(vbase + (size_t)(key + 1) * kQkvCols + 8 * c) : z8;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KC; ++r) {
      const int idx = tid + NT * r;
      store16(&Ks[buf][(idx >> 3) * kKld + 8 * (idx & 7)], rk[r]);
    }
#pragma unroll
    for (int r = 0; r < VP; ++r) {
      const int idx = tid + NT * r;
      const int kp = idx >> 3, c = idx & 7;
      // V^T[d][key]: the two keys of a pair share one 32-bit LDS word.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f16x2 pr = {rv0[r][e], rv1[r][e]};
        *reinterpret_cast<f16x2*>(&Vts[buf][(8 * c + e) * kVld + 2 * kp]) = pr;
      }
    }
  };

  const float c_scale = kLog2e / 8.0f;  // log2(e) / sqrt(64)
  float m_run = -INFINITY;              // running max of raw scores for this lane's query
  float l_run = 0.0f;                   // this lane's partial sum (half of the keys)
  f32x16 oacc[2] = {(f32x16){}, (f32x16){}};
  const bool wave_active = __builtin_amdgcn_readfirstlane(
      (int)(q_begin + 32 * wave < seg0 + seg_len));

  gload(k_lo);
  sstore(0);
  __syncthreads();
  const int n_tiles = (k_hi - k_lo + kKeyTile - 1) / kKeyTile;
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int kt = k_lo + it * kKeyTile;
    if (it + 1 < n_tiles) gload(kt + kKeyTile);

    if (wave_active) {
      // S^T for keys kt + 32 kb + (8 i + 4 g + j), query l32.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = (f32x16){};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f16x8 kf = load16(&Ks[buf][(32 * kb + l32) * kKld + 16 * s + 8 * g]);
          sacc[kb] = mfma_32x32x16(kf, qf[s], sacc[kb]);
        }
      }
      if (kt + kKeyTile > k_hi) {  // partial last tile: mask keys >= k_hi
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kt + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
            if (key >= k_hi) sacc[kb][e] = -INFINITY;
          }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sacc[kb][e]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = (m_run == -INFINITY) ? 0.0f : exp2_fast((m_run - m_new) * c_scale);
      const float mc = (m_new == -INFINITY) ? 0.0f : m_new * c_scale;
      m_run = m_new;
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(fmaf(sacc[kb][e], c_scale, -mc));
          sacc[kb][e] = p;
          lsum += p;
        }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;

      // O^T += V^T P^T over four 16-key steps sigma = (kb, hb).
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {
        const int kb = sg >> 1, hb = sg & 1;
        const f16x8 pf = pack8(sacc[kb][8 * hb + 0], sacc[kb][8 * hb + 1], sacc[kb][8 * hb + 2],
                               sacc[kb][8 * hb + 3], sacc[kb][8 * hb + 4], sacc[kb][8 * hb + 5],
                               sacc[kb][8 * hb + 6], sacc[kb][8 * hb + 7]);
        const int base = 32 * kb + 16 * hb + 4 * g;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const f16* vrow = &Vts[buf][(32 * db + l32) * kVld];
          const f16x4 v_lo = *reinterpret_cast<const f16x4*>(vrow + base);
          const f16x4 v_hi = *reinterpret_cast<const f16x4*>(vrow + base + 8);
          const f16x8 vf = {v_lo[0], v_lo[1], v_lo[2], v_lo[3], v_hi[0], v_hi[1], v_hi[2], v_hi[3]};
          oacc[db] = mfma_32x32x16(vf, pf, oacc[db]);
        }
      }
    }
    if (it + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 lo = pack_rne(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv);
      const f16x2 hi = pack_rne(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
      *reinterpret_cast<f16x4*>(out_row + 32 * db + 8 * i + 4 * g) = (f16x4){lo[0], lo[1], hi[0], hi[1]};
    }
}

}  // namespace

hipError_t launch_flash_attn(const void* qkv, void* O, int batch, int seq_len, int chunk_len,
                             const int32_t* valid_host, hipStream_t stream) {
  constexpr int NW = 4;
  constexpr int BM = 32 * NW;
  const int seg_len_max = chunk_len > 0 ? chunk_len : seq_len;
  const int n_segs = (seq_len + seg_len_max - 1) / seg_len_max;
  const int tiles_per_seg = (seg_len_max + BM - 1) / BM;
  for (int w0 = 0; w0 < batch; w0 += kMaxBatchPerLaunch) {
    const int nb = min(kMaxBatchPerLaunch, batch - w0);
    ValidLens vl;
    for (int b = 0; b < nb; ++b) vl.v[b] = valid_host ? valid_host[w0 + b] : seq_len;
    for (int b = nb; b < kMaxBatchPerLaunch; ++b) vl.v[b] = 0;
    dim3 grid(nb * n_segs * tiles_per_seg, kHeads);
    hipLaunchKernelGGL((flash_attn_kernel<NW>), grid, dim3(NW * kWave), 0, stream,
                       static_cast<const f16*>(qkv), static_cast<f16*>(O), seq_len, seg_len_max,
                       n_segs, tiles_per_seg, w0, vl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace edda
