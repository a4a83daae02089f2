// Kernels 4 and 5: LayerNorm and the column gather of the convolutional stem.
//
// LayerNorm: one wave per row (the row arithmetic is layer_norm_row), 4 rows per
// workgroup.  HBM-bound: 2 bytes read and 2 written per element.
//
// Column gather (im2col) of a kernel-3, padding-1 convolution with stride s: output row
// t of window b holds, for tap = 0, 1, 2, the C input channels of frame s*t + tap - 1
// (zeros outside the window), so the convolution becomes one GEMM with K = 3C.  A
// thread writes 8 consecutive columns (16 bytes); it reads them with one 16-byte load
// when the channels are contiguous in the input, else element by element (the
// channel-major mel input, read once per window).
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layer_norm_row.hpp"

namespace edda {
namespace {

constexpr int kLnRowsPerBlock = 4;

template <int kGroups>  // 4-feature groups per lane: features = 256 * kGroups
__global__ __launch_bounds__(kLnRowsPerBlock * kWave) void layer_norm_kernel(
    const f16* __restrict__ x, int rows, const f16* __restrict__ gamma, const f16* __restrict__ beta,
    f16* __restrict__ y) {
  constexpr int kFeatures = 256 * kGroups;
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * kLnRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  // Output rows written through to memory (sc1), as the GEMM's: no dirty lines left for the
  // end-of-kernel L2 write-back.  The row's base is wave-uniform.
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc(y + (size_t)row * kFeatures, (short)0, 0x7fffffff, 0x00020000);
  layer_norm_row<kGroups>(x + (size_t)row * kFeatures, gamma, beta, lane, [&](int f, f16x4 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), yr, 2 * f, 0, 16);
  });
}

template <int kGroups>
hipError_t launch_ln(const void* x, int rows, const void* gamma, const void* beta, void* y, hipStream_t stream) {
  const int blocks = (rows + kLnRowsPerBlock - 1) / kLnRowsPerBlock;
  hipLaunchKernelGGL(layer_norm_kernel<kGroups>, dim3(blocks), dim3(kLnRowsPerBlock * kWave), 0, stream,
                     static_cast<const f16*>(x), rows, static_cast<const f16*>(gamma),
                     static_cast<const f16*>(beta), static_cast<f16*>(y));
  return hipGetLastError();
}

// One thread per 8 output columns; total = rows_out * 3C / 8 threads.
__global__ __launch_bounds__(256) void im2col3_kernel(const f16* __restrict__ x, long x_batch, int t_in,
                                                      int channels, long ts, long cs, int stride, int t_out,
                                                      long total, bool vec, f16* __restrict__ cols) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int row_chunks = 3 * channels / 8;
  const long r = idx / row_chunks;
  const int col = (int)(idx - r * row_chunks) * 8;
  const int b = (int)(r / t_out), t = (int)(r - (long)b * t_out);
  const int tap = col / channels, c0 = col - tap * channels;
  const int src = stride * t + tap - 1;
  f16x8 out = {};
  if (src >= 0 && src < t_in) {
    const f16* p = x + b * x_batch + (long)src * ts + (long)c0 * cs;
    if (vec) {
      out = load16(p);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = p[(long)e * cs];
    }
  }
  store16(cols + r * (3L * channels) + col, out);
}

}  // namespace

namespace {
template <int G>
hipError_t launch_ln_groups(int groups, const void* x, int rows, const void* gamma, const void* beta, void* y,
                            hipStream_t stream) {
  if constexpr (G > 16) {
    return hipErrorInvalidValue;
  } else {
    if (groups == G) return launch_ln<G>(x, rows, gamma, beta, y, stream);
    return launch_ln_groups<G + 1>(groups, x, rows, gamma, beta, y, stream);
  }
}
}  // namespace

hipError_t launch_layer_norm(const void* x, int rows, int features, const void* gamma, const void* beta,
                             void* y, hipStream_t stream) {
  if (features % 256 != 0) return hipErrorInvalidValue;
  return launch_ln_groups<1>(features / 256, x, rows, gamma, beta, y, stream);
}

hipError_t launch_im2col3(const void* x, int batch, long x_batch, int t_in, int channels, long ts, long cs,
                          int stride, void* cols, hipStream_t stream) {
  const int t_out = (t_in - 1) / stride + 1;
  const long total = (long)batch * t_out * (3L * channels / 8);
  // 16-byte loads need contiguous channels and 16-byte aligned rows.
  const bool vec = cs == 1 && ts % 8 == 0 && x_batch % 8 == 0 && ((uintptr_t)x & 15) == 0;
  const long blocks = (total + 255) / 256;
  if (blocks >= (1L << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(im2col3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const f16*>(x),
                     x_batch, t_in, channels, ts, cs, stride, t_out, total, vec, static_cast<f16*>(cols));
  return hipGetLastError();
}

}  // namespace edda
