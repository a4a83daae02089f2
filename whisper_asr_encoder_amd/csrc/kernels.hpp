// Internal launchers (host side) for the gfx950 kernels. Shapes are validated by
// the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace edda {

// C[M, N] = A[M, K] * Bt[N, K]^T (+ bias[N]); fp16 in/out, fp32 accumulation.
// Requires N % 64 == 0 and K % 64 == 0; any M >= 1.
hipError_t launch_gemm_bias(const void* A, const void* Bt, const void* bias, void* C, int M, int N,
                            int K, hipStream_t stream);

// C = act(A * Bt^T + bias) + residual[m % res_period] (act 0 none, 1 GELU; bias and
// residual may be null; residual may be C itself). Same shape rules as launch_gemm_bias.
hipError_t launch_gemm(const void* A, const void* Bt, const void* bias, const void* residual, int res_period,
                       int act, void* C, int M, int N, int K, hipStream_t stream);

// Row-wise LayerNorm over `features` (multiple of 256, at most 4096), eps 1e-5.
hipError_t launch_layer_norm(const void* x, int rows, int features, const void* gamma, const void* beta,
                             void* y, hipStream_t stream);

// Columns of a kernel-3, padding-1 convolution: cols[b*T_out + t][tap*C + c] =
// x_b[stride*t + tap - 1][c] (0 outside), x_b element (t, c) at x + b*x_batch + t*ts + c*cs.
// C % 8 == 0.
hipError_t launch_im2col3(const void* x, int batch, long x_batch, int t_in, int channels, long ts, long cs,
                          int stride, void* cols, hipStream_t stream);

// C = act(A * Bt^T + bias) + residual for M <= 16 rows (N % 16 == 0, K % 32 == 0):
// weights streamed straight into registers, 8-way K split inside a workgroup.
// scales != null: Bt holds Q8_0 int8 codes [N][K] and scales fp16 [K / 32][N] (the weight
// of (n, k) is scales[k / 32][n] * codes[n][k]); every skinny launcher takes them the same way.
hipError_t launch_skinny_gemm(const void* A, const void* Bt, const void* bias, const void* residual, int res_period,
                              int act, void* C, int M, int N, int K, hipStream_t stream,
                              const void* scales = nullptr);

// Q8_0 codes [rows][cols] and scales [cols / 32][rows] of fp16 weights [rows][cols].
hipError_t launch_quantize_q8_0(const void* w, int rows, int cols, void* codes, void* scales, hipStream_t stream);

// Cache slots of the (at most 16) block tokens, passed by value.
struct Slots {
  int32_t s[16];
};

// As launch_skinny_gemm (no residual) with A's rows (K = 1280) first normalised by
// LayerNorm(gamma, beta) inside the kernel.  With k_cache: C is a packed QKV block
// (N = 3840, act 0) whose K and V columns are also stored into k_cache / v_cache rows
// slots[m] ([slot][1280]).
hipError_t launch_skinny_ln_gemm(const void* A, const void* gamma, const void* beta, const void* Bt, const void* bias,
                                 int act, void* C, int M, int N, void* k_cache, void* v_cache, const Slots* slots,
                                 hipStream_t stream, const void* scales = nullptr);

// Split-K form of launch_skinny_gemm (act 0) for narrow outputs: skinny_splits(N, K)
// workgroups per 16-column block, each over a K range; the last to finish sums their fp32
// partials (part: skinny_split_part_bytes(N, K) bytes) in split order and applies the
// epilogue.  counters: N / 16 uint32 counters 64 bytes apart, zero before the call and left
// zero by it.  One split runs launch_skinny_gemm.
int skinny_splits(int N, int K);
size_t skinny_split_part_bytes(int N, int K);
hipError_t launch_skinny_gemm_split(const void* A, const void* Bt, const void* bias, const void* residual,
                                    int res_period, int act, void* C, int M, int N, int K, void* counters,
                                    void* part, hipStream_t stream, const void* scales = nullptr);

// Flash attention over a packed [batch*seq_len, 3840] QKV buffer into O [batch*seq_len, 1280].
// chunk_len 0 = whole window; valid[b] = number of admitted key positions of window b.
hipError_t launch_flash_attn(const void* qkv, void* O, int batch, int seq_len, int chunk_len,
                             const int32_t* valid_host, hipStream_t stream);

// Split-KV verification attention. part_ml / part_o may be null when n_splits == 1.
// mask_mode: 0 explicit rows (mask), 1 none, 2 causal block; sinks: fp32 [n_heads] or null.
// q rows are q_stride elements apart (n_heads * 64 for a contiguous [n_q, n_heads, 64] tensor).
int verify_num_splits(int n_kv);
// n uint32 words at p set to zero by a kernel on `stream` (no memset node in a captured graph).
hipError_t launch_zero_words(void* p, int n, hipStream_t stream);
size_t verify_workspace_bytes(int n_q, int n_kv, int n_heads);
hipError_t launch_verify(const void* q, int q_stride, int n_q, const void* k, const void* v, int n_kv, int n_heads,
                         int mask_mode, const uint32_t* mask, const float* sinks, void* o, void* workspace,
                         hipStream_t stream);

// The decoder's verification layer, n_layers consecutive layers of it, in one launch of
// `workgroups` persistent workgroups (kernel 8, fp16 or Q8_0 projection weights, n_kv <= 512).
// Layer l's w: ln1_gamma, ln1_beta, w_qkv, b_qkv, w_o, b_o, ln2_gamma, ln2_beta, w_q_cross,
// b_q_cross, w_o_cross, b_o_cross, ln3_gamma, ln3_beta, w_fc1, b_fc1, w_fc2, b_fc2 (biases may be
// null); scales: the Q8_0 scales of the six matrices (w: codes), or all null for every layer.
// Workspace rows of layer l at lws + l * lws_stride + off_*: qkv [16][3840], o, qc, x1, x2, y
// [16][1280], h [16][1280], f [16][5120] (byte offsets; no two overlap); y of layer l is the
// input of layer l + 1 (the last layer writes p.y).  verify_counters: 20 per-head counters 256
// bytes apart; ctl: 2 counters 256 bytes apart; flags: n_layers * decoder_fused_items(n_frames)
// words; all zero before the launch and left zero by it.  part: decoder_fused_part_bytes.
constexpr int kDecoderFusedMaxLayers = 8;
struct DecoderFusedLayer {
  const void* w[18];
  const void* scales[6];
  void* k_cache;
  void* v_cache;
  const void* cross_k;
  const void* cross_v;
};
struct DecoderFusedParams {
  const void* x;
  void* y;
  int n_q;
  Slots slots;
  int n_kv;
  const uint32_t* mask;  // rows [n_q][ceil(n_kv / 32)] or null (every slot admitted)
  int n_frames;
  int n_layers;
  DecoderFusedLayer layer[kDecoderFusedMaxLayers];
  void* lws;
  size_t lws_stride;
  uint32_t off_qkv, off_o, off_x1, off_qc, off_h, off_x2, off_f, off_y;
  void* verify_counters;
  void* ctl;
  void* flags;
  void* part;
  int workgroups;
};
constexpr int kDecoderFusedMaxItems = 768;
int decoder_fused_items(int n_frames);
bool decoder_fused_supported(int n_q, int n_kv, int n_frames);
size_t decoder_fused_part_bytes(int n_q, int n_frames);
hipError_t launch_decoder_layer_fused(const DecoderFusedParams& p, hipStream_t stream);

}  // namespace edda
