// C ABI of libedda.so: argument validation, workspace sizing, error text and
// dispatch of the gfx950 kernels onto the caller's stream.  Every check runs on
// the host before anything is enqueued; nothing falls back silently.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/edda.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

edda_status fail(edda_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

edda_status ok() {
  g_last_error.clear();
  return EDDA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

edda_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(EDDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxRows = (int64_t)1 << 31;

// The GEMM's tile map handles fewer than 65536 tiles (128 rows by at least 64 columns).
bool gemm_tiles_ok(int64_t rows, int64_t n) { return ((rows + 127) / 128) * (n / 64) < 65536; }

// Scratch of edda_verify_attn_noalloc: the verification workspace (arrival counters, then the
// fp32 partial results of the key splits) for up to EDDA_NOALLOC_MAX_KV keys, 16 queries and 20
// heads, as a device array of this library (one copy per GPU, held until the process ends).
// Host code never passes `scratch` itself to a kernel: its name is only a host-side stand-in;
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocSplits = (EDDA_NOALLOC_MAX_KV + 127) / 128;
constexpr size_t kNoAllocScratchBytes =
    EDDA_VERIFY_COUNTER_BYTES + kNoAllocSplits * EDDA_MAX_VERIFY_QUERIES * EDDA_N_HEADS * (2 + EDDA_HEAD_DIM) * 4;
static_assert(EDDA_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "scratch size in the public header");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch`, looked up on the first call on the device; that
// call also clears the arrival counters with a kernel on its stream (every later call leaves
// them zero, as the verification kernels reset their counters).
edda_status noalloc_scratch(const char* fn, hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EDDA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(EDDA_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(EDDA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    e = edda::launch_zero_words(p, EDDA_VERIFY_COUNTER_BYTES / 4, stream);
    if (e != hipSuccess) return fail(EDDA_ERR_HIP, "%s: clearing the counters: %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EDDA_OK;
}

}  // namespace

extern "C" {

const char* edda_last_error(void) { return g_last_error.c_str(); }

const char* edda_version(void) { return "edda 0.1 (gfx950)"; }

edda_status edda_qkv_pack(const void* x, int64_t rows, const void* w_qkv, const void* b_qkv,
                          void* qkv, void* stream) {
  if (!x || !w_qkv || !qkv) return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_qkv_pack: x, w_qkv and qkv must be non-null");
  if (rows < 1 || rows >= kMaxRows / EDDA_QKV_COLS)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_qkv_pack: rows = %lld out of range", (long long)rows);
  if (!aligned(x, 16) || !aligned(w_qkv, 16) || !aligned(qkv, 16) || (b_qkv && !aligned(b_qkv, 16)))
    return fail(EDDA_ERR_MISALIGNED, "edda_qkv_pack: pointers must be 16-byte aligned");
  return from_hip(edda::launch_gemm_bias(x, w_qkv, b_qkv, qkv, (int)rows, EDDA_QKV_COLS, EDDA_D_MODEL,
                                         static_cast<hipStream_t>(stream)),
                  "edda_qkv_pack launch");
}

size_t edda_encoder_workspace_bytes(int32_t batch, int32_t seq_len) {
  if (batch < 1 || seq_len < 1) return 0;
  const int64_t rows = (int64_t)batch * seq_len;
  if (rows >= kMaxRows / EDDA_QKV_COLS) return 0;
  return (size_t)rows * EDDA_D_MODEL * 2;
}

namespace {
edda_status check_encoder_shape(const char* fn, int32_t batch, int32_t seq_len, int32_t chunk_len,
                                const int32_t* valid_len) {
  if (batch < 1 || seq_len < 1)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: batch = %d and seq_len = %d must be >= 1", fn, batch, seq_len);
  const int64_t rows = (int64_t)batch * seq_len;
  if (rows >= kMaxRows / EDDA_QKV_COLS)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: batch*seq_len = %lld too large", fn, (long long)rows);
  if (chunk_len < 0 || chunk_len > seq_len)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: chunk_len = %d outside {0} U [1, seq_len = %d]", fn, chunk_len, seq_len);
  if (valid_len) {
    for (int32_t b = 0; b < batch; ++b)
      if (valid_len[b] < 1 || valid_len[b] > seq_len)
        return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: valid_len[%d] = %d outside [1, %d]", fn, b, valid_len[b], seq_len);
  }
  return EDDA_OK;
}
}  // namespace

edda_status edda_flash_attn(const void* qkv, int32_t batch, int32_t seq_len, int32_t chunk_len,
                            const int32_t* valid_len, void* o, void* stream) {
  if (!qkv || !o) return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_flash_attn: qkv and o must be non-null");
  edda_status st = check_encoder_shape("edda_flash_attn", batch, seq_len, chunk_len, valid_len);
  if (st != EDDA_OK) return st;
  if (!aligned(qkv, 16) || !aligned(o, 16))
    return fail(EDDA_ERR_MISALIGNED, "edda_flash_attn: pointers must be 16-byte aligned");
  return from_hip(edda::launch_flash_attn(qkv, o, batch, seq_len, chunk_len, valid_len,
                                          static_cast<hipStream_t>(stream)),
                  "edda_flash_attn launch");
}

edda_status edda_encoder_attn(const void* qkv, int32_t batch, int32_t seq_len, int32_t chunk_len,
                              const int32_t* valid_len, const void* w_o, const void* b_o, void* y,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!qkv || !w_o || !y)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_encoder_attn: qkv, w_o and y must be non-null");
  edda_status st = check_encoder_shape("edda_encoder_attn", batch, seq_len, chunk_len, valid_len);
  if (st != EDDA_OK) return st;
  const int64_t rows = (int64_t)batch * seq_len;
  if (!aligned(qkv, 16) || !aligned(w_o, 16) || !aligned(y, 16) || (b_o && !aligned(b_o, 16)) ||
      (workspace && !aligned(workspace, 16)))
    return fail(EDDA_ERR_MISALIGNED, "edda_encoder_attn: pointers must be 16-byte aligned");
  const size_t need = edda_encoder_workspace_bytes(batch, seq_len);
  if (!workspace || workspace_bytes < need)
    return fail(EDDA_ERR_WORKSPACE, "edda_encoder_attn: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = edda::launch_flash_attn(qkv, workspace, batch, seq_len, chunk_len, valid_len, s);
  if (e != hipSuccess) return from_hip(e, "edda_encoder_attn flash-attention launch");
  return from_hip(edda::launch_gemm_bias(workspace, w_o, b_o, y, (int)rows, EDDA_D_MODEL, EDDA_D_MODEL, s),
                  "edda_encoder_attn output-projection launch");
}

edda_status edda_verify_attn_noalloc(const void* q, int32_t n_q, const void* k, const void* v, int32_t n_kv,
                                     const uint32_t* mask_rows, void* o, void* stream) {
  const char* fn = "edda_verify_attn_noalloc";
  if (!q || !k || !v || !o) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: q, k, v and o must be non-null", fn);
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_q = %d outside [1, %d]", fn, n_q, EDDA_MAX_VERIFY_QUERIES);
  if (n_kv < 1) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_kv = %d out of range", fn, n_kv);
  if (n_kv > EDDA_NOALLOC_MAX_KV)
    return fail(EDDA_ERR_UNSUPPORTED, "%s: n_kv = %d beyond the static scratch's limit of %d keys "
                "(use edda_verify_attn with a workspace)", fn, n_kv, EDDA_NOALLOC_MAX_KV);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || (mask_rows && !aligned(mask_rows, 4)))
    return fail(EDDA_ERR_MISALIGNED, "%s: q/k/v/o must be 16-byte and mask_rows 4-byte aligned", fn);
  const size_t need = edda::verify_workspace_bytes(n_q, n_kv, EDDA_N_HEADS);
  if (need > kNoAllocScratchBytes)
    return fail(EDDA_ERR_UNSUPPORTED, "%s: %zu bytes of scratch needed, %zu held", fn, need, kNoAllocScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    const edda_status st = noalloc_scratch(fn, s, &ws);
    if (st != EDDA_OK) return st;
  }
  return from_hip(edda::launch_verify(q, EDDA_D_MODEL, n_q, k, v, n_kv, EDDA_N_HEADS,
                                      mask_rows ? EDDA_MASK_ROWS : EDDA_MASK_NONE, mask_rows, nullptr, o, ws, s),
                  "edda_verify_attn_noalloc launch");
}

size_t edda_verify_workspace_bytes(int32_t n_q, int32_t n_kv) {
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES || n_kv < 1) return 0;
  return edda::verify_workspace_bytes(n_q, n_kv, EDDA_N_HEADS);
}

edda_status edda_verify_attn(const void* q, int32_t n_q, const void* k, const void* v, int32_t n_kv,
                             const uint32_t* mask_rows, void* o, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_verify_attn: q, k, v and o must be non-null");
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_verify_attn: n_q = %d outside [1, %d]", n_q, EDDA_MAX_VERIFY_QUERIES);
  if (n_kv < 1 || (int64_t)n_kv * EDDA_D_MODEL >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_verify_attn: n_kv = %d out of range", n_kv);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (mask_rows && !aligned(mask_rows, 4)) || (workspace && !aligned(workspace, 16)))
    return fail(EDDA_ERR_MISALIGNED, "edda_verify_attn: q/k/v/o/workspace must be 16-byte and mask_rows 4-byte aligned");
  const size_t need = edda::verify_workspace_bytes(n_q, n_kv, EDDA_N_HEADS);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EDDA_ERR_WORKSPACE, "edda_verify_attn: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  return from_hip(edda::launch_verify(q, EDDA_D_MODEL, n_q, k, v, n_kv, EDDA_N_HEADS,
                                      mask_rows ? EDDA_MASK_ROWS : EDDA_MASK_NONE, mask_rows, nullptr, o, workspace,
                                      static_cast<hipStream_t>(stream)),
                  "edda_verify_attn launch");
}


// ---------------------------------------------------------------------------------------
// The rest of the encoder: fused linear layers, LayerNorm, the pre-norm layer, the stem.
// ---------------------------------------------------------------------------------------

edda_status edda_linear(const void* x, int64_t rows, int32_t in_features, const void* w, int32_t out_features,
                        const void* bias, int32_t activation, const void* residual, int64_t residual_rows,
                        void* y, void* stream) {
  if (!x || !w || !y) return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_linear: x, w and y must be non-null");
  if (rows < 1 || in_features < 1 || out_features < 1)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_linear: rows, in_features and out_features must be >= 1");
  if (activation != EDDA_ACT_NONE && activation != EDDA_ACT_GELU)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_linear: unknown activation %d", activation);
  if (residual && residual_rows < 1)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_linear: residual_rows = %lld must be >= 1", (long long)residual_rows);
  if (in_features % 64 || out_features % 64)
    return fail(EDDA_ERR_UNSUPPORTED, "edda_linear: in_features = %d and out_features = %d must be multiples of 64",
                in_features, out_features);
  const int64_t width = in_features > out_features ? in_features : out_features;
  if (rows >= kMaxRows / width || (residual && residual_rows >= kMaxRows / out_features) ||
      !gemm_tiles_ok(rows, out_features))
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_linear: rows = %lld too large", (long long)rows);
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || (bias && !aligned(bias, 16)) ||
      (residual && !aligned(residual, 16)))
    return fail(EDDA_ERR_MISALIGNED, "edda_linear: pointers must be 16-byte aligned");
  return from_hip(edda::launch_gemm(x, w, bias, residual, residual ? (int)residual_rows : 1, activation, y,
                                    (int)rows, out_features, in_features, static_cast<hipStream_t>(stream)),
                  "edda_linear launch");
}

edda_status edda_layer_norm(const void* x, int64_t rows, int32_t features, const void* gamma, const void* beta,
                            void* y, void* stream) {
  if (!x || !gamma || !beta || !y)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_layer_norm: x, gamma, beta and y must be non-null");
  if (rows < 1 || features < 1)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_layer_norm: rows and features must be >= 1");
  if (features % 256 || features > 4096)
    return fail(EDDA_ERR_UNSUPPORTED, "edda_layer_norm: features = %d must be a multiple of 256, at most 4096",
                features);
  if (rows >= kMaxRows / features) return fail(EDDA_ERR_INVALID_ARGUMENT, "edda_layer_norm: rows too large");
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(beta, 16) || !aligned(y, 16))
    return fail(EDDA_ERR_MISALIGNED, "edda_layer_norm: pointers must be 16-byte aligned");
  return from_hip(edda::launch_layer_norm(x, (int)rows, features, gamma, beta, y, static_cast<hipStream_t>(stream)),
                  "edda_layer_norm launch");
}

size_t edda_encoder_layer_workspace_bytes(int32_t batch, int32_t seq_len) {
  if (batch < 1 || seq_len < 1) return 0;
  const int64_t rows = (int64_t)batch * seq_len;
  if (rows >= kMaxRows / EDDA_D_FF) return 0;
  return (size_t)rows * (EDDA_D_FF + 2 * EDDA_D_MODEL) * 2;
}

edda_status edda_encoder_layer(const void* x, int32_t batch, int32_t seq_len, int32_t chunk_len,
                               const int32_t* valid_len, const edda_encoder_layer_weights* wt, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "edda_encoder_layer";
  if (!x || !wt || !y) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: x, weights and y must be non-null", fn);
  const void* required[] = {wt->ln1_gamma, wt->ln1_beta, wt->w_qkv, wt->w_o, wt->ln2_gamma, wt->ln2_beta,
                            wt->w_fc1, wt->w_fc2};
  for (const void* p : required)
    if (!p) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: every LayerNorm and weight-matrix pointer is required", fn);
  edda_status st = check_encoder_shape(fn, batch, seq_len, chunk_len, valid_len);
  if (st != EDDA_OK) return st;
  const int64_t rows = (int64_t)batch * seq_len;
  if (rows >= kMaxRows / EDDA_D_FF || !gemm_tiles_ok(rows, EDDA_D_FF))
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: batch*seq_len = %lld too large", fn, (long long)rows);
  const void* all[] = {x, y, workspace, wt->ln1_gamma, wt->ln1_beta, wt->w_qkv, wt->b_qkv, wt->w_o, wt->b_o,
                       wt->ln2_gamma, wt->ln2_beta, wt->w_fc1, wt->b_fc1, wt->w_fc2, wt->b_fc2};
  for (const void* p : all)
    if (p && !aligned(p, 16)) return fail(EDDA_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", fn);
  const size_t need = edda_encoder_layer_workspace_bytes(batch, seq_len);
  if (!workspace || workspace_bytes < need)
    return fail(EDDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  // Workspace: big [rows, 5120] (QKV, later the MLP hidden layer), h [rows, 1280] (LN1 out,
  // then O, then LN2 out), x1 [rows, 1280].
  char* big = static_cast<char*>(workspace);
  char* h = big + rows * EDDA_D_FF * 2;
  char* x1 = h + rows * EDDA_D_MODEL * 2;
  const int m = (int)rows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = edda::launch_layer_norm(x, m, EDDA_D_MODEL, wt->ln1_gamma, wt->ln1_beta, h, s)) != hipSuccess)
    return from_hip(e, "edda_encoder_layer LN1 launch");
  if ((e = edda::launch_gemm(h, wt->w_qkv, wt->b_qkv, nullptr, 1, EDDA_ACT_NONE, big, m, EDDA_QKV_COLS,
                             EDDA_D_MODEL, s)) != hipSuccess)
    return from_hip(e, "edda_encoder_layer QKV launch");
  if ((e = edda::launch_flash_attn(big, h, batch, seq_len, chunk_len, valid_len, s)) != hipSuccess)
    return from_hip(e, "edda_encoder_layer attention launch");
  if ((e = edda::launch_gemm(h, wt->w_o, wt->b_o, x, m, EDDA_ACT_NONE, x1, m, EDDA_D_MODEL, EDDA_D_MODEL, s)) !=
      hipSuccess)
    return from_hip(e, "edda_encoder_layer output-projection launch");
  if ((e = edda::launch_layer_norm(x1, m, EDDA_D_MODEL, wt->ln2_gamma, wt->ln2_beta, h, s)) != hipSuccess)
    return from_hip(e, "edda_encoder_layer LN2 launch");
  if ((e = edda::launch_gemm(h, wt->w_fc1, wt->b_fc1, nullptr, 1, EDDA_ACT_GELU, big, m, EDDA_D_FF, EDDA_D_MODEL,
                             s)) != hipSuccess)
    return from_hip(e, "edda_encoder_layer fc1 launch");
  return from_hip(edda::launch_gemm(big, wt->w_fc2, wt->b_fc2, x1, m, EDDA_ACT_NONE, y, m, EDDA_D_MODEL, EDDA_D_FF, s),
                  "edda_encoder_layer fc2 launch");
}

namespace {
int64_t stem_frames_out(int32_t n_frames) { return (int64_t)(n_frames - 1) / 2 + 1; }
}  // namespace

size_t edda_encoder_stem_workspace_bytes(int32_t batch, int32_t n_mels, int32_t n_frames) {
  if (batch < 1 || n_mels < 1 || n_frames < 1) return 0;
  const int64_t r1 = (int64_t)batch * n_frames, r2 = (int64_t)batch * stem_frames_out(n_frames);
  if (r1 >= kMaxRows / (3 * EDDA_D_MODEL) || (int64_t)n_mels * 3 >= kMaxRows / r1 ||
      !gemm_tiles_ok(r1, EDDA_D_MODEL))
    return 0;
  return (size_t)(r1 * 3 * n_mels + r1 * EDDA_D_MODEL + r2 * 3 * EDDA_D_MODEL) * 2;
}

edda_status edda_encoder_stem(const void* mel, int32_t batch, int32_t n_mels, int32_t n_frames,
                              const void* conv1_w, const void* conv1_b, const void* conv2_w, const void* conv2_b,
                              const void* pos, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "edda_encoder_stem";
  if (!mel || !conv1_w || !conv2_w || !pos || !y)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: mel, conv1_w, conv2_w, pos and y must be non-null", fn);
  if (batch < 1 || n_mels < 1 || n_frames < 1)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: batch, n_mels and n_frames must be >= 1", fn);
  if (n_mels % 64) return fail(EDDA_ERR_UNSUPPORTED, "%s: n_mels = %d must be a multiple of 64", fn, n_mels);
  const size_t need = edda_encoder_stem_workspace_bytes(batch, n_mels, n_frames);
  if (need == 0) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: batch * n_frames too large", fn);
  const void* all[] = {mel, conv1_w, conv1_b, conv2_w, conv2_b, pos, y, workspace};
  for (const void* p : all)
    if (p && !aligned(p, 16)) return fail(EDDA_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", fn);
  if (!workspace || workspace_bytes < need)
    return fail(EDDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  const int64_t t2 = stem_frames_out(n_frames);
  const int64_t r1 = (int64_t)batch * n_frames, r2 = (int64_t)batch * t2;
  char* cols1 = static_cast<char*>(workspace);
  char* h1 = cols1 + r1 * 3 * n_mels * 2;
  char* cols2 = h1 + r1 * EDDA_D_MODEL * 2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  // Frame t, channel c of window b sits at mel[b][c][t].
  if ((e = edda::launch_im2col3(mel, batch, (long)n_mels * n_frames, n_frames, n_mels, 1, n_frames, 1, cols1, s)) !=
      hipSuccess)
    return from_hip(e, "edda_encoder_stem column gather (conv1) launch");
  if ((e = edda::launch_gemm(cols1, conv1_w, conv1_b, nullptr, 1, EDDA_ACT_GELU, h1, (int)r1, EDDA_D_MODEL,
                             3 * n_mels, s)) != hipSuccess)
    return from_hip(e, "edda_encoder_stem conv1 launch");
  if ((e = edda::launch_im2col3(h1, batch, (long)n_frames * EDDA_D_MODEL, n_frames, EDDA_D_MODEL, EDDA_D_MODEL, 1, 2,
                                cols2, s)) != hipSuccess)
    return from_hip(e, "edda_encoder_stem column gather (conv2) launch");
  return from_hip(edda::launch_gemm(cols2, conv2_w, conv2_b, pos, (int)t2, EDDA_ACT_GELU, y, (int)r2, EDDA_D_MODEL,
                                    3 * EDDA_D_MODEL, s),
                  "edda_encoder_stem conv2 launch");
}


// ---------------------------------------------------------------------------------------
// The decoder's verification layer.
// ---------------------------------------------------------------------------------------

namespace {
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of the decoder layer: the verification workspace (counters first), then h, qkv,
// o, x1, x2 and the MLP hidden layer, each 256-byte aligned.
// Split-K counters of the decoder layer's block GEMMs: after the 20 verification counter
// lines (256 bytes each) inside the zeroed counter region; 64 bytes per 16-column block.
constexpr size_t kSplitCounterOffset = (size_t)EDDA_N_HEADS * 256;
static_assert(kSplitCounterOffset + (EDDA_D_MODEL / 16) * 64 <= EDDA_VERIFY_COUNTER_BYTES,
              "split-K counters must fit in the counter region");
// The single-launch layer's ticket and exit counters, then one done flag per work item: the
// region's last free lines.
constexpr size_t kFusedCtlOffset = 12288;
constexpr size_t kFusedFlagOffset = kFusedCtlOffset + 2 * 256;
static_assert(kSplitCounterOffset + (EDDA_D_MODEL / 16) * 64 <= kFusedCtlOffset &&
                  kFusedFlagOffset + edda::kDecoderFusedMaxItems * 4 <= EDDA_VERIFY_COUNTER_BYTES,
              "fused-layer counters and flags must fit in the counter region");
// Persistent workgroups of the single-launch layer: one per compute unit of an MI355X.
constexpr int kFusedWorkgroups = 256;

struct DecoderWs {
  size_t verify, h, qkv, o, x1, x2, f, qc, total;
};

DecoderWs decoder_ws(int32_t n_q, int32_t n_kv, int32_t n_frames) {
  DecoderWs w{};
  size_t v1 = edda::verify_workspace_bytes(n_q, n_kv, EDDA_N_HEADS);
  size_t v2 = edda::verify_workspace_bytes(n_q, n_frames, EDDA_N_HEADS);
  // The block GEMMs with 1280 outputs split K; their partials reuse the region after the
  // counters (launches on one stream never overlap), their counters sit in the counter
  // lines the 20-head verification leaves unused.
  const size_t v3 = EDDA_VERIFY_COUNTER_BYTES + std::max(edda::skinny_split_part_bytes(EDDA_D_MODEL, EDDA_D_MODEL),
                                                         edda::skinny_split_part_bytes(EDDA_D_MODEL, EDDA_D_FF));
  const size_t v4 = EDDA_VERIFY_COUNTER_BYTES + edda::decoder_fused_part_bytes(n_q, n_frames);
  size_t off = align256(std::max(std::max(v1, v2), std::max(v3, v4)));
  w.verify = 0;
  const size_t row = (size_t)n_q * 2;
  // h, o and f hold 16 rows whatever n_q: the single-launch layer keeps them in MFMA fragment
  // order, which spans all 16 rows of the block GEMMs' operand.
  const size_t row16 = (size_t)EDDA_MAX_VERIFY_QUERIES * 2;
  w.h = off;
  w.qkv = w.h + align256(row16 * EDDA_D_MODEL);
  w.o = w.qkv + align256(row * EDDA_QKV_COLS);
  w.x1 = w.o + align256(row16 * EDDA_D_MODEL);
  w.x2 = w.x1 + align256(row * EDDA_D_MODEL);
  w.f = w.x2 + align256(row * EDDA_D_MODEL);
  w.qc = w.f + align256(row16 * EDDA_D_FF);  // the single-launch layer's cross query
  w.total = w.qc + align256(row * EDDA_D_MODEL);
  return w;
}
}  // namespace

size_t edda_decoder_verify_workspace_bytes(int32_t n_q, int32_t n_kv, int32_t n_frames) {
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES || n_kv < 1 || n_frames < 1) return 0;
  if ((int64_t)n_kv * EDDA_D_MODEL >= kMaxRows || (int64_t)n_frames * EDDA_D_MODEL >= kMaxRows) return 0;
  return decoder_ws(n_q, n_kv, n_frames).total;
}

namespace {
// One projection matrix: fp16 [out, in] (scales null) or Q8_0 codes with their scales.
struct Mat {
  const void* w;
  const void* scales;
};
struct DecoderMats {
  const void *ln1_gamma, *ln1_beta;
  Mat qkv;
  const void* b_qkv;
  Mat o;
  const void* b_o;
  const void *ln2_gamma, *ln2_beta;
  Mat q_cross;
  const void* b_q_cross;
  Mat o_cross;
  const void* b_o_cross;
  const void *ln3_gamma, *ln3_beta;
  Mat fc1;
  const void* b_fc1;
  Mat fc2;
  const void* b_fc2;
};

// One layer's pointers for the single-launch layer kernel.
void fused_layer_ptrs(const DecoderMats& wt, bool q8, void* k_cache, void* v_cache, const void* cross_k,
                      const void* cross_v, edda::DecoderFusedLayer* d) {
  const void* w[18] = {wt.ln1_gamma, wt.ln1_beta, wt.qkv.w,     wt.b_qkv,     wt.o.w,       wt.b_o,
                       wt.ln2_gamma, wt.ln2_beta, wt.q_cross.w, wt.b_q_cross, wt.o_cross.w, wt.b_o_cross,
                       wt.ln3_gamma, wt.ln3_beta, wt.fc1.w,     wt.b_fc1,     wt.fc2.w,     wt.b_fc2};
  for (int i = 0; i < 18; ++i) d->w[i] = w[i];
  const Mat* m6[6] = {&wt.qkv, &wt.o, &wt.q_cross, &wt.o_cross, &wt.fc1, &wt.fc2};
  for (int i = 0; i < 6; ++i) d->scales[i] = q8 ? m6[i]->scales : nullptr;
  d->k_cache = k_cache, d->v_cache = v_cache, d->cross_k = cross_k, d->cross_v = cross_v;
}

edda_status decoder_layer(const char* fn, const void* x, int32_t n_q, const int32_t* slots, void* k_cache,
                          void* v_cache, int32_t cache_slots, int32_t n_kv, const uint32_t* mask_rows,
                          const void* cross_k, const void* cross_v, int32_t n_frames, const DecoderMats* wt, void* y,
                          void* workspace, size_t workspace_bytes, void* stream, bool q8) {
  if (!x || !slots || !k_cache || !v_cache || !cross_k || !cross_v || !wt || !y)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: x, slots, caches, cross K/V, weights and y must be non-null", fn);
  const Mat mats[] = {wt->qkv, wt->o, wt->q_cross, wt->o_cross, wt->fc1, wt->fc2};
  const void* required[] = {wt->ln1_gamma, wt->ln1_beta, wt->ln2_gamma, wt->ln2_beta, wt->ln3_gamma, wt->ln3_beta};
  for (const void* p : required)
    if (!p) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: every LayerNorm and weight-matrix pointer is required", fn);
  for (const Mat& m : mats)
    if (!m.w || (q8 && !m.scales))
      return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: every LayerNorm and weight-matrix pointer is required", fn);
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_q = %d outside [1, %d]", fn, n_q, EDDA_MAX_VERIFY_QUERIES);
  if (cache_slots < 1 || n_kv < 1 || n_kv > cache_slots || (int64_t)cache_slots * EDDA_D_MODEL >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_kv = %d must be in [1, cache_slots = %d]", fn, n_kv, cache_slots);
  if (n_frames < 1 || (int64_t)n_frames * EDDA_D_MODEL >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_frames = %d out of range", fn, n_frames);
  edda::Slots sl{};
  for (int32_t t = 0; t < n_q; ++t) {
    if (slots[t] < 0 || slots[t] >= n_kv)
      return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: slots[%d] = %d outside [0, n_kv = %d)", fn, t, slots[t], n_kv);
    for (int32_t u = 0; u < t; ++u)
      if (slots[u] == slots[t]) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: slot %d repeated", fn, slots[t]);
    sl.s[t] = slots[t];
  }
  const void* all[] = {x, y, k_cache, v_cache, cross_k, cross_v, workspace, wt->ln1_gamma, wt->ln1_beta, wt->b_qkv,
                       wt->b_o, wt->ln2_gamma, wt->ln2_beta, wt->b_q_cross, wt->b_o_cross, wt->ln3_gamma,
                       wt->ln3_beta, wt->b_fc1, wt->b_fc2};
  for (const void* p : all)
    if (p && !aligned(p, 16)) return fail(EDDA_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", fn);
  for (const Mat& m : mats)
    if (!aligned(m.w, 16) || (m.scales && !aligned(m.scales, 16)))
      return fail(EDDA_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", fn);
  if (mask_rows && !aligned(mask_rows, 4)) return fail(EDDA_ERR_MISALIGNED, "%s: mask_rows must be 4-byte aligned", fn);
  const DecoderWs L = decoder_ws(n_q, n_kv, n_frames);
  if (!workspace || workspace_bytes < L.total)
    return fail(EDDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                workspace ? workspace_bytes : (size_t)0);
  char* ws = static_cast<char*>(workspace);
  void *h = ws + L.h, *qkv = ws + L.qkv, *o = ws + L.o, *x1 = ws + L.x1, *x2 = ws + L.x2, *f = ws + L.f;
  void* const sk_counters = ws + kSplitCounterOffset;
  void* const sk_part = ws + EDDA_VERIFY_COUNTER_BYTES;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = EDDA_D_MODEL;
  hipError_t e;
#define EDDA_STEP(call, what)             \
  if ((e = (call)) != hipSuccess) {       \
    char msg[96];                         \
    snprintf(msg, sizeof msg, "%s " what " launch", fn); \
    return from_hip(e, msg);              \
  }
  if (edda::decoder_fused_supported(n_q, n_kv, n_frames)) {
    // One launch: the eight steps below as work items of persistent workgroups.
    edda::DecoderFusedParams p{};
    p.x = x, p.y = y, p.n_q = n_q, p.slots = sl, p.n_kv = n_kv, p.mask = mask_rows, p.n_frames = n_frames;
    p.n_layers = 1;
    fused_layer_ptrs(*wt, q8, k_cache, v_cache, cross_k, cross_v, &p.layer[0]);
    // This workspace's rows as a one-layer block (offsets from its start).
    p.lws = ws, p.lws_stride = 0;
    p.off_qkv = (uint32_t)L.qkv, p.off_o = (uint32_t)L.o, p.off_x1 = (uint32_t)L.x1, p.off_qc = (uint32_t)L.qc;
    p.off_h = (uint32_t)L.h, p.off_x2 = (uint32_t)L.x2, p.off_f = (uint32_t)L.f, p.off_y = 0;  // y: the output
    p.verify_counters = ws, p.ctl = ws + kFusedCtlOffset, p.flags = ws + kFusedFlagOffset, p.part = sk_part;
    p.workgroups = kFusedWorkgroups;
    EDDA_STEP(edda::launch_decoder_layer_fused(p, s), "single-launch layer");
    return ok();
  }
  // Eight launches: LayerNorms run inside the block GEMMs that consume them, and the QKV
  // epilogue writes the block's K and V rows into their cache slots.
  EDDA_STEP(edda::launch_skinny_ln_gemm(x, wt->ln1_gamma, wt->ln1_beta, wt->qkv.w, wt->b_qkv, EDDA_ACT_NONE, qkv, n_q,
                                        EDDA_QKV_COLS, k_cache, v_cache, &sl, s, wt->qkv.scales),
            "LN1 + QKV + cache append");
  EDDA_STEP(edda::launch_verify(qkv, EDDA_QKV_COLS, n_q, k_cache, v_cache, n_kv, EDDA_N_HEADS,
                                mask_rows ? EDDA_MASK_ROWS : EDDA_MASK_NONE, mask_rows, nullptr, o, ws, s),
            "self-attention");
  EDDA_STEP(edda::launch_skinny_gemm_split(o, wt->o.w, wt->b_o, x, n_q, EDDA_ACT_NONE, x1, n_q, D, D, sk_counters,
                                           sk_part, s, wt->o.scales),
            "self output projection");
  EDDA_STEP(edda::launch_skinny_ln_gemm(x1, wt->ln2_gamma, wt->ln2_beta, wt->q_cross.w, wt->b_q_cross, EDDA_ACT_NONE,
                                        o, n_q, D, nullptr, nullptr, nullptr, s, wt->q_cross.scales),
            "LN2 + cross query");
  EDDA_STEP(edda::launch_verify(o, D, n_q, cross_k, cross_v, n_frames, EDDA_N_HEADS, EDDA_MASK_NONE, nullptr,
                                nullptr, h, ws, s),
            "cross-attention");
  EDDA_STEP(edda::launch_skinny_gemm_split(h, wt->o_cross.w, wt->b_o_cross, x1, n_q, EDDA_ACT_NONE, x2, n_q, D, D,
                                           sk_counters, sk_part, s, wt->o_cross.scales),
            "cross output projection");
  EDDA_STEP(edda::launch_skinny_ln_gemm(x2, wt->ln3_gamma, wt->ln3_beta, wt->fc1.w, wt->b_fc1, EDDA_ACT_GELU, f, n_q,
                                        EDDA_D_FF, nullptr, nullptr, nullptr, s, wt->fc1.scales),
            "LN3 + fc1");
  EDDA_STEP(edda::launch_skinny_gemm_split(f, wt->fc2.w, wt->b_fc2, x2, n_q, EDDA_ACT_NONE, y, n_q, D, EDDA_D_FF,
                                           sk_counters, sk_part, s, wt->fc2.scales),
            "fc2");
#undef EDDA_STEP
  return ok();
}
}  // namespace

edda_status edda_decoder_verify_layer(const void* x, int32_t n_q, const int32_t* slots, void* k_cache,
                                      void* v_cache, int32_t cache_slots, int32_t n_kv,
                                      const uint32_t* mask_rows, const void* cross_k, const void* cross_v,
                                      int32_t n_frames, const edda_decoder_layer_weights* wt, void* y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "edda_decoder_verify_layer";
  if (!wt) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: x, slots, caches, cross K/V, weights and y must be non-null", fn);
  const DecoderMats m{wt->ln1_gamma, wt->ln1_beta, {wt->w_qkv, nullptr}, wt->b_qkv, {wt->w_o, nullptr}, wt->b_o,
                      wt->ln2_gamma, wt->ln2_beta, {wt->w_q_cross, nullptr}, wt->b_q_cross, {wt->w_o_cross, nullptr},
                      wt->b_o_cross, wt->ln3_gamma, wt->ln3_beta, {wt->w_fc1, nullptr}, wt->b_fc1,
                      {wt->w_fc2, nullptr}, wt->b_fc2};
  return decoder_layer(fn, x, n_q, slots, k_cache, v_cache, cache_slots, n_kv, mask_rows, cross_k, cross_v, n_frames,
                       &m, y, workspace, workspace_bytes, stream, false);
}

edda_status edda_decoder_verify_layer_q8(const void* x, int32_t n_q, const int32_t* slots, void* k_cache,
                                         void* v_cache, int32_t cache_slots, int32_t n_kv,
                                         const uint32_t* mask_rows, const void* cross_k, const void* cross_v,
                                         int32_t n_frames, const edda_decoder_layer_weights_q8* wt, void* y,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "edda_decoder_verify_layer_q8";
  if (!wt) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: x, slots, caches, cross K/V, weights and y must be non-null", fn);
  auto M = [](const edda_q8_matrix& q) { return Mat{q.codes, q.scales}; };
  const DecoderMats m{wt->ln1_gamma, wt->ln1_beta, M(wt->w_qkv), wt->b_qkv, M(wt->w_o), wt->b_o,
                      wt->ln2_gamma, wt->ln2_beta, M(wt->w_q_cross), wt->b_q_cross, M(wt->w_o_cross),
                      wt->b_o_cross, wt->ln3_gamma, wt->ln3_beta, M(wt->w_fc1), wt->b_fc1, M(wt->w_fc2), wt->b_fc2};
  return decoder_layer(fn, x, n_q, slots, k_cache, v_cache, cache_slots, n_kv, mask_rows, cross_k, cross_v, n_frames,
                       &m, y, workspace, workspace_bytes, stream, true);
}

// ---------------------------------------------------------------------------------------
// Several decoder layers per launch.
// ---------------------------------------------------------------------------------------

namespace {
// Workspace of edda_decoder_verify_stack: the counter region (as for one layer: verification
// counters, then the single-launch kernel's ticket and exit counters), the items' done flags
// (both zero-initialised, EDDA_DECODER_STACK_ZERO_BYTES), the cross-attention partials, the
// carry rows between launches, then one block of rows per layer of a launch.
struct StackWs {
  size_t part, carry, blocks, block, total;
  size_t qkv, o, x1, qc, h, x2, f, y;  // offsets within a block
};
constexpr size_t kStackFlagOffset = EDDA_VERIFY_COUNTER_BYTES;
static_assert(kStackFlagOffset + (size_t)edda::kDecoderFusedMaxLayers * edda::kDecoderFusedMaxItems * 4 <=
                  EDDA_DECODER_STACK_ZERO_BYTES,
              "stack flags must fit in the zeroed region");

StackWs stack_ws(int32_t n_q, int32_t n_frames) {
  StackWs w{};
  const size_t rows = (size_t)EDDA_MAX_VERIFY_QUERIES * 2;  // bytes per feature column of a 16-row block
  w.part = EDDA_DECODER_STACK_ZERO_BYTES;
  w.carry = w.part + align256(edda::decoder_fused_part_bytes(n_q, n_frames));
  w.blocks = w.carry + align256(rows * EDDA_D_MODEL);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align256(bytes); return at; };
  w.qkv = take(rows * EDDA_QKV_COLS);
  w.o = take(rows * EDDA_D_MODEL);
  w.x1 = take(rows * EDDA_D_MODEL);
  w.qc = take(rows * EDDA_D_MODEL);
  w.h = take(rows * EDDA_D_MODEL);
  w.x2 = take(rows * EDDA_D_MODEL);
  w.f = take(rows * EDDA_D_FF);
  w.y = take(rows * EDDA_D_MODEL);
  w.block = off;
  w.total = w.blocks + (size_t)edda::kDecoderFusedMaxLayers * w.block;
  return w;
}
}  // namespace

size_t edda_decoder_verify_stack_workspace_bytes(int32_t n_q, int32_t n_kv, int32_t n_frames) {
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES || n_kv < 1 || n_frames < 1) return 0;
  if (!edda::decoder_fused_supported(n_q, n_kv, n_frames)) return 0;
  return stack_ws(n_q, n_frames).total;
}

}  // extern "C"

namespace {
// The layer's matrices in the form the single-launch kernel takes.
DecoderMats stack_mats(const edda_decoder_layer_weights& wt) {
  return DecoderMats{wt.ln1_gamma, wt.ln1_beta, {wt.w_qkv, nullptr}, wt.b_qkv, {wt.w_o, nullptr}, wt.b_o,
                     wt.ln2_gamma, wt.ln2_beta, {wt.w_q_cross, nullptr}, wt.b_q_cross, {wt.w_o_cross, nullptr},
                     wt.b_o_cross, wt.ln3_gamma, wt.ln3_beta, {wt.w_fc1, nullptr}, wt.b_fc1,
                     {wt.w_fc2, nullptr}, wt.b_fc2};
}
DecoderMats stack_mats(const edda_decoder_layer_weights_q8& wt) {
  auto M = [](const edda_q8_matrix& q) { return Mat{q.codes, q.scales}; };
  return DecoderMats{wt.ln1_gamma, wt.ln1_beta, M(wt.w_qkv), wt.b_qkv, M(wt.w_o), wt.b_o,
                     wt.ln2_gamma, wt.ln2_beta, M(wt.w_q_cross), wt.b_q_cross, M(wt.w_o_cross),
                     wt.b_o_cross, wt.ln3_gamma, wt.ln3_beta, M(wt.w_fc1), wt.b_fc1, M(wt.w_fc2), wt.b_fc2};
}

template <typename Layer>
edda_status decoder_stack(const char* fn, const void* x, int32_t n_q, const int32_t* slots, int32_t cache_slots,
                          int32_t n_kv, const uint32_t* mask_rows, int32_t n_frames, const Layer* layers,
                          int32_t n_layers, void* y, void* workspace, size_t workspace_bytes, void* stream,
                          bool q8) {
  if (!x || !slots || !layers || !y)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: x, slots, layers and y must be non-null", fn);
  if (n_layers < 1) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_layers = %d must be >= 1", fn, n_layers);
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_q = %d outside [1, %d]", fn, n_q, EDDA_MAX_VERIFY_QUERIES);
  if (cache_slots < 1 || n_kv < 1 || n_kv > cache_slots || (int64_t)cache_slots * EDDA_D_MODEL >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_kv = %d must be in [1, cache_slots = %d]", fn, n_kv, cache_slots);
  if (n_frames < 1 || (int64_t)n_frames * EDDA_D_MODEL >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_frames = %d out of range", fn, n_frames);
  if (!edda::decoder_fused_supported(n_q, n_kv, n_frames))
    return fail(EDDA_ERR_UNSUPPORTED,
                "%s: n_kv = %d (at most %d) or n_frames = %d: run edda_decoder_verify_layer per layer", fn, n_kv,
                EDDA_DECODER_STACK_MAX_KV, n_frames);
  edda::Slots sl{};
  for (int32_t t = 0; t < n_q; ++t) {
    if (slots[t] < 0 || slots[t] >= n_kv)
      return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: slots[%d] = %d outside [0, n_kv = %d)", fn, t, slots[t], n_kv);
    for (int32_t u = 0; u < t; ++u)
      if (slots[u] == slots[t]) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: slot %d repeated", fn, slots[t]);
    sl.s[t] = slots[t];
  }
  if (!aligned(x, 16) || !aligned(y, 16) || (workspace && !aligned(workspace, 256)))
    return fail(EDDA_ERR_MISALIGNED, "%s: x and y must be 16-byte, the workspace 256-byte aligned", fn);
  if (mask_rows && !aligned(mask_rows, 4)) return fail(EDDA_ERR_MISALIGNED, "%s: mask_rows must be 4-byte aligned", fn);
  for (int32_t l = 0; l < n_layers; ++l) {
    const Layer& L = layers[l];
    const DecoderMats m = stack_mats(L.weights);
    const void* required[] = {m.ln1_gamma, m.ln1_beta, m.qkv.w,     m.o.w,       m.ln2_gamma, m.ln2_beta,
                              m.q_cross.w, m.o_cross.w, m.ln3_gamma, m.ln3_beta, m.fc1.w,     m.fc2.w,
                              L.k_cache,   L.v_cache,   L.cross_k,   L.cross_v};
    for (const void* q : required)
      if (!q)
        return fail(EDDA_ERR_INVALID_ARGUMENT,
                    "%s: layer %d: every LayerNorm, weight-matrix, cache and cross K/V pointer is required", fn, l);
    const Mat* mats[] = {&m.qkv, &m.o, &m.q_cross, &m.o_cross, &m.fc1, &m.fc2};
    for (const Mat* mt : mats)
      if (q8 && !mt->scales)
        return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: layer %d: every Q8_0 matrix needs its scales", fn, l);
    const void* all[] = {m.ln1_gamma, m.ln1_beta, m.qkv.w,     m.b_qkv,     m.o.w,       m.b_o,       m.ln2_gamma,
                         m.ln2_beta,  m.q_cross.w, m.b_q_cross, m.o_cross.w, m.b_o_cross, m.ln3_gamma, m.ln3_beta,
                         m.fc1.w,     m.b_fc1,     m.fc2.w,     m.b_fc2,     L.k_cache,   L.v_cache,   L.cross_k,
                         L.cross_v,   m.qkv.scales, m.o.scales, m.q_cross.scales, m.o_cross.scales, m.fc1.scales,
                         m.fc2.scales};
    for (const void* q : all)
      if (q && !aligned(q, 16)) return fail(EDDA_ERR_MISALIGNED, "%s: layer %d: pointers must be 16-byte aligned", fn, l);
  }
  const StackWs W = stack_ws(n_q, n_frames);
  if (!workspace || workspace_bytes < W.total)
    return fail(EDDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, W.total,
                workspace ? workspace_bytes : (size_t)0);
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Launches of up to kDecoderFusedMaxLayers layers; between two launches the activations go
  // through the carry rows (a launch may read and then overwrite them: it reads its input only
  // in its first layer and writes its output in its last).
  const int G = edda::kDecoderFusedMaxLayers;
  for (int32_t l0 = 0; l0 < n_layers; l0 += G) {
    const int n = std::min<int32_t>(G, n_layers - l0);
    edda::DecoderFusedParams p{};
    p.x = l0 == 0 ? x : ws + W.carry;
    p.y = l0 + n == n_layers ? y : ws + W.carry;
    p.n_q = n_q, p.slots = sl, p.n_kv = n_kv, p.mask = mask_rows, p.n_frames = n_frames, p.n_layers = n;
    for (int i = 0; i < n; ++i) {
      const Layer& L = layers[l0 + i];
      fused_layer_ptrs(stack_mats(L.weights), q8, L.k_cache, L.v_cache, L.cross_k, L.cross_v, &p.layer[i]);
    }
    p.lws = ws + W.blocks, p.lws_stride = W.block;
    p.off_qkv = (uint32_t)W.qkv, p.off_o = (uint32_t)W.o, p.off_x1 = (uint32_t)W.x1, p.off_qc = (uint32_t)W.qc;
    p.off_h = (uint32_t)W.h, p.off_x2 = (uint32_t)W.x2, p.off_f = (uint32_t)W.f, p.off_y = (uint32_t)W.y;
    p.verify_counters = ws, p.ctl = ws + kFusedCtlOffset, p.flags = ws + kStackFlagOffset, p.part = ws + W.part;
    p.workgroups = kFusedWorkgroups;
    const hipError_t e = edda::launch_decoder_layer_fused(p, s);
    if (e != hipSuccess) {
      char msg[96];
      snprintf(msg, sizeof msg, "%s launch (layers %d..%d)", fn, l0, l0 + n - 1);
      return from_hip(e, msg);
    }
  }
  return ok();
}

}  // namespace

extern "C" {

edda_status edda_decoder_verify_stack(const void* x, int32_t n_q, const int32_t* slots, int32_t cache_slots,
                                      int32_t n_kv, const uint32_t* mask_rows, int32_t n_frames,
                                      const edda_decoder_stack_layer* layers, int32_t n_layers, void* y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decoder_stack("edda_decoder_verify_stack", x, n_q, slots, cache_slots, n_kv, mask_rows, n_frames, layers,
                       n_layers, y, workspace, workspace_bytes, stream, false);
}

edda_status edda_decoder_verify_stack_q8(const void* x, int32_t n_q, const int32_t* slots, int32_t cache_slots,
                                         int32_t n_kv, const uint32_t* mask_rows, int32_t n_frames,
                                         const edda_decoder_stack_layer_q8* layers, int32_t n_layers, void* y,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return decoder_stack("edda_decoder_verify_stack_q8", x, n_q, slots, cache_slots, n_kv, mask_rows, n_frames, layers,
                       n_layers, y, workspace, workspace_bytes, stream, true);
}

edda_status edda_quantize_q8_0(const void* w, int32_t rows, int32_t cols, void* codes, void* scales, void* stream) {
  const char* fn = "edda_quantize_q8_0";
  if (!w || !codes || !scales) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: w, codes and scales must be non-null", fn);
  if (rows < 1 || cols < 32 || (int64_t)rows * cols >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: rows = %d, cols = %d out of range", fn, rows, cols);
  if (cols % 32) return fail(EDDA_ERR_UNSUPPORTED, "%s: cols = %d must be a multiple of 32", fn, cols);
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 2))
    return fail(EDDA_ERR_MISALIGNED, "%s: w and codes must be 16-byte, scales 2-byte aligned", fn);
  return from_hip(edda::launch_quantize_q8_0(w, rows, cols, codes, scales, static_cast<hipStream_t>(stream)),
                  "edda_quantize_q8_0 launch");
}

edda_status edda_linear_q8(const void* x, int64_t rows, int32_t in_features, const void* codes, const void* scales,
                           int32_t out_features, const void* bias, int32_t activation, const void* residual,
                           int64_t residual_rows, void* y, void* stream) {
  const char* fn = "edda_linear_q8";
  if (!x || !codes || !scales || !y) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: x, codes, scales and y must be non-null", fn);
  if (rows < 1 || in_features < 1 || out_features < 1)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: rows, in_features and out_features must be >= 1", fn);
  if (activation != EDDA_ACT_NONE && activation != EDDA_ACT_GELU)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: unknown activation %d", fn, activation);
  if (residual && residual_rows < 1)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: residual_rows = %lld must be >= 1", fn, (long long)residual_rows);
  if ((int64_t)in_features * out_features >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: weight matrix too large", fn);
  if (rows > EDDA_MAX_VERIFY_QUERIES || in_features % 32 || out_features % 16)
    return fail(EDDA_ERR_UNSUPPORTED, "%s: rows = %lld (at most 16), in_features = %d (multiple of 32), "
                "out_features = %d (multiple of 16)", fn, (long long)rows, in_features, out_features);
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 16) || !aligned(y, 16) || (bias && !aligned(bias, 16)) ||
      (residual && !aligned(residual, 16)))
    return fail(EDDA_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", fn);
  return from_hip(edda::launch_skinny_gemm(x, codes, bias, residual, residual ? (int)residual_rows : 1, activation, y,
                                           (int)rows, out_features, in_features, static_cast<hipStream_t>(stream),
                                           scales),
                  "edda_linear_q8 launch");
}

edda_status edda_cross_kv(const void* enc, int32_t n_frames, const void* w_k, const void* w_v, const void* b_v,
                          void* cross_k, void* cross_v, void* stream) {
  const char* fn = "edda_cross_kv";
  if (!enc || !w_k || !w_v || !cross_k || !cross_v)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: enc, w_k, w_v, cross_k and cross_v must be non-null", fn);
  if (n_frames < 1 || n_frames >= kMaxRows / EDDA_D_MODEL || !gemm_tiles_ok(n_frames, EDDA_D_MODEL))
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_frames = %d out of range", fn, n_frames);
  const void* all[] = {enc, w_k, w_v, b_v, cross_k, cross_v};
  for (const void* p : all)
    if (p && !aligned(p, 16)) return fail(EDDA_ERR_MISALIGNED, "%s: pointers must be 16-byte aligned", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = edda::launch_gemm(enc, w_k, nullptr, nullptr, 1, EDDA_ACT_NONE, cross_k, n_frames, EDDA_D_MODEL,
                                   EDDA_D_MODEL, s);
  if (e != hipSuccess) return from_hip(e, "edda_cross_kv key projection launch");
  return from_hip(edda::launch_gemm(enc, w_v, b_v, nullptr, 1, EDDA_ACT_NONE, cross_v, n_frames, EDDA_D_MODEL,
                                    EDDA_D_MODEL, s),
                  "edda_cross_kv value projection launch");
}


size_t edda_verify_workspace_bytes_ex(int32_t n_q, int32_t n_kv, int32_t n_heads) {
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES || n_kv < 1 || n_heads < 1 || n_heads > EDDA_MAX_VERIFY_HEADS)
    return 0;
  if ((int64_t)n_kv * n_heads * 64 >= kMaxRows) return 0;
  return edda::verify_workspace_bytes(n_q, n_kv, n_heads);
}

edda_status edda_verify_attn_ex(const void* q, int32_t n_q, const void* k, const void* v, int32_t n_kv,
                                int32_t n_heads, int32_t mask_mode, const uint32_t* mask_rows, const float* sinks,
                                void* o, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "edda_verify_attn_ex";
  if (!q || !k || !v || !o) return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: q, k, v and o must be non-null", fn);
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_q = %d outside [1, %d]", fn, n_q, EDDA_MAX_VERIFY_QUERIES);
  if (n_heads < 1 || n_heads > EDDA_MAX_VERIFY_HEADS)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_heads = %d outside [1, %d]", fn, n_heads, EDDA_MAX_VERIFY_HEADS);
  if (n_kv < 1 || (int64_t)n_kv * n_heads * 64 >= kMaxRows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: n_kv = %d out of range", fn, n_kv);
  if (mask_mode != EDDA_MASK_ROWS && mask_mode != EDDA_MASK_NONE && mask_mode != EDDA_MASK_CAUSAL_BLOCK)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: unknown mask_mode %d", fn, mask_mode);
  if (mask_mode == EDDA_MASK_ROWS && !mask_rows)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: EDDA_MASK_ROWS needs mask_rows", fn);
  if (mask_mode == EDDA_MASK_CAUSAL_BLOCK && n_q > n_kv)
    return fail(EDDA_ERR_INVALID_ARGUMENT, "%s: a causal block needs n_q <= n_kv", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (mask_mode == EDDA_MASK_ROWS && !aligned(mask_rows, 4)) || (sinks && !aligned(sinks, 4)) ||
      (workspace && !aligned(workspace, 16)))
    return fail(EDDA_ERR_MISALIGNED, "%s: q/k/v/o/workspace must be 16-byte, mask_rows and sinks 4-byte aligned", fn);
  const size_t need = edda::verify_workspace_bytes(n_q, n_kv, n_heads);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EDDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  return from_hip(edda::launch_verify(q, n_heads * 64, n_q, k, v, n_kv, n_heads, mask_mode,
                                      mask_mode == EDDA_MASK_ROWS ? mask_rows : nullptr, sinks, o, workspace,
                                      static_cast<hipStream_t>(stream)),
                  "edda_verify_attn_ex launch");
}

}  // extern "C"
