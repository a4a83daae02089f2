// C ABI of libedda.so: argument validation, workspace sizing, error text and
// dispatch of the gfx950 kernels onto the caller's stream.  Every check runs on
// the host before anything is enqueued; nothing falls back silently.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
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

size_t edda_verify_workspace_bytes(int32_t n_q, int32_t n_kv) {
  if (n_q < 1 || n_q > EDDA_MAX_VERIFY_QUERIES || n_kv < 1) return 0;
  return edda::verify_workspace_bytes(n_q, n_kv);
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
  const size_t need = edda::verify_workspace_bytes(n_q, n_kv);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EDDA_ERR_WORKSPACE, "edda_verify_attn: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  return from_hip(edda::launch_verify(q, n_q, k, v, n_kv, mask_rows, o, workspace,
                                      static_cast<hipStream_t>(stream)),
                  "edda_verify_attn launch");
}

}  // extern "C"
