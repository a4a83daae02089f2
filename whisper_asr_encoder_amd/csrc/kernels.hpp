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

// Flash attention over a packed [batch*seq_len, 3840] QKV buffer into O [batch*seq_len, 1280].
// chunk_len 0 = whole window; valid[b] = number of admitted key positions of window b.
hipError_t launch_flash_attn(const void* qkv, void* O, int batch, int seq_len, int chunk_len,
                             const int32_t* valid_host, hipStream_t stream);

// Split-KV verification attention. part_ml / part_o may be null when n_splits == 1.
int verify_num_splits(int n_kv);
size_t verify_workspace_bytes(int n_q, int n_kv);
hipError_t launch_verify(const void* q, int n_q, const void* k, const void* v, int n_kv,
                         const uint32_t* mask, void* o, void* workspace, hipStream_t stream);

}  // namespace edda
