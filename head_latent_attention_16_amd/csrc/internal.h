// Host-side launchers behind the C ABI.  Each returns hipSuccess or the HIP
// error of the failed launch; arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

struct Shape {
  int n_h, d_c, d_r, d_h, d_v, d_model, d_q;
  double rope_base;
  float scale;   // softmax scale (already resolved)
  bool bf16;
};

// ---- generic kernels: any dims, fp32 or bf16 storage, fp32 math -------------
// Y[M,N] (fp32) = X[M,K] . W[N,K]^T ; X is fp32 or storage type, W storage type.
hipError_t launch_linear_generic(const Shape& s, int M, int N, int K, const void* X, bool x_f32,
                                 const void* W, float* Y, hipStream_t st);
// q (fp32 or storage type) [B, n_h, d_h + d_r] -> q_lat, q_pe (storage type).
hipError_t launch_absorb_generic(const Shape& s, int B, const void* q, bool q_f32, const void* W_UK,
                                 const int32_t* pos, void* q_lat, void* q_pe, hipStream_t st);
// New rows -> cache: c from c_src (row stride c_stride elements), un-rotated
// k from k_src (stride k_stride); both fp32 or both the storage type.
hipError_t launch_append_generic(const Shape& s, int B, int n_new, const void* c_src,
                                 size_t c_stride, const void* k_src, size_t k_stride, bool src_f32,
                                 void* cache, const int32_t* offsets, int32_t* lens,
                                 int32_t* err_flag, hipStream_t st);
// B sequences with n_q query tokens each (n_q = 1: one decode query; n_q > 1:
// the last n_q cached rows are the step's tokens, token i sees rows up to
// lens[b] - n_q + i).  q_lat, q_pe, o_lat, lse are [B, n_q, n_h, ...].
hipError_t launch_decode_generic(const Shape& s, int B, int n_q, const void* q_lat, const void* q_pe,
                                 const void* cache, const int32_t* offsets, const int32_t* lens,
                                 float* o_lat, float* lse, int32_t* err_flag, hipStream_t st);
// In place on fp32 rows (stride ld): x[:cols] / sqrt(mean(x[:cols]^2) + eps) * w.
hipError_t launch_rmsnorm(const Shape& s, float* x, int rows, int cols, size_t ld, const void* w,
                          float eps, hipStream_t st);
// o[b,h,:] = W_UV[h] . o_lat[b,h,:] (fp32 out)
hipError_t launch_uv_generic(const Shape& s, int B, const float* o_lat, const void* W_UV, float* o,
                             hipStream_t st);

// ---- V3 fast path (bf16, d_c = 512, d_r = 64, n_h = 128) --------------------
bool decode_v3_supported(const Shape& s);
size_t decode_v3_workspace(const Shape& s, int B, int n_q, int64_t total_rows_hint, int num_cu);
hipError_t launch_decode_v3(const Shape& s, int B, int n_q, const void* q_lat, const void* q_pe,
                            const void* cache, const int32_t* offsets, const int32_t* lens,
                            int64_t total_rows_hint, float* o_lat, float* lse, int32_t* err_flag,
                            void* ws, size_t ws_bytes, int num_cu, hipStream_t st);

// bf16 per-head projections at n_h = 128, d_h = d_v = 128, d_c = 512, d_r = 64.
bool proj_v3_supported(const Shape& s);
// q (bf16, or fp32 when q_f32) [B, n_h, d_h + d_r] -> q_lat, q_pe (bf16).
hipError_t launch_absorb_v3(const Shape& s, int B, const void* q, bool q_f32, const void* W_UK,
                            const int32_t* pos, void* q_lat, void* q_pe, hipStream_t st);

// bf16-weight linear layer Y[M,N] (fp32) = X[M,K] . W^T, X bf16 or fp32.
// Rows n < N1 of W come from W1 (stride K), rows >= N1 from W2 (W2 == NULL:
// all rows from W1).  Needs N % 32 == 0 and K % 256 == 0, and a workspace of
// gemm_v3_workspace(M, N, K) bytes for the split partials (may be 0).
bool gemm_v3_supported(int M, int N, int K);
size_t gemm_v3_workspace(int M, int N, int K);
hipError_t launch_gemm_v3(int M, int N, int N1, int K, const void* X, bool x_f32, const void* W1,
                          const void* W2, float* Y, void* ws, hipStream_t st);
// o[b,h,:] = W_UV[h] . o_lat[b,h,:] (fp32 in and out).
hipError_t launch_uv_v3(const Shape& s, int B, const float* o_lat, const void* W_UV, float* o,
                        hipStream_t st);

// Device properties of the current device (cached per device, thread-safe).
struct DeviceInfo {
  int device;
  int num_cu;
  bool gfx950;
};
hipError_t current_device_info(DeviceInfo* out);

}  // namespace mla
