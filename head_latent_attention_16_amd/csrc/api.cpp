// C ABI of libmla.so: argument validation, workspace sizing and dispatch.
// Every entry point checks its arguments before making any HIP call, so the
// error paths can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>

#include <mutex>

#include "../../include/mla.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];
hipError_t g_info_err[kMaxDevices];

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] && strcmp(v, "0") != 0;
}

// Host-side validation of the dimension record.  Returns MLA_OK or an error.
mla_status_t check_dims(const mla_dims_t* d, Shape* s) {
  if (!d) return MLA_ERR_NULL;
  if (d->dtype != MLA_DT_BF16 && d->dtype != MLA_DT_F32) return MLA_ERR_DTYPE;
  if (d->n_h < 1 || d->d_c < 1 || d->d_r < 2 || (d->d_r & 1) || d->d_h < 1 || d->d_v < 1)
    return MLA_ERR_SHAPE;
  if (d->d_model < 0 || d->d_q < 0) return MLA_ERR_SHAPE;
  if (!(d->rope_base > 0.f) || !isfinite(d->rope_base)) return MLA_ERR_SHAPE;
  if (isnan(d->softmax_scale) || isinf(d->softmax_scale)) return MLA_ERR_SHAPE;
  // Widths the kernels can hold: the generic decode keeps a row in 20
  // registers per lane and the latent accumulator in 16.
  if (d->d_c > 1024 || d->d_c + d->d_r > 1280) return MLA_ERR_SHAPE;
  if (s) {
    s->n_h = d->n_h;
    s->d_c = d->d_c;
    s->d_r = d->d_r;
    s->d_h = d->d_h;
    s->d_v = d->d_v;
    s->d_model = d->d_model;
    s->d_q = d->d_q;
    s->rope_base = (double)d->rope_base;
    s->scale = d->softmax_scale > 0.f ? d->softmax_scale
                                      : (float)(1.0 / sqrt((double)(d->d_h + d->d_r)));
    s->bf16 = d->dtype == MLA_DT_BF16;
  }
  return MLA_OK;
}

size_t elem_bytes(const Shape& s) { return s.bf16 ? 2 : 4; }

mla_status_t device_ready(DeviceInfo* info) {
  hipError_t e = current_device_info(info);
  if (e != hipSuccess || !info->gfx950) return MLA_ERR_DEVICE;
  return MLA_OK;
}

mla_status_t launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

bool force_generic() { return env_flag("MLA_FORCE_GENERIC"); }

// Linear layers: the MFMA kernel for bf16 weights when the sizes suit it,
// the generic kernel otherwise.  Both paths of a call site are chosen by the
// same predicate in the workspace query and in the call.  The MFMA kernel
// takes bf16 activations: an intermediate that feeds it (c^Q, o) is rounded
// to bf16 once by the kernel that produces it, as in bf16 inference; the
// generic kernel keeps fp32 intermediates.
bool fast_linear(const Shape& s, int M, int N, int K) {
  return !force_generic() && s.bf16 && gemm_v3_supported(M, N, K);
}
size_t linear_ws(const Shape& s, int M, int N, int K) {
  return fast_linear(s, M, N, K) ? gemm_v3_workspace(M, N, K) : 0;
}
// Y = X W^T in fp32, X in the storage type (the caller has checked which
// path runs when X is an fp32 intermediate).
hipError_t linear(const Shape& s, int M, int N, int K, const void* X, bool x_f32, const void* W,
                  float* Y, void* part, hipStream_t st) {
  if (fast_linear(s, M, N, K)) return launch_gemm_v3(M, N, N, K, X, W, nullptr, Y, nullptr, part, st);
  return launch_linear_generic(s, M, N, K, X, x_f32, W, Y, st);
}

// Workspace layouts (byte offsets, each region 256-aligned).
// absorb from h_t: [c^Q fp32 | c^Q bf16 (fast W^UQ) | q (fp32; bf16 from the
// fast W^UQ) | split partials of the linear layers]
size_t absorb_ws(const Shape& s, int B, bool from_hidden) {
  if (!from_hidden) return 0;
  const int qw = s.n_h * (s.d_h + s.d_r);
  const int kq = s.d_q > 0 ? s.d_q : s.d_model;
  const bool uq_fast = fast_linear(s, B, qw, kq);
  size_t cq = s.d_q > 0 ? align256((size_t)B * s.d_q * sizeof(float)) : 0;
  size_t cqb = s.d_q > 0 && uq_fast ? align256((size_t)B * s.d_q * sizeof(uint16_t)) : 0;
  size_t q = align256((size_t)B * qw * (uq_fast ? sizeof(uint16_t) : sizeof(float)));
  size_t part = linear_ws(s, B, qw, kq);
  if (s.d_q > 0) {
    const size_t p1 = linear_ws(s, B, s.d_q, s.d_model);
    if (p1 > part) part = p1;
  }
  return cq + cqb + q + align256(part);
}
// Fused rope+latent key projection: one linear layer of d_c + d_r outputs
// whose rows come from W_DKV then W_KR.
bool fused_kv(const Shape& s, int M) { return fast_linear(s, M, s.d_c + s.d_r, s.d_model) && s.d_c % 32 == 0; }
size_t append_ws(const Shape& s, int B, int n_new, bool from_hidden) {
  if (!from_hidden) return 0;
  const int M = B * n_new;
  size_t part = 0;
  if (fused_kv(s, M)) {
    part = gemm_v3_workspace(M, s.d_c + s.d_r, s.d_model);
  } else {
    part = linear_ws(s, M, s.d_c, s.d_model);
    const size_t p2 = linear_ws(s, M, s.d_r, s.d_model);
    if (p2 > part) part = p2;
  }
  return align256((size_t)M * (s.d_c + s.d_r) * sizeof(float)) + align256(part);
}
// project_out with u: [o fp32 (when o is not given) | o bf16 (fast W^O) |
// split partials of W^O]
size_t project_ws(const Shape& s, int B, bool with_u) {
  if (!with_u) return 0;
  const size_t n = (size_t)B * s.n_h * s.d_v;
  const bool o_fast = fast_linear(s, B, s.d_model, s.n_h * s.d_v);
  return align256(n * sizeof(float)) + (o_fast ? align256(n * sizeof(uint16_t)) : 0) +
         align256(linear_ws(s, B, s.d_model, s.n_h * s.d_v));
}
// Query tokens per call (B n_q): the combine and generic decode grids index
// them in their second dimension.
constexpr int64_t kMaxQueryTokens = 65535;
// Only sizes the launch; clamped so that hint * n_q stays far from overflow.
int64_t clamp_hint(int64_t hint) { return hint < 1 ? 1 : (hint > (int64_t(1) << 40) ? int64_t(1) << 40 : hint); }

size_t decode_ws(const Shape& s, int B, int n_q, int64_t hint, int num_cu) {
  if (!force_generic() && decode_v3_supported(s))
    return decode_v3_workspace(s, B, n_q, clamp_hint(hint), num_cu);
  return 0;
}

RowMap contiguous_map(const int32_t* offsets) {
  RowMap m;
  m.offsets = offsets;
  m.table = nullptr;
  m.max_blocks = m.shift = m.num_blocks = 0;
  return m;
}

// Host-side validation of a paged pool description (see mla_decode_attn_paged).
mla_status_t paged_map(int32_t num_blocks, int32_t block_rows, const int32_t* block_table,
                       int32_t max_blocks, RowMap* out) {
  if (num_blocks < 1 || max_blocks < 1 || block_rows < 32 || block_rows > (1 << 20) ||
      (block_rows & (block_rows - 1)) != 0)
    return MLA_ERR_SHAPE;
  // a sequence's capacity max_blocks * block_rows must be an int32 length
  if ((int64_t)max_blocks * block_rows > INT32_MAX) return MLA_ERR_SHAPE;
  int shift = 0;
  while ((1 << shift) < block_rows) ++shift;
  out->offsets = nullptr;
  out->table = block_table;
  out->max_blocks = max_blocks;
  out->shift = shift;
  out->num_blocks = num_blocks;
  return MLA_OK;
}

// scales != NULL: `cache` holds E4M3 codes with one fp32 scale per row.
mla_status_t decode_common(const mla_dims_t* dims, int32_t B, int32_t n_q, const void* q_lat,
                           const void* q_pe, const void* cache, const float* scales, const RowMap& map,
                           const int32_t* lens, int64_t total_rows_hint, float* o_lat, float* lse,
                           int32_t* err_flag, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (B < 0 || n_q < 1 || (int64_t)B * n_q > kMaxQueryTokens) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (total_rows_hint < 1) return MLA_ERR_SHAPE;
  if (!q_lat || !q_pe || !cache || !(map.paged() ? map.table : map.offsets) || !lens || !o_lat)
    return MLA_ERR_NULL;
  total_rows_hint = clamp_hint(total_rows_hint);
  DeviceInfo info;
  const bool fast = !force_generic() && decode_v3_supported(s);
  // The workspace requirement depends on the device's CU count; size it
  // before touching the device only when the fast path needs it.
  if (fast) {
    if (!ws) return MLA_ERR_WORKSPACE;
    if ((st = device_ready(&info)) != MLA_OK) return st;
    const size_t need = decode_v3_workspace(s, B, n_q, total_rows_hint, info.num_cu);
    if (ws_bytes < need) return MLA_ERR_WORKSPACE;
    return launched(launch_decode_v3(s, B, n_q, q_lat, q_pe, cache, scales, map, lens, total_rows_hint,
                                     o_lat, lse, err_flag, ws, ws_bytes, info.num_cu,
                                     (hipStream_t)stream));
  }
  if ((st = device_ready(&info)) != MLA_OK) return st;
  return launched(launch_decode_generic(s, B, n_q, q_lat, q_pe, cache, scales, map, lens, o_lat, lse,
                                        err_flag, (hipStream_t)stream));
}

// ---- fixed scratch for mla_decode_attn_noalloc -----------------------------
// Device memory the library owns: one copy of this array on every device the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns for
// the current device, looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(52) << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (looked up on first use).
hipError_t scratch_ptr_current(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int num_cu_or_default() {
  DeviceInfo info;
  if (current_device_info(&info) == hipSuccess && info.num_cu > 0) return info.num_cu;
  return 256;
}

}  // namespace

hipError_t current_device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    hipDeviceProp_t p;
    hipError_t err = hipGetDeviceProperties(&p, dev);
    g_info_err[dev] = err;
    if (err == hipSuccess) {
      g_info[dev].device = dev;
      g_info[dev].num_cu = p.multiProcessorCount;
      g_info[dev].gfx950 = strncmp(p.gcnArchName, "gfx950", 6) == 0;
    }
  });
  if (g_info_err[dev] != hipSuccess) return g_info_err[dev];
  *out = g_info[dev];
  return hipSuccess;
}

}  // namespace mla

using namespace mla;

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int32_t st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a size is out of range or the dims are unsupported";
    case MLA_ERR_DTYPE: return "unknown element type";
    case MLA_ERR_WORKSPACE: return "workspace smaller than required";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_DEVICE: return "no usable gfx950 device is current";
  }
  return "unknown status";
}

size_t mla_cache_row_bytes(const mla_dims_t* dims) {
  Shape s;
  if (check_dims(dims, &s) != MLA_OK) return 0;
  return (size_t)(s.d_c + s.d_r) * elem_bytes(s);
}

size_t mla_absorb_q_workspace(const mla_dims_t* dims, int32_t B, int32_t from_hidden) {
  Shape s;
  if (check_dims(dims, &s) != MLA_OK || B < 0) return 0;
  return absorb_ws(s, B, from_hidden != 0);
}

}  // extern "C"

namespace {
// q_norm_w != NULL: c^Q is normalised in place (root-mean-square, eps) between
// the two query projections.
mla_status_t absorb_common(const mla_dims_t* dims, int32_t B, const void* h_t, const void* W_DQ,
                           const void* q_norm_w, float eps, const void* W_UQ, const void* q,
                           const void* W_UK, const int32_t* pos, void* q_lat, void* q_pe, void* ws,
                           size_t ws_bytes, void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (B < 0) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!W_UK || !pos || !q_lat || !q_pe) return MLA_ERR_NULL;
  const bool from_hidden = h_t != nullptr;
  if (from_hidden) {
    if (!W_UQ) return MLA_ERR_NULL;
    if (s.d_model < 1) return MLA_ERR_SHAPE;
    if ((s.d_q > 0) != (W_DQ != nullptr)) return s.d_q > 0 ? MLA_ERR_NULL : MLA_ERR_SHAPE;
  } else if (!q) {
    return MLA_ERR_NULL;
  }
  const size_t need = absorb_ws(s, B, from_hidden);
  if (need > 0 && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  DeviceInfo info;
  if ((st = device_ready(&info)) != MLA_OK) return st;
  hipStream_t hs = (hipStream_t)stream;

  // Inputs given in the storage type are fp32 exactly when the storage is fp32.
  const bool storage_f32 = !s.bf16;
  const void* qsrc = q;
  bool q_f32 = storage_f32;
  if (from_hidden) {
    // regions as absorb_ws
    char* w = (char*)ws;
    const int qw = s.n_h * (s.d_h + s.d_r);
    const int kq = s.d_q > 0 ? s.d_q : s.d_model;
    const bool uq_fast = fast_linear(s, B, qw, kq);
    float* cq = (float*)w;
    if (s.d_q > 0) w += align256((size_t)B * s.d_q * sizeof(float));
    void* cqb = w;
    if (s.d_q > 0 && uq_fast) w += align256((size_t)B * s.d_q * sizeof(uint16_t));
    void* qbuf = w;
    w += align256((size_t)B * qw * (uq_fast ? sizeof(uint16_t) : sizeof(float)));
    void* part = w;
    const void* x = h_t;   // the input of W^UQ
    bool x_f32 = storage_f32;
    if (s.d_q > 0) {
      hipError_t e;
      if (uq_fast && !q_norm_w && fast_linear(s, B, s.d_q, s.d_model)) {
        e = launch_gemm_v3(B, s.d_q, s.d_q, s.d_model, h_t, W_DQ, nullptr, nullptr, cqb, part, hs);
      } else {
        e = linear(s, B, s.d_q, s.d_model, h_t, storage_f32, W_DQ, cq, part, hs);
        if (e == hipSuccess && q_norm_w)
          e = launch_rmsnorm(s, cq, B, s.d_q, (size_t)s.d_q, q_norm_w, eps, uq_fast ? cqb : nullptr, hs);
        else if (e == hipSuccess && uq_fast)
          e = launch_to_bf16(cq, cqb, (size_t)B * s.d_q, hs);
      }
      if (e != hipSuccess) return MLA_ERR_LAUNCH;
      x = uq_fast ? cqb : (const void*)cq;
      x_f32 = !uq_fast;
    }
    hipError_t e = uq_fast ? launch_gemm_v3(B, qw, qw, kq, x, W_UQ, nullptr, nullptr, qbuf, part, hs)
                           : linear(s, B, qw, kq, x, x_f32, W_UQ, (float*)qbuf, part, hs);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
    qsrc = qbuf;
    q_f32 = !uq_fast;
  }
  if (!force_generic() && proj_v3_supported(s))
    return launched(launch_absorb_v3(s, B, qsrc, q_f32, W_UK, pos, q_lat, q_pe, hs));
  return launched(launch_absorb_generic(s, B, qsrc, q_f32, W_UK, pos, q_lat, q_pe, hs));
}
}  // namespace

extern "C" {

mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t B, const void* h_t, const void* W_DQ,
                          const void* W_UQ, const void* q, const void* W_UK, const int32_t* pos,
                          void* q_lat, void* q_pe, void* ws, size_t ws_bytes, void* stream) {
  return absorb_common(dims, B, h_t, W_DQ, nullptr, 0.f, W_UQ, q, W_UK, pos, q_lat, q_pe, ws, ws_bytes,
                       stream);
}

mla_status_t mla_absorb_q_normed(const mla_dims_t* dims, int32_t B, const void* h_t, const void* W_DQ,
                                 const void* q_norm_w, float eps, const void* W_UQ, const void* W_UK,
                                 const int32_t* pos, void* q_lat, void* q_pe, void* ws, size_t ws_bytes,
                                 void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (!(eps >= 0.f) || !std::isfinite(eps) || s.d_q < 1) return MLA_ERR_SHAPE;
  if (B > 0 && (!h_t || !W_DQ || !q_norm_w)) return MLA_ERR_NULL;
  return absorb_common(dims, B, h_t, W_DQ, q_norm_w, eps, W_UQ, nullptr, W_UK, pos, q_lat, q_pe, ws,
                       ws_bytes, stream);
}

size_t mla_append_cache_workspace(const mla_dims_t* dims, int32_t B, int32_t n_new,
                                  int32_t from_hidden) {
  Shape s;
  if (check_dims(dims, &s) != MLA_OK || B < 0 || n_new < 0) return 0;
  return append_ws(s, B, n_new, from_hidden != 0);
}

}  // extern "C"

namespace {
// kv_norm_w != NULL: the new latents c^KV are normalised in place
// (root-mean-square, eps) before they are written.
// scales != NULL: `cache` receives E4M3 codes with one fp32 scale per row.
mla_status_t append_common(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                           const void* W_DKV, const void* kv_norm_w, float eps, const void* W_KR,
                           const void* kv_raw, void* cache, float* scales, const RowMap& map,
                           int32_t* lens, int32_t* err_flag, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (B < 0 || n_new < 0) return MLA_ERR_SHAPE;
  if (B == 0 || n_new == 0) return MLA_OK;
  if (!cache || !(map.paged() ? map.table : map.offsets) || !lens) return MLA_ERR_NULL;
  const bool from_hidden = h_t != nullptr;
  if (from_hidden) {
    if (!W_DKV || !W_KR) return MLA_ERR_NULL;
    if (s.d_model < 1) return MLA_ERR_SHAPE;
  } else if (!kv_raw) {
    return MLA_ERR_NULL;
  }
  const size_t need = append_ws(s, B, n_new, from_hidden);
  if (need > 0 && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  DeviceInfo info;
  if ((st = device_ready(&info)) != MLA_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  const size_t D = (size_t)(s.d_c + s.d_r);
  // the row writer: the storage type, or 8-bit codes with a row scale
  auto write_rows = [&](const void* c_src, size_t c_stride, const void* k_src, size_t k_stride, bool src_f32) {
    return scales ? launch_append_fp8(s, B, n_new, c_src, c_stride, k_src, k_stride, src_f32, cache, scales, map,
                                      lens, err_flag, hs)
                  : launch_append_generic(s, B, n_new, c_src, c_stride, k_src, k_stride, src_f32, cache, map,
                                          lens, err_flag, hs);
  };
  if (from_hidden) {
    // c = x W_DKV^T and k = x W_KR^T into fp32 scratch, then rotate + write.
    const int M = B * n_new;
    float* kc = (float*)ws;
    void* part = (char*)ws + align256((size_t)M * D * sizeof(float));
    if (fused_kv(s, M)) {
      // one [M, d_c + d_r] product: row i = [c_i | k_i]
      hipError_t e = launch_gemm_v3(M, (int)D, s.d_c, s.d_model, h_t, W_DKV, W_KR, kc, nullptr, part, hs);
      if (e != hipSuccess) return MLA_ERR_LAUNCH;
      if (kv_norm_w && launch_rmsnorm(s, kc, M, s.d_c, D, kv_norm_w, eps, nullptr, hs) != hipSuccess)
        return MLA_ERR_LAUNCH;
      return launched(write_rows(kc, D, kc + s.d_c, D, true));
    }
    float* kr = kc + (size_t)M * s.d_c;
    hipError_t e = linear(s, M, s.d_c, s.d_model, h_t, !s.bf16, W_DKV, kc, part, hs);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
    if (kv_norm_w && launch_rmsnorm(s, kc, M, s.d_c, (size_t)s.d_c, kv_norm_w, eps, nullptr, hs) != hipSuccess)
      return MLA_ERR_LAUNCH;
    e = linear(s, M, s.d_r, s.d_model, h_t, !s.bf16, W_KR, kr, part, hs);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
    return launched(write_rows(kc, (size_t)s.d_c, kr, (size_t)s.d_r, true));
  }
  const char* raw = (const char*)kv_raw;
  // kv_raw is in the storage type: fp32 rows are read as fp32, bf16 rows as bf16.
  return launched(write_rows(raw, D, raw + (size_t)s.d_c * elem_bytes(s), D, !s.bf16));
}
}  // namespace

extern "C" {

mla_status_t mla_append_cache(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                              const void* W_DKV, const void* W_KR, const void* kv_raw, void* cache,
                              const int32_t* offsets, int32_t* lens, int32_t* err_flag, void* ws,
                              size_t ws_bytes, void* stream) {
  return append_common(dims, B, n_new, h_t, W_DKV, nullptr, 0.f, W_KR, kv_raw, cache, nullptr, contiguous_map(offsets), lens,
                       err_flag, ws, ws_bytes, stream);
}

mla_status_t mla_append_cache_normed(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                                     const void* W_DKV, const void* kv_norm_w, float eps,
                                     const void* W_KR, void* cache, const int32_t* offsets,
                                     int32_t* lens, int32_t* err_flag, void* ws, size_t ws_bytes,
                                     void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return MLA_ERR_SHAPE;
  if (B > 0 && n_new > 0 && (!h_t || !kv_norm_w)) return MLA_ERR_NULL;
  return append_common(dims, B, n_new, h_t, W_DKV, kv_norm_w, eps, W_KR, nullptr, cache, nullptr, contiguous_map(offsets), lens,
                       err_flag, ws, ws_bytes, stream);
}

size_t mla_decode_attn_workspace(const mla_dims_t* dims, int32_t B, int64_t total_rows_hint) {
  return mla_decode_attn_causal_workspace(dims, B, 1, total_rows_hint);
}

mla_status_t mla_decode_attn(const mla_dims_t* dims, int32_t B, const void* q_lat,
                             const void* q_pe, const void* cache, const int32_t* offsets,
                             const int32_t* lens, int64_t total_rows_hint, float* o_lat,
                             float* lse, int32_t* err_flag, void* ws, size_t ws_bytes,
                             void* stream) {
  return decode_common(dims, B, 1, q_lat, q_pe, cache, nullptr, contiguous_map(offsets), lens, total_rows_hint, o_lat, lse,
                       err_flag, ws, ws_bytes, stream);
}

size_t mla_decode_attn_causal_workspace(const mla_dims_t* dims, int32_t B, int32_t n_q,
                                        int64_t total_rows_hint) {
  Shape s;
  if (check_dims(dims, &s) != MLA_OK || B < 0 || n_q < 1 || (int64_t)B * n_q > kMaxQueryTokens) return 0;
  return decode_ws(s, B, n_q, total_rows_hint, num_cu_or_default());
}

mla_status_t mla_decode_attn_causal(const mla_dims_t* dims, int32_t B, int32_t n_q,
                                    const void* q_lat, const void* q_pe, const void* cache,
                                    const int32_t* offsets, const int32_t* lens,
                                    int64_t total_rows_hint, float* o_lat, float* lse,
                                    int32_t* err_flag, void* ws, size_t ws_bytes, void* stream) {
  return decode_common(dims, B, n_q, q_lat, q_pe, cache, nullptr, contiguous_map(offsets), lens, total_rows_hint, o_lat, lse,
                       err_flag, ws, ws_bytes, stream);
}

mla_status_t mla_decode_attn_noalloc(const mla_dims_t* dims, int32_t B, const void* q_lat,
                                     const void* q_pe, const void* cache, const int32_t* offsets,
                                     const int32_t* lens, int64_t total_rows_hint, float* o_lat,
                                     float* lse, int32_t* err_flag, void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (B < 0 || B > kMaxQueryTokens) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (total_rows_hint < 1) return MLA_ERR_SHAPE;
  if (!q_lat || !q_pe || !cache || !offsets || !lens || !o_lat) return MLA_ERR_NULL;
  DeviceInfo info;
  if ((st = device_ready(&info)) != MLA_OK) return st;
  const size_t need = decode_ws(s, B, 1, total_rows_hint, info.num_cu);
  if (need > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && scratch_ptr_current(&ws) != hipSuccess) return MLA_ERR_DEVICE;
  return decode_common(dims, B, 1, q_lat, q_pe, cache, nullptr, contiguous_map(offsets), lens, total_rows_hint, o_lat, lse,
                       err_flag, ws, need, stream);
}

mla_status_t mla_decode_attn_paged(const mla_dims_t* dims, int32_t B, const void* q_lat,
                                   const void* q_pe, const void* pool, int32_t num_blocks,
                                   int32_t block_rows, const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* lens, int64_t total_rows_hint, float* o_lat,
                                   float* lse, int32_t* err_flag, void* ws, size_t ws_bytes,
                                   void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  RowMap map;
  if ((st = paged_map(num_blocks, block_rows, block_table, max_blocks, &map)) != MLA_OK) return st;
  return decode_common(dims, B, 1, q_lat, q_pe, pool, nullptr, map, lens, total_rows_hint, o_lat, lse, err_flag,
                       ws, ws_bytes, stream);
}

mla_status_t mla_append_cache_paged(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                                    const void* W_DKV, const void* W_KR, const void* kv_raw, void* pool,
                                    int32_t num_blocks, int32_t block_rows, const int32_t* block_table,
                                    int32_t max_blocks, int32_t* lens, int32_t* err_flag, void* ws,
                                    size_t ws_bytes, void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  RowMap map;
  if ((st = paged_map(num_blocks, block_rows, block_table, max_blocks, &map)) != MLA_OK) return st;
  return append_common(dims, B, n_new, h_t, W_DKV, nullptr, 0.f, W_KR, kv_raw, pool, nullptr, map, lens, err_flag,
                       ws, ws_bytes, stream);
}

mla_status_t mla_decode_attn_fp8(const mla_dims_t* dims, int32_t B, const void* q_lat, const void* q_pe,
                                 const uint8_t* cache8, const float* scales, const int32_t* offsets,
                                 const int32_t* lens, int64_t total_rows_hint, float* o_lat, float* lse,
                                 int32_t* err_flag, void* ws, size_t ws_bytes, void* stream) {
  if (dims && B > 0 && !scales) return MLA_ERR_NULL;
  return decode_common(dims, B, 1, q_lat, q_pe, cache8, scales, contiguous_map(offsets), lens, total_rows_hint,
                       o_lat, lse, err_flag, ws, ws_bytes, stream);
}

mla_status_t mla_append_cache_fp8(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                                  const void* W_DKV, const void* W_KR, const void* kv_raw, uint8_t* cache8,
                                  float* scales, const int32_t* offsets, int32_t* lens, int32_t* err_flag,
                                  void* ws, size_t ws_bytes, void* stream) {
  if (dims && B > 0 && n_new > 0 && !scales) return MLA_ERR_NULL;
  return append_common(dims, B, n_new, h_t, W_DKV, nullptr, 0.f, W_KR, kv_raw, cache8, scales,
                       contiguous_map(offsets), lens, err_flag, ws, ws_bytes, stream);
}

size_t mla_prefill_attn_workspace(const mla_dims_t* dims, int32_t B, int32_t n_q, int64_t cache_rows) {
  Shape s;
  if (check_dims(dims, &s) != MLA_OK || !prefill_v3_supported(s) || B < 0 || B > 65535 || n_q < 1 ||
      cache_rows < 1)
    return 0;
  return prefill_v3_workspace(B, n_q, cache_rows);
}

mla_status_t mla_prefill_attn(const mla_dims_t* dims, int32_t B, int32_t n_q, const void* q, const void* cache,
                              int64_t cache_rows, const int32_t* offsets, const int32_t* lens, const void* W_UK,
                              const void* W_UV, float* o, float* lse, int32_t* err_flag, void* ws,
                              size_t ws_bytes, void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (!prefill_v3_supported(s)) return MLA_ERR_SHAPE;
  if (B < 0 || B > 65535 || n_q < 1 || cache_rows < 1 || cache_rows > INT32_MAX) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !cache || !offsets || !lens || !W_UK || !W_UV || !o) return MLA_ERR_NULL;
  if (!ws || ws_bytes < prefill_v3_workspace(B, n_q, cache_rows)) return MLA_ERR_WORKSPACE;
  DeviceInfo info;
  if ((st = device_ready(&info)) != MLA_OK) return st;
  return launched(launch_prefill_v3(s, B, n_q, q, cache, cache_rows, offsets, lens, W_UK, W_UV, o, lse, err_flag,
                                    ws, (hipStream_t)stream));
}

size_t mla_project_out_workspace(const mla_dims_t* dims, int32_t B, int32_t with_u) {
  Shape s;
  if (check_dims(dims, &s) != MLA_OK || B < 0) return 0;
  return project_ws(s, B, with_u != 0);
}

mla_status_t mla_project_out(const mla_dims_t* dims, int32_t B, const float* o_lat,
                             const void* W_UV, const void* W_O, float* o, float* u, void* ws,
                             size_t ws_bytes, void* stream) {
  Shape s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (B < 0) return MLA_ERR_SHAPE;
  if (B == 0 || (!o && !u)) return MLA_OK;
  if (!o_lat || !W_UV) return MLA_ERR_NULL;
  if (u) {
    if (!W_O) return MLA_ERR_NULL;
    if (s.d_model < 1) return MLA_ERR_SHAPE;
  }
  const size_t need = u ? project_ws(s, B, true) : 0;
  if (need > 0 && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  DeviceInfo info;
  if ((st = device_ready(&info)) != MLA_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  // workspace: regions as project_ws
  const size_t n = (size_t)B * s.n_h * s.d_v;
  const int kin = s.n_h * s.d_v;
  const bool o_fast = u && fast_linear(s, B, s.d_model, kin);
  const bool uv_fast = !force_generic() && proj_v3_supported(s);
  char* w = (char*)ws;
  float* of = o ? o : (float*)w;   // fp32 o
  if (u) w += align256(n * sizeof(float));
  void* obf = o_fast ? (void*)w : nullptr;   // bf16 o for the fast W^O
  if (o_fast) w += align256(n * sizeof(uint16_t));
  void* part = w;
  hipError_t e;
  if (uv_fast) {
    e = launch_uv_v3(s, B, o_lat, W_UV, o || !o_fast ? of : nullptr, obf, hs);
  } else {
    e = launch_uv_generic(s, B, o_lat, W_UV, of, hs);
    if (e == hipSuccess && o_fast) e = launch_to_bf16(of, obf, n, hs);
  }
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  if (u) {
    e = o_fast ? launch_gemm_v3(B, s.d_model, s.d_model, kin, obf, W_O, nullptr, u, nullptr, part, hs)
               : linear(s, B, s.d_model, kin, of, true, W_O, u, part, hs);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

}  // extern "C"
