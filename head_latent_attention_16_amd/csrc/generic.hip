// Generic MLA kernels: any head count and widths, fp32 or bf16 storage, fp32
// arithmetic.  They serve the small fp32 configuration and any dims the MFMA
// fast path does not cover; they favour obviousness over speed.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int kMaxRowPerLane = 20;   // (d_c + d_r) <= 64 * 20 = 1280
constexpr int kMaxLatPerLane = 16;   // d_c <= 1024

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i) { return to_f32(p[i]); }
__device__ __forceinline__ float ld_any(const void* p, bool f32, size_t i) {
  return f32 ? ((const float*)p)[i] : (float)((const __bf16*)p)[i];
}

// Y[m, n] = sum_k X[m, k] W[n, k].  One wave per (n, group of 8 rows m).
template <typename T>
__global__ void __launch_bounds__(64) k_linear(int M, int N, int K, const void* X, bool x_f32,
                                               const T* __restrict__ W, float* __restrict__ Y) {
  const int n = blockIdx.x;
  const int m0 = blockIdx.y * 8;
  const int lane = threadIdx.x;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const T* w = W + (size_t)n * K;
  for (int k = lane; k < K; k += 64) {
    float wk = ld(w, k);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (m0 + i < M) acc[i] += wk * ld_any(X, x_f32, (size_t)(m0 + i) * K + k);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = wave_sum(acc[i]);
    if (lane == 0 && m0 + i < M) Y[(size_t)(m0 + i) * N + n] = v;
  }
}

// q_lat[b,h,c] = sum_k qC[b,h,k] W_UK[h,k,c];  q_pe = RoPE(qR, pos[b]).
template <typename T>
__global__ void __launch_bounds__(256) k_absorb(int n_h, int d_c, int d_r, int d_h, double base,
                                                const void* q, bool q_f32, const T* __restrict__ W_UK,
                                                const int32_t* __restrict__ pos, T* __restrict__ q_lat,
                                                T* __restrict__ q_pe) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t qrow = ((size_t)b * n_h + h) * (d_h + d_r);
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < d_h; ++k)
      acc += ld_any(q, q_f32, qrow + k) * ld(W_UK, ((size_t)h * d_h + k) * d_c + c);
    q_lat[((size_t)b * n_h + h) * d_c + c] = from_f32<T>(acc);
  }
  const int half = d_r / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float cs, sn;
    rope_cos_sin(pos[b], i, d_r, base, &cs, &sn);
    float lo = ld_any(q, q_f32, qrow + d_h + i);
    float hi = ld_any(q, q_f32, qrow + d_h + half + i);
    T* out = q_pe + ((size_t)b * n_h + h) * d_r;
    out[i] = from_f32<T>(lo * cs - hi * sn);
    out[half + i] = from_f32<T>(hi * cs + lo * sn);
  }
}

// One block per sequence: writes its n_new rows, then bumps lens[b].  Row
// i of sequence b takes c from c_src + (b*n_new + i)*c_stride and the
// un-rotated k from k_src + (b*n_new + i)*k_stride.
template <typename T>
__global__ void __launch_bounds__(256) k_append(int n_new, int d_c, int d_r, double base,
                                                const void* c_src, size_t c_stride,
                                                const void* k_src, size_t k_stride, bool src_f32,
                                                T* __restrict__ cache, RowMap map,
                                                int32_t* __restrict__ lens, int32_t* err_flag) {
  const int b = blockIdx.x;
  const int D = d_c + d_r;
  const int len = lens[b];
  if (len < 0 || (int64_t)len + n_new > map.capacity(b)) {
    if (threadIdx.x == 0 && err_flag) atomicOr(err_flag, MLA_DEVERR_OVERFLOW);
    return;
  }
  // every destination row must map to a valid block before anything is written
  bool bad = false;
  for (int i = 0; i < n_new; ++i) bad |= map.row(b, (int64_t)len + i) < 0;
  if (bad) {
    if (threadIdx.x == 0 && err_flag) atomicOr(err_flag, MLA_DEVERR_TABLE);
    return;
  }
  const int half = d_r / 2;
  for (int i = 0; i < n_new; ++i) {
    const size_t idx = (size_t)b * n_new + i;
    const size_t cs = idx * c_stride, ks = idx * k_stride;
    T* dst = cache + (size_t)map.row(b, (int64_t)len + i) * D;
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
      if (src_f32)
        dst[c] = from_f32<T>(((const float*)c_src)[cs + c]);
      else
        dst[c] = ((const T*)c_src)[cs + c];   // bit-exact copy
    }
    for (int j = threadIdx.x; j < half; j += blockDim.x) {
      float cn, sn;
      rope_cos_sin((int64_t)len + i, j, d_r, base, &cn, &sn);
      float lo = ld_any(k_src, src_f32, ks + j);
      float hi = ld_any(k_src, src_f32, ks + half + j);
      dst[d_c + j] = from_f32<T>(lo * cn - hi * sn);
      dst[d_c + half + j] = from_f32<T>(hi * cn + lo * sn);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) lens[b] = len + n_new;
}

// 8-bit cache rows: one block per sequence.  For each new row its d_c + d_r
// values in fp32 (c copied, k rotated as in k_append) are staged in LDS, the
// row's largest magnitude amax comes from a block reduction, and the row is
// stored as E4M3 codes of x / 2^e (round to nearest even) with scale 2^e,
// e the smallest integer with amax <= 448 2^e (clamped to [-120, 120]; an
// all-zero row: codes 0, scale 1).  Dividing by a power of two is exact, so
// the codes depend only on the row's fp32 values.
__global__ void __launch_bounds__(256) k_append_fp8(int n_new, int d_c, int d_r, double base,
                                                    const void* c_src, size_t c_stride,
                                                    const void* k_src, size_t k_stride, bool src_f32,
                                                    uint8_t* __restrict__ cache, float* __restrict__ scales,
                                                    RowMap map, int32_t* __restrict__ lens, int32_t* err_flag) {
  extern __shared__ float row[];   // d_c + d_r
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int D = d_c + d_r;
  const int len = lens[b];
  if (len < 0 || (int64_t)len + n_new > map.capacity(b)) {
    if (threadIdx.x == 0 && err_flag) atomicOr(err_flag, MLA_DEVERR_OVERFLOW);
    return;
  }
  bool bad = false;
  for (int i = 0; i < n_new; ++i) bad |= map.row(b, (int64_t)len + i) < 0;
  if (bad) {
    if (threadIdx.x == 0 && err_flag) atomicOr(err_flag, MLA_DEVERR_TABLE);
    return;
  }
  const int half = d_r / 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = 0; i < n_new; ++i) {
    const size_t idx = (size_t)b * n_new + i;
    const size_t cs = idx * c_stride, ks = idx * k_stride;
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) row[c] = ld_any(c_src, src_f32, cs + c);
    for (int j = threadIdx.x; j < half; j += blockDim.x) {
      float cn, sn;
      rope_cos_sin((int64_t)len + i, j, d_r, base, &cn, &sn);
      const float lo = ld_any(k_src, src_f32, ks + j);
      const float hi = ld_any(k_src, src_f32, ks + half + j);
      row[d_c + j] = lo * cn - hi * sn;
      row[d_c + half + j] = hi * cn + lo * sn;
    }
    __syncthreads();
    float m = 0.f;
    for (int f = threadIdx.x; f < D; f += blockDim.x) m = fmaxf(m, fabsf(row[f]));
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int E = 0;
    const float mant = frexpf(amax, &E);          // amax = mant 2^E, 0.5 <= mant < 1
    int e = amax == 0.f ? 0 : (mant <= 0.875f ? E - 9 : E - 8);   // 448 = 0.875 2^9
    e = e < -120 ? -120 : (e > 120 ? 120 : e);
    const float inv = ldexpf(1.f, -e);
    const int64_t r = map.row(b, (int64_t)len + i);
    uint8_t* dst = cache + (size_t)r * D;
    for (int pr = threadIdx.x; 2 * pr < D; pr += blockDim.x) {
      const int f = 2 * pr;
      const float v0 = fminf(fmaxf(row[f] * inv, -448.f), 448.f);
      const float v1 = f + 1 < D ? fminf(fmaxf(row[f + 1] * inv, -448.f), 448.f) : 0.f;
      const int code = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
      dst[f] = (uint8_t)(code & 0xff);
      if (f + 1 < D) dst[f + 1] = (uint8_t)((code >> 8) & 0xff);
    }
    if (threadIdx.x == 0) scales[r] = ldexpf(1.f, e);
    __syncthreads();   // row[] and red[] are reused by the next row
  }
  if (threadIdx.x == 0) lens[b] = len + n_new;
}

// One block (4 waves) per (head, sequence).  Each wave streams every 4th row,
// keeps an online softmax (running max m, sum l, accumulator), and the four
// partial states are merged through LDS at the end.
// F8: the cache holds E4M3 codes with one fp32 scale per row (scales).
template <typename T, bool F8>
__global__ void __launch_bounds__(256) k_decode(int n_h, int d_c, int d_r, int n_q, float scale_log2,
                                                const T* __restrict__ q_lat, const T* __restrict__ q_pe,
                                                const void* __restrict__ cache, const float* __restrict__ scales,
                                                RowMap map,
                                                const int32_t* __restrict__ lens,
                                                float* __restrict__ o_lat, float* __restrict__ lse,
                                                int32_t* err_flag) {
  extern __shared__ float smem[];
  // block (h, v): head h of query token i = v % n_q of sequence b = v / n_q,
  // which sees rows 0 .. lens[b] - n_q + i of the sequence
  const int h = blockIdx.x, v = blockIdx.y;
  const int b = v / n_q, tok = v - b * n_q;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int D = d_c + d_r;
  const int all = lens[b];
  float* out = o_lat + ((size_t)v * n_h + h) * d_c;
  int bad = all < n_q || all > map.capacity(b) ? MLA_DEVERR_LENS : 0;
  const int len = all - (n_q - 1 - tok);
  // paged rows: every block the sequence uses must be a valid pool block
  if (!bad && map.paged()) {
    const int nblk = (int)(((int64_t)len + (int64_t(1) << map.shift) - 1) >> map.shift);
    int any = 0;
    for (int k = threadIdx.x; k < nblk; k += blockDim.x) any |= map.row(b, (int64_t)k << map.shift) < 0;
    if (__syncthreads_or(any)) bad = MLA_DEVERR_TABLE;
  }
  if (bad) {
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) out[c] = __builtin_nanf("");
    if (threadIdx.x == 0) {
      if (lse) lse[(size_t)v * n_h + h] = __builtin_nanf("");
      if (err_flag) atomicOr(err_flag, bad);
    }
    return;
  }
  float q[kMaxRowPerLane];
#pragma unroll
  for (int k = 0; k < kMaxRowPerLane; ++k) {
    int f = lane + 64 * k;
    float x = 0.f;
    if (f < d_c) x = ld(q_lat, ((size_t)v * n_h + h) * d_c + f);
    else if (f < D) x = ld(q_pe, ((size_t)v * n_h + h) * d_r + (f - d_c));
    q[k] = x;
  }
  float acc[kMaxLatPerLane];
#pragma unroll
  for (int k = 0; k < kMaxLatPerLane; ++k) acc[k] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j = wave; j < len; j += nw) {
    const int64_t rj = map.row(b, j);
    // element f of row rj: the stored value, or code value x row scale
    const float rs = F8 ? scales[rj] : 1.f;
    auto elem = [&](int f) -> float {
      if constexpr (F8) return __builtin_amdgcn_cvt_f32_fp8((int)((const uint8_t*)cache)[(size_t)rj * D + f], 0) * rs;
      else return ld((const T*)cache + (size_t)rj * D, f);
    };
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxRowPerLane; ++k) {
      int f = lane + 64 * k;
      if (f < D) s += q[k] * elem(f);
    }
    s = wave_sum(s) * scale_log2;
    float mn = fmaxf(m, s);
    float a = exp2f(m - mn);
    float p = exp2f(s - mn);
    l = l * a + p;
#pragma unroll
    for (int k = 0; k < kMaxLatPerLane; ++k) {
      int f = lane + 64 * k;
      if (f < d_c) acc[k] = acc[k] * a + p * elem(f);
    }
    m = mn;
  }
  // merge the waves' states
  float* sm = smem;                         // [nw]
  float* sl = smem + nw;                    // [nw]
  float* sacc = smem + 2 * nw;              // [nw][d_c]
  if (lane == 0) { sm[wave] = m; sl[wave] = l; }
#pragma unroll
  for (int k = 0; k < kMaxLatPerLane; ++k) {
    int f = lane + 64 * k;
    if (f < d_c) sacc[wave * d_c + f] = acc[k];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, sm[w]);
  float L = 0.f;
  for (int w = 0; w < nw; ++w) L += (sm[w] == -INFINITY) ? 0.f : sl[w] * exp2f(sm[w] - M);
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float acc_c = 0.f;
    for (int w = 0; w < nw; ++w)
      if (sm[w] != -INFINITY) acc_c += sacc[w * d_c + c] * exp2f(sm[w] - M);
    out[c] = acc_c / L;
  }
  if (threadIdx.x == 0 && lse) lse[(size_t)v * n_h + h] = (M + log2f(L)) * kLn2;
}

// o[b,h,v] = sum_c W_UV[h,v,c] o_lat[b,h,c]; one wave per (v-group of 4, h, b).
template <typename T>
__global__ void __launch_bounds__(64) k_uv(int n_h, int d_c, int d_v, const float* __restrict__ o_lat,
                                           const T* __restrict__ W_UV, float* __restrict__ o) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const float* x = o_lat + ((size_t)b * n_h + h) * d_c;
  for (int vi = 0; vi < 4; ++vi) {
    int v = blockIdx.x * 4 + vi;
    if (v >= d_v) break;
    const T* w = W_UV + ((size_t)h * d_v + v) * d_c;
    float acc = 0.f;
    for (int c = lane; c < d_c; c += 64) acc += ld(w, c) * x[c];
    acc = wave_sum(acc);
    if (lane == 0) o[((size_t)b * n_h + h) * d_v + v] = acc;
  }
}

}  // namespace

hipError_t launch_linear_generic(const Shape& s, int M, int N, int K, const void* X, bool x_f32,
                                 const void* W, float* Y, hipStream_t st) {
  dim3 grid(N, (M + 7) / 8);
  if (s.bf16)
    k_linear<__bf16><<<grid, 64, 0, st>>>(M, N, K, X, x_f32, (const __bf16*)W, Y);
  else
    k_linear<float><<<grid, 64, 0, st>>>(M, N, K, X, x_f32, (const float*)W, Y);
  return hipGetLastError();
}

hipError_t launch_absorb_generic(const Shape& s, int B, const void* q, bool q_f32, const void* W_UK,
                                 const int32_t* pos, void* q_lat, void* q_pe, hipStream_t st) {
  dim3 grid(s.n_h, B);
  if (s.bf16)
    k_absorb<__bf16><<<grid, 256, 0, st>>>(s.n_h, s.d_c, s.d_r, s.d_h, s.rope_base, q, q_f32,
                                           (const __bf16*)W_UK, pos, (__bf16*)q_lat, (__bf16*)q_pe);
  else
    k_absorb<float><<<grid, 256, 0, st>>>(s.n_h, s.d_c, s.d_r, s.d_h, s.rope_base, q, q_f32,
                                          (const float*)W_UK, pos, (float*)q_lat, (float*)q_pe);
  return hipGetLastError();
}

hipError_t launch_append_generic(const Shape& s, int B, int n_new, const void* c_src,
                                 size_t c_stride, const void* k_src, size_t k_stride, bool src_f32,
                                 void* cache, const RowMap& map, int32_t* lens,
                                 int32_t* err_flag, hipStream_t st) {
  if (s.bf16)
    k_append<__bf16><<<B, 256, 0, st>>>(n_new, s.d_c, s.d_r, s.rope_base, c_src, c_stride, k_src,
                                        k_stride, src_f32, (__bf16*)cache, map, lens, err_flag);
  else
    k_append<float><<<B, 256, 0, st>>>(n_new, s.d_c, s.d_r, s.rope_base, c_src, c_stride, k_src,
                                       k_stride, src_f32, (float*)cache, map, lens, err_flag);
  return hipGetLastError();
}

hipError_t launch_append_fp8(const Shape& s, int B, int n_new, const void* c_src, size_t c_stride,
                             const void* k_src, size_t k_stride, bool src_f32, void* cache, float* scales,
                             const RowMap& map, int32_t* lens, int32_t* err_flag, hipStream_t st) {
  k_append_fp8<<<B, 256, sizeof(float) * (size_t)(s.d_c + s.d_r), st>>>(
      n_new, s.d_c, s.d_r, s.rope_base, c_src, c_stride, k_src, k_stride, src_f32, (uint8_t*)cache, scales, map,
      lens, err_flag);
  return hipGetLastError();
}

hipError_t launch_decode_generic(const Shape& s, int B, int n_q, const void* q_lat, const void* q_pe,
                                 const void* cache, const float* scales, const RowMap& map,
                                 const int32_t* lens, float* o_lat, float* lse, int32_t* err_flag,
                                 hipStream_t st) {
  const int threads = 256, nw = threads / 64;
  size_t smem = sizeof(float) * (2 * nw + (size_t)nw * s.d_c);
  dim3 grid(s.n_h, B * n_q);
  float sl2 = s.scale * kLog2e;
  if (s.bf16 && scales)
    k_decode<__bf16, true><<<grid, threads, smem, st>>>(s.n_h, s.d_c, s.d_r, n_q, sl2, (const __bf16*)q_lat,
                                                        (const __bf16*)q_pe, cache, scales, map,
                                                        lens, o_lat, lse, err_flag);
  else if (s.bf16)
    k_decode<__bf16, false><<<grid, threads, smem, st>>>(s.n_h, s.d_c, s.d_r, n_q, sl2, (const __bf16*)q_lat,
                                                         (const __bf16*)q_pe, cache, nullptr, map,
                                                         lens, o_lat, lse, err_flag);
  else if (scales)
    k_decode<float, true><<<grid, threads, smem, st>>>(s.n_h, s.d_c, s.d_r, n_q, sl2, (const float*)q_lat,
                                                       (const float*)q_pe, cache, scales, map,
                                                       lens, o_lat, lse, err_flag);
  else
    k_decode<float, false><<<grid, threads, smem, st>>>(s.n_h, s.d_c, s.d_r, n_q, sl2, (const float*)q_lat,
                                                        (const float*)q_pe, cache, nullptr, map,
                                                        lens, o_lat, lse, err_flag);
  return hipGetLastError();
}

// Root-mean-square norm of the first `cols` fp32 values of each row (row
// stride `stride`), in place: x / sqrt(mean(x^2) + eps) * w, w in the storage type.
// One block of 256 per row: a sum of squares per lane, wave sums, four waves.
template <typename T>
__global__ void __launch_bounds__(256) k_rmsnorm(float* __restrict__ x, int cols, size_t stride,
                                                 const T* __restrict__ w, float eps, __bf16* __restrict__ out) {
  __shared__ float red[4];
  float* row = x + (size_t)blockIdx.x * stride;
  float ss = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) {
    const float v = row[c];
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)cols + eps);
  if (out) {
    __bf16* orow = out + (size_t)blockIdx.x * cols;
    for (int c = threadIdx.x; c < cols; c += 256) orow[c] = (__bf16)(row[c] * r * ld(w, c));
  } else {
    for (int c = threadIdx.x; c < cols; c += 256) row[c] = row[c] * r * ld(w, c);
  }
}

__global__ void __launch_bounds__(256) k_to_bf16(size_t n, const float* __restrict__ x, __bf16* __restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) y[i] = (__bf16)x[i];
}

hipError_t launch_rmsnorm(const Shape& s, float* x, int rows, int cols, size_t ld, const void* w,
                          float eps, void* out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (s.bf16)
    k_rmsnorm<__bf16><<<rows, 256, 0, st>>>(x, cols, ld, (const __bf16*)w, eps, (__bf16*)out);
  else
    k_rmsnorm<float><<<rows, 256, 0, st>>>(x, cols, ld, (const float*)w, eps, (__bf16*)out);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* x, void* y, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_to_bf16<<<(unsigned)blocks, 256, 0, st>>>(n, x, (__bf16*)y);
  return hipGetLastError();
}

hipError_t launch_uv_generic(const Shape& s, int B, const float* o_lat, const void* W_UV, float* o,
                             hipStream_t st) {
  dim3 grid((s.d_v + 3) / 4, s.n_h, B);
  if (s.bf16)
    k_uv<__bf16><<<grid, 64, 0, st>>>(s.n_h, s.d_c, s.d_v, o_lat, (const __bf16*)W_UV, o);
  else
    k_uv<float><<<grid, 64, 0, st>>>(s.n_h, s.d_c, s.d_v, o_lat, (const float*)W_UV, o);
  return hipGetLastError();
}

}  // namespace mla
