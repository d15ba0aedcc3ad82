// Device-side helpers shared by the MLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> f32.  Widening is exact; narrowing rounds to nearest even
// (gfx950 lowers the conversion to v_cvt_pk_bf16_f32).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// RoPE angle for pair i of a d_r-wide rotate-half rotation at position pos:
// pos * base^(-2i/d_r), formed in double, returned as (cos, sin) in float.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int i, int d_r, double base, float* c,
                                             float* s) {
  double theta = pow(base, -2.0 * (double)i / (double)d_r);
  double ang = (double)pos * theta;
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

}  // namespace mla
