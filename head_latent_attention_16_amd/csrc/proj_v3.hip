// Per-head projections around the latent attention, DeepSeek-V3 dims, bf16.
//
// absorb: q_lat[b,h,:] = W_UK[h]^T q^C[b,h,:]   ("MLA模型结构详解", section
//         "为什么矩阵吸收很关键": q^C . (W^UK c) = (q^C W^UK) . c), plus
//         q_pe[b,h,:] = RoPE(q^R[b,h,:], pos[b]) on the decoupled part.
// uv:     o[b,h,:] = W_UV[h] o_lat[b,h,:]        (worked example step 5).
//
// Both are batched skinny products (M = batch, 128 x 512 weight per head) whose
// cost is streaming the 16.8 MB weight once; they run on bf16 MFMA with fp32
// accumulation.  W_UK[h] is [d_h=128][d_c=512] with the contraction index d_h
// strided, so its tile is staged in LDS and read with transpose reads; W_UV[h]
// is [d_v][d_c] with the contraction index contiguous and is read directly.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int NH = 128, DH = 128, DC = 512, DR = 64, DV = 128;
constexpr int QW = DH + DR;   // per-head width of the given query [q^C | q^R]

// ---------------------------------------------------------------------------
// absorb: one workgroup per (head, quarter of the 512 latent columns).
//   q_lat^T[cols x batch] = W_UK[h]^T[cols x k] . q_C^T[k x batch]   (32x32x16)
// LDS holds W_UK[h][0:128][128 columns] with rows padded to 288 bytes so the
// 4-row x 32-byte transpose reads of a 16-lane group fall in distinct banks;
// wave w owns column block w of the quarter.  The weight and query loads are
// issued first and the workgroup's share of the RoPE (pairs 8 qt .. 8 qt + 7 of
// this head, every batch row) is computed while they are in flight.
// ---------------------------------------------------------------------------
constexpr int ABS_COLS = 128;
constexpr int ABS_ROWB = ABS_COLS * 2 + 32;   // 288
constexpr int ABS_THREADS = 256;
constexpr int ABS_WPT = DH * ABS_COLS / 8 / ABS_THREADS;   // 16-byte weight pieces per thread
constexpr int ABS_QROWB = DH * 2 + 16;                      // staged query row (bf16) + pad

// cos and sin of pos * base^(-2i/d_r): the angle is formed in double and
// reduced modulo 2 pi in double (2 pi as a sum of two doubles), and the
// reduced angle, at most pi in magnitude, goes to single-precision sincos.
__device__ __forceinline__ void rope_cs_reduced(int64_t pos, int i, int d_r, double log2_base, float* c,
                                                float* s) {
  const double theta = exp2(-2.0 * (double)i / (double)d_r * log2_base);
  const double ang = (double)pos * theta;
  const double k = rint(ang * 0.15915494309189535);   // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, ang);
  r = fma(-k, 2.4492935982947064e-16, r);
  sincosf((float)r, s, c);
}

// q is bf16, or fp32 (QF32: the query computed from the hidden state), which
// enters the bf16 product as hi + lo (two MFMAs per step).
template <bool QF32>
__global__ void __launch_bounds__(ABS_THREADS) k_absorb_v3(int B, double rope_base,
                                                           const void* __restrict__ qv,
                                                           const __bf16* __restrict__ W_UK,
                                                           const int32_t* __restrict__ pos,
                                                           __bf16* __restrict__ q_lat,
                                                           __bf16* __restrict__ q_pe) {
  __shared__ __attribute__((aligned(16))) char w[DH * ABS_ROWB];
  // fp32 query: one batch block's q_C of this head as bf16 hi and lo planes,
  // split once per workgroup instead of once per wave
  __shared__ __attribute__((aligned(16))) char qs[QF32 ? 2 : 1][QF32 ? 32 * ABS_QROWB : 16];
  const int h = blockIdx.x, qt = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g32 = lane >> 5;

  // W_UK[h][:, 128 qt .. +128]: 128 rows x 16 pieces of 16 B, into registers
  const __bf16* src = W_UK + (size_t)h * DH * DC + qt * ABS_COLS;
  floatx4 wv[ABS_WPT];
#pragma unroll
  for (int j = 0; j < ABS_WPT; ++j) {
    const int idx = j * ABS_THREADS + tid, r = idx >> 4, c = idx & 15;
    wv[j] = *(const floatx4*)(src + (size_t)r * DC + c * 8);
  }

  // B operand: q_C[bq][h][16 ks + 8 g32 .. +8] (and its low part)
  bf16x8 qb[DH / 16];
  // fp32: the batch block's 32 x 128 query values, 16 per thread, read here
  // and split into the LDS planes by stage_q (after the previous block's
  // fragment reads); bf16: the B fragments straight into registers.
  floatx4 qf[QF32 ? 4 : 1];
  auto load_q = [&](int nb) {
    if constexpr (QF32) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = u * ABS_THREADS + tid, r = idx >> 5, c4 = idx & 31;   // row, 4-float piece
        const int bq = nb * 32 + r;
        qf[u] = bq < B ? *(const floatx4*)((const float*)qv + ((size_t)bq * NH + h) * QW + 4 * c4)
                       : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
      const int bq = nb * 32 + (lane & 31);
      const bool bok = bq < B;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        const size_t e0 = ((size_t)(bok ? bq : 0) * NH + h) * QW + 16 * ks + 8 * g32;
        qb[ks] = bok ? *(const bf16x8*)((const __bf16*)qv + e0) : bf16x8{};
      }
    }
  };
  auto stage_q = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = u * ABS_THREADS + tid, r = idx >> 5, c4 = idx & 31;
      bf16x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)qf[u][e];
        lo[e] = (__bf16)(qf[u][e] - (float)hi[e]);
      }
      *(bf16x4*)(qs[0] + r * ABS_QROWB + 8 * c4) = hi;
      *(bf16x4*)(qs[QF32 ? 1 : 0] + r * ABS_QROWB + 8 * c4) = lo;
    }
  };
  load_q(0);

  // RoPE on the decoupled part: q_pe = rotate(q^R, pos[b]), pairs 8 qt .. +8.
  {
    const double log2_base = log2(rope_base);
    for (int idx = tid; idx < B * 8; idx += ABS_THREADS) {
      const int b = idx >> 3, i = 8 * qt + (idx & 7);
      const size_t e0 = ((size_t)b * NH + h) * QW + DH;
      float lo, hi;
      if constexpr (QF32) {
        lo = ((const float*)qv)[e0 + i];
        hi = ((const float*)qv)[e0 + DR / 2 + i];
      } else {
        lo = (float)((const __bf16*)qv)[e0 + i];
        hi = (float)((const __bf16*)qv)[e0 + DR / 2 + i];
      }
      float cs, sn;
      rope_cs_reduced(pos[b], i, DR, log2_base, &cs, &sn);
      __bf16* out = q_pe + ((size_t)b * NH + h) * DR;
      out[i] = (__bf16)(lo * cs - hi * sn);
      out[DR / 2 + i] = (__bf16)(hi * cs + lo * sn);
    }
  }

#pragma unroll
  for (int j = 0; j < ABS_WPT; ++j) {
    const int idx = j * ABS_THREADS + tid, r = idx >> 4, c = idx & 15;
    *(floatx4*)(w + r * ABS_ROWB + c * 16) = wv[j];
  }
  if constexpr (QF32) stage_q();
  __syncthreads();

  // Transpose-read addressing (see the decode kernel): in 16-lane group G,
  // lane i reads 8 bytes of row r0 + i/4 at columns c0 + 4 (i & 3); lane j of
  // the group then holds column c0 + j for rows r0 .. r0+3.
  const int G = lane >> 4, i16 = lane & 15;
  const int h16 = G & 1;
  const uint32_t tr_off = (uint32_t)((i16 >> 2) * ABS_ROWB + 32 * h16 + 8 * (i16 & 3));

  for (int nb = 0; nb * 32 < B; ++nb) {
    if (nb > 0) {
      load_q(nb);
      if constexpr (QF32) {
        __syncthreads();   // every wave is done with the previous block's planes
        stage_q();
        __syncthreads();
      }
    }
    const int bq = nb * 32 + (lane & 31);
    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      const char* p = w + (16 * ks + 8 * g32) * ABS_ROWB + 64 * wave + tr_off;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(MLA_LDS char*)p);
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(MLA_LDS char*)(p + 4 * ABS_ROWB));
      const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if constexpr (QF32) {
        // B fragment: batch row lane & 31, k = 16 ks + 8 g32 .. +8, from both planes
        const int off = (lane & 31) * ABS_QROWB + (16 * ks + 8 * g32) * 2;
        const bf16x8 bh = *(const bf16x8*)(qs[0] + off);
        const bf16x8 bl = *(const bf16x8*)(qs[1] + off);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], acc, 0, 0, 0);
      }
    }
    // lane: batch bq, columns 8 (i/4) + 4 g32 + i%4 of the block
    if (bq < B) {
      __bf16* dst = q_lat + ((size_t)bq * NH + h) * DC + qt * ABS_COLS + 32 * wave + 4 * g32;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const bf16x4 v = {(__bf16)acc[4 * q4 + 0], (__bf16)acc[4 * q4 + 1],
                          (__bf16)acc[4 * q4 + 2], (__bf16)acc[4 * q4 + 3]};
        *(bf16x4*)(dst + 8 * q4) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// uv: one workgroup per (head, 32-row block of W_UV); it keeps its 32 x 512
// weight block in registers and walks the batch in blocks of 32.  The four
// waves split the 512-long contraction and add their partial sums through LDS.
//   o^T[v x batch] = W_UV[h][v x c] . o_lat^T[c x batch]   (32x32x16)
// o_lat is fp32; it enters the bf16 product as hi + lo with hi = bf16(x) and
// lo = bf16(x - hi), two MFMAs per step, so the result keeps about 16
// significant bits of o_lat instead of the 8 a single bf16 rounding leaves.
// ---------------------------------------------------------------------------
constexpr int UV_KS = DC / 16 / 4;   // 8 k-steps per wave

__device__ __forceinline__ void split_bf16(const floatx4& x0, const floatx4& x1, bf16x8& hi,
                                           bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (__bf16)x0[i];
    hi[4 + i] = (__bf16)x1[i];
    lo[i] = (__bf16)(x0[i] - (float)hi[i]);
    lo[4 + i] = (__bf16)(x1[i] - (float)hi[4 + i]);
  }
}

__global__ void __launch_bounds__(256) k_uv_v3(int B, const float* __restrict__ o_lat,
                                               const __bf16* __restrict__ W_UV,
                                               float* __restrict__ o) {
  __shared__ floatx16 red[3][64];
  const int h = blockIdx.x, vb = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g32 = lane >> 5;
  const int v = 32 * vb + (lane & 31);
  const __bf16* wrow = W_UV + ((size_t)h * DV + v) * DC;
  bf16x8 aw[UV_KS];
#pragma unroll
  for (int j = 0; j < UV_KS; ++j) aw[j] = *(const bf16x8*)(wrow + 16 * (wave * UV_KS + j) + 8 * g32);

  for (int nb = 0; nb * 32 < B; ++nb) {
    const int bq = 32 * nb + (lane & 31);
    const bool bok = bq < B;
    const float* orow = o_lat + ((size_t)(bok ? bq : 0) * NH + h) * DC;
    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < UV_KS; ++j) {
      const int c = 16 * (wave * UV_KS + j) + 8 * g32;
      floatx4 x0 = *(const floatx4*)(orow + c);
      floatx4 x1 = *(const floatx4*)(orow + c + 4);
      if (!bok) x0 = x1 = floatx4{0.f, 0.f, 0.f, 0.f};
      bf16x8 hi, lo;
      split_bf16(x0, x1, hi, lo);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[j], hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[j], lo, acc, 0, 0, 0);
    }
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w2 = 0; w2 < 3; ++w2) {
        const floatx16 r = red[w2][lane];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += r[i];
      }
      // lane: batch bq, rows v = 32 vb + 8 (i/4) + 4 g32 + i%4
      if (bok) {
        float* dst = o + ((size_t)bq * NH + h) * DV + 32 * vb + 4 * g32;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(floatx4*)(dst + 8 * q4) =
              floatx4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
      }
    }
    __syncthreads();
  }
}

}  // namespace

bool proj_v3_supported(const Shape& s) {
  return s.bf16 && s.n_h == NH && s.d_c == DC && s.d_r == DR && s.d_h == DH && s.d_v == DV;
}

hipError_t launch_absorb_v3(const Shape& s, int B, const void* q, bool q_f32, const void* W_UK,
                            const int32_t* pos, void* q_lat, void* q_pe, hipStream_t st) {
  const dim3 grid(NH, DC / ABS_COLS);
  if (q_f32)
    k_absorb_v3<true><<<grid, ABS_THREADS, 0, st>>>(B, s.rope_base, q, (const __bf16*)W_UK, pos,
                                                    (__bf16*)q_lat, (__bf16*)q_pe);
  else
    k_absorb_v3<false><<<grid, ABS_THREADS, 0, st>>>(B, s.rope_base, q, (const __bf16*)W_UK, pos,
                                                     (__bf16*)q_lat, (__bf16*)q_pe);
  return hipGetLastError();
}

hipError_t launch_uv_v3(const Shape&, int B, const float* o_lat, const void* W_UV, float* o,
                        hipStream_t st) {
  k_uv_v3<<<dim3(NH, DV / 32), 256, 0, st>>>(B, o_lat, (const __bf16*)W_UV, o);
  return hipGetLastError();
}

}  // namespace mla
