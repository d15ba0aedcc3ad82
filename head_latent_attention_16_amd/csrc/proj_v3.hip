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

// cos and sin of pos * theta, theta = base^(-2i/d_r): the angle is formed
// in double and reduced modulo 2 pi in double (2 pi as a sum of two
// doubles), and the reduced angle, at most pi in magnitude, goes to
// single-precision sincos.
__device__ __forceinline__ void rope_cs_reduced(int64_t pos, double theta, float* c, float* s) {
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
  // one batch block's q_C of this head, staged once per workgroup (fp32
  // query: as bf16 hi and lo planes)
  __shared__ __attribute__((aligned(16))) char qs[QF32 ? 2 : 1][32 * ABS_QROWB];
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

  // The batch block's 32 x 128 query values are read with whole-row pieces
  // (fp32: 16 per thread; bf16: 16 per thread as two 16-byte pieces) and
  // written to LDS by stage_q (fp32 split into the hi and lo planes), where
  // every wave reads its B fragments.
  floatx4 qf[QF32 ? 4 : 1];
  bf16x8 qh[QF32 ? 1 : 2];
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
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = u * ABS_THREADS + tid, r = idx >> 4, c8 = idx & 15;   // row, 8-value piece
        const int bq = nb * 32 + r;
        qh[u] = bq < B ? *(const bf16x8*)((const __bf16*)qv + ((size_t)bq * NH + h) * QW + 8 * c8) : bf16x8{};
      }
    }
  };
  auto stage_q = [&]() {
    if constexpr (QF32) {
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
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = u * ABS_THREADS + tid, r = idx >> 4, c8 = idx & 15;
        *(bf16x8*)(qs[0] + r * ABS_QROWB + 16 * c8) = qh[u];
      }
    }
  };
  load_q(0);

  // RoPE on the decoupled part: q_pe = rotate(q^R, pos[b]), pairs 8 qt .. +8.
  // Item idx = (batch row idx / 8, pair 8 qt + idx % 8); a thread's items
  // all have pair 8 qt + tid % 8, and the loads of RP items are issued
  // before any of them is used (B = 64: 10.4 -> 10.0 us).
  {
    static_assert(ABS_THREADS % 8 == 0, "one pair per thread");
    constexpr int RP = 4;
    const int i = 8 * qt + (tid & 7);
    const double theta = exp2(-2.0 * (double)i / (double)DR * log2(rope_base));
    for (int base = 0; base < B * 8; base += RP * ABS_THREADS) {
      float lo[RP], hi[RP];
      int64_t pb[RP];
#pragma unroll
      for (int u = 0; u < RP; ++u) {
        const int idx = base + u * ABS_THREADS + tid;
        const int b = min(idx >> 3, B - 1);
        const size_t e0 = ((size_t)b * NH + h) * QW + DH;
        if constexpr (QF32) {
          lo[u] = ((const float*)qv)[e0 + i];
          hi[u] = ((const float*)qv)[e0 + DR / 2 + i];
        } else {
          lo[u] = (float)((const __bf16*)qv)[e0 + i];
          hi[u] = (float)((const __bf16*)qv)[e0 + DR / 2 + i];
        }
        pb[u] = pos[b];
      }
#pragma unroll
      for (int u = 0; u < RP; ++u) {
        const int idx = base + u * ABS_THREADS + tid;
        if (idx >= B * 8) break;
        float cs, sn;
        rope_cs_reduced(pb[u], theta, &cs, &sn);
        __bf16* out = q_pe + ((size_t)(idx >> 3) * NH + h) * DR;
        out[i] = (__bf16)(lo[u] * cs - hi[u] * sn);
        out[DR / 2 + i] = (__bf16)(hi[u] * cs + lo[u] * sn);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < ABS_WPT; ++j) {
    const int idx = j * ABS_THREADS + tid, r = idx >> 4, c = idx & 15;
    *(floatx4*)(w + r * ABS_ROWB + c * 16) = wv[j];
  }
  stage_q();
  __syncthreads();

  // Transpose-read addressing (see the decode kernel): in 16-lane group G,
  // lane i reads 8 bytes of row r0 + i/4 at columns c0 + 4 (i & 3); lane j of
  // the group then holds column c0 + j for rows r0 .. r0+3.
  const int G = lane >> 4, i16 = lane & 15;
  const int h16 = G & 1;
  const uint32_t tr_off = (uint32_t)((i16 >> 2) * ABS_ROWB + 32 * h16 + 8 * (i16 & 3));

  for (int nb = 0; nb * 32 < B; ++nb) {
    const bool more = (nb + 1) * 32 < B;
    if (more) load_q(nb + 1);   // in flight during this block's MFMAs
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
      // B fragment: batch row lane & 31, k = 16 ks + 8 g32 .. +8 (from both planes)
      const int off = (lane & 31) * ABS_QROWB + (16 * ks + 8 * g32) * 2;
      const bf16x8 bh = *(const bf16x8*)(qs[0] + off);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
      if constexpr (QF32) {
        const bf16x8 bl = *(const bf16x8*)(qs[1] + off);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);
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
    if (more) {
      __syncthreads();   // every wave is done with this block's fragments
      stage_q();
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// uv: one workgroup per (head, block of 32 batch rows).  Wave w owns the
// head's value rows 32 w .. +32 over the whole 512-long contraction, with
// its 32 x 512 block of W_UV in registers; the block's 32 o_lat rows are read
// once by the workgroup (whole rows, 4 KiB per workgroup instruction), split
// into bf16 hi and lo planes in LDS, and read by all four waves, so no
// partial sums cross waves and each o_lat byte leaves L2 once.
//   o^T[v x batch] = W_UV[h][v x c] . o_lat^T[c x batch]   (32x32x16)
// o_lat is fp32; it enters the bf16 product as hi + lo with hi = bf16(x) and
// lo = bf16(x - hi), two MFMAs per step, so the result keeps about 16
// significant bits of o_lat instead of the 8 a single bf16 rounding leaves.
// Plane rows are 1 KiB; the 16-byte chunk c of row r is stored at
// c ^ (r % 16), so 16 rows at one chunk hit 16 distinct bank groups.
// (The previous layout, four workgroups per head splitting W_UV's rows and
// each reading every o_lat row of the head, took 12.9 us at B = 64: the
// o_lat reads from L2 were four times the bytes.)
// ---------------------------------------------------------------------------
constexpr int UV_KS = DC / 16;            // 32 k-steps
constexpr int UV_PF = 4;                  // fragment steps read ahead
constexpr int UV_ROWB = DC * 2;           // 1024 bytes per plane row
constexpr int UV_PLANE = 32 * UV_ROWB;    // 32 KiB
constexpr int UV_SMALL_B = 32;   // batches up to this use two workgroups per head

template <int VW>   // waves per workgroup: value rows 32 VW (blockIdx.x % (4 / VW)) .. of head blockIdx.x / (4 / VW)
__global__ void __launch_bounds__(64 * VW) k_uv_v3(int B, const float* __restrict__ o_lat,
                                                   const __bf16* __restrict__ W_UV,
                                                   float* __restrict__ o, __bf16* __restrict__ ob) {
  constexpr int NT = 64 * VW, NL = 4096 / NT;   // threads, o_lat loads per thread
  __shared__ __attribute__((aligned(16))) char xs[2][UV_PLANE];   // [hi, lo]
  const int h = blockIdx.x / (4 / VW), b0 = 32 * blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, g32 = lane >> 5, n32 = lane & 31;
  const int wave = (blockIdx.x % (4 / VW)) * VW + (tid >> 6);   // value rows 32 wave .. +32

  // o_lat: load i of thread t is float4 number f = NT i + t of the block,
  // row f / 128 (clamped to the last batch row), columns 4 (f % 128) .. +4
  floatx4 xl[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = NT * i + tid;
    const int bq = min(b0 + (f >> 7), B - 1);
    xl[i] = *(const floatx4*)(o_lat + ((size_t)bq * NH + h) * DC + 4 * (f & 127));
  }
  // the wave's W_UV rows: lane n32 holds row 32 w + n32, k = 16 j + 8 g32 .. +8
  const __bf16* wrow = W_UV + ((size_t)h * DV + 32 * wave + n32) * DC + 8 * g32;
  bf16x8 aw[UV_KS];
#pragma unroll
  for (int j = 0; j < UV_KS; ++j) aw[j] = *(const bf16x8*)(wrow + 16 * j);

  MLA_LDS char* hp = (MLA_LDS char*)xs[0];
  MLA_LDS char* lp = (MLA_LDS char*)xs[1];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = NT * i + tid;
    const int r = f >> 7, q = f & 127;   // columns 4 q .. +4: chunk q / 2, half q % 2
    bf16x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = (__bf16)xl[i][e];
      lo[e] = (__bf16)(xl[i][e] - (float)hi[e]);
    }
    const int off = r * UV_ROWB + ((((q >> 1) ^ (r & 15)) << 4) | ((q & 1) << 3));
    *(MLA_LDS bf16x4*)(hp + off) = hi;
    *(MLA_LDS bf16x4*)(lp + off) = lo;
  }
  __syncthreads();

  floatx16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // B fragment of step j: batch row n32 of the block, k = 16 j + 8 g32 .. +8
  // (chunk 2 j + g32), hi and lo planes, read UV_PF steps ahead of their
  // MFMAs (the scheduling barriers keep that order; left to itself the
  // compiler read most fragments just before their MFMA behind a full wait)
  auto frag_off = [&](int j) { return n32 * UV_ROWB + (((2 * j + g32) ^ (n32 & 15)) << 4); };
  bf16x8 fh[UV_PF], fl[UV_PF];
#pragma unroll
  for (int j = 0; j < UV_PF; ++j) {
    fh[j] = *(const MLA_LDS bf16x8*)(hp + frag_off(j));
    fl[j] = *(const MLA_LDS bf16x8*)(lp + frag_off(j));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < UV_KS; ++j) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[j], fh[j % UV_PF], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[j], fl[j % UV_PF], acc, 0, 0, 0);
    if (j + UV_PF < UV_KS) {
      fh[j % UV_PF] = *(const MLA_LDS bf16x8*)(hp + frag_off(j + UV_PF));
      fl[j % UV_PF] = *(const MLA_LDS bf16x8*)(lp + frag_off(j + UV_PF));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane: batch row b0 + n32, value rows v = 32 w + 8 (i/4) + 4 g32 + i%4
  const int bq = b0 + n32;
  if (bq >= B) return;
  const size_t at = ((size_t)bq * NH + h) * DV + 32 * wave + 4 * g32;
  if (o) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *(floatx4*)(o + at + 8 * q4) = floatx4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
  }
  if (ob) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *(bf16x4*)(ob + at + 8 * q4) = bf16x4{(__bf16)acc[4 * q4], (__bf16)acc[4 * q4 + 1],
                                            (__bf16)acc[4 * q4 + 2], (__bf16)acc[4 * q4 + 3]};
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

hipError_t launch_uv_v3(const Shape&, int B, const float* o_lat, const void* W_UV, float* o, void* ob,
                        hipStream_t st) {
  if (B <= UV_SMALL_B)
    k_uv_v3<2><<<dim3(2 * NH, (B + 31) / 32), 128, 0, st>>>(B, o_lat, (const __bf16*)W_UV, o, (__bf16*)ob);
  else
    k_uv_v3<4><<<dim3(NH, (B + 31) / 32), 256, 0, st>>>(B, o_lat, (const __bf16*)W_UV, o, (__bf16*)ob);
  return hipGetLastError();
}

}  // namespace mla
