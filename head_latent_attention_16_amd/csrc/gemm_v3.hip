// Weight-streaming linear layers of the MLA layer at decode batch sizes:
//   Y[M, N] (fp32) = X[M, K] . W[N, K]^T
// ("MLA模型结构详解", worked example: the query path W^DQ, W^UQ, the latent
// and rope key projections W^DKV, W^KR, and the output projection W^O.)
//
// M is the decode batch (tens to a few hundred rows) while N x K is a weight
// of up to 7168 x 16384, so every weight byte is used by only M rows: the
// layer is bound by streaming W from HBM once.  Layout of the work:
// * A workgroup owns 128 output columns (32 per wave) and up to 128 rows,
//   over a range of K; several K ranges ("splits") per column block give the
//   chip enough independent streams, and a second kernel adds the split
//   partials in a fixed order (deterministic).
// * v_mfma_f32_32x32x16_bf16 with A = X (rows), B = W^T: both operands are
//   "8 consecutive k per lane", so W fragments come straight from global
//   memory into registers (64 contiguous bytes per lane per 64-wide k chunk,
//   PD chunks in flight) and X fragments from LDS.
// * Within a 64-wide k chunk, lane half g holds k = 32 g + 8 j .. +8 for
//   k-step j; A and B use the same order, so the dot products are unchanged.
// * fp32 X (an intermediate such as c^Q, or the attention output o) enters
//   the bf16 MFMA as hi + lo with hi = bf16(x), lo = bf16(x - hi): two MFMAs
//   per step, about 16 significant bits of x instead of 8.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int GT = 256;           // threads per workgroup
constexpr int GMB = 4;            // 32-row blocks per workgroup (128 rows)
constexpr int GMR = GMB * 32;     // rows per workgroup
constexpr int GNW = 32;           // output columns per wave
constexpr int GNT = 4 * GNW;      // columns per workgroup
constexpr int KC = 64;            // k per chunk
constexpr int XROWB = KC * 2;     // LDS bytes per row per chunk (bf16)
constexpr int PD = 4;             // chunks of X and W in flight per wave
constexpr int TARGET_WG = 384;

struct GemmArgs {
  const void* X;        // [M][K], bf16 or fp32
  const __bf16* W1;     // rows 0 .. N1-1: W1[n][K]
  const __bf16* W2;     // rows N1 .. N-1: W2[n - N1][K] (may equal W1 + N1 K)
  float* Y;             // [M][N] when splits == 1
  float* part;          // [splits][M][N] when splits > 1
  int M, N, N1, K;
  int kper;             // k per split, a multiple of KC
  int splits;
};

// X chunk rows are 128 bytes (8 chunks of 16 B) in LDS; the 16-byte chunk c
// of row r is stored at c ^ ((r >> 1) & 7), which makes the 16-lane groups
// of both the staging writes and the fragment reads hit 16 distinct bank
// groups.
__device__ __forceinline__ int xsw(int r) { return (r >> 1) & 7; }

template <bool XF32>
__global__ void __launch_bounds__(GT, 1) k_gemm(GemmArgs a) {
  constexpr int NPLANE = XF32 ? 2 : 1;   // hi (and lo) planes
  __shared__ __attribute__((aligned(16))) char xs[2][NPLANE][GMR * XROWB];

  const int nb = blockIdx.x, sk = blockIdx.y, mc = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, g32 = lane >> 5, n32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = nb * GNT + wave * GNW;
  const bool active = n0 < a.N;   // wave-uniform
  const int m0 = mc * GMR;
  const int kb = sk * a.kper;
  const int ke = min(a.K, kb + a.kper);
  const int nch = (ke - kb) / KC;

  // Waves past N (only in the last column block) stream row 0 and store nothing.
  const int nrow = active ? n0 + n32 : 0;
  const __bf16* wrow = (nrow < a.N1 ? a.W1 + (size_t)nrow * a.K
                                    : a.W2 + (size_t)(nrow - a.N1) * a.K) + kb + 32 * g32;

  // X staging: thread t fills row t/2, k half t&1 (32 values) of a chunk.
  const int xr = tid >> 1, xh = tid & 1;
  const bool xrow_ok = m0 + xr < a.M;
  const size_t xoff = (size_t)(xrow_ok ? m0 + xr : 0) * a.K + kb + 32 * xh;

  floatx16 acc[GMB];
#pragma unroll
  for (int i = 0; i < GMB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  bf16x8 wf[PD][4];
  auto load_w = [&](int slot, int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) wf[slot][j] = *(const bf16x8*)(wrow + (size_t)c * KC + 8 * j);
  };
  // X staging registers, PD chunks deep: X(k) and W(k) are issued together
  // (X first), so waiting for X(c+1) before storing it to LDS never forces a
  // newer W chunk to complete -- vmcnt completes in issue order.
  floatx4 xf[XF32 ? PD : 1][8];
  bf16x8 xb[XF32 ? 1 : PD][4];
  // Every global load in the main loop is unconditional (indices are clamped
  // to valid data and rows past M are zeroed when stored to LDS), so that the
  // compiler can count outstanding loads exactly.
  auto load_x = [&](int slot, int c) {
    if constexpr (XF32) {
      const float* src = (const float*)a.X + xoff + (size_t)c * KC;
#pragma unroll
      for (int i = 0; i < 8; ++i) xf[slot][i] = *(const floatx4*)(src + 4 * i);
    } else {
      const __bf16* src = (const __bf16*)a.X + xoff + (size_t)c * KC;
#pragma unroll
      for (int i = 0; i < 4; ++i) xb[slot][i] = *(const bf16x8*)(src + 8 * i);
    }
  };
  auto store_x = [&](int slot, int stage) {
    const int sw = xsw(xr);
    if constexpr (XF32) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = xrow_ok ? xf[slot][2 * q + (e >> 2)][e & 3] : 0.f;
          hi[e] = (__bf16)x;
          lo[e] = (__bf16)(x - (float)hi[e]);
        }
        const int off = xr * XROWB + (((4 * xh + q) ^ sw) << 4);
        *(bf16x8*)(xs[stage][0] + off) = hi;
        *(bf16x8*)(xs[stage][NPLANE - 1] + off) = lo;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int off = xr * XROWB + (((4 * xh + q) ^ sw) << 4);
        *(bf16x8*)(xs[stage][0] + off) = xrow_ok ? xb[slot][q] : bf16x8{};
      }
    }
  };

#pragma unroll
  for (int s = 0; s < PD; ++s) {
    load_x(s, min(s, nch - 1));
    load_w(s, min(s, nch - 1));
  }
  store_x(0, 0);
  __syncthreads();

  // A-fragment LDS offsets for step j of block mb: row 32 mb + n32,
  // logical chunk 4 g32 + j.
  uint32_t aoff[GMB];
#pragma unroll
  for (int mb = 0; mb < GMB; ++mb) aoff[mb] = (uint32_t)((32 * mb + n32) * XROWB);
  const int asw = xsw(n32);   // (32 mb + n32) >> 1 & 7 == n32 >> 1 & 7

  // nch is a multiple of PD (K % (KC PD) == 0 and kper is a multiple of
  // KC PD), so the unrolled body has no early exit.
  for (int cb = 0; cb < nch; cb += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int c = cb + s;
      const int stage = c & 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = ((4 * g32 + j) ^ asw) << 4;
#pragma unroll
        for (int mb = 0; mb < GMB; ++mb) {
          const bf16x8 xa = *(const bf16x8*)(xs[stage][0] + aoff[mb] + ch);
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, wf[s][j], acc[mb], 0, 0, 0);
          if constexpr (XF32) {
            const bf16x8 xl = *(const bf16x8*)(xs[stage][NPLANE - 1] + aoff[mb] + ch);
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, wf[s][j], acc[mb], 0, 0, 0);
          }
        }
      }
      // keep the issue order: MFMAs, then chunk c+PD's loads (X first), then
      // the staging of X(c+1)
      __builtin_amdgcn_sched_barrier(0);
      load_x(s, min(c + PD, nch - 1));
      load_w(s, min(c + PD, nch - 1));
      __builtin_amdgcn_sched_barrier(0);
      // after the last chunk this rewrites the idle stage with data nobody reads
      store_x((s + 1) % PD, stage ^ 1);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (!active) return;
  // D layout: lane holds column n0 + n32, rows 32 mb + 8 (e/4) + 4 g32 + e%4.
  float* out = a.splits == 1 ? a.Y : a.part + (size_t)sk * a.M * a.N;
#pragma unroll
  for (int mb = 0; mb < GMB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 32 * mb + 8 * (e >> 2) + 4 * g32 + (e & 3);
      if (m < a.M) out[(size_t)m * a.N + n0 + n32] = acc[mb][e];
    }
}

// Y = sum over splits of the partials, in split order.
__global__ void __launch_bounds__(256) k_split_sum(int splits, size_t n4, const floatx4* __restrict__ part,
                                                   floatx4* __restrict__ Y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    floatx4 s = part[i];
    for (int k = 1; k < splits; ++k) {
      const floatx4 v = part[(size_t)k * n4 + i];
      s[0] += v[0];
      s[1] += v[1];
      s[2] += v[2];
      s[3] += v[3];
    }
    Y[i] = s;
  }
}

struct Plan {
  int nblk, mch, kper, splits;
};

Plan plan(int M, int N, int K) {
  Plan p;
  p.nblk = (N + GNT - 1) / GNT;
  p.mch = (M + GMR - 1) / GMR;
  const int kgr = K / (KC * PD);   // groups of PD chunks
  int splits = (TARGET_WG + p.nblk * p.mch - 1) / (p.nblk * p.mch);
  int cap = kgr / 2;   // every split streams at least 2 groups (512 k)
  if (cap < 1) cap = 1;
  if (splits > cap) splits = cap;
  if (splits < 1) splits = 1;
  const int per = (kgr + splits - 1) / splits;
  p.kper = per * KC * PD;
  p.splits = (kgr + per - 1) / per;
  return p;
}

}  // namespace

bool gemm_v3_supported(int M, int N, int K) {
  return M >= 1 && N >= 32 && N % 32 == 0 && K >= KC * PD && K % (KC * PD) == 0;
}

size_t gemm_v3_workspace(int M, int N, int K) {
  if (!gemm_v3_supported(M, N, K)) return 0;
  const Plan p = plan(M, N, K);
  return p.splits > 1 ? ((size_t)p.splits * M * N * sizeof(float) + 255) / 256 * 256 : 0;
}

hipError_t launch_gemm_v3(int M, int N, int N1, int K, const void* X, bool x_f32, const void* W1,
                          const void* W2, float* Y, void* ws, hipStream_t st) {
  const Plan p = plan(M, N, K);
  GemmArgs a;
  a.X = X;
  a.W1 = (const __bf16*)W1;
  a.W2 = (const __bf16*)(W2 ? W2 : W1);
  a.Y = Y;
  a.part = (float*)ws;
  a.M = M;
  a.N = N;
  a.N1 = W2 ? N1 : N;
  a.K = K;
  a.kper = p.kper;
  a.splits = p.splits;
  dim3 grid(p.nblk, p.splits, p.mch);
  if (x_f32)
    k_gemm<true><<<grid, GT, 0, st>>>(a);
  else
    k_gemm<false><<<grid, GT, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const size_t n4 = (size_t)M * N / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_split_sum<<<(unsigned)blocks, 256, 0, st>>>(p.splits, n4, (const floatx4*)ws, (floatx4*)Y);
  return hipGetLastError();
}

}  // namespace mla
