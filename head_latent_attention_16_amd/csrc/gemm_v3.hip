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
//   PD chunks in flight) and X fragments from LDS, read FPF MFMAs ahead.
// * Within a 64-wide k chunk, lane half g holds k = 32 g + 8 j .. +8 for
//   k-step j; A and B use the same order, so the dot products are unchanged.
// * fp32 X (an intermediate such as c^Q, or the attention output o) enters
//   the bf16 MFMA as hi + lo with hi = bf16(x), lo = bf16(x - hi): two MFMAs
//   per step, about 16 significant bits of x instead of 8.  The split is done
//   once per call by k_hilo into two bf16 planes in the workspace, not by
//   every column block that stages the same X.
// * X is loaded in whole-row 16-byte pieces (every wave instruction reads
//   full cache lines) and staged in LDS one chunk ahead.  The X and W loads
//   of the chunk PD ahead and that staging are spread over the MFMA stream
//   of the current chunk instead of stalling between chunks.
// * The K splits are chosen so that all workgroups run in one round on the
//   256 compute units.
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
constexpr int SLOTS = 256;        // workgroups per round (one per compute unit)
constexpr int FPF = 8;            // A fragments read ahead

struct GemmArgs {
  const __bf16* X;      // [NPL][M][K] bf16: X, or its hi and lo planes
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

// hi = bf16(x), lo = bf16(x - hi) of fp32 X [n4 x 4], planes [2][n4 x 4]
__global__ void __launch_bounds__(256) k_hilo(size_t n4, const floatx4* __restrict__ X, bf16x4* __restrict__ hi,
                                              bf16x4* __restrict__ lo) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const floatx4 x = X[i];
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (__bf16)x[e];
      l[e] = (__bf16)(x[e] - (float)h[e]);
    }
    hi[i] = h;
    lo[i] = l;
  }
}

template <int NPLANE>   // 1: bf16 X; 2: hi and lo planes of fp32 X
__global__ void __launch_bounds__(GT, 1) k_gemm(GemmArgs a) {
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

  // X staging, coalesced: load i of thread t covers 16 bytes at flat index
  // f = 256 i + t of a plane's chunk, so each wave instruction reads whole
  // rows: 8 per row (rows 32 i + t / 8), four per plane.
  constexpr int XPR = 8;               // 16-byte pieces per row per chunk
  const int xq = tid % XPR;            // this thread's piece within its row
  const int xrb = tid / XPR;           // its row within each group of 256 pieces
  constexpr int XRS = 256 / XPR;       // rows per load index

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
  // X staging registers, PD chunks deep: X(k) and W(k) are issued in the
  // same chunk (X first), so waiting for X(c+1) before storing it to LDS
  // never forces a newer W chunk to complete -- vmcnt completes in issue
  // order.  Piece i = 4 p + i4 is row group i4 of plane p.
  constexpr int XPIECES = 4 * NPLANE;       // 16-byte X loads per thread per chunk
  bf16x8 xb[PD][XPIECES];
  // Every global load in the main loop is unconditional (indices are clamped
  // to valid data and rows past M are zeroed when stored to LDS), so that the
  // compiler can count outstanding loads exactly.
  const size_t plane = (size_t)a.M * a.K;
  auto xrow_src = [&](int i) {
    return (size_t)(i >> 2) * plane + (size_t)min(m0 + xrb + XRS * (i & 3), a.M - 1) * a.K + kb;
  };
  auto load_x_piece = [&](int slot, int c, int i) {
    xb[slot][i] = *(const bf16x8*)(a.X + xrow_src(i) + (size_t)c * KC + 8 * xq);
  };
  auto store_x_piece = [&](int slot, int stage, int i) {
    const int r = xrb + XRS * (i & 3);
    const int off = r * XROWB + ((xq ^ xsw(r)) << 4);
    *(bf16x8*)(xs[stage][i >> 2] + off) = m0 + r < a.M ? xb[slot][i] : bf16x8{};
  };

#pragma unroll
  for (int s = 0; s < PD; ++s) {
#pragma unroll
    for (int i = 0; i < XPIECES; ++i) load_x_piece(s, min(s, nch - 1), i);
    load_w(s, min(s, nch - 1));
  }
#pragma unroll
  for (int i = 0; i < XPIECES; ++i) store_x_piece(0, 0, i);
  __syncthreads();

  // A-fragment LDS offsets for step j of block mb: row 32 mb + n32,
  // logical chunk 4 g32 + j.
  uint32_t aoff[GMB];
#pragma unroll
  for (int mb = 0; mb < GMB; ++mb) aoff[mb] = (uint32_t)((32 * mb + n32) * XROWB);
  const int asw = xsw(n32);   // (32 mb + n32) >> 1 & 7 == n32 >> 1 & 7

  constexpr int NF = 4 * NPLANE * GMB;      // MFMAs (= A fragments) per chunk
  constexpr int PER_J = NPLANE * GMB;       // MFMAs per W fragment
  constexpr int ST0 = NF / 2 - XPIECES;     // first step of the X staging
  // (steps ST0, ST0 + 2, ... stage X(c + 1); after the last chunk this
  // rewrites the idle stage with data nobody reads)

  // Chunk c: NF steps, each one MFMA and the A-fragment read FPF ahead; the
  // loads of chunk c + PD (X pieces first, then each W fragment as soon as
  // the MFMAs of chunk c are done with its register) and the staging of
  // X(c + 1) into the other LDS stage ride along in the MFMA gaps.
  // nch is a multiple of PD (K % (KC PD) == 0 and kper is a multiple of
  // KC PD), so the unrolled body has no early exit.
  for (int cb = 0; cb < nch; cb += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int c = cb + s;
      const int stage = s & 1;   // == c & 1: cb is a multiple of PD (even)
      const int cn = min(c + PD, nch - 1);
      auto frag_addr = [&](int f) {
        const int mb = f % GMB, pl = (f / GMB) % NPLANE, j = f / PER_J;
        return xs[stage][pl] + aoff[mb] + (((4 * g32 + j) ^ asw) << 4);
      };
      bf16x8 fr[FPF];
#pragma unroll
      for (int f = 0; f < FPF; ++f) fr[f] = *(const bf16x8*)frag_addr(f);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int mb = f % GMB, j = f / PER_J;
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % FPF], wf[s][j], acc[mb], 0, 0, 0);
        if (f + FPF < NF) fr[f % FPF] = *(const bf16x8*)frag_addr(f + FPF);
        if (f < XPIECES) load_x_piece(s, cn, f);
        if (f % PER_J == PER_J - 1 && j < 3)   // W fragment j of chunk c is done
          wf[s][j] = *(const bf16x8*)(wrow + (size_t)cn * KC + 8 * j);
        if (f >= ST0 && f < ST0 + 2 * XPIECES && (f - ST0) % 2 == 0)
          store_x_piece((s + 1) % PD, stage ^ 1, (f - ST0) / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      wf[s][3] = *(const bf16x8*)(wrow + (size_t)cn * KC + 24);
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
  int splits = SLOTS / (p.nblk * p.mch);   // one round of workgroups
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

// Workspace: the split partials [splits][M][N] fp32 (when splits > 1), then
// for fp32 X its hi and lo planes [2][M][K] bf16.
static size_t part_bytes(const Plan& p, int M, int N) {
  return p.splits > 1 ? ((size_t)p.splits * M * N * sizeof(float) + 255) / 256 * 256 : 0;
}

size_t gemm_v3_workspace(int M, int N, int K, bool x_f32) {
  if (!gemm_v3_supported(M, N, K)) return 0;
  const Plan p = plan(M, N, K);
  return part_bytes(p, M, N) + (x_f32 ? ((size_t)2 * M * K * sizeof(__bf16) + 255) / 256 * 256 : 0);
}

hipError_t launch_gemm_v3(int M, int N, int N1, int K, const void* X, bool x_f32, const void* W1,
                          const void* W2, float* Y, void* ws, hipStream_t st) {
  const Plan p = plan(M, N, K);
  GemmArgs a;
  a.X = (const __bf16*)X;
  if (x_f32) {
    __bf16* planes = (__bf16*)((char*)ws + part_bytes(p, M, N));
    const size_t n4 = (size_t)M * K / 4;   // K is a multiple of 256
    size_t blocks = (n4 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    k_hilo<<<(unsigned)blocks, 256, 0, st>>>(n4, (const floatx4*)X, (bf16x4*)planes,
                                              (bf16x4*)(planes + (size_t)M * K));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.X = planes;
  }
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
    k_gemm<2><<<grid, GT, 0, st>>>(a);
  else
    k_gemm<1><<<grid, GT, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const size_t n4 = (size_t)M * N / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_split_sum<<<(unsigned)blocks, 256, 0, st>>>(p.splits, n4, (const floatx4*)ws, (floatx4*)Y);
  return hipGetLastError();
}

}  // namespace mla
