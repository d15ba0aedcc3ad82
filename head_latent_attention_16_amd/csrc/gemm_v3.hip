// Weight-streaming linear layers of the MLA layer at decode batch sizes:
//   Y[M, N] (fp32, or rounded once to bf16) = X[M, K] . W[N, K]^T, X bf16
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
// * Both operands go through LDS: per 64-wide k chunk the workgroup's W tile
//   (128 columns x 128 bytes) and X tile (128 rows x 128 bytes per plane) are
//   copied straight from global memory into LDS stages with
//   global_load_lds_dwordx4, eight lanes per 128-byte row, so every wave
//   instruction covers whole 64-byte segments (a lane loading 16 bytes of
//   its own W row would touch 64 segments per instruction and keep the
//   address unit busy for four times as long).  Several chunks are in
//   flight; completion is counted by hand with s_waitcnt vmcnt.
// * v_mfma_f32_32x32x16_bf16 with A = X (rows), B = W^T: both fragments are
//   "8 consecutive k per lane" reads from LDS; within a 64-wide k chunk, lane
//   half g holds k = 32 g + 8 j .. +8 for k-step j, in both operands.
// * Intermediate activations that feed a layer (c^Q, the query q, the
//   attention output o) are rounded to bf16 once by the kernel that produces
//   them, as everywhere in bf16 inference; a layer can write its own output
//   that way (Yb), from its epilogue or from the split sum.
// * The K splits are chosen so that all workgroups run in one round on the
//   256 compute units.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int GW = 4;             // waves per workgroup
constexpr int GT = 64 * GW;       // threads per workgroup
constexpr int GMB = 4;            // 32-row blocks per workgroup (128 rows)
constexpr int GMR = GMB * 32;     // rows per workgroup
constexpr int GNW = 32;           // output columns per wave
constexpr int GNT = GW * GNW;     // columns per workgroup
constexpr int KC = 64;            // k per chunk
constexpr int ROWB = KC * 2;      // LDS bytes per row (or column) per chunk (bf16)
constexpr int WTB = GNT * ROWB;   // W tile per chunk
constexpr int XTB = GMR * ROWB;   // X tile per chunk: 16 KiB
constexpr int KGROUP = 256;       // k granularity of the split plan
constexpr int SLOTS = 256;        // workgroups per round (one per compute unit)
constexpr int FPF = 8;            // A fragments read ahead

// Stage = [W tile | X tile]; as many stages as fit in 144 KiB of LDS.
constexpr int STAGE = WTB + XTB;
constexpr int NST = 144 * 1024 / STAGE;
constexpr int DPW = STAGE / 1024 / GW;   // DMAs per wave per chunk
static_assert(STAGE % (1024 * GW) == 0 && NST >= 3, "stage plan");

struct GemmArgs {
  const __bf16* X;      // [M][K]
  const __bf16* W1;     // rows 0 .. N1-1: W1[n][K]
  const __bf16* W2;     // rows N1 .. N-1: W2[n - N1][K] (may equal W1 + N1 K)
  float* Y;             // [M][N] fp32 output (when Yb is NULL)
  __bf16* Yb;           // [M][N] bf16 output, rounded once from the fp32 sum
  float* part;          // [splits][M][N] when splits > 1
  int M, N, N1, K;
  int kper;             // k per split, a multiple of KGROUP
  int splits;
};

// Tile rows are 128 bytes (8 chunks of 16 B) in LDS; the 16-byte chunk c of
// row r is stored at c ^ ((r >> 1) & 7), which makes the 16-lane groups of
// the fragment reads hit 16 distinct bank groups.
__device__ __forceinline__ int xsw(int r) { return (r >> 1) & 7; }

// Direct global -> LDS, 16 bytes per lane from a per-lane address (lane i's
// bytes land at M0 + 16 i).  Issued from inline asm so that the compiler does
// not add waits it cannot size; completion is counted by hand below.
__device__ __forceinline__ void gdma_16B(uint32_t lds_addr, const char* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
               : "m0");
}

template <int N>
__device__ __forceinline__ void gwait_vm_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__global__ void __launch_bounds__(GT, 1) k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[NST * STAGE];

  const int nb = blockIdx.x, sk = blockIdx.y, mc = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, g32 = lane >> 5, n32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = nb * GNT;        // the workgroup's first column
  const int m0 = mc * GMR;
  const int kb = sk * a.kper;
  const int ke = min(a.K, kb + a.kper);
  const int nch = (ke - kb) / KC;   // >= 1
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MLA_LDS char*)lds;

  // DMA plan of one chunk: instruction q = DPW wave + k fills the 1024 bytes
  // at 1024 q of the stage (the W tile, then the X tile); lane i writes the
  // 16 bytes at 16 u of its tile, u = 64 q' + i (q' = q, or q minus the W
  // tile's instructions), which hold logical chunk (u % 8) ^ xsw(r) of tile
  // row r = u / 8.  Rows past M and columns past N read the last valid row
  // (their results are not stored).
  const char* src[DPW];
#pragma unroll
  for (int k = 0; k < DPW; ++k) {
    const int q = wave * DPW + k;
    const bool wpart = q < WTB / 1024;
    const int u = 64 * (wpart ? q : q - WTB / 1024) + lane;
    const int r = u >> 3;
    const int c = (u & 7) ^ xsw(r);
    if (wpart) {
      const int n = min(nw + r, a.N - 1);
      const __bf16* row = n < a.N1 ? a.W1 + (size_t)n * a.K : a.W2 + (size_t)(n - a.N1) * a.K;
      src[k] = (const char*)(row + kb + 8 * c);
    } else {
      const int m = min(m0 + r, a.M - 1);
      src[k] = (const char*)(a.X + (size_t)m * a.K + kb + 8 * c);
    }
  }
  // DMA k of chunk t into its stage; t past the end re-copies the last chunk
  // into the free stage, so every chunk index issues exactly DPW DMAs and
  // the wait count below is constant.
  auto dma = [&](int k, int t) {
    const int q = wave * DPW + k;
    gdma_16B(lds0 + (uint32_t)((t % NST) * STAGE + q * 1024), src[k] + (size_t)min(t, nch - 1) * ROWB);
  };

  floatx16 acc[GMB];
#pragma unroll
  for (int i = 0; i < GMB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  // fragment offsets: A = X row 32 mb + n32, B = W column 32 wave + n32, both
  // at logical chunk 4 g32 + j, stored at (4 g32 + j) ^ xsw(n32)
  const int asw = xsw(n32);
  const uint32_t arow = (uint32_t)(n32 * ROWB);
  const uint32_t brow = (uint32_t)((GNW * wave + n32) * ROWB);

  constexpr int NF = 4 * GMB;   // MFMAs (= A fragments) per chunk
  constexpr int PER_J = GMB;    // MFMAs per W fragment

#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
#pragma unroll
    for (int k = 0; k < DPW; ++k) dma(k, t);

  // Chunk c: every wave has finished chunk c - 1 and chunk c has landed
  // (only chunks c + 1 .. c + NST - 2 may still be in flight); chunk
  // c + NST - 1 goes into the stage of chunk c - 1, its DMAs spread over the
  // MFMAs of chunk c.
  for (int c0 = 0; c0 < nch; c0 += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int c = c0 + s;
      if (c >= nch) break;
      gwait_vm_then_barrier<(NST - 2) * DPW>();
      const MLA_LDS char* st = (const MLA_LDS char*)lds + s * STAGE;
      auto frag_addr = [&](int f) {
        const int mb = f % GMB, j = f / PER_J;
        return st + WTB + mb * 32 * ROWB + arow + (((4 * g32 + j) ^ asw) << 4);
      };
      bf16x8 wf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[j] = *(const MLA_LDS bf16x8*)(st + brow + (((4 * g32 + j) ^ asw) << 4));
      bf16x8 fr[FPF];
#pragma unroll
      for (int f = 0; f < FPF; ++f) fr[f] = *(const MLA_LDS bf16x8*)frag_addr(f);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int mb = f % GMB, j = f / PER_J;
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % FPF], wf[j], acc[mb], 0, 0, 0);
        if (f + FPF < NF) fr[f % FPF] = *(const MLA_LDS bf16x8*)frag_addr(f + FPF);
#pragma unroll
        for (int k = 0; k < DPW; ++k)
          if (f == (k * NF) / DPW) dma(k, c + NST - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the last DMAs (past the end) must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const int n0 = nw + GNW * wave;
  if (n0 >= a.N) return;   // wave-uniform
  // D layout: lane holds column n0 + n32, rows 32 mb + 8 (e/4) + 4 g32 + e%4.
  if (a.splits == 1 && a.Yb) {
#pragma unroll
    for (int mb = 0; mb < GMB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * mb + 8 * (e >> 2) + 4 * g32 + (e & 3);
        if (m < a.M) a.Yb[(size_t)m * a.N + n0 + n32] = (__bf16)acc[mb][e];
      }
    return;
  }
  float* out = a.splits == 1 ? a.Y : a.part + (size_t)sk * a.M * a.N;
#pragma unroll
  for (int mb = 0; mb < GMB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 32 * mb + 8 * (e >> 2) + 4 * g32 + (e & 3);
      if (m < a.M) out[(size_t)m * a.N + n0 + n32] = acc[mb][e];
    }
}

// Y (or Yb, rounded once) = sum over splits of the partials, in split order.
__global__ void __launch_bounds__(256) k_split_sum(int splits, size_t n4, const floatx4* __restrict__ part,
                                                   floatx4* __restrict__ Y, bf16x4* __restrict__ Yb) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    floatx4 s = part[i];
    for (int k = 1; k < splits; ++k) {
      const floatx4 v = part[(size_t)k * n4 + i];
      s[0] += v[0];
      s[1] += v[1];
      s[2] += v[2];
      s[3] += v[3];
    }
    if (Yb)
      Yb[i] = bf16x4{(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
    else
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
  const int kgr = K / KGROUP;   // groups of k
  int splits = SLOTS / (p.nblk * p.mch);   // one round of workgroups
  int cap = kgr / 2;   // every split streams at least 2 groups (512 k)
  if (cap < 1) cap = 1;
  if (splits > cap) splits = cap;
  if (splits < 1) splits = 1;
  const int per = (kgr + splits - 1) / splits;
  p.kper = per * KGROUP;
  p.splits = (kgr + per - 1) / per;
  return p;
}

}  // namespace

bool gemm_v3_supported(int M, int N, int K) {
  return M >= 1 && N >= 32 && N % 32 == 0 && K >= KGROUP && K % KGROUP == 0;
}

// Workspace: the split partials [splits][M][N] fp32 (when splits > 1).
size_t gemm_v3_workspace(int M, int N, int K) {
  if (!gemm_v3_supported(M, N, K)) return 0;
  const Plan p = plan(M, N, K);
  return p.splits > 1 ? ((size_t)p.splits * M * N * sizeof(float) + 255) / 256 * 256 : 0;
}

hipError_t launch_gemm_v3(int M, int N, int N1, int K, const void* X, const void* W1, const void* W2,
                          float* Y, void* Yb, void* ws, hipStream_t st) {
  const Plan p = plan(M, N, K);
  GemmArgs a;
  a.X = (const __bf16*)X;
  a.W1 = (const __bf16*)W1;
  a.W2 = (const __bf16*)(W2 ? W2 : W1);
  a.Y = Y;
  a.Yb = (__bf16*)Yb;
  a.part = (float*)ws;
  a.M = M;
  a.N = N;
  a.N1 = W2 ? N1 : N;
  a.K = K;
  a.kper = p.kper;
  a.splits = p.splits;
  dim3 grid(p.nblk, p.splits, p.mch);
  k_gemm<<<grid, GT, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const size_t n4 = (size_t)M * N / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_split_sum<<<(unsigned)blocks, 256, 0, st>>>(p.splits, n4, (const floatx4*)ws, (floatx4*)Y, (bf16x4*)Yb);
  return hipGetLastError();
}

}  // namespace mla
