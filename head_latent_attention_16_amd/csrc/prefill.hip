// The un-absorbed ("naive") branch of MLA for many new tokens (prefill).
//
// What is computed ("MLA模型结构详解：从公式到推理代码", section "结合 DeepSeek 推理代码看
// MLA", the naive branch; worked example step 4 for the causal mask): the full
// per-head keys and values are recovered from the latent cache,
//   k_j = [W^UK[h] c_j | kR_j],   v_j = W^UV[h] c_j,
// and each new token i (at row p_i = lens[b] - n_q + i of its sequence)
// attends causally to rows 0 .. p_i:
//   o[b,i,h] = sum_{j <= p_i} softmax_j(scale [q^C; RoPE(q^R, p_i)] . k_j) v_j.
// Per (query, key) pair this costs 2 n_h (d_h + d_R + d_v) flops instead of
// the absorbed route's 2 n_h (2 d_c + d_R): the up-projection is paid once
// per key row and amortised over the new tokens.
//
// The explicit keys and values live in an fp16 workspace (11 significant
// bits: rounding them to bf16 would add an error comparable to the whole
// tolerance when a token sees few keys), so the attention runs on fp16 MFMA;
// the explicit keys, values and queries must lie within the fp16 range.
//
// Kernels (gfx950, wave64, MFMA with fp32 accumulation):
// * k_rope_table: cos and sin of each new token's rotation angles (fp64
//   angle); k_prefill rotates q^R with them as it loads the query (fp16).
// * k_upproj: KV[r, h] = [W^UK[h] c_r | W^UV[h] c_r] (fp16) for every cache
//   row r, a bf16 [rows x 512] . [512 x n_h 256] GEMM; a workgroup owns one head's 256
//   output columns for 256 rows, the 512-deep reduction in 64-wide chunks
//   double-buffered in LDS through direct global -> LDS loads.
// * k_prefill: flash attention per (sequence, head, 256 new tokens): eight
//   waves of 32 tokens; 64-key blocks of [K^C | k^R]
//   (384 B per row) and V (256 B per row) are DMA'd into three LDS stages,
//   two blocks ahead; S^T = K Q^T and
//   O^T += V^T P^T on v_mfma_f32_32x32x16_f16 (V^T fragments by transpose
//   reads) in 32-key steps, an online softmax in base 2 with the running
//   max, the causal mask on the diagonal blocks.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int PN_H = 128, PD_C = 512, PD_R = 64, PD_H = 128, PD_V = 128;
constexpr int PQK = PD_H + PD_R;          // 192 query/key width
constexpr int KVW = PD_H + PD_V;          // 256 up-projected columns per head
constexpr int CROWB = (PD_C + PD_R) * 2;  // 1152 cache row bytes

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx4v __attribute__((ext_vector_type(4)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ const char* uni_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// Direct global -> LDS, 16 bytes per lane (lane i's bytes land at M0 + 16 i);
// completion is counted by hand (s_waitcnt vmcnt) before the barrier that
// publishes the stage.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const char* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
               : "m0");
}

template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// Rotation angles of the new tokens: table[t][i] = (cos, sin)(pos_t theta_i),
// pos_t the token's row, i < d_R / 2 (fp64 angle, see rope_cos_sin).  The
// attention kernel rotates each token's q^R with them as it loads the query,
// so the 128 heads of a token share one angle computation and no rotated
// copy of the queries is written.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_rope_table(int64_t ntok, int n_q, double base,
                                                    const int32_t* __restrict__ lens, float2* __restrict__ table) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= ntok * (PD_R / 2)) return;
  const int64_t t = idx / (PD_R / 2);
  const int i = (int)(idx - t * (PD_R / 2));
  const int b = (int)(t / n_q), k = (int)(t - (int64_t)b * n_q);
  const int64_t pos = (int64_t)lens[b] - n_q + k;
  float c, sn;
  rope_cos_sin(pos < 0 ? 0 : pos, i, PD_R, base, &c, &sn);
  table[idx] = make_float2(c, sn);
}

// k^R in fp16: kr[r] = cache[r, d_c ..] (one thread per value).
__global__ void __launch_bounds__(256) k_kr_f16(int64_t rows, const __bf16* __restrict__ cache,
                                                _Float16* __restrict__ kr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * PD_R) return;
  const int64_t r = i / PD_R;
  const int c = (int)(i - r * PD_R);
  kr[i] = (_Float16)(float)cache[r * (PD_C + PD_R) + PD_C + c];
}

// ---------------------------------------------------------------------------
// Up-projection GEMM.  KV^T tile of one head: rows of the output are the 256
// weight rows (W^UK[h] then W^UV[h]), columns U_ROWS = 256 cache rows.  Wave
// w: weight rows 64 w .. +64 (two 32-row blocks) for all 256 cache rows
// (eight blocks): 16 accumulators (in the accumulation registers).  Per
// 64-wide k chunk the stage holds W [256 x 64] (32 KiB) and X [256 x 64]
// (32 KiB), rows of 128 B with the 16-byte chunk c of row r at
// c ^ ((r >> 1) & 7).  Each workgroup streams its head's 256 KiB of weights
// once per 256 rows (128 rows per workgroup: 0.91 ms at B = 4, T = 4096;
// 256 rows: 0.84 ms).
// ---------------------------------------------------------------------------
constexpr int U_ROWS = 256;                      // cache rows per workgroup
constexpr int U_KC = 64;                         // k per chunk
constexpr int U_WB = KVW * U_KC * 2;             // 32768
constexpr int U_XB = U_ROWS * U_KC * 2;          // 32768
constexpr int U_STAGE = U_WB + U_XB;             // 65536
constexpr int U_DPW = U_STAGE / 1024 / 4;        // DMAs per wave per chunk
static_assert(U_DPW * 4 * 1024 == U_STAGE, "whole DMA instructions per wave");

__device__ __forceinline__ int usw(int r) { return (r >> 1) & 7; }

__global__ void __launch_bounds__(256, 1) k_upproj(int rows, const __bf16* __restrict__ cache,
                                                   const __bf16* __restrict__ W_UK,
                                                   const __bf16* __restrict__ W_UV, _Float16* __restrict__ kv) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * U_STAGE];
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * U_ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MLA_LDS char*)lds;
  const char* wuk = (const char*)(W_UK + (size_t)h * PD_H * PD_C);
  const char* wuv = (const char*)(W_UV + (size_t)h * PD_V * PD_C);
  const char* crow = (const char*)cache;

  // DMA k of this wave for chunk kc: LDS chunk p = 64 (U_DPW wave + k) + lane
  // of the stage; p < 2048: W row p / 8, else X row (p - 2048) / 8; physical
  // 16-byte position p % 8 holds logical chunk (p % 8) ^ usw(row).
  auto dma_chunk = [&](int kc, int stage) {
#pragma unroll
    for (int k = 0; k < U_DPW; ++k) {
      const int p = 64 * (U_DPW * wave + k) + lane;
      const char* src;
      if (p < U_WB / 16) {
        const int wr = p >> 3, c = (p & 7) ^ usw(wr);
        src = (wr < PD_H ? wuk + (size_t)wr * PD_C * 2 : wuv + (size_t)(wr - PD_H) * PD_C * 2) + kc * U_KC * 2 + c * 16;
      } else {
        const int xr = (p - U_WB / 16) >> 3, c = (p & 7) ^ usw(xr);
        const int r = min(r0 + xr, rows - 1);   // rows past the end repeat the last one
        src = crow + (size_t)r * CROWB + kc * U_KC * 2 + c * 16;
      }
      dma16(lds0 + (uint32_t)(stage * U_STAGE + (U_DPW * wave + k) * 1024), src);
    }
  };

  constexpr int NJ = U_ROWS / 32;   // 32-row blocks of cache rows
  floatx16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  constexpr int NCH = PD_C / U_KC;   // 8 chunks
  dma_chunk(0, 0);
  const int n32 = lane & 31, g = lane >> 5;
  for (int kc = 0; kc < NCH; ++kc) {
    if (kc + 1 < NCH) {
      dma_chunk(kc + 1, (kc + 1) & 1);
      vm_wait_barrier<U_DPW>();   // chunk kc landed (only kc + 1 is in flight)
    } else {
      vm_wait_barrier<0>();
    }
    const MLA_LDS char* Ws = (const MLA_LDS char*)lds + (kc & 1) * U_STAGE;
    const MLA_LDS char* Xs = Ws + U_WB;
#pragma unroll
    for (int ks = 0; ks < U_KC / 16; ++ks) {
      const int c = 2 * ks + g;   // logical 16-byte chunk of this lane's 8 k values
      bf16x8 A[2], Bx[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int wr = 64 * wave + 32 * i + n32;
        A[i] = *(const MLA_LDS bf16x8*)(Ws + wr * 128 + ((c ^ usw(wr)) << 4));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int xr = 32 * j + n32;
        Bx[j] = *(const MLA_LDS bf16x8*)(Xs + xr * 128 + ((c ^ usw(xr)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], Bx[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_barrier" ::: "memory");   // the stage is refilled next
  }
  // acc[i][j]: weight rows 64 wave + 32 i + {8 (e / 4) + 4 g + e % 4}, cache
  // row 32 j + n32; four consecutive weight rows -> 8 contiguous bytes.
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = r0 + 32 * j + n32;
    if (r >= rows) continue;
    _Float16* out = kv + ((size_t)r * PN_H + h) * KVW;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        halfx4v v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (_Float16)acc[i][j][4 * q4 + e];
        *(halfx4v*)(out + 64 * wave + 32 * i + 8 * q4 + 4 * g) = v;
      }
  }
}

// ---------------------------------------------------------------------------
// Causal flash attention over the explicit keys and values.
// Key block stage: K [64 x 192] (rows of 384 B, 24 chunks; chunk c of row r at
// c ^ ((r >> 1) & 7)) then V [64 x 128] (rows of 256 B, 16 chunks; chunk c of
// row r at c ^ (4 (r & 3))).  40 KiB = 5 DMAs per wave of eight; three stages.
// ---------------------------------------------------------------------------
constexpr int F_WAVES = 8;                // waves per workgroup
constexpr int F_TB = 1;                   // 32-token blocks per wave
constexpr int F_TQ = F_WAVES * 32 * F_TB; // new tokens per workgroup (256)
constexpr int F_KB = 64;                  // keys per block
constexpr int F_NST = 3;                  // LDS stages: two blocks in flight
constexpr float F_SLACK = 8.f;            // log2 headroom of the softmax reference
constexpr float F_WMAX = 256.f;           // 2^F_SLACK: the largest weight kept
constexpr int F_KROWB = PQK * 2;          // 384
constexpr int F_VROWB = PD_V * 2;         // 256
constexpr int F_KB_BYTES = F_KB * F_KROWB;   // 24576
constexpr int F_STAGE = F_KB_BYTES + F_KB * F_VROWB;   // 40960
constexpr int F_DPW = F_STAGE / 1024 / F_WAVES;    // DMAs per wave and block
static_assert(F_DPW * F_WAVES * 1024 == F_STAGE, "whole DMA instructions per wave");

__device__ __forceinline__ int ksw(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int vsw(int r) { return 4 * (r & 3); }

struct PrefillArgs {
  const __bf16* q;          // [B, n_q, n_h, 192] (q^R not rotated)
  const float2* rope;       // [B n_q, 32] (cos, sin) of each token
  const _Float16* kr;      // [rows, 64]
  const _Float16* kv;      // [rows, n_h, 256]
  const int32_t* offsets;
  const int32_t* lens;
  float* o;                // [B, n_q, n_h, 128]
  float* lse;              // [B, n_q, n_h] or NULL
  int32_t* err_flag;
  int B, n_q, rows;
  float scale_log2;
};

// One workgroup of F_WAVES waves per compute unit (120 KiB of LDS, two waves
// per SIMD), 256 new tokens: each key block streamed into LDS serves all of
// them.  Each wave holds F_TB blocks of 32 tokens; with more than one, every
// key and value fragment read from LDS feeds F_TB MFMAs (two blocks per wave
// with four waves needs more than one wave's registers: it spilled and ran
// 3x slower).
__global__ void __launch_bounds__(64 * F_WAVES, 1) k_prefill(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[F_NST * F_STAGE];
  // Work item of this workgroup.  Workgroups are dealt to the 8 XCDs
  // round-robin in launch order; each XCD takes a contiguous run of work
  // items instead, so the token blocks of one (sequence, head), which stream
  // the same keys and values, share that XCD's L2 (B = 4, T = 4096, 128
  // tokens per workgroup: 5.9 -> 4.1 ms).  Within a (sequence, head) the
  // longest token blocks go first.
  const int nqb = gridDim.x;
  const int total = nqb * gridDim.y * gridDim.z;
  const int L = blockIdx.x + nqb * (blockIdx.y + gridDim.y * blockIdx.z);
  const int W = (total % 8 == 0) ? (L % 8) * (total / 8) + L / 8 : L;
  const int qb = nqb - 1 - W % nqb, h = (W / nqb) % gridDim.y, b = W / (nqb * gridDim.y);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, g = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MLA_LDS char*)lds;

  const int len = a.lens[b];
  const int off = a.offsets[b];
  const int cap = a.offsets[b + 1] - off;
  const int i0 = qb * F_TQ;                       // first token of the workgroup
  const int nq_wg = min(F_TQ, a.n_q - i0);        // tokens of the workgroup
  const bool valid = len >= a.n_q && len <= cap && (int64_t)off + len <= a.rows && off >= 0;
  // token block j of this wave: tokens i0 + 32 (F_TB wave + j) + n32 (the
  // column of S^T this lane holds); lanes past the workgroup's tokens take
  // its last token and store nothing
  int tok[F_TB], pos[F_TB], bfirst[F_TB];
  bool tok_ok[F_TB];
#pragma unroll
  for (int j = 0; j < F_TB; ++j) {
    const int tw = 32 * (F_TB * wave + j);
    tok[j] = i0 + tw + n32;
    tok_ok[j] = tw + n32 < nq_wg;
    pos[j] = len - a.n_q + min(tok[j], a.n_q - 1);
    bfirst[j] = len - a.n_q + i0 + min(tw, nq_wg - 1);   // the block's first position
  }
  if (!valid) {
#pragma unroll
    for (int j = 0; j < F_TB; ++j)
      if (tok_ok[j]) {
        float* orow = a.o + (((size_t)b * a.n_q + tok[j]) * PN_H + h) * PD_V;
        for (int c = g; c < PD_V; c += 2) orow[c] = __builtin_nanf("");
        if (g == 0 && a.lse) a.lse[((size_t)b * a.n_q + tok[j]) * PN_H + h] = __builtin_nanf("");
      }
    if (tid == 0 && qb == 0 && h == 0 && a.err_flag) atomicOr(a.err_flag, MLA_DEVERR_LENS);
    return;
  }
  const int p_first = len - a.n_q + i0;           // position of the workgroup's first token
  const int p_last = p_first + nq_wg - 1;
  const int nblk = (p_last + 1 + F_KB - 1) / F_KB;     // key blocks any token sees
  // the wave's last position; a wave without tokens only helps with the loads
  const bool idle = 32 * F_TB * wave >= nq_wg;
  const int wpos_last = p_first + min(32 * F_TB * wave + 32 * F_TB - 1, nq_wg - 1);

  // Q^T fragments (B operand) of block j: token n32, features 16 kk + 8 g,
  // in fp16.  Rope feature r = 16 (kk - 8) + 8 g + e pairs with r + 32: the
  // lane holds both (kk = 8 with 10, 9 with 11) and rotates them with the
  // angle of frequency r (rotate-half).
  halfx8 q[F_TB][PQK / 16];
#pragma unroll
  for (int j = 0; j < F_TB; ++j) {
    const size_t t = (size_t)b * a.n_q + min(tok[j], a.n_q - 1);
    const __bf16* qr = a.q + (t * PN_H + h) * PQK;
    bf16x8 raw[PQK / 16];
#pragma unroll
    for (int kk = 0; kk < PQK / 16; ++kk) raw[kk] = *(const bf16x8*)(qr + 16 * kk + 8 * g);
#pragma unroll
    for (int kk = 0; kk < PD_H / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) q[j][kk][e] = (_Float16)(float)raw[kk][e];
    const float2* rt = a.rope + t * (PD_R / 2);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {          // kk = 8 + hh pairs with 10 + hh
      const int kl = PD_H / 16 + hh, khi = kl + 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = rt[16 * hh + 8 * g + e];
        const float lo = (float)raw[kl][e], hi = (float)raw[khi][e];
        q[j][kl][e] = (_Float16)(lo * cs.x - hi * cs.y);
        q[j][khi][e] = (_Float16)(hi * cs.x + lo * cs.y);
      }
    }
  }

  const char* kvb = (const char*)(a.kv + (size_t)h * KVW);     // row r at kvb + r * n_h * 512
  const size_t kv_row = (size_t)PN_H * KVW * 2;
  // DMA k of this wave for key block kb: stage chunk p = 64 (F_DPW wave + k)
  // + lane; p < 1536: K row p / 24, physical chunk p % 24 holding logical
  // chunk (p % 24) ^ ksw(row) (logical < 16: K^C from kv, else k^R);
  // else V row (p - 1536) / 16, logical chunk ((p - 1536) % 16) ^ vsw(row).
  // A block whose rows all lie before the sequence's end takes each source
  // as block 0's plus kb blocks of its stride (K^C and V rows are kv_row
  // apart, k^R rows 128 B); the last block clamps its rows one by one.
  const char* src0[F_DPW];
  uint32_t bstep[F_DPW];
#pragma unroll
  for (int k = 0; k < F_DPW; ++k) {
    const int p = 64 * (F_DPW * wave + k) + lane;
    if (p < F_KB_BYTES / 16) {
      const int kr = p / 24, pc = p - kr * 24, c = pc ^ ksw(kr);
      const size_t row = (size_t)off + kr;
      src0[k] = c < 16 ? kvb + row * kv_row + c * 16 : (const char*)(a.kr + row * PD_R) + (c - 16) * 16;
      bstep[k] = c < 16 ? (uint32_t)(F_KB * kv_row) : (uint32_t)(F_KB * PD_R * 2);
    } else {
      const int pv = p - F_KB_BYTES / 16;
      const int vr = pv >> 4, c = (pv & 15) ^ vsw(vr);
      src0[k] = kvb + ((size_t)off + vr) * kv_row + PD_H * 2 + c * 16;
      bstep[k] = (uint32_t)(F_KB * kv_row);
    }
  }
  auto dma_block = [&](int kb, int stage) {
    if ((kb + 1) * F_KB <= len) {
#pragma unroll
      for (int k = 0; k < F_DPW; ++k)
        dma16(lds0 + (uint32_t)(stage * F_STAGE + (F_DPW * wave + k) * 1024), src0[k] + (size_t)kb * bstep[k]);
      return;
    }
#pragma unroll
    for (int k = 0; k < F_DPW; ++k) {
      const int p = 64 * (F_DPW * wave + k) + lane;
      const char* src;
      if (p < F_KB_BYTES / 16) {
        const int kr = p / 24, pc = p - kr * 24, c = pc ^ ksw(kr);
        const int j = min(kb * F_KB + kr, len - 1);
        const size_t row = (size_t)off + j;
        src = c < 16 ? kvb + row * kv_row + c * 16 : (const char*)(a.kr + row * PD_R) + (c - 16) * 16;
      } else {
        const int pv = p - F_KB_BYTES / 16;
        const int vr = pv >> 4, c = (pv & 15) ^ vsw(vr);
        const int j = min(kb * F_KB + vr, len - 1);
        src = kvb + ((size_t)off + j) * kv_row + PD_H * 2 + c * 16;
      }
      dma16(lds0 + (uint32_t)(stage * F_STAGE + (F_DPW * wave + k) * 1024), src);
    }
  };

  floatx16 O[F_TB][PD_V / 32];
#pragma unroll
  for (int j = 0; j < F_TB; ++j)
#pragma unroll
    for (int cb = 0; cb < PD_V / 32; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) O[j][cb][e] = 0.f;
  float m_run[F_TB], l_run[F_TB];   // running max (log2 units) and this lane's share of the sum
#pragma unroll
  for (int j = 0; j < F_TB; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }

  // transpose-read bases for V^T fragments: group G = lane / 16, i = lane % 16
  // reads 8 bytes of key row 16 kk2 + 8 rd + rr (rr = 4 g + i / 4) at value
  // columns 32 cb + 16 (G & 1) + 4 (i & 3).
  const int Gq = lane >> 4, i16 = lane & 15;
  const int rr = 4 * g + (i16 >> 2);

  // Block kb + F_NST - 1 goes into the stage of block kb - 1, which every
  // wave has finished (the barrier at the end of its step); indices past
  // the last block repeat it into the free stage, so the wait count is
  // constant.
#pragma unroll
  for (int k = 0; k < F_NST - 1; ++k) dma_block(min(k, nblk - 1), k);
  for (int kb = 0; kb < nblk; ++kb) {
    dma_block(min(kb + F_NST - 1, nblk - 1), (kb + F_NST - 1) % F_NST);
    vm_wait_barrier<(F_NST - 1) * F_DPW>();   // block kb has landed
    const MLA_LDS char* Ks = (const MLA_LDS char*)lds + (kb % F_NST) * F_STAGE;
    const MLA_LDS char* Vs = Ks + F_KB_BYTES;
    // The block's two 32-key halves are taken one after the other, each a
    // step of the online softmax for both token blocks: S^T[32 keys x 32
    // tokens] = K Q^T, the causal mask, the running max (rescaling what was
    // accumulated when it moves), the weights, O^T += V^T P^T.
#pragma unroll 1
    for (int t = 0; t < F_KB / 32; ++t) {
      const int kbase = kb * F_KB + 32 * t;
      // every token of the wave precedes these keys: all weights are 0 and
      // the running max stays, so the step changes nothing
      if (idle || kbase > wpos_last) continue;
      floatx16 S[F_TB];
#pragma unroll
      for (int j = 0; j < F_TB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[j][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < PQK / 16; ++kk) {
        const int kr = 32 * t + n32, c = 2 * kk + g;
        const halfx8 kf = *(const MLA_LDS halfx8*)(Ks + kr * F_KROWB + ((c ^ ksw(kr)) << 4));
#pragma unroll
        for (int j = 0; j < F_TB; ++j) S[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, q[j][kk], S[j], 0, 0, 0);
      }
      // weights as the PV operand: P[j][kk2] holds keys 32 t + 16 kk2 + {4 g + 0..3, 8 + 4 g + 0..3}
      halfx8 P[F_TB][2];
#pragma unroll
      for (int j = 0; j < F_TB; ++j) {
        // key of S[e] is kbase + 8 (e / 4) + 4 g + e % 4.  Off the diagonal
        // (every key of this half at or before the block's first token)
        // nothing is masked; on it, masked scores become -inf.  The max is
        // taken on the raw scores (the scale is positive) and the scale is
        // folded into the exponent's fma.
        // (pos <= len - 1, so key <= pos also keeps key < len)
        if (kbase + 31 > bfirst[j]) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kbase + 8 * (e >> 2) + 4 * g + (e & 3);
            S[j][e] = key <= pos[j] ? S[j][e] : -INFINITY;
          }
        }
        // The weights against the reference m_run, in fp32.  The reference
        // moves (rescaling what was accumulated) only when some token's
        // weight would pass 2^F_SLACK: weights that large are exact enough in
        // fp16 and their sums in fp32, and the rescale is then rare instead
        // of happening in most steps.  The check takes the max of the
        // exponentials (canonical results, one instruction per three of
        // them); the token's max score over both lane halves is formed only
        // when the reference moves, and the weights are then recomputed.
        // Every token sees key 0 in its first step: before it m_run = -inf,
        // its weight is +inf and the reference becomes finite (masked scores
        // give NaN there, which the max ignores, and 0 after it).
        float w[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) w[e] = __builtin_amdgcn_exp2f(fmaf(S[j][e], a.scale_log2, -m_run[j]));
        float wmax = fmaxf(fmaxf(w[0], w[1]), w[2]);
#pragma unroll
        for (int e = 3; e < 16; e += 2) wmax = fmaxf(wmax, fmaxf(w[e], w[e + 1]));
        if (__any(wmax > F_WMAX)) {
          float pmax = fmaxf(S[j][0], S[j][1]);
#pragma unroll
          for (int e = 2; e < 16; e += 2) pmax = fmaxf(pmax, fmaxf(S[j][e], S[j][e + 1]));
          int ln = lane;
          asm volatile("" : "+v"(ln));
          const float bmax =
              fmaxf(pmax, __int_as_float(__builtin_amdgcn_ds_bpermute(((ln & 63) ^ 32) << 2, __float_as_int(pmax))));
          const float m_new = fmaxf(m_run[j], bmax * a.scale_log2);
          const float al = __builtin_amdgcn_exp2f(m_run[j] - m_new);
          l_run[j] *= al;
#pragma unroll
          for (int cb = 0; cb < PD_V / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[j][cb][e] *= al;
          m_run[j] = m_new;
#pragma unroll
          for (int e = 0; e < 16; ++e) w[e] = __builtin_amdgcn_exp2f(fmaf(S[j][e], a.scale_log2, -m_new));
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) P[j][e >> 3][e & 7] = (_Float16)w[e];
        // l sums the same fp16 weights, two per dot instruction
        const halfx2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const halfx2 pr = {P[j][e >> 3][e & 7], P[j][e >> 3][(e & 7) + 1]};
          l_run[j] = __builtin_amdgcn_fdot2(pr, one2, l_run[j], false);
        }
      }
      // O^T[value cols x tokens] += V^T . P^T, four 32-column blocks
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
        for (int cb = 0; cb < PD_V / 32; ++cb) {
          halfx4v part[2];
#pragma unroll
          for (int rd = 0; rd < 2; ++rd) {
            const int vr = 32 * t + 16 * kk2 + 8 * rd + rr;
            const int c = 2 * (2 * cb + (Gq & 1)) + ((i16 & 3) >> 1);     // logical 16-byte chunk
            const MLA_LDS char* pa = Vs + vr * F_VROWB + ((c ^ vsw(vr)) << 4) + 8 * (i16 & 1);
            part[rd] = __builtin_bit_cast(halfx4v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)pa));
          }
          const halfx8 vf = {part[0][0], part[0][1], part[0][2], part[0][3],
                             part[1][0], part[1][1], part[1][2], part[1][3]};
#pragma unroll
          for (int j = 0; j < F_TB; ++j)
            O[j][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, P[j][kk2], O[j][cb], 0, 0, 0);
        }
    }
    asm volatile("s_barrier" ::: "memory");   // every wave is done with this stage
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the repeated last blocks land before the LDS is released
  // normalise and store: O[j][cb][e] is value column 32 cb + 8 (e / 4) + 4 g + e % 4
#pragma unroll
  for (int j = 0; j < F_TB; ++j) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const float l = l_run[j] + __int_as_float(__builtin_amdgcn_ds_bpermute(((ln & 63) ^ 32) << 2, __float_as_int(l_run[j])));
    if (!tok_ok[j]) continue;
    float* orow = a.o + (((size_t)b * a.n_q + tok[j]) * PN_H + h) * PD_V;
    const float inv = 1.f / l;
#pragma unroll
    for (int cb = 0; cb < PD_V / 32; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const floatx4 v = {O[j][cb][4 * q4] * inv, O[j][cb][4 * q4 + 1] * inv, O[j][cb][4 * q4 + 2] * inv,
                           O[j][cb][4 * q4 + 3] * inv};
        *(floatx4*)(orow + 32 * cb + 8 * q4 + 4 * g) = v;
      }
    if (g == 0 && a.lse) a.lse[((size_t)b * a.n_q + tok[j]) * PN_H + h] = (m_run[j] + log2f(l)) * kLn2;
  }
}

}  // namespace

bool prefill_v3_supported(const Shape& s) {
  return s.bf16 && s.n_h == PN_H && s.d_c == PD_C && s.d_r == PD_R && s.d_h == PD_H && s.d_v == PD_V;
}

// workspace: explicit keys and values [rows, n_h, 256] fp16, k^R [rows, 64]
// fp16, rotation table [B n_q, 32] (cos, sin) (each 256-byte aligned)
size_t prefill_v3_workspace(int B, int n_q, int64_t rows) {
  const size_t kv = (size_t)rows * PN_H * KVW * 2;
  const size_t kr = (size_t)rows * PD_R * 2;
  const size_t qr = (size_t)B * n_q * (PD_R / 2) * sizeof(float2);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(kv) + al(kr) + al(qr);
}

hipError_t launch_prefill_v3(const Shape& s, int B, int n_q, const void* q, const void* cache, int64_t rows,
                             const int32_t* offsets, const int32_t* lens, const void* W_UK, const void* W_UV,
                             float* o, float* lse, int32_t* err_flag, void* ws, hipStream_t st) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  _Float16* kv = (_Float16*)ws;
  _Float16* kr = (_Float16*)((char*)ws + al((size_t)rows * PN_H * KVW * 2));
  float2* rope = (float2*)((char*)kr + al((size_t)rows * PD_R * 2));
  const int64_t ntok = (int64_t)B * n_q;
  k_rope_table<<<(unsigned)((ntok * (PD_R / 2) + 255) / 256), 256, 0, st>>>(ntok, n_q, s.rope_base, lens, rope);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_kr_f16<<<(unsigned)((rows * PD_R + 255) / 256), 256, 0, st>>>(rows, (const __bf16*)cache, kr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_upproj<<<dim3(PN_H, (unsigned)((rows + U_ROWS - 1) / U_ROWS)), 256, 0, st>>>(
      (int)rows, (const __bf16*)cache, (const __bf16*)W_UK, (const __bf16*)W_UV, kv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillArgs a;
  a.q = (const __bf16*)q;
  a.rope = rope;
  a.kr = kr;
  a.kv = kv;
  a.offsets = offsets;
  a.lens = lens;
  a.o = o;
  a.lse = lse;
  a.err_flag = err_flag;
  a.B = B;
  a.n_q = n_q;
  a.rows = (int)rows;
  a.scale_log2 = s.scale * kLog2e;
  k_prefill<<<dim3((n_q + F_TQ - 1) / F_TQ, PN_H, B), 64 * F_WAVES, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
