// Latent-space MLA decode attention for DeepSeek-V3 dims on gfx950.
//
// What is computed ("MLA模型结构详解：从公式到推理代码", worked example steps 4-5):
//   s_j   = scale * (q_lat[h] . c_j + q_pe[h] . kR_j)          per head h, row j
//   o_lat = sum_j softmax_j(s) c_j,  lse = log sum_j exp(s_j)
// over the rows [c_j | kR_j] (512 + 64 bf16) of each sequence's cache region.
//
// Design (MI355X):
// * The cache is read exactly once.  A workgroup owns a contiguous range of
//   cache rows and ALL 128 heads: every 32-row tile is DMA'd from HBM into LDS
//   once (global_load_lds_dwordx4, 16 B per lane) and then feeds both
//   contractions of all four waves: S^T = K . Q^T (QK, 576-deep) and
//   O^T += C^T . P^T (PV, over the tile's 32 rows, first 512 columns).
// * Four waves, one per SIMD; wave w owns heads 32w..32w+31.  Its Q
//   (32 heads x 576 bf16) lives in 144 VGPRs and its output accumulator O^T
//   (512 cols x 32 heads fp32) in 256 accumulation registers.  Each LDS byte
//   of a tile is read by four waves (not eight): LDS read bandwidth, not the
//   matrix cores, is the scarcer resource for these access patterns.
// * Both contractions use v_mfma_f32_32x32x16_bf16.  QK reads row-major
//   16-byte fragments; PV needs 8 rows of one column per lane and gets them
//   with ds_read_b64_tr_b16 transpose reads from the same row-major tile.
//   The PV reduction order over rows is permuted to match the accumulator
//   layout of S, so P goes from the QK result to the PV operand in registers.
// * LDS rows are 1152 B with 16-byte chunks XOR-swizzled per row so that the
//   row-strided reads of both contractions are free of bank conflicts.
// * Four LDS stages (144 KiB): while tile i is used, tiles i+1..i+3 are in
//   flight.
// * Softmax in base 2 against a per-piece reference max fixed by the piece's
//   first tile: later scores may exceed it (p up to 2^64 stays far from fp32
//   overflow), so the accumulator is never rescaled inside the loop -- the
//   accumulators stay in AGPRs.  The final normalisation uses the same
//   reference, so the result is exact.  If a later score exceeds the
//   reference by more than 2^64 the piece is flagged and the combine kernel
//   recomputes that sequence with a plain online-softmax loop.
// * Split-T: the rows of the whole batch are divided over G workgroups (one
//   per CU) by cost -- each sequence start that would fall inside a range is
//   charged a fixed setup cost, and without such starts the split is the
//   even one; a workgroup's range may cross sequence boundaries and emits one
//   partial (O, m, l) per sequence piece; a combine kernel merges the pieces
//   of each sequence by log-sum-exp.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int NH = 128;
constexpr int DC = 512;
constexpr int DR = 64;
constexpr int DK = DC + DR;            // 576
constexpr int ROWB = DK * 2;           // 1152 bytes per cache row
constexpr int CHUNKS = ROWB / 16;      // 72
constexpr int TILE = 32;               // rows per tile
constexpr int TILEB = TILE * ROWB;     // 36864 bytes
constexpr int NSTAGE = 4;
constexpr int WAVES = 4;                              // one per SIMD
constexpr int HPW = NH / WAVES;                       // 32 heads per wave
constexpr int THREADS = WAVES * 64;
constexpr int DMA_PER_TILE = TILEB / 1024;            // 36 wave-instructions
constexpr int DMA_PER_WAVE = DMA_PER_TILE / WAVES;    // 9
constexpr int KSTEPS = DK / 16;                       // 36 k-steps of 16 features
constexpr int QK_PF = 6;                              // QK fragments in flight
constexpr int PV_PF = 4;                              // PV fragment pairs in flight
constexpr float OVF_TH = 64.0f;                       // log2 units
constexpr int MIN_ROWS_PER_WG = 256;
// Batches up to SPL_MAXB sequences are scanned inside the split kernel (the
// prefix sits in LDS next to the stages); larger ones by a scan kernel.
constexpr int SPL_MAXB = 1024;
constexpr int SPL_PER = SPL_MAXB / THREADS;           // sequences per lane

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
// Largest |O / l| a partial may carry in fp16 (max finite 65504); a piece
// above it is flagged and its sequence recomputed by the fallback.
constexpr float PART_MAX = 65000.0f;


// 8-bit cache rows (E4M3 codes, one power-of-two scale per row, stored as
// fp32): a 32-row tile is 18 KiB of codes plus 128 bytes of scales.  Each
// wave issues five DMAs per tile: waves 0-2 five 1 KiB code chunks each,
// wave 3 the last three chunks, the scales (one dword per lane) and a repeat
// of the last chunk, so that every wave waits for the same count.  The codes
// stay 8-bit in LDS: QK reads 16-byte fragments (two MFMAs' worth) and PV
// 8-bit transpose fragments straight into registers and converts them there
// (QK with its row's scale; for PV the scale is folded into the weights), so
// a tile costs half the LDS reads of the 16-bit path and no converted copy.
constexpr int F8_ROWB = DK;                       // 576 bytes per row
constexpr int F8_CHUNKS = F8_ROWB / 16;           // 36 chunks of 16 bytes
constexpr int F8_TILEB = TILE * F8_ROWB;          // 18432
constexpr int F8_STAGE = F8_TILEB + 256;          // codes + scale area
constexpr int F8_DPW = 5;
constexpr int QK_PF8 = 4;                         // 16-byte QK fragments in flight
constexpr int PV_PF8 = 6;                         // PV transpose fragments in flight
static_assert(F8_TILEB / 1024 == 18 && NSTAGE * F8_STAGE <= NSTAGE * TILEB, "8-bit tile layout");

static_assert(DMA_PER_TILE * 1024 == TILEB, "tile must be whole KiB");
static_assert(DMA_PER_WAVE * WAVES == DMA_PER_TILE, "DMA split over the waves");

// Partial record of one (workgroup, sequence) piece.
struct PartialLayout {
  size_t o_off;    // fp16 [slots][NH / 32][DC / 32][2 KiB] O / l of the piece, lane order
  size_t ml_off;   // float [slots][NH][2]   (m in log2 units, l)
  size_t pre_off;  // int64 [B + 1] prefix of valid lengths (scan kernel path)
  size_t flag_off; // int32 [slots][WAVES] the piece needs the fallback recompute
  size_t rec_off;  // WgRec [G] each workgroup's row range and first sequence
  size_t si_off;   // int4 [B] first range holding the sequence, ranges, valid length
  size_t cnt_off;  // int32 [B + 1] charged sequence starts before b (scan kernel path)
  size_t bytes;
};

// A split workgroup's share: rows [start, end) of the concatenated valid
// lengths, starting in sequence b.  Written by the scan kernel so that the
// split kernel needs one load instead of a chain of dependent ones.
struct WgRec {
  int64_t start, end;            // rows [start, end) of the concatenated lengths
  int64_t seq_begin, seq_end;    // prefix[b], prefix[b + 1] of its first sequence
  int32_t b, off_b;              // that sequence and its cache offset
  int32_t pad[2];
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline PartialLayout partial_layout(int B, int G) {
  PartialLayout L;
  size_t slots = (size_t)G + (size_t)B;   // slot = g + b  <  G + B - 1
  L.pre_off = 0;
  L.flag_off = align256(sizeof(int64_t) * (B + 1));
  L.o_off = L.flag_off + align256(sizeof(int32_t) * WAVES * slots);
  L.ml_off = L.o_off + align256(slots * NH * DC * sizeof(_Float16));
  L.rec_off = L.ml_off + align256(slots * NH * 2 * sizeof(float));
  L.si_off = L.rec_off + align256(sizeof(WgRec) * (size_t)G);
  L.cnt_off = L.si_off + align256(sizeof(int4) * (size_t)B);
  L.bytes = L.cnt_off + align256(sizeof(int32_t) * ((size_t)B + 1));
  return L;
}

// Ranges: workgroup g owns positions [floor(g n / G), floor((g + 1) n / G))
// of a line of n positions.  All quantities are integers below 2^52, held
// exactly in fp64; quotients come from a reciprocal and are corrected to the
// exact floor by one comparison each way (the estimate is off by at most one).
__device__ __forceinline__ double floor_q(double x, double d, double inv_d) {
  double q = floor(x * inv_d);
  if (q * d > x) q -= 1.0;
  else if ((q + 1.0) * d <= x) q += 1.0;
  return q;
}

struct Line {
  double n, G, inv_n, inv_G;
  int Gi;
  __device__ Line(int64_t n_, int G_)
      : n((double)n_), G((double)G_), inv_n(1.0 / (double)n_), inv_G(1.0 / (double)G_), Gi(G_) {}
  __device__ int64_t start(int g) const { return (int64_t)floor_q((double)g * n, G, inv_G); }
  // the range holding position p (0 <= p < n): the largest g with
  // start(g) <= p, i.e. g n < (p + 1) G
  __device__ int range_of(int64_t p) const {
    const int g = (int)floor_q(((double)p + 1.0) * G - 1.0, n, inv_n);
    return g < Gi - 1 ? g : Gi - 1;
  }
};

// Cost-balanced ranges.  A workgroup pays a fixed setup for every piece it
// processes (query load, pipeline fill, partial store: about SEG_ROWS rows
// of loop time).  Under the plain even split of the rows, a sequence start
// strictly inside a range adds a piece to that range; each such start is
// charged SEG_ROWS virtual rows placed just before the sequence's first real
// row, and the virtual line (rows plus charges) is split evenly instead.
// Sequence b then spans [V_b - SEG_ROWS f_b, V_b + len_b) of the virtual
// line, V_b = prefix[b] + SEG_ROWS c_b, with f_b its charge flag and c_b the
// number of charged starts up to and including b.  When every sequence start
// falls on a range boundary (equal lengths) nothing is charged and the split
// is the plain one.
constexpr int64_t SEG_ROWS = 224;

// Whether the plain split of the rows puts the sequence start p0 strictly
// inside a range.
__device__ __forceinline__ bool interior_start(int64_t p0, const Line& rows) {
  if (p0 <= 0) return false;
  const double gs = floor_q((double)p0 * rows.G + rows.n - 1.0, rows.n, rows.inv_n);   // ceil(p0 G / n)
  return !(gs < rows.G && rows.start((int)gs) == p0);
}

// What the combine needs of a valid sequence whose real rows sit at virtual
// [vb, vb + len): the first range holding it, how many ranges it spans, and
// its length (0: invalid, the result is NaN).
__device__ __forceinline__ int4 seq_info(int64_t vb, int64_t len, const Line& vline) {
  if (len <= 0) return make_int4(0, 0, 0, 0);
  const int lo = vline.range_of(vb);
  return make_int4(lo, vline.range_of(vb + len - 1) - lo + 1, (int)len, 0);
}

// ---------------------------------------------------------------------------
// Scheduler: validate lengths, prefix-sum the valid ones (invalid -> 0).
// ---------------------------------------------------------------------------
// Several new tokens per step: query token i < n_q of sequence b is handled as
// sequence v = b n_q + i with its own queries and outputs.  The step's tokens
// are the last n_q of the lens[b] cached rows, and token i sees rows
// 0 .. lens[b] - n_q + i (causal mask).  Sequence b is valid when
// n_q <= lens[b] <= offsets[b+1] - offsets[b]; n_q = 1 is the plain decode.
__device__ __forceinline__ int seq_of(int v, int n_q) { return n_q == 1 ? v : v / n_q; }

// Rows seen by sequence v (>= 1), or 0 if its sequence is invalid.
__device__ __forceinline__ int vseq_len(const int32_t* lens, const RowMap& map, int v, int n_q) {
  const int b = seq_of(v, n_q);
  const int len = lens[b];
  return len >= n_q && (int64_t)len <= map.capacity(b) ? len - (n_q - 1 - (v - b * n_q)) : 0;
}

constexpr int SCHED_THREADS = 1024;
constexpr int SCHED_PER = 4;
constexpr int SCHED_LDS_B = 4096;   // prefix kept in LDS up to this many sequences

// One workgroup of 1024 threads, four sequences per thread per chunk.
// (1) Inclusive scan of the valid lengths (wave scans, then a scan of the 16
// wave totals), written to prefix[] and, for B up to SCHED_LDS_B, to LDS.
// (2) The same scan of the charge flags of the sequence starts (exclusive
// counts in cnt[]).  (3) One lane per range g: its virtual bounds, mapped to
// rows through the sequence whose virtual span holds them (binary search).
// (4) One lane per sequence: the first range holding it and how many ranges
// it spans.
__device__ __forceinline__ int64_t block_scan_1024(int64_t tsum, int64_t* wsum, int lane, int wave,
                                                   int64_t& chunk_total) {
  int64_t x = tsum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int64_t w = lane < SCHED_THREADS / 64 ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < SCHED_THREADS / 64; o <<= 1) {
      const int64_t y = __shfl_up(w, o, 64);
      if (lane >= o) w += y;
    }
    if (lane < SCHED_THREADS / 64) wsum[lane] = w;   // inclusive over waves
  }
  __syncthreads();
  const int64_t excl = (wave > 0 ? wsum[wave - 1] : 0) + x - tsum;
  chunk_total = wsum[SCHED_THREADS / 64 - 1];
  __syncthreads();   // wsum is reused by the next chunk
  return excl;
}

__global__ void __launch_bounds__(SCHED_THREADS) k_sched(int B, int n_q, int G,
                                                         RowMap map,
                                                         const int32_t* __restrict__ lens,
                                                         int64_t* __restrict__ prefix,
                                                         int32_t* __restrict__ cnt,
                                                         WgRec* __restrict__ rec,
                                                         int4* __restrict__ seqinfo, int32_t* err_flag) {
  __shared__ int64_t wsum[SCHED_THREADS / 64];
  __shared__ int64_t s_pre[SCHED_LDS_B + 1];
  __shared__ int32_t s_cnt[SCHED_LDS_B + 1];
  const bool in_lds = B <= SCHED_LDS_B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    prefix[0] = 0;
    s_pre[0] = 0;
    cnt[0] = 0;
    s_cnt[0] = 0;
  }
  int64_t carry = 0;
  for (int base = 0; base < B; base += SCHED_THREADS * SCHED_PER) {
    int64_t v[SCHED_PER];
    int64_t tsum = 0;
#pragma unroll
    for (int j = 0; j < SCHED_PER; ++j) {
      const int b = base + SCHED_PER * tid + j;
      v[j] = 0;
      if (b < B) {
        const int len = vseq_len(lens, map, b, n_q);
        if (len > 0)
          v[j] = len;
        else if (err_flag)
          atomicOr(err_flag, MLA_DEVERR_LENS);
      }
      tsum += v[j];
    }
    int64_t ct;
    int64_t run = carry + block_scan_1024(tsum, wsum, lane, wave, ct);
#pragma unroll
    for (int j = 0; j < SCHED_PER; ++j) {
      const int b = base + SCHED_PER * tid + j;
      run += v[j];
      if (b < B) {
        prefix[b + 1] = run;
        if (in_lds) s_pre[b + 1] = run;
      }
    }
    carry += ct;
  }
  const int64_t total = carry;
  if (total <= 0) {   // no valid sequence: the combine writes NaN everywhere
    for (int g = tid; g < G; g += SCHED_THREADS) {
      WgRec r = {};
      rec[g] = r;
    }
    for (int b = tid; b < B; b += SCHED_THREADS) seqinfo[b] = make_int4(0, 0, 0, 0);
    return;
  }
  __syncthreads();   // prefix[] written by every lane
  auto pre = [&](int i) -> int64_t { return in_lds ? s_pre[i] : prefix[i]; };
  const Line rows_line(total, G);
  // charged starts: exclusive counts cnt[b], cnt[B] = all of them
  int64_t fcarry = 0;
  for (int base = 0; base < B; base += SCHED_THREADS * SCHED_PER) {
    int f[SCHED_PER];
    int64_t fsum = 0;
#pragma unroll
    for (int j = 0; j < SCHED_PER; ++j) {
      const int b = base + SCHED_PER * tid + j;
      f[j] = b < B && pre(b + 1) > pre(b) && interior_start(pre(b), rows_line) ? 1 : 0;
      fsum += f[j];
    }
    int64_t ct;
    int64_t run = fcarry + block_scan_1024(fsum, wsum, lane, wave, ct);
#pragma unroll
    for (int j = 0; j < SCHED_PER; ++j) {
      const int b = base + SCHED_PER * tid + j;
      run += f[j];
      if (b < B) {
        cnt[b + 1] = (int32_t)run;   // charged starts among 0 .. b
        if (in_lds) s_cnt[b + 1] = (int32_t)run;
      }
    }
    fcarry += ct;
  }
  __syncthreads();
  auto cnt_of = [&](int i) -> int64_t { return in_lds ? s_cnt[i] : cnt[i]; };
  const int64_t tv = total + SEG_ROWS * fcarry;
  const Line vline(tv, G);
  // virtual span of sequence b starts at prefix[b] + SEG_ROWS cnt[b] (the
  // charge, if any, comes first); its rows start at V_b = prefix[b] + SEG_ROWS cnt[b + 1]
  auto span_start = [&](int b) -> int64_t { return pre(b) + SEG_ROWS * cnt_of(b); };
  auto to_row = [&](int64_t vpos) -> int64_t {
    if (vpos >= tv) return total;
    int lo = 0, hi = B - 1;   // largest b with span_start(b) <= vpos: a valid sequence
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (span_start(mid) <= vpos) lo = mid;
      else hi = mid - 1;
    }
    const int64_t vb = pre(lo) + SEG_ROWS * cnt_of(lo + 1);
    return pre(lo) + (vpos > vb ? vpos - vb : 0);
  };
  for (int g = tid; g < G; g += SCHED_THREADS) {
    const int64_t start = to_row(vline.start(g));
    // the sequence holding row start (start < total: a charge is always
    // followed by its sequence's rows)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre(mid) <= start) lo = mid;
      else hi = mid - 1;
    }
    WgRec r;
    r.start = start;
    r.end = to_row(vline.start(g + 1));
    r.seq_begin = pre(lo);
    r.seq_end = pre(lo + 1);
    r.b = lo;
    r.off_b = map.paged() ? 0 : map.offsets[seq_of(lo, n_q)];
    r.pad[0] = r.pad[1] = 0;
    rec[g] = r;
  }
  for (int b = tid; b < B; b += SCHED_THREADS)
    seqinfo[b] = seq_info(pre(b) + SEG_ROWS * cnt_of(b + 1), pre(b + 1) - pre(b), vline);
}

// ---------------------------------------------------------------------------
// Split kernel.
// ---------------------------------------------------------------------------
struct SplitArgs {
  const WgRec* rec;      // scan-kernel path only
  const int32_t* lens;   // in-kernel scan path only
  int32_t* err_flag;
  int4* seqinfo;         // written by the in-kernel scan path
  int32_t* flags;        // [slots][WAVES]
  float* o_lat;   // a sequence handled whole by one workgroup is written here
  float* lse;
  const __bf16* q_lat;
  const __bf16* q_pe;
  const char* cache;     // the cache, or the block pool (paged), or 8-bit codes
  const float* scales;   // 8-bit cache: one scale per row
  RowMap map;
  const int64_t* prefix;
  _Float16* part_o;
  float* part_ml;
  int B;     // sequences as the kernels see them: one per query token
  int n_q;   // query tokens per sequence of the caller
  int G;
  float scale_log2;
};

// Wave-uniform values read from LDS or memory arrive in vector registers;
// these move them to scalar registers so they do not occupy VGPRs.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uniform_i32(int v) { return (int)__builtin_amdgcn_readfirstlane((uint32_t)v); }

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// The same DMA from a per-lane 64-bit address.
__device__ __forceinline__ void dma_16B_at(uint32_t lds_addr, const char* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
               : "m0");
}

__device__ __forceinline__ void dma_16B(uint32_t lds_addr, uint32_t voff, const char* base) {
  // Direct global -> LDS: lane i's 16 bytes land at M0 + 16 i.  Issued from
  // inline asm so that the compiler does not add a conservative vmcnt(0)
  // before every LDS read (it cannot see which stage the DMA targets);
  // completion is tracked by hand with s_waitcnt vmcnt before the barrier.
  // No "memory" clobber: the target stage is never read between a DMA and
  // the barrier asm (itself a compiler memory barrier) that precedes its
  // first use, and without it LDS reads may be scheduled across the DMA.
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(uniform_ptr(base))
               : "m0");
}

// One int32 of wave-uniform address through the scalar unit, waited for in
// the same statement (vector loads would disturb the hand-counted vmcnt of
// the tile DMAs).  Used only where no LDS read is in flight.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(v)
               : "s"(uniform_ptr((const char*)p))
               : "memory");
  return v;
}

// Direct global -> LDS of one dword per lane (lane i's 4 bytes land at M0 + 4 i).
__device__ __forceinline__ void dma_4B_at(uint32_t lds_addr, const char* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
               : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier_all_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The QK accumulator S is kept in VGPRs with MFMAs written as asm: the
// builtin form puts every accumulator in AGPRs, and with the 256-register
// O accumulator there S would displace an O block and be copied back and
// forth every tile.  Hazards the compiler cannot see in asm are covered by
// construction: the first MFMA takes srcC = 0 (no VALU-written input), a
// chain only accumulates into the same registers (forwarded by the
// hardware), and mfma_drain's 24 wait states precede any other use of S.
// Value of lane ^ 32 (the other half of the wave), with the lane index
// taken opaque so that the compiler does not keep the permute address live
// across the kernel.
__device__ __forceinline__ float swap_halves(float v, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  ln &= 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute((ln ^ 32) << 2, __float_as_int(v)));
}

// max of three floats as one instruction (fmaxf chains would add a
// canonicalising max per operand)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ void mfma_first(floatx16& S, const bf16x8& A, const bf16x8& B) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(S) : "v"(A), "v"(B));
}
// The same, for an A operand converted by VALU instructions just before: a
// VALU write of a VGPR that an MFMA reads needs two wait states, which the
// compiler cannot see to insert in front of an asm MFMA.  (Later fragments
// of the 8-bit path are converted two MFMAs ahead of their use.)
__device__ __forceinline__ void mfma_first_valu(floatx16& S, const bf16x8& A, const bf16x8& B) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(S) : "v"(A), "v"(B));
}
__device__ __forceinline__ void mfma_acc(floatx16& S, const bf16x8& A, const bf16x8& B) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(S) : "v"(A), "v"(B));
}
__device__ __forceinline__ void mfma_drain(floatx16& S) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(S));
}

// Bank swizzle of a 1152-byte row in LDS.  gfx950's LDS has 64 four-byte
// banks; a 16-byte read by 16 lanes or an 8-byte read by 32 lanes is served in
// one pass when the lanes hit 16 distinct 16-byte bank groups.  Row r starts
// at bank group 8 r (mod 16), and its 16-byte chunk c is stored at
// c ^ swz(r), swz = bit-reverse of bits 1..3 of r.  Then (a) 16 consecutive
// rows at one chunk (the QK fragment read) and (b) 8 aligned rows x 2 aligned
// chunks (one 32-lane half of a PV transpose read) cover 16 distinct groups.
__device__ __forceinline__ int swz(int r) {
  return ((r & 2) << 1) | ((r & 4) >> 1) | ((r & 8) >> 3);
}

// Bank swizzle of a 576-byte 8-bit row: its 16-byte chunk c is stored at
// c ^ f8sw(r) (within the aligned group of four chunks).  Row r starts at
// bank group 4 r (mod 16), so with f8sw = bits 2..3 of r (a) 16 consecutive
// rows at one chunk (a QK fragment read) and (b) rows {0..3, 8..11} or
// {4..7, 12..15} (mod 16) at two neighbouring chunks (one 32-lane half of a
// PV transpose read) each cover 16 distinct groups.
__device__ __forceinline__ int f8sw(int r) { return (r >> 2) & 3; }

// 8-bit cache: DMA slot k of wave w -> code chunk (0..17) of the tile, or -1
// for the scales (wave 3, slot 3); wave 3's slot 4 repeats chunk 17.
__device__ __forceinline__ int f8_chunk(int w, int k) {
  if (w < 3) return 5 * w + k;
  return k < 3 ? 15 + k : (k == 3 ? -1 : 17);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// eight E4M3 codes (two dwords, byte order) -> eight bf16 of code x s
// (exact for a power-of-two s: the products are bf16 values)
__device__ __forceinline__ bf16x8 cvt8(uint32_t w0, uint32_t w1, float s) {
  const bf16x2v a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false);
  const bf16x2v b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true);
  const bf16x2v c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false);
  const bf16x2v d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Wave w owns heads 32w .. 32w+31.  Per 32-row tile it computes
//   S^T[32 rows x 32 heads] = K[rows x 576] . Q^T[576 x heads]          (36 MFMA 32x32x16)
//   O^T[512 cols x 32 heads] += C^T[cols x 32 rows] . P^T[rows x heads]  (32 MFMA 32x32x16)
// One wave per SIMD holds Q (144 VGPRs) and O (256 accumulation registers);
// latency is hidden inside the wave by loading LDS fragments several
// steps ahead of the MFMA that consumes them.
// MODE: 0 contiguous bf16 cache, 1 paged bf16 pool, 2 contiguous 8-bit cache.
template <bool SCAN, int MODE>
__global__ void __launch_bounds__(THREADS, 1) k_split(SplitArgs a) {
  constexpr bool PAGED = MODE == 1;
  constexpr bool FP8 = MODE == 2;
  constexpr int DPW = FP8 ? F8_DPW : DMA_PER_WAVE;   // DMAs per wave and tile
  // (the 8-bit stages use the first NSTAGE * F8_STAGE bytes; all of it
  // stages the query rows at the start of a piece)
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * TILEB];
  // in-kernel scan (SCAN): prefix of the valid lengths and the offsets
  __shared__ int64_t s_pre[SCAN ? SPL_MAXB + 1 : 1];
  __shared__ int32_t s_off[SCAN ? SPL_MAXB : 1];
  __shared__ int64_t s_wsum[WAVES];
  __shared__ int32_t s_fsum[WAVES];
  __shared__ int16_t s_c[SCAN ? SPL_MAXB + 1 : 1];   // charge flags, then counts
  __shared__ int32_t s_first;
  __shared__ int64_t s_rows[2];   // this workgroup's first row, end row

  // Range index of this workgroup.  Workgroups are dealt to the 8 XCDs
  // round-robin (block i runs on XCD i % 8); giving each XCD a contiguous
  // run of ranges keeps the workgroups of one sequence on one XCD, where they
  // share its L2 for the query and neighbouring rows.
  const int g = (a.G % 8 == 0) ? (int)(blockIdx.x % 8) * (a.G / 8) + (int)(blockIdx.x / 8)
                               : (int)blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane_id = threadIdx.x & 63;

  // This workgroup's rows [start, end) and the sequence b holding row start.
  int64_t start, end, seq_begin0, seq_end0;
  int b0, off0;
  if (SCAN && a.B <= 64) {
    // Up to 64 sequences: wave 0 does all of it, one sequence per lane, with
    // wave-level scans and no workgroup barrier until the results are in LDS.
    const int B = a.B, G = a.G;
    int bad = 0;
    int4 sinfo = make_int4(0, 0, 0, 0);
    bool own_info = false;
    if (wave == 0) {
      const int l = lane_id;
      const bool in = l < B;
      const int len = vseq_len(a.lens, a.map, min(l, B - 1), a.n_q);
      const int o0 = PAGED ? 0 : a.map.offsets[seq_of(min(l, B - 1), a.n_q)];
      const bool ok = len > 0;
      const int64_t v = in && ok ? len : 0;
      bad = in && !ok ? 1 : 0;
      int64_t x = v;   // inclusive prefix of the valid lengths
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o, 64);
        if (l >= o) x += y;
      }
      const int64_t total = __shfl(x, 63, 64);
      const int64_t p0 = x - v;   // first row of sequence l
      if (in) {
        s_off[l] = o0;
        s_pre[l + 1] = x;
      }
      if (l == 0) s_pre[0] = 0;
      const Line rows_line(total > 0 ? total : 1, G);
      const int f = v > 0 && interior_start(p0, rows_line) ? 1 : 0;
      int c = f;   // charged starts up to and including l
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(c, o, 64);
        if (l >= o) c += y;
      }
      const int nchg = __shfl(c, 63, 64);
      const int64_t tv = total + SEG_ROWS * nchg;   // the virtual line
      const Line vline(tv > 0 ? tv : 1, G);
      const int64_t vs = total > 0 ? vline.start(g) : 0;
      const int64_t ve = total > 0 ? vline.start(g + 1) : 0;
      const int64_t vb = p0 + SEG_ROWS * c;
      const int64_t lo = vb - SEG_ROWS * f, hi = vb + v;
      const bool hs = v > 0 && lo <= vs && vs < hi;   // at most one lane each
      const bool he = v > 0 && lo <= ve && ve < hi;
      if (l == 0) {
        s_first = 0;
        s_rows[0] = 0;
        s_rows[1] = ve >= tv ? total : -1;   // ve == tv lies in no span
        s_wsum[0] = total;
      }
      if (hs) {
        s_first = l;
        s_rows[0] = p0 + (vs > vb ? vs - vb : 0);
      }
      if (he && ve < tv) s_rows[1] = p0 + (ve > vb ? ve - vb : 0);
      own_info = in && l % G == g;   // one workgroup per sequence
      if (own_info) sinfo = seq_info(vb, v, vline);
    }
    bad = __syncthreads_or(bad);
    if (g == 0 && threadIdx.x == 0 && bad && a.err_flag) atomicOr(a.err_flag, MLA_DEVERR_LENS);
    if (own_info) a.seqinfo[lane_id] = sinfo;
    if (s_wsum[0] <= 0) return;   // no valid sequence: the combine writes NaN
    start = uniform_i64(s_rows[0]);
    end = uniform_i64(s_rows[1]);
    b0 = uniform_i32(s_first);
    seq_begin0 = uniform_i64(s_pre[b0]);
    seq_end0 = uniform_i64(s_pre[b0 + 1]);
    off0 = uniform_i32(s_off[b0]);
  } else if constexpr (SCAN) {
    // Every workgroup scans the (at most SPL_MAXB) lengths itself: four
    // sequences per lane, a wave scan, then the four wave totals.
    const int tid = threadIdx.x;
    const int B = a.B, G = a.G;
    // all loads first (indices clamped), so they share one round trip
    int lenj[SPL_PER], offj[SPL_PER];
#pragma unroll
    for (int j = 0; j < SPL_PER; ++j) {
      const int bb = min(tid * SPL_PER + j, B - 1);
      lenj[j] = vseq_len(a.lens, a.map, bb, a.n_q);
      offj[j] = PAGED ? 0 : a.map.offsets[seq_of(bb, a.n_q)];
    }
    int64_t v[SPL_PER];
    int64_t tsum = 0;
    int bad = 0;
#pragma unroll
    for (int j = 0; j < SPL_PER; ++j) {
      const int bb = tid * SPL_PER + j;
      const bool in = bb < B;
      const bool ok = lenj[j] > 0;
      v[j] = in && ok ? lenj[j] : 0;
      bad |= in && !ok ? 1 : 0;
      if (in) s_off[bb] = offj[j];
      tsum += v[j];
    }
    int64_t x = tsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(x, o, 64);
      if (lane_id >= o) x += y;
    }
    if (lane_id == 63) s_wsum[wave] = x;
    if (tid == 0) {
      s_pre[0] = 0;
      s_first = 0;
      s_rows[0] = 0;
      s_rows[1] = -1;   // set below: the end row, or the total when the end is the line's end
    }
    __syncthreads();
    int64_t total = 0, run = x - tsum;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      total += s_wsum[w];
      if (w < wave) run += s_wsum[w];
    }
#pragma unroll
    for (int j = 0; j < SPL_PER; ++j) {
      const int bb = tid * SPL_PER + j;
      run += v[j];
      if (bb < B) s_pre[bb + 1] = run;
    }
    __syncthreads();
    // Charged sequence starts (see SEG_ROWS).  The per-sequence work below
    // takes sequence tid + THREADS k on lane tid, so that a small batch
    // spreads over many lanes; the scans take SPL_PER consecutive sequences
    // per lane.  s_c[b + 1] first holds the flag of sequence b, then the
    // number of charged starts among 0 .. b.
    {
      const Line rows_line(total > 0 ? total : 1, G);
#pragma unroll
      for (int k = 0; k < SPL_PER; ++k) {
        const int bb = tid + THREADS * k;
        if (bb < B)
          s_c[bb + 1] = (int16_t)(s_pre[bb + 1] > s_pre[bb] && interior_start(s_pre[bb], rows_line) ? 1 : 0);
      }
    }
    __syncthreads();
    int f[SPL_PER];
    int fsum = 0;
#pragma unroll
    for (int j = 0; j < SPL_PER; ++j) {
      const int bb = tid * SPL_PER + j;
      f[j] = bb < B ? s_c[bb + 1] : 0;
      fsum += f[j];
    }
    int fx = fsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(fx, o, 64);
      if (lane_id >= o) fx += y;
    }
    if (lane_id == 63) s_fsum[wave] = fx;
    __syncthreads();
    int nchg = 0, c = fx - fsum;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      nchg += s_fsum[w];
      if (w < wave) c += s_fsum[w];
    }
#pragma unroll
    for (int j = 0; j < SPL_PER; ++j) {
      const int bb = tid * SPL_PER + j;
      c += f[j];
      if (bb < B) s_c[bb + 1] = (int16_t)c;
    }
    if (tid == 0) s_c[0] = 0;
    const int64_t tv = total + SEG_ROWS * nchg;   // the virtual line
    const Line vline(tv > 0 ? tv : 1, G);
    const int64_t vs = total > 0 ? vline.start(g) : 0;
    const int64_t ve = total > 0 ? vline.start(g + 1) : 0;
    __syncthreads();
    // each lane maps the virtual bounds through its sequences, whose spans
    // [V - SEG_ROWS f, V + len) tile the virtual line
    int4 sinfo[SPL_PER];
#pragma unroll
    for (int k = 0; k < SPL_PER; ++k) {
      const int bb = tid + THREADS * k;
      if (bb < B) {
        const int64_t p0 = s_pre[bb], len = s_pre[bb + 1] - p0;
        const int cb = s_c[bb + 1], fb = cb - s_c[bb];
        const int64_t vb = p0 + SEG_ROWS * cb;
        if (len > 0) {
          const int64_t lo = vb - SEG_ROWS * fb, hi = vb + len;
          if (lo <= vs && vs < hi) {   // one writer each
            s_first = bb;
            s_rows[0] = p0 + (vs > vb ? vs - vb : 0);
          }
          if (lo <= ve && ve < hi) s_rows[1] = p0 + (ve > vb ? ve - vb : 0);
        }
        if (bb % G == g) sinfo[k] = seq_info(vb, len, vline);   // one workgroup per sequence
      }
    }
    bad = __syncthreads_or(bad);
    if (g == 0 && tid == 0 && bad && a.err_flag) atomicOr(a.err_flag, MLA_DEVERR_LENS);
    // what the combine needs of each sequence (written by one workgroup;
    // stored after the barrier, which would otherwise wait for the stores)
#pragma unroll
    for (int k = 0; k < SPL_PER; ++k) {
      const int bb = tid + THREADS * k;
      if (bb < B && bb % G == g) a.seqinfo[bb] = sinfo[k];
    }
    start = s_rows[0];
    end = ve >= tv ? total : s_rows[1];   // ve == tv lies in no span
    if (total <= 0) return;   // no valid sequence: the combine writes NaN
    start = uniform_i64(start);
    end = uniform_i64(end);
    b0 = uniform_i32(s_first);
    seq_begin0 = uniform_i64(s_pre[b0]);
    seq_end0 = uniform_i64(s_pre[b0 + 1]);
    off0 = uniform_i32(s_off[b0]);
  } else {
    const WgRec rec = a.rec[g];
    start = uniform_i64(rec.start);
    end = uniform_i64(rec.end);
    seq_begin0 = uniform_i64(rec.seq_begin);
    seq_end0 = uniform_i64(rec.seq_end);
    b0 = uniform_i32(rec.b);
    off0 = uniform_i32(rec.off_b);
  }
  auto pre = [&](int i) -> int64_t {
    if constexpr (SCAN) return uniform_i64(s_pre[i]);
    else return uniform_i64(a.prefix[i]);
  };
  auto off_of = [&](int i) -> int {
    if constexpr (SCAN) return uniform_i32(s_off[i]);
    else if constexpr (PAGED) return 0;
    else return uniform_i32(a.map.offsets[seq_of(i, a.n_q)]);
  };

  if (start >= end) {
    // An empty range (fewer rows than workgroups) can fall inside the span of
    // ranges the combine walks for sequence b0: leave it a zero partial
    // with weight 0 there (m = -inf, l = 0) and no fallback flag.
    if (seq_end0 > seq_begin0) {
      const size_t slot = (size_t)g + (size_t)b0;
      uint4* po = (uint4*)(a.part_o + slot * NH * DC);
      for (int i = threadIdx.x; i < NH * DC / 8; i += THREADS) po[i] = make_uint4(0, 0, 0, 0);
      if (threadIdx.x < NH)
        ((float2*)a.part_ml)[slot * NH + threadIdx.x] = make_float2(-INFINITY, 0.f);
      if (threadIdx.x < WAVES) a.flags[slot * WAVES + threadIdx.x] = 0;
    }
    return;
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)(MLA_LDS char*)lds;

  // QK A-fragment (32x32x16): row n32, logical chunk 2 kk + g32 stored at
  // (2 kk + g32) ^ swz(n32).  For kk = 4u + v the low three bits are
  // (2v + g32) ^ swz(n32); the rest is the constant 8u chunks.
  // These lane-dependent offsets are rebuilt at the start of every QK / PV
  // block from an opaque copy of the lane index (a handful of VALU
  // instructions) rather than kept in registers across the whole loop.
  auto make_qk_off = [&](uint32_t (&o)[4]) {
    int ln = lane_id;
    asm volatile("" : "+v"(ln));
    ln &= 63;
    const int n = ln & 31, h = ln >> 5;
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = (uint32_t)(n * ROWB + (((2 * v + h) ^ swz(n)) << 4));
  };

  // PV A-fragment via transpose reads.  In each 16-lane group G (i = lane%16),
  // lane i reads 8 bytes of row 16 kk2 + 8 rd + rr, rr = 4 g32 + i/4, at
  // columns 32 cb + 16 (G & 1) + 4 (i & 3); after the transpose lane j of the
  // group holds column 32 cb + 16 (G & 1) + j for four consecutive rows.
  // Logical chunk 4 cb + e sits at (4 cb + e) ^ swz(8 rd + rr)
  //   = 4 (cb ^ bb) + (e ^ ff),  bb = bit 2 of swz, ff = its low two bits.
  auto make_tr_base = [&](uint32_t (&t)[2][2]) {
    int ln = lane_id;
    asm volatile("" : "+v"(ln));
    ln &= 63;
    const int Gq = ln >> 4;
    const int i16 = ln & 15;
    const int rr = 4 * (ln >> 5) + (i16 >> 2);
    const int e = 2 * (Gq & 1) + ((i16 & 3) >> 1);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int sw = swz(8 * rd + rr);
      const int bb = sw >> 2, ff = sw & 3;
      const uint32_t base = (uint32_t)((8 * rd + rr) * ROWB + ((e ^ ff) << 4) + 8 * (i16 & 1));
      t[rd][0] = base + (uint32_t)(bb << 6);   // cb even: cb ^ bb = cb + bb
      t[rd][1] = base - (uint32_t)(bb << 6);   // cb odd:  cb ^ bb = cb - bb
    }
  };

  int b = b0;   // first sequence touching [start, end)

  int64_t pos = start;
  bool first_segment = true;
  while (pos < end) {
    // Lane-derived values are rebuilt for every piece from an opaque copy of
    // the lane index, so none of them stays live (and spilled) across the
    // previous piece's epilogue.
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    lane &= 63;
    const int g32 = lane >> 5;          // which half of the wave
    const int n32 = lane & 31;          // head within the wave / row within the tile
    const int head = wave * HPW + n32;

    // DMA: wave-instruction j = 9 wave + k covers LDS chunks [64 j, 64 j + 64);
    // lane i fills chunk p = 64 j + i, which holds logical chunk
    // (p % 72) ^ swz(row) of row p / 72.  The 64 chunks span at most two rows
    // (72 > 64), so everything but a per-lane select is wave-uniform.
    // The nine per-lane source offsets (< 36864) are kept as 16-bit pairs in
    // five registers; each DMA extracts its own with one instruction.
    uint32_t dma_pk[(DMA_PER_WAVE + 1) / 2];
  #pragma unroll
    for (int j = 0; j < (DMA_PER_WAVE + 1) / 2; ++j) dma_pk[j] = 0;
  #pragma unroll
    for (int k = 0; k < DPW; ++k) {
      uint32_t off;
      if constexpr (FP8) {
        // 8-bit: LDS chunk p = 64 j + i of the tile holds logical chunk
        // (p % 36) ^ f8sw(row) of row p / 36 (the scale slot's offset is unused)
        const int j = f8_chunk(wave, k);
        const int p = 64 * (j < 0 ? 0 : j) + lane;
        const int r = p / F8_CHUNKS;
        const int c = (p % F8_CHUNKS) ^ f8sw(r);
        off = (uint32_t)(r * F8_ROWB + c * 16);
      } else {
        const int p = (wave * DMA_PER_WAVE + k) * 64 + lane;
        const int r = p / CHUNKS;
        const int c = (p % CHUNKS) ^ swz(r);
        off = (uint32_t)(r * ROWB + c * 16);
      }
      dma_pk[k >> 1] |= off << (16 * (k & 1));
    }
    auto dma_off = [&](int k) -> uint32_t { return (dma_pk[k >> 1] >> (16 * (k & 1))) & 0xffffu; };

    // The record describes the first sequence; later ones are looked up.
    int64_t seq_begin, seq_endx;
    int off_b;
    if (first_segment) {
      seq_begin = seq_begin0;
      seq_endx = seq_end0;
      off_b = off0;
    } else {
      while (pre(b + 1) <= pos) ++b;
      seq_begin = pre(b);
      seq_endx = pre(b + 1);
      off_b = off_of(b);
    }
    const int64_t seg_end = end < seq_endx ? end : seq_endx;
    const int t0 = (int)(pos - seq_begin);
    const int seg_len = (int)(seg_end - pos);
    const int ntiles = (seg_len + TILE - 1) / TILE;
    const char* rows = a.cache + ((size_t)off_b + (size_t)t0) * (FP8 ? F8_ROWB : ROWB);
    // paged: this sequence's row of the block table
    const int32_t* tbl = PAGED ? a.map.table + (size_t)seq_of(b, a.n_q) * a.map.max_blocks : nullptr;

    if (!first_segment) barrier_all_lds();   // previous segment's tiles fully consumed
    first_segment = false;

    // Q fragments (B operand of QK): head n32, features 16 kk + 8 g32 .. +8.
    // A wave's 32 query rows [q_lat | q_pe] (1152 B each, like cache rows)
    // are DMA'd into stage `wave` in the tile layout -- whole rows, so every
    // DMA instruction reads full cache lines -- and then read out with the
    // QK fragment pattern.  The stages are free until the tiles are issued.
    bf16x8 q[KSTEPS];
    {
      const char* qlb = (const char*)(a.q_lat + ((size_t)b * NH + wave * HPW) * DC);
      const char* qpb = (const char*)(a.q_pe + ((size_t)b * NH + wave * HPW) * DR);
      const uint32_t qstage = lds0 + (uint32_t)(wave * TILEB);
#pragma unroll 4
      for (int j = 0; j < TILEB / 1024; ++j) {
        const int p = 64 * j + lane;
        const int r = p / CHUNKS;
        const int c = (p % CHUNKS) ^ swz(r);
        const char* src = c < DC / 8 ? qlb + r * (DC * 2) + c * 16 : qpb + r * (DR * 2) + (c - DC / 8) * 16;
        dma_16B_at(qstage + (uint32_t)(j * 1024), src);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's own stage
      uint32_t qo[4];
      make_qk_off(qo);
      const MLA_LDS char* T = (const MLA_LDS char*)lds + wave * TILEB;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        if constexpr (FP8) {
          // 8-bit path: MFMA kk takes features 32 (kk/2) + 16 g32 + 8 (kk%2) .. +8,
          // the order of its 16-byte code fragments (logical bf16 chunk
          // 4 (kk/2) + 2 g32 + kk%2, stored at that ^ swz(n32))
          const int L = 4 * (kk >> 1) + 2 * g32 + (kk & 1);
          q[kk] = *(const MLA_LDS bf16x8*)(T + n32 * ROWB + ((L ^ swz(n32)) << 4));
        } else {
          q[kk] = *(const MLA_LDS bf16x8*)(T + qo[kk & 3] + (kk >> 2) * 128);
        }
      }
      barrier_all_lds();   // every wave has its Q before the tiles overwrite the stages
    }

    // Every tile index t gets exactly DMA_PER_WAVE DMA instructions per wave,
    // issued in order t = 0, 1, 2, ...  Tile t goes into stage t % NSTAGE.
    // Row clamping keeps every source byte inside the piece:
    //  * t < ntiles, partial tile: lanes whose chunk lies in a row at or past
    //    nvalid load the last valid 16 bytes instead, so the whole stage
    //    holds finite cache values (their scores are masked out);
    //  * t >= ntiles (past the end of the piece): a copy of the last tile
    //    (just fetched, so served by L2) into the stage that tile t would
    //    use -- it is free, and no later tile of this piece uses it.
    // With a fixed count per tile the wait for tile `it` is always the same.
    //
    // Paged rows: the tile's (at most 32) rows lie in at most two pool blocks
    // (a block holds >= 32 rows).  Lanes whose byte offset in the tile is
    // below thr read from block 0 at a0 + offset, the others from block 1 at
    // a1 + offset (a1 is block 1's address shifted back by the rows of block
    // 0 in the tile), so one compare and select per DMA picks the source.
    // An id outside [0, num_blocks) is replaced by block 0 (nothing outside
    // the pool is read) and the piece is flagged; its sequence's result is
    // then NaN with MLA_DEVERR_TABLE.
    struct TileSrc {
      const char* a0;
      const char* a1;
      uint32_t thr, bound;
      const char* scl;   // 8-bit cache: the tile's first scale
      int nv;            // 8-bit cache: valid rows in the tile (clamped to TILE)
    };
    bool bad_tbl = false;
    auto dma_src = [&](int t) -> TileSrc {
      const int ts = t < ntiles ? t : ntiles - 1;
      const int nv = seg_len - ts * TILE;
      TileSrc r;
      r.bound = nv >= TILE ? (uint32_t)TILEB - 16u : (uint32_t)(nv * ROWB - 16);
      r.scl = nullptr;
      r.nv = 0;
      if constexpr (FP8) {
        r.bound = nv >= TILE ? (uint32_t)F8_TILEB - 16u : (uint32_t)(nv * F8_ROWB - 16);
        r.a0 = r.a1 = rows + (size_t)ts * F8_TILEB;
        r.thr = 0xffffffffu;
        r.scl = (const char*)(a.scales + (size_t)off_b + (size_t)t0 + (size_t)ts * TILE);
        r.nv = nv < TILE ? nv : TILE;
      } else if constexpr (!PAGED) {
        r.a0 = r.a1 = rows + (size_t)ts * TILEB;
        r.thr = 0xffffffffu;
      } else {
        const int sh = a.map.shift;
        const int brows = 1 << sh;
        const int R0 = t0 + ts * TILE;   // the tile's first row in the sequence
        const int rin = R0 & (brows - 1);
        const int blk = R0 >> sh;
        const int nrow = nv < TILE ? nv : TILE;
        int id0 = sload_i32(tbl + blk);
        int id1 = rin + nrow > brows ? sload_i32(tbl + blk + 1) : id0;
        if ((unsigned)id0 >= (unsigned)a.map.num_blocks) { id0 = 0; bad_tbl = true; }
        if ((unsigned)id1 >= (unsigned)a.map.num_blocks) { id1 = 0; bad_tbl = true; }
        r.a0 = a.cache + (((int64_t)id0 << sh) + rin) * (int64_t)ROWB;
        r.a1 = a.cache + (((int64_t)id1 << sh) + rin - brows) * (int64_t)ROWB;
        r.thr = (uint32_t)((brows - rin) * ROWB);
      }
      return r;
    };
    auto dma = [&](uint32_t lds_addr, uint32_t off, const TileSrc& src) {
      if constexpr (!PAGED) dma_16B(lds_addr, off, src.a0);
      else dma_16B_at(lds_addr, (off < src.thr ? src.a0 : src.a1) + off);
    };
    // LDS stage (DMA target) of tile t
    auto stage_of = [&](int t) -> uint32_t {
      return lds0 + (uint32_t)((t % NSTAGE) * (FP8 ? F8_STAGE : TILEB));
    };
    // the k-th DMA of this wave for a tile
    auto dma_slot = [&](int k, uint32_t stage_lds, const TileSrc& src) {
      if constexpr (FP8) {
        const int j = f8_chunk(wave, k);
        if (j < 0) {
          dma_4B_at(stage_lds + F8_TILEB, src.scl + 4 * (lane_id < src.nv ? lane_id : src.nv - 1));
        } else {
          dma_16B(stage_lds + (uint32_t)(j * 1024), min(dma_off(k), src.bound), src.a0);
        }
      } else {
        dma(stage_lds + (uint32_t)((wave * DMA_PER_WAVE + k) * 1024), min(dma_off(k), src.bound), src);
      }
    };
    auto issue_tile = [&](int t) {
      const TileSrc src = dma_src(t);
      const uint32_t stage_lds = stage_of(t);
#pragma unroll
      for (int k = 0; k < DPW; ++k) dma_slot(k, stage_lds, src);
    };
    // tile read by QK / PV for tile t (its stage)
    auto ctile = [&](int t) -> const MLA_LDS char* {
      return (const MLA_LDS char*)lds + (t % NSTAGE) * (FP8 ? F8_STAGE : TILEB);
    };
    // Wait for tile `it`: the tiles it+1 and it+2 were issued after it.

    // Three tiles ahead: tile it+3 goes into the stage of tile it-1.
    for (int t = 0; t < NSTAGE - 1; ++t) issue_tile(t);

    floatx16 O[DC / 32];
#pragma unroll
    for (int cb = 0; cb < DC / 32; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[cb][i] = 0.f;
    float m_ref = 0.f;         // reference max of scaled scores (log2 units)
    float l_run = 0.f;         // this lane's share of the sum of weights
    float s_thr = INFINITY;    // raw-score bound of the overflow check
    bool ovf_any = false;      // a score of this lane exceeded it

    // ---- S^T = K . Q^T of tile t, fragments loaded QK_PF steps ahead ----
    auto qk = [&](int t, floatx16& S) {
      const MLA_LDS char* T = ctile(t);
      uint32_t qk_off[4];
      make_qk_off(qk_off);
      bf16x8 kf[QK_PF];
#pragma unroll
      for (int j = 0; j < QK_PF; ++j)
        kf[j] = *(const MLA_LDS bf16x8*)(T + qk_off[j & 3] + (j >> 2) * 128);
      // (MFMA, load) pairs in program order, pinned by scheduling barriers:
      // the MFMAs are asm statements, which the scheduler's instruction
      // groups do not recognise, and without the barriers it sank every
      // fragment load to just before its MFMA behind a full LDS wait.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        if (kk == 0)
          mfma_first(S, kf[0], q[0]);
        else
          mfma_acc(S, kf[kk % QK_PF], q[kk]);
        const int nk = kk + QK_PF;
        if (nk < KSTEPS)
          kf[kk % QK_PF] = *(const MLA_LDS bf16x8*)(T + qk_off[nk & 3] + (nk >> 2) * 128);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_drain(S);
    };

    // ---- softmax of one tile: lane holds head n32, rows 8 (i/4) + 4 g32 + i%4 ----
    // Every weight is bf16(2^fma(S, scale log2 e, -m_ref)) with m_ref fixed by
    // the first tile as the max of separately rounded products; at the
    // maximal score the fma leaves only that product's rounding error, so the
    // weight rounds to exactly 1.  l sums the same bf16 weights that enter PV,
    // so O / l is an exactly normalised average of the rows.  A score more
    // than 2^64 above the reference flags the piece for the fallback.  Rows
    // at or past nvalid (a partial tile) get weight 0.  No branches: the
    // instructions interleave with the next tile's QK MFMAs.
    // Row of score i is 8 (i/4) + i%4 + 4 g32: "row < n" is tested as
    // 4 g32 < n - (8 (i/4) + i%4), one lane value against wave-uniform bounds.
    const int row4 = 4 * g32;
    auto row_lt = [&](int i, int n) { return row4 < n - (8 * (i >> 2) + (i & 3)); };
    // weights of scores 2j, 2j+1 -> P pair j; smax tracks the unmasked max
    auto sm_pair = [&](const floatx16& S, int j, int nvalid, bf16x8 (&P)[2], float& smax) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * j + e;
        const bool ok = row_lt(i, nvalid);
        smax = fmaxf(smax, ok ? S[i] : -INFINITY);
        const float x = ok ? fmaf(S[i], a.scale_log2, -m_ref) : -INFINITY;
        P[i >> 3][i & 7] = (__bf16)__builtin_amdgcn_exp2f(x);
      }
    };
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    auto sm_sum = [&](const bf16x8 (&P)[2], int j) {
      const bf16x2 pr = {P[j >> 2][2 * (j & 3)], P[j >> 2][2 * (j & 3) + 1]};
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_run, false);
    };
    auto softmax = [&](const floatx16& S, int nvalid, bf16x8 (&P)[2]) {
      float smax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) sm_pair(S, j, nvalid, P, smax);
#pragma unroll
      for (int j = 0; j < 8; ++j) sm_sum(P, j);
      ovf_any = ovf_any || (smax > s_thr);
    };

    // ---- 8-bit path: fragments straight from the code tile ----
    // QK A-fragment pair c2 (MFMAs 2 c2 and 2 c2 + 1): lane (n32, g32) reads the
    // 16 codes of row n32 at logical chunk 2 c2 + g32 (features 32 c2 + 16 g32
    // .. +16: the first eight feed MFMA 2 c2, the rest MFMA 2 c2 + 1), stored at
    // 4 (c2 / 2) + ((2 (c2 % 2) + g32) ^ f8sw(n32)).
    auto make_qk8_off = [&](uint32_t (&o)[2]) {
      int ln = lane_id;
      asm volatile("" : "+v"(ln));
      ln &= 63;
      const int n = ln & 31, h = ln >> 5;
#pragma unroll
      for (int v = 0; v < 2; ++v) o[v] = (uint32_t)(n * F8_ROWB + (((2 * v + h) ^ f8sw(n)) << 4));
    };
    auto qk8_frag = [&](const MLA_LDS char* Tt, const uint32_t (&o)[2], int c2) -> u32x4 {
      return *(const MLA_LDS u32x4*)(Tt + o[c2 & 1] + (c2 >> 1) * 64);
    };
    // scale of this lane's QK row (n32) of a tile
    auto row_scale = [&](const MLA_LDS char* Tt) -> float {
      int ln = lane_id;
      asm volatile("" : "+v"(ln));
      ln &= 31;
      return *(const MLA_LDS float*)(Tt + F8_TILEB + 4 * ln);
    };
    // PV A-fragment by 8-bit transpose reads.  In each 16-lane group G
    // (i = lane % 16) lanes 2k and 2k+1 read the two 8-byte halves of row
    // rho_k = 16 kk2 + 8 (k / 4) + 4 g32 + k % 4 at columns 32 cb + 16 (G & 1)
    // .. +16; after the transpose lane j of the group holds column
    // 32 cb + 16 (G & 1) + j of rows rho_0 .. rho_7, the rows whose weights
    // the lane holds in P[kk2].  f8sw(rho_k) = 2 (k / 4) + g32 for both kk2,
    // so logical chunk 2 cb + (G & 1) sits at 4 (cb / 2) + ((2 (cb % 2) + (G & 1)) ^ f).
    auto make_tr8_base = [&](uint32_t (&t)[2]) {
      int ln = lane_id;
      asm volatile("" : "+v"(ln));
      ln &= 63;
      const int i16 = ln & 15, k = i16 >> 1;
      const int rho = 8 * (k >> 2) + 4 * (ln >> 5) + (k & 3);
      const int f = f8sw(rho);
      const int gh = (ln >> 4) & 1;
#pragma unroll
      for (int v = 0; v < 2; ++v)
        t[v] = (uint32_t)(rho * F8_ROWB + (((2 * v + gh) ^ f) << 4) + 8 * (i16 & 1));
    };
    // QK of tile t (no softmax beside it): the prologue
    auto qk8 = [&](int t, floatx16& S) {
      const MLA_LDS char* Tt = ctile(t);
      uint32_t o8[2];
      make_qk8_off(o8);
      const float sq = row_scale(Tt);
      u32x4 kf[QK_PF8];
#pragma unroll
      for (int j = 0; j < QK_PF8; ++j) kf[j] = qk8_frag(Tt, o8, j);
      bf16x8 A[3];
      A[0] = cvt8(kf[0][0], kf[0][1], sq);
      A[1] = cvt8(kf[0][2], kf[0][3], sq);
      kf[0] = qk8_frag(Tt, o8, QK_PF8);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        if (kk == 0)
          mfma_first_valu(S, A[0], q[0]);
        else
          mfma_acc(S, A[kk % 3], q[kk]);
        __builtin_amdgcn_sched_barrier(0);
        const int nk = kk + 2;
        if (nk < KSTEPS) {
          const int c2 = nk >> 1;
          const u32x4 f = kf[c2 % QK_PF8];
          A[nk % 3] = (nk & 1) ? cvt8(f[2], f[3], sq) : cvt8(f[0], f[1], sq);
          if ((nk & 1) && c2 + QK_PF8 < KSTEPS / 2) kf[c2 % QK_PF8] = qk8_frag(Tt, o8, c2 + QK_PF8);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_drain(S);
    };
    // softmax of tile it spread over the QK steps of tile it+1: one pair of
    // weights after each odd step, their row sums later (the 16-bit loop
    // below writes the same steps inline)
    auto sm_step = [&](int kk, const floatx16& Sc, float& smax, float (&x)[16], float (&e)[16],
                       bf16x8 (&P)[2]) {
      if (kk < 16) {
        x[kk] = fmaf(Sc[kk], a.scale_log2, -m_ref);
        if (kk & 1) smax = max3f(smax, Sc[kk - 1], Sc[kk]);
      }
      if (kk >= 4 && kk < 20) e[kk - 4] = __builtin_amdgcn_exp2f(x[kk - 4]);
      if (kk >= 9 && kk < 25 && (kk & 1)) {
        const int j = (kk - 9) / 2;
        P[j >> 2][2 * (j & 3)] = (__bf16)e[2 * j];
        P[j >> 2][2 * (j & 3) + 1] = (__bf16)e[2 * j + 1];
      }
      if (kk >= 26 && kk < 34) sm_sum(P, kk - 26);
    };

    // ---- prologue: QK of tile 0 and the reference max ----
    floatx16 S_cur;
    wait_vm_then_barrier<(NSTAGE - 2) * DPW>();   // tile 0 landed
    if constexpr (FP8) {
      qk8(0, S_cur);
    } else {
      qk(0, S_cur);
    }
    {
      float mloc = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = __fmul_rn(S_cur[i], a.scale_log2);
        mloc = fmaxf(mloc, row_lt(i, seg_len) ? v : -INFINITY);
      }
      m_ref = fmaxf(mloc, swap_halves(mloc, lane));
      s_thr = (m_ref + OVF_TH) / a.scale_log2;
    }

    // ---- 8-bit software pipeline: the same steps, fragments converted in registers ----
    if constexpr (FP8) {
      for (int it = 0; it < ntiles; ++it) {
        const int nvalid = seg_len - it * TILE;
        const TileSrc nsrc = dma_src(it + NSTAGE - 1);
        const MLA_LDS char* T = ctile(it);
        bf16x8 P[2], Pv[2];
        floatx16 S_next;
        uint32_t tr8b[2];
        i32x2 pa8[PV_PF8];
        auto pv8_frag = [&](int j) {
          const int kk2 = j / (DC / 32), cb = j % (DC / 32);
          pa8[j % PV_PF8] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (MLA_LDS i32x2*)(T + tr8b[cb & 1] + kk2 * 16 * F8_ROWB + (cb >> 1) * 64));
        };
        // PV weights with the row scales folded in: weight i of this lane
        // belongs to row 8 (i / 4) + 4 g32 + i % 4; bf16 x power of two is exact
        floatx4 s4[4];
        auto load_s4 = [&]() {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            s4[r4] = *(const MLA_LDS floatx4*)(T + F8_TILEB + 4 * (8 * r4 + 4 * g32));
        };
        auto pv_scale = [&](int j) {
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int i = 2 * j + e2;
            Pv[i >> 3][i & 7] = (__bf16)((float)P[i >> 3][i & 7] * s4[i >> 2][i & 3]);
          }
        };
        if (it + 1 < ntiles) {
          uint32_t o8[2];
          make_qk8_off(o8);
          wait_vm_then_barrier<(NSTAGE - 3) * DPW>();
          floatx16 Sc = S_cur;
          asm volatile("" : "+v"(Sc));
          const MLA_LDS char* Tn = ctile(it + 1);
          const float sq = row_scale(Tn);
          u32x4 kf[QK_PF8];
#pragma unroll
          for (int j = 0; j < QK_PF8; ++j) kf[j] = qk8_frag(Tn, o8, j);
          bf16x8 A[3];
          A[0] = cvt8(kf[0][0], kf[0][1], sq);
          A[1] = cvt8(kf[0][2], kf[0][3], sq);
          kf[0] = qk8_frag(Tn, o8, QK_PF8);
          float smax = -INFINITY;
          float x[16], e[16];
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            if (kk == 0)
              mfma_first_valu(S_next, A[0], q[0]);
            else
              mfma_acc(S_next, A[kk % 3], q[kk]);
            __builtin_amdgcn_sched_barrier(0);
            // fragment of MFMA kk+2, converted two steps ahead of its use
            const int nk = kk + 2;
            if (nk < KSTEPS) {
              const int c2 = nk >> 1;
              const u32x4 f = kf[c2 % QK_PF8];
              A[nk % 3] = (nk & 1) ? cvt8(f[2], f[3], sq) : cvt8(f[0], f[1], sq);
              if ((nk & 1) && c2 + QK_PF8 < KSTEPS / 2) kf[c2 % QK_PF8] = qk8_frag(Tn, o8, c2 + QK_PF8);
            }
            sm_step(kk, Sc, smax, x, e, P);
            if (kk == 20) load_s4();
            if (kk >= 26 && kk < 34) pv_scale(kk - 26);
            if (kk == KSTEPS - PV_PF8 - 2) make_tr8_base(tr8b);
            if (kk >= KSTEPS - PV_PF8 - 1 && kk < KSTEPS - 1) pv8_frag(kk - (KSTEPS - PV_PF8 - 1));
            __builtin_amdgcn_sched_barrier(0);
          }
          mfma_drain(S_next);
          ovf_any = ovf_any || (smax > s_thr);
        } else {
          barrier_all_lds();
          floatx16 Sc = S_cur;
          asm volatile("" : "+v"(Sc));
          softmax(Sc, nvalid, P);
          load_s4();
#pragma unroll
          for (int j = 0; j < 8; ++j) pv_scale(j);
          make_tr8_base(tr8b);
#pragma unroll
          for (int j = 0; j < PV_PF8; ++j) pv8_frag(j);
        }

        // ---- O^T += C^T . P'^T; tile it+3's DMAs spread as in the 16-bit loop ----
        {
          const int nt = it + NSTAGE - 1;
          const uint32_t stage_lds = stage_of(nt);
          bf16x8 cf = cvt8((uint32_t)pa8[0][0], (uint32_t)pa8[0][1], 1.0f);
#pragma unroll
          for (int s = 0; s < 2 * (DC / 32); ++s) {
            const int kk2 = s / (DC / 32), cb = s % (DC / 32);
            // fragment s + PV_PF8 into the slot of fragment s (converted)
            if (s + PV_PF8 < 2 * (DC / 32)) pv8_frag(s + PV_PF8);
            O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf, Pv[kk2], O[cb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < 2 * (DC / 32)) {
              cf = cvt8((uint32_t)pa8[(s + 1) % PV_PF8][0], (uint32_t)pa8[(s + 1) % PV_PF8][1], 1.0f);
            }
            if (s % 3 == 2 && s / 3 < DPW) dma_slot(s / 3, stage_lds, nsrc);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        S_cur = S_next;
      }
    } else {

    // ---- software pipeline: [QK(it+1) || softmax(it)], then PV(it) ----
    for (int it = 0; it < ntiles; ++it) {
      const int nvalid = seg_len - it * TILE;
      // source of tile it+3, DMA'd during PV below (paged: its block ids are
      // fetched here, where no LDS read is in flight)
      const TileSrc nsrc = dma_src(it + NSTAGE - 1);
      const MLA_LDS char* T = ctile(it);
      bf16x8 P[2];
      floatx16 S_next;
      // PV A-fragments of tile it, PV_PF pairs ahead of their MFMAs.  The
      // first pairs are read during the last QK steps (tile it is resident
      // throughout), so PV starts without waiting on transpose reads.
      uint32_t tr_base[2][2];
      bf16x4 pa[PV_PF][2];
      auto pv_pair = [&](int j) {
        const int kk2 = j / (DC / 32), cb = j % (DC / 32);
        const MLA_LDS char* p0 = T + tr_base[0][cb & 1] + kk2 * 16 * ROWB + cb * 64;
        const MLA_LDS char* p1 = T + tr_base[1][cb & 1] + kk2 * 16 * ROWB + cb * 64;
        pa[j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p0);
        pa[j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p1);
      };
      // (The empty asm statements pin the softmax inside each branch: the
      // compiler would otherwise hoist the common code above the branch, out
      // of reach of the QK MFMAs it is meant to overlap.)
      if (it + 1 < ntiles) {
        // Tile it+1 landed (only tile it+2 was issued after it); the barrier
        // also means every wave is past PV(it-1), so that tile's stage may be
        // refilled below.
        uint32_t qk_off[4];
        make_qk_off(qk_off);   // lane arithmetic only: ahead of the wait
        wait_vm_then_barrier<(NSTAGE - 3) * DPW>();
        floatx16 Sc = S_cur;
        asm volatile("" : "+v"(Sc));
        // QK of tile it+1 with the softmax of tile it in its MFMA gaps: one
        // pair of weights after each odd MFMA, their row sums later; the
        // scheduling barriers keep every step where it is written, so the
        // fragment prefetch and the VALU placement stay as planned.
        const MLA_LDS char* Tn = ctile(it + 1);
        bf16x8 kf[QK_PF];
#pragma unroll
        for (int j = 0; j < QK_PF; ++j)
          kf[j] = *(const MLA_LDS bf16x8*)(Tn + qk_off[j & 3] + (j >> 2) * 128);
        // Tile it is full here (only the last tile of a piece can be
        // partial, and it takes the other branch): no row masking.  Each
        // weight's fma, exp2, bf16 packing and row sum sit several MFMAs
        // apart, so no VALU instruction waits on the one before it.
        float smax = -INFINITY;
        float x[16], e[16];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          if (kk == 0)
            mfma_first(S_next, kf[0], q[0]);
          else
            mfma_acc(S_next, kf[kk % QK_PF], q[kk]);
          const int nk = kk + QK_PF;
          if (nk < KSTEPS)
            kf[kk % QK_PF] = *(const MLA_LDS bf16x8*)(Tn + qk_off[nk & 3] + (nk >> 2) * 128);
          if (kk < 16) {
            x[kk] = fmaf(Sc[kk], a.scale_log2, -m_ref);
            if (kk & 1) smax = max3f(smax, Sc[kk - 1], Sc[kk]);
          }
          if (kk >= 4 && kk < 20) e[kk - 4] = __builtin_amdgcn_exp2f(x[kk - 4]);
          if (kk >= 9 && kk < 25 && (kk & 1)) {
            const int j = (kk - 9) / 2;
            P[j >> 2][2 * (j & 3)] = (__bf16)e[2 * j];
            P[j >> 2][2 * (j & 3) + 1] = (__bf16)e[2 * j + 1];
          }
          if (kk >= 26 && kk < 34) sm_sum(P, kk - 26);
          if (kk == KSTEPS - PV_PF - 2) make_tr_base(tr_base);
          if (kk >= KSTEPS - PV_PF - 1 && kk < KSTEPS - 1) pv_pair(kk - (KSTEPS - PV_PF - 1));
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_drain(S_next);
        ovf_any = ovf_any || (smax > s_thr);
      } else {
        barrier_all_lds();
        floatx16 Sc = S_cur;
        asm volatile("" : "+v"(Sc));
        softmax(Sc, nvalid, P);
        make_tr_base(tr_base);
#pragma unroll
        for (int j = 0; j < PV_PF; ++j) pv_pair(j);
      }


      // ---- O^T += C^T . P^T over 2 row halves x 16 column blocks ----
      // Tile it+3 goes into the stage of tile it-1; its nine DMA instructions
      // per wave are spread over the loop: the address unit moves 64 B per
      // clock, so issuing them back to back stalls the wave for ~600 cycles.
      {
        const int nt = it + NSTAGE - 1;
        const uint32_t stage_lds = stage_of(nt);
        // DMA k goes out after MFMA 3k+2 (its source offset is recomputed
        // there: a few VALU instructions in the MFMA gaps, no registers held).
#pragma unroll
        for (int s = 0; s < 2 * (DC / 32); ++s) {
          const int kk2 = s / (DC / 32), cb = s % (DC / 32);
          const bf16x4 lo = pa[s % PV_PF][0], hi = pa[s % PV_PF][1];
          const bf16x8 cf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const int ns = s + PV_PF;
          if (ns < 2 * (DC / 32)) {
            const int nk2 = ns / (DC / 32), ncb = ns % (DC / 32);
            const MLA_LDS char* p0 = T + tr_base[0][ncb & 1] + nk2 * 16 * ROWB + ncb * 64;
            const MLA_LDS char* p1 = T + tr_base[1][ncb & 1] + nk2 * 16 * ROWB + ncb * 64;
            pa[s % PV_PF][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p0);
            pa[s % PV_PF][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p1);
          }
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf, P[kk2], O[cb], 0, 0, 0);
          if (s % 3 == 2 && s / 3 < DPW) dma_slot(s / 3, stage_lds, nsrc);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV_PF, 1);
#pragma unroll
        for (int s2 = 0; s2 < 2 * (DC / 32) - PV_PF; ++s2) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PV_PF, 1);
      }
      S_cur = S_next;
    }
    }   // 16-bit loop
    const size_t slot = (size_t)g + (size_t)b;
    // DMAs issued during the last tiles only fill stages this piece no
    // longer reads; they must land before a next piece reuses the stages.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const float l_tot = l_run + swap_halves(l_run, lane);
    const float inv_l = 1.0f / l_tot;
    if (t0 == 0 && seg_end == seq_endx) {
      // ---- the whole sequence is in this piece: final output, fp32 ----
      float* out = a.o_lat + ((size_t)b * NH + head) * DC;
#pragma unroll
      for (int cb = 0; cb < DC / 32; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const floatx4 v = {O[cb][4 * q4 + 0] * inv_l, O[cb][4 * q4 + 1] * inv_l,
                             O[cb][4 * q4 + 2] * inv_l, O[cb][4 * q4 + 3] * inv_l};
          *(floatx4*)(out + 32 * cb + 8 * q4 + 4 * g32) = v;
          __builtin_amdgcn_sched_barrier(0);
        }
      if (g32 == 0 && a.lse) a.lse[(size_t)b * NH + head] = (m_ref + log2f(l_tot)) * kLn2;
      const int flag = (__any(ovf_any) ? 1 : 0) | (bad_tbl ? 2 : 0);
      if (lane == 0) a.flags[slot * WAVES + wave] = flag;
      pos = seg_end;
      continue;
    }
    // ---- emit the partial (O / l in fp16, m, l) of this piece ----
    // The normalised rows are weighted averages of cache rows, so fp16
    // (11-bit significand, finer than the bf16 weights and queries that bound
    // the result) holds them; a piece whose values exceed the fp16 range is
    // flagged for the fallback instead.  The values leave in the
    // accumulator's own lane order (the combine kernel reads that order), so
    // every store instruction writes 512 contiguous bytes.
    _Float16* po = a.part_o + (slot * NH + wave * HPW) * DC;   // this wave's 32 heads
    float amax = 0.f;
#pragma unroll
    for (int cb = 0; cb < DC / 32; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        halfx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = O[cb][4 * q4 + e] * inv_l;
          amax = fmaxf(amax, fabsf(x));
          v[e] = (_Float16)x;
        }
        *(halfx4*)(po + (cb * 4 + q4) * 256 + 4 * lane) = v;
        // one group of four at a time: converting all 256 accumulators at
        // once would need as many VGPRs
        __builtin_amdgcn_sched_barrier(0);
      }
    const int flag = (__any(ovf_any || amax > PART_MAX) ? 1 : 0) | (bad_tbl ? 2 : 0);
    if (lane == 0) a.flags[slot * WAVES + wave] = flag;
    if (g32 == 0) {
      float* pm = a.part_ml + (slot * NH + head) * 2;
      pm[0] = m_ref;
      pm[1] = l_tot;
    }
    pos = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Combine: merge the pieces of each (sequence, head) by log-sum-exp.
// ---------------------------------------------------------------------------
struct CombineArgs {
  const __bf16* q_lat;
  const __bf16* q_pe;
  const __bf16* cache;
  const uint8_t* cache8;   // 8-bit cache (codes) or NULL
  const float* scales;     // its row scales
  RowMap map;
  const int4* seqinfo;
  const int32_t* flags;
  const _Float16* part_o;
  const float* part_ml;
  float* o_lat;
  float* lse;
  int32_t* err_flag;
  int B;     // one per query token, as in the split kernel
  int n_q;
  int G;
  int cpw;   // column blocks per combine workgroup
  float scale_log2;
};

// Fallback for a flagged sequence: a plain online softmax over all its rows
// (the block's waves take alternate rows, 64 lanes across the 576 features,
// running max with rescale), then the wave states are merged.
constexpr int CMB_THREADS = 256;
constexpr int CMB_WAVES = CMB_THREADS / 64;

__device__ void recompute_head(const CombineArgs& a, int b, int h, int len) {
  __shared__ float st_m[CMB_WAVES], st_l[CMB_WAVES];
  __shared__ float st_o[CMB_WAVES][DC];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float q[DK / 64];
#pragma unroll
  for (int k = 0; k < DK / 64; ++k) {
    const int f = lane + 64 * k;
    q[k] = f < DC ? (float)a.q_lat[((size_t)b * NH + h) * DC + f]
                  : (float)a.q_pe[((size_t)b * NH + h) * DR + (f - DC)];
  }
  float acc[DC / 64];
#pragma unroll
  for (int k = 0; k < DC / 64; ++k) acc[k] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int seq = seq_of(b, a.n_q);
  for (int j = wave; j < len; j += CMB_WAVES) {
    // (every block of a sequence that reaches this fallback was validated by
    // the split kernel; the check only keeps a bad id from being followed)
    const int64_t rj = a.map.row(seq, j);
    if (rj < 0) continue;
    // the row's values: bf16, or 8-bit code value x row scale
    float rv[DK / 64];
    if (a.cache8) {
      const uint8_t* r8 = a.cache8 + (size_t)rj * DK;
      const float sc = a.scales[rj];
#pragma unroll
      for (int k = 0; k < DK / 64; ++k) rv[k] = __builtin_amdgcn_cvt_f32_fp8((int)r8[lane + 64 * k], 0) * sc;
    } else {
      const __bf16* r = a.cache + (size_t)rj * DK;
#pragma unroll
      for (int k = 0; k < DK / 64; ++k) rv[k] = (float)r[lane + 64 * k];
    }
    float sdot = 0.f;
#pragma unroll
    for (int k = 0; k < DK / 64; ++k) sdot += q[k] * rv[k];
    const float x = wave_sum(sdot) * a.scale_log2;
    const float mn = fmaxf(m, x);
    const float al = exp2f(m - mn);
    const float p = exp2f(x - mn);
    l = l * al + p;
#pragma unroll
    for (int k = 0; k < DC / 64; ++k) acc[k] = acc[k] * al + p * rv[k];
    m = mn;
  }
  if (lane == 0) { st_m[wave] = m; st_l[wave] = l; }
#pragma unroll
  for (int k = 0; k < DC / 64; ++k) st_o[wave][lane + 64 * k] = acc[k];
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < CMB_WAVES; ++w) M = fmaxf(M, st_m[w]);
  float wt[CMB_WAVES], L = 0.f;
#pragma unroll
  for (int w = 0; w < CMB_WAVES; ++w) {
    wt[w] = st_m[w] == -INFINITY ? 0.f : exp2f(st_m[w] - M);
    L += st_l[w] * wt[w];
  }
  float* out = a.o_lat + ((size_t)b * NH + h) * DC;
  for (int c = threadIdx.x; c < DC; c += blockDim.x) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < CMB_WAVES; ++w) v += st_o[w][c] * wt[w];
    out[c] = v / L;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[(size_t)b * NH + h] = (M + log2f(L)) * kLn2;
  __syncthreads();   // the LDS state is reused by the next head
}

// One workgroup per (32-head block, CPW 32-column blocks, sequence).  A
// piece's partial O is stored in the split kernel's accumulator lane order:
// for each (piece, head block, column block) 2 KiB of fp16, entry t =
// 64 q4 + lane holding columns 8 q4 + 4 (lane / 32) + [0, 4) of head
// lane % 32.  Lane t of this block reads entry t of every piece, so each
// piece is one contiguous 2 KiB read.  Each lane forms the weights of its
// own head itself: with the common max M of the pieces' m, piece i weighs
// 2^(m_i - M) l_i.  Pieces over empty ranges carry m = -inf, l = 0 and zero
// rows.  The result is transposed through LDS so that every head's 32
// columns leave as one 128-byte store.  The combine is bound by the latency
// of its partial loads, not by their bytes: a sequence of up to 16 pieces
// has the loads of several column blocks (a "round", up to CMB_MAXLD
// 8-byte loads per lane) issued together, and a round's results leave
// through LDS behind one barrier.  Sequences of more than 16 pieces take a
// grouped loop over the pieces instead (cmb_large).
constexpr int CMB_HB = HPW;          // heads per block (one split-kernel wave)
constexpr int CMB_CB = 32;           // columns per block (one accumulator tile)
constexpr int CMB_NCB = DC / CMB_CB;
constexpr size_t CMB_SLOT = (size_t)NH * DC;   // fp16 per slot
constexpr size_t CMB_CHUNK = (size_t)CMB_HB * CMB_CB;   // fp16 per (piece, head block, column block)
constexpr int CMB_MAXLD = 32;        // partial loads per lane in one round
constexpr int CMB_MAXCG = 8;         // column blocks per round
constexpr int CMB_ROW = CMB_MAXCG * CMB_CB + 1;   // LDS row of the transpose (odd: no bank conflicts)

// Writes CG normalised 32 x 32 blocks (column blocks cb .. cb + CG - 1)
// through LDS: lane t holds head t % 32, columns 8 (t / 64) + 4 ((t / 32) % 2)
// ..+4 of each block; every head's CG 32 consecutive columns are written as
// 16-byte pieces, eight lanes per 128 bytes.
template <int CG>
__device__ __forceinline__ void cmb_store(const CombineArgs& a, float (*s_out)[CMB_ROW], int b, int hb, int cb,
                                          const float4 (&acc)[CG], float inv) {
  const int tid = threadIdx.x;
  const int n32 = tid & 31, cols = 8 * (tid >> 6) + 4 * ((tid >> 5) & 1);
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    s_out[n32][CMB_CB * c + cols + 0] = acc[c].x * inv;
    s_out[n32][CMB_CB * c + cols + 1] = acc[c].y * inv;
    s_out[n32][CMB_CB * c + cols + 2] = acc[c].z * inv;
    s_out[n32][CMB_CB * c + cols + 3] = acc[c].w * inv;
  }
  __syncthreads();
  const int h_r = tid >> 3, c_r = (tid & 7) * 4;
  float* row = a.o_lat + ((size_t)b * NH + hb * CMB_HB + h_r) * DC + cb * CMB_CB + c_r;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const float* sv = &s_out[h_r][CMB_CB * c + c_r];
    *(float4*)(row + CMB_CB * c) = make_float4(sv[0], sv[1], sv[2], sv[3]);
  }
  __syncthreads();   // s_out is reused by the next round
}

// Loads of one round: column blocks cb .. cb + CG - 1 of every piece (piece
// indices past the last are clamped to it; their weight is 0).
template <int NP, int CG>
__device__ __forceinline__ void cmb_round_load(const _Float16* po, int cb, int npiece, halfx4 (&v)[CG][NP]) {
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int k = i < npiece ? i : npiece - 1;
      v[c][i] = *(const halfx4*)(po + (size_t)k * CMB_SLOT + (size_t)(cb + c) * CMB_CHUNK);
    }
}

// Up to NP pieces, CG column blocks per round.  The (m, l) of all pieces and
// the first round's partials are loaded before the fallback flags are
// examined, so both share one round trip.  Returns 1 if the sequence must
// take the fallback, 2 if one workgroup held it whole (the split kernel wrote
// its result), else 0 with M, L of this lane's head.
template <int NP, int CG>
__device__ int cmb_small(const CombineArgs& a, float (*s_out)[CMB_ROW], int b, int hb, int cb0, int cpw,
                         int npiece, size_t slot0, int flag, float& M, float& L) {
  static_assert(NP * CG <= CMB_MAXLD && CG <= CMB_MAXCG, "round size");
  const int tid = threadIdx.x, n32 = tid & 31;
  const float2* ml = (const float2*)a.part_ml + slot0 * NH + hb * CMB_HB + n32;
  const _Float16* po = a.part_o + slot0 * CMB_SLOT + (size_t)hb * CMB_NCB * CMB_CHUNK + 4 * tid;
  float2 m2[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) m2[i] = ml[(size_t)(i < npiece ? i : npiece - 1) * NH];
  halfx4 v[CG][NP];
  cmb_round_load<NP, CG>(po, cb0, npiece, v);
  if (__syncthreads_or(flag)) return 1;
  if (npiece == 1) return 2;
  float w[NP];
  M = -INFINITY;
#pragma unroll
  for (int i = 0; i < NP; ++i)
    if (i < npiece) M = fmaxf(M, m2[i].x);
  L = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const bool use = i < npiece && m2[i].x != -INFINITY;
    w[i] = use ? exp2f(m2[i].x - M) * m2[i].y : 0.f;   // 2^(m - M) l
    L += w[i];
  }
  const float inv = 1.f / L;
  for (int r = 0; r < cpw; r += CG) {
    if (r > 0) cmb_round_load<NP, CG>(po, cb0 + r, npiece, v);
    float4 acc[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        acc[c].x += w[i] * (float)v[c][i][0];
        acc[c].y += w[i] * (float)v[c][i][1];
        acc[c].z += w[i] * (float)v[c][i][2];
        acc[c].w += w[i] * (float)v[c][i][3];
      }
    }
    cmb_store<CG>(a, s_out, b, hb, cb0 + r, acc, inv);
  }
  return 0;
}

// The round size for NP pieces: as many of the workgroup's cpw column blocks
// as CMB_MAXLD loads per lane allow, 16 for sequences of 9 to 16 pieces
// (cpw and the round size are powers of two).  Measured per call (ragged
// B = 64 / layer B = 128 / uniform B = 16, rounds of at most 16 or 32
// loads): 16.7 / 18.1 / 8.7 and 15.4 / 17.1 / 9.1 us, against 19.0 / 22.7 /
// 8.4 with one column block per round; more than 16 pieces (long B = 8)
// went from 11.6 to 12.0 us in one round of 32 and take the grouped loop.
template <int NP>
__device__ int cmb_small_any(const CombineArgs& a, float (*s_out)[CMB_ROW], int b, int hb, int cb0, int cpw,
                             int npiece, size_t slot0, int flag, float& M, float& L) {
  constexpr int LD = NP >= 16 ? 16 : CMB_MAXLD;
  constexpr int MAXCG = LD / NP < CMB_MAXCG ? LD / NP : CMB_MAXCG;
  const int cg = cpw < MAXCG ? cpw : MAXCG;
  if constexpr (MAXCG >= 8)
    if (cg == 8) return cmb_small<NP, 8>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
  if constexpr (MAXCG >= 4)
    if (cg == 4) return cmb_small<NP, 4>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
  if constexpr (MAXCG >= 2)
    if (cg == 2) return cmb_small<NP, 2>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
  return cmb_small<NP, 1>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
}

// Any number of pieces: one pass per column block, 16 pieces at a time,
// the running max M moving only between groups (rescaling what was
// accumulated so far).
__device__ void cmb_large(const CombineArgs& a, float (*s_out)[CMB_ROW], int b, int hb, int cb0, int cpw,
                          int npiece, size_t slot0, float& M, float& L) {
  const int tid = threadIdx.x, n32 = tid & 31;
  const float2* ml = (const float2*)a.part_ml + slot0 * NH + hb * CMB_HB + n32;
  constexpr int GRP = 16;
  for (int c = 0; c < cpw; ++c) {
    const _Float16* po = a.part_o + slot0 * CMB_SLOT + ((size_t)hb * CMB_NCB + cb0 + c) * CMB_CHUNK + 4 * tid;
    float4 acc[1] = {make_float4(0.f, 0.f, 0.f, 0.f)};
    M = -INFINITY;
    L = 0.f;
    for (int i = 0; i < npiece; i += GRP) {
      halfx4 v[GRP];
      float2 m2[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const int k = i + j < npiece ? i + j : npiece - 1;   // clamped; weight 0 below
        v[j] = *(const halfx4*)(po + (size_t)k * CMB_SLOT);
        m2[j] = ml[(size_t)k * NH];
      }
      float Mg = M;
#pragma unroll
      for (int j = 0; j < GRP; ++j)
        if (i + j < npiece) Mg = fmaxf(Mg, m2[j].x);
      if (Mg > M) {   // M = -inf only before any finite piece: nothing to rescale
        const float r = M == -INFINITY ? 0.f : exp2f(M - Mg);
        acc[0].x *= r;
        acc[0].y *= r;
        acc[0].z *= r;
        acc[0].w *= r;
        L *= r;
        M = Mg;
      }
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const bool use = i + j < npiece && m2[j].x != -INFINITY;
        const float w = use ? exp2f(m2[j].x - M) * m2[j].y : 0.f;   // 2^(m - M) l
        L += w;
        acc[0].x += w * (float)v[j][0];
        acc[0].y += w * (float)v[j][1];
        acc[0].z += w * (float)v[j][2];
        acc[0].w += w * (float)v[j][3];
      }
    }
    cmb_store<1>(a, s_out, b, hb, cb0 + c, acc, 1.f / L);
  }
}

__global__ void __launch_bounds__(CMB_THREADS) k_combine(CombineArgs a) {
  __shared__ float s_out[CMB_HB][CMB_ROW];
  const int cpw = a.cpw;
  const int ngrp = CMB_NCB / cpw;
  const int hb = blockIdx.x / ngrp, cb0 = (blockIdx.x % ngrp) * cpw, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int4 si = a.seqinfo[b];   // first range, ranges, valid length
  // this block's share of the result set to NaN
  auto write_nan = [&]() {
    const float nan = __builtin_nanf("");
    const int h_r = tid >> 3, c_r = (tid & 7) * 4;
    for (int c = 0; c < cpw; ++c) {
      float4* out = (float4*)(a.o_lat + ((size_t)b * NH + hb * CMB_HB + h_r) * DC + (cb0 + c) * CMB_CB + c_r);
      *out = make_float4(nan, nan, nan, nan);
    }
    if (cb0 == 0 && tid < CMB_HB && a.lse) a.lse[(size_t)b * NH + hb * CMB_HB + tid] = nan;
  };
  if (si.z <= 0) {   // invalid length: NaN result (the error flag is set)
    write_nan();
    return;
  }
  const int npiece = si.y;
  const size_t slot0 = (size_t)si.x + (size_t)b;   // piece i is slot slot0 + i
  int flag = 0;
  for (int k = tid; k < npiece * WAVES; k += CMB_THREADS) flag |= a.flags[slot0 * WAVES + k];
  // A flagged piece (reached by every thread of the block together): a block
  // id outside the pool (bit 2) makes the sequence's result NaN; otherwise a
  // piece overflowed (bit 1) and the blocks of this head block share its
  // heads out and recompute whole rows each.
  auto fallback = [&]() {
    if (__syncthreads_or(flag & 2)) {
      write_nan();
      if (tid == 0 && a.err_flag) atomicOr(a.err_flag, MLA_DEVERR_TABLE);
      return;
    }
    for (int k = blockIdx.x % ngrp; k < CMB_HB; k += ngrp) recompute_head(a, b, hb * CMB_HB + k, si.z);
  };
  float M, L;
  int r;
  if (npiece <= 2) r = cmb_small_any<2>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
  else if (npiece <= 4) r = cmb_small_any<4>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
  else if (npiece <= 8) r = cmb_small_any<8>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
  else if (npiece <= 16) r = cmb_small_any<16>(a, s_out, b, hb, cb0, cpw, npiece, slot0, flag, M, L);
  else {
    r = __syncthreads_or(flag) ? 1 : 0;
    if (r == 0) cmb_large(a, s_out, b, hb, cb0, cpw, npiece, slot0, M, L);
  }
  if (r == 1) return fallback();
  if (r == 2) return;   // one workgroup held the whole sequence and wrote it
  if (cb0 == 0 && tid < CMB_HB && a.lse) {
    // lanes 0..31 hold heads 0..31 (n32 = tid); M, L are per head
    a.lse[(size_t)b * NH + hb * CMB_HB + tid] = (M + log2f(L)) * kLn2;
  }
}

constexpr int MAX_G = 256;   // split workgroups per call (one per compute unit)

int choose_groups(int64_t total_rows_hint, int num_cu) {
  int64_t g = (total_rows_hint + MIN_ROWS_PER_WG - 1) / MIN_ROWS_PER_WG;
  if (g < 1) g = 1;
  if (g > num_cu) g = num_cu;
  if (g > MAX_G) g = MAX_G;
  return (int)g;
}

}  // namespace

bool decode_v3_supported(const Shape& s) {
  return s.bf16 && s.n_h == NH && s.d_c == DC && s.d_r == DR;
}

// B sequences of n_q query tokens each run as B n_q sequences (one per token,
// see seq_of); the rows they process add up to about n_q times the hint.
size_t decode_v3_workspace(const Shape&, int B, int n_q, int64_t total_rows_hint, int num_cu) {
  return partial_layout(B * n_q, choose_groups(total_rows_hint * n_q, num_cu)).bytes;
}

hipError_t launch_decode_v3(const Shape& s, int B_seq, int n_q, const void* q_lat, const void* q_pe,
                            const void* cache, const float* scales, const RowMap& map, const int32_t* lens,
                            int64_t total_rows_hint, float* o_lat, float* lse, int32_t* err_flag,
                            void* ws, size_t, int num_cu, hipStream_t st) {
  const int B = B_seq * n_q;
  const int G = choose_groups(total_rows_hint * n_q, num_cu);
  const PartialLayout L = partial_layout(B, G);
  char* w = (char*)ws;
  int64_t* prefix = (int64_t*)(w + L.pre_off);
  WgRec* rec = (WgRec*)(w + L.rec_off);
  int4* seqinfo = (int4*)(w + L.si_off);
  int32_t* flags = (int32_t*)(w + L.flag_off);
  SplitArgs a;
  a.rec = rec;
  a.lens = lens;
  a.err_flag = err_flag;
  a.seqinfo = seqinfo;
  a.flags = flags;
  a.o_lat = o_lat;
  a.lse = lse;
  a.q_lat = (const __bf16*)q_lat;
  a.q_pe = (const __bf16*)q_pe;
  a.cache = (const char*)cache;
  a.scales = scales;
  a.map = map;
  a.prefix = prefix;
  a.part_o = (_Float16*)(w + L.o_off);
  a.part_ml = (float*)(w + L.ml_off);
  a.B = B;
  a.n_q = n_q;
  a.G = G;
  a.scale_log2 = s.scale * kLog2e;
  // 8-bit cache (scales given), paged pool, or contiguous bf16 cache
  const int mode = scales ? 2 : map.paged() ? 1 : 0;
  if (B <= SPL_MAXB) {
    if (mode == 2) k_split<true, 2><<<G, THREADS, 0, st>>>(a);
    else if (mode == 1) k_split<true, 1><<<G, THREADS, 0, st>>>(a);
    else k_split<true, 0><<<G, THREADS, 0, st>>>(a);
  } else {
    k_sched<<<1, SCHED_THREADS, 0, st>>>(B, n_q, G, map, lens, prefix, (int32_t*)(w + L.cnt_off), rec, seqinfo,
                                         err_flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mode == 2) k_split<false, 2><<<G, THREADS, 0, st>>>(a);
    else if (mode == 1) k_split<false, 1><<<G, THREADS, 0, st>>>(a);
    else k_split<false, 0><<<G, THREADS, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CombineArgs c;
  c.q_lat = a.q_lat;
  c.q_pe = a.q_pe;
  c.cache = (const __bf16*)cache;
  c.cache8 = scales ? (const uint8_t*)cache : nullptr;
  c.scales = scales;
  c.map = map;
  c.err_flag = err_flag;
  c.seqinfo = seqinfo;
  c.flags = flags;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  c.o_lat = o_lat;
  c.lse = lse;
  c.B = B;
  c.n_q = n_q;
  c.G = G;
  c.scale_log2 = a.scale_log2;
  // about G / B pieces per sequence: fewer pieces, more column blocks per
  // workgroup (CPW * pieces loads in flight per lane), but not so many that
  // large batches lose workgroups, and at most four since the loads of a
  // workgroup's blocks are issued in rounds.  Measured (mean of 300 calls,
  // this rule against halved and doubled thresholds): ragged B=64 (G/B = 4)
  // 16.4 us at 4 against 17.4 at 8 and 26.1 at 16; layer B=128 (2) 17.4 at 4
  // against 19.7 at 8; uniform B=16 (16) 8.7 at 2 against 9.9 at 1 and 9.5 at
  // 4; long B=8 (32) 11.6 at 1 against 13.5 at 2.
  int cpw = 1;
  while (cpw < 4 && cpw * G < 32 * B && cpw * B < 512) cpw *= 2;
  c.cpw = cpw;
  k_combine<<<dim3((NH / CMB_HB) * (CMB_NCB / cpw), B), CMB_THREADS, 0, st>>>(c);
  return hipGetLastError();
}

}  // namespace mla
