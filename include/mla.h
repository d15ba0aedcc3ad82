/*
 * mla.h -- C ABI of libmla.so: one decode step of Multi-head Latent Attention
 * (MLA) over a compressed latent KV cache, computed in latent space by matrix
 * absorption, on AMD MI355X (gfx950).
 *
 * The problem as the pages state it ("MLA模型结构详解：从公式到推理代码",
 * gentlecold.top, sections "MLA 的核心结构" and "一个实际推理示例"): given the new
 * token's hidden state h_t, the weights W^DKV, W^KR, W^UK, W^UV, W^O (and for a
 * compressed query W^DQ, W^UQ) and a cache holding, for every past token, only
 * the latent c^KV (d_c numbers) and the shared RoPE key k^R (d_R numbers),
 * produce the layer output.  The four calls below are the steps of that path:
 *
 *   mla_absorb_q      query side: q = W^UQ W^DQ h_t (or q given), then the
 *                     latent query q_lat = W^UK^T q^C per head and q_pe = RoPE(q^R)
 *   mla_append_cache  new row [c^KV | RoPE(k^R)] written at each sequence's end
 *   mla_decode_attn   o_lat = softmax(scale (q_lat.c + q_pe.k^R)) . c  (the hot loop)
 *                     (mla_decode_attn_causal: n_q new tokens per sequence,
 *                     causally masked among themselves)
 *   mla_project_out   o = W^UV o_lat per head, u = W^O flatten(o)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer to row-major, contiguous memory
 *   that the caller allocated and owns.  The library allocates nothing and
 *   keeps no per-call state; it caches device properties per device only.
 * - ``stream`` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues work on it and returns; there is no host synchronisation inside.
 * - Every call validates its arguments on the host first.  A return of
 *   MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE, MLA_ERR_WORKSPACE or
 *   MLA_ERR_DEVICE means nothing was enqueued and no output was touched.
 *   MLA_ERR_LAUNCH (the HIP runtime refused a launch) can come after earlier
 *   kernels of the same call were already enqueued: scratch, and outputs
 *   those kernels write, are then unspecified until the call succeeds.
 * - Element types follow ``dims->dtype``: with MLA_DT_BF16 every ``void*``
 *   tensor is bf16, with MLA_DT_F32 it is float32.  Outputs typed ``float*``
 *   are always float32.  Index arrays are int32.
 * - Conditions only the device can see (a length out of range, a full cache
 *   region) are reported through an optional device ``err_flag`` (int32):
 *   the kernels OR in the MLA_DEVERR_* bits below; the caller clears it.
 * - Calls that overlap on one stream are ordered; calls on different streams
 *   that write the same buffers race.
 *
 * Cache layout: ``cache`` is [rows, d_c + d_R]; row r = [c^KV (d_c) | k^R (d_R)]
 * with k^R already rotated to the row's position (the worked example caches the
 * RoPE'd k_pe).  Sequence b owns rows offsets[b] .. offsets[b+1]-1 (its
 * capacity) and uses the first lens[b] of them, the row at index t holding the
 * token at position t.  For V3 dims in bf16 a row is 1152 bytes.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds mla_decode_attn_causal, mla_absorb_q_normed, mla_append_cache_normed;
 * the decode entry points reject more than 65535 query tokens up front.
 * 3: adds mla_decode_attn_noalloc, the paged pool (mla_decode_attn_paged,
 * mla_append_cache_paged), MLA_DEVERR_TABLE and the 8-bit cache
 * (mla_append_cache_fp8, mla_decode_attn_fp8) and the un-absorbed prefill
 * (mla_prefill_attn). */
#define MLA_ABI_VERSION 3

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,       /* a required pointer is NULL                          */
  MLA_ERR_SHAPE = 2,      /* a size is out of range or dims are unsupported      */
  MLA_ERR_DTYPE = 3,      /* unknown dims->dtype                                 */
  MLA_ERR_WORKSPACE = 4,  /* ws_bytes smaller than the matching *_workspace()    */
  MLA_ERR_LAUNCH = 5,     /* the HIP runtime refused a launch                    */
  MLA_ERR_DEVICE = 6      /* no usable gfx950 device is current                  */
} mla_status_t;

typedef enum { MLA_DT_BF16 = 0, MLA_DT_F32 = 1 } mla_dtype_t;

/* Device-side error bits OR-ed into *err_flag. */
#define MLA_DEVERR_LENS 1       /* lens[b] < 1 or lens[b] > offsets[b+1]-offsets[b]   */
#define MLA_DEVERR_OVERFLOW 2   /* an appended row would not fit in its region        */
#define MLA_DEVERR_TABLE 4      /* a paged block id is outside [0, num_blocks)        */

/* Model dimensions ("MLA模型结构详解", section "结合 DeepSeek 推理代码看 MLA":
 * n_heads, kv_lora_rank = d_c, qk_nope_head_dim = d_h, qk_rope_head_dim = d_R,
 * v_head_dim = d_v; q_lora_rank = d_q).  DeepSeek-V3: 128, 512, 64, 128, 128,
 * d_model 7168, d_q 1536. */
typedef struct {
  int32_t n_h;            /* query heads                                     */
  int32_t d_c;            /* latent width (kv_lora_rank)                     */
  int32_t d_r;            /* decoupled RoPE width, even                      */
  int32_t d_h;            /* per-head content query/key width                */
  int32_t d_v;            /* per-head value width                            */
  int32_t d_model;        /* hidden size (0 if no projection from h_t is used) */
  int32_t d_q;            /* query latent width (0: no query compression)    */
  float rope_base;        /* RoPE base; 10000                                */
  float softmax_scale;    /* <= 0 selects 1/sqrt(d_h + d_r)                  */
  int32_t dtype;          /* mla_dtype_t                                     */
} mla_dims_t;

/* Query side ("MLA模型结构详解", section "MLA 的核心结构": c^Q = W^DQ h_t,
 * q^C = W^UQ c^Q; worked example steps 1 and 4; key identity
 * q^C.(W^UK c) = (q^C W^UK).c; RoPE on q^R per head).
 *
 * Source of the per-head query [q^C (d_h) | q^R (d_R)]:
 *   h_t != NULL: q = W_UQ (W_DQ h_t), h_t [B, d_model], W_DQ [d_q, d_model],
 *                W_UQ [n_h*(d_h+d_r), d_q] with rows head-major, each head
 *                [d_h content | d_r rope].  With dims->d_q == 0, W_DQ must be
 *                NULL and q = W_UQ h_t, W_UQ [n_h*(d_h+d_r), d_model].
 *   h_t == NULL: q [B, n_h, d_h + d_r] is given.
 * Outputs: q_lat [B, n_h, d_c] with q_lat[b,h,:] = W_UK[h]^T q^C[b,h,:]
 *          (W_UK [n_h, d_h, d_c]), q_pe [B, n_h, d_r] = RoPE(q^R[b,h,:], pos[b])
 *          (rotate-half, theta_i = base^(-2i/d_r), angle formed in fp64),
 *          both in dims->dtype, rounded to nearest even once from fp32.
 * Precision from h_t with bf16 storage: the products accumulate in fp32, and
 * c^Q and q are rounded once to bf16 before the next product (as in bf16
 * inference) wherever the matrix-core layer runs (N a multiple of 32, K a
 * multiple of 256); other shapes keep them in fp32.
 * pos [B] int32 device: the query position (the new token's index).
 * ws: device scratch of at least mla_absorb_q_workspace(dims, B, h_t != NULL)
 *     bytes (may be NULL when that is 0). */
mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t B, const void* h_t, const void* W_DQ,
                          const void* W_UQ, const void* q, const void* W_UK, const int32_t* pos,
                          void* q_lat, void* q_pe, void* ws, size_t ws_bytes, void* stream);
size_t mla_absorb_q_workspace(const mla_dims_t* dims, int32_t B, int32_t from_hidden);

/* mla_absorb_q from h_t with a norm on the compressed query.  No page prints
 * this norm: "MLA模型结构详解" (section "结合 DeepSeek 推理代码看 MLA" and
 * worked example step 3) shows norm(kv_latent) on the latent side only.  It
 * is a reading beyond the pages that completes a DeepSeek-V3-style query path
 * with the same root-mean-square norm as the latent side (kind and epsilon
 * are readings too):
 *   c^Q = W_DQ h_t,  c^Q <- c^Q / sqrt(mean(c^Q^2) + eps) * q_norm_w,  q = W_UQ c^Q,
 * then as mla_absorb_q.  q_norm_w [d_q] in dims->dtype; the norm runs in fp32
 * on the fp32 c^Q (its result is then rounded as c^Q is in mla_absorb_q).  Needs d_q >= 1, h_t, W_DQ, q_norm_w (MLA_ERR_NULL), and a
 * finite eps >= 0 (MLA_ERR_SHAPE).  ws: mla_absorb_q_workspace(dims, B, 1). */
mla_status_t mla_absorb_q_normed(const mla_dims_t* dims, int32_t B, const void* h_t,
                                 const void* W_DQ, const void* q_norm_w, float eps,
                                 const void* W_UQ, const void* W_UK, const int32_t* pos,
                                 void* q_lat, void* q_pe, void* ws, size_t ws_bytes, void* stream);

/* Append n_new tokens per sequence ("MLA模型结构详解", worked example steps 2-3:
 * kv_and_pe = wkv_a(x) split into the latent and k_pe, RoPE(k_pe), written at
 * index start_pos; c^KV = W^DKV h_t, k^R = RoPE(W^KR h_t)).
 * For b < B, i < n_new: row offsets[b] + lens[b] + i  <-  [c | RoPE(k, lens[b] + i)]
 *   with (c, k) = (W_DKV x, W_KR x), x = h_t[b, i, :] (h_t [B, n_new, d_model],
 *   W_DKV [d_c, d_model], W_KR [d_r, d_model]); or, if h_t == NULL, (c, k) taken
 *   from kv_raw[b, i, :] = [c | un-rotated k] (kv_raw [B, n_new, d_c + d_r];
 *   the c part is copied bit-exactly).
 * Then lens[b] += n_new.  No other row is written.  If the rows do not fit in
 * the region (lens[b] + n_new > offsets[b+1] - offsets[b]) nothing is written
 * for b, lens[b] is unchanged and MLA_DEVERR_OVERFLOW is set.
 * ws: at least mla_append_cache_workspace(dims, B, n_new, h_t != NULL) bytes. */
mla_status_t mla_append_cache(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                              const void* W_DKV, const void* W_KR, const void* kv_raw, void* cache,
                              const int32_t* offsets, int32_t* lens, int32_t* err_flag, void* ws,
                              size_t ws_bytes, void* stream);
size_t mla_append_cache_workspace(const mla_dims_t* dims, int32_t B, int32_t n_new,
                                  int32_t from_hidden);

/* mla_append_cache from h_t with the latent norm of the inference code
 * ("MLA模型结构详解", section "结合 DeepSeek 推理代码看 MLA" and worked example
 * step 3: cache(norm(kv_latent)); kind and epsilon unstated there, read as a
 * root-mean-square norm):
 *   c^KV = W_DKV x,  c^KV <- c^KV / sqrt(mean(c^KV^2) + eps) * kv_norm_w,
 * k^R = RoPE(W_KR x) as in mla_append_cache (not normalised).  kv_norm_w [d_c]
 * in dims->dtype; the norm runs in fp32 before the row is rounded to the
 * storage type.  Needs h_t, W_DKV, W_KR, kv_norm_w (MLA_ERR_NULL) and a finite
 * eps >= 0 (MLA_ERR_SHAPE).  ws: mla_append_cache_workspace(dims, B, n_new, 1). */
mla_status_t mla_append_cache_normed(const mla_dims_t* dims, int32_t B, int32_t n_new,
                                     const void* h_t, const void* W_DKV, const void* kv_norm_w,
                                     float eps, const void* W_KR, void* cache,
                                     const int32_t* offsets, int32_t* lens, int32_t* err_flag,
                                     void* ws, size_t ws_bytes, void* stream);

/* Latent-space attention of one query per sequence ("MLA模型结构详解", worked
 * example steps 4-5: score = (score_C + score_R) x scale, softmax, z = A . kv_cache;
 * value identity sum_j a_j W^UV c_j = W^UV sum_j a_j c_j).
 *   o_lat[b,h,:] = sum_{j < lens[b]} p_j c_j,
 *   p = softmax_j( scale * (q_lat[b,h,:].c_j + q_pe[b,h,:].kR_j) ),
 *   (c_j, kR_j) = row offsets[b] + j,  scale = dims->softmax_scale or 1/sqrt(d_h+d_r).
 *   lse[b,h] = log sum_j exp(scale * score_j)  (natural log; lse may be NULL).
 * q_lat [B, n_h, d_c], q_pe [B, n_h, d_r] in dims->dtype; o_lat [B, n_h, d_c] fp32.
 * No mask: every cached row precedes the query.  lens[b] must be in
 * [1, offsets[b+1]-offsets[b]]; a sequence violating it gets NaN outputs and
 * MLA_DEVERR_LENS.  B <= 65535 (else MLA_ERR_SHAPE).  total_rows_hint (> 0) is
 * the expected sum of lens and only sizes the launch (the number of row
 * ranges the batch is split into): any hint gives a correct result, but the
 * split points, and with them the low-order bits of o_lat and lse, can change
 * with it (within the same rounding bounds).
 * ws: at least mla_decode_attn_workspace(dims, B, total_rows_hint) bytes. */
mla_status_t mla_decode_attn(const mla_dims_t* dims, int32_t B, const void* q_lat,
                             const void* q_pe, const void* cache, const int32_t* offsets,
                             const int32_t* lens, int64_t total_rows_hint, float* o_lat,
                             float* lse, int32_t* err_flag, void* ws, size_t ws_bytes,
                             void* stream);
size_t mla_decode_attn_workspace(const mla_dims_t* dims, int32_t B, int64_t total_rows_hint);

/* mla_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, kernels and results as mla_decode_attn
 * with the same arguments, but the scratch is a fixed array inside the
 * library (52 MiB on each device it runs on, held until the process ends)
 * instead of a caller workspace.  The call allocates and frees nothing.
 * Limit: the scratch mla_decode_attn_workspace(dims, B, total_rows_hint)
 * would ask for must fit in 52 MiB (at V3 dims on a 256-CU MI355X: up to
 * 156 sequences; other dims need none); larger requests return
 * MLA_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one device shares that device's
 * scratch: calls that overlap on one device (different streams or threads)
 * race and must be serialised by the caller. */
mla_status_t mla_decode_attn_noalloc(const mla_dims_t* dims, int32_t B, const void* q_lat,
                                     const void* q_pe, const void* cache, const int32_t* offsets,
                                     const int32_t* lens, int64_t total_rows_hint, float* o_lat,
                                     float* lse, int32_t* err_flag, void* stream);

/* Several new tokens per sequence in one step ("MLA模型结构详解", worked
 * example step 4: with more than one new token the inference code masks the
 * scores causally before the softmax).  The step's n_q tokens are the last
 * n_q of the lens[b] cached rows (appended first, e.g. by mla_append_cache
 * with n_new = n_q), and token i < n_q attends to rows 0 .. lens[b] - n_q + i:
 *   o_lat[b,i,h,:] = sum_{j <= lens[b]-n_q+i} p_j c_j,
 *   p = softmax_j( scale * (q_lat[b,i,h,:].c_j + q_pe[b,i,h,:].kR_j) ),
 *   lse[b,i,h] as in mla_decode_attn.
 * q_lat [B, n_q, n_h, d_c], q_pe [B, n_q, n_h, d_r] in dims->dtype; o_lat
 * [B, n_q, n_h, d_c] fp32; lse [B, n_q, n_h] fp32 or NULL.  n_q = 1 is exactly
 * mla_decode_attn.  Needs 1 <= n_q and B * n_q <= 65535 (else MLA_ERR_SHAPE);
 * lens[b] must be in [n_q, offsets[b+1]-offsets[b]], else all n_q tokens of
 * sequence b get NaN outputs and MLA_DEVERR_LENS.  total_rows_hint (> 0) is
 * the expected sum of lens.  Each token is run as a sequence of its own over
 * its rows (so a row is streamed once per token that sees it; neighbouring
 * tokens of a sequence share the reads through the cache hierarchy).
 * ws: at least mla_decode_attn_causal_workspace(dims, B, n_q, total_rows_hint)
 * bytes. */
mla_status_t mla_decode_attn_causal(const mla_dims_t* dims, int32_t B, int32_t n_q,
                                    const void* q_lat, const void* q_pe, const void* cache,
                                    const int32_t* offsets, const int32_t* lens,
                                    int64_t total_rows_hint, float* o_lat, float* lse,
                                    int32_t* err_flag, void* ws, size_t ws_bytes, void* stream);
size_t mla_decode_attn_causal_workspace(const mla_dims_t* dims, int32_t B, int32_t n_q,
                                        int64_t total_rows_hint);

/* Many new tokens at once (prefill) by the un-absorbed branch
 * ("MLA模型结构详解", section "结合 DeepSeek 推理代码看 MLA": the naive branch
 * recovers the full keys and values, k^C = W^UK c and v = W^UV c, and scores
 * [q^C; q^R] . [k^C; k^R]; worked example step 4: causal mask).  For a long
 * prompt the explicit keys cost d_h + d_R + d_v per (token, key, head) against
 * the absorbed route's 2 d_c + d_R, and the up-projection is paid once per
 * cached row.
 *   The step's n_q tokens are the last n_q of the lens[b] cached rows (append
 *   them first, e.g. mla_append_cache with n_new = n_q); token i sits at row
 *   p = lens[b] - n_q + i and sees rows 0 .. p:
 *   o[b,i,h,:] = sum_{j <= p} softmax_j(scale [q^C; RoPE(q^R, p)] . [W_UK[h] c_j; kR_j]) W_UV[h] c_j
 *   lse[b,i,h] = log sum_j exp(scale ...).
 * q [B, n_q, n_h, d_h + d_r] (per head [content | rope], q^R NOT yet rotated:
 * it is rotated at p) in dims->dtype; cache [cache_rows, d_c + d_r] with
 * sequence b at rows offsets[b] ..; W_UK [n_h, d_h, d_c], W_UV [n_h, d_v, d_c];
 * o [B, n_q, n_h, d_v] fp32; lse [B, n_q, n_h] fp32 or NULL.  Every cache row
 * 0 .. cache_rows - 1 is up-projected (into the workspace, fp16), so pass the
 * rows the batch occupies.  V3 dims in bf16 only (else MLA_ERR_SHAPE);
 * B <= 65535.  lens[b] must be in [n_q, offsets[b+1] - offsets[b]] with
 * offsets[b] + lens[b] <= cache_rows, else sequence b's outputs are NaN and
 * MLA_DEVERR_LENS is set.
 * The explicit keys, values and queries are held in fp16 (finer than bf16,
 * so a token that sees few keys keeps the tolerance); they must lie within
 * the fp16 range.
 * ws: at least mla_prefill_attn_workspace(dims, B, n_q, cache_rows) bytes
 * (cache_rows x n_h x (d_h + d_v) x 2 for the explicit keys and values). */
mla_status_t mla_prefill_attn(const mla_dims_t* dims, int32_t B, int32_t n_q, const void* q, const void* cache,
                              int64_t cache_rows, const int32_t* offsets, const int32_t* lens, const void* W_UK,
                              const void* W_UV, float* o, float* lse, int32_t* err_flag, void* ws,
                              size_t ws_bytes, void* stream);
size_t mla_prefill_attn_workspace(const mla_dims_t* dims, int32_t B, int32_t n_q, int64_t cache_rows);

/* Paged latent cache pool, shared by the layers of a model.
 *
 * The pages give the per-token cache of a whole model as layers x (d_c + d_R)
 * numbers ("MLA latent attention / KV cache", section "MLA 的思路：把 KV 压缩成一个
 * 小向量": 61 x 576 x 2 B, about 68 KB per token for DeepSeek-V3) and name
 * PagedAttention-style memory management as the system-level companion of
 * MLA ("给 KV Cache 瘦身：MQA · GQA · MLA", section "易错点与常见追问") without
 * describing it.  Reading: the cache rows of every layer and sequence live in
 * one pool of fixed-size blocks, pool [num_blocks, block_rows, d_c + d_R] in
 * dims->dtype; each (layer, sequence) owns a list of blocks, and a layer's
 * call gets that layer's block table, block_table [B, max_blocks] int32
 * (device): row t of sequence b is row t % block_rows of block
 * block_table[b * max_blocks + t / block_rows].  block_rows is a power of two
 * >= 32 (at most 2^20) and max_blocks * block_rows <= 2^31 - 1; else
 * MLA_ERR_SHAPE.  Only the entries of the blocks a call touches are read;
 * an id outside [0, num_blocks) is never followed (MLA_DEVERR_TABLE; the
 * sequence's outputs are NaN, or nothing is appended for it).
 *
 * mla_decode_attn_paged: mla_decode_attn over the pool (lens[b] <=
 * max_blocks * block_rows, else MLA_DEVERR_LENS).  Same results as
 * mla_decode_attn over a contiguous cache holding the same rows, with the
 * same total_rows_hint (the split points depend on lens only); ws: at least
 * mla_decode_attn_workspace(dims, B, total_rows_hint) bytes.
 * mla_append_cache_paged: mla_append_cache into the pool (row lens[b] + i of
 * sequence b; capacity max_blocks * block_rows); ws: at least
 * mla_append_cache_workspace(dims, B, n_new, h_t != NULL) bytes. */
mla_status_t mla_decode_attn_paged(const mla_dims_t* dims, int32_t B, const void* q_lat,
                                   const void* q_pe, const void* pool, int32_t num_blocks,
                                   int32_t block_rows, const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* lens, int64_t total_rows_hint, float* o_lat,
                                   float* lse, int32_t* err_flag, void* ws, size_t ws_bytes,
                                   void* stream);
mla_status_t mla_append_cache_paged(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                                    const void* W_DKV, const void* W_KR, const void* kv_raw, void* pool,
                                    int32_t num_blocks, int32_t block_rows, const int32_t* block_table,
                                    int32_t max_blocks, int32_t* lens, int32_t* err_flag, void* ws,
                                    size_t ws_bytes, void* stream);

/* Low-precision latent cache.  "给 KV Cache 瘦身：MQA · GQA · MLA" (section
 * "易错点与常见追问") names KV quantisation as the companion of MLA, and
 * "MLA模型结构详解" (worked example step 3) notes that precision changes the
 * real footprint; neither fixes a format.  Reading: each row [c^KV | k^R] is
 * stored as d_c + d_R OCP E4M3 codes (1 byte each; largest finite 448) with
 * one power-of-two scale per row (stored as fp32): scale = 2^e with e the
 * smallest integer for which amax <= 448 2^e (clamped to [-120, 120]), amax
 * = max |x| over the row's d_c + d_R values (k^R after its rotation), and
 * code = E4M3(x / scale) rounded to nearest even; an all-zero row gets codes
 * 0 and scale 1.  A row then holds (d_c + d_R) + 4 bytes: 580 at V3 dims,
 * about half of the 1152-byte bf16 row.  The row's value is value(code) x
 * scale, exactly representable in bf16, which is what the decode feeds to the
 * matrix cores.
 *
 * mla_append_cache_fp8: mla_append_cache writing codes into cache8 [rows,
 * d_c + d_r] (uint8) and the row's scale into scales [rows] (fp32); h_t,
 * the weights and kv_raw are in dims->dtype.
 * mla_decode_attn_fp8: mla_decode_attn over such a cache (q_lat, q_pe in
 * dims->dtype); ws: at least mla_decode_attn_workspace(dims, B, hint) bytes.
 * Inputs must be finite. */
mla_status_t mla_append_cache_fp8(const mla_dims_t* dims, int32_t B, int32_t n_new, const void* h_t,
                                  const void* W_DKV, const void* W_KR, const void* kv_raw, uint8_t* cache8,
                                  float* scales, const int32_t* offsets, int32_t* lens, int32_t* err_flag,
                                  void* ws, size_t ws_bytes, void* stream);
mla_status_t mla_decode_attn_fp8(const mla_dims_t* dims, int32_t B, const void* q_lat, const void* q_pe,
                                 const uint8_t* cache8, const float* scales, const int32_t* offsets,
                                 const int32_t* lens, int64_t total_rows_hint, float* o_lat, float* lse,
                                 int32_t* err_flag, void* ws, size_t ws_bytes, void* stream);

/* Output side ("MLA模型结构详解", worked example step 5: multiply by the value
 * part of wkv_b per head, flatten heads, output projection).
 *   o[b,h,:] = W_UV[h] o_lat[b,h,:]      W_UV [n_h, d_v, d_c], o [B, n_h, d_v] fp32
 *   u[b,:]   = W_O flatten(o[b])          W_O [d_model, n_h*d_v] (input index h*d_v + v),
 *                                         u [B, d_model] fp32
 * o or u may be NULL to skip storing it (W_O may be NULL when u is NULL).  With
 * bf16 weights the products run on bf16 matrix cores with fp32 accumulation;
 * the fp32 o_lat enters W_UV as two bf16 operands, the rounded value
 * hi = bf16(x) and the remainder lo = bf16(x - hi), both multiplied by the
 * weight, so it keeps about 16 significant bits; o enters W_O rounded once to
 * bf16 (as in bf16 inference) wherever the matrix-core layer runs (d_model a
 * multiple of 32, n_h d_v a multiple of 256), in fp32 otherwise; the o
 * stored for the caller is the fp32 product.
 * ws: at least mla_project_out_workspace(dims, B, u != NULL) bytes. */
mla_status_t mla_project_out(const mla_dims_t* dims, int32_t B, const float* o_lat,
                             const void* W_UV, const void* W_O, float* o, float* u, void* ws,
                             size_t ws_bytes, void* stream);
size_t mla_project_out_workspace(const mla_dims_t* dims, int32_t B, int32_t with_u);

/* Bytes of one cache row: (d_c + d_r) * element size (1152 for V3 bf16);
 * 0 if dims is NULL or invalid. */
size_t mla_cache_row_bytes(const mla_dims_t* dims);

/* Static, NUL-terminated description of a status code (any int32 value;
 * values that are not an mla_status_t give "unknown status"). */
const char* mla_status_string(int32_t status);

/* MLA_ABI_VERSION of the built library. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
