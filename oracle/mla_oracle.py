"""Plain fp64 CPU oracle for one MLA decode step.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this module.  The HIP library never calls it and it
shares no code, constants or helpers with ``head_latent_attention_16_amd``.

What it computes, and where the pages say so
--------------------------------------------
Page abbreviations used in the citations below:

* [MLA-struct]  "MLA模型结构详解：从公式到推理代码" (gentlecold.top) -- the
  formal source: equations, data-flow chart, both inference branches and a
  shape-by-shape worked decode step.
* [MLA-visual]  "DeepSeek-V2 MLA" visual reading (syt-nju.github.io,
  files/visual-reading/deepseek-v2-mla) -- method narrative and the per-token
  cache-size table.
* [KV-2026]     "MLA latent attention / KV cache" (ai.saiita.com.cn,
  mla-latent-attention-kv-cache-2026) -- DeepSeek-V3 cache arithmetic.
* [KV-slim]     "给 KV Cache 瘦身：MQA · GQA · MLA" (bilibili-notes) -- the
  7B example and the 576-numbers / ~70 KB figure.

The oracle deliberately takes the *un-absorbed* route ([MLA-struct], section
"MLA 的核心结构"): the content keys and values of every cached token are
materialised explicitly (k^C = W^UK c^KV, v^C = W^UV c^KV), the per-head query
and key are the concatenations [q^C; RoPE(q^R)] and [k^C; k^R] with k^R shared
by all heads ([MLA-struct], section "RoPE 为什么要解耦"), the score is their dot
product times the softmax scale, the softmax is the textbook two-pass one, and
the head output is the probability-weighted sum of the explicit values.  The
absorbed route used by the GPU path is an exact re-association of this
([MLA-struct], section "为什么矩阵吸收很关键", the two associativity identities),
so the two must agree up to rounding.

Readings of points the pages leave open:

* softmax scale = 1 / sqrt(d_h + d_R) applied to the sum of the content and
  RoPE scores (the pages write "x scale" without a value);
* RoPE is rotate-half with base 10000: theta_i = base^(-2 i / d_R), pairs
  (i, i + d_R/2); angles pos * theta_i are formed in fp64;
* the cache always holds the already-rotated k^R (the worked example writes the
  RoPE'd k_pe into pe_cache);
* no causal mask is applied to a single decode query: it sits at a position
  >= every cached row, so the mask passes everything; with n_q new tokens
  (latent_attention_causal) they are the last n_q cached rows and token i
  sees rows 0 .. T - n_q + i;
* the latent ``norm(...)`` of the inference code is not applied by default
  (c^KV = W^DKV h_t is the equation's definition); when asked for, it is a
  root-mean-square norm with a per-feature weight and eps = 1e-6 (the pages
  name neither its kind nor its epsilon) on c^KV before caching, which is
  where the pages print it.  The same norm on the compressed query c^Q
  before its up-projection is a reading BEYOND the pages (no page prints a
  norm on c^Q; it completes the query path of a DeepSeek-V3-style layer by
  symmetry with the latent side) and is applied only when asked for;
* weights are [out, in] row-major: W_UK [n_h, d_h, d_c], W_UV [n_h, d_v, d_c],
  W_UQ rows head-major with [d_h content | d_R rope] per head, W_O input index
  h * d_v + v ("flatten head").

Everything is float64.  Inputs given as bf16 bit patterns are widened exactly
by the caller before they reach this module.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "rope",
    "softmax_two_pass",
    "explicit_kv",
    "attend_explicit",
    "decode_explicit",
    "absorb_query",
    "latent_attention",
    "latent_attention_causal",
    "prefill_explicit",
    "append_rows",
    "rms_norm",
    "query_path",
    "project_out",
    "layer_step",
    "cache_elems_per_token_layer",
    "cache_bytes_per_token",
    "paged_rows",
    "pool_bytes_per_token",
    "e4m3_value",
    "e4m3_encode",
    "e4m3_decode",
    "row_scale_exponent",
    "quantize_rows",
    "dequantize_rows",
]


# ---------------------------------------------------------------------------
# RoPE on the decoupled positional part.
# [MLA-visual], section on decoupled RoPE: the query RoPE part is per head,
# the key RoPE part k^R = RoPE(W^KR h_t) is one vector shared by all heads.
# Rotation convention (rotate-half, base 10000, fp64 angles) is a reading.
# ---------------------------------------------------------------------------
def rope(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis of ``x`` (length d_R, even) by position ``pos``.

    x'_i        = x_i cos(pos*theta_i) - x_{i+d/2} sin(pos*theta_i)
    x'_{i+d/2}  = x_{i+d/2} cos(pos*theta_i) + x_i sin(pos*theta_i)
    theta_i     = base ** (-2 i / d),  i < d/2.
    ``pos`` broadcasts against x.shape[:-1].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE dimension must be even")
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * cos - hi * sin, hi * cos + lo * sin], axis=-1)


# ---------------------------------------------------------------------------
# Softmax: textbook two-pass form over the last axis.
# [MLA-struct], worked example step 4: score -> (causal mask) -> softmax.
# ---------------------------------------------------------------------------
def softmax_two_pass(s: np.ndarray):
    """Return (p, lse) with p = exp(s - max) / sum exp(s - max)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    p = e / z
    lse = (m + np.log(z))[..., 0]
    return p, lse


# ---------------------------------------------------------------------------
# The un-absorbed ("naive") route.
# [MLA-struct], section "MLA 的核心结构": k^C_t = W^UK c^KV_t, v^C_t = W^UV c^KV_t;
# section "RoPE 为什么要解耦": q_{t,i} = [q^C_{t,i}; q^R_{t,i}],
# k_{t,i} = [k^C_{t,i}; k^R_t] with k^R_t shared by every head i.
# ---------------------------------------------------------------------------
def explicit_kv(c: np.ndarray, k_rot: np.ndarray, W_UK_h: np.ndarray, W_UV_h: np.ndarray):
    """Explicit keys [T, d_h + d_R] and values [T, d_v] of one head."""
    k_content = c @ W_UK_h.T          # k^C_j = W^UK c_j   -> [T, d_h]
    v_content = c @ W_UV_h.T          # v^C_j = W^UV c_j   -> [T, d_v]
    keys = np.concatenate([k_content, k_rot], axis=1)
    return keys, v_content


def attend_explicit(q_C_h, q_R_rot_h, c, k_rot, W_UK_h, W_UV_h, scale):
    """One head, one query, explicit K/V.

    Returns (o_h [d_v], o_lat_h [d_c], lse_h).  ``o_lat_h`` = sum_j p_j c_j is
    the latent aggregate that W^UV maps to o_h ([MLA-struct], value identity);
    it is returned so the GPU's latent output can be compared directly.
    """
    keys, values = explicit_kv(c, k_rot, W_UK_h, W_UV_h)
    q = np.concatenate([q_C_h, q_R_rot_h])           # [d_h + d_R]
    s = (keys @ q) * scale                            # [T]
    p, lse = softmax_two_pass(s)
    o_h = p @ values                                  # sum_j p_j v_j
    o_lat_h = p @ c                                   # sum_j p_j c_j
    return o_h, o_lat_h, float(lse)


def decode_explicit(q_C, q_R, pos, c, k_rot, W_UK, W_UV, scale, base=10000.0):
    """All heads of one sequence.

    q_C [n_h, d_h], q_R [n_h, d_R] (not yet rotated), pos = query position,
    c [T, d_c], k_rot [T, d_R] (rotated keys as cached), W_UK [n_h, d_h, d_c],
    W_UV [n_h, d_v, d_c].  Returns o [n_h, d_v], o_lat [n_h, d_c], lse [n_h].
    """
    c = np.asarray(c, np.float64)
    k_rot = np.asarray(k_rot, np.float64)
    q_R_rot = rope(q_R, pos, base)
    n_h = q_C.shape[0]
    o = np.empty((n_h, W_UV.shape[1]))
    o_lat = np.empty((n_h, c.shape[1]))
    lse = np.empty(n_h)
    for h in range(n_h):
        o[h], o_lat[h], lse[h] = attend_explicit(
            q_C[h], q_R_rot[h], c, k_rot, W_UK[h], W_UV[h], scale)
    return o, o_lat, lse


# ---------------------------------------------------------------------------
# What the latent-space call computes, stated as its own definition:
# o_lat[h] = sum_j softmax_j(scale (q_lat[h].c_j + q_pe[h].k^R_j)) c_j.
# [MLA-struct], worked example steps 4-5 (score_C + score_R, z = A . kv_cache).
# ---------------------------------------------------------------------------
def absorb_query(q_C, W_UK):
    """q_lat[h] = W_UK[h]^T q_C[h]  ([MLA-struct], key identity q.(W c) = (q W).c)."""
    return np.einsum("hk,hkc->hc", np.asarray(q_C, np.float64), np.asarray(W_UK, np.float64))


def latent_attention(q_lat, q_pe, c, k_rot, scale):
    """o_lat [n_h, d_c] and lse [n_h] from latent queries (q_pe already rotated)."""
    s = (np.asarray(q_lat, np.float64) @ np.asarray(c, np.float64).T
         + np.asarray(q_pe, np.float64) @ np.asarray(k_rot, np.float64).T) * scale
    p, lse = softmax_two_pass(s)
    return p @ np.asarray(c, np.float64), lse


# ---------------------------------------------------------------------------
# Several new tokens in one step.  [MLA-struct], worked example step 4 and the
# inference code's mask: with more than one new token the score matrix gets a
# causal mask before the softmax, so a token sees every earlier row and itself
# but none of the tokens after it.  Reading: the n_q new tokens are the last
# n_q of the T cached rows (appended before the attention), token i sits at
# row T - n_q + i, and a masked score is -inf (weight exactly 0).
# ---------------------------------------------------------------------------
def latent_attention_causal(q_lat, q_pe, c, k_rot, scale):
    """o_lat [n_q, n_h, d_c] and lse [n_q, n_h] for q_lat [n_q, n_h, d_c],
    q_pe [n_q, n_h, d_R] (rotated) over the T rows c [T, d_c], k_rot [T, d_R]."""
    q_lat = np.asarray(q_lat, np.float64)
    q_pe = np.asarray(q_pe, np.float64)
    c = np.asarray(c, np.float64)
    k_rot = np.asarray(k_rot, np.float64)
    n_q, T = q_lat.shape[0], c.shape[0]
    s = (q_lat @ c.T + q_pe @ k_rot.T) * scale                       # [n_q, n_h, T]
    row = np.arange(T)[None, :]
    tok = (T - n_q + np.arange(n_q))[:, None]
    s = np.where((row <= tok)[:, None, :], s, -np.inf)                # causal mask
    p, lse = softmax_two_pass(s)
    return p @ c, lse


# ---------------------------------------------------------------------------
# The un-absorbed ("naive") branch for many new tokens.  [MLA-struct], section
# "结合 DeepSeek 推理代码看 MLA", the `naive` branch: the full keys and values
# are recovered from the latent (k^C = W^UK c, v = W^UV c), the key gets the
# shared RoPE key concatenated, scores are [q^C; q^R] . [k^C; k^R], and the
# output is the weighted sum of the explicit values; worked example step 4:
# the scores are causally masked.  Reading: the n_q new tokens are the last n_q
# of the T cached rows (appended first, as in the absorbed branch), token i
# sits at row T - n_q + i and sees rows 0 .. T - n_q + i; q^R is rotated at
# the token's position.
# ---------------------------------------------------------------------------
def prefill_explicit(q_C, q_R, c, k_rot, W_UK, W_UV, scale, base=10000.0):
    """o [n_q, n_h, d_v] and lse [n_q, n_h] of n_q new tokens of one sequence.

    q_C [n_q, n_h, d_h], q_R [n_q, n_h, d_R] (not rotated), c [T, d_c],
    k_rot [T, d_R] (rotated, as cached), W_UK [n_h, d_h, d_c], W_UV [n_h, d_v, d_c].
    """
    q_C = np.asarray(q_C, np.float64)
    q_R = np.asarray(q_R, np.float64)
    c = np.asarray(c, np.float64)
    k_rot = np.asarray(k_rot, np.float64)
    n_q, n_h = q_C.shape[0], q_C.shape[1]
    T = c.shape[0]
    pos = T - n_q + np.arange(n_q)                                   # token positions = rows
    q_R_rot = rope(q_R, pos[:, None], base)                          # [n_q, n_h, d_R]
    o = np.empty((n_q, n_h, np.asarray(W_UV).shape[1]))
    lse = np.empty((n_q, n_h))
    visible = np.arange(T)[None, :] <= pos[:, None]                 # causal mask [n_q, T]
    for h in range(n_h):
        keys, values = explicit_kv(c, k_rot, np.asarray(W_UK[h], np.float64), np.asarray(W_UV[h], np.float64))
        q = np.concatenate([q_C[:, h], q_R_rot[:, h]], axis=1)       # [n_q, d_h + d_R]
        s = np.where(visible, (q @ keys.T) * scale, -np.inf)
        p, lse[:, h] = softmax_two_pass(s)
        o[:, h] = p @ values
    return o, lse


# ---------------------------------------------------------------------------
# New-token projections and the cache row.
# [MLA-struct], section "MLA 的核心结构": c^KV_t = W^DKV h_t; c^Q_t = W^DQ h_t,
# q^C_t = W^UQ c^Q_t; worked example steps 1-3 (q split per head into
# [128 content | 64 rope]; kv_and_pe split into latent and k_pe; RoPE(k_pe);
# write at index start_pos).
# ---------------------------------------------------------------------------
def append_rows(x, W_DKV, W_KR, pos, base=10000.0, kv_norm_w=None, eps=1e-6):
    """Cache rows for new tokens: (c_new [n, d_c], k_rot [n, d_R]).

    x [n, d_model] are the new tokens' hidden states, pos [n] their positions.
    With ``kv_norm_w`` the latent is normalised before it is cached (rms_norm).
    """
    x = np.asarray(x, np.float64)
    c_new = x @ np.asarray(W_DKV, np.float64).T
    if kv_norm_w is not None:
        c_new = rms_norm(c_new, kv_norm_w, eps)
    k_raw = x @ np.asarray(W_KR, np.float64).T
    return c_new, rope(k_raw, np.asarray(pos), base)


# ---------------------------------------------------------------------------
# The latent norms.  [MLA-struct], section "结合 DeepSeek 推理代码看 MLA" (both
# branches of the pseudocode) and worked example step 3: the compressed latent
# is passed through norm(kv_latent) before it is cached; the pages name
# neither the kind of norm nor its epsilon.  Reading: root-mean-square norm
# over the latent's features with a learned per-feature weight,
# y = x / sqrt(mean(x^2) + eps) * w, eps = 1e-6.
# The norm on the compressed query c^Q (query_path with q_norm_w) is a
# reading beyond the pages: none of them prints it.
# ---------------------------------------------------------------------------
def rms_norm(x, w, eps=1e-6):
    """Row-wise x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, np.float64)


def query_path(h, W_DQ, W_UQ, n_h, d_h, d_r, q_norm_w=None, eps=1e-6):
    """q_C [n, n_h, d_h] and q_R [n, n_h, d_R] (un-rotated) from hidden states h [n, d].

    With ``W_DQ`` None the query is projected directly (q = W_UQ h), as in a
    configuration without query compression.  With ``q_norm_w`` the compressed
    query c^Q is normalised (rms_norm) before the up-projection.
    """
    c_Q = np.asarray(h, np.float64)
    if W_DQ is not None:
        c_Q = c_Q @ np.asarray(W_DQ, np.float64).T
        if q_norm_w is not None:
            c_Q = rms_norm(c_Q, q_norm_w, eps)
    q = (c_Q @ np.asarray(W_UQ, np.float64).T).reshape(len(c_Q), n_h, d_h + d_r)
    return q[..., :d_h], q[..., d_h:]


# ---------------------------------------------------------------------------
# Output side.  [MLA-struct], worked example step 5: o = W^UV z per head, then
# flatten heads and apply the output projection W_O.
# ---------------------------------------------------------------------------
def project_out(o_lat, W_UV, W_O=None):
    """o [B, n_h, d_v] = W_UV[h] o_lat[b, h];  u [B, d_model] = W_O flatten(o[b])."""
    o_lat = np.asarray(o_lat, np.float64)
    o = np.einsum("hvc,bhc->bhv", np.asarray(W_UV, np.float64), o_lat)
    u = None
    if W_O is not None:
        u = o.reshape(o.shape[0], -1) @ np.asarray(W_O, np.float64).T
    return o, u


def layer_step(h_t, W, prior_c, prior_k, dims, scale, base=10000.0, seqs=None, norms=False, eps=1e-6):
    """One full MLA decode layer step for selected sequences, explicit route.

    h_t [B, d_model]; W: dict with W_DQ, W_UQ, W_DKV, W_KR, W_UK, W_UV, W_O;
    prior_c[b] [T_b, d_c], prior_k[b] [T_b, d_R] (rotated).  The new token of
    sequence b sits at position t_b = T_b: its row is appended at that index,
    and the query uses the same position ([MLA-struct], worked example step 3:
    write at start_pos, visible length start_pos + 1).  With ``norms`` the
    latent norm on c^KV (W["kv_norm_w"], printed on the pages) and the
    query-side norm on c^Q (W["q_norm_w"], a reading beyond the pages) are
    applied.
    Returns dict of per-sequence results keyed by b.
    """
    n_h, d_h, d_r = dims["n_h"], dims["d_h"], dims["d_r"]
    seqs = range(len(h_t)) if seqs is None else seqs
    out = {}
    for b in seqs:
        x = np.asarray(h_t[b:b + 1], np.float64)
        t = len(prior_c[b])
        q_C, q_R = query_path(x, W["W_DQ"], W["W_UQ"], n_h, d_h, d_r,
                              q_norm_w=W["q_norm_w"] if norms else None, eps=eps)
        c_new, k_new = append_rows(x, W["W_DKV"], W["W_KR"], [t], base,
                                   kv_norm_w=W["kv_norm_w"] if norms else None, eps=eps)
        c_all = np.concatenate([np.asarray(prior_c[b], np.float64), c_new])
        k_all = np.concatenate([np.asarray(prior_k[b], np.float64), k_new])
        o, o_lat, lse = decode_explicit(q_C[0], q_R[0], t, c_all, k_all,
                                        W["W_UK"], W["W_UV"], scale, base)
        u = o.reshape(1, -1) @ np.asarray(W["W_O"], np.float64).T
        out[b] = dict(o=o, o_lat=o_lat, lse=lse, u=u[0], c_new=c_new[0], k_new=k_new[0],
                      q_C=q_C[0], q_R=q_R[0])
    return out


# ---------------------------------------------------------------------------
# A paged pool shared by the layers of a model.  [KV-2026], section "MLA 的思路：
# 把 KV 压缩成一个小向量": the model-wide cache per token is layers x (d_c + d_R)
# numbers; [KV-slim], section "易错点与常见追问", names PagedAttention-style memory
# management without describing it.  Reading: fixed-size blocks of
# block_rows rows, a block table per (layer, sequence); row t of a sequence is
# row t % block_rows of block table[t // block_rows].
# ---------------------------------------------------------------------------
def paged_rows(pool, table_row, n, block_rows):
    """Rows 0 .. n-1 of one sequence of a paged pool, in order: row t is pool
    row table_row[t // block_rows] * block_rows + t % block_rows."""
    pool = np.asarray(pool)
    t = np.arange(n, dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[t // block_rows]
    if n and (blocks.min() < 0 or blocks.max() * block_rows >= len(pool)):
        raise IndexError("block id outside the pool")
    return pool[blocks * block_rows + t % block_rows]


def pool_bytes_per_token(layers: int, d_c: int, d_r: int, bytes_per_elem: int) -> int:
    """Bytes one token occupies across the layers of a pooled latent cache."""
    return layers * (d_c + d_r) * bytes_per_elem


# ---------------------------------------------------------------------------
# A low-precision latent cache.  [KV-slim], section "易错点与常见追问", names KV
# quantisation (INT8/INT4) as a companion of MLA; [MLA-struct], worked example
# step 3 notes that precision and quantisation change the real memory
# footprint.  Neither page fixes a format or a scale.  Reading: each cached row
# [c^KV | k^R] (d_c + d_R numbers) is stored as 8-bit floats in the OCP E4M3
# format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
# finite 448, smallest subnormal 2^-9, codes 0x7F / 0xFF are NaN) with one
# power-of-two scale per row, s = 2^e with e the smallest integer for which
# amax <= 448 * 2^e (amax = max |x| over the row; e clamped to [-120, 120]; an
# all-zero row has s = 1), and code = E4M3(x / s) rounded to nearest, ties to
# even.  A power-of-two scale keeps x / s exact and makes value(code) * s
# exactly representable in bf16, so a kernel may feed the dequantised row to
# bf16 matrix cores without a further rounding.  A row dequantises to
# value(code) * s.
# ---------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    """The number an E4M3 code stands for (the format's definition)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_POS = np.array([e4m3_value(c) for c in range(0x7F)])   # codes 0x00 .. 0x7E, increasing


def e4m3_encode(x) -> np.ndarray:
    """Round float32 values to E4M3 codes: nearest, ties to the even code,
    |x| >= 448 saturating to +-448 (NaN maps to 0x7F)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    neg = np.signbit(x)
    i = np.searchsorted(_E4M3_POS, np.minimum(a, 448.0))       # first code >= a
    i = np.minimum(i, 0x7E)
    lo = np.maximum(i - 1, 0)
    exact = _E4M3_POS[i] == a
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[i] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 0))
    code = np.where(exact | pick_hi, i, lo)
    code = np.where(a >= 448.0, 0x7E, code).astype(np.uint8)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    table = np.array([e4m3_value(c) for c in range(256)])
    return table[np.asarray(codes, dtype=np.uint8)]


def row_scale_exponent(amax: float) -> int:
    """Smallest e with amax <= 448 * 2^e (amax > 0), clamped to [-120, 120]."""
    m, E = math.frexp(float(amax))            # amax = m 2^E, 0.5 <= m < 1
    e = E - 9 if m <= 0.875 else E - 8        # 448 = 0.875 * 2^9
    return max(-120, min(120, e))


def quantize_rows(x):
    """Per-row E4M3 quantisation of float32 rows with a power-of-two scale:
    (codes uint8 [n, D], scales float32 [n])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    e = np.array([row_scale_exponent(a) if a > 0 else 0 for a in amax.reshape(-1)], np.int64).reshape(amax.shape)
    scale = np.ldexp(np.float32(1), e).astype(np.float32)
    v = np.ldexp(x.astype(np.float64), -e[..., None])          # exact: a power-of-two rescale
    return e4m3_encode(np.clip(v, -448.0, 448.0).astype(np.float32)), scale


def dequantize_rows(codes, scales):
    """value(code) * scale, in float64."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


# ---------------------------------------------------------------------------
# Cache-size arithmetic.  [MLA-visual], cache-size table: MHA 2 n_h d_h l,
# GQA 2 n_g d_h l, MQA 2 d_h l, MLA (d_c + d_h^R) l elements per token.
# ---------------------------------------------------------------------------
def cache_elems_per_token_layer(kind: str, n_h=None, d_h=None, n_g=None, d_c=None, d_r=None) -> int:
    if kind == "mha":
        return 2 * n_h * d_h
    if kind == "gqa":
        return 2 * n_g * d_h
    if kind == "mqa":
        return 2 * d_h
    if kind == "mla":
        return d_c + d_r
    raise ValueError(kind)


def cache_bytes_per_token(kind: str, layers: int, bytes_per_elem: int, **dims) -> int:
    return layers * bytes_per_elem * cache_elems_per_token_layer(kind, **dims)


def scale_for(d_h: int, d_r: int) -> float:
    """Softmax scale reading: 1 / sqrt(d_h + d_R)."""
    return 1.0 / math.sqrt(d_h + d_r)
