"""Seeded synthetic MLA decode workloads.

This module only draws numbers and lays them out; it holds none of the
method's arithmetic (no RoPE, no projection, no attention), so both the fp64
oracle and the HIP path can take their inputs from it.

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload, seed 0):
draw order is lengths, cache c_KV, cache k_R, q_C, q_R, then the weights in the
order W_DQ, W_UQ, W_DKV, W_KR, W_UK, W_UV, W_O, then h_t -- each only if the
workload has it.  Normal draws are ``standard_normal(float32) * std``; bf16
workloads round them to bf16 with round-to-nearest-even.  Ragged lengths are
integers drawn uniformly with both ends included.  Weight std is
fan_in ** -0.5 (the "N(0, 1/fan_in)" of the workload statement read as a
variance).  Large arrays are drawn in row chunks from the same stream.

The five workloads mirror the statement of the decode problem at DeepSeek-V3
dimensions (n_h=128, d_c=512, d_R=64, d_h=d_v=128, d=7168, d_q=1536):

* ``tiny``     fp32, B=1, n_h=4, d_c=32, d_R=8, d_h=d_v=16, T=64, query at T;
                 k_R drawn raw and rotated when appended at positions 0..T-1.
* ``uniform``  B=16, T=4096, attention only.
* ``ragged``   B=64, T uniform in [1024, 32768], attention only.
* ``long``     B=8, T=131072, attention only.
* ``layer``    full layer step, B=128, prior T uniform in [512, 8192], h_t given.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

V3_DIMS = dict(n_h=128, d_c=512, d_r=64, d_h=128, d_v=128, d_model=7168, d_q=1536)
TINY_DIMS = dict(n_h=4, d_c=32, d_r=8, d_h=16, d_v=16, d_model=0, d_q=0)

_CHUNK = 1 << 22  # elements per draw chunk


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


@dataclasses.dataclass
class Workload:
    """Host-side arrays of one workload.

    Floating arrays are stored as bf16 bit patterns (uint16) when
    ``dtype == 'bf16'`` and as float32 when ``dtype == 'f32'``.
    ``cache`` is [rows, d_c + d_R] with sequence b occupying rows
    ``offsets[b] .. offsets[b] + lens[b] - 1`` and capacity
    ``offsets[b+1] - offsets[b]``.  For attention-only workloads the query
    position of sequence b is ``lens[b]``.
    """

    name: str
    dtype: str
    dims: Dict[str, int]
    B: int
    lens: np.ndarray             # int32 [B] rows already in the cache
    offsets: np.ndarray          # int32 [B+1] region starts (+ end)
    cache: np.ndarray            # [rows, d_c + d_R]; k_R part already rotated
    q_C: Optional[np.ndarray] = None       # [B, n_h, d_h]
    q_R: Optional[np.ndarray] = None       # [B, n_h, d_R] (not rotated)
    W: Dict[str, np.ndarray] = dataclasses.field(default_factory=dict)
    h_t: Optional[np.ndarray] = None       # [B, d_model]
    kv_raw: Optional[np.ndarray] = None    # tiny: [B, T, d_c + d_R] un-rotated rows
    seed: int = 0
    n_q: int = 1                 # query tokens per sequence (q_C, q_R hold B n_q rows)

    @property
    def row_elems(self) -> int:
        return self.dims["d_c"] + self.dims["d_r"]

    def f64(self, a: np.ndarray) -> np.ndarray:
        """Exact float64 view of a stored array."""
        if a.dtype == np.uint16:
            return bf16_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)

    def seq_rows(self, b: int) -> np.ndarray:
        o = int(self.offsets[b])
        return self.cache[o:o + int(self.lens[b])]

    @property
    def total_rows(self) -> int:
        return int(np.sum(self.lens, dtype=np.int64))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _offsets(caps: np.ndarray) -> np.ndarray:
    off = np.zeros(len(caps) + 1, dtype=np.int64)
    off[1:] = np.cumsum(caps)
    if off[-1] >= 2 ** 31:
        raise ValueError("cache rows exceed int32 offsets")
    return off.astype(np.int32)


def _cache(rng, lens, caps, d_c, d_r, dtype):
    """Cache region with c_KV ~ N(0,1) then k_R ~ N(0,1) drawn for the used rows."""
    offsets = _offsets(caps)
    rows = int(offsets[-1])
    used = int(np.sum(lens, dtype=np.int64))
    c = _normal(rng, (used, d_c), 1.0)
    k = _normal(rng, (used, d_r), 1.0)
    cache = np.zeros((rows, d_c + d_r), dtype=np.uint16 if dtype == "bf16" else np.float32)
    src = 0
    for b, t in enumerate(lens):
        o = int(offsets[b])
        cache[o:o + t, :d_c] = _store(c[src:src + t], dtype)
        cache[o:o + t, d_c:] = _store(k[src:src + t], dtype)
        src += t
    return offsets, cache


def tiny(seed: int = 0) -> Workload:
    """fp32, B=1, n_h=4, d_c=32, d_R=8, d_h=d_v=16, T=64; rows appended raw."""
    d = dict(TINY_DIMS)
    B, T = 1, 64
    rng = np.random.default_rng(seed)
    lens = np.full(B, T, dtype=np.int32)
    c = _normal(rng, (B * T, d["d_c"]), 1.0)
    k = _normal(rng, (B * T, d["d_r"]), 1.0)
    q_C = _normal(rng, (B, d["n_h"], d["d_h"]), 1.0)
    q_R = _normal(rng, (B, d["n_h"], d["d_r"]), 1.0)
    W_UK = _normal(rng, (d["n_h"], d["d_h"], d["d_c"]), d["d_c"] ** -0.5)
    W_UV = _normal(rng, (d["n_h"], d["d_v"], d["d_c"]), d["d_c"] ** -0.5)
    kv_raw = np.concatenate([c, k], axis=1).reshape(B, T, -1).astype(np.float32)
    offsets = _offsets(np.full(B, T, dtype=np.int64))
    # The cache starts empty: rows are appended (and k_R rotated) at positions 0..T-1.
    cache = np.full((int(offsets[-1]), d["d_c"] + d["d_r"]), np.nan, dtype=np.float32)
    return Workload("tiny", "f32", d, B, lens, offsets, cache, q_C=q_C, q_R=q_R,
                    W=dict(W_UK=W_UK, W_UV=W_UV), kv_raw=kv_raw, seed=seed)


def attention_only(name: str, B: int, lens: np.ndarray, rng, seed: int) -> Workload:
    d = dict(V3_DIMS)
    lens = np.asarray(lens, dtype=np.int32)
    offsets, cache = _cache(rng, lens, lens.astype(np.int64), d["d_c"], d["d_r"], "bf16")
    q_C = bf16_bits(_normal(rng, (B, d["n_h"], d["d_h"]), 1.0))
    q_R = bf16_bits(_normal(rng, (B, d["n_h"], d["d_r"]), 1.0))
    W_UK = bf16_bits(_normal(rng, (d["n_h"], d["d_h"], d["d_c"]), d["d_c"] ** -0.5))
    W_UV = bf16_bits(_normal(rng, (d["n_h"], d["d_v"], d["d_c"]), d["d_c"] ** -0.5))
    return Workload(name, "bf16", d, B, lens, offsets, cache, q_C=q_C, q_R=q_R,
                    W=dict(W_UK=W_UK, W_UV=W_UV), seed=seed)


def uniform(seed: int = 0, B: int = 16, T: int = 4096) -> Workload:
    rng = np.random.default_rng(seed)
    return attention_only("uniform", B, np.full(B, T, dtype=np.int32), rng, seed)


def ragged(seed: int = 0, B: int = 64, lo: int = 1024, hi: int = 32768) -> Workload:
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    return attention_only("ragged", B, lens, rng, seed)


def long_context(seed: int = 0, B: int = 8, T: int = 131072) -> Workload:
    rng = np.random.default_rng(seed)
    return attention_only("long", B, np.full(B, T, dtype=np.int32), rng, seed)


def causal(seed: int = 0, B: int = 16, T: int = 4096, n_q: int = 4) -> Workload:
    """Several new tokens per sequence: the uniform cache, whose last n_q rows
    are the step's tokens, and queries for B n_q tokens (q_C [B n_q, n_h, d_h],
    token i of sequence b in row b n_q + i, at position T - n_q + i)."""
    d = dict(V3_DIMS)
    rng = np.random.default_rng(seed)
    lens = np.full(B, T, dtype=np.int32)
    offsets, cache = _cache(rng, lens, lens.astype(np.int64), d["d_c"], d["d_r"], "bf16")
    q_C = bf16_bits(_normal(rng, (B * n_q, d["n_h"], d["d_h"]), 1.0))
    q_R = bf16_bits(_normal(rng, (B * n_q, d["n_h"], d["d_r"]), 1.0))
    W_UK = bf16_bits(_normal(rng, (d["n_h"], d["d_h"], d["d_c"]), d["d_c"] ** -0.5))
    W_UV = bf16_bits(_normal(rng, (d["n_h"], d["d_v"], d["d_c"]), d["d_c"] ** -0.5))
    return Workload("causal", "bf16", d, B, lens, offsets, cache, q_C=q_C, q_R=q_R,
                    W=dict(W_UK=W_UK, W_UV=W_UV), seed=seed, n_q=n_q)


def layer(seed: int = 0, B: int = 128, lo: int = 512, hi: int = 8192, spare: int = 1) -> Workload:
    """Full decode-layer step: prior cache, weights and h_t; ``spare`` free rows per sequence."""
    d = dict(V3_DIMS)
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    offsets, cache = _cache(rng, lens, lens.astype(np.int64) + spare, d["d_c"], d["d_r"], "bf16")
    n_h, d_h, d_r, d_c, d_v = d["n_h"], d["d_h"], d["d_r"], d["d_c"], d["d_v"]
    dm, dq = d["d_model"], d["d_q"]
    W = {}
    W["W_DQ"] = bf16_bits(_normal(rng, (dq, dm), dm ** -0.5))
    W["W_UQ"] = bf16_bits(_normal(rng, (n_h * (d_h + d_r), dq), dq ** -0.5))
    W["W_DKV"] = bf16_bits(_normal(rng, (d_c, dm), dm ** -0.5))
    W["W_KR"] = bf16_bits(_normal(rng, (d_r, dm), dm ** -0.5))
    W["W_UK"] = bf16_bits(_normal(rng, (n_h, d_h, d_c), d_c ** -0.5))
    W["W_UV"] = bf16_bits(_normal(rng, (n_h, d_v, d_c), d_c ** -0.5))
    W["W_O"] = bf16_bits(_normal(rng, (dm, n_h * d_v), (n_h * d_v) ** -0.5))
    h_t = bf16_bits(_normal(rng, (B, dm), 1.0))
    # weights of the optional latent norms, 1 + N(0, 0.1^2) per feature (drawn
    # last, so that every other input is the same with or without them)
    W["q_norm_w"] = bf16_bits(1.0 + _normal(rng, (dq,), 0.1))
    W["kv_norm_w"] = bf16_bits(1.0 + _normal(rng, (d_c,), 0.1))
    return Workload("layer", "bf16", d, B, lens, offsets, cache, W=W, h_t=h_t, seed=seed)


@dataclasses.dataclass
class PagedPool:
    """A block pool holding the rows of several layers' caches.

    ``pool`` is [num_blocks * block_rows, d_c + d_R] (same storage as the
    workload's cache); layer l's block table is ``tables[l]`` [B, max_blocks]
    (int32; unused entries -1).  Row t of sequence b in layer l is pool row
    tables[l][b, t // block_rows] * block_rows + t % block_rows.
    """

    pool: np.ndarray
    tables: np.ndarray           # int32 [layers, B, max_blocks]
    block_rows: int
    num_blocks: int

    @property
    def max_blocks(self) -> int:
        return int(self.tables.shape[2])


def paged_pool(caches, lens, caps, block_rows: int = 64, seed: int = 0, spare_blocks: int = 0) -> PagedPool:
    """Lay the rows of one or more layers' caches out in a shared block pool.

    ``caches[l]`` is layer l's contiguous cache with sequence b in rows
    offsets[b] .. offsets[b] + lens[b] - 1 (offsets = cumulative ``caps``);
    each (layer, sequence) gets ceil(caps[b] / block_rows) blocks, and block
    ids are a seeded random permutation over all layers (so neighbouring rows
    of a sequence are not neighbours in the pool).  Unused rows of the pool
    hold bf16/fp32 NaN so that a wrong row shows.  Layout only: no arithmetic.
    """
    caps = np.asarray(caps, np.int64)
    lens = np.asarray(lens, np.int64)
    L = len(caches)
    B = len(lens)
    nblk = (caps + block_rows - 1) // block_rows
    max_blocks = int(max(1, nblk.max()))
    total = int(nblk.sum()) * L + spare_blocks
    perm = np.random.default_rng(seed + 7919).permutation(total).astype(np.int64)
    D = caches[0].shape[1]
    dt = caches[0].dtype
    pool = np.empty((total * block_rows, D), dtype=dt)
    pool[...] = np.uint16(0x7FC0) if dt == np.uint16 else np.float32("nan")
    tables = np.full((L, B, max_blocks), -1, dtype=np.int32)
    offsets = np.zeros(B + 1, np.int64)
    offsets[1:] = np.cumsum(caps)
    k = 0
    for l in range(L):
        for b in range(B):
            for j in range(int(nblk[b])):
                blk = int(perm[k])
                k += 1
                tables[l, b, j] = blk
                lo = j * block_rows
                n = int(min(block_rows, lens[b] - lo))
                if n > 0:
                    src = int(offsets[b]) + lo
                    pool[blk * block_rows: blk * block_rows + n] = caches[l][src:src + n]
    return PagedPool(pool=pool, tables=tables, block_rows=block_rows, num_blocks=total)


WORKLOADS = {
    "tiny": tiny,
    "uniform": uniform,
    "ragged": ragged,
    "long": long_context,
    "layer": layer,
    "causal": causal,
}


def make(name: str, seed: int = 0, **kw) -> Workload:
    return WORKLOADS[name](seed=seed, **kw)


def ragged_lens(seed: int = 0, B: int = 64, lo: int = 1024, hi: int = 32768) -> np.ndarray:
    """The ragged workload's lengths alone (they are the first draw of its stream)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=B).astype(np.int32)
