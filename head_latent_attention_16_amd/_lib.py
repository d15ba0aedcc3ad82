"""ctypes binding of libmla.so (C ABI in include/mla.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, scratch is allocated with torch when the
caller does not pass one.  Every step of the computation runs in the HIP
kernels of the library; if the library is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB_PATH selects another build of the same library (the host-sanitized
# one used by the CPU ABI checks); by default the in-tree libmla.so.
LIB_PATH = os.environ.get("MLA_LIB_PATH") or os.path.join(_HERE, "libmla.so")

MLA_OK = 0
STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE",
          4: "MLA_ERR_WORKSPACE", 5: "MLA_ERR_LAUNCH", 6: "MLA_ERR_DEVICE"}
DEVERR_LENS = 1
DEVERR_OVERFLOW = 2
DEVERR_TABLE = 4
DT_BF16, DT_F32 = 0, 1

EXPORTS = ("mla_absorb_q", "mla_absorb_q_workspace", "mla_append_cache",
           "mla_append_cache_workspace", "mla_decode_attn", "mla_decode_attn_workspace",
           "mla_decode_attn_causal", "mla_decode_attn_causal_workspace",
           "mla_absorb_q_normed", "mla_append_cache_normed",
           "mla_project_out", "mla_project_out_workspace", "mla_cache_row_bytes",
           "mla_status_string", "mla_abi_version", "mla_decode_attn_noalloc",
           "mla_decode_attn_paged", "mla_append_cache_paged", "mla_append_cache_fp8",
           "mla_decode_attn_fp8", "mla_prefill_attn", "mla_prefill_attn_workspace")


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


class Dims(ctypes.Structure):
    _fields_ = [("n_h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("d_v", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_q", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32)]

    @classmethod
    def make(cls, n_h, d_c, d_r, d_h, d_v, d_model=0, d_q=0, rope_base=10000.0,
             softmax_scale=0.0, dtype="bf16"):
        dt = {"bf16": DT_BF16, "f32": DT_F32}[dtype] if isinstance(dtype, str) else int(dtype)
        return cls(n_h, d_c, d_r, d_h, d_v, d_model, d_q, rope_base, softmax_scale, dt)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == DT_BF16 else torch.float32


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with `python -m head_latent_attention_16_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(Dims)
    sig = {
        "mla_absorb_q": ([D, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "mla_absorb_q_workspace": ([D, i32, i32], sz),
        "mla_absorb_q_normed": ([D, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "mla_append_cache_normed": ([D, i32, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, sz,
                                     vp], i32),
        "mla_append_cache": ([D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "mla_append_cache_workspace": ([D, i32, i32, i32], sz),
        "mla_decode_attn": ([D, i32, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp], i32),
        "mla_decode_attn_workspace": ([D, i32, i64], sz),
        "mla_decode_attn_noalloc": ([D, i32, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp], i32),
        "mla_decode_attn_paged": ([D, i32, vp, vp, vp, i32, i32, vp, i32, vp, i64, vp, vp, vp, vp, sz, vp],
                                  i32),
        "mla_append_cache_paged": ([D, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, sz, vp],
                                   i32),
        "mla_append_cache_fp8": ([D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "mla_decode_attn_fp8": ([D, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp], i32),
        "mla_prefill_attn": ([D, i32, i32, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "mla_prefill_attn_workspace": ([D, i32, i32, i64], sz),
        "mla_decode_attn_causal": ([D, i32, i32, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp], i32),
        "mla_decode_attn_causal_workspace": ([D, i32, i32, i64], sz),
        "mla_project_out": ([D, i32, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "mla_project_out_workspace": ([D, i32, i32], sz),
        "mla_cache_row_bytes": ([D], sz),
        "mla_status_string": ([i32], ctypes.c_char_p),
        "mla_abi_version": ([], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


# ---------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(name, st):
    if st != MLA_OK:
        raise MLAError(name, st)


def _need(t, numel, dtype, what):
    if t is None:
        return
    if t.numel() != numel:
        raise ValueError(f"{what}: expected {numel} elements, got {t.numel()}")
    if t.dtype != dtype:
        raise ValueError(f"{what}: expected {dtype}, got {t.dtype}")


def _workspace(nbytes: int, ws: Optional[torch.Tensor], device):
    if nbytes == 0:
        return ws
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel() * ws.element_size()} < {nbytes}")
    return ws


def _ws_args(ws):
    if ws is None:
        return None, 0
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def cache_row_bytes(dims: Dims) -> int:
    return int(lib().mla_cache_row_bytes(ctypes.byref(dims)))


def decode_attn_workspace(dims: Dims, B: int, total_rows_hint: int) -> int:
    return int(lib().mla_decode_attn_workspace(ctypes.byref(dims), B, int(total_rows_hint)))


def decode_attn_causal_workspace(dims: Dims, B: int, n_q: int, total_rows_hint: int) -> int:
    return int(lib().mla_decode_attn_causal_workspace(ctypes.byref(dims), B, n_q, int(total_rows_hint)))


def absorb_q(dims: Dims, q_lat, q_pe, W_UK, pos, q=None, h_t=None, W_DQ=None, W_UQ=None,
             ws=None, stream=None):
    """q_lat[b,h] = W_UK[h]^T q^C[b,h], q_pe[b,h] = RoPE(q^R[b,h], pos[b]).

    q [B, n_h, d_h + d_r] given, or computed from h_t [B, d_model] as
    W_UQ (W_DQ h_t) (W_DQ None when dims.d_q == 0)."""
    L = lib()
    B = q_lat.shape[0]
    dt = dims.torch_dtype
    _dev(q_lat, q_pe, W_UK, pos, q, h_t, W_DQ, W_UQ)
    _need(q_lat, B * dims.n_h * dims.d_c, dt, "q_lat")
    _need(q_pe, B * dims.n_h * dims.d_r, dt, "q_pe")
    _need(W_UK, dims.n_h * dims.d_h * dims.d_c, dt, "W_UK")
    _need(pos, B, torch.int32, "pos")
    _need(q, B * dims.n_h * (dims.d_h + dims.d_r), dt, "q")
    _need(h_t, B * dims.d_model, dt, "h_t")
    nbytes = int(L.mla_absorb_q_workspace(ctypes.byref(dims), B, int(h_t is not None)))
    ws = _workspace(nbytes, ws, q_lat.device)
    w, wn = _ws_args(ws)
    st = L.mla_absorb_q(ctypes.byref(dims), B, _ptr(h_t), _ptr(W_DQ), _ptr(W_UQ), _ptr(q),
                        _ptr(W_UK), _ptr(pos), _ptr(q_lat), _ptr(q_pe), w, wn, _stream(stream))
    _check("mla_absorb_q", st)


def append_cache(dims: Dims, cache, offsets, lens, n_new: int, kv_raw=None, h_t=None,
                 W_DKV=None, W_KR=None, err_flag=None, ws=None, stream=None):
    """Append n_new rows per sequence at offsets[b] + lens[b]; lens[b] += n_new."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(cache, offsets, lens, kv_raw, h_t, W_DKV, W_KR, err_flag)
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(lens, B, torch.int32, "lens")
    _need(kv_raw, B * n_new * (dims.d_c + dims.d_r), dt, "kv_raw")
    _need(h_t, B * n_new * dims.d_model, dt, "h_t")
    if cache.dtype != dt:
        raise ValueError("cache dtype")
    nbytes = int(L.mla_append_cache_workspace(ctypes.byref(dims), B, n_new, int(h_t is not None)))
    ws = _workspace(nbytes, ws, cache.device)
    w, wn = _ws_args(ws)
    st = L.mla_append_cache(ctypes.byref(dims), B, n_new, _ptr(h_t), _ptr(W_DKV), _ptr(W_KR),
                            _ptr(kv_raw), _ptr(cache), _ptr(offsets), _ptr(lens), _ptr(err_flag),
                            w, wn, _stream(stream))
    _check("mla_append_cache", st)


def decode_attn(dims: Dims, q_lat, q_pe, cache, offsets, lens, o_lat, lse=None,
                total_rows_hint: Optional[int] = None, err_flag=None, ws=None, stream=None):
    """o_lat[b,h] = sum_j softmax_j(scale (q_lat.c_j + q_pe.kR_j)) c_j over the b-th region."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(q_lat, q_pe, cache, offsets, lens, o_lat, lse, err_flag)
    _need(q_lat, B * dims.n_h * dims.d_c, dt, "q_lat")
    _need(q_pe, B * dims.n_h * dims.d_r, dt, "q_pe")
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(o_lat, B * dims.n_h * dims.d_c, torch.float32, "o_lat")
    _need(lse, B * dims.n_h, torch.float32, "lse")
    if cache.dtype != dt:
        raise ValueError("cache dtype")
    hint = int(total_rows_hint) if total_rows_hint is not None else max(1, cache.shape[0])
    nbytes = decode_attn_workspace(dims, B, hint)
    ws = _workspace(nbytes, ws, cache.device)
    w, wn = _ws_args(ws)
    st = L.mla_decode_attn(ctypes.byref(dims), B, _ptr(q_lat), _ptr(q_pe), _ptr(cache),
                           _ptr(offsets), _ptr(lens), hint, _ptr(o_lat), _ptr(lse),
                           _ptr(err_flag), w, wn, _stream(stream))
    _check("mla_decode_attn", st)


def decode_attn_noalloc(dims: Dims, q_lat, q_pe, cache, offsets, lens, o_lat, lse=None,
                        total_rows_hint: Optional[int] = None, err_flag=None, stream=None):
    """decode_attn with the library's fixed scratch instead of a workspace
    (the call allocates nothing)."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(q_lat, q_pe, cache, offsets, lens, o_lat, lse, err_flag)
    _need(q_lat, B * dims.n_h * dims.d_c, dt, "q_lat")
    _need(q_pe, B * dims.n_h * dims.d_r, dt, "q_pe")
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(o_lat, B * dims.n_h * dims.d_c, torch.float32, "o_lat")
    _need(lse, B * dims.n_h, torch.float32, "lse")
    if cache.dtype != dt:
        raise ValueError("cache dtype")
    hint = int(total_rows_hint) if total_rows_hint is not None else max(1, cache.shape[0])
    st = L.mla_decode_attn_noalloc(ctypes.byref(dims), B, _ptr(q_lat), _ptr(q_pe), _ptr(cache),
                                   _ptr(offsets), _ptr(lens), hint, _ptr(o_lat), _ptr(lse),
                                   _ptr(err_flag), _stream(stream))
    _check("mla_decode_attn_noalloc", st)


def decode_attn_paged(dims: Dims, q_lat, q_pe, pool, block_rows: int, block_table, lens, o_lat, lse=None,
                      total_rows_hint: Optional[int] = None, err_flag=None, ws=None, stream=None):
    """decode_attn over a block pool: row t of sequence b is row
    t % block_rows of block block_table[b, t // block_rows]."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(q_lat, q_pe, pool, block_table, lens, o_lat, lse, err_flag)
    _need(q_lat, B * dims.n_h * dims.d_c, dt, "q_lat")
    _need(q_pe, B * dims.n_h * dims.d_r, dt, "q_pe")
    _need(o_lat, B * dims.n_h * dims.d_c, torch.float32, "o_lat")
    _need(lse, B * dims.n_h, torch.float32, "lse")
    if pool.dtype != dt or block_table.dtype != torch.int32 or block_table.dim() != 2 \
            or block_table.shape[0] != B:
        raise ValueError("pool dtype or block table shape")
    nrows = pool.numel() // (dims.d_c + dims.d_r)
    hint = int(total_rows_hint) if total_rows_hint is not None else max(1, nrows)
    ws = _workspace(decode_attn_workspace(dims, B, hint), ws, pool.device)
    w, wn = _ws_args(ws)
    st = L.mla_decode_attn_paged(ctypes.byref(dims), B, _ptr(q_lat), _ptr(q_pe), _ptr(pool),
                                 nrows // block_rows, block_rows, _ptr(block_table), block_table.shape[1],
                                 _ptr(lens), hint, _ptr(o_lat), _ptr(lse), _ptr(err_flag), w, wn,
                                 _stream(stream))
    _check("mla_decode_attn_paged", st)


def append_cache_paged(dims: Dims, pool, block_rows: int, block_table, lens, n_new: int, kv_raw=None,
                       h_t=None, W_DKV=None, W_KR=None, err_flag=None, ws=None, stream=None):
    """append_cache into a block pool (row lens[b] + i of sequence b)."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(pool, block_table, lens, kv_raw, h_t, W_DKV, W_KR, err_flag)
    _need(lens, B, torch.int32, "lens")
    _need(kv_raw, B * n_new * (dims.d_c + dims.d_r), dt, "kv_raw")
    _need(h_t, B * n_new * dims.d_model, dt, "h_t")
    if pool.dtype != dt or block_table.dtype != torch.int32 or block_table.dim() != 2 \
            or block_table.shape[0] != B:
        raise ValueError("pool dtype or block table shape")
    nrows = pool.numel() // (dims.d_c + dims.d_r)
    nbytes = int(L.mla_append_cache_workspace(ctypes.byref(dims), B, n_new, int(h_t is not None)))
    ws = _workspace(nbytes, ws, pool.device)
    w, wn = _ws_args(ws)
    st = L.mla_append_cache_paged(ctypes.byref(dims), B, n_new, _ptr(h_t), _ptr(W_DKV), _ptr(W_KR),
                                  _ptr(kv_raw), _ptr(pool), nrows // block_rows, block_rows,
                                  _ptr(block_table), block_table.shape[1], _ptr(lens), _ptr(err_flag), w, wn,
                                  _stream(stream))
    _check("mla_append_cache_paged", st)


def append_cache_fp8(dims: Dims, cache8, scales, offsets, lens, n_new: int, kv_raw=None, h_t=None,
                     W_DKV=None, W_KR=None, err_flag=None, ws=None, stream=None):
    """append_cache into an 8-bit cache: E4M3 codes cache8 [rows, d_c + d_r]
    (uint8) and one fp32 scale per row in scales [rows]."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(cache8, scales, offsets, lens, kv_raw, h_t, W_DKV, W_KR, err_flag)
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(lens, B, torch.int32, "lens")
    _need(kv_raw, B * n_new * (dims.d_c + dims.d_r), dt, "kv_raw")
    _need(h_t, B * n_new * dims.d_model, dt, "h_t")
    rows = cache8.numel() // (dims.d_c + dims.d_r)
    _need(scales, rows, torch.float32, "scales")
    if cache8.dtype != torch.uint8:
        raise ValueError("cache8 must be uint8")
    nbytes = int(L.mla_append_cache_workspace(ctypes.byref(dims), B, n_new, int(h_t is not None)))
    ws = _workspace(nbytes, ws, cache8.device)
    w, wn = _ws_args(ws)
    st = L.mla_append_cache_fp8(ctypes.byref(dims), B, n_new, _ptr(h_t), _ptr(W_DKV), _ptr(W_KR), _ptr(kv_raw),
                                _ptr(cache8), _ptr(scales), _ptr(offsets), _ptr(lens), _ptr(err_flag), w, wn,
                                _stream(stream))
    _check("mla_append_cache_fp8", st)


def decode_attn_fp8(dims: Dims, q_lat, q_pe, cache8, scales, offsets, lens, o_lat, lse=None,
                    total_rows_hint: Optional[int] = None, err_flag=None, ws=None, stream=None):
    """decode_attn over an 8-bit cache (codes x row scale)."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(q_lat, q_pe, cache8, scales, offsets, lens, o_lat, lse, err_flag)
    _need(q_lat, B * dims.n_h * dims.d_c, dt, "q_lat")
    _need(q_pe, B * dims.n_h * dims.d_r, dt, "q_pe")
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(o_lat, B * dims.n_h * dims.d_c, torch.float32, "o_lat")
    _need(lse, B * dims.n_h, torch.float32, "lse")
    rows = cache8.numel() // (dims.d_c + dims.d_r)
    _need(scales, rows, torch.float32, "scales")
    if cache8.dtype != torch.uint8:
        raise ValueError("cache8 must be uint8")
    hint = int(total_rows_hint) if total_rows_hint is not None else max(1, rows)
    ws = _workspace(decode_attn_workspace(dims, B, hint), ws, cache8.device)
    w, wn = _ws_args(ws)
    st = L.mla_decode_attn_fp8(ctypes.byref(dims), B, _ptr(q_lat), _ptr(q_pe), _ptr(cache8), _ptr(scales),
                               _ptr(offsets), _ptr(lens), hint, _ptr(o_lat), _ptr(lse), _ptr(err_flag), w, wn,
                               _stream(stream))
    _check("mla_decode_attn_fp8", st)


def prefill_attn_workspace(dims: Dims, B: int, n_q: int, cache_rows: int) -> int:
    return int(lib().mla_prefill_attn_workspace(ctypes.byref(dims), B, n_q, int(cache_rows)))


def prefill_attn(dims: Dims, q, cache, offsets, lens, W_UK, W_UV, o, lse=None, err_flag=None, ws=None,
                 stream=None):
    """Un-absorbed causal attention of the last n_q cached tokens of each
    sequence; q [B, n_q, n_h, d_h + d_r] (q^R not rotated), o [B, n_q, n_h, d_v]."""
    L = lib()
    B, n_q = q.shape[0], q.shape[1]
    dt = dims.torch_dtype
    _dev(q, cache, offsets, lens, W_UK, W_UV, o, lse, err_flag)
    _need(q, B * n_q * dims.n_h * (dims.d_h + dims.d_r), dt, "q")
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(lens, B, torch.int32, "lens")
    _need(W_UK, dims.n_h * dims.d_h * dims.d_c, dt, "W_UK")
    _need(W_UV, dims.n_h * dims.d_v * dims.d_c, dt, "W_UV")
    _need(o, B * n_q * dims.n_h * dims.d_v, torch.float32, "o")
    _need(lse, B * n_q * dims.n_h, torch.float32, "lse")
    if cache.dtype != dt:
        raise ValueError("cache dtype")
    rows = cache.numel() // (dims.d_c + dims.d_r)
    ws = _workspace(prefill_attn_workspace(dims, B, n_q, rows), ws, cache.device)
    w, wn = _ws_args(ws)
    st = L.mla_prefill_attn(ctypes.byref(dims), B, n_q, _ptr(q), _ptr(cache), rows, _ptr(offsets), _ptr(lens),
                            _ptr(W_UK), _ptr(W_UV), _ptr(o), _ptr(lse), _ptr(err_flag), w, wn, _stream(stream))
    _check("mla_prefill_attn", st)


def project_out(dims: Dims, o_lat, W_UV, o=None, u=None, W_O=None, ws=None, stream=None):
    """o[b,h] = W_UV[h] o_lat[b,h]; u[b] = W_O flatten(o[b])."""
    L = lib()
    B = o_lat.shape[0]
    dt = dims.torch_dtype
    _dev(o_lat, W_UV, o, u, W_O)
    _need(o_lat, B * dims.n_h * dims.d_c, torch.float32, "o_lat")
    _need(W_UV, dims.n_h * dims.d_v * dims.d_c, dt, "W_UV")
    _need(o, B * dims.n_h * dims.d_v, torch.float32, "o")
    _need(u, B * dims.d_model, torch.float32, "u")
    nbytes = int(L.mla_project_out_workspace(ctypes.byref(dims), B, int(u is not None)))
    ws = _workspace(nbytes, ws, o_lat.device)
    w, wn = _ws_args(ws)
    st = L.mla_project_out(ctypes.byref(dims), B, _ptr(o_lat), _ptr(W_UV), _ptr(W_O), _ptr(o),
                           _ptr(u), w, wn, _stream(stream))
    _check("mla_project_out", st)


def decode_attn_causal(dims: Dims, n_q: int, q_lat, q_pe, cache, offsets, lens, o_lat, lse=None,
                       total_rows_hint: Optional[int] = None, err_flag=None, ws=None, stream=None):
    """n_q new tokens per sequence (the last n_q cached rows): token i of
    sequence b attends to rows 0 .. lens[b] - n_q + i.  q_lat, q_pe, o_lat,
    lse are [B, n_q, n_h, ...]."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(q_lat, q_pe, cache, offsets, lens, o_lat, lse, err_flag)
    _need(q_lat, B * n_q * dims.n_h * dims.d_c, dt, "q_lat")
    _need(q_pe, B * n_q * dims.n_h * dims.d_r, dt, "q_pe")
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(o_lat, B * n_q * dims.n_h * dims.d_c, torch.float32, "o_lat")
    _need(lse, B * n_q * dims.n_h, torch.float32, "lse")
    if cache.dtype != dt:
        raise ValueError("cache dtype")
    hint = int(total_rows_hint) if total_rows_hint is not None else max(1, cache.shape[0])
    nbytes = decode_attn_causal_workspace(dims, B, n_q, hint)
    ws = _workspace(nbytes, ws, cache.device)
    w, wn = _ws_args(ws)
    st = L.mla_decode_attn_causal(ctypes.byref(dims), B, n_q, _ptr(q_lat), _ptr(q_pe), _ptr(cache),
                                  _ptr(offsets), _ptr(lens), hint, _ptr(o_lat), _ptr(lse),
                                  _ptr(err_flag), w, wn, _stream(stream))
    _check("mla_decode_attn_causal", st)


def absorb_q_normed(dims: Dims, q_lat, q_pe, W_UK, pos, h_t, W_DQ, q_norm_w, W_UQ, eps=1e-6,
                    ws=None, stream=None):
    """absorb_q from h_t with c^Q normalised (root-mean-square, weight q_norm_w)
    between W_DQ and W_UQ."""
    L = lib()
    B = q_lat.shape[0]
    dt = dims.torch_dtype
    _dev(q_lat, q_pe, W_UK, pos, h_t, W_DQ, q_norm_w, W_UQ)
    _need(q_lat, B * dims.n_h * dims.d_c, dt, "q_lat")
    _need(q_pe, B * dims.n_h * dims.d_r, dt, "q_pe")
    _need(pos, B, torch.int32, "pos")
    _need(h_t, B * dims.d_model, dt, "h_t")
    _need(q_norm_w, dims.d_q, dt, "q_norm_w")
    ws = _workspace(int(L.mla_absorb_q_workspace(ctypes.byref(dims), B, 1)), ws, q_lat.device)
    w, wn = _ws_args(ws)
    st = L.mla_absorb_q_normed(ctypes.byref(dims), B, _ptr(h_t), _ptr(W_DQ), _ptr(q_norm_w), float(eps),
                               _ptr(W_UQ), _ptr(W_UK), _ptr(pos), _ptr(q_lat), _ptr(q_pe), w, wn,
                               _stream(stream))
    _check("mla_absorb_q_normed", st)


def append_cache_normed(dims: Dims, cache, offsets, lens, n_new: int, h_t, W_DKV, kv_norm_w, W_KR,
                        eps=1e-6, err_flag=None, ws=None, stream=None):
    """append_cache from h_t with c^KV normalised (root-mean-square, weight
    kv_norm_w) before it is written."""
    L = lib()
    B = lens.shape[0]
    dt = dims.torch_dtype
    _dev(cache, offsets, lens, h_t, W_DKV, kv_norm_w, W_KR, err_flag)
    _need(offsets, B + 1, torch.int32, "offsets")
    _need(h_t, B * n_new * dims.d_model, dt, "h_t")
    _need(kv_norm_w, dims.d_c, dt, "kv_norm_w")
    ws = _workspace(int(L.mla_append_cache_workspace(ctypes.byref(dims), B, n_new, 1)), ws, cache.device)
    w, wn = _ws_args(ws)
    st = L.mla_append_cache_normed(ctypes.byref(dims), B, n_new, _ptr(h_t), _ptr(W_DKV), _ptr(kv_norm_w),
                                   float(eps), _ptr(W_KR), _ptr(cache), _ptr(offsets), _ptr(lens),
                                   _ptr(err_flag), w, wn, _stream(stream))
    _check("mla_append_cache_normed", st)
