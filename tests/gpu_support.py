"""Helpers shared by the GPU parity tests: upload a workload, run the HIP
path through the C ABI, compute the oracle on the same values, compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray) -> torch.Tensor:
    """Upload a stored array (bf16 bits as uint16, or float32/int32) unchanged."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def dims_of(w: I.Workload) -> L.Dims:
    d = w.dims
    return L.Dims.make(d["n_h"], d["d_c"], d["d_r"], d["d_h"], d["d_v"], d_model=d["d_model"],
                       d_q=d["d_q"], dtype=w.dtype)


def query_concat(w: I.Workload) -> np.ndarray:
    """[q_C | q_R] per head, exactly the stored values."""
    return np.ascontiguousarray(np.concatenate([w.q_C, w.q_R], axis=-1))


class Uploaded:
    """Device copies of a workload's inputs."""

    def __init__(self, w: I.Workload):
        self.w = w
        self.dims = dims_of(w)
        self.cache = dev(w.cache)
        self.offsets = dev(w.offsets)
        self.lens = dev(w.lens)
        self.W = {k: dev(v) for k, v in w.W.items()}
        self.q = dev(query_concat(w)) if w.q_C is not None else None
        self.h_t = dev(w.h_t) if w.h_t is not None else None


def run_attention(u: Uploaded, hint=None, pos=None):
    """absorb_q (q given) -> decode_attn -> project_out (o only)."""
    w, d = u.w, u.dims
    B, n_h = w.B, d.n_h
    dt = d.torch_dtype
    q_lat = torch.empty(B, n_h, d.d_c, dtype=dt, device="cuda")
    q_pe = torch.empty(B, n_h, d.d_r, dtype=dt, device="cuda")
    pos = u.lens.clone() if pos is None else pos
    L.absorb_q(d, q_lat, q_pe, u.W["W_UK"], pos, q=u.q)
    o_lat = torch.empty(B, n_h, d.d_c, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hint = hint if hint is not None else w.total_rows
    ws, check_canary = canaried_workspace(L.decode_attn_workspace(d, B, hint))
    L.decode_attn(d, q_lat, q_pe, u.cache, u.offsets, u.lens, o_lat, lse,
                  total_rows_hint=hint, err_flag=err, ws=ws)
    o = torch.empty(B, n_h, d.d_v, dtype=torch.float32, device="cuda")
    L.project_out(d, o_lat, u.W["W_UV"], o=o)
    torch.cuda.synchronize()
    check_canary()
    return dict(q_lat=q_lat, q_pe=q_pe, o_lat=o_lat, lse=lse, o=o, err=int(err.item()))


CANARY_BYTES = 4096


def canaried_workspace(nbytes: int):
    """A workspace of exactly nbytes (as the library asked for) followed, in
    the same allocation, by canary bytes; the returned check asserts that no
    kernel wrote past the end of the workspace."""
    buf = torch.empty(nbytes + CANARY_BYTES, dtype=torch.uint8, device="cuda")
    buf[nbytes:].fill_(0xA5)

    def check():
        tail = buf[nbytes:].cpu()
        assert bool((tail == 0xA5).all()), "a kernel wrote past the end of its workspace"

    return buf[:nbytes], check


def oracle_seq(w: I.Workload, b: int, heads=None, pos=None):
    """Explicit-route oracle for sequence b (selected heads)."""
    d = w.dims
    heads = list(range(d["n_h"])) if heads is None else list(heads)
    rows = w.f64(w.seq_rows(b))
    c, kr = rows[:, :d["d_c"]], rows[:, d["d_c"]:]
    q_C = w.f64(w.q_C[b])[heads]
    q_R = w.f64(w.q_R[b])[heads]
    W_UK = w.f64(w.W["W_UK"])[heads]
    W_UV = w.f64(w.W["W_UV"])[heads]
    p = int(w.lens[b]) if pos is None else pos
    return O.decode_explicit(q_C, q_R, p, c, kr, W_UK, W_UV, O.scale_for(d["d_h"], d["d_r"]))


def compare(got, ref, what, max_abs=1e-2, mean_abs=1e-3, norm_max=3e-2, norm_mean=3e-3):
    """Tolerance gate: raw max/mean abs error, plus an RMS-normalised guard."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    diff = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    stats = dict(max_abs=float(diff.max()), mean_abs=float(diff.mean()),
                 norm_max=float(diff.max() / rms), norm_mean=float(diff.mean() / rms), rms=rms)
    say(f"  {what}: " + " ".join(f"{k}={v:.3g}" for k, v in stats.items()))
    assert stats["max_abs"] <= max_abs, (what, stats)
    assert stats["mean_abs"] <= mean_abs, (what, stats)
    assert stats["norm_max"] <= norm_max, (what, stats)
    assert stats["norm_mean"] <= norm_mean, (what, stats)
    return stats
