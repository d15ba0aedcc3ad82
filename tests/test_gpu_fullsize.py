"""GPU parity at the full benchmark sizes, in the launch configuration the
benchmark times (same seeded workloads, total-rows hint, split kernel and
combine), on sampled (sequence, head) outputs that the fp64 oracle computes
one by one: uniform B=16 T=4096, ragged B=64 T in [1024, 32768], long context
B=8 T=131072, the full layer step at B=128, and the several-new-tokens step
(B=16, T=4096, n_q=4)."""

import numpy as np
import pytest
import torch

import oracle as O
from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I

from gpu_support import Uploaded, compare, dev, dims_of, host_f64, oracle_seq, run_attention, say

pytestmark = pytest.mark.gpu


def _samples(name, w):
    lens = w.lens
    if name == "uniform":
        return {0: [0, 40, 77], 7: [31, 63], 15: [64, 127]}
    if name == "ragged":
        return {0: [5, 33], int(np.argmax(lens)): [100, 50], int(np.argmin(lens)): [0, 127], w.B - 1: [64]}
    return {0: [3, 45], w.B - 1: [64, 127]}


@pytest.mark.parametrize("name", ["uniform", "ragged", "long"])
def test_full_size_attention(name):
    w = I.make(name)
    say(f"full size {name}: B={w.B} rows={w.total_rows}")
    u = Uploaded(w)
    r = run_attention(u)
    assert r["err"] == 0
    o, o_lat, lse = host_f64(r["o"]), host_f64(r["o_lat"]), host_f64(r["lse"])
    assert np.all(np.isfinite(o_lat)) and np.all(np.isfinite(lse))
    for b, heads in _samples(name, w).items():
        ro, ro_lat, rlse = oracle_seq(w, b, heads=heads)
        tag = f"{name} b={b} T={int(w.lens[b])} heads={heads}"
        compare(o_lat[b][heads], ro_lat, f"{tag} o_lat")
        compare(o[b][heads], ro, f"{tag} o")
        compare(lse[b][heads], rlse, f"{tag} lse", max_abs=2e-2, mean_abs=2e-3, norm_max=1e-2, norm_mean=2e-3)
    # every head (all four 32-head groups of the split kernel) of two
    # sequences: the latent definition evaluated by the oracle on the
    # kernel's own q_lat / q_pe (that definition is pinned to the explicit
    # route on the CPU)
    ql, qp = host_f64(r["q_lat"]), host_f64(r["q_pe"])
    two = [int(np.argmin(w.lens)), int(np.argmax(w.lens))] if name == "ragged" else [0, w.B - 1]
    for b in two:
        rows = w.f64(w.seq_rows(b))
        ref, rl = O.latent_attention(ql[b], qp[b], rows[:, :512], rows[:, 512:], O.scale_for(128, 64))
        compare(o_lat[b], ref, f"{name} b={b} all heads o_lat")
        compare(lse[b], rl, f"{name} b={b} all heads lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2,
                norm_mean=1e-3)


@pytest.mark.parametrize("norms", [False, True])
def test_full_size_layer_step(norms):
    """B=128, prior T in [512, 8192]: query path from h_t, append, attention,
    up-projection and output projection (with norms: the latent norms on c^Q
    and c^KV, as bench.py --workload layer --norms); sequences 0, 64 and 127
    checked."""
    w = I.layer()
    check = [0, 64, 127]
    d = dims_of(w)
    dd = w.dims
    B = w.B
    say(f"full size layer: B={B} prior rows={w.total_rows} norms={norms}")
    cache, offsets, lens = dev(w.cache), dev(w.offsets), dev(w.lens)
    W = {k: dev(v) for k, v in w.W.items()}
    h_t = dev(w.h_t)
    pos = lens.clone()
    q_lat = torch.empty(B, dd["n_h"], dd["d_c"], dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(B, dd["n_h"], dd["d_r"], dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if norms:
        L.absorb_q_normed(d, q_lat, q_pe, W["W_UK"], pos, h_t, W["W_DQ"], W["q_norm_w"], W["W_UQ"])
        L.append_cache_normed(d, cache, offsets, lens, 1, h_t, W["W_DKV"], W["kv_norm_w"], W["W_KR"],
                              err_flag=err)
    else:
        L.absorb_q(d, q_lat, q_pe, W["W_UK"], pos, h_t=h_t, W_DQ=W["W_DQ"], W_UQ=W["W_UQ"])
        L.append_cache(d, cache, offsets, lens, 1, h_t=h_t, W_DKV=W["W_DKV"], W_KR=W["W_KR"], err_flag=err)
    o_lat = torch.empty(B, dd["n_h"], dd["d_c"], dtype=torch.float32, device="cuda")
    lse = torch.empty(B, dd["n_h"], dtype=torch.float32, device="cuda")
    L.decode_attn(d, q_lat, q_pe, cache, offsets, lens, o_lat, lse,
                  total_rows_hint=int(w.total_rows) + B, err_flag=err)
    o = torch.empty(B, dd["n_h"], dd["d_v"], dtype=torch.float32, device="cuda")
    u = torch.empty(B, dd["d_model"], dtype=torch.float32, device="cuda")
    L.project_out(d, o_lat, W["W_UV"], o=o, u=u, W_O=W["W_O"])
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    Wf = {k: w.f64(v) for k, v in w.W.items()}
    prior_c = {b: w.f64(w.seq_rows(b))[:, :dd["d_c"]] for b in check}
    prior_k = {b: w.f64(w.seq_rows(b))[:, dd["d_c"]:] for b in check}
    ref = O.layer_step(w.f64(w.h_t), Wf, prior_c, prior_k, dd, O.scale_for(dd["d_h"], dd["d_r"]), seqs=check,
                       norms=norms)
    for b in check:
        rb = ref[b]
        compare(host_f64(o_lat[b]), rb["o_lat"], f"layer b={b} o_lat")
        compare(host_f64(o[b]), rb["o"], f"layer b={b} o")
        compare(host_f64(lse[b]), rb["lse"], f"layer b={b} lse", max_abs=2e-2, mean_abs=2e-3,
                norm_max=1e-2, norm_mean=2e-3)
        compare(host_f64(u[b]), rb["u"], f"layer b={b} u")


def test_full_size_causal_step():
    """Several new tokens, as bench.py --workload causal times them: B=16,
    T=4096, n_q=4; absorb (token i of sequence b at position T - 4 + i),
    mla_decode_attn_causal, up-projection.  Sampled (sequence, token, heads)
    against the oracle's explicit route over each token's prefix."""
    w = I.causal()
    n_q, B, T = w.n_q, w.B, int(w.lens[0])
    d = dims_of(w)
    say(f"full size causal: B={B} T={T} n_q={n_q}")
    u = Uploaded(w)
    BQ = B * n_q
    q_lat = torch.empty(BQ, 128, 512, dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(BQ, 128, 64, dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty(BQ, 128, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(BQ, 128, dtype=torch.float32, device="cuda")
    o = torch.empty(BQ, 128, 128, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.tensor([T - n_q + i for _ in range(B) for i in range(n_q)], dtype=torch.int32, device="cuda")
    L.absorb_q(d, q_lat, q_pe, u.W["W_UK"], pos, q=u.q)
    L.decode_attn_causal(d, n_q, q_lat, q_pe, u.cache, u.offsets, u.lens, o_lat, lse,
                         total_rows_hint=w.total_rows, err_flag=err)
    L.project_out(d, o_lat, u.W["W_UV"], o=o)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o, o_lat, lse = host_f64(o), host_f64(o_lat), host_f64(lse)
    assert np.all(np.isfinite(o_lat)) and np.all(np.isfinite(lse))
    W_UK, W_UV = w.f64(w.W["W_UK"]), w.f64(w.W["W_UV"])
    scale = O.scale_for(128, 64)
    for b, i, heads in ((0, 0, [0, 77]), (0, 3, [5]), (9, 1, [31, 100]), (15, 2, [127])):
        n = T - n_q + i + 1
        rows = w.f64(w.seq_rows(b))[:n]
        t = b * n_q + i
        ro, ro_lat, rlse = O.decode_explicit(w.f64(w.q_C[t])[heads], w.f64(w.q_R[t])[heads], T - n_q + i,
                                             rows[:, :512], rows[:, 512:], W_UK[heads], W_UV[heads], scale)
        tag = f"causal b={b} token={i} rows={n} heads={heads}"
        compare(o_lat[t][heads], ro_lat, f"{tag} o_lat")
        compare(o[t][heads], ro, f"{tag} o")
        compare(lse[t][heads], rlse, f"{tag} lse", max_abs=2e-2, mean_abs=2e-3, norm_max=1e-2, norm_mean=2e-3)
