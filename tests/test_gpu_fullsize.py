"""GPU parity at the full benchmark sizes, in the launch configuration the
benchmark times (same seeded workloads, total-rows hint, split kernel and
combine), on sampled (sequence, head) outputs that the fp64 oracle computes
one by one: uniform B=16 T=4096, ragged B=64 T in [1024, 32768], long context
B=8 T=131072, and the full layer step at B=128."""

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
        return {0: [0, 77], 7: [31], 15: [64, 127]}
    if name == "ragged":
        return {0: [5], int(np.argmax(lens)): [100], int(np.argmin(lens)): [0, 127], w.B - 1: [64]}
    return {0: [3], w.B - 1: [64, 127]}


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


def test_full_size_layer_step():
    """B=128, prior T in [512, 8192]: query path from h_t, append, attention,
    up-projection and output projection; sequences 0, 64 and 127 checked."""
    w = I.layer()
    check = [0, 64, 127]
    d = dims_of(w)
    dd = w.dims
    B = w.B
    say(f"full size layer: B={B} prior rows={w.total_rows}")
    cache, offsets, lens = dev(w.cache), dev(w.offsets), dev(w.lens)
    W = {k: dev(v) for k, v in w.W.items()}
    h_t = dev(w.h_t)
    pos = lens.clone()
    q_lat = torch.empty(B, dd["n_h"], dd["d_c"], dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(B, dd["n_h"], dd["d_r"], dtype=torch.bfloat16, device="cuda")
    L.absorb_q(d, q_lat, q_pe, W["W_UK"], pos, h_t=h_t, W_DQ=W["W_DQ"], W_UQ=W["W_UQ"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
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
    ref = O.layer_step(w.f64(w.h_t), Wf, prior_c, prior_k, dd, O.scale_for(dd["d_h"], dd["d_r"]), seqs=check)
    for b in check:
        rb = ref[b]
        compare(host_f64(o_lat[b]), rb["o_lat"], f"layer b={b} o_lat")
        compare(host_f64(o[b]), rb["o"], f"layer b={b} o")
        compare(host_f64(lse[b]), rb["lse"], f"layer b={b} lse", max_abs=2e-2, mean_abs=2e-3,
                norm_max=1e-2, norm_mean=2e-3)
        compare(host_f64(u[b]), rb["u"], f"layer b={b} u")
