"""GPU parity of the full decode-layer step at DeepSeek-V3 dims (bf16 weights):
query path from the hidden state, append of the new token's latent row,
latent attention, up-projection and output projection, against the fp64
oracle's explicit route.  The batch sizes cover one row and more than one
128-row block of the linear layers (a partial second block)."""

import numpy as np
import pytest
import torch

import oracle as O
from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I

from gpu_support import compare, dev, dims_of, host_f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,lo,hi,check", [(1, 40, 40, [0]), (130, 1, 90, [0, 31, 32, 127, 128, 129])])
def test_layer_step_v3(B, lo, hi, check):
    w = I.layer(seed=3, B=B, lo=lo, hi=hi, spare=2)
    say(f"layer: B={B} T_prior in [{lo},{hi}] checked seqs {check}")
    d = dims_of(w)
    dd = w.dims
    n_h, d_c, d_r = dd["n_h"], dd["d_c"], dd["d_r"]
    cache, offsets, lens = dev(w.cache), dev(w.offsets), dev(w.lens)
    W = {k: dev(v) for k, v in w.W.items()}
    h_t = dev(w.h_t)
    pos = lens.clone()
    q_lat = torch.empty(B, n_h, d_c, dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(B, n_h, d_r, dtype=torch.bfloat16, device="cuda")
    L.absorb_q(d, q_lat, q_pe, W["W_UK"], pos, h_t=h_t, W_DQ=W["W_DQ"], W_UQ=W["W_UQ"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.append_cache(d, cache, offsets, lens, 1, h_t=h_t, W_DKV=W["W_DKV"], W_KR=W["W_KR"],
                   err_flag=err)
    o_lat = torch.empty(B, n_h, d_c, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    L.decode_attn(d, q_lat, q_pe, cache, offsets, lens, o_lat, lse,
                  total_rows_hint=int(w.total_rows) + B, err_flag=err)
    o = torch.empty(B, n_h, dd["d_v"], dtype=torch.float32, device="cuda")
    u = torch.empty(B, dd["d_model"], dtype=torch.float32, device="cuda")
    L.project_out(d, o_lat, W["W_UV"], o=o, u=u, W_O=W["W_O"])
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(lens.cpu().numpy(), w.lens + 1)

    Wf = {k: w.f64(v) for k, v in w.W.items()}
    prior_c = {b: w.f64(w.seq_rows(b))[:, :d_c] for b in check}
    prior_k = {b: w.f64(w.seq_rows(b))[:, d_c:] for b in check}
    ref = O.layer_step(w.f64(w.h_t), Wf, prior_c, prior_k, dd, O.scale_for(dd["d_h"], d_r),
                       seqs=check)
    got_cache = host_f64(cache)
    for b in check:
        r = ref[b]
        # the appended row: the projections rounded once to bf16 (k after RoPE)
        row = got_cache[int(w.offsets[b]) + int(w.lens[b])]
        cmax = np.max(np.abs(r["c_new"]))
        assert np.max(np.abs(row[:d_c] - r["c_new"])) <= 2.0 ** -8 * cmax + 1e-6, b
        kmax = np.max(np.abs(r["k_new"]))
        assert np.max(np.abs(row[d_c:] - r["k_new"])) <= 2.0 ** -7 * kmax + 1e-6, b
        # rows other than the new one are untouched
        t0 = int(w.offsets[b])
        assert np.array_equal(got_cache[t0:t0 + int(w.lens[b])], w.f64(w.seq_rows(b))), b
        # query path + absorption: q_lat within one bf16 rounding of W_UK^T q_C
        want = O.absorb_query(r["q_C"], Wf["W_UK"])
        got = host_f64(q_lat[b])
        assert np.max(np.abs(got - want)) <= 2.0 ** -7 * np.max(np.abs(want)), b
        compare(host_f64(o_lat[b]), r["o_lat"], f"o_lat[{b}]")
        compare(host_f64(o[b]), r["o"], f"o[{b}]")
        compare(host_f64(lse[b]), r["lse"], f"lse[{b}]")
        compare(host_f64(u[b]), r["u"], f"u[{b}]")


def test_append_selection_matrix_bit_exact():
    """h_t through the fused W_DKV | W_KR MFMA GEMM with 0/1 selection
    weights: every product is exact and the fp32 sums add zeros, so the
    cached c^KV is exactly the selected features of h_t; at position 0 the
    rotation is the identity, so k^R is exact too.  At later positions k^R is
    within one bf16 rounding of the fp64 rotation of the selected features."""
    B, D, dm = 128, 576, 7168
    rng = np.random.default_rng(77)
    d = L.Dims.make(128, 512, 64, 128, 128, d_model=dm, d_q=1536, dtype="bf16")
    h = I.bf16_bits(rng.standard_normal((B, dm), dtype=np.float32))
    pick = rng.permutation(dm)[:D]
    W = np.zeros((D, dm), np.float32)
    W[np.arange(D), pick] = 1.0
    Wb = I.bf16_bits(W)
    pos = rng.integers(0, 5000, size=B).astype(np.int32)
    pos[:64] = 0
    caps = pos.astype(np.int64) + 1
    offsets = np.concatenate([[0], np.cumsum(caps)]).astype(np.int32)
    cache = torch.zeros(int(offsets[-1]), D, dtype=torch.bfloat16, device="cuda")
    lens = dev(pos.copy())
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.append_cache(d, cache, dev(offsets), lens, 1, h_t=dev(h), W_DKV=dev(Wb[:512]), W_KR=dev(Wb[512:]),
                   err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and np.array_equal(lens.cpu().numpy(), pos + 1)
    got = cache.view(torch.int16).cpu().numpy().view(np.uint16)
    rows = got[offsets[:-1] + pos]
    sel = h[:, pick]
    assert np.array_equal(rows[:, :512], sel[:, :512])                   # c^KV bit-exact
    assert np.array_equal(rows[:64, 512:], sel[:64, 512:])               # k^R at position 0
    kr = O.rope(I.bf16_to_f32(sel[64:, 512:]).astype(np.float64), pos[64:].astype(np.float64))
    gk = I.bf16_to_f32(rows[64:, 512:]).astype(np.float64)
    ulp = np.maximum(np.abs(kr), 1e-30) * 2.0 ** -8
    assert np.all(np.abs(gk - kr) <= ulp + 1e-12), float(np.max(np.abs(gk - kr) / ulp))
