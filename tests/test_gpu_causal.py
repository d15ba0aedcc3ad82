"""GPU parity of mla_decode_attn_causal: n_q new tokens per sequence, the last
n_q cached rows, token i attending to rows 0 .. lens[b] - n_q + i (the causal
mask of the worked example's inference code), against the oracle's
latent_attention_causal."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I

from gpu_support import Uploaded, compare, dev, host_f64, say

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(192)


def _case(lens, n_q, seed):
    rng = np.random.default_rng(seed)
    w = I.attention_only("causal", len(lens), np.asarray(lens, np.int32), rng, seed)
    q_lat = I.bf16_bits(rng.standard_normal((w.B, n_q, 128, 512)).astype(np.float32) * 0.05)
    q_pe = I.bf16_bits(rng.standard_normal((w.B, n_q, 128, 64)).astype(np.float32))
    return w, q_lat, q_pe


def _run(w, n_q, q_lat, q_pe, lens=None):
    u = Uploaded(w)
    B = w.B
    o_lat = torch.empty(B, n_q, 128, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, n_q, 128, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens_t = u.lens if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    L.decode_attn_causal(u.dims, n_q, dev(q_lat), dev(q_pe), u.cache, u.offsets, lens_t, o_lat, lse,
                         total_rows_hint=w.total_rows, err_flag=err)
    torch.cuda.synchronize()
    return host_f64(o_lat), host_f64(lse), int(err.item())


def _check_seq(w, got, glse, q_lat, q_pe, b, n_q):
    rows = w.f64(w.seq_rows(b))
    ref, lse = O.latent_attention_causal(w.f64(q_lat[b]), w.f64(q_pe[b]), rows[:, :512], rows[:, 512:],
                                         SCALE)
    compare(got[b], ref, f"b={b} T={rows.shape[0]} n_q={n_q} o_lat")
    compare(glse[b], lse, f"b={b} lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2, norm_mean=1e-3)


@pytest.mark.parametrize("n_q", [1, 2, 5])
def test_causal_matches_oracle(n_q):
    """Lengths from exactly n_q (the first token sees one row) over tile and
    piece boundaries to a few thousand rows."""
    lens = [n_q, n_q + 1, 33, 64 + n_q, 300, 2500]
    w, q_lat, q_pe = _case(lens, n_q, seed=40 + n_q)
    say(f"causal n_q={n_q} lens={lens}")
    got, glse, err = _run(w, n_q, q_lat, q_pe)
    assert err == 0
    for b in range(w.B):
        _check_seq(w, got, glse, q_lat, q_pe, b, n_q)
    # the first token of the sequence holding only the step's tokens sees row 0 alone
    row0 = w.f64(w.seq_rows(0))[0, :512]
    assert np.max(np.abs(got[0, 0] - row0[None])) <= 1e-6 * np.max(np.abs(row0))


def test_causal_single_token_is_the_plain_decode():
    """n_q = 1 runs the same kernels on the same split as mla_decode_attn:
    bit-identical outputs."""
    lens = [7, 129, 1000, 4096]
    w, q_lat, q_pe = _case(lens, 1, seed=50)
    say(f"causal n_q=1 vs decode_attn lens={lens}")
    got, glse, err = _run(w, 1, q_lat, q_pe)
    assert err == 0
    u = Uploaded(w)
    o_lat = torch.empty(w.B, 128, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.B, 128, dtype=torch.float32, device="cuda")
    L.decode_attn(u.dims, dev(q_lat[:, 0]), dev(q_pe[:, 0]), u.cache, u.offsets, u.lens, o_lat, lse,
                  total_rows_hint=w.total_rows)
    torch.cuda.synchronize()
    assert np.array_equal(got[:, 0], host_f64(o_lat))
    assert np.array_equal(glse[:, 0], host_f64(lse))


@pytest.mark.parametrize("B,n_q", [(16, 4), (13, 5), (40, 4), (300, 4), (1024, 5)])
def test_causal_many_tokens(B, n_q):
    """B n_q = 64 token-sequences is the largest count the split kernel scans
    in one wave, 65 and 160 go through its block scan, 1200 through the
    separate scan kernel, 5120 past what the scan kernel holds in LDS;
    sampled sequences (and the last) are checked."""
    rng = np.random.default_rng(B * 7 + n_q)
    lens = rng.integers(n_q, 90, size=B).astype(np.int32)
    w, q_lat, q_pe = _case(lens, n_q, seed=B + n_q)
    say(f"causal B={B} n_q={n_q} lens in [{n_q}, 90) total={int(lens.sum())}")
    got, glse, err = _run(w, n_q, q_lat, q_pe)
    assert err == 0
    for b in sorted(set(range(0, B, 17)) | {B - 1}):
        _check_seq(w, got, glse, q_lat, q_pe, b, n_q)


def test_causal_invalid_lengths_flagged():
    """lens[b] < n_q or above the capacity: every token of that sequence is NaN
    and the flag is set; the other sequences are unaffected."""
    n_q = 3
    w, q_lat, q_pe = _case([40, 50, 60], n_q, seed=60)
    say("causal invalid lengths")
    got, glse, err = _run(w, n_q, q_lat, q_pe, lens=[40, 2, 61])
    assert err & L.DEVERR_LENS
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    assert np.all(np.isnan(glse[1])) and np.all(np.isnan(glse[2]))
    _check_seq(w, got, glse, q_lat, q_pe, 0, n_q)


def test_causal_generic_fp32():
    """The plain kernel for any dims (fp32 storage, the tiny configuration's
    n_h=4, d_c=32, d_R=8): same masking rule."""
    n_h, d_c, d_r, n_q = 4, 32, 8, 3
    lens = np.array([3, 20, 64], np.int32)
    offsets = np.array([0, 5, 30, 100], np.int32)
    rng = np.random.default_rng(70)
    cache = rng.standard_normal((100, d_c + d_r)).astype(np.float32)
    q_lat = rng.standard_normal((3, n_q, n_h, d_c)).astype(np.float32)
    q_pe = rng.standard_normal((3, n_q, n_h, d_r)).astype(np.float32)
    d = L.Dims.make(n_h, d_c, d_r, 16, 16, dtype="f32")
    o_lat = torch.empty(3, n_q, n_h, d_c, dtype=torch.float32, device="cuda")
    lse = torch.empty(3, n_q, n_h, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("causal generic fp32")
    L.decode_attn_causal(d, n_q, torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_pe).cuda(),
                         torch.from_numpy(cache).cuda(), torch.from_numpy(offsets).cuda(),
                         torch.from_numpy(lens).cuda(), o_lat, lse, total_rows_hint=87, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got, glse = host_f64(o_lat), host_f64(lse)
    scale = 1 / math.sqrt(16 + 8)
    for b in range(3):
        rows = cache[offsets[b]:offsets[b] + lens[b]].astype(np.float64)
        ref, rlse = O.latent_attention_causal(q_lat[b].astype(np.float64), q_pe[b].astype(np.float64),
                                              rows[:, :d_c], rows[:, d_c:], scale)
        assert np.max(np.abs(got[b] - ref)) <= 1e-4 * max(1.0, np.max(np.abs(ref))), b
        assert np.max(np.abs(glse[b] - rlse)) <= 1e-4 * max(1.0, np.max(np.abs(rlse))), b
