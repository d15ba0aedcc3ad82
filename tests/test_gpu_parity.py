"""GPU parity of the HIP path against the fp64 oracle, at sizes the oracle
finishes in seconds (several tiles, ragged tails), plus the method's special
cases.  Every call goes through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I

from gpu_support import Uploaded, canaried_workspace, compare, dev, host_f64, oracle_seq, run_attention, say

pytestmark = pytest.mark.gpu

V3 = dict(n_h=128, d_c=512, d_r=64, d_h=128, d_v=128)


def v3_dims(**kw):
    d = dict(V3, d_model=7168, d_q=1536, dtype="bf16")
    d.update(kw)
    return L.Dims.make(**d)


def small_v3(lens, seed=0):
    rng = np.random.default_rng(seed)
    return I.attention_only("small", len(lens), np.asarray(lens, np.int32), rng, seed)


# ---------------------------------------------------------------------------
def test_tiny_fp32_end_to_end():
    """fp32, n_h=4, d_c=32, d_R=8, T=64: append raw rows (RoPE at 0..63),
    absorb the query at position 64, decode, project; generic kernels."""
    w = I.tiny()
    say("tiny: B=1 n_h=4 d_c=32 d_r=8 T=64 fp32")
    u = Uploaded(w)
    d = u.dims
    u.lens.zero_()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.append_cache(d, u.cache, u.offsets, u.lens, 64, kv_raw=dev(w.kv_raw), err_flag=err)
    torch.cuda.synchronize()
    assert int(u.lens[0].item()) == 64 and int(err.item()) == 0
    raw = w.kv_raw[0].astype(np.float64)
    c, kr = raw[:, :32], O.rope(raw[:, 32:], np.arange(64))
    got_cache = u.cache.cpu().numpy().astype(np.float64)
    assert np.array_equal(got_cache[:, :32], raw[:, :32])          # bit-exact copy
    compare(got_cache[:, 32:], kr, "cache k_R (rotated)", max_abs=2e-6, mean_abs=1e-6)
    r = run_attention(u, pos=torch.full((1,), 64, dtype=torch.int32, device="cuda"))
    o, o_lat, lse = O.decode_explicit(w.q_C[0].astype(np.float64), w.q_R[0].astype(np.float64), 64,
                                      c, kr, w.W["W_UK"].astype(np.float64),
                                      w.W["W_UV"].astype(np.float64), O.scale_for(16, 8))
    compare(host_f64(r["o_lat"])[0], o_lat, "o_lat", max_abs=1e-5, mean_abs=1e-6)
    compare(host_f64(r["o"])[0], o, "o", max_abs=1e-5, mean_abs=1e-6)
    compare(host_f64(r["lse"])[0], lse, "lse", max_abs=1e-5, mean_abs=1e-6)
    assert r["err"] == 0


@pytest.mark.parametrize("lens", [[300, 77], [1, 31, 32, 33, 64, 100, 257]])
def test_v3_attention_small(lens):
    """V3 dims, bf16: q given -> absorb -> decode (MFMA split kernel) -> W_UV."""
    w = small_v3(lens)
    say(f"v3 small: lens={lens}")
    u = Uploaded(w)
    r = run_attention(u)
    assert r["err"] == 0
    for b in range(w.B):
        o, o_lat, lse = oracle_seq(w, b)
        compare(host_f64(r["o_lat"][b]), o_lat, f"b={b} T={lens[b]} o_lat")
        compare(host_f64(r["o"][b]), o, f"b={b} o")
        compare(host_f64(r["lse"][b]), lse, f"b={b} lse", max_abs=2e-2, mean_abs=2e-3,
                norm_max=1e-2, norm_mean=2e-3)


@pytest.mark.parametrize("B", [31, 32, 33, 65])
def test_project_out_batch_blocks(B):
    """W_UV at batch sizes around the up-projection kernel's switch from two
    workgroups of two waves per head (B <= 32) to one of four waves per
    32-row batch block, with a partial last block: o against the fp64
    definition o[b,h] = W_UV[h] o_lat[b,h] for every (row, head)."""
    w = small_v3([1] * B, seed=B)
    u = Uploaded(w)
    say(f"project_out: B={B}")
    rng = np.random.default_rng(100 + B)
    o_lat = rng.standard_normal((B, 128, 512)).astype(np.float32)
    o = torch.empty(B, 128, 128, dtype=torch.float32, device="cuda")
    L.project_out(u.dims, dev(o_lat), u.W["W_UV"], o=o)
    torch.cuda.synchronize()
    ref, _ = O.project_out(o_lat, w.f64(w.W["W_UV"]))
    # o_lat enters as bf16 hi + lo (about 16 significant bits), fp32 sums
    compare(host_f64(o), ref, f"B={B} o", max_abs=1e-3, mean_abs=1e-4, norm_max=1e-3, norm_mean=1e-4)


def test_absorb_query_v3():
    """q_lat = W_UK^T q_C within one bf16 rounding; q_pe = RoPE(q_R, pos)."""
    w = small_v3([5, 9, 1000])
    u = Uploaded(w)
    r = run_attention(u)
    d = w.dims
    for b in range(w.B):
        want = O.absorb_query(w.f64(w.q_C[b]), w.f64(w.W["W_UK"]))
        got = host_f64(r["q_lat"][b])
        rel = np.abs(got - want) / np.maximum(np.abs(want), 1e-3)
        assert np.max(np.abs(got - want)) <= 2.0 ** -7 * np.max(np.abs(want))
        assert np.median(rel) < 2.0 ** -8
        pe = O.rope(w.f64(w.q_R[b]), int(w.lens[b]))
        assert np.max(np.abs(host_f64(r["q_pe"][b]) - pe)) <= 2.0 ** -7 * np.max(np.abs(pe))


def test_absorb_query_large_positions():
    """Query RoPE at positions up to 2^31 - 1 (angles up to about 2e9 rad,
    reduced modulo 2 pi in double before the single-precision sine and cosine):
    q_pe within one bf16 rounding of the fp64 rotation; q_lat unaffected."""
    w = small_v3([5, 9, 17, 33])
    u = Uploaded(w)
    pos = np.array([131072, 1048577, 123456789, 2 ** 31 - 1], np.int32)
    q_lat = torch.empty(w.B, 128, 512, dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(w.B, 128, 64, dtype=torch.bfloat16, device="cuda")
    L.absorb_q(u.dims, q_lat, q_pe, u.W["W_UK"], dev(pos), q=u.q)
    torch.cuda.synchronize()
    for b in range(w.B):
        pe = O.rope(w.f64(w.q_R[b]), int(pos[b]))
        assert np.max(np.abs(host_f64(q_pe[b]) - pe)) <= 2.0 ** -7 * np.max(np.abs(pe)), (b, int(pos[b]))
        want = O.absorb_query(w.f64(w.q_C[b]), w.f64(w.W["W_UK"]))
        assert np.max(np.abs(host_f64(q_lat[b]) - want)) <= 2.0 ** -7 * np.max(np.abs(want))


def _decode_only(w, q_lat_bits, q_pe_bits, hint=None):
    u = Uploaded(w)
    d = u.dims
    B = w.B
    o_lat = torch.empty(B, 128, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, 128, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.decode_attn(d, dev(q_lat_bits), dev(q_pe_bits), u.cache, u.offsets, u.lens, o_lat, lse,
                  total_rows_hint=hint if hint is not None else w.total_rows, err_flag=err)
    torch.cuda.synchronize()
    return host_f64(o_lat), host_f64(lse), int(err.item())


@pytest.mark.parametrize("hint", [None, 1, 10 ** 7])
def test_decode_latent_definition(hint):
    """mla_decode_attn alone against its definition (latent queries given);
    the hint changes how rows are split over workgroups, never the result."""
    lens = [1, 2, 31, 32, 33, 63, 64, 65, 250, 513]
    w = small_v3(lens, seed=3)
    rng = np.random.default_rng(5)
    q_lat = I.bf16_bits(rng.standard_normal((w.B, 128, 512)).astype(np.float32) * 0.05)
    q_pe = I.bf16_bits(rng.standard_normal((w.B, 128, 64)).astype(np.float32))
    say(f"decode-only lens={lens} hint={hint}")
    got, glse, err = _decode_only(w, q_lat, q_pe, hint)
    assert err == 0
    scale = 1 / math.sqrt(192)
    for b in range(w.B):
        rows = w.f64(w.seq_rows(b))
        ref, lse = O.latent_attention(w.f64(q_lat[b]), w.f64(q_pe[b]), rows[:, :512], rows[:, 512:], scale)
        compare(got[b], ref, f"b={b} T={lens[b]} o_lat")
        compare(glse[b], lse, f"b={b} lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2, norm_mean=1e-3)


@pytest.mark.parametrize("hint_scale", [0.125, 1, 4])
def test_decode_piece_counts(hint_scale):
    """Sequences of 40 to 9000 rows under three row hints, so that the split
    kernel cuts them into anything from one piece to a few dozen, and the
    combine merges them with one to four 32-column blocks per workgroup:
    rounds of partial loads at two, four and eight pieces, one and several
    rounds at sixteen, and the grouped loop past sixteen.  Every head of
    every sequence against the latent definition; the workspace canaries
    stay intact."""
    lens = [40, 700, 1500, 3000, 6000, 9000]
    w = small_v3(lens, seed=21)
    rng = np.random.default_rng(22)
    q_lat = I.bf16_bits(rng.standard_normal((w.B, 128, 512)).astype(np.float32) * 0.05)
    q_pe = I.bf16_bits(rng.standard_normal((w.B, 128, 64)).astype(np.float32))
    hint = max(1, int(w.total_rows * hint_scale))
    say(f"decode-only piece counts lens={lens} hint={hint}")
    u = Uploaded(w)
    o_lat = torch.empty(w.B, 128, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.B, 128, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws, check_canary = canaried_workspace(L.decode_attn_workspace(u.dims, w.B, hint))
    L.decode_attn(u.dims, dev(q_lat), dev(q_pe), u.cache, u.offsets, u.lens, o_lat, lse,
                  total_rows_hint=hint, err_flag=err, ws=ws)
    torch.cuda.synchronize()
    check_canary()
    assert int(err.item()) == 0
    got, glse = host_f64(o_lat), host_f64(lse)
    scale = 1 / math.sqrt(192)
    for b in range(w.B):
        rows = w.f64(w.seq_rows(b))
        ref, rlse = O.latent_attention(w.f64(q_lat[b]), w.f64(q_pe[b]), rows[:, :512], rows[:, 512:], scale)
        compare(got[b], ref, f"b={b} T={lens[b]} o_lat")
        compare(glse[b], rlse, f"b={b} lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2, norm_mean=1e-3)


def test_decode_more_workgroups_than_rows():
    """Fewer rows than split workgroups (a large hint over a small batch):
    most workgroup ranges are empty, several fall inside one sequence's span
    and must count as weight-0 pieces there."""
    lens = [1, 2, 3, 40, 5, 70, 1, 33]
    w = small_v3(lens, seed=11)
    rng = np.random.default_rng(12)
    q_lat = I.bf16_bits(rng.standard_normal((w.B, 128, 512)).astype(np.float32) * 0.05)
    q_pe = I.bf16_bits(rng.standard_normal((w.B, 128, 64)).astype(np.float32))
    say(f"decode-only lens={lens} hint=10**7 (empty ranges)")
    got, glse, err = _decode_only(w, q_lat, q_pe, 10 ** 7)
    assert err == 0
    scale = 1 / math.sqrt(192)
    for b in range(w.B):
        rows = w.f64(w.seq_rows(b))
        ref, lse = O.latent_attention(w.f64(q_lat[b]), w.f64(q_pe[b]), rows[:, :512], rows[:, 512:], scale)
        compare(got[b], ref, f"b={b} T={lens[b]} o_lat")
        compare(glse[b], lse, f"b={b} lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2, norm_mean=1e-3)


@pytest.mark.parametrize("B", [1024, 1100, 5000])
def test_decode_large_batch(B):
    """Many short sequences: B = 1024 is the largest batch whose lengths the
    split kernel scans itself, B = 1100 goes through the separate scan
    kernel, and B = 5000 exceeds what the scan kernel keeps in LDS (its
    prefix and charge counts are then read back from memory).  Every 37th
    sequence and the last ones are checked."""
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 41, size=B).astype(np.int32)
    w = small_v3(lens, seed=B)
    q_lat = I.bf16_bits(rng.standard_normal((B, 128, 512)).astype(np.float32) * 0.05)
    q_pe = I.bf16_bits(rng.standard_normal((B, 128, 64)).astype(np.float32))
    say(f"decode-only B={B} lens in [1, 40] total={int(lens.sum())}")
    got, glse, err = _decode_only(w, q_lat, q_pe)
    assert err == 0
    scale = 1 / math.sqrt(192)
    for b in sorted(set(range(0, B, 37)) | {B - 2, B - 1}):
        rows = w.f64(w.seq_rows(b))
        ref, lse = O.latent_attention(w.f64(q_lat[b]), w.f64(q_pe[b]), rows[:, :512], rows[:, 512:], scale)
        compare(got[b], ref, f"b={b} T={lens[b]} o_lat")
        compare(glse[b], lse, f"b={b} lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2, norm_mean=1e-3)


def test_single_row_is_exact():
    """T = 1: the only weight is exp2(0) = 1, so o_lat is the row itself, bit for bit."""
    w = small_v3([1, 1, 1])
    rng = np.random.default_rng(7)
    q_lat = I.bf16_bits(rng.standard_normal((3, 128, 512)).astype(np.float32))
    q_pe = I.bf16_bits(rng.standard_normal((3, 128, 64)).astype(np.float32))
    got, glse, err = _decode_only(w, q_lat, q_pe)
    for b in range(3):
        row = w.f64(w.seq_rows(b))[0, :512]
        assert np.array_equal(got[b], np.broadcast_to(row, (128, 512)))
        s = (w.f64(q_lat[b]) @ w.f64(w.seq_rows(b))[0, :512]
             + w.f64(q_pe[b]) @ w.f64(w.seq_rows(b))[0, 512:]) / math.sqrt(192)
        assert np.max(np.abs(glse[b] - s)) < 1e-3 * max(1.0, np.max(np.abs(s)))


def test_zero_query_gives_exact_mean():
    """q = 0: uniform weights; rows of small integers make the mean exact."""
    T = 128
    w = small_v3([T, 37])
    rng = np.random.default_rng(9)
    ints = rng.integers(-8, 9, size=w.cache.shape).astype(np.float32)
    w.cache[:] = I.bf16_bits(ints)
    z = np.zeros((2, 128, 512), np.uint16)
    zp = np.zeros((2, 128, 64), np.uint16)
    got, glse, err = _decode_only(w, z, zp)
    for b, t in enumerate([T, 37]):
        mean = w.f64(w.seq_rows(b))[:, :512].mean(axis=0)
        tol = 0.0 if t == T else 1e-6
        assert np.max(np.abs(got[b] - mean[None])) <= tol
        assert np.allclose(glse[b], math.log(t), atol=1e-5)


def test_dominant_row_and_fallback():
    """A row whose score exceeds the first tile's by far more than 2^64 forces
    the flagged-sequence recompute; the answer is that row."""
    w = small_v3([700, 300])
    rng = np.random.default_rng(11)
    q_lat = I.bf16_bits(rng.standard_normal((2, 128, 512)).astype(np.float32) * 0.02)
    q_pe = np.zeros((2, 128, 64), np.float32)
    q_pe[:, :, 0] = 1.0
    q_pe = I.bf16_bits(q_pe)
    # sequence 0: row 600 has k_R[0] = 2000 -> score jump ~2000/sqrt(192)*log2(e) ~ 208 (log2)
    o0 = int(w.offsets[0])
    kr = w.cache[o0 + 600, 512:].copy()
    kr[0] = I.bf16_bits(np.array([2000.0], np.float32))[0]
    w.cache[o0 + 600, 512:] = kr
    # sequence 1: a moderate jump (~2^10) that the fast path absorbs without fallback
    o1 = int(w.offsets[1])
    w.cache[o1 + 250, 512] = I.bf16_bits(np.array([120.0], np.float32))[0]
    got, glse, err = _decode_only(w, q_lat, q_pe)
    assert err == 0
    scale = 1 / math.sqrt(192)
    for b in range(2):
        rows = w.f64(w.seq_rows(b))
        ref, lse = O.latent_attention(w.f64(q_lat[b]), w.f64(q_pe[b]), rows[:, :512], rows[:, 512:], scale)
        compare(got[b], ref, f"b={b} o_lat")
        assert np.max(np.abs(glse[b] - lse)) < 1e-3 * np.max(np.abs(lse))
    assert np.allclose(got[0], w.f64(w.seq_rows(0))[600, :512][None], atol=1e-5)


def test_partial_outside_fp16_range_falls_back():
    """A piece whose normalised partial exceeds the fp16 range (one row of
    3e7 among N(0,1) rows, zero query so every weight is 1) is flagged and the
    sequence recomputed: the result is the exact mean of its rows."""
    w = small_v3([3000, 500])
    o0 = int(w.offsets[0])
    w.cache[o0 + 1500, :512] = I.bf16_bits(np.full(512, 3.0e7, np.float32))
    q_lat = I.bf16_bits(np.zeros((2, 128, 512), np.float32))
    q_pe = I.bf16_bits(np.zeros((2, 128, 64), np.float32))
    got, glse, err = _decode_only(w, q_lat, q_pe)
    assert err == 0
    for b in range(2):
        rows = w.f64(w.seq_rows(b))[:, :512]
        mean = rows.mean(axis=0)
        assert np.all(np.isfinite(got[b])), b
        assert np.max(np.abs(got[b] - mean[None])) <= 1e-5 * np.max(np.abs(mean)) + 1e-4, b
        assert np.max(np.abs(glse[b] - math.log(rows.shape[0]))) < 1e-4, b


def test_invalid_lengths_flagged():
    w = small_v3([40, 50, 60])
    u = Uploaded(w)
    d = u.dims
    lens = torch.tensor([40, 0, 61], dtype=torch.int32, device="cuda")   # 0 and > capacity
    q_lat = torch.zeros(3, 128, 512, dtype=torch.bfloat16, device="cuda")
    q_pe = torch.zeros(3, 128, 64, dtype=torch.bfloat16, device="cuda")
    o_lat = torch.zeros(3, 128, 512, dtype=torch.float32, device="cuda")
    lse = torch.zeros(3, 128, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.decode_attn(d, q_lat, q_pe, u.cache, u.offsets, lens, o_lat, lse, total_rows_hint=150, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & L.DEVERR_LENS
    o = o_lat.cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    mean = w.f64(w.seq_rows(0))[:, :512].mean(axis=0)
    assert np.max(np.abs(o[0] - mean[None])) < 1e-5


def test_append_raw_bit_exact_with_canaries():
    """Rows land at offsets[b] + lens[b]; the latent part is copied bit for
    bit; k_R is rotated to its position (exactly at position 0); nothing else
    in the cache changes; a full region is refused and flagged."""
    d = v3_dims()
    B = 4
    caps = np.array([3, 5, 2, 4])
    offsets = np.concatenate([[0], np.cumsum(caps)]).astype(np.int32)
    lens0 = np.array([0, 2, 2, 3], np.int32)       # sequence 2 is full
    canary = np.uint16(0x7FA5)                      # a NaN pattern
    cache = np.full((offsets[-1], 576), canary, np.uint16)
    rng = np.random.default_rng(13)
    kv = I.bf16_bits(rng.standard_normal((B, 1, 576)).astype(np.float32))
    dc, do, dl = dev(cache), dev(offsets), dev(lens0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.append_cache(d, dc, do, dl, 1, kv_raw=dev(kv), err_flag=err)
    torch.cuda.synchronize()
    got = dc.view(torch.int16).cpu().numpy().view(np.uint16)
    assert list(dl.cpu().numpy()) == [1, 3, 2, 4]
    assert int(err.item()) & L.DEVERR_OVERFLOW
    expect = cache.copy()
    for b in range(B):
        if b == 2:
            continue
        r = offsets[b] + lens0[b]
        assert np.array_equal(got[r, :512], kv[b, 0, :512]), b
        kr = O.rope(I.bf16_to_f32(kv[b, 0, 512:]).astype(np.float64), int(lens0[b]))
        g = I.bf16_to_f32(got[r, 512:]).astype(np.float64)
        if lens0[b] == 0:
            assert np.array_equal(got[r, 512:], kv[b, 0, 512:])
        else:
            assert np.all(np.abs(g - kr) <= 2.0 ** -8 * np.abs(kr) + 1e-30)
        expect[r] = got[r]
    assert np.array_equal(got, expect)           # every other row still holds the canary


def test_decode_is_deterministic():
    w = small_v3([900, 1500, 33], seed=21)
    u = Uploaded(w)
    a = run_attention(u)
    b = run_attention(u)
    assert torch.equal(a["o_lat"], b["o_lat"]) and torch.equal(a["lse"], b["lse"])
