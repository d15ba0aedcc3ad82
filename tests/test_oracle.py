"""Pins for the fp64 oracle: each test ties it to something other than itself.

Sources of truth used here: numbers and shapes printed on the pages (fixtures
under tests/golden/ with their citations), the associativity identities the
pages state for absorption, an independent library routine (torch's
scaled_dot_product_attention in float64), a pure-Python brute force on tiny
inputs, closed forms and invariants of RoPE and softmax, and special cases
whose answer is known without running attention.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from head_latent_attention_16_amd import inputs as I

RTOL = 1e-12


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


def rand_case(rng, n_h=3, d_c=12, d_r=6, d_h=5, d_v=7, T=9):
    """Non-square, mutually distinct dims so that a transposed operand cannot pass."""
    return dict(
        q_C=rng.standard_normal((n_h, d_h)),
        q_R=rng.standard_normal((n_h, d_r)),
        c=rng.standard_normal((T, d_c)),
        k=rng.standard_normal((T, d_r)),
        W_UK=rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c),
        W_UV=rng.standard_normal((n_h, d_v, d_c)) / math.sqrt(d_c),
        pos=T,
        scale=1.0 / math.sqrt(d_h + d_r),
    )


# ---------------------------------------------------------------------------
# Cache-size arithmetic against the printed numbers
# ---------------------------------------------------------------------------
UNITS = {"B": 1, "kB": 1e3, "KiB": 1024, "MB": 1e6, "MiB": 2 ** 20, "GB": 1e9, "GiB": 2 ** 30}


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_cache_sizes_match_pages(golden_dir):
    g = _golden(golden_dir, "cache_sizes.json")
    sizes = {}
    for e in g["entries"]:
        got = O.cache_bytes_per_token(e["kind"], e["layers"], e["bytes_per_elem"], **e["dims"])
        assert got == e["exact_bytes"], e["id"]
        printed = e["printed"] * UNITS[e["unit"]]
        assert abs(got - printed) <= max(0.5, e["rel_tol"] * printed + 0.05 * UNITS[e["unit"]]), e["id"]
        sizes[e["id"]] = got
    for e in g["context_totals"]:
        total = sizes[e["per_token_id"]] * e["tokens"]
        printed = e["printed"] * UNITS[e["unit"]]
        assert abs(total - printed) <= e["rel_tol"] * printed, e["id"]
    for e in g["ratios"]:
        if "num" in e:
            pct = 100.0 * sizes[e["num"]] / sizes[e["den"]]
        else:
            pct = 100.0 * e["num_elems"] / e["den_elems"]
        assert abs(pct - e["printed_percent"]) <= e["abs_tol_percent"] + 1e-9, e["id"]


def test_cache_size_table_forms():
    # [MLA-visual] cache-size table: with d_c = 4 d_h and d_R = d_h / 2 the MLA
    # cache is 9/2 d_h per layer, i.e. GQA with 2.25 groups.
    for d_h in (64, 128, 256):
        mla = O.cache_elems_per_token_layer("mla", d_c=4 * d_h, d_r=d_h // 2)
        assert mla * 2 == 9 * d_h
        assert O.cache_elems_per_token_layer("gqa", n_g=1, d_h=d_h) == O.cache_elems_per_token_layer("mqa", d_h=d_h)
        assert mla / O.cache_elems_per_token_layer("gqa", n_g=1, d_h=d_h) == 2.25
    # MHA is GQA with one group per head.
    assert O.cache_elems_per_token_layer("mha", n_h=128, d_h=128) == O.cache_elems_per_token_layer("gqa", n_g=128, d_h=128)
    # V3 row: 576 elements = 1152 bytes in bf16.
    assert O.cache_elems_per_token_layer("mla", d_c=512, d_r=64) * 2 == 1152


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def test_rope_matches_complex_rotation():
    # Independent statement of rotate-half RoPE: pair (x_i, x_{i+d/2}) is the
    # complex number x_i + j x_{i+d/2}, multiplied by exp(j pos theta_i).
    rng = np.random.default_rng(1)
    for d in (2, 4, 8, 64):
        x = rng.standard_normal((5, d))
        pos = np.array([0, 1, 7, 1000, 131072])
        z = x[:, : d // 2] + 1j * x[:, d // 2:]
        theta = np.array([10000.0 ** (-(2.0 * i) / d) for i in range(d // 2)])
        zr = z * np.exp(1j * pos[:, None] * theta[None, :])
        want = np.concatenate([zr.real, zr.imag], axis=1)
        # cos/sin of an angle A carry ~A*eps of argument-rounding error
        tol = 8e-16 * (1.0 + pos[:, None]) * np.max(np.abs(x))
        assert np.all(np.abs(O.rope(x, pos) - want) <= tol)


def test_rope_two_dim_closed_form():
    # d_R = 2: theta_0 = 1, so RoPE is the plane rotation by `pos` radians.
    x = np.array([0.3, -1.7])
    for p in (0, 1, 2, 5, 4096):
        c, s = math.cos(p), math.sin(p)
        want = np.array([c * x[0] - s * x[1], s * x[0] + c * x[1]])
        assert np.allclose(O.rope(x, p), want, rtol=0, atol=1e-15)


def test_rope_properties():
    rng = np.random.default_rng(2)
    d = 64
    x = rng.standard_normal((4, d))
    y = rng.standard_normal((4, d))
    # position 0 is the identity, bit for bit
    assert np.array_equal(O.rope(x, 0), x)
    # a rotation preserves the norm
    r = O.rope(x, 12345)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # composition adds positions
    assert rel_err(O.rope(O.rope(x, 100), 23), O.rope(x, 123)) < 1e-12
    # scores depend only on the relative position
    for p, j, delta in ((5, 3, 11), (4096, 17, 1000), (0, 0, 77)):
        a = np.sum(O.rope(x, p) * O.rope(y, j), axis=1)
        b = np.sum(O.rope(x, p + delta) * O.rope(y, j + delta), axis=1)
        assert np.allclose(a, b, rtol=1e-11, atol=1e-12)
    # the last pair rotates slowest: theta = base^(-(d-2)/d)
    e_last = np.zeros(d)
    e_last[d // 2 - 1] = 1.0
    ang = math.atan2(O.rope(e_last, 1000)[d - 1], O.rope(e_last, 1000)[d // 2 - 1])
    assert abs(ang - 1000 * 10000.0 ** (-(d - 2) / d)) < 1e-12


# ---------------------------------------------------------------------------
# Softmax
# ---------------------------------------------------------------------------
def test_softmax_rows_and_lse():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((6, 40)) * 3
    p, lse = O.softmax_two_pass(s)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p > 0)
    want = np.log(np.sum(np.exp(s), axis=1))
    assert np.allclose(lse, want, rtol=1e-14)
    # shift invariance and no overflow for large logits
    p2, lse2 = O.softmax_two_pass(s + 1000.0)
    assert np.allclose(p2, p, rtol=1e-12)
    assert np.allclose(lse2, lse + 1000.0, rtol=1e-14)


def test_split_softmax_combine_equals_whole():
    # What the split-T combine relies on: merging per-chunk (max, sum, weighted
    # sum) by log-sum-exp reproduces the softmax over the whole row.
    rng = np.random.default_rng(4)
    s = rng.standard_normal(100) * 4
    v = rng.standard_normal((100, 7))
    p, lse = O.softmax_two_pass(s)
    whole = p @ v
    cuts = [0, 13, 14, 60, 100]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        m = s[a:b].max()
        e = np.exp(s[a:b] - m)
        parts.append((m, e.sum(), e @ v[a:b]))
    M = max(m for m, _, _ in parts)
    L = sum(l * math.exp(m - M) for m, l, _ in parts)
    acc = sum(o * math.exp(m - M) for m, _, o in parts) / L
    assert rel_err(acc, whole) < 1e-13
    assert abs((M + math.log(L)) - lse) < 1e-13


# ---------------------------------------------------------------------------
# Attention: explicit route vs absorbed route vs library routine vs brute force
# ---------------------------------------------------------------------------
def test_absorbed_equals_explicit():
    # [MLA-struct] absorption identities: q.(W^UK c) = (q W^UK).c and
    # sum_j a_j W^UV c_j = W^UV sum_j a_j c_j.
    rng = np.random.default_rng(5)
    for T in (1, 2, 9, 200):
        k = rand_case(rng, T=T)
        o, o_lat, lse = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"], k["k"],
                                          k["W_UK"], k["W_UV"], k["scale"])
        q_lat = O.absorb_query(k["q_C"], k["W_UK"])
        q_pe = O.rope(k["q_R"], k["pos"])
        o_lat2, lse2 = O.latent_attention(q_lat, q_pe, k["c"], k["k"], k["scale"])
        o2, _ = O.project_out(o_lat2[None], k["W_UV"])
        assert rel_err(o_lat2, o_lat) < RTOL
        assert rel_err(o2[0], o) < RTOL
        assert np.max(np.abs(lse2 - lse)) < 1e-12


def test_concat_score_equals_split_score():
    # [q^C; q^R].[k^C; k^R] equals the sum of the content and rope dot products.
    rng = np.random.default_rng(6)
    k = rand_case(rng)
    h = 1
    keys, _ = O.explicit_kv(k["c"], k["k"], k["W_UK"][h], k["W_UV"][h])
    qr = O.rope(k["q_R"][h], k["pos"])
    s_cat = keys @ np.concatenate([k["q_C"][h], qr])
    s_split = (k["c"] @ k["W_UK"][h].T) @ k["q_C"][h] + k["k"] @ qr
    assert rel_err(s_cat, s_split) < RTOL


def test_explicit_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(7)
    for T in (1, 5, 64, 300):
        k = rand_case(rng, n_h=4, d_c=32, d_r=8, d_h=16, d_v=16, T=T)
        o, _, _ = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"], k["k"],
                                    k["W_UK"], k["W_UV"], k["scale"])
        c = torch.from_numpy(k["c"])
        kr = torch.from_numpy(k["k"])
        qr = torch.from_numpy(O.rope(k["q_R"], k["pos"]))
        qc = torch.from_numpy(k["q_C"])
        Wk = torch.from_numpy(k["W_UK"])
        Wv = torch.from_numpy(k["W_UV"])
        K = torch.cat([torch.matmul(c, Wk.transpose(1, 2).contiguous()),
                       kr.unsqueeze(0).expand(Wk.shape[0], -1, -1)], dim=-1)      # [h, T, d_h + d_r]
        V = torch.matmul(c, Wv.transpose(1, 2).contiguous())                     # [h, T, d_v]
        q = torch.cat([qc, qr], dim=-1).unsqueeze(1)                             # [h, 1, d_h + d_r]
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=k["scale"])[:, 0]
        assert rel_err(o, ref.numpy()) < 1e-12


def _brute_force(q_C, q_R, pos, c, kr, W_UK, W_UV, scale):
    """Scalar loops with math.* only: no numpy arithmetic."""
    n_h, d_h = len(q_C), len(q_C[0])
    d_r = len(q_R[0])
    T, d_c = len(c), len(c[0])
    d_v = len(W_UV[0])
    half = d_r // 2
    out = []
    for h in range(n_h):
        qr = [0.0] * d_r
        for i in range(half):
            th = pos * 10000.0 ** (-2.0 * i / d_r)
            qr[i] = q_R[h][i] * math.cos(th) - q_R[h][i + half] * math.sin(th)
            qr[i + half] = q_R[h][i + half] * math.cos(th) + q_R[h][i] * math.sin(th)
        scores = []
        for j in range(T):
            s = 0.0
            for a in range(d_h):
                kc = 0.0
                for e in range(d_c):
                    kc += W_UK[h][a][e] * c[j][e]
                s += q_C[h][a] * kc
            for i in range(d_r):
                s += qr[i] * kr[j][i]
            scores.append(s * scale)
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        z = sum(w)
        o = []
        for v in range(d_v):
            acc = 0.0
            for j in range(T):
                vj = 0.0
                for e in range(d_c):
                    vj += W_UV[h][v][e] * c[j][e]
                acc += w[j] / z * vj
            o.append(acc)
        out.append(o)
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(8)
    for (n_h, d_c, d_r, d_h, d_v, T) in ((1, 4, 2, 3, 2, 1), (2, 4, 2, 3, 2, 5), (2, 3, 4, 2, 3, 4)):
        k = rand_case(rng, n_h=n_h, d_c=d_c, d_r=d_r, d_h=d_h, d_v=d_v, T=T)
        o, _, _ = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"], k["k"],
                                    k["W_UK"], k["W_UV"], k["scale"])
        bf = _brute_force(k["q_C"].tolist(), k["q_R"].tolist(), k["pos"], k["c"].tolist(),
                          k["k"].tolist(), k["W_UK"].tolist(), k["W_UV"].tolist(), k["scale"])
        assert rel_err(o, bf) < RTOL


def test_brute_force_tiny_workload_heads():
    # The tiny fp32 workload itself (n_h=4, d_c=32, d_R=8, d_h=16, T=64), on a row subset.
    w = I.tiny()
    raw = w.kv_raw[0].astype(np.float64)
    c = raw[:, :32]
    kr = O.rope(raw[:, 32:], np.arange(64))
    o, _, _ = O.decode_explicit(w.q_C[0].astype(np.float64), w.q_R[0].astype(np.float64), 64,
                                c, kr, w.W["W_UK"].astype(np.float64), w.W["W_UV"].astype(np.float64),
                                O.scale_for(16, 8))
    bf = _brute_force(w.q_C[0].astype(np.float64).tolist(), w.q_R[0].astype(np.float64).tolist(), 64,
                      c.tolist(), kr.tolist(), w.W["W_UK"].astype(np.float64).tolist(),
                      w.W["W_UV"].astype(np.float64).tolist(), O.scale_for(16, 8))
    assert rel_err(o, bf) < RTOL


# ---------------------------------------------------------------------------
# Special cases with known answers
# ---------------------------------------------------------------------------
def test_single_row_returns_that_row():
    rng = np.random.default_rng(9)
    k = rand_case(rng, T=1)
    o, o_lat, lse = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"], k["k"],
                                      k["W_UK"], k["W_UV"], k["scale"])
    for h in range(len(o)):
        assert np.array_equal(o_lat[h], k["c"][0])
        assert rel_err(o[h], k["W_UV"][h] @ k["c"][0]) < RTOL


def test_zero_query_gives_mean():
    rng = np.random.default_rng(10)
    k = rand_case(rng, T=16)
    z_C = np.zeros_like(k["q_C"])
    z_R = np.zeros_like(k["q_R"])
    _, o_lat, lse = O.decode_explicit(z_C, z_R, k["pos"], k["c"], k["k"], k["W_UK"], k["W_UV"], k["scale"])
    assert np.allclose(o_lat, k["c"].mean(axis=0)[None], rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(16), atol=1e-14)


def test_identical_rows_and_dominant_row():
    rng = np.random.default_rng(11)
    k = rand_case(rng, T=8)
    c = np.repeat(k["c"][:1], 8, axis=0)
    kr = np.repeat(k["k"][:1], 8, axis=0)
    _, o_lat, _ = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], c, kr, k["W_UK"], k["W_UV"], k["scale"])
    assert np.allclose(o_lat, c[0][None], rtol=1e-14, atol=1e-14)
    # make row 5's rope key align with a huge rotated query -> its weight -> 1
    q_R = k["q_R"].copy()
    kr = k["k"].copy()
    qr = O.rope(q_R, k["pos"])
    kr[5] = 1e3 * qr[0] / np.linalg.norm(qr[0])
    _, o_lat, _ = O.decode_explicit(k["q_C"][:1], q_R[:1], k["pos"], k["c"], kr,
                                    k["W_UK"][:1], k["W_UV"][:1], k["scale"])
    assert np.allclose(o_lat[0], k["c"][5], atol=1e-9)


def test_row_permutation_invariance():
    rng = np.random.default_rng(12)
    k = rand_case(rng, T=30)
    perm = rng.permutation(30)
    a = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"], k["k"], k["W_UK"], k["W_UV"], k["scale"])
    b = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"][perm], k["k"][perm], k["W_UK"], k["W_UV"], k["scale"])
    for x, y in zip(a, b):
        assert rel_err(x, y) < 1e-12


def test_rope_key_shared_by_heads():
    # k^R has no head index: giving every head the same q^R yields identical
    # rope scores across heads, so heads with equal content parts agree exactly.
    rng = np.random.default_rng(13)
    k = rand_case(rng, n_h=3, T=10)
    q_C = np.repeat(k["q_C"][:1], 3, axis=0)
    q_R = np.repeat(k["q_R"][:1], 3, axis=0)
    W_UK = np.repeat(k["W_UK"][:1], 3, axis=0)
    _, o_lat, lse = O.decode_explicit(q_C, q_R, k["pos"], k["c"], k["k"], W_UK, k["W_UV"], k["scale"])
    assert np.array_equal(o_lat[0], o_lat[1]) and np.array_equal(o_lat[0], o_lat[2])


# ---------------------------------------------------------------------------
# Projections, query path, append and the full layer step
# ---------------------------------------------------------------------------
def test_query_path_head_layout():
    # W_UQ rows are head-major with [d_h content | d_R rope] per head; with a
    # selection matrix the split can be read off exactly.
    n_h, d_h, d_r, d_q, d = 3, 4, 2, 5, 7
    rng = np.random.default_rng(14)
    h = rng.standard_normal((2, d))
    W_DQ = rng.standard_normal((d_q, d))
    rows = n_h * (d_h + d_r)
    W_UQ = np.zeros((rows, d_q))
    W_UQ[np.arange(rows), np.arange(rows) % d_q] = np.arange(1, rows + 1)
    q_C, q_R = O.query_path(h, W_DQ, W_UQ, n_h, d_h, d_r)
    cq = h @ W_DQ.T
    for b in range(2):
        for hh in range(n_h):
            for i in range(d_h):
                r = hh * (d_h + d_r) + i
                assert q_C[b, hh, i] == cq[b, r % d_q] * (r + 1)
            for i in range(d_r):
                r = hh * (d_h + d_r) + d_h + i
                assert q_R[b, hh, i] == cq[b, r % d_q] * (r + 1)


def test_project_out_flatten_order():
    # u = W_O flatten(o) with the flat index h * d_v + v.
    n_h, d_v, d_c, dm = 3, 4, 6, 5
    rng = np.random.default_rng(15)
    o_lat = rng.standard_normal((2, n_h, d_c))
    W_UV = rng.standard_normal((n_h, d_v, d_c))
    W_O = np.zeros((dm, n_h * d_v))
    W_O[0, 1 * d_v + 2] = 1.0   # u[:,0] picks head 1, value dim 2
    W_O[4, 2 * d_v + 0] = 2.0
    o, u = O.project_out(o_lat, W_UV, W_O)
    for b in range(2):
        for hh in range(n_h):
            assert rel_err(o[b, hh], W_UV[hh] @ o_lat[b, hh]) < RTOL
        assert u[b, 0] == o[b, 1, 2]
        assert u[b, 4] == 2.0 * o[b, 2, 0]
        assert u[b, 1] == 0.0


def test_append_rows_selection_weights():
    d, d_c, d_r = 10, 4, 2
    rng = np.random.default_rng(16)
    x = rng.standard_normal((3, d))
    W_DKV = np.eye(d_c, d)
    W_KR = np.zeros((d_r, d))
    W_KR[0, 5] = 1.0
    W_KR[1, 6] = 1.0
    c, kr = O.append_rows(x, W_DKV, W_KR, [0, 1, 2])
    assert np.array_equal(c, x[:, :d_c])
    assert np.array_equal(kr[0], x[0, 5:7])      # position 0: no rotation
    assert rel_err(kr[2], O.rope(x[2, 5:7], 2)) < RTOL
    assert abs(np.linalg.norm(kr[1]) - np.linalg.norm(x[1, 5:7])) < 1e-14


def test_layer_step_consistent_and_shapes(golden_dir):
    # The page's worked example (n_heads=16, dim=2048, start_pos=1024): every
    # printed shape, and the layer step equals its pieces composed by hand.
    g = _golden(golden_dir, "worked_example_shapes.json")
    cfg = g["config"]
    n_h, dm, d_c, d_h, d_r, d_v = (cfg["n_heads"], cfg["dim"], cfg["kv_lora_rank"],
                                   cfg["qk_nope_head_dim"], cfg["qk_rope_head_dim"], cfg["v_head_dim"])
    T0 = cfg["start_pos"]
    rng = np.random.default_rng(17)
    x = rng.standard_normal((1, dm))
    W = dict(
        W_DQ=None,
        W_UQ=rng.standard_normal((n_h * (d_h + d_r), dm)) / math.sqrt(dm),
        W_DKV=rng.standard_normal((d_c, dm)) / math.sqrt(dm),
        W_KR=rng.standard_normal((d_r, dm)) / math.sqrt(dm),
        W_UK=rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c),
        W_UV=rng.standard_normal((n_h, d_v, d_c)) / math.sqrt(d_c),
        W_O=rng.standard_normal((dm, n_h * d_v)) / math.sqrt(n_h * d_v),
    )
    prior_c = [rng.standard_normal((T0, d_c))]
    prior_k = [rng.standard_normal((T0, d_r))]
    scale = O.scale_for(d_h, d_r)
    res = O.layer_step(x, W, prior_c, prior_k, dict(n_h=n_h, d_h=d_h, d_r=d_r), scale)[0]
    S = g["shapes"]
    q_C, q_R = O.query_path(x, None, W["W_UQ"], n_h, d_h, d_r)
    assert [1, 1] + list(np.concatenate([q_C, q_R], -1)[0].shape) == S["q"]
    assert [1, 1] + list(q_C[0].shape) == S["q_nope"]
    assert [1, 1] + list(q_R[0].shape) == S["q_pe"]
    c_new, k_new = O.append_rows(x, W["W_DKV"], W["W_KR"], [T0])
    assert [1, 1, c_new.shape[1] + k_new.shape[1]] == S["kv_and_pe"]
    assert [1, 1, c_new.shape[1]] == S["kv_latent"] and [1, 1, k_new.shape[1]] == S["k_pe"]
    c_all = np.concatenate([prior_c[0], c_new])
    k_all = np.concatenate([prior_k[0], k_new])
    assert [1] + list(c_all.shape) == S["kv_cache_visible"]
    assert [1] + list(k_all.shape) == S["pe_cache_visible"]
    q_lat = O.absorb_query(q_C[0], W["W_UK"])
    assert [1, 1] + list(q_lat.shape) == S["q_nope_absorb"]
    s = q_lat @ c_all.T
    assert [1, 1] + list(s.shape) == S["score_C"]
    z, lse = O.latent_attention(q_lat, O.rope(q_R[0], T0), c_all, k_all, scale)
    assert [1, 1] + list(z.shape) == S["z"]
    o, u = O.project_out(z[None], W["W_UV"], W["W_O"])
    assert [1, 1] + list(o[0].shape) == S["o"]
    assert [1, 1] + list(u[0].shape) == S["u"]
    assert rel_err(res["o_lat"], z) < 1e-11
    assert rel_err(res["u"], u[0]) < 1e-11
    assert rel_err(res["lse"], lse) < 1e-12
    assert g["elements_per_token_layer"]["mla"] == d_c + d_r
    assert g["elements_per_token_layer"]["full_kv"] == n_h * (d_h + d_r + d_v)


# ---------------------------------------------------------------------------
# The softmax scale against the values the workload statements write out.
# ---------------------------------------------------------------------------
def _scale_pinned(scale_fn, golden):
    return all(abs(scale_fn(e["d_h"], e["d_r"]) - e["value"]) <= 1e-15 * e["value"]
               for e in golden["entries"])


def test_softmax_scale_matches_workload_statements(golden_dir, monkeypatch):
    g = _golden(golden_dir, "softmax_scale.json")
    assert _scale_pinned(O.scale_for, g)
    # the explicit route applies it to the sum of the content and RoPE scores:
    # one row, so lse is that scaled score exactly
    rng = np.random.default_rng(26)
    for e in g["entries"]:
        k = rand_case(rng, n_h=2, d_c=12, d_r=e["d_r"], d_h=e["d_h"], d_v=5, T=1)
        _, _, lse = O.decode_explicit(k["q_C"], k["q_R"], 1, k["c"], k["k"], k["W_UK"], k["W_UV"],
                                      O.scale_for(e["d_h"], e["d_r"]))
        raw = (np.einsum("hk,hkc,c->h", k["q_C"], k["W_UK"], k["c"][0])
               + O.rope(k["q_R"], 1) @ k["k"][0])
        assert rel_err(lse, raw * e["value"]) < RTOL
    # planted mistakes: 1/sqrt(d_h) (content width only) and 1/(d_h + d_R)
    monkeypatch.setattr(O.mla_oracle, "scale_for", lambda d_h, d_r: 1.0 / math.sqrt(d_h))
    assert not _scale_pinned(O.mla_oracle.scale_for, g)
    monkeypatch.setattr(O.mla_oracle, "scale_for", lambda d_h, d_r: 1.0 / (d_h + d_r))
    assert not _scale_pinned(O.mla_oracle.scale_for, g)


# ---------------------------------------------------------------------------
# The latent norms (root-mean-square reading).
def test_rms_norm_matches_torch_and_closed_forms():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((5, 512)) * 3.0
    w = 1.0 + 0.1 * rng.standard_normal(512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(w), eps=1e-6)
    assert rel_err(O.rms_norm(x, w, 1e-6), ref.numpy()) < 1e-12
    # a constant row a: every output is a / sqrt(a^2 + eps) times its weight
    a = 0.37
    y = O.rms_norm(np.full((1, 8), a), np.arange(1.0, 9.0), 1e-6)
    assert rel_err(y[0], a / math.sqrt(a * a + 1e-6) * np.arange(1.0, 9.0)) < RTOL
    # unit weight, eps 0: the output's root mean square is exactly 1 and
    # rescaling the input changes nothing
    z = O.rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(np.sqrt(np.mean(z * z, axis=1)), 1.0, rtol=1e-14, atol=0)
    assert rel_err(O.rms_norm(5.5 * x, np.ones(512), 0.0), z) < RTOL


def test_norms_sit_on_the_latents():
    # the kv norm acts on c^KV only (k^R untouched); the query norm on c^Q
    rng = np.random.default_rng(25)
    x = rng.standard_normal((3, 40))
    W_DKV, W_KR = rng.standard_normal((12, 40)), rng.standard_normal((6, 40))
    g = 1.0 + 0.2 * rng.standard_normal(12)
    c0, k0 = O.append_rows(x, W_DKV, W_KR, [4, 5, 6])
    c1, k1 = O.append_rows(x, W_DKV, W_KR, [4, 5, 6], kv_norm_w=g)
    assert rel_err(k1, k0) == 0.0
    assert rel_err(c1, O.rms_norm(x @ W_DKV.T, g)) < RTOL
    W_DQ, W_UQ = rng.standard_normal((10, 40)), rng.standard_normal((2 * 7, 10))
    gq = 1.0 + 0.2 * rng.standard_normal(10)
    qc, qr = O.query_path(x, W_DQ, W_UQ, 2, 4, 3, q_norm_w=gq)
    q = O.rms_norm(x @ W_DQ.T, gq) @ W_UQ.T
    assert rel_err(np.concatenate([qc, qr], -1).reshape(3, -1), q) < RTOL


# ---------------------------------------------------------------------------
# Several new tokens per step (causal mask).
def _causal_case(rng, T, n_q, n_h=3, d_c=12, d_r=6):
    return (rng.standard_normal((n_q, n_h, d_c)), rng.standard_normal((n_q, n_h, d_r)),
            rng.standard_normal((T, d_c)), rng.standard_normal((T, d_r)), 0.3)


def test_causal_matches_torch_sdpa_mask_fp64():
    # torch's attention with a boolean lower-triangular mask, offset so that
    # query i of n_q keeps keys j <= T - n_q + i; keys [c | k^R], values c.
    rng = np.random.default_rng(21)
    for T, n_q in ((1, 1), (5, 5), (9, 3), (64, 4), (300, 7)):
        ql, qp, c, kr, scale = _causal_case(rng, T, n_q)
        n_h = ql.shape[1]
        o, lse = O.latent_attention_causal(ql, qp, c, kr, scale)
        K = torch.from_numpy(np.concatenate([c, kr], 1)).unsqueeze(0).expand(n_h, -1, -1)
        V = torch.from_numpy(c).unsqueeze(0).expand(n_h, -1, -1)
        q = torch.from_numpy(np.concatenate([ql, qp], 2)).transpose(0, 1).contiguous()   # [n_h, n_q, D]
        mask = torch.ones(n_q, T, dtype=torch.bool).tril(T - n_q)
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=scale)
        assert rel_err(o, ref.transpose(0, 1).numpy()) < 1e-12
        sc = torch.matmul(q, K.transpose(1, 2).contiguous()) * scale
        ref_lse = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1)           # [n_h, n_q]
        assert rel_err(lse, ref_lse.transpose(0, 1).numpy()) < 1e-12


def test_causal_token_equals_decode_over_its_prefix():
    # token i of the step is a single-query decode over rows 0 .. T - n_q + i;
    # with n_q = 1 the step is the plain decode over all T rows
    rng = np.random.default_rng(22)
    for T, n_q in ((7, 1), (12, 4), (6, 6)):
        ql, qp, c, kr, scale = _causal_case(rng, T, n_q)
        o, lse = O.latent_attention_causal(ql, qp, c, kr, scale)
        for i in range(n_q):
            n = T - n_q + i + 1
            oi, lsei = O.latent_attention(ql[i], qp[i], c[:n], kr[:n], scale)
            assert rel_err(o[i], oi) < RTOL and rel_err(lse[i], lsei) < RTOL
        # an off-by-one mask (token i seeing one row fewer) is a different result
        if n_q > 1 and T > n_q:
            n = T - n_q + 1
            oi, _ = O.latent_attention(ql[1], qp[1], c[:n], kr[:n], scale)
            assert rel_err(o[1], oi) > 1e-3


def test_causal_first_token_of_fresh_sequence_sees_one_row():
    # a sequence whose cache holds only the step's tokens: token 0 attends to
    # row 0 alone, so its output is that row and its lse is that score
    rng = np.random.default_rng(23)
    ql, qp, c, kr, scale = _causal_case(rng, 4, 4)
    o, lse = O.latent_attention_causal(ql, qp, c, kr, scale)
    for h in range(ql.shape[1]):
        assert rel_err(o[0, h], c[0]) < RTOL
        s0 = (ql[0, h] @ c[0] + qp[0, h] @ kr[0]) * scale
        assert abs(lse[0, h] - s0) < 1e-12 * max(1.0, abs(s0))


# ---------------------------------------------------------------------------
# A planted mistake must be caught (mutations applied to a copy of the oracle
# on the CPU; the pins above must reject each of them).
# ---------------------------------------------------------------------------
def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(18)
    k = rand_case(rng, n_h=4, d_c=32, d_r=8, d_h=16, d_v=16, T=40)
    ref = O.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"], k["k"], k["W_UK"], k["W_UV"], k["scale"])[0]

    def sdpa_ref():
        c = torch.from_numpy(k["c"])
        qr = torch.from_numpy(O.rope(k["q_R"], k["pos"]))
        Wk = torch.from_numpy(k["W_UK"])
        Wv = torch.from_numpy(k["W_UV"])
        K = torch.cat([torch.matmul(c, Wk.transpose(1, 2).contiguous()),
                       torch.from_numpy(k["k"]).unsqueeze(0).expand(4, -1, -1)], -1)
        V = torch.matmul(c, Wv.transpose(1, 2).contiguous())
        q = torch.cat([torch.from_numpy(k["q_C"]), qr], -1).unsqueeze(1)
        return torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=k["scale"])[:, 0].numpy()

    assert rel_err(ref, sdpa_ref()) < 1e-12
    orig_kv = O.mla_oracle.explicit_kv

    def dropped_rope_term(c, kr, Wk, Wv):
        keys, v = orig_kv(c, kr, Wk, Wv)
        keys[:, Wk.shape[0]:] = 0.0
        return keys, v

    monkeypatch.setattr(O.mla_oracle, "explicit_kv", dropped_rope_term)
    bad = O.mla_oracle.decode_explicit(k["q_C"], k["q_R"], k["pos"], k["c"], k["k"], k["W_UK"], k["W_UV"], k["scale"])[0]
    assert rel_err(bad, sdpa_ref()) > 1e-3
    monkeypatch.setattr(O.mla_oracle, "explicit_kv", orig_kv)
    # wrong RoPE sign
    bad_rope = lambda x, p, base=10000.0: O.mla_oracle.rope(x, -np.asarray(p), base)  # noqa: E731
    x = rng.standard_normal((3, 8))
    z = x[:, :4] + 1j * x[:, 4:]
    th = np.array([10000.0 ** (-(2.0 * i) / 8) for i in range(4)])
    zr = z * np.exp(1j * 9 * th)
    assert rel_err(bad_rope(x, 9), np.concatenate([zr.real, zr.imag], 1)) > 1e-3


# ---------------------------------------------------------------------------
# The paged pool reading: rows gathered through a block table.
# ---------------------------------------------------------------------------
def _scatter_by_hand(rows_per_seq, block_rows, rng):
    """An independent pure-Python scatter into a pool with shuffled blocks."""
    nblk = [(len(r) + block_rows - 1) // block_rows for r in rows_per_seq]
    ids = list(rng.permutation(sum(nblk) + 3))
    pool = [[float("nan")] * 3 for _ in range((sum(nblk) + 3) * block_rows)]
    tables = []
    for rows in rows_per_seq:
        tab = [int(ids.pop()) for _ in range((len(rows) + block_rows - 1) // block_rows)]
        for t, row in enumerate(rows):
            pool[tab[t // block_rows] * block_rows + t % block_rows] = list(row)
        tables.append(tab)
    return np.array(pool), tables


def test_paged_rows_round_trip_and_brute_force():
    rng = np.random.default_rng(30)
    for block_rows in (1, 4, 32):
        seqs = [rng.standard_normal((n, 3)) for n in (1, 5, block_rows, block_rows + 1, 3 * block_rows + 2)]
        pool, tables = _scatter_by_hand(seqs, block_rows, rng)
        for rows, tab in zip(seqs, tables):
            got = O.paged_rows(pool, tab, len(rows), block_rows)
            assert np.array_equal(got, rows)
            # a prefix is the prefix of the rows
            assert np.array_equal(O.paged_rows(pool, tab, 1, block_rows), rows[:1])
    # a mistaken reading (block-major within the table, t % n_blocks) does not round-trip
    seqs = [rng.standard_normal((9, 3))]
    pool, tables = _scatter_by_hand(seqs, 4, rng)
    tab = np.asarray(tables[0])
    t = np.arange(9)
    wrong = pool[tab[t % len(tab)] * 4 + t // len(tab)]
    assert not np.array_equal(wrong, seqs[0])
    with pytest.raises(IndexError):
        O.paged_rows(pool, [len(pool)], 1, 4)


def test_pool_bytes_per_token_matches_pages(golden_dir):
    # a pool shared by DeepSeek-V3's 61 layers: 61 x 576 bf16 per token, the
    # pages' ~68 KB (exactly 70,272 B); 32K tokens of one sequence ~ 2.1 GB
    g = _golden(golden_dir, "cache_sizes.json")
    e = {x["id"]: x for x in g["entries"]}
    per_tok = O.pool_bytes_per_token(61, 512, 64, 2)
    assert per_tok == e["v3_mla_per_token"]["exact_bytes"] == 70272
    assert abs(per_tok * 32768 / 2 ** 30 - 2.1) / 2.1 < 0.03


# ---------------------------------------------------------------------------
# The low-precision cache reading: E4M3 codes with one scale per row.
# ---------------------------------------------------------------------------
def _e4m3_by_hand(v):
    """Pure-Python nearest E4M3 code by search over every code of v's sign:
    clamp to [-448, 448], nearest value, ties to the even code (whose last
    bit, the mantissa's, is 0)."""
    if math.isnan(v):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0x00
    t = max(-448.0, min(448.0, v))
    best = None
    for m in range(0x7F):
        c = sign | m
        d = abs(O.e4m3_value(c) - t)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e4m3_format_points():
    # values fixed by the format's definition
    assert O.e4m3_value(0x7E) == 448.0 and math.isnan(O.e4m3_value(0x7F)) and math.isnan(O.e4m3_value(0xFF))
    assert O.e4m3_value(0x01) == 2.0 ** -9 and O.e4m3_value(0x08) == 2.0 ** -6 and O.e4m3_value(0x38) == 1.0
    assert O.e4m3_value(0x80) == 0.0 and O.e4m3_value(0xBE) == -1.75
    vals = [O.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))                     # increasing, no duplicates
    # every finite code round-trips
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes).astype(np.float32)), codes)


def test_e4m3_rounding_ties_and_saturation():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 17.0: 0x58, 19.0: 0x5A, 464.0: 0x7E, 500.0: 0x7E, 1e9: 0x7E,
             2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, -448.0: 0xFE, -1e9: 0xFE}
    for v, code in cases.items():
        assert int(O.e4m3_encode(np.float32(v))) == code, (v, hex(int(O.e4m3_encode(np.float32(v)))), hex(code))
    rng = np.random.default_rng(31)
    xs = np.concatenate([rng.standard_normal(300) * 50, rng.uniform(-470, 470, 300),
                         rng.standard_normal(100) * 2.0 ** -7]).astype(np.float32)
    got = O.e4m3_encode(xs)
    for x, c in zip(xs, got):
        assert int(c) == _e4m3_by_hand(float(x)), (float(x), hex(int(c)))


def test_quantize_rows_bounds_and_special_rows():
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((50, 576)) * rng.uniform(0.01, 100, (50, 1))).astype(np.float32)
    codes, scales = O.quantize_rows(x)
    deq = O.dequantize_rows(codes, scales)
    amax = np.max(np.abs(x), axis=1)
    # the scale is the smallest power of two that brings amax within 448
    e = np.log2(scales.astype(np.float64))
    assert np.all(e == np.round(e))
    assert np.all(amax <= 448 * scales) and np.all(amax > 224 * scales)
    # every element within half an E4M3 step (relative 2^-4 of its binade),
    # or half the subnormal step 2^-10 * scale
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None] * 2.0 ** -10) * (1 + 1e-12)
    assert np.all(err <= bound)
    # the dequantised values are exactly representable in bf16
    assert np.array_equal(I.bf16_to_f32(I.bf16_bits(deq.astype(np.float32))).astype(np.float64), deq)
    # an all-zero row: scale 1, zero codes; a row of powers of two: exact
    c0, s0 = O.quantize_rows(np.zeros((1, 8), np.float32))
    assert s0[0] == 1.0 and not c0.any()
    p2 = np.array([[-3.25, 1.0, 0.5, 448.0 * 4, -2.0 ** -3]], np.float32)
    c1, s1 = O.quantize_rows(p2)
    assert s1[0] == 4.0 and np.array_equal(O.dequantize_rows(c1, s1), p2.astype(np.float64))
    # the exponent rule at its boundaries: amax = 448 2^e -> e; just above -> e + 1
    assert O.row_scale_exponent(448.0) == 0 and O.row_scale_exponent(448.0 * 2 ** -5) == -5
    assert O.row_scale_exponent(np.nextafter(np.float32(448.0), np.float32(1e9))) == 1
    assert O.row_scale_exponent(224.0) == -1 and O.row_scale_exponent(225.0) == 0
    # a planted mistake: rounding toward zero instead of to nearest breaks the
    # half-step bound
    v = x / scales[:, None]
    mags = np.array([O.e4m3_value(c) for c in range(0x7F)])
    toward0 = np.sign(v) * mags[np.searchsorted(mags, np.abs(v), side="right") - 1]
    bad = np.abs(toward0 * scales[:, None] - x)
    assert np.any(bad > bound)


# ---------------------------------------------------------------------------
# The un-absorbed branch for many new tokens (prefill).
# ---------------------------------------------------------------------------
def _prefill_case(rng, T, n_q, n_h=3, d_c=12, d_r=6, d_h=5, d_v=7):
    return (rng.standard_normal((n_q, n_h, d_h)), rng.standard_normal((n_q, n_h, d_r)),
            rng.standard_normal((T, d_c)), rng.standard_normal((T, d_r)),
            rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c), rng.standard_normal((n_h, d_v, d_c)) / math.sqrt(d_c),
            1.0 / math.sqrt(d_h + d_r))


def test_prefill_token_equals_decode_over_prefix():
    # token i is a single-query explicit decode over rows 0 .. T - n_q + i at
    # its own position; an off-by-one mask is a different result
    rng = np.random.default_rng(40)
    for T, n_q in ((1, 1), (9, 9), (20, 6)):
        qc, qr, c, kr, Wk, Wv, sc = _prefill_case(rng, T, n_q)
        o, lse = O.prefill_explicit(qc, qr, c, kr, Wk, Wv, sc)
        for i in range(n_q):
            n = T - n_q + i + 1
            oi, _, li = O.decode_explicit(qc[i], qr[i], n - 1, c[:n], kr[:n], Wk, Wv, sc)
            assert rel_err(o[i], oi) < RTOL and rel_err(lse[i], li) < RTOL
        if n_q > 1 and T > n_q:
            n = T - n_q + 1
            wrong, _, _ = O.decode_explicit(qc[1], qr[1], n, c[:n], kr[:n], Wk, Wv, sc)
            assert rel_err(o[1], wrong) > 1e-3


def test_prefill_matches_torch_causal_sdpa_and_absorbed_route():
    rng = np.random.default_rng(41)
    T, n_q = 30, 30
    qc, qr, c, kr, Wk, Wv, sc = _prefill_case(rng, T, n_q)
    o, lse = O.prefill_explicit(qc, qr, c, kr, Wk, Wv, sc)
    # torch's attention with is_causal over explicit K, V (a fresh prompt: n_q = T)
    qrot = O.rope(qr, np.arange(T)[:, None])
    q = torch.from_numpy(np.concatenate([qc, qrot], 2)).transpose(0, 1).contiguous()          # [n_h, T, D]
    K = torch.from_numpy(np.concatenate([np.einsum("tc,hkc->htk", c, Wk),
                                         np.broadcast_to(kr, (3, T, kr.shape[1]))], 2)).contiguous()
    V = torch.from_numpy(np.einsum("tc,hvc->htv", c, Wv)).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, is_causal=True, scale=sc)
    assert rel_err(o, ref.transpose(0, 1).numpy()) < 1e-12
    # the absorbed route: latent causal attention, then W_UV per head
    q_lat = np.einsum("thk,hkc->thc", qc, Wk)
    z, lse2 = O.latent_attention_causal(q_lat, qrot, c, kr, sc)
    assert rel_err(np.einsum("hvc,thc->thv", Wv, z), o) < 1e-12
    assert rel_err(lse2, lse) < 1e-12
