"""The un-absorbed prefill branch (explicit K/V up-projection, causal flash
attention) against the oracle's explicit route, and against the absorbed
route of the same step (mla_absorb_q + mla_decode_attn_causal + W^UV)."""

import numpy as np
import pytest
import torch

import oracle as O
from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I

from gpu_support import compare, dev, host_f64, say

pytestmark = pytest.mark.gpu

V3 = L.Dims.make(128, 512, 64, 128, 128, d_model=7168, d_q=1536, dtype="bf16")
SCALE = O.scale_for(128, 64)


def _case(lens, n_q, seed, caps=None):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    caps = lens.astype(np.int64) if caps is None else np.asarray(caps, np.int64)
    offsets = np.concatenate([[0], np.cumsum(caps)]).astype(np.int32)
    rows = int(offsets[-1])
    cache = I.bf16_bits(rng.standard_normal((rows, 576), dtype=np.float32))
    B = len(lens)
    q = I.bf16_bits(rng.standard_normal((B, n_q, 128, 192), dtype=np.float32))
    W_UK = I.bf16_bits(rng.standard_normal((128, 128, 512), dtype=np.float32) * np.float32(512 ** -0.5))
    W_UV = I.bf16_bits(rng.standard_normal((128, 128, 512), dtype=np.float32) * np.float32(512 ** -0.5))
    return dict(lens=lens, offsets=offsets, cache=cache, q=q, W_UK=W_UK, W_UV=W_UV, n_q=n_q, B=B)


def _run(c):
    B, n_q = c["B"], c["n_q"]
    o = torch.full((B, n_q, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, n_q, 128), float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.prefill_attn(V3, dev(c["q"]), dev(c["cache"]), dev(c["offsets"]), dev(c["lens"]), dev(c["W_UK"]),
                   dev(c["W_UV"]), o, lse, err_flag=err)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse), int(err.item())


def _oracle(c, b, toks, heads):
    f = lambda a: I.bf16_to_f32(a).astype(np.float64)
    o0 = int(c["offsets"][b])
    rows = f(c["cache"][o0:o0 + int(c["lens"][b])])
    q = f(c["q"][b])
    o, lse = O.prefill_explicit(q[:, heads, :128], q[:, heads, 128:], rows[:, :512], rows[:, 512:],
                                f(c["W_UK"])[heads], f(c["W_UV"])[heads], SCALE)
    return o[toks], lse[toks]


@pytest.mark.parametrize("lens,n_q", [([300, 77], 77), ([1, 40, 129], 1), ([200, 200, 513], 200)])
def test_prefill_small(lens, n_q):
    c = _case(lens, n_q, seed=sum(lens) + n_q)
    say(f"prefill: lens={lens} n_q={n_q}")
    o, lse, err = _run(c)
    assert err == 0
    heads = list(range(0, 128, 3))
    for b in range(c["B"]):
        toks = sorted({0, n_q // 2, n_q - 1})
        ro, rl = _oracle(c, b, toks, heads)
        compare(o[b][toks][:, heads], ro, f"b={b} toks={toks} o")
        compare(lse[b][toks][:, heads], rl, f"b={b} lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2,
                norm_mean=1e-3)


def test_prefill_matches_absorbed_route():
    """The same step by the absorbed route: q_lat = W_UK^T q^C, q_pe rotated,
    latent causal attention, then W_UV -- the two branches agree."""
    lens, n_q = [150, 64], 64
    c = _case(lens, n_q, seed=9)
    o, lse, err = _run(c)
    assert err == 0
    B = c["B"]
    q = dev(c["q"]).view(B * n_q, 128, 192)
    pos = torch.tensor([int(c["lens"][b]) - n_q + i for b in range(B) for i in range(n_q)], dtype=torch.int32,
                       device="cuda")
    q_lat = torch.empty(B * n_q, 128, 512, dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(B * n_q, 128, 64, dtype=torch.bfloat16, device="cuda")
    L.absorb_q(V3, q_lat, q_pe, dev(c["W_UK"]), pos, q=q)
    o_lat = torch.empty(B * n_q, 128, 512, dtype=torch.float32, device="cuda")
    lse2 = torch.empty(B * n_q, 128, dtype=torch.float32, device="cuda")
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.decode_attn_causal(V3, n_q, q_lat, q_pe, dev(c["cache"]), dev(c["offsets"]), dev(c["lens"]), o_lat, lse2,
                         err_flag=err2)
    o2 = torch.empty(B * n_q, 128, 128, dtype=torch.float32, device="cuda")
    L.project_out(V3, o_lat, dev(c["W_UV"]), o=o2)
    torch.cuda.synchronize()
    assert int(err2.item()) == 0
    compare(o.reshape(B * n_q, 128, 128), host_f64(o2), "explicit vs absorbed o", max_abs=1e-2, mean_abs=1e-3)
    compare(lse.reshape(B * n_q, 128), host_f64(lse2), "explicit vs absorbed lse", max_abs=1e-2, mean_abs=1e-3,
            norm_max=1e-2, norm_mean=1e-3)


def test_prefill_long_prompt():
    """A fresh 4096-token prompt and a 2048-token continuation of a
    1024-token prefix: sampled tokens (first, last, block edges) and heads."""
    c = _case([4096, 3072], 2048, seed=4096)
    say("prefill: lens=[4096, 3072] n_q=2048")
    o, lse, err = _run(c)
    assert err == 0
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    heads = [0, 37, 64, 127]
    for b in range(2):
        toks = [0, 127, 128, 1000, 2047]
        ro, rl = _oracle(c, b, toks, heads)
        compare(o[b][toks][:, heads], ro, f"long b={b} o")
        compare(lse[b][toks][:, heads], rl, f"long b={b} lse", max_abs=1e-2, mean_abs=1e-3, norm_max=1e-2,
                norm_mean=1e-3)


def test_prefill_benchmark_configuration():
    """The configuration the benchmark times: four fresh 4096-token prompts,
    every token new (n_q = T = 4096).  Sampled tokens (first, tile and block
    edges, last) and heads of the first and last prompt against the
    explicit route."""
    c = _case([4096] * 4, 4096, seed=44)
    say("prefill: B=4 fresh prompts of 4096 tokens (n_q=4096)")
    o, lse, err = _run(c)
    assert err == 0
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    heads = [5, 100]
    toks = [0, 1, 31, 32, 255, 256, 2047, 4095]
    for b in (0, 3):
        ro, rl = _oracle(c, b, toks, heads)
        compare(o[b][toks][:, heads], ro, f"bench config b={b} o")
        compare(lse[b][toks][:, heads], rl, f"bench config b={b} lse", max_abs=1e-2, mean_abs=1e-3,
                norm_max=1e-2, norm_mean=1e-3)


def test_prefill_invalid_lengths():
    c = _case([100, 50], 60, seed=3, caps=[100, 80])   # sequence 1 has fewer rows than tokens
    o, lse, err = _run(c)
    assert err & L.DEVERR_LENS
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(lse[1]))
    assert np.all(np.isfinite(o[0]))
    ro, rl = _oracle(c, 0, [0, 59], [5, 99])
    compare(o[0][[0, 59]][:, [5, 99]], ro, "valid sequence o")
