"""mla_decode_attn_noalloc (the library's fixed scratch, no allocation)
against mla_decode_attn with a caller workspace, on two calls in a row, the
second with a smaller batch; plus its size limit."""

import numpy as np
import pytest
import torch

from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I

from gpu_support import Uploaded, compare, host_f64, oracle_seq, say

pytestmark = pytest.mark.gpu


def _queries(u):
    w, d = u.w, u.dims
    q_lat = torch.empty(w.B, d.n_h, d.d_c, dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(w.B, d.n_h, d.d_r, dtype=torch.bfloat16, device="cuda")
    L.absorb_q(d, q_lat, q_pe, u.W["W_UK"], u.lens.clone(), q=u.q)
    return q_lat, q_pe


def _both(u, hint):
    w, d = u.w, u.dims
    q_lat, q_pe = _queries(u)
    out = {}
    for name in ("ws", "noalloc"):
        o_lat = torch.full((w.B, d.n_h, d.d_c), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((w.B, d.n_h), float("nan"), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if name == "ws":
            L.decode_attn(d, q_lat, q_pe, u.cache, u.offsets, u.lens, o_lat, lse, total_rows_hint=hint,
                          err_flag=err)
        else:
            L.decode_attn_noalloc(d, q_lat, q_pe, u.cache, u.offsets, u.lens, o_lat, lse,
                                  total_rows_hint=hint, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        out[name] = (o_lat, lse)
    return out


@pytest.mark.parametrize("second", [[40, 1, 700], [3]])
def test_noalloc_matches_workspace_entry(second):
    # first call: 9 sequences over many split pieces; second: a smaller batch
    for lens in ([4100, 37, 1, 800, 2000, 257, 5000, 64, 3333], second):
        rng = np.random.default_rng(len(lens))
        w = I.attention_only("noalloc", len(lens), np.asarray(lens, np.int32), rng, 0)
        say(f"noalloc: lens={lens}")
        u = Uploaded(w)
        r = _both(u, w.total_rows)
        (a, la), (b, lb) = r["ws"], r["noalloc"]
        # same kernels, same split: identical bits
        assert torch.equal(a, b) and torch.equal(la, lb)
        for bb in (0, w.B - 1):
            _, ro_lat, rlse = oracle_seq(w, bb, heads=[0, 45, 127])
            compare(host_f64(b[bb])[[0, 45, 127]], ro_lat, f"noalloc b={bb} o_lat")
            compare(host_f64(lb[bb])[[0, 45, 127]], rlse, f"noalloc b={bb} lse", max_abs=2e-2, mean_abs=2e-3,
                    norm_max=1e-2, norm_mean=2e-3)


def test_noalloc_rejects_batches_beyond_its_scratch():
    d = L.Dims.make(128, 512, 64, 128, 128, dtype="bf16")
    B = 400
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    q = torch.zeros(B, 128, 512, dtype=torch.bfloat16, device="cuda")
    qp = torch.zeros(B, 128, 64, dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros(B, 576, dtype=torch.bfloat16, device="cuda")
    offs = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    o = torch.zeros(B, 128, 512, dtype=torch.float32, device="cuda")
    with pytest.raises(L.MLAError) as e:
        L.decode_attn_noalloc(d, q, qp, cache, offs, lens, o, total_rows_hint=1 << 20, err_flag=t)
    assert e.value.status == 4
    # the same batch with the workspace entry point works
    L.decode_attn(d, q, qp, cache, offs, lens, o, total_rows_hint=1 << 20, err_flag=t)
    torch.cuda.synchronize()
    assert int(t.item()) == 0 and torch.isfinite(o).all()
