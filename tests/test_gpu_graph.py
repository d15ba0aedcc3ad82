"""The decode step captured in a HIP graph (as the benchmark runs it) gives,
replay after replay, bit-for-bit the results of the same calls launched
eagerly: every kernel of the path is deterministic and none of them records a
memset node.  Eager work and synchronisations run between the replays."""

import numpy as np
import pytest
import torch

from head_latent_attention_16_amd import _lib as L
from head_latent_attention_16_amd import inputs as I

from gpu_support import Uploaded, dev, dims_of, say

pytestmark = pytest.mark.gpu


def _attention_step(u, d, out):
    L.absorb_q(d, out["q_lat"], out["q_pe"], u.W["W_UK"], u.lens, q=u.q)
    L.decode_attn(d, out["q_lat"], out["q_pe"], u.cache, u.offsets, u.lens, out["o_lat"],
                  out["lse"], total_rows_hint=int(u.w.total_rows), ws=out["ws"])
    L.project_out(d, out["o_lat"], u.W["W_UV"], o=out["o"])


def _buffers(w, d, hint):
    B, n_h = w.B, d.n_h
    return dict(q_lat=torch.empty(B, n_h, d.d_c, dtype=torch.bfloat16, device="cuda"),
                q_pe=torch.empty(B, n_h, d.d_r, dtype=torch.bfloat16, device="cuda"),
                o_lat=torch.empty(B, n_h, d.d_c, dtype=torch.float32, device="cuda"),
                lse=torch.empty(B, n_h, dtype=torch.float32, device="cuda"),
                o=torch.empty(B, n_h, d.d_v, dtype=torch.float32, device="cuda"),
                ws=torch.empty(L.decode_attn_workspace(d, B, hint), dtype=torch.uint8,
                               device="cuda"))


def test_attention_step_graph_replays_match_eager():
    rng = np.random.default_rng(5)
    w = I.attention_only("graph", 3, np.array([300, 77, 1000], np.int32), rng, 5)
    other = I.attention_only("graph2", 2, np.array([64, 513], np.int32), rng, 6)
    u, uo = Uploaded(w), Uploaded(other)
    d = dims_of(w)
    say("graph: attention step B=3 lens [300, 77, 1000], 4 replays")
    ref = _buffers(w, d, w.total_rows)
    _attention_step(u, d, ref)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items() if k != "ws"}

    out = _buffers(w, d, w.total_rows)
    side = _buffers(other, d, other.total_rows)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        _attention_step(u, d, out)
    for rep in range(4):
        for v in (out["q_lat"], out["q_pe"], out["o_lat"], out["lse"], out["o"]):
            v.fill_(float("nan"))
        _attention_step(uo, d, side)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("q_lat", "q_pe", "o_lat", "lse", "o"):
            assert torch.equal(out[k], ref[k]), (rep, k)


@pytest.mark.parametrize("two_streams,B,lo,hi", [(False, 4, 20, 200), (True, 4, 20, 200),
                                                 (True, 128, 512, 8192)])
def test_layer_step_graph_replays_match_eager(two_streams, B, lo, hi):
    """Full layer step (query path, append, attention, projections): the graph
    and an eager twin advance identical state copies; after every replay the
    outputs, the appended rows and the lengths agree bit for bit.  With
    two_streams the graph runs the append on a second stream beside the
    query path while the eager twin runs everything on one stream; the
    last case is the full-size layer workload (B = 128, T_prior in [512,
    8192]), as the benchmark runs it."""
    w = I.layer(seed=7, B=B, lo=lo, hi=hi, spare=8)
    d = dims_of(w)
    dd = w.dims
    B, n_h = w.B, dd["n_h"]
    say(f"graph: layer step B={B} T_prior in [{lo}, {hi}], 3 replays, two streams {two_streams}")

    def state():
        return dict(cache=dev(w.cache), offsets=dev(w.offsets), lens=dev(w.lens),
                    pos=dev(w.lens), h_t=dev(w.h_t), **{k: dev(v) for k, v in w.W.items()})

    def bufs():
        hint = int(w.total_rows) + 8 * B
        b = _buffers(w, d, hint)
        b["u"] = torch.empty(B, dd["d_model"], dtype=torch.float32, device="cuda")
        import ctypes
        lib = L.lib()
        b["ws_abs"] = torch.empty(max(1, lib.mla_absorb_q_workspace(ctypes.byref(d), B, 1)),
                                  dtype=torch.uint8, device="cuda")
        b["ws_app"] = torch.empty(max(1, lib.mla_append_cache_workspace(ctypes.byref(d), B, 1, 1)),
                                  dtype=torch.uint8, device="cuda")
        b["ws_prj"] = torch.empty(max(1, lib.mla_project_out_workspace(ctypes.byref(d), B, 1)),
                                  dtype=torch.uint8, device="cuda")
        b["hint"] = hint
        return b

    def append(s, b):
        L.append_cache(d, s["cache"], s["offsets"], s["lens"], 1, h_t=s["h_t"], W_DKV=s["W_DKV"],
                       W_KR=s["W_KR"], ws=b["ws_app"])

    def step(s, b, side=None):
        s["pos"].copy_(s["lens"])
        if side is not None:
            # the append on a second stream, forked after the positions are
            # copied and joined before the attention call (as the benchmark runs it)
            main = torch.cuda.current_stream()
            forked = torch.cuda.Event()
            forked.record(main)
            side.wait_event(forked)
            with torch.cuda.stream(side):
                append(s, b)
            appended = torch.cuda.Event()
            appended.record(side)
        L.absorb_q(d, b["q_lat"], b["q_pe"], s["W_UK"], s["pos"], h_t=s["h_t"], W_DQ=s["W_DQ"],
                   W_UQ=s["W_UQ"], ws=b["ws_abs"])
        if side is not None:
            main.wait_event(appended)
        else:
            append(s, b)
        L.decode_attn(d, b["q_lat"], b["q_pe"], s["cache"], s["offsets"], s["lens"], b["o_lat"],
                      b["lse"], total_rows_hint=b["hint"], ws=b["ws"])
        L.project_out(d, b["o_lat"], s["W_UV"], o=b["o"], u=b["u"], W_O=s["W_O"], ws=b["ws_prj"])

    se, be = state(), bufs()     # eager twin, one stream
    sg, bg = state(), bufs()     # graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step(sg, bg, side=torch.cuda.Stream() if two_streams else None)
    for rep in range(3):
        step(se, be)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sg["lens"], se["lens"]), rep
        assert torch.equal(sg["cache"], se["cache"]), rep
        for k in ("q_lat", "q_pe", "o_lat", "lse", "o", "u"):
            assert torch.equal(bg[k], be[k]), (rep, k)
    assert np.array_equal(se["lens"].cpu().numpy(), w.lens + 3)
