"""Benchmark one MLA decode step on one MI355X through the C ABI.

    python bench.py [--steps K] [--warmup W] [--workload ragged|uniform|long|layer|causal]

The default workload is the ragged batch (B=64, T uniform in [1024, 32768]),
the largest attention-only workload that fits one GPU.

A step is one pass of the decode hot path over one batch:
  attention-only workloads (uniform, ragged, long):
      mla_absorb_q (q given) -> mla_decode_attn -> mla_project_out (o)
  layer workload: mla_absorb_q (from h_t) and mla_append_cache (from h_t),
      the append on a second stream beside the query path (--one-stream:
      one after the other), -> mla_decode_attn -> mla_project_out (o and u);
      with --norms the _normed variants of the first two (latent norms on
      c^Q and c^KV)
  causal workload (--n-q new tokens per sequence, the cache's last rows):
      mla_absorb_q (B n_q queries) -> mla_decode_attn_causal -> mla_project_out (o)
Warmup steps replay the same step graphs back to back right before the
timed steps, so the timed steps run at the sustained shader clock.
Inputs are seeded synthetic tensors of the DeepSeek-V3 shapes, resident in
HBM before timing; several independent copies of all inputs are rotated so
that consecutive steps do not hit in the 256 MB Infinity Cache.

Prints ONE JSON line on stdout (progress goes to stderr).  ``value`` is
cache-tokens/s of the whole step; ``roofline`` is for the mla_decode_attn call
(its kernels: split attention with the length scan, combine), timed with HIP
events on the launch stream inside the timed loop.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode cache-tokens/s & HBM GB/s (% roofline), V3 dims, B×T at 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # 200 warmup steps (tens of ms of back-to-back work) bring the shader
    # clock to its sustained level before the timed steps; after 10 the
    # clock is still rising and a step measures ~20% slower
    p.add_argument("--warmup", type=int, default=200)
    # default: the largest single-GPU attention workload (ragged, 1.29 GB of cache per step)
    p.add_argument("--workload", default="ragged",
                   choices=["uniform", "ragged", "long", "layer", "causal", "paged", "fp8", "prefill"])
    p.add_argument("--prefill-len", type=int, default=4096, help="prefill workload: prompt tokens per sequence")
    p.add_argument("--prefill-batch", type=int, default=4, help="prefill workload: sequences")
    p.add_argument("--block-rows", type=int, default=64, help="paged workload: rows per pool block")
    p.add_argument("--n-q", type=int, default=4, help="causal workload: new tokens per sequence")
    p.add_argument("--norms", action="store_true",
                   help="layer workload: root-mean-square latent norms on c^Q and c^KV")
    p.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = auto)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="launch each kernel from the host")
    p.add_argument("--one-stream", action="store_true",
                   help="layer workload: run the append on the same stream as the query path")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="first run one plain device-to-device copy of MIB MiB (a reference "
                        "for the HBM byte counters of a profiler run)")
    return p.parse_args()


def algorithmic(w, row_bytes=None):
    """Bytes and FLOPs of one attention call: the cache read once, q in, o_lat
    out; with n_q tokens per sequence token i scores T - n_q + i + 1 rows.
    row_bytes: bytes of one cached row (default bf16: 2 (d_c + d_r))."""
    n_h, d_c, d_r, n_q = w.dims["n_h"], w.dims["d_c"], w.dims["d_r"], w.n_q
    tokens = int(w.total_rows)
    nq_tok = w.B * n_q
    rb = row_bytes if row_bytes is not None else (d_c + d_r) * 2
    byts = tokens * rb + nq_tok * n_h * (d_c + d_r) * 2 + nq_tok * n_h * d_c * 4
    scored = n_q * tokens - w.B * (n_q * (n_q - 1) // 2)     # rows seen, summed over tokens
    flops = scored * 2 * n_h * ((d_c + d_r) + d_c)
    return tokens, byts, flops


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "head_latent_attention_16_amd", "csrc", "decode_v3.hip")


def measured_traffic(workload):
    """HBM bytes per mla_decode_attn call from the recorded counter runs, or None.

    The record holds FETCH_SIZE + WRITE_SIZE of the call's kernels, scaled by a
    plain copy of known size, and the SHA-256 of the kernel source it was taken
    with: a changed kernel makes the figure stale, so it is not reported."""
    import hashlib
    try:
        rec = None
        for line in open(TRAFFIC_FILE):
            line = line.strip()
            if line.startswith("{") and '"workload"' in line:
                r = json.loads(line)
                if r.get("workload") == workload:
                    rec = r
        if rec is None:
            return None
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        return rec["bytes_per_call"] if rec.get("kernel_sha256") == src else None
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(w, budget_s):
    """Time the fp64 oracle (explicit route) on whole sequences until the budget is used."""
    import oracle as O
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')} ({info[0].get('architecture')})"
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    d = w.dims
    scale = O.scale_for(d["d_h"], d["d_r"])
    W_UK, W_UV = w.f64(w.W["W_UK"]), w.f64(w.W["W_UV"])
    done_tokens, heads_done, t0 = 0, 0, time.perf_counter()
    b = 0
    while time.perf_counter() - t0 < budget_s and b < w.B:
        rows = w.f64(w.seq_rows(b))
        c, kr = rows[:, :d["d_c"]], rows[:, d["d_c"]:]
        if w.q_C is not None:
            q_C, q_R, pos = w.f64(w.q_C[b]), w.f64(w.q_R[b]), int(w.lens[b])
        else:
            q_C, q_R = O.query_path(w.f64(w.h_t[b:b + 1]), w.f64(w.W["W_DQ"]), w.f64(w.W["W_UQ"]),
                                    d["n_h"], d["d_h"], d["d_r"])
            q_C, q_R, pos = q_C[0], q_R[0], int(w.lens[b])
        # all heads of this sequence, one head at a time, stop at the budget
        for h in range(d["n_h"]):
            O.decode_explicit(q_C[h:h + 1], q_R[h:h + 1], pos, c, kr, W_UK[h:h + 1], W_UV[h:h + 1], scale)
            heads_done += 1
            done_tokens += len(rows)
            if time.perf_counter() - t0 >= budget_s:
                break
        b += 1
    dt = time.perf_counter() - t0
    per_token_heads = done_tokens / d["n_h"]        # cache-tokens with all heads processed
    rate = per_token_heads / dt
    return {"value": rate, "unit": "cache-tokens/s", "cores": int(threads),
            "extrapolated_full_workload_s": float(w.total_rows) / rate if rate > 0 else None,
            "kind": "oracle", "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "blas": blas,
            "sample": f"fp64 explicit route, {heads_done} (sequence, head) pairs over "
                      f"{b} sequence(s) of the same workload in {dt:.1f} s; value = "
                      f"head-weighted cache tokens / s"}


def bench_prefill(args):
    """Un-absorbed prefill of B fresh prompts of T tokens (every token is new:
    n_q = T), mla_prefill_attn timed: explicit K/V up-projection of the B T
    cache rows, then causal attention.  Compute-bound: reported against the
    dense fp16/bf16 MFMA peak."""
    import torch

    from head_latent_attention_16_amd import _lib as L
    from head_latent_attention_16_amd import inputs as I

    torch.cuda.set_device(0)
    B, T = args.prefill_batch, args.prefill_len
    rng = np.random.default_rng(0)
    log(f"generating prefill B={B} T={T} ...")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    lens = np.full(B, T, np.int32)
    offsets = (np.arange(B + 1) * T).astype(np.int32)
    cache = dev(I.bf16_bits(rng.standard_normal((B * T, 576), dtype=np.float32)))
    q = dev(I.bf16_bits(rng.standard_normal((B, T, 128, 192), dtype=np.float32)))
    W_UK = dev(I.bf16_bits(rng.standard_normal((128, 128, 512), dtype=np.float32) * np.float32(512 ** -0.5)))
    W_UV = dev(I.bf16_bits(rng.standard_normal((128, 128, 512), dtype=np.float32) * np.float32(512 ** -0.5)))
    dims = L.Dims.make(128, 512, 64, 128, 128, dtype="bf16")
    o = torch.empty(B, T, 128, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, T, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(L.prefill_attn_workspace(dims, B, T, B * T), dtype=torch.uint8, device="cuda")
    lens_d, offs_d = torch.from_numpy(lens).cuda(), torch.from_numpy(offsets).cuda()

    def step():
        L.prefill_attn(dims, q, cache, offs_d, lens_d, W_UK, W_UV, o, lse, ws=ws)

    # a step is milliseconds long: 20 of them already reach the sustained clock
    warm = min(args.warmup, 20)
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for a, b in ev:
        a.record()
        step()
        b.record()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    pairs = B * T * (T + 1) // 2
    flops_attn = pairs * 128 * 2 * (192 + 128)
    flops_up = 2 * B * T * 512 * (128 * 256)
    flops = flops_attn + flops_up
    tf = flops / (call_ms * 1e-3) / 1e12
    log(f"prefill {call_ms * 1e3:.0f} us per call, {tf:.0f} TFLOP/s")
    out = {
        "metric": METRIC, "value": B * T / (ms * 1e-3), "unit": "new-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"un-absorbed prefill, B={B} fresh prompts of T={T} tokens (DeepSeek-V3 dims "
                               f"n_h=128 d_c=512 d_R=64 d_h=d_v=128), explicit K/V in fp16",
                   "B": B, "new_tokens": B * T, "step": "prefill_attn (up-projection + causal attention)"},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "mla_prefill_attn (k_rope_table, k_kr_f16, k_upproj, k_prefill)",
                     "call_us": call_ms * 1e3, "flops": flops, "flops_upproj": flops_up, "flops_attention": flops_attn},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    from head_latent_attention_16_amd import _lib as L
    from head_latent_attention_16_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "prefill":
        return bench_prefill(args)
    torch.cuda.set_device(0)
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read and written")
        del src, dst
    name = args.workload
    spare = args.warmup + args.steps + 2
    log(f"generating workload {name} ...")
    t0 = time.perf_counter()
    w = (I.layer(spare=spare) if name == "layer"
         else I.causal(n_q=args.n_q) if name == "causal"
         else I.make("ragged") if name in ("paged", "fp8") else I.make(name))
    paged = name == "paged"
    fp8 = name == "fp8"
    n_q = w.n_q
    log(f"  done in {time.perf_counter() - t0:.1f}s: B={w.B} total_rows={w.total_rows}")
    d = w.dims
    layer = name == "layer"
    dims = L.Dims.make(d["n_h"], d["d_c"], d["d_r"], d["d_h"], d["d_v"], d_model=d["d_model"],
                       d_q=d["d_q"], dtype="bf16")

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    if fp8:
        # the ragged batch's rows as E4M3 codes with one fp32 scale per row
        # (quantised on the host here; mla_append_cache_fp8 writes the same
        # codes on the device)
        import oracle as O
        codes, scales = O.quantize_rows(I.bf16_to_f32(w.cache))
        base = {"cache": dev(codes), "scales": dev(scales), "offsets": dev(w.offsets), "lens": dev(w.lens)}
        del codes, scales
    elif paged:
        # the ragged batch's rows in a pool of block_rows-row blocks with shuffled ids
        pp = I.paged_pool([w.cache], w.lens, w.lens, args.block_rows, seed=1)
        base = {"cache": dev(pp.pool), "table": dev(pp.tables[0]), "offsets": dev(w.offsets),
                "lens": dev(w.lens)}
        del pp
    else:
        base = {"cache": dev(w.cache), "offsets": dev(w.offsets), "lens": dev(w.lens)}
    for k, v in w.W.items():
        base[k] = dev(v)
    if layer:
        base["h_t"] = dev(w.h_t)
        base["pos"] = dev(w.lens)   # the query position of each step (lens before its append)
    else:
        base["q"] = dev(np.ascontiguousarray(np.concatenate([w.q_C, w.q_R], -1)))
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    copies = args.copies or max(2, math.ceil(2.5 * MALL_BYTES / per_copy))
    log(f"  {per_copy / 1e6:.1f} MB of inputs per copy, rotating {copies} copies")
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]

    B, n_h = w.B, d["n_h"]
    BQ = B * n_q   # query tokens
    hint = int(w.total_rows) + (B if layer else 0)
    q_lat = torch.empty(BQ, n_h, d["d_c"], dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty(BQ, n_h, d["d_r"], dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty(BQ, n_h, d["d_c"], dtype=torch.float32, device="cuda")
    lse = torch.empty(BQ, n_h, dtype=torch.float32, device="cuda")
    o = torch.empty(BQ, n_h, d["d_v"], dtype=torch.float32, device="cuda")
    # causal: token i of sequence b sits at position lens[b] - n_q + i
    tok_pos = torch.from_numpy((np.repeat(w.lens.astype(np.int64), n_q) - n_q
                                + np.tile(np.arange(n_q), B)).astype(np.int32)).cuda()
    u = torch.empty(B, d["d_model"], dtype=torch.float32, device="cuda") if layer else None
    ws_dec = torch.empty(L.decode_attn_causal_workspace(dims, B, n_q, hint), dtype=torch.uint8, device="cuda")

    def attend(s):
        if fp8:
            L.decode_attn_fp8(dims, q_lat, q_pe, s["cache"], s["scales"], s["offsets"], s["lens"], o_lat, lse,
                              total_rows_hint=hint, ws=ws_dec)
        elif paged:
            L.decode_attn_paged(dims, q_lat, q_pe, s["cache"], args.block_rows, s["table"], s["lens"], o_lat, lse,
                                total_rows_hint=hint, ws=ws_dec)
        elif n_q > 1:
            L.decode_attn_causal(dims, n_q, q_lat, q_pe, s["cache"], s["offsets"], s["lens"], o_lat, lse,
                                 total_rows_hint=hint, ws=ws_dec)
        else:
            L.decode_attn(dims, q_lat, q_pe, s["cache"], s["offsets"], s["lens"], o_lat, lse,
                          total_rows_hint=hint, ws=ws_dec)
    lib = L.lib()
    import ctypes
    ws_abs = torch.empty(max(1, lib.mla_absorb_q_workspace(ctypes.byref(dims), B, int(layer))),
                         dtype=torch.uint8, device="cuda")
    ws_app = torch.empty(max(1, lib.mla_append_cache_workspace(ctypes.byref(dims), B, 1, 1)),
                         dtype=torch.uint8, device="cuda")
    ws_prj = torch.empty(max(1, lib.mla_project_out_workspace(ctypes.byref(dims), B, int(layer))),
                         dtype=torch.uint8, device="cuda")

    # Layer step: the latent append (W^DKV|W^KR, the row write and the length
    # increment) does not depend on the query path (W^DQ, W^UQ, absorption),
    # so it runs on a second stream, forked after the query positions are
    # copied from the lengths and joined before the attention call.
    side = torch.cuda.Stream() if layer and not args.one_stream else None

    def append(s):
        if args.norms:
            L.append_cache_normed(dims, s["cache"], s["offsets"], s["lens"], 1, s["h_t"], s["W_DKV"],
                                  s["kv_norm_w"], s["W_KR"], ws=ws_app)
        else:
            L.append_cache(dims, s["cache"], s["offsets"], s["lens"], 1, h_t=s["h_t"],
                           W_DKV=s["W_DKV"], W_KR=s["W_KR"], ws=ws_app)

    def step(c):
        """One pass of the hot path over input copy c (launches only)."""
        s = sets[c]
        if layer:
            # query position = the length before this step's append
            s["pos"].copy_(s["lens"])
            if side is not None:
                main = torch.cuda.current_stream()
                forked = torch.cuda.Event()
                forked.record(main)
                side.wait_event(forked)
                with torch.cuda.stream(side):
                    append(s)
                appended = torch.cuda.Event()
                appended.record(side)
            if args.norms:
                L.absorb_q_normed(dims, q_lat, q_pe, s["W_UK"], s["pos"], s["h_t"], s["W_DQ"], s["q_norm_w"],
                                  s["W_UQ"], ws=ws_abs)
            else:
                L.absorb_q(dims, q_lat, q_pe, s["W_UK"], s["pos"], h_t=s["h_t"], W_DQ=s["W_DQ"],
                           W_UQ=s["W_UQ"], ws=ws_abs)
            if side is not None:
                main.wait_event(appended)
            else:
                append(s)
        else:
            L.absorb_q(dims, q_lat, q_pe, s["W_UK"], tok_pos if n_q > 1 else s["lens"], q=s["q"])
        attend(s)
        if layer:
            L.project_out(dims, o_lat, s["W_UV"], o=o, u=u, W_O=s["W_O"], ws=ws_prj)
        else:
            L.project_out(dims, o_lat, s["W_UV"], o=o)

    # The step's kernels are captured once per input copy into a HIP graph and
    # replayed, so the timed region holds device work only (no per-launch
    # host overhead between the ~6 kernels of a step).  Warmup step j runs on
    # copy j % copies: the first one eagerly (before any capture), the rest
    # as graph replays, so each graph's one-time upload to the device happens
    # in the warmup and not in the timed steps.
    n_eager = args.warmup if args.no_graph else min(args.warmup, 1)
    log(f"warmup {args.warmup} steps ({n_eager} eager) ...")
    for i in range(n_eager):
        step(i % copies)
    torch.cuda.synchronize()
    graphs = None
    if not args.no_graph:
        log(f"capturing {copies} step graphs ...")
        graphs = []
        cap = torch.cuda.Stream()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(c)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(n_eager, args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
    log(f"timing {args.steps} steps ...")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        if graphs is not None:
            graphs[(args.warmup + i) % copies].replay()
        else:
            step((args.warmup + i) % copies)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    # Roofline: mla_decode_attn alone (its split and combine kernels),
    # HIP events on the launch stream around each call, same input rotation.
    ev = []
    for i in range(args.steps):
        s = sets[(args.warmup + i) % copies]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        attend(s)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    # 8-bit rows: d_c + d_r codes and a 4-byte scale
    tokens, byts, flops = algorithmic(w, row_bytes=(d["d_c"] + d["d_r"] + 4) if fp8 else None)
    if layer:
        # Every step appends one row per sequence to the copy it uses: step j
        # (j = warmup + i) on copy j % copies attends over the prior rows plus
        # the floor(j / copies) + 1 rows appended to that copy so far.  The
        # decode-only timing pass afterwards sees each copy at its final size.
        per_copy_steps = [sum(1 for j in range(args.warmup + args.steps) if j % copies == c)
                          for c in range(copies)]
        grown = [B * (j // copies + 1) for j in range(args.warmup, args.warmup + args.steps)]
        tokens += sum(grown) / len(grown)
        dec_rows = [B * per_copy_steps[(args.warmup + i) % copies] for i in range(args.steps)]
        extra = sum(dec_rows) / len(dec_rows)
        n_h, d_c, d_r = d["n_h"], d["d_c"], d["d_r"]
        byts += extra * (d_c + d_r) * 2
        flops += extra * 2 * n_h * ((d_c + d_r) + d_c)
    achieved = byts / (dec_ms * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us, decode_attn {dec_ms * 1e3:.1f} us, {achieved:.0f} GB/s, "
        f"{flops / (dec_ms * 1e-3) / 1e12:.0f} TFLOP/s")
    wl = {"uniform": f"uniform B={w.B} T={int(w.lens[0])}",
          "ragged": f"ragged B={w.B} T~U[1024,32768] sum={w.total_rows}",
          "long": f"long-context B={w.B} T={int(w.lens[0])}",
          "layer": f"full layer step B={w.B} prior T~U[512,8192] sum={w.total_rows}",
          "causal": f"causal B={w.B} T={int(w.lens[0])} n_q={n_q} new tokens per sequence",
          "paged": f"ragged B={w.B} T~U[1024,32768] sum={w.total_rows} in a paged pool of "
                   f"{args.block_rows}-row blocks",
          "fp8": f"ragged B={w.B} T~U[1024,32768] sum={w.total_rows}, 8-bit E4M3 cache rows with a "
                 f"per-row scale"}[name]
    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "cache-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl + " (DeepSeek-V3 dims n_h=128 d_c=512 d_R=64)",
                   "B": w.B, "cache_tokens": tokens,
                   "step": ("absorb_q_normed+append_normed+decode_attn+project_out(o,u)" if args.norms
                            else "absorb_q+append+decode_attn+project_out(o,u)") if layer
                   else "absorb_q+decode_attn_causal+project_out(o)" if n_q > 1
                   else "absorb_q+decode_attn_paged+project_out(o)" if paged
                   else "absorb_q+decode_attn_fp8+project_out(o)" if fp8
                   else "absorb_q+decode_attn+project_out(o)",
                   "input_copies_rotated": copies,
                   "launch": ("host launches" if args.no_graph else "one HIP graph per input copy")
                   + (", the append on a second stream" if side is not None else "")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(name if name != "causal" else f"causal_nq{n_q}"),
                     "kernel": ("mla_decode_attn_causal" if n_q > 1 else "mla_decode_attn_paged" if paged
                                else "mla_decode_attn_fp8" if fp8 else "mla_decode_attn")
                     + " (split attention with length scan + combine)",
                     "decode_us": dec_ms * 1e3, "algorithmic_bytes": byts,
                     "mfma_tflops": flops / (dec_ms * 1e-3) / 1e12,
                     "mfma_frac": flops / (dec_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    # the binding roof: the one whose time at peak is longer (8-bit rows carry
    # 480 FLOP per byte, past the bf16 ridge, so the matrix cores bind there)
    mfma_tflops = flops / (dec_ms * 1e-3) / 1e12
    if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > byts / (HBM_PEAK_GBS * 1e9):
        out["roofline"].update({"bound": "mfma", "achieved": mfma_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": mfma_tflops / MFMA_BF16_PEAK_TFLOPS,
                                "hbm_gbs": achieved, "hbm_frac": achieved / HBM_PEAK_GBS})
    if not args.no_cpu_baseline and n_q == 1:
        log(f"oracle baseline on the host ({args.cpu_seconds:.0f} s budget) ...")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
