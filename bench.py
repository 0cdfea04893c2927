#!/usr/bin/env python3
"""Decode throughput of the DMS hot path on one MI355X.

Workload: Qwen3-8B-shaped attention layer (hidden 4096, 32 query / 8 KV heads,
head_dim 128, bf16), B = 8 sequences with an 8192-token prompt, window 512,
block 256, per-head eviction fractions drawn from U[0.85, 0.92].  The cache of
every one of 36 layers (Qwen3-8B depth) is built separately, so one decode
step streams ~1.7 GB of live K/V, far more than the 256 MB Infinity Cache.

A step is one decode token for every sequence through all 36 layers: per layer
one dms_decode_step launch (RMSNorm + linear adapter + threshold, delayed
eviction with in-place slot reuse, and the attention over the live slots).
(--path prepare: dms_decode_prepare -> dms_decode_attn; --path unfused:
dms_decide -> dms_append_evict -> dms_decode_attn.)  Steps are captured as HIP
graphs and replayed; inputs (hidden states, Q, K, V of every step) are
resident in HBM before the timed region.

Output: one JSON line (metric, value = decode tokens/s per layer, roofline of
the step's dominant kernel, CPU-oracle baseline, prefill figures).
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DMS decode tok/s/layer + HBM GB/s vs peak, Qwen3-8B layer shape, ctx 8K, B=8"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def traffic_from_profiles(kind: str):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/*.json), if
    they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kind}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from learned_kv_cache_amd.counters import source_hash
    if rec.get("source_hash") != source_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------


class Layer:
    def __init__(self, idx, cfg, wl, dms, torch, gen, steps_total):
        self.idx = idx
        B, H, Hq, Hkv, D = wl.B, wl.hidden, wl.Hq, wl.Hkv, wl.D
        self.cache = dms.DmsCache(cfg)
        self.W = (torch.randn(Hkv, H, generator=gen, device="cuda") / math.sqrt(H)).contiguous()
        self.gamma = torch.ones(H, device="cuda")
        lo, hi = wl.p_range
        self.p_h = lo + (hi - lo) * torch.rand(Hkv, generator=gen, device="cuda")
        self.seed = 1_000_003 * (idx + 1)
        S = steps_total
        self.h_dec = torch.randn(S, B, H, generator=gen, device="cuda").to(torch.bfloat16)
        self.q_dec = torch.randn(S, B, Hq, D, generator=gen, device="cuda").to(torch.bfloat16)
        self.k_dec = torch.randn(S, B, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
        self.v_dec = torch.randn(S, B, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
        self.evict = torch.empty(B * Hkv, dtype=torch.uint8, device="cuda")
        self.out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
        self.off = torch.zeros(Hkv, device="cuda")


def prompt_chunk(layer, c, wl, torch):
    """Hidden states, K and V of prompt chunk c (regenerated from its own seed)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(layer.seed + 17 * c)
    h = torch.randn(wl.B, wl.chunk, wl.hidden, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(wl.B, wl.chunk, wl.Hkv, wl.D, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(wl.B, wl.chunk, wl.Hkv, wl.D, generator=g, device="cuda").to(torch.bfloat16)
    return h, k, v


def calibrate_and_fill(layer, wl, dms, torch):
    """Per-head offsets so that a fraction p_h of the run's tokens is evicted
    (midpoint of the order statistics around the (1-p) quantile of the
    pre-offset logits), then the 8192-token prompt goes in through
    dms_decide + dms_append_evict in chunks of 4096."""
    B, Hkv, C = wl.B, wl.Hkv, wl.chunk
    n_chunks = wl.prefill // C
    zero = torch.zeros(Hkv, device="cuda")
    logits = []
    ev = torch.empty(B * Hkv * C, dtype=torch.uint8, device="cuda")
    for c in range(n_chunks):
        h, _, _ = prompt_chunk(layer, c, wl, torch)
        lg = torch.empty(B, Hkv, C, device="cuda")
        dms.dms_decide(layer.cache, h, layer.gamma, layer.W, None, zero, None, B, C, lg, ev)
        logits.append(lg.permute(1, 0, 2).reshape(Hkv, -1))
    S = layer.h_dec.shape[0]
    lg = torch.empty(S * B, Hkv, 1, device="cuda")
    evd = torch.empty(S * B * Hkv, dtype=torch.uint8, device="cuda")
    dms.dms_decide(layer.cache, layer.h_dec, layer.gamma, layer.W, None, zero, None, S * B, 1, lg, evd)
    logits.append(lg.permute(1, 0, 2).reshape(Hkv, -1))
    allv = torch.cat(logits, dim=1)
    srt, _ = torch.sort(allv, dim=1)
    n = srt.shape[1]
    kept = torch.round((1.0 - layer.p_h) * n).long().clamp(1, n - 1)
    lo = srt.gather(1, (kept - 1)[:, None])[:, 0]
    hi = srt.gather(1, kept[:, None])[:, 0]
    layer.off.copy_(0.5 * (lo + hi))
    for c in range(n_chunks):
        h, k, v = prompt_chunk(layer, c, wl, torch)
        dms.dms_decide(layer.cache, h, layer.gamma, layer.W, None, layer.off, None, B, C, None, ev)
        dms.dms_append_evict(layer.cache, None, k, v, ev, B, C)


def calibrate_and_fill_ragged(layer, wl, ctx, dms, torch):
    """As calibrate_and_fill, for prompts of per-sequence lengths ctx[b]:
    each sequence's prompt goes in alone, in chunks of up to 4096 tokens
    (each chunk's rows drawn from its own seed)."""
    Hkv, C, H = wl.Hkv, wl.chunk, wl.hidden
    zero = torch.zeros(Hkv, device="cuda")

    def chunk(b, c0, n):
        g = torch.Generator(device="cuda")
        g.manual_seed(layer.seed + 17 * c0 + 7919 * (b + 1))
        h = torch.randn(1, n, H, generator=g, device="cuda").to(torch.bfloat16)
        k = torch.randn(1, n, Hkv, wl.D, generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn(1, n, Hkv, wl.D, generator=g, device="cuda").to(torch.bfloat16)
        return h, k, v

    spans = [(b, c0, min(C, int(ctx[b]) - c0)) for b in range(wl.B) for c0 in range(0, int(ctx[b]), C)]
    ev = torch.empty(Hkv * C, dtype=torch.uint8, device="cuda")
    logits = []
    for b, c0, n in spans:
        h, _, _ = chunk(b, c0, n)
        lg = torch.empty(1, Hkv, n, device="cuda")
        dms.dms_decide(layer.cache, h, layer.gamma, layer.W, None, zero, None, 1, n, lg, ev[: Hkv * n])
        logits.append(lg[0])
    S = layer.h_dec.shape[0]
    lg = torch.empty(S * wl.B, Hkv, 1, device="cuda")
    evd = torch.empty(S * wl.B * Hkv, dtype=torch.uint8, device="cuda")
    dms.dms_decide(layer.cache, layer.h_dec, layer.gamma, layer.W, None, zero, None, S * wl.B, 1, lg, evd)
    logits.append(lg.permute(1, 0, 2).reshape(Hkv, -1))
    allv = torch.cat(logits, dim=1)
    srt, _ = torch.sort(allv, dim=1)
    n_all = srt.shape[1]
    kept = torch.round((1.0 - layer.p_h) * n_all).long().clamp(1, n_all - 1)
    layer.off.copy_(0.5 * (srt.gather(1, (kept - 1)[:, None])[:, 0] + srt.gather(1, kept[:, None])[:, 0]))
    for b, c0, n in spans:
        h, k, v = chunk(b, c0, n)
        seq = torch.tensor([b], dtype=torch.int32, device="cuda")
        dms.dms_decide(layer.cache, h, layer.gamma, layer.W, None, layer.off, None, 1, n, None, ev[: Hkv * n])
        dms.dms_append_evict(layer.cache, seq, k, v, ev[: Hkv * n], 1, n)


def step_bindings(layers, wl, dms, torch, S):
    """One dms_step_layers binding per decode step s: every layer's inputs and
    outputs of step s (the tensors are bound, not copied, so no copy runs in
    the timed region) and all B rows in order."""
    seq = torch.arange(wl.B, dtype=torch.int32, device="cuda")
    binds = []
    for s in range(S):
        io = [dict(hidden=L.h_dec[s], rms_gamma=L.gamma, W=L.W, offsets=L.off, q_inout=L.q_dec[s], k=L.k_dec[s],
                   v=L.v_dec[s], out=L.out, evict_out=L.evict) for L in layers]
        binds.append(dms.StepLayers([L.cache for L in layers], io))
    return seq, binds


def decode_step(layers, s, wl, dms, path, ws, binds=None):
    """One decode step over every layer; `ws` is the decode workspace all
    layers share (their calls run in stream order)."""
    B = wl.B
    if path == "layers":
        seq, b = binds
        b[s].run(seq, B, workspace=ws)
        return
    for L in layers:
        if path == "step":
            dms.dms_decode_step(L.cache, None, L.h_dec[s], L.gamma, L.W, None, L.off, L.q_dec[s], L.k_dec[s],
                                L.v_dec[s], L.out, B, None, L.evict, workspace=ws)
            continue
        if path == "prepare":
            dms.dms_decode_prepare(L.cache, None, L.h_dec[s], L.gamma, L.W, None, L.off, None, L.k_dec[s],
                                   L.v_dec[s], B, None, L.evict)
        else:
            dms.dms_decide(L.cache, L.h_dec[s], L.gamma, L.W, None, L.off, None, B, 1, None, L.evict)
            dms.dms_append_evict(L.cache, None, L.k_dec[s], L.v_dec[s], L.evict, B, 1)
        dms.dms_decode_attn(L.cache, None, L.q_dec[s], L.out, B, workspace=ws)


# ---------------------------------------------------------------------------


def run_decode(args, dms, synth, torch, extra_paths=()):
    """The headline decode figures (path args.path), then those of each path
    in extra_paths on the same caches (the step inputs are replayed; the
    caches hold room for every run), under "paths"."""
    wl = synth.QWEN8B_DECODE
    S = args.warmup + args.steps
    max_tokens = wl.prefill + S * (1 + len(extra_paths))
    pool_pages = wl.B * wl.Hkv * math.ceil(max_tokens / wl.block)
    cfg = dms.make_config(
        max_batch=wl.B, num_q_heads=wl.Hq, num_kv_heads=wl.Hkv, head_dim=wl.D, hidden=wl.hidden,
        window=wl.window, block_size=wl.block, max_tokens_per_seq=max_tokens, pool_pages=pool_pages,
        max_chunk=wl.chunk, kv_dtype="bf16", decide_mode="linear", alpha_per="head")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + wl.cfg_id)
    layers = []
    t0 = time.time()
    for i in range(args.layers):
        L = Layer(i, cfg, wl, dms, torch, gen, S)
        calibrate_and_fill(L, wl, dms, torch)
        layers.append(L)
    torch.cuda.synchronize()
    for L in layers:
        st = dms.dms_cache_status(L.cache)
        assert st == 0, f"device status {st:#x}"
    log(f"{args.layers} layers filled with {wl.prefill} tokens x {wl.B} sequences in {time.time() - t0:.1f}s")

    out = time_decode(layers, wl, dms, torch, S, args.warmup, args.steps, args.path, args.attn_reps, args.eager)
    for path in extra_paths:
        r = time_decode(layers, wl, dms, torch, S, args.warmup, args.steps, path, args.attn_reps, args.eager)
        out.setdefault("paths", {})[path] = {k: r[k] for k in ("value", "ms_per_step", "layer_step_us",
                                                               "launch_bytes", "launch_gbs", "one_launch")}
    return out


def time_decode(layers, wl, dms, torch, S, warmup, steps, path, attn_reps, eager=False):
    """Replays `steps` timed decode steps (after `warmup`) over the layer
    caches from one captured graph per step, then the attention alone; HIP
    events on the launch stream; figures per layer step."""
    ws = dms.decode_workspace(layers[0].cache.cfg, wl.B)
    binds = None
    if path == "layers":
        binds = step_bindings(layers, wl, dms, torch, S)
        one = binds[1][0].one_launch(wl.B)
        log(f"{wl.name}: dms_step_layers over {len(layers)} layers, one launch: {one}")
    graphs = []
    if not eager:
        for s in range(S):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                decode_step(layers, s, wl, dms, path, ws, binds)
            graphs.append(g)
        torch.cuda.synchronize()
        log(f"captured {S} step graphs")

    def step(s):
        if graphs:
            graphs[s].replay()
        else:
            decode_step(layers, s, wl, dms, path, ws, binds)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    live0 = [dms.dms_cache_stats(L.cache) for L in layers]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for s in range(warmup, S):
        step(s)
    ev1.record()
    torch.cuda.synchronize()
    elapsed_ms = ev0.elapsed_time(ev1)
    live1 = [dms.dms_cache_stats(L.cache) for L in layers]
    for L in layers:
        st = dms.dms_cache_status(L.cache)
        assert st == 0, f"device status {st:#x}"
    ms_per_step = elapsed_ms / steps
    tok_s_layer = wl.B * steps * len(layers) / (elapsed_ms / 1e3)
    log(f"{wl.name}: timed {steps} steps: {ms_per_step:.3f} ms/step, {tok_s_layer / 1e6:.3f} M tok/s/layer")

    # Decode attention alone (context for the two-call paths): one graph
    # holding the dms_decode_attn calls of all layers (the cache state does not
    # change), replayed; HIP events on the launch stream around the replays;
    # average per call.
    reps = attn_reps
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for L in layers:
            dms.dms_decode_attn(L.cache, None, L.q_dec[S - 1], L.out, wl.B, workspace=ws)
    ga.replay()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(reps):
        ga.replay()
    a1.record()
    torch.cuda.synchronize()
    attn_us = a0.elapsed_time(a1) * 1e3 / (reps * len(layers))

    elem = 1 if wl.kv_dtype == "fp8" else 2
    row_bytes = wl.D * elem
    kv_live = float(np.mean([s["bytes_live"] for s in live1]))          # K+V bytes the attention reads
    kv_live_mid = float(np.mean([(a["bytes_live"] + b["bytes_live"]) / 2 for a, b in zip(live0, live1)]))
    qo_bytes = 2 * wl.B * wl.Hq * wl.D * 2
    pages = float(np.mean([s["pages_in_use"] for s in live1]))
    scale_bytes = pages * 8 if wl.kv_dtype == "fp8" else 0.0
    attn_bytes = kv_live + qo_bytes + pages * 4 + scale_bytes
    attn_gbs = attn_bytes / (attn_us * 1e-6) / 1e9
    mean_L = kv_live / (wl.B * wl.Hkv * 2 * row_bytes)
    step_bytes = kv_live_mid + qo_bytes
    # one dms_decode_step launch: the live K/V after the append (the current
    # token's row comes from the input), Q and O, the hidden state, the adapter
    # row and gamma, the new K/V rows written into the pages, the page ids
    pages_mid = float(np.mean([(a["pages_in_use"] + b["pages_in_use"]) / 2 for a, b in zip(live0, live1)]))
    launch_bytes = (kv_live_mid + qo_bytes + wl.B * wl.hidden * 2 + wl.Hkv * wl.hidden * 4 + wl.hidden * 4
                    + wl.B * wl.Hkv * 2 * row_bytes + pages_mid * 4)
    layer_us = ms_per_step * 1e3 / len(layers)
    stats = live1[0]
    return {
        "launch_bytes": launch_bytes,
        "launch_gbs": launch_bytes / (layer_us * 1e-6) / 1e9,
        "value": tok_s_layer,
        "ms_per_step": ms_per_step,
        "attn_us": attn_us,
        "attn_bytes": attn_bytes,
        "attn_gbs": attn_gbs,
        "mean_live_slots_per_head": mean_L,
        "layer_step_us": layer_us,
        "step_kv_gbs": step_bytes * len(layers) / (ms_per_step * 1e-3) / 1e9,
        "kv_bytes_resident_per_layer": float(np.mean([s["bytes_allocated"] for s in live1])),
        "kv_bytes_live_per_layer": kv_live,
        "dense_bf16_kv_bytes_per_layer": float(wl.B * wl.Hkv * (wl.prefill + S) * 2 * wl.D * 2),
        "cache_cr": stats["cache_cr"],
        "graphs": bool(graphs),
        "one_launch": None if binds is None else binds[1][0].one_launch(wl.B),
    }


def run_other_decode(dms, synth, torch, wl, n_layers, steps, warmup, paths=("step",)):
    """A further decode configuration, reported beside the headline: wl's
    layer shape and prompts (uniform, or per-sequence log-uniform lengths),
    n_layers separate layer caches (enough to exceed the Infinity Cache),
    each step path of `paths` in turn on the same caches (the step inputs are
    replayed; the caches hold room for every run).  Returns the
    per-layer-step figures of time_decode for the first path, and those of
    the others under "paths"."""
    S = warmup + steps
    cap = S * len(paths)
    if wl.ctx_range is None:
        ctx = np.full(wl.B, wl.prefill)
    else:
        rng = np.random.default_rng(1000 + wl.cfg_id)
        lo, hi = wl.ctx_range
        ctx = np.round(np.exp(rng.uniform(math.log(lo), math.log(hi), wl.B))).astype(np.int64)
    max_tokens = int(ctx.max()) + cap
    pool_pages = int(sum(wl.Hkv * math.ceil((int(c) + cap) / wl.block) for c in ctx))
    cfg = dms.make_config(
        max_batch=wl.B, num_q_heads=wl.Hq, num_kv_heads=wl.Hkv, head_dim=wl.D, hidden=wl.hidden,
        window=wl.window, block_size=wl.block, max_tokens_per_seq=max_tokens, pool_pages=pool_pages,
        max_chunk=wl.chunk, kv_dtype=wl.kv_dtype, decide_mode="linear", alpha_per="head")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + wl.cfg_id)
    layers = []
    t0 = time.time()
    for i in range(n_layers):
        L = Layer(i, cfg, wl, dms, torch, gen, S)
        if wl.ctx_range is None:
            calibrate_and_fill(L, wl, dms, torch)
        else:
            calibrate_and_fill_ragged(L, wl, ctx, dms, torch)
        layers.append(L)
    torch.cuda.synchronize()
    for L in layers:
        st = dms.dms_cache_status(L.cache)
        assert st == 0, f"device status {st:#x}"
    log(f"{wl.name}: {n_layers} layers filled (mean prompt {ctx.mean():.0f}) in {time.time() - t0:.1f}s")
    keys = ("value", "layer_step_us", "attn_us", "attn_gbs", "attn_bytes", "launch_bytes", "launch_gbs",
            "mean_live_slots_per_head", "kv_bytes_live_per_layer", "cache_cr", "one_launch")
    out = {"workload": wl.name, "layers": n_layers, "batch": wl.B, "kv_dtype": wl.kv_dtype,
           "mean_prompt": float(ctx.mean()), "steps": steps, "path": paths[0]}
    for i, path in enumerate(paths):
        r = time_decode(layers, wl, dms, torch, S, warmup, steps, path, 10)
        if i == 0:
            out.update({k: r[k] for k in keys})
            out["attn_frac_hbm_peak"] = r["attn_gbs"] / HBM_PEAK_GBS
        else:
            out.setdefault("paths", {})[path] = {k: r[k] for k in keys}
    del layers
    torch.cuda.empty_cache()
    return out


def run_prefill(args, dms, synth, torch, variant="qneuron"):
    """32K-token prompt in 4096-token chunks: per chunk dms_decide ->
    dms_prefill_attn -> dms_append_evict, each call timed with HIP events on
    the launch stream.  variant "qneuron": decision from the last query
    element (offset 5); "linear": RMSNorm + linear adapter over a
    4096-wide bf16 hidden state (a = 100, offset 5)."""
    wl = synth.QWEN8B_PREFILL32K if variant == "qneuron" else synth.QWEN8B_PREFILL32K_LINEAR
    T, C = wl.prefill, wl.chunk
    nch = T // C
    cfg = dms.make_config(
        max_batch=1, num_q_heads=wl.Hq, num_kv_heads=wl.Hkv, head_dim=wl.D, hidden=wl.hidden,
        window=wl.window, block_size=wl.block, max_tokens_per_seq=T, pool_pages=wl.Hkv * (T // wl.block),
        max_chunk=C, kv_dtype="bf16", decide_mode=wl.decide, alpha_per="head")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + wl.cfg_id)
    q = torch.randn(nch, 1, C, wl.Hq, wl.D, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn(nch, 1, C, wl.Hkv, wl.D, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(nch, 1, C, wl.Hkv, wl.D, generator=gen, device="cuda").to(torch.bfloat16)
    h = W = gamma = None
    if variant == "linear":
        h = torch.randn(nch, 1, C, wl.hidden, generator=gen, device="cuda").to(torch.bfloat16)
        W = torch.randn(wl.Hkv, wl.hidden, generator=gen, device="cuda") / math.sqrt(wl.hidden)
        gamma = torch.ones(wl.hidden, device="cuda")
    off = torch.full((wl.Hkv,), float(wl.fixed_offset), device="cuda")
    ev = torch.empty(nch, wl.Hkv * C, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, C, wl.Hq, wl.D, dtype=torch.bfloat16, device="cuda")

    def once(qq, ev_times=None):
        cache = dms.DmsCache(cfg)
        for c in range(nch):
            e = ev_times[c] if ev_times else None
            if e:
                e[0].record()
            if variant == "qneuron":
                dms.dms_decide(cache, None, None, None, None, off, qq[c], 1, C, None, ev[c])
            else:
                dms.dms_decide(cache, h[c], gamma, W, None, off, None, 1, C, None, ev[c])
            if e:
                e[1].record()
            dms.dms_prefill_attn(cache, None, qq[c], k[c], v[c], ev[c], out, 1, C)
            if e:
                e[2].record()
            dms.dms_append_evict(cache, None, k[c], v[c], ev[c], 1, C)
            if e:
                e[3].record()
        return cache

    once(q.clone())
    torch.cuda.synchronize()
    qq = q.clone()
    times = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nch)]
    once(qq, times)
    torch.cuda.synchronize()
    decide_ms = sum(t[0].elapsed_time(t[1]) for t in times)
    attn_ms = sum(t[1].elapsed_time(t[2]) for t in times)
    append_ms = sum(t[2].elapsed_time(t[3]) for t in times)
    total_ms = times[0][0].elapsed_time(times[-1][3])
    # useful flops: 4 * D per (query head, visible key) pair; |V(i)| = (i+1) - #{j <= i-w: e_j}
    e = ev.view(nch, wl.Hkv, C).permute(1, 0, 2).reshape(wl.Hkv, T).to(torch.int64)
    ce = torch.cumsum(e, dim=1)
    i = torch.arange(T, device="cuda")
    evicted_out = torch.where(i >= wl.window, ce[:, (i - wl.window).clamp(min=0)], torch.zeros_like(ce))
    vis = (i + 1)[None, :] - evicted_out
    useful = 4.0 * wl.D * wl.g * float(vis.sum())
    res = {
        "workload": wl.name,
        "tokens": T,
        "ms_per_prompt": total_ms,
        "tok_s": T / (total_ms / 1e3),
        "decide_ms": decide_ms,
        "attn_ms": attn_ms,
        "append_ms": append_ms,
        "useful_tflop": useful / 1e12,
        "attn_tflops": useful / (attn_ms * 1e-3) / 1e12,
        "frac_bf16_peak": useful / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "evict_fraction": float(e.float().mean()),
    }
    # the decisions alone, back to back on the GPU: the 8 chunks' calls captured
    # in a graph and replayed (the per-call events above include the host's
    # launch time, which these short kernels do not cover)
    cache = dms.DmsCache(cfg)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in range(nch):
            if variant == "qneuron":
                dms.dms_decide(cache, None, None, None, None, off, qq[c], 1, C, None, ev[c])
            else:
                dms.dms_decide(cache, h[c], gamma, W, None, off, None, 1, C, None, ev[c])
    graph.replay()
    torch.cuda.synchronize()
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    res["decide_ms_graph"] = e0.elapsed_time(e1) / reps
    if variant == "linear":
        hbytes = T * wl.hidden * 2
        res["decide_hbm_gbs"] = hbytes / (res["decide_ms_graph"] * 1e-3) / 1e9
    return res


def run_train_fwd(args, dms, torch):
    """Training-mode forward (gate + soft-eviction attention) at the Qwen3-8B
    layer shape: B = 2 sequences of T = 4096 tokens, window 512, gate logits
    from N(0, 3) logits plus logistic noise at tau = 0.1; each call timed with
    HIP events on the launch stream.  Useful work: 4 * D flops per (query
    head, causal key) pair (training keeps every causal key).  The backward
    (dq, dk, dv and the gate-logit gradient from a seeded N(0, 1) output
    gradient) is timed the same way; its useful work is the five products of
    the softmax backward, 10 * D flops per pair."""
    B, T, Hq, Hkv, D, w = 2, 4096, 32, 8, 128, 512
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    q = torch.randn(B, T, Hq, D, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn(B, T, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, T, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
    logits = 3.0 * torch.randn(B, Hkv, T, generator=gen, device="cuda")
    u = torch.rand(B, Hkv, T, generator=gen, device="cuda").clamp(1e-6, 1 - 1e-6)
    noise = torch.log(u) - torch.log1p(-u)
    y = torch.empty_like(logits)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, device="cuda")

    def once():
        dms.dms_train_gate(logits, noise, 0.1, y, None, None)
        dms.dms_train_attn_fwd(q, k, v, y, out, lse, window=w)

    for _ in range(3):
        once()
    torch.cuda.synchronize()
    reps = 20
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(reps):
        dms.dms_train_gate(logits, noise, 0.1, y, None, None)
    e1.record()
    for _ in range(reps):
        dms.dms_train_attn_fwd(q, k, v, y, out, lse, window=w)
    e2.record()
    torch.cuda.synchronize()
    gate_ms = e0.elapsed_time(e1) / reps
    attn_ms = e1.elapsed_time(e2) / reps
    useful = 4.0 * D * Hq * B * T * (T + 1) / 2

    dout = torch.randn(B, T, Hq, D, generator=gen, device="cuda").to(torch.bfloat16)
    dq = torch.empty(q.shape, device="cuda")
    dk, dv = torch.empty(k.shape, device="cuda"), torch.empty(v.shape, device="cuda")
    dy = torch.empty_like(logits)
    ws = torch.empty(dms.dms_train_attn_bwd_workspace_bytes(B, T, Hq), dtype=torch.uint8, device="cuda")

    def bwd():
        dms.dms_train_attn_bwd(q, k, v, out, dout, y, lse, dq, dk, dv, dy, window=w, workspace=ws)

    for _ in range(3):
        bwd()
    torch.cuda.synchronize()
    b0, b1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    b0.record()
    for _ in range(reps):
        bwd()
    b1.record()
    torch.cuda.synchronize()
    bwd_ms = b0.elapsed_time(b1) / reps
    useful_bwd = 2.5 * useful
    return {
        "workload": "qwen3-8b_layer_train_fwd_b2_t4096_w512",
        "attn_ms": attn_ms,
        "gate_ms": gate_ms,
        "useful_tflop": useful / 1e12,
        "attn_tflops": useful / (attn_ms * 1e-3) / 1e12,
        "frac_bf16_peak": useful / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "tok_s": B * T / ((attn_ms + gate_ms) * 1e-3),
        "bwd_ms": bwd_ms,
        "bwd_useful_tflop": useful_bwd / 1e12,
        "bwd_tflops": useful_bwd / (bwd_ms * 1e-3) / 1e12,
        "bwd_frac_bf16_peak": useful_bwd / (bwd_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        # one layer's attention training step: gate, forward and backward
        "step_ms": gate_ms + attn_ms + bwd_ms,
        "step_tok_s": B * T / ((gate_ms + attn_ms + bwd_ms) * 1e-3),
    }


def run_kvzap(args, dms, torch):
    """KVzap scorers at the KVzap-mlp page's Qwen3-8B shape (hidden 4096, inner
    512, 8 KV heads) and the linear scorer (4096 -> 8), bf16 hidden states,
    f32 weights: one 4096-token prefill chunk and one B = 8 decode step each,
    timed with HIP events over repeated calls on the launch stream.  Work per
    token: MLP 2 * 4096 * 512 + 2 * 512 * 8 flops; bytes: hidden 8 KB per
    token, weights once per call (MLP 8 MB + 16 KB, linear 128 KB).  The calls
    are replayed from a HIP graph (50 per replay): GPU time per call."""
    H, Hm, Hkv = 4096, 512, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(777)
    W1 = torch.randn(Hm, H, generator=gen, device="cuda") / math.sqrt(H)
    b1 = 0.1 * torch.randn(Hm, generator=gen, device="cuda")
    W2 = torch.randn(Hkv, Hm, generator=gen, device="cuda") / math.sqrt(Hm)
    b2 = torch.full((Hkv,), -4.0, device="cuda")
    Wl = torch.randn(Hkv, H, generator=gen, device="cuda") / math.sqrt(H)
    bl = torch.full((Hkv,), -4.0, device="cuda")
    res = {"workload": "kvzap_qwen3-8b_h4096_inner512_kv8"}
    for name, B, T in (("chunk4096", 1, 4096), ("decode_b8", 8, 1)):
        h = torch.randn(B, T, H, generator=gen, device="cuda").to(torch.bfloat16)
        ev = torch.empty(B * Hkv * T, dtype=torch.uint8, device="cuda")
        sc = torch.empty(B * Hkv * T, device="cuda")
        ws = torch.empty(dms.dms_kvzap_workspace_bytes(B, T, Hkv, Hm), dtype=torch.uint8, device="cuda")
        calls = {
            "mlp": lambda: dms.dms_kvzap_score(h, W1, b1, ev, W2=W2, b2=b2, threshold=-4.0, scores_out=sc,
                                               workspace=ws),
            "linear": lambda: dms.dms_kvzap_score(h, Wl, bl, ev, threshold=-4.0, scores_out=sc),
        }
        for kind, fn in calls.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            # 50 calls captured in one graph, so that host launch costs stay out of the figure
            reps = 50
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(reps):
                    fn()
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            N = B * T
            flops = 2.0 * N * (H * Hm + Hm * Hkv) if kind == "mlp" else 2.0 * N * H * Hkv
            wbytes = 4.0 * (Hm * H + Hkv * Hm) if kind == "mlp" else 4.0 * Hkv * H
            nbytes = 2.0 * N * H + wbytes + 5.0 * N * Hkv
            res[f"{kind}_{name}_us"] = us
            res[f"{kind}_{name}_tflops"] = flops / (us * 1e-6) / 1e12
            res[f"{kind}_{name}_gbs"] = nbytes / (us * 1e-6) / 1e9
    res["mlp_chunk4096_frac_fp32_mfma_peak"] = res["mlp_chunk4096_tflops"] / FP32_PEAK_TFLOPS
    return res


def cpu_baseline(steps: int):
    """The CPU oracle (float64 NumPy) on a bounded sample of the same decode
    workload: one layer, B = 8, 8192-token prompt, `steps` decode steps of
    decide + cache simulation + masked attention.  Prompt state is built
    untimed."""
    import oracle
    from learned_kv_cache_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    wl = synth.QWEN8B_DECODE
    d = synth.draw(wl, run_id=7)
    B, Hkv = wl.B, wl.Hkv
    pre = []
    for b in range(B):
        lg, _ = oracle.decide_linear(d.tensor("h", b)[None, : wl.prefill], d.gamma, d.W, np.zeros(Hkv),
                                     alpha_scale=wl.alpha_scale, eps=1e-6)
        pre.append(lg[0])
    off = np.array([synth.offset_for_fraction(np.concatenate([p[k] for p in pre]), d.p_h[k]) for k in range(Hkv)])
    e_hist = [(p - off[:, None] > 0).astype(np.uint8) for p in pre]
    steps = min(steps, wl.decode_steps)
    sim = oracle.CacheSim(B, Hkv, wl.window, wl.block, wl.prefill + wl.decode_steps, B * Hkv * 64)
    for s in range(0, wl.prefill, wl.chunk):
        sim.append(list(range(B)), np.stack([e[:, s:s + wl.chunk] for e in e_hist]))
    K = [d.tensor("k", b, keep=True) for b in range(B)]
    V = [d.tensor("v", b, keep=True) for b in range(B)]
    hd = [d.decode_rows("h", b) for b in range(B)]
    qd = [d.decode_rows("q", b) for b in range(B)]
    scale = 1.0 / math.sqrt(wl.D)
    t0 = time.perf_counter()
    for i in range(steps):
        t = wl.prefill + i
        h = np.stack([hd[b][i] for b in range(B)])[:, None]
        _, e = oracle.decide_linear(h, d.gamma, d.W, off, alpha_scale=wl.alpha_scale, eps=1e-6)
        sim.append(list(range(B)), e)
        for b in range(B):
            e_hist[b] = np.concatenate([e_hist[b], e[b]], axis=1)
            oracle.attention_rows(qd[b][i][None], K[b][: t + 1], V[b][: t + 1], e_hist[b], wl.window, [t], scale)
    dt = time.perf_counter() - t0
    # the same loop with BLAS held to one thread, on a quarter of the steps
    from threadpoolctl import threadpool_limits
    steps1 = min(max(4, steps // 4), wl.decode_steps - steps)
    sim1 = __import__("copy").deepcopy(sim)
    e1 = [x.copy() for x in e_hist]
    with threadpool_limits(1):
        t1 = time.perf_counter()
        for i in range(steps, steps + steps1):
            t = wl.prefill + i
            h = np.stack([hd[b][i] for b in range(B)])[:, None]
            _, e = oracle.decide_linear(h, d.gamma, d.W, off, alpha_scale=wl.alpha_scale, eps=1e-6)
            sim1.append(list(range(B)), e)
            for b in range(B):
                e1[b] = np.concatenate([e1[b], e[b]], axis=1)
                oracle.attention_rows(qd[b][i][None], K[b][: t + 1], V[b][: t + 1], e1[b], wl.window, [t], scale)
        dt1 = max(time.perf_counter() - t1, 1e-9)
    return {
        "value": B * steps / dt,
        "unit": "tok/s/layer",
        "cores": blas_threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{steps} decode steps of one Qwen3-8B-shaped layer, B=8, ctx 8192 (float64 NumPy: "
                  f"decide + cache simulation + masked attention); prompt state built untimed",
        "seconds": dt,
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas_threads": blas_threads,
        "one_thread": {"value": B * steps1 / dt1 if steps1 > 0 else None, "steps": steps1, "seconds": dt1,
                       "blas_threads": 1},
    }


def measure_peaks(dms, torch) -> dict:
    """The box's own rates (libdms_probe): a streaming read of a 4 GiB buffer
    (16 times the Infinity Cache) over 15 launch shapes, best of them, and a
    dense bf16 matrix-core loop (8 independent 16x16x32 products per wave,
    8 waves per CU); HIP events on the launch stream around repeated calls."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(8 * cus * 8, dtype=torch.int32, device="cuda")
    best = (0.0, None)
    sweep = []
    # one to eight workgroups per CU, 4 to 16 loads of 16 bytes in flight per thread
    for grid, unroll in [(cus * w, u) for w in (1, 2, 3, 4, 8) for u in (4, 8, 16)]:
        dms.probe_read(buf, grid, unroll, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            nbytes = dms.probe_read(buf, grid, unroll, sink)
        e1.record()
        torch.cuda.synchronize()
        gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        sweep.append({"grid": grid, "unroll": unroll, "gbs": round(gbs, 1)})
        if gbs > best[0]:
            best = (gbs, {"grid": grid, "unroll": unroll, "bytes": nbytes})
    del buf
    grid, iters = 2 * cus, 20000
    dms.probe_mfma_bf16(grid, 200, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = sum(dms.probe_mfma_bf16(grid, iters, sink) for _ in range(5))
    e1.record()
    torch.cuda.synchronize()
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"hbm_read_gbs": best[0], "hbm_read_shape": best[1], "hbm_read_sweep": sweep, "bf16_mfma_tflops": tflops,
            "hbm_nominal_gbs": HBM_PEAK_GBS, "bf16_nominal_tflops": BF16_PEAK_TFLOPS, "compute_units": cus}


def copy_calibration(mib: int, torch) -> None:
    """A plain read-once/write-once elementwise kernel over `mib` MiB of bf16
    (torch.neg), run 4 times: its FETCH_SIZE and WRITE_SIZE readings scale the
    counters of the other kernels (learned_kv_cache_amd.counters)."""
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 4 x {mib} MiB read + write")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--attn-reps", type=int, default=20)
    ap.add_argument("--eager", action="store_true", help="launch kernels directly instead of replaying graphs")
    ap.add_argument("--path", choices=("step", "layers", "prepare", "unfused"), default="step",
                    help="step: one dms_decode_step launch per layer; layers: one dms_step_layers launch for "
                         "every layer; prepare: dms_decode_prepare -> dms_decode_attn; unfused: dms_decide -> "
                         "dms_append_evict -> dms_decode_attn")
    ap.add_argument("--cpu-steps", type=int, default=96)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured HBM / bf16 peak probes")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="end with a plain elementwise copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the DMS decode path is timed on a single GPU", file=sys.stderr)
        return 2
    import torch
    from learned_kv_cache_amd import dms, synth
    dms.lib()
    torch.cuda.set_device(0)
    dec = run_decode(args, dms, synth, torch, () if args.path == "layers" else ("layers",))
    for p, r in dec.get("paths", {}).items():
        log(f"headline [{p}]: {r['layer_step_us']:.2f} us per layer step, one launch {r['one_launch']}")
    pre = None
    if not args.no_prefill:
        pre = {v: run_prefill(args, dms, synth, torch, v) for v in ("qneuron", "linear")}
        for v, r in pre.items():
            log(f"prefill {v}: {r['ms_per_prompt']:.1f} ms per 32K prompt (decide {r['decide_ms']:.2f}, "
                f"{r['decide_ms_graph']:.3f} in a graph, attention {r['attn_ms']:.2f} = {r['attn_tflops']:.1f} TFLOP/s, "
                f"append {r['append_ms']:.2f} ms)")
    train = None
    if not args.no_prefill:
        train = run_train_fwd(args, dms, torch)
        log(f"training forward: {train['attn_ms']:.3f} ms attention = {train['attn_tflops']:.1f} TFLOP/s, "
            f"gate {train['gate_ms'] * 1e3:.1f} us; backward {train['bwd_ms']:.3f} ms = "
            f"{train['bwd_tflops']:.1f} TFLOP/s; step {train['step_ms']:.3f} ms = {train['step_tok_s'] / 1e6:.2f} M tok/s")
    others = None
    if not args.no_prefill:
        # Llama-3.2-1B has 16 layers; the fp8 serving figure rotates 4 layer caches
        others = {
            "llama1b_ctx8k_b1": run_other_decode(dms, synth, torch, synth.LLAMA1B_DECODE, 16, 64, 4,
                                                 ("step", "layers")),
            "qwen8b_fp8kv_b64": run_other_decode(dms, synth, torch, synth.QWEN8B_FP8_SERVING, 4, 32, 4),
        }
        for k, r in others.items():
            log(f"{k}: {r['layer_step_us']:.2f} us per layer step ({r['value'] / 1e6:.3f} M tok/s/layer), "
                f"attention {r['attn_us']:.2f} us = {r['attn_gbs']:.0f} GB/s")
            for p, rp in r.get("paths", {}).items():
                log(f"{k} [{p}]: {rp['layer_step_us']:.2f} us per layer step, one launch {rp['one_launch']}")
    kvzap = None
    if not args.no_prefill:
        kvzap = run_kvzap(args, dms, torch)
        log(f"kvzap: mlp chunk {kvzap['mlp_chunk4096_us']:.1f} us ({kvzap['mlp_chunk4096_tflops']:.1f} TFLOP/s), "
            f"mlp decode {kvzap['mlp_decode_b8_us']:.1f} us ({kvzap['mlp_decode_b8_gbs']:.0f} GB/s), "
            f"linear chunk {kvzap['linear_chunk4096_us']:.1f} us ({kvzap['linear_chunk4096_gbs']:.0f} GB/s), "
            f"linear decode {kvzap['linear_decode_b8_us']:.1f} us")
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks(dms, torch)
        log(f"peaks: HBM read {peaks['hbm_read_gbs']:.0f} GB/s {peaks['hbm_read_shape']}, "
            f"bf16 matrix cores {peaks['bf16_mfma_tflops']:.0f} TFLOP/s")
        for r in (pre or {}).values():
            r["frac_bf16_measured"] = r["attn_tflops"] / peaks["bf16_mfma_tflops"]
        if train:
            train["frac_bf16_measured"] = train["attn_tflops"] / peaks["bf16_mfma_tflops"]
            train["bwd_frac_bf16_measured"] = train["bwd_tflops"] / peaks["bf16_mfma_tflops"]
        for r in (others or {}).values():
            r["attn_frac_hbm_measured"] = r["attn_gbs"] / peaks["hbm_read_gbs"]
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(args.cpu_steps)
        log(f"cpu baseline {cpu['value']:.1f} tok/s/layer in {cpu['seconds']:.1f}s")
    if args.path == "layers":
        traffic = traffic_from_profiles("decode_layers")
        roof = {"kernel": "decode_layers_kernel (dms_step_layers_run)", "achieved": dec["launch_gbs"],
                "algorithmic_bytes_per_launch": dec["launch_bytes"] * args.layers,
                "avg_launch_us": dec["ms_per_step"] * 1e3}
    elif args.path == "step":
        traffic = traffic_from_profiles("decode_step")
        roof = {"kernel": "decode_step_kernel (dms_decode_step)", "achieved": dec["launch_gbs"],
                "algorithmic_bytes_per_launch": dec["launch_bytes"], "avg_launch_us": dec["layer_step_us"]}
    else:
        traffic = traffic_from_profiles("decode_attn")
        roof = {"kernel": "decode_attn_fast_kernel (dms_decode_attn)", "achieved": dec["attn_gbs"],
                "algorithmic_bytes_per_launch": dec["attn_bytes"], "avg_launch_us": dec["attn_us"]}
    steps_desc = {
        "step": "per layer: dms_decode_step (decide + append + attention, one launch)",
        "layers": "every layer in one dms_step_layers launch (per layer: decide + append + attention; "
                  "a grid barrier between layers)",
        "prepare": "per layer: dms_decode_prepare (decide + append) -> dms_decode_attn",
        "unfused": "per layer: dms_decide -> dms_append_evict -> dms_decode_attn",
    }
    line = {
        "metric": METRIC,
        "value": dec["value"],
        "unit": "tok/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "qwen3-8b_layer_ctx8k_b8_decode",
            "layers": args.layers, "batch": 8, "ctx": 8192, "hidden": 4096, "q_heads": 32, "kv_heads": 8,
            "head_dim": 128, "window": 512, "block": 256, "evict_fraction": [0.85, 0.92],
            "step": steps_desc[args.path],
            "graphs": dec["graphs"], "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "kernel": roof["kernel"],
            "bound": "hbm",
            "achieved": roof["achieved"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": roof["achieved"] / HBM_PEAK_GBS,
            "traffic": traffic,
            "peak_measured": None if peaks is None else peaks["hbm_read_gbs"],
            "frac_measured": None if peaks is None else roof["achieved"] / peaks["hbm_read_gbs"],
            "algorithmic_bytes_per_launch": roof["algorithmic_bytes_per_launch"],
            "avg_launch_us": roof["avg_launch_us"],
        },
        "other_paths": {p: dict(r, frac=r["launch_gbs"] / HBM_PEAK_GBS, step=steps_desc[p])
                        for p, r in dec.get("paths", {}).items()},
        "attn_only": {"kernel": "decode_attn_fast_kernel (dms_decode_attn)", "avg_launch_us": dec["attn_us"],
                      "achieved_gbs": dec["attn_gbs"], "algorithmic_bytes_per_launch": dec["attn_bytes"]},
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
        "cpu_baseline_detail": None if cpu is None else {k: cpu[k] for k in ("host_cpus", "blas_threads", "seconds",
                                                                             "one_thread")},
        "peaks": peaks,
        "layer_step_us": dec["layer_step_us"],
        "step_kv_gbs": dec["step_kv_gbs"],
        "mean_live_slots_per_head": dec["mean_live_slots_per_head"],
        "kv_bytes_resident_per_layer": dec["kv_bytes_resident_per_layer"],
        "kv_bytes_live_per_layer": dec["kv_bytes_live_per_layer"],
        "dense_bf16_kv_bytes_per_layer": dec["dense_bf16_kv_bytes_per_layer"],
        "cache_cr": dec["cache_cr"],
        "prefill": pre,
        "train_fwd": train,
        "kvzap": kvzap,
        "other_decode": others,
    }
    print(json.dumps(line), flush=True)
    if args.copy_calib:
        copy_calibration(args.copy_calib, torch)
    return 0


if __name__ == "__main__":
    sys.exit(main())
