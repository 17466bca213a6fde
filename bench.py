#!/usr/bin/env python3
"""Benchmark: decode attention over a low-rank KV cache on one MI355X.

Workload (default): Llama-3.1-8B geometry, 32 layers, batch 16, 32 query /
8 kv heads, head_dim 128, context 32768, layer-varying ranks (r_K, r_V) =
(32, 96) on even and (48, 112) on odd layers, bfloat16 cache.  One step is
the whole hot path over one batch: for every layer, compress a 4096-token
prefill chunk (K and V) into rows [N-1-4096, N-1); then for every layer,
compress the appended token (K and V) into row N-1 and attend one query per
head over all N tokens.
All inputs are synthetic, seeded, and resident in HBM before timing.

Reported `value`: decode microseconds per layer-step, i.e. one
lrkv_decode_step per layer (the attention kernel, whose extra workgroup per
(batch, kv head) compresses and stores the appended token, + the merge
kernel), averaged over the 32 layers and the timed steps, measured with HIP
events on the launch stream around each layer's two launches.  The timed
steps alternate: in even-numbered ones an extra event between the two
launches times the attention kernel alone (the roofline's duration), the
odd-numbered ones give the layer-step figure.  The roofline entry is for the attention kernel
(split_bf16_kernel, the dominant one): its algorithmic bytes per launch (key
and value coefficient rows, both bases, the queries, the appended token in and
its coefficient rows out) over its average launch time.  `cpu_baseline` times the float64 CPU oracle on a
bounded sample of the same decode and scales it to a layer-step.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-cpu-baseline]
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

METRIC = "decode attn μs/layer-step & achieved HBM GB/s (% peak) at ctx 8K-128K"
HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published figure


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the variant, hybrid and 32-layer-step figures")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the 32-layer-step figures (their HIP graph replays; for counter passes)")
    p.add_argument("--only", choices=("hybrid", "sweep"),
                   help="run only the hybrid 128K figures or only the 32-layer-step sweep (for profiling)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle sample")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", flush=True)
        return 2

    import torch
    import decode_attention_lrkv_amd as lrkv
    from decode_attention_lrkv_amd import bytes_model as bm
    import lrkv_synth as synth

    lrkv.library()   # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        threads = min(16, len(os.sched_getaffinity(0)))
        fig = (bench_hybrid if args.only == "hybrid" else bench_step_sweep)(torch, lrkv, bm, synth, dev, threads)
        print(json.dumps({args.only: fig}), flush=True)
        return 0
    w = synth.BATCHED_32K
    L, B, Hq, H, d = w.layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    N = w.n_ctx[0]
    cap = N
    P = w.prefill
    p0 = N - 1 - P                      # first row of the prefill chunk
    threads = min(16, len(os.sched_getaffinity(0)))

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------- inputs (generated once per layer parity, copied per layer)
    t_gen = time.time()
    base = {}
    for par in (0, 1):
        rk, rv = w.ranks(par)
        ck = np.zeros((B, H, cap, rk), np.uint16)
        cv = np.zeros((B, H, cap, rv), np.uint16)
        ck[:, :, :p0] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, par, "k", b, h, p0, exact=False),
                                          threads=threads).store
        cv[:, :, :p0] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, par, "v", b, h, p0, exact=False),
                                          threads=threads).store
        xk = synth.tokens_major(synth.stack_heads(
            w, lambda b, h: synth.full_tokens(w, par, "k", b, h, P, synth.PART_PREFILL), threads=threads)).store
        xv = synth.tokens_major(synth.stack_heads(
            w, lambda b, h: synth.full_tokens(w, par, "v", b, h, P, synth.PART_PREFILL), threads=threads)).store
        base[par] = dict(
            rk=rk, rv=rv,
            ck=dev_bf16(ck), cv=dev_bf16(synth.to_value_octets(cv)),
            xk=dev_bf16(xk), xv=dev_bf16(xv),
            bk=dev_bf16(synth.basis(w, par, "k").store), bv=dev_bf16(synth.basis(w, par, "v").store))
        del ck, cv, xk, xv
    layers = []
    for l in range(L):
        bs = base[l % 2]
        xa_k = synth.tokens_major(synth.stack_heads(
            w, lambda b, h: synth.full_tokens(w, l, "k", b, h, 1, synth.PART_APPEND), threads=threads)).store
        xa_v = synth.tokens_major(synth.stack_heads(
            w, lambda b, h: synth.full_tokens(w, l, "v", b, h, 1, synth.PART_APPEND), threads=threads)).store
        layers.append(dict(
            rk=bs["rk"], rv=bs["rv"], bk=bs["bk"], bv=bs["bv"],
            ck=bs["ck"].clone(), cv=bs["cv"].clone(),       # distinct addresses per layer
            xk=bs["xk"].clone(), xv=bs["xv"].clone(),
            ak=dev_bf16(xa_k), av=dev_bf16(xa_v),
            q=dev_bf16(synth.query(w, l).store),
            out=torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev),
            lse=torch.empty((B, Hq), dtype=torch.float32, device=dev)))
    del base
    ws_bytes = max(lrkv.decode_step_workspace_bytes(B, Hq, H, d, lay["rk"], lay["rv"], cap, N) for lay in layers)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)   # decode workspaces start zero-filled
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t_gen:.1f}s: {torch.cuda.memory_allocated() / 2**30:.1f} GiB on device, "
        f"workspace {ws_bytes / 2**20:.2f} MiB")

    # ---------------- one step: prefill chunk of every layer, then one decode step of every layer
    def step(ev=None, split=True):
        for l, lay in enumerate(layers):
            if ev: ev["pre"][l][0].record()
            lrkv.compress_kv(lay["xk"], lay["xv"], lay["bk"], lay["bv"], lay["ck"], lay["cv"], p0)
            if ev: ev["pre"][l][1].record()
        for l, lay in enumerate(layers):
            # lrkv_decode_step as its two launches; in a split step an event
            # between them times the attention kernel (which also compresses
            # and stores the appended token) alone
            if ev: ev["dec"][l][0].record()
            lrkv.decode_step_partial(lay["q"], lay["ak"], lay["av"], lay["bk"], lay["ck"], lay["bv"], lay["cv"], N, ws)
            if ev and split: ev["dec"][l][1].record()
            lrkv.decode_step_merge(lay["out"], lay["lse"], N, ws, H, lay["rk"], lay["rv"], cap)
            if ev: ev["dec"][l][2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    mk = lambda n: [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    events = [{"pre": [mk(2) for _ in range(L)], "dec": [mk(3) for _ in range(L)]} for _ in range(K)]
    torch.cuda.synchronize()
    # Even-numbered steps are split (an event between the attention and the
    # merge launch of every layer, for the kernel's own time); the layer-step
    # figure comes from the odd-numbered steps, whose two launches follow each
    # other with no event between them (an event there adds a few us), or
    # from every step when only one is timed.
    split = lambda k: k % 2 == 0
    t0 = time.perf_counter()
    for k in range(K):
        step(events[k], split(k))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {K} steps in {wall:.3f}s")

    prefill_us, decode_us, attn_us, merge_us = [], [], [], []
    attn_by_par = {0: [], 1: []}
    whole = [k for k in range(K) if not split(k)] or list(range(K))
    for k in range(K):
        for l in range(L):
            ep, ed = events[k]["pre"][l], events[k]["dec"][l]
            prefill_us.append(ep[0].elapsed_time(ep[1]) * 1e3)
            if k in whole:
                decode_us.append(ed[0].elapsed_time(ed[2]) * 1e3)
            if split(k):
                attn_us.append(ed[0].elapsed_time(ed[1]) * 1e3)
                merge_us.append(ed[1].elapsed_time(ed[2]) * 1e3)
                attn_by_par[l % 2].append(attn_us[-1])

    # ---------------- bytes and rates
    app_bytes = {p: bm.compress_bytes(B, 1, H, d, w.ranks(p)[0]) + bm.compress_bytes(B, 1, H, d, w.ranks(p)[1])
                 for p in (0, 1)}
    dec_bytes = {p: bm.decode_bytes(B, Hq, H, d, *w.ranks(p), N) for p in (0, 1)}
    attn_bytes = {p: bm.step_kernel_bytes(B, Hq, H, d, *w.ranks(p), N) for p in (0, 1)}
    pre_bytes = {p: bm.compress_bytes(B, P, H, d, w.ranks(p)[0]) + bm.compress_bytes(B, P, H, d, w.ranks(p)[1])
                 for p in (0, 1)}
    mean = lambda xs: float(np.mean(xs))
    dec_us = mean(decode_us)
    dec_gbps = sum((dec_bytes[l % 2] + app_bytes[l % 2]) for l in range(L)) * len(whole) / (sum(decode_us) * 1e-6) / 1e9
    attn_mean = {p: mean(attn_by_par[p]) for p in (0, 1)}
    attn_gbps = sum(attn_bytes[l % 2] for l in range(L)) * (len(attn_us) // L) / (sum(attn_us) * 1e-6) / 1e9
    pre_gbps = sum(pre_bytes[l % 2] for l in range(L)) * K / (sum(prefill_us) * 1e-6) / 1e9
    step_decode_us = dec_us * L
    tok_s = B / (step_decode_us * 1e-6)

    # a plain device copy of 4 GiB for context (practical bandwidth ceiling)
    src = torch.empty(2 ** 31, dtype=torch.uint16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    peak_dev = device_peak_gbps(lrkv)
    result = {
        "metric": METRIC,
        "value": round(dec_us, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "batch": B, "n_q_heads": Hq, "n_kv_heads": H,
                   "head_dim": d, "context": N, "ranks_even": list(w.ranks(0)), "ranks_odd": list(w.ranks(1)),
                   "prefill_chunk": P, "cache_dtype": "bf16", "accumulate": "fp32"},
        "decode_us_per_layer_step": stats(decode_us),
        "decode_GBps": round(dec_gbps, 1),
        "decode_pct_peak": round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
        "device_peak": peak_dev,
        "attn_tokens_per_s": round(tok_s, 1),
        "decode_us_per_step_32_layers": round(step_decode_us, 1),
        "attn_kernel_us": {"even": stats(attn_by_par[0]), "odd": stats(attn_by_par[1])},
        "merge_us": stats(merge_us),
        "prefill_compress_us_per_layer": stats(prefill_us),
        "prefill_compress_GBps": round(pre_gbps, 1),
        "device_copy_GBps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": "split_bf16_kernel",
                     "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": round(sum(attn_bytes[l % 2] for l in range(L)) / L)},
    }

    if not args.no_extra:
        result["variants_32k"] = bench_variants(torch, lrkv, bm, synth, dev, layers, ws, dev_bf16)
    del layers, ws
    torch.cuda.empty_cache()
    if not args.no_extra:
        result["hybrid_128k"] = bench_hybrid(torch, lrkv, bm, synth, dev, threads)
        if not args.no_sweep:
            result["step_32layer_sweep"] = bench_step_sweep(torch, lrkv, bm, synth, dev, threads)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def bench_variants(torch, lrkv, bm, synth, dev, layers, ws, dev_bf16):
    """Variants of the decode on the same 32-layer batched caches, each timed
    per call (TIMED_ITERS calls after WARM_ITERS, cycling over the layers):
    - latent queries and outputs (projections that absorb the bases: no fold,
      no lift, no basis read);
    - the decode step with a separate, non-orthogonal key encoder (decoder D
      folds the query, encoder E compresses the appended key), and the plain
      decode step timed the same way for comparison;
    - the Oja update of both bases of a layer, from its 4096-token prefill
      chunk and at decode shape (the step's one appended token per sequence).
    Each decode figure is two launches (attention + merge)."""
    w = synth.BATCHED_32K
    B, Hq, H, d, L = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.layers
    N = w.n_ctx[0]
    lat = {p: dev_bf16(synth.latent_query(w, p).store) for p in (0, 1)}
    tf = {p: tuple(dev_bf16(x.store) for x in synth.key_transform(w, p, "k")) for p in (0, 1)}
    outs = {p: torch.empty((B, Hq, w.ranks(p)[1]), dtype=torch.bfloat16, device=dev) for p in (0, 1)}

    def latent(i):
        lay = layers[i % L]
        lrkv.decode_attn_latent(lat[i % 2], lay["ck"], lay["cv"], N, d, out=outs[i % 2], lse=lay["lse"],
                                workspace=ws)

    def transform_step(i):
        lay = layers[i % L]
        enc, dec = tf[i % 2]
        lrkv.decode_step(lay["q"], lay["ak"], lay["av"], dec, lay["ck"], lay["bv"], lay["cv"], N, out=lay["out"],
                         lse=lay["lse"], workspace=ws, enc_k=enc)

    def plain_step(i):
        lay = layers[i % L]
        lrkv.decode_step(lay["q"], lay["ak"], lay["av"], lay["bk"], lay["ck"], lay["bv"], lay["cv"], N,
                         out=lay["out"], lse=lay["lse"], workspace=ws)

    # Oja update of both bases of a layer (float32 master bases; the bfloat16
    # copies go to buffers of their own, so the caches' bases stay as they are)
    # from the layer's 4096-token prefill chunk, and from the decode step's
    # appended token (batch 16 x 1 token)
    oja = {p: [] for p in (0, 1)}
    oja_dec = {p: [] for p in (0, 1)}
    for l, lay in enumerate(layers[:2]):
        for key, x in (("bk", "xk"), ("bv", "xv")):
            b32 = lay[key].float().contiguous()
            oja[l].append((lay[x], b32, torch.empty_like(lay[key])))
            tok = lay["ak" if key == "bk" else "av"].view(B, 1, H, d)
            oja_dec[l].append((tok, b32.clone(), torch.empty_like(lay[key])))
    P = layers[0]["xk"].shape[1]
    oja_ws = torch.empty(max(lrkv.oja_workspace_bytes(B, H, d, r, P) for p in (0, 1) for r in w.ranks(p)),
                         dtype=torch.uint8, device=dev)

    def oja_layer(i):
        for x, b32, b16 in oja[i % 2]:
            lrkv.oja_update(x, b32, 1e-9, basis_bf16=b16, workspace=oja_ws)

    def oja_decode(i):
        for x, b32, b16 in oja_dec[i % 2]:
            lrkv.oja_update(x, b32, 1e-9, basis_bf16=b16, workspace=oja_ws)

    lat_us = _timed(torch, latent)
    tf_us = _timed(torch, transform_step)
    plain_us = _timed(torch, plain_step)
    oja_us = _timed(torch, oja_layer)
    oja_dec_us = _timed(torch, oja_decode)
    oja_bytes = sum(bm.oja_bytes(B, P, H, d, r) for p in (0, 1) for r in w.ranks(p)) / 2
    oja_flops = sum(bm.oja_flops(B, P, H, d, r) for p in (0, 1) for r in w.ranks(p)) / 2
    oja_dec_bytes = sum(bm.oja_bytes(B, 1, H, d, r) for p in (0, 1) for r in w.ranks(p)) / 2
    lat_bytes = sum(bm.latent_decode_bytes(B, Hq, H, *w.ranks(p), N) for p in (0, 1)) / 2
    return {"latent_decode_us_per_layer": lat_us,
            "latent_decode_GBps": round(lat_bytes / (lat_us["mean"] * 1e-6) / 1e9, 1),
            "transform_step_us_per_layer": tf_us,
            "plain_step_us_per_layer": plain_us,
            "oja_update_us_per_layer": oja_us,
            "oja_update_GBps": round(oja_bytes / (oja_us["mean"] * 1e-6) / 1e9, 1),
            "oja_update_TFLOPs": round(oja_flops / (oja_us["mean"] * 1e-6) / 1e12, 1),
            "oja_update_decode_us_per_layer": oja_dec_us,
            "oja_update_decode_GBps": round(oja_dec_bytes / (oja_dec_us["mean"] * 1e-6) / 1e9, 1),
            "note": "same caches and context as the main figure, layers cycled call after call (no prefill "
                    "between them); two launches per decode call; the Oja update is of both bases of a layer "
                    "(three launches per basis through the Gram matrix), from its 4096-token prefill chunk and at decode shape "
                    "(batch 16 x the step's one appended token)"}


TIMED_ITERS = 200   # timed calls per figure
WARM_ITERS = 20     # untimed calls before them


def stats(us):
    """mean and p10 / p50 / p90 of per-call times (microseconds)."""
    a = np.asarray(us, dtype=np.float64)
    return {"mean": round(float(a.mean()), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p50": round(float(np.percentile(a, 50)), 3), "p90": round(float(np.percentile(a, 90)), 3),
            "n": int(a.size)}


def _timed(torch, fn, iters=TIMED_ITERS, warm=WARM_ITERS):
    """Call fn(i) `warm` times untimed, then `iters` times, each call between
    its own pair of HIP events on the current stream (the stream the library
    launches on).  Returns stats() of the per-call times in microseconds."""
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return stats([a.elapsed_time(b) * 1e3 for a, b in ev])


def _back_to_back(torch, fn, iters=TIMED_ITERS, warm=WARM_ITERS):
    """Mean microseconds per call of `iters` calls issued in a row between
    one pair of HIP events on the current stream (after `warm` untimed calls)."""
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / iters, 3)


def bench_hybrid(torch, lrkv, bm, synth, dev, threads):
    """Hybrid cache at 131072 tokens: selection + compaction of every token, then decode.

    Three caches rotate so that the 256 MB last-level cache cannot hold the
    working set between decode calls.
    """
    w = synth.HYBRID_128K
    n = w.n_ctx[0]
    H, d = w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(0)
    t0 = time.time()
    inj = synth.injected_set(w, 0, 0, n)
    k = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.hybrid_tokens(w, 0, "k", b, h, n, inj),
                                             threads=threads)).store
    v = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.hybrid_tokens(w, 0, "v", b, h, n, inj),
                                             threads=threads)).store
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    kd, vd = dv(k), dv(v)
    # three input sets (the token order rotated by a third) so that no call
    # finds its keys and values in the last-level cache from the call before
    kvs = [(kd, vd)] + [(torch.roll(kd, j * n // 3, dims=1), torch.roll(vd, j * n // 3, dims=1)) for j in (1, 2)]
    bk, bv, q = dv(synth.basis(w, 0, "k").store), dv(synth.basis(w, 0, "v").store), dv(synth.query(w, 0).store)
    side_cap = 8192
    caches = [lrkv.HybridCache(1, w.n_q_heads, H, d, rk, rv, n, side_cap, dev) for _ in range(3)]
    cws = torch.empty(lrkv.compress_hybrid_workspace_bytes(1, w.n_q_heads, H, d, rk, rv, n, n),
                      dtype=torch.uint8, device=dev)

    def compress(i):
        c = caches[i % 3]
        c.n_lr.zero_()
        c.n_side.zero_()
        lrkv.compress_hybrid(c, *kvs[i % 3], bk, bv, 0.5, 0, workspace=cws)

    comp_us = _timed(torch, compress)
    n_side = int(caches[0].n_side[0, 0].item())
    dws = torch.zeros(lrkv.decode_workspace_bytes(1, w.n_q_heads, H, d, rk, rv, n, 0, side_cap),
                      dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((1, w.n_q_heads), dtype=torch.float32, device=dev)
    dec_call = lambda i: lrkv.decode_attn_hybrid(q, bk, bv, caches[i % 3], out=out, lse=lse, workspace=dws)
    dec_us = _timed(torch, dec_call)
    dec_b2b = _back_to_back(torch, dec_call)
    comp_bytes = (2 * n * H * d * 2 + (n - n_side) * H * (rk + rv) * 2 + n_side * H * (2 * d * 2 + 4)
                  + H * d * (rk + rv) * 2)
    dec_bytes = bm.decode_bytes(1, w.n_q_heads, H, d, rk, rv, n, side_tokens=n_side)
    log(f"hybrid figures in {time.time() - t0:.1f}s")
    return {"workload": w.name, "context": n, "side_tokens_per_kv_head": n_side,
            "compress_us": comp_us, "compress_bytes": comp_bytes,
            "compress_GBps": round(comp_bytes / comp_us["mean"] / 1e3, 1),
            "decode_us": dec_us, "decode_bytes": dec_bytes,
            "decode_GBps": round(dec_bytes / dec_us["mean"] / 1e3, 1),
            "decode_pct_peak": round(100 * dec_bytes / dec_us["mean"] / 1e3 / HBM_PEAK_GBPS, 2),
            "decode_pct_peak_p50": round(100 * dec_bytes / dec_us["p50"] / 1e3 / HBM_PEAK_GBPS, 2),
            "decode_us_back_to_back": dec_b2b,
            "decode_pct_peak_back_to_back": round(100 * dec_bytes / dec_b2b / 1e3 / HBM_PEAK_GBPS, 2),
            "note": "decode_us: each call between its own pair of events (the event commands between calls "
                    "add about 2 us); decode_us_back_to_back: TIMED_ITERS calls in a row between one pair"}


def bench_step_sweep(torch, lrkv, bm, synth, dev, threads):
    """32-layer decode step at batch 1, context 256 / 2048 / 8192: one
    lrkv_decode_step per layer (append + attention [+ merge]), eager and as a
    HIP graph replayed at one context; the same step through the device-length
    entry point as one graph that advances the context by one token per
    replay (the graph appends a token to every layer's cache and increments
    the length); and, for comparison, the unfused sequence (compress launch +
    decode) as a graph, and the attention alone on latent queries
    (lrkv_decode_attn_latent per layer: no fold, no lift, no appended token)
    as a graph."""
    w = synth.LLAMA_STEP
    L, Hq, H, d = w.layers, w.n_q_heads, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(0)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    bk, bv = dv(synth.basis(w, 0, "k").store), dv(synth.basis(w, 0, "v").store)
    grow = TIMED_ITERS + WARM_ITERS          # tokens the advancing graph appends
    res = {}
    for n in w.n_ctx:
        cap = (n + grow + 7) // 8 * 8
        ck0 = np.zeros((1, H, cap, rk), np.uint16)
        cv0 = np.zeros((1, H, cap, rv), np.uint16)
        ck0[:, :, :n] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, 0, "k", b, h, n, exact=False),
                                          threads=threads).store
        cv0[:, :, :n] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, 0, "v", b, h, n, exact=False),
                                          threads=threads).store
        ck0, cv0 = dv(ck0), dv(synth.to_value_octets(cv0))
        lay = [dict(ck=ck0.clone(), cv=cv0.clone(), q=dv(synth.query(w, l).store),
                    ak=dv(synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(
                        w, l, "k", b, h, 1, synth.PART_APPEND))).store),
                    av=dv(synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(
                        w, l, "v", b, h, 1, synth.PART_APPEND))).store),
                    out=torch.empty((1, Hq, d), dtype=torch.bfloat16, device=dev),
                    lse=torch.empty((1, Hq), dtype=torch.float32, device=dev)) for l in range(L)]
        ws = torch.zeros(max(lrkv.decode_workspace_bytes(1, Hq, H, d, rk, rv, cap, n),
                             lrkv.decode_step_workspace_bytes(1, Hq, H, d, rk, rv, cap, n),
                             lrkv.decode_step_workspace_bytes(1, Hq, H, d, rk, rv, cap, n + grow)),
                         dtype=torch.uint8, device=dev)
        seq_lens = torch.full((1,), n, dtype=torch.int32, device=dev)

        def step(_i=0):      # one lrkv_decode_step per layer at context n
            for x in lay:
                lrkv.decode_step(x["q"], x["ak"], x["av"], bk, x["ck"], bv, x["cv"], n, out=x["out"], lse=x["lse"],
                                 workspace=ws)

        def step_advancing():   # the same with the length on the device, then one more token
            for x in lay:
                lrkv.decode_step_seqlens(x["q"], x["ak"], x["av"], bk, x["ck"], bv, x["cv"], seq_lens, n + grow,
                                         out=x["out"], lse=x["lse"], workspace=ws)
            seq_lens.add_(1)

        def step_unfused(_i=0):   # compress of the token, then the decode
            for x in lay:
                lrkv.compress_kv(x["ak"], x["av"], bk, bv, x["ck"], x["cv"], n - 1)
                lrkv.decode_attn(x["q"], bk, x["ck"], bv, x["cv"], n, out=x["out"], lse=x["lse"], workspace=ws)

        for x in lay:   # latent queries for projections that absorb the bases (no fold, no lift)
            x["ql"] = x["q"][..., :rk].contiguous()
            x["ol"] = torch.empty((1, Hq, rv), dtype=torch.bfloat16, device=dev)

        def step_latent(_i=0):   # the attention alone on latent queries (no appended token)
            for x in lay:
                lrkv.decode_attn_latent(x["ql"], x["ck"], x["cv"], n, d, out=x["ol"], lse=x["lse"], workspace=ws)

        def graph_of(fn):
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                fn()
            return g

        eager = _timed(torch, step)
        g = graph_of(step)
        graph = _timed(torch, lambda i: g.replay())
        g2 = graph_of(step_unfused)
        graph_unfused = _timed(torch, lambda i: g2.replay())
        g4 = graph_of(step_latent)
        latent = _timed(torch, lambda i: g4.replay())
        g3 = graph_of(step_advancing)       # the eager warm-up and the capture leave the length at n + 1
        seq_lens.fill_(n)
        torch.cuda.synchronize()
        advancing = _timed(torch, lambda i: g3.replay())
        reached = int(seq_lens.item())
        step_bytes = L * (bm.decode_bytes(1, Hq, H, d, rk, rv, n) + bm.compress_bytes(1, 1, H, d, rk)
                          + bm.compress_bytes(1, 1, H, d, rv))
        res[str(n)] = {"eager_us_per_step": eager, "graph_us_per_step": graph,
                       "graph_us_per_layer": round(graph["mean"] / L, 2),
                       "advancing_graph_us_per_step": advancing,
                       "advancing_context_range": [n + WARM_ITERS, reached - 1],
                       "unfused_graph_us_per_step": graph_unfused,
                       "latent_attn_graph_us_per_step": latent,
                       "graph_GBps_effective": round(step_bytes / graph["mean"] / 1e3, 1)}
        del lay, g, g2, g3, g4, ws
        torch.cuda.empty_cache()
    return {"workload": w.name, "layers": L, "by_context": res,
            "note": "working set <= 0.6 GB per step; 'effective' bandwidth can include last-level-cache hits; "
                    "the latent graph attends rows [0, n) with no appended token; "
                    "the advancing graph appends one token per replay (its context grows from n by "
                    f"{WARM_ITERS} warm-up and {TIMED_ITERS} timed replays)"}


def device_peak_gbps(lrkv):
    """HBM peak from the device's own properties (memory clock x bus width),
    next to the published 8 TB/s.  The attributes are read through the HIP
    runtime the library itself uses (hipDeviceGetAttribute, attributes 59 =
    memory bus width in bits and 60 = peak memory clock in kHz in
    hip_runtime_api.h).  The double-data-rate formula clock x 2 x width / 8 is
    the one the properties are usually read with; HBM's actual transfers per
    clock are not among the properties, so the figure is reported as read."""
    import ctypes
    try:
        lib = lrkv.library()
        get = lib.hipDeviceGetAttribute
        get.restype = ctypes.c_int
        get.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
        dev = ctypes.c_int(0)
        lib.hipGetDevice.argtypes = [ctypes.POINTER(ctypes.c_int)]
        lib.hipGetDevice(ctypes.byref(dev))
        width, clock = ctypes.c_int(0), ctypes.c_int(0)
        if get(ctypes.byref(width), 59, dev.value) or get(ctypes.byref(clock), 60, dev.value):
            return None
    except (AttributeError, OSError):
        return None
    ddr = clock.value * 1e3 * 2 * width.value / 8 / 1e9
    return {"memory_clock_khz": clock.value, "memory_bus_width_bits": width.value,
            "clock_x2_x_width_GBps": round(ddr, 1), "published_GBps": HBM_PEAK_GBPS}


# the sources the attention kernel is compiled from; the counter record is
# valid for the kernel built from exactly these
KERNEL_SOURCES = ("decode_body.h", "decode_split.hip", "lrkv_device.h", "lrkv_internal.h")


def kernel_sources_sha256():
    """SHA-256 over the attention kernel's sources, in KERNEL_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_lrkv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, or None when the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "split_bf16_kernel_llama8b-b16-32k.txt")
    try:
        rec = next(json.loads(l.split("TRAFFIC", 1)[1]) for l in open(path) if l.strip().startswith("TRAFFIC"))
        sha = kernel_sources_sha256()
    except (OSError, StopIteration, ValueError):
        return None
    return rec["mean_bytes_per_launch"] if rec.get("kernel_src_sha256") == sha else None


def cpu_baseline(w, budget_s):
    """Time the float64 CPU oracle on a bounded sample of the same decode layer-step.

    Sample: whole (batch, kv head) units of the decode (reconstruct K_hat and
    V_hat of all N tokens, attend the 4 query heads; plus compressing the
    appended token), alternating odd and even layers, until the budget is
    spent; the mean per unit times B * Hkv units is the layer-step estimate.
    """
    import lrkv_synth as synth
    from oracle import lrkv_oracle as O
    try:
        from threadpoolctl import threadpool_info
        n_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        n_threads = None
    N = w.n_ctx[0]
    g = w.group
    times = []
    t_start = time.time()
    u = 0
    while time.time() - t_start < budget_s or len(times) < 2:
        layer = u % 2
        b, h = (u // 2) % w.batch, (u // (2 * w.batch)) % w.n_kv_heads
        ck = synth.direct_coeffs(w, layer, "k", b, h, N - 1).exact
        cv = synth.direct_coeffs(w, layer, "v", b, h, N - 1).exact
        xk = synth.full_tokens(w, layer, "k", b, h, 1, synth.PART_APPEND).exact
        xv = synth.full_tokens(w, layer, "v", b, h, 1, synth.PART_APPEND).exact
        bk = synth.basis(w, layer, "k").exact
        bv = synth.basis(w, layer, "v").exact
        q = synth.query(w, layer).exact
        t0 = time.perf_counter()
        ak = O.round_storage(O.compress(xk[None, :, None, :], bk[h:h + 1]), "bf16")[0, 0]
        av = O.round_storage(O.compress(xv[None, :, None, :], bv[h:h + 1]), "bf16")[0, 0]
        rows = [(b, h * g + j) for j in range(g)]
        O.decode_rows(q, bk, {(b, h): np.concatenate([ck, ak])}, bv, {(b, h): np.concatenate([cv, av])},
                      N, rows)
        times.append(time.perf_counter() - t0)
        u += 1
    per_unit = float(np.mean(times))
    us = per_unit * w.batch * w.n_kv_heads * 1e6
    spread = stats(np.asarray(times) * w.batch * w.n_kv_heads * 1e6)
    return {"value": round(us, 1), "unit": "us/layer-step", "cores": n_threads, "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)),
            "per_unit_scaled_us": {k: spread[k] for k in ("p10", "p50", "p90")},
            "sample": f"{len(times)} (batch, kv-head) units of the decode at N={N} (reconstruct K_hat, V_hat; "
                      f"attend {g} query heads; compress the appended token), odd and even layers alternating, "
                      f"mean {per_unit:.3f}s per unit, scaled x{w.batch * w.n_kv_heads} to one layer-step"}


if __name__ == "__main__":
    sys.exit(main())
