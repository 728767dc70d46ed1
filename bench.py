"""Benchmark of host-streamed paged attention on one MI355X.

One step = kvs_attend over every layer of the workload (one pass of the hot
path: ring copies, page gathers, dequantization, attention, split-K combine).

Default workload: resident decode at 32 Ki context (16 layers, 24 query / 4 kv
heads, d = 128, 128 resident pages per layer, one query token). `value` is
the KV bytes attended per second (all 16 layers' pages, 436,207,616 B per
step) over the timed steps. Alongside it:
  * roofline: the attention kernel's algorithmic bytes per launch (one layer,
    27,262,976 B) over its average launch duration (HIP events carried by
    each launch's dispatch on the compute stream, timed region), against
    8 TB/s HBM;
  * streamed: the same measurement at 256 Ki context with 103 resident pages
    per layer and the rest streamed through a 48-page ring, against the host
    link rate measured in the same run (1 GiB pinned copy, best of 5);
  * verify / prefill: the speculative-verify block (4 query tokens at 160 Ki
    context, 180 resident pages per layer) and the prefill ubatch (256 query
    tokens over a 128 Ki prefix, 10 % resident), each streamed through the ring
    against the measured link, plus the matrix-core kernel on the same shapes
    with every page resident: KV bytes against HBM for verify, flops against
    the dense f16 matrix peak for prefill;
  * cpu_baseline: the float64 CPU oracle on a bounded sample of layers of the
    same workload, on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-streamed] [--no-multi] [--no-cpu]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# The pool configuration each workload runs with (ring, chunk and split-K
# group sizes in pages). The full-size parity tests use the same table. The
# streamed decode runs through the 16-page ring its workload specifies; a
# 48-page ring is timed beside it as a labelled variant.
STREAMED_RING48 = dict(ring_pages=48, chunk_pages=4, group_pages=1)

POOL_CFG = {
    "resident_decode_32k": dict(ring_pages=48, chunk_pages=4, group_pages=1),
    "streamed_decode_256k": dict(ring_pages=16, chunk_pages=4, group_pages=1),
    "spec_verify_160k": dict(ring_pages=48, chunk_pages=4, group_pages=2),
    "prefill_ubatch_128k": dict(ring_pages=96, chunk_pages=16, group_pages=8),
}

METRIC = "streamed attention KV GB/s + decode attn tok/s at 32K/256K ctx, % of HBM/link roofline"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense f16 matrix peak of MI355X
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gen_layers(wl, geom, threads):
    from kvs_synth import layer_records
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda l: layer_records(wl.cid, l, wl.n_kv, geom), range(wl.n_layers)))


def setup(wl, cfg_kw, threads, type_v="q4_0"):
    import torch
    import host_streamed_paged_amd as kvs
    from kvs_synth import KVGeometry, make_q, residency_mask

    geom = KVGeometry(wl.n_kv_heads, wl.head_dim, type_v=type_v)
    t0 = time.time()
    recs = gen_layers(wl, geom, threads)
    host = [torch.from_numpy(r).pin_memory() for r in recs]
    log(f"{wl.name}: generated and pinned {sum(r.nbytes for r in recs) / 2**30:.2f} GiB in {time.time() - t0:.1f}s")
    masks = [residency_mask(wl.cid, l, wl.n_pages, wl.resident_pages, wl.own_page_resident)
             for l in range(wl.n_layers)]
    cfg = kvs.Config(n_layers=wl.n_layers, n_kv_heads=wl.n_kv_heads, n_q_heads=wl.n_q_heads,
                     max_pages=wl.n_pages, max_q_tokens=wl.n_q,
                     type_v=kvs.TYPE_Q8_0 if type_v == "q8_0" else kvs.TYPE_Q4_0, **cfg_kw)
    arena = kvs.Pool.arena_for(cfg, int(sum(int(m.sum()) for m in masks)))
    pool = kvs.Pool(cfg, arena)
    for l in range(wl.n_layers):
        pool.host_pages_set(l, host[l])
        pool.page_table_set(l, masks[l])
    qs = [torch.from_numpy(make_q(wl.cid, l, wl.n_q, wl.n_q_heads, wl.head_dim, wl.q_dtype)).cuda()
          for l in range(wl.n_layers)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for q in qs]
    return dict(recs=recs, host=host, masks=masks, cfg=cfg, arena=arena, pool=pool, qs=qs, outs=outs)


def run_steps(wl, st, n, stream, prefetch=True):
    """n steps of kvs_attend over every layer; the first ring chunk of layer
    l + 1 is prefetched as soon as layer l has been issued."""
    pool = st["pool"]
    for _ in range(n):
        for l in range(wl.n_layers):
            pool.attend(l, st["qs"][l], wl.n_kv, wl.q_pos0, wl.scale, wl.causal, st["outs"][l], None,
                        stream=stream)
            if prefetch:
                pool.stream_enqueue((l + 1) % wl.n_layers)


def timed_run(wl, st, steps, warmup):
    """Eager timing: every step issues kvs_attend per layer from Python, with
    the attention and combine launches bracketed by HIP events."""
    import torch
    stream = torch.cuda.current_stream()
    pool = st["pool"]
    run_steps(wl, st, warmup, stream)
    torch.cuda.synchronize()
    for kind in (0, 1):
        pool.profile_read(kind, reset=True)
    pool.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    run_steps(wl, st, steps, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pool.profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    n_att, ms_att = pool.profile_read(0, reset=True)
    n_cmb, ms_cmb = pool.profile_read(1, reset=True)
    return dict(ms_per_step=ms, wall_ms_per_step=wall * 1e3 / steps, attn_launches=n_att,
                attn_ms_total=ms_att, combine_launches=n_cmb, combine_ms_total=ms_cmb, steps=steps)


def graph_run(wl, st, steps, warmup):
    """Steady-state timing: the whole L-layer step (every kvs_attend call)
    captured once in a HIP graph and replayed, as a serving loop replays its
    decode step; the host issues one launch per step."""
    import torch
    pool = st["pool"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_steps(wl, st, 2, s, prefetch=False)          # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_steps(wl, st, 1, s, prefetch=False)
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del g
    return dict(ms_per_step=e0.elapsed_time(e1) / steps, wall_ms_per_step=wall * 1e3 / steps)


def streamed_run(wl, st, steps, warmup):
    """Eager timing of a streamed workload (ring launches cannot be captured
    in a graph): HIP events around the steps only, no per-launch events."""
    import torch
    stream = torch.cuda.current_stream()
    run_steps(wl, st, warmup, stream)
    torch.cuda.synchronize()
    st["pool"].profile_enable(False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    run_steps(wl, st, steps, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return dict(ms_per_step=e0.elapsed_time(e1) / steps, wall_ms_per_step=wall * 1e3 / steps)


def q8_leg(args, link):
    """The q8_0 K / q8_0 V pair on the two decode shapes: resident 32 Ki
    (graph replay of the 16-layer step, plus the eager per-kernel time) and,
    unless streamed legs are off, streamed 256 Ki through its 16-page ring."""
    from kvs_synth import WORKLOADS
    wl = WORKLOADS["resident_decode_32k"]
    st = setup(wl, POOL_CFG[wl.name], args.threads, type_v="q8_0")
    r = timed_run(wl, st, args.steps, args.warmup)
    gr = graph_run(wl, st, args.steps, args.warmup)
    pb = st["recs"][0].shape[1]
    kv_bytes = wl.n_layers * wl.n_pages * pb
    avg_att = r["attn_ms_total"] / max(1, r["attn_launches"])
    out = {"cache": "q8_0 K / q8_0 V", "page_bytes": pb,
           "resident": {"workload": wl.name, "ms_per_step": round(gr["ms_per_step"], 5),
                        "kv_gbs": round(kv_bytes / (gr["ms_per_step"] / 1e3) / 1e9, 2),
                        "attn_tok_s": round(1 / (gr["ms_per_step"] / 1e3), 1),
                        "attention_kernel_us": round(avg_att * 1e3, 3),
                        "kernel_frac_of_hbm": round(wl.n_pages * pb / (avg_att / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                        "combine_avg_us": round(r["combine_ms_total"] / max(1, r["combine_launches"]) * 1e3, 3)}}
    log(f"q8_0/q8_0 {wl.name}: graph {gr['ms_per_step']:.4f} ms/step, attention kernel {avg_att * 1e3:.2f} us")
    st["pool"].close()
    del st
    if not args.no_streamed and link:
        swl = WORKLOADS["streamed_decode_256k"]
        sst = setup(swl, POOL_CFG[swl.name], args.threads, type_v="q8_0")
        sr = streamed_run(swl, sst, args.streamed_steps, 2)
        spb = sst["recs"][0].shape[1]
        streamed_bytes = sum(int((1 - m).sum()) for m in sst["masks"]) * spb
        sec = sr["ms_per_step"] / 1e3
        out["streamed"] = {"workload": swl.name, "ms_per_step": round(sr["ms_per_step"], 4),
                           "streamed_gbs": round(streamed_bytes / sec / 1e9, 2),
                           "frac_of_link": round(streamed_bytes / sec / 1e9 / link, 4),
                           "attn_tok_s": round(1 / sec, 3)}
        log(f"q8_0/q8_0 {swl.name}: {sr['ms_per_step']:.3f} ms/step, streamed {streamed_bytes / sec / 1e9:.2f} GB/s")
        sst["pool"].close()
        del sst
    return out


def append_leg(wl, st, steps, link):
    """kvs_append on the resident decode pool (every page resident): a step's
    new rows quantized into Q8_0 / Q4_0 and written to each layer's host record
    and resident slot. One row per layer (a decode step) and a 256-row ubatch
    per layer, at the cache's last positions; eager calls over all layers,
    HIP events around `steps` such passes."""
    import torch
    pool, L, H, D = st["pool"], wl.n_layers, wl.n_kv_heads, wl.head_dim
    gen = torch.Generator(device="cuda").manual_seed(7)
    out = {"note": "host record and device slot both written; bytes = rows x kv heads x 208 (136 B K + 72 B V)"}
    for name, n in (("decode_row", 1), ("ubatch_256", 256)):
        k = torch.randn((n, H, D), device="cuda", generator=gen)
        v = torch.randn((n, H, D), device="cuda", generator=gen)
        pos0 = wl.n_kv - n
        for l in range(L):
            pool.append(l, k, v, pos0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            for l in range(L):
                pool.append(l, k, v, pos0)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (steps * L)
        nbytes = n * H * 208
        out[name] = {"rows": n, "us_per_layer": round(us, 3), "bytes_per_layer": nbytes,
                     "host_write_gbs": round(nbytes / us / 1e3, 3)}
        if link:
            out[name]["frac_of_link"] = round(nbytes / us / 1e3 / link, 4)
    return out


def variant_leg(wl, st, cfg_kw, steps, link, flags, how):
    """A second pool over the same pinned host records and residency, with
    another ring geometry or mode, timed the same way."""
    import host_streamed_paged_amd as kvs
    cfg = kvs.Config(n_layers=wl.n_layers, n_kv_heads=wl.n_kv_heads, n_q_heads=wl.n_q_heads,
                     max_pages=wl.n_pages, max_q_tokens=wl.n_q, flags=flags, **cfg_kw)
    arena = kvs.Pool.arena_for(cfg, int(sum(int(m.sum()) for m in st["masks"])))
    pool = kvs.Pool(cfg, arena)
    for l in range(wl.n_layers):
        pool.host_pages_set(l, st["host"][l])
        pool.page_table_set(l, st["masks"][l])
    sr = streamed_run(wl, dict(st, pool=pool, cfg=cfg, arena=arena), steps, 2)
    pool.close()
    pb = st["recs"][0].shape[1]
    streamed_bytes = sum(int((1 - m).sum()) for m in st["masks"]) * pb
    sec = sr["ms_per_step"] / 1e3
    log(f"{wl.name} {how}: {sr['ms_per_step']:.3f} ms/step, streamed {streamed_bytes / sec / 1e9:.2f} GB/s")
    return {"ms_per_step": round(sr["ms_per_step"], 4), "streamed_gbs": round(streamed_bytes / sec / 1e9, 2),
            "frac_of_link": round(streamed_bytes / sec / 1e9 / link, 4) if link else None, "how": how, **cfg_kw}


def zero_copy_leg(wl, st, cfg_kw, steps, link):
    """The A/B against the ring (KVS_FLAG_ZERO_COPY): the attention kernels
    read the streamed pages in place over the link instead of through the
    ring."""
    import host_streamed_paged_amd as kvs
    return variant_leg(wl, st, cfg_kw, steps, link, kvs.FLAG_ZERO_COPY,
                       "zero-copy: attention kernels read streamed pages in place from pinned host memory; "
                       "no ring, no copies")


def allowed_keys(wl):
    """Keys each query row may attend, summed over the block's query tokens."""
    if not wl.causal:
        return wl.n_q * wl.n_kv
    return sum(min(wl.n_kv, wl.q_pos0 + i + 1) for i in range(wl.n_q))


def multi_leg(name, cfg_kw, threads, link, steps, kind, zero_copy=True):
    """A multi-query workload: the streamed step through the ring, then the
    same shapes with every page resident to time the matrix-core kernel."""
    import dataclasses
    from kvs_synth import WORKLOADS
    wl = WORKLOADS[name]
    st = setup(wl, cfg_kw, threads)
    sr = streamed_run(wl, st, steps, 2)
    pb = st["recs"][0].shape[1]
    streamed_bytes = sum(int((1 - m).sum()) for m in st["masks"]) * pb
    total_bytes = wl.n_layers * wl.n_pages * pb
    sec = sr["ms_per_step"] / 1e3
    st["pool"].close()
    zc = zero_copy_leg(wl, st, cfg_kw, steps, link) if zero_copy else None
    del st
    out = {
        "workload": name, "context": wl.n_kv, "query_tokens": wl.n_q, "resident_pages_per_layer": wl.resident_pages,
        "ms_per_step": round(sr["ms_per_step"], 4), "q_tok_s": round(wl.n_q / sec, 2),
        "kv_gbs": round(total_bytes / sec / 1e9, 2), "streamed_gbs": round(streamed_bytes / sec / 1e9, 2),
        "link_gbs_measured": round(link, 2), "frac_of_link": round(streamed_bytes / sec / 1e9 / link, 4),
        "streamed_bytes_per_step": streamed_bytes, **cfg_kw,
    }
    if zc:
        out["zero_copy"] = zc
    log(f"{name}: {sr['ms_per_step']:.3f} ms/step, streamed {streamed_bytes / sec / 1e9:.2f} GB/s of link {link:.2f}")
    rwl = dataclasses.replace(wl, resident_pages=wl.n_pages)
    rst = setup(rwl, cfg_kw, threads)
    r = timed_run(rwl, rst, 5, 2)
    gr = graph_run(rwl, rst, 10, 2)
    rst["pool"].close()
    del rst
    # per layer: the whole kvs_attend call (attention and combine launches)
    # replayed as a HIP graph of the 16-layer step, as for decode, and the
    # attention launches' own durations (eager, events on their dispatches)
    layers_timed = r["steps"] * wl.n_layers
    layer_ms = gr["ms_per_step"] / wl.n_layers
    att_ms = r["attn_ms_total"] / max(1, layers_timed)
    layer_bytes = wl.n_pages * pb
    flops = 4 * wl.n_q_heads * wl.head_dim * allowed_keys(wl)
    kname = "prefill_kernel (256-row workgroups, pages converted in the workgroup)" if kind == "prefill" \
        else "verify_kernel (one 8-wave workgroup per kv head with every row, pages converted in the kernel)"
    k = {"kernel": kname + ", all pages resident", "layer_us": round(layer_ms * 1e3, 2),
         "attn_us_per_layer": round(att_ms * 1e3, 2), "attn_launches": r["attn_launches"],
         "combine_us_per_layer": round(r["combine_ms_total"] / max(1, layers_timed) * 1e3, 2),
         "bytes_per_layer": layer_bytes, "flops_per_layer": flops,
         "achieved_gbs": round(layer_bytes / (layer_ms / 1e3) / 1e9, 1),
         "achieved_tflops": round(flops / (layer_ms / 1e3) / 1e12, 1),
         "kernel_gbs": round(layer_bytes / (att_ms / 1e3) / 1e9, 1),
         "kernel_tflops": round(flops / (att_ms / 1e3) / 1e12, 1),
         "timing": "achieved_*: whole layer (attention and combine launches, HIP-graph replay of the "
                   "16-layer step); kernel_*: the attention launches' summed durations"}
    if kind == "verify":
        k.update(bound="hbm", frac=round(k["achieved_gbs"] / HBM_PEAK_GBS, 4), peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        k.update(bound="mfma", frac=round(k["achieved_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                 peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s")
    out["resident_kernel"] = k
    log(f"{name} all-resident: {layer_ms * 1e3:.1f} us per layer ({att_ms * 1e3:.1f} us attention), "
        f"{k['achieved_gbs']} GB/s, {k['achieved_tflops']} TFLOP/s")
    return out


# Sources of the decode kernel, whose HBM traffic the stored counters record:
# its own file and the headers it includes.
DECODE_SOURCES = ("kvs_decode.hip", "kvs_device.h", "kvs_internal.h")


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "host_streamed_paged_amd", "csrc")
    for f in DECODE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"attend_{workload}_counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except OSError:
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def measure_link():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8).pin_memory()
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    best = math.inf
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del src, dst
    return n / best / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, recs, qs_np, min_s=10.0, max_s=30.0):
    """The float64 oracle, one layer at a time, in whole passes over the
    workload's layers until at least min_s of work (a pass that would run past
    max_s stops at the layer where it gets there). `cores` is the number of
    host cores this process may run on; numpy's BLAS threads are reported
    beside it."""
    from oracle import attend_layer
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    t0 = time.perf_counter()
    layers = 0
    while True:
        l = layers % wl.n_layers
        attend_layer(recs[l], qs_np[l], n_kv=wl.n_kv, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                     scale=wl.scale, causal=wl.causal, q_pos0=wl.q_pos0)
        layers += 1
        el = time.perf_counter() - t0
        if (layers % wl.n_layers == 0 and el >= min_s) or el >= max_s:
            break
    dt = time.perf_counter() - t0
    layer_bytes = wl.n_pages * recs[0].shape[1]
    return {
        "value": round(layers * layer_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "blas_threads": int(blas_threads),
        "kind": "oracle",
        "sample": f"{wl.name}: {layers} layer passes ({layers / wl.n_layers:.2f} x the {wl.n_layers}-layer step; "
                  f"float64 numpy, one layer at a time), {dt:.1f}s; decode attn tok/s equivalent "
                  f"{layers / wl.n_layers / dt:.4f}",
        "attn_tok_s": round(layers / wl.n_layers / dt, 5),
    }


KERNEL_ONLY = {"decode": "resident_decode_32k", "verify": "spec_verify_160k", "prefill": "prefill_ubatch_128k"}


def kernels_only(name, args):
    """The kernels of one workload with every page resident: `steps` eager
    passes over its layers after `warmup`, per-launch HIP events."""
    import dataclasses
    from kvs_synth import WORKLOADS
    wl = WORKLOADS[name]
    rwl = dataclasses.replace(wl, resident_pages=wl.n_pages)
    st = setup(rwl, POOL_CFG[name], args.threads)
    r = timed_run(rwl, st, args.steps, args.warmup)
    gr = graph_run(rwl, st, args.steps, args.warmup)
    st["pool"].close()
    layers = r["steps"] * wl.n_layers
    per = {k: round(r[f"{k}_ms_total"] / max(1, layers) * 1e3, 3) for k in ("attn", "combine")}
    print(json.dumps({"workload": name, "all_resident": True, "layers_timed": layers,
                      "attn_launches": r["attn_launches"],
                      "combine_launches": r["combine_launches"], "us_per_layer": per,
                      "layer_us": round(r["ms_per_step"] / wl.n_layers * 1e3, 3),
                      "graph_layer_us": round(gr["ms_per_step"] / wl.n_layers * 1e3, 3),
                      "flops_per_layer": 4 * wl.n_q_heads * wl.head_dim * allowed_keys(wl),
                      "bytes_per_layer": wl.n_pages * st["recs"][0].shape[1]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="resident_decode_32k")
    ap.add_argument("--no-streamed", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-multi", action="store_true", help="skip the verify and prefill workloads")
    ap.add_argument("--no-zero-copy", action="store_true", help="skip the zero-copy A/B runs")
    ap.add_argument("--no-q8", action="store_true", help="skip the q8_0 K / q8_0 V decode legs")
    ap.add_argument("--streamed-steps", type=int, default=10)
    ap.add_argument("--threads", type=int, default=min(16, len(os.sched_getaffinity(0))))
    ap.add_argument("--kernels-only", choices=sorted(KERNEL_ONLY), default=None,
                    help="only time the attention (and staging, combine) launches of one workload with every page "
                         "resident, eager with HIP events, and print one JSON line: the run profilers wrap")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run torch device-to-device copies of MIB MiB (the reference kernel of known "
                         "traffic for scaling the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the streamed-attention path runs on a single device "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "launches": 3}), flush=True)
        return
    import host_streamed_paged_amd as kvs
    from kvs_synth import WORKLOADS

    kvs.lib()
    torch.cuda.set_device(0)
    if args.kernels_only:
        kernels_only(KERNEL_ONLY[args.kernels_only], args)
        return
    wl = WORKLOADS[args.workload]
    cfg_kw = POOL_CFG[args.workload] if args.workload in POOL_CFG else POOL_CFG["resident_decode_32k"]
    st = setup(wl, cfg_kw, args.threads)
    r = timed_run(wl, st, args.steps, args.warmup)          # eager, per-kernel events
    gr = graph_run(wl, st, args.steps, args.warmup)        # graph replay of the whole step
    kv_bytes = wl.n_layers * wl.n_pages * st["recs"][0].shape[1]
    value = kv_bytes / (gr["ms_per_step"] / 1e3) / 1e9
    layer_bytes = wl.n_pages * st["recs"][0].shape[1]
    avg_att = r["attn_ms_total"] / max(1, r["attn_launches"])
    achieved = layer_bytes / (avg_att / 1e3) / 1e9
    traffic = stored_traffic(wl.name)
    log(f"{wl.name}: graph {gr['ms_per_step']:.4f} ms/step ({value:.1f} GB/s), eager {r['ms_per_step']:.4f} ms/step, "
        f"attention kernel {avg_att * 1e3:.2f} us ({achieved:.0f} GB/s), "
        f"combine {r['combine_ms_total'] / max(1, r['combine_launches']) * 1e3:.2f} us")
    qs_np = [q.cpu().numpy() for q in st["qs"]]
    recs = st["recs"]
    link = None
    if not args.no_streamed or not args.no_multi:
        link = measure_link()
    appended = append_leg(wl, st, args.steps, link)
    log(f"append: decode row {appended['decode_row']['us_per_layer']:.2f} us/layer, 256-row ubatch "
        f"{appended['ubatch_256']['us_per_layer']:.2f} us/layer ({appended['ubatch_256']['host_write_gbs']:.2f} GB/s)")
    st["pool"].close()
    del st

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gr["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mixed(i8,f16,f32)",
        "dtype_note": "Q8_0 codes exact on int8 (decode, 16-bit fixed-point query limbs) or f16 (matrix-core "
                      "paths) matrix operands; probabilities and V elements in f16; float32 block scales, "
                      "scores, softmax and accumulation",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "layers": wl.n_layers, "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
            "head_dim": wl.head_dim, "context": wl.n_kv, "pages_per_layer": wl.n_pages,
            "resident_pages_per_layer": wl.resident_pages, "query_tokens": wl.n_q, "cache": "q8_0 K / q4_0 V",
            "kv_bytes_per_step": kv_bytes, **cfg_kw,
        },
        "attn_tok_s": round(wl.n_q / (gr["ms_per_step"] / 1e3), 1),
        "timing": "HIP-graph replay of the 16-layer step (one host launch per step)",
        "wall_ms_per_step": round(gr["wall_ms_per_step"], 5),
        "eager_ms_per_step": round(r["ms_per_step"], 5),
        "eager_wall_ms_per_step": round(r["wall_ms_per_step"], 5),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "decode_kernel<6> (resident launch, eager pass with HIP events)", "bytes_per_launch": layer_bytes,
            "avg_launch_us": round(avg_att * 1e3, 3), "launches": r["attn_launches"],
        },
        "combine_avg_us": round(r["combine_ms_total"] / max(1, r["combine_launches"]) * 1e3, 3),
        "append": appended,
    }
    if not args.no_streamed:
        swl = WORKLOADS["streamed_decode_256k"]
        scfg = POOL_CFG["streamed_decode_256k"]
        sst = setup(swl, scfg, args.threads)
        sr = streamed_run(swl, sst, args.streamed_steps, 2)
        st_info = sst["pool"].status()
        pb = sst["recs"][0].shape[1]
        streamed_bytes = sum(int((1 - m).sum()) for m in sst["masks"]) * pb
        total_bytes = swl.n_layers * swl.n_pages * pb
        sec = sr["ms_per_step"] / 1e3
        res_bytes = swl.n_layers * swl.resident_pages * pb
        result["streamed"] = {
            "workload": swl.name, "context": swl.n_kv, "resident_pages_per_layer": swl.resident_pages,
            "ms_per_step": round(sr["ms_per_step"], 4), "attn_tok_s": round(1 / sec, 3),
            "kv_gbs": round(total_bytes / sec / 1e9, 2), "streamed_gbs": round(streamed_bytes / sec / 1e9, 2),
            "link_gbs_measured": round(link, 2), "frac_of_link": round(streamed_bytes / sec / 1e9 / link, 4),
            "streamed_bytes_per_step": streamed_bytes, "kv_bytes_per_step": total_bytes,
            "ring_copy_launches_per_step": round(st_info.copies_issued / (args.streamed_steps + 2), 1),
            "resident_bytes_per_step": res_bytes,
            "schedule": f"ring {scfg['ring_pages']} pages in {scfg['chunk_pages']}-page chunks; copy workgroups "
                        "inside the compute launches; the compute lanes take chunks in turn",
        }
        log(f"{swl.name}: {sr['ms_per_step']:.3f} ms/step, streamed {streamed_bytes / sec / 1e9:.2f} GB/s "
            f"of link {link:.2f} GB/s")
        sst["pool"].close()
        result["streamed"]["ring48_variant"] = variant_leg(
            swl, sst, STREAMED_RING48, args.streamed_steps, link, 0,
            "variant: the same step through a 48-page ring in 4-page chunks (three compute lanes)")
        if not args.no_zero_copy:
            result["streamed"]["zero_copy"] = zero_copy_leg(swl, sst, scfg, args.streamed_steps, link)
        del sst

    if not args.no_q8:
        result["q8_0_v"] = q8_leg(args, link)

    if not args.no_multi:
        result["verify"] = multi_leg("spec_verify_160k", POOL_CFG["spec_verify_160k"], args.threads, link, 8, "verify",
                                     not args.no_zero_copy)
        result["prefill"] = multi_leg("prefill_ubatch_128k", POOL_CFG["prefill_ubatch_128k"], args.threads, link, 6, "prefill",
                                      not args.no_zero_copy)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, recs, qs_np)
        log(f"cpu baseline: {result['cpu_baseline']['value']} GB/s on {result['cpu_baseline']['cores']} threads")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
