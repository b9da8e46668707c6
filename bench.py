#!/usr/bin/env python3
"""Benchmark of the RidgeFill hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input, resident in HBM:
  fit : zero the statistics, accumulate every calibration chunk (rf_gram_accumulate), solve
        the ridge maps of every filled layer (rf_solve, bf16 maps out), and fold them into the
        layers' K/V projections (rf_fill_compose);
  fill: fill every prompt token of every filled layer with those maps (rf_fill_composed: the
        same caches as rf_fill, from the composed maps).
After the timed steps the direct fill (rf_fill: map product, then the K/V product) is timed
alternated with the composed one and reported under ``fill_direct``.
Default workload: the Llama-8B-shaped configuration (d=4096, 32 layers split at 16, GQA
8 x 128, RoPE base 5e5, calibration N=65536 in 32768-row chunks, lambda=0.1, T=16384).

Prints one JSON line.  ``value`` is filled tokens per second of fill time; the fit's rows
per second, per-phase times, the dominant kernel's roofline and the CPU oracle baseline ride
along.  After the timed steps, and outside them, the fill is timed once more with its maps streamed
from page-locked host memory (``fill_streamed``), and the token-wise cache translators
(KV-Lingo page, section 3.1) are timed on their own workload (28 -> 36 layers of 8 x 128 KV
heads, two source layers per target layer, 16384 tokens) and reported under ``translate``.
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector, published
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
# HBM bytes of one rf_gram_accumulate call (32768 rows, d=4096, 16 targets): the per-launch
# means (KiB) of two rocprofv3 --pmc runs of this benchmark (FETCH_SIZE, then WRITE_SIZE), and
# the factors that turn each counter into bytes (what it reads for a 1 GiB device copy: 524308
# KiB fetched, 1048576 KiB written).  The traffic profile under profiles/ gives the commands.
# The figures belong to the kernel sources they were taken on: once those hash differently the
# traffic is reported as null until the counters are taken again.
GRAM_COUNTERS = {"fetch_kib": 18663133.4, "write_kib": 1170264.8, "fetch_scale": 2.0, "write_scale": 1.0,
                 "sources": ("gram.hip", "rf_pipe.h", "rf_mfma.h", "rf_internal.h"),
                 "sources_sha256": "d42f46872c572f7c18d519612984773770d6d0ed1c2e64e9e65fa311c30fdf9a"}
METRIC = "filled tokens/sec (all filled layers) + % bf16 MFMA peak; ridge-fit rows/sec"


def gram_traffic():
    """Scaled HBM bytes of one Gram launch, or None when the kernel's sources have changed since
    the counters were read."""
    import hashlib
    h = hashlib.sha256()
    for name in GRAM_COUNTERS["sources"]:
        with open(os.path.join(ROOT, "linear_kv_cache_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != GRAM_COUNTERS["sources_sha256"]:
        return None
    return int((GRAM_COUNTERS["fetch_kib"] * GRAM_COUNTERS["fetch_scale"] +
                GRAM_COUNTERS["write_kib"] * GRAM_COUNTERS["write_scale"]) * 1024)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def composed_flop_per_token_layer(d: int, kvw: int) -> int:
    """FLOP the composed fill executes per token and layer: the triangular quadratic form (each
    256-feature tile reads the columns from its own first feature on) and the K/V product."""
    return 2 * 256 * sum(d - 256 * i for i in range(d // 256)) + 2 * d * 2 * kvw


def alternate(stream, fns, steps):
    """Median milliseconds of each callable, called in turn ``steps`` times (same clock and
    power state for all)."""
    import torch

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    for fn in fns:
        timed(fn)
    ms = [[] for _ in fns]
    for _ in range(steps):
        for i, fn in enumerate(fns):
            ms[i].append(timed(fn))
    return [statistics.median(m) for m in ms]


def cpu_translate_baseline(n_tokens: int):
    """Time the oracle's translation (fp64 NumPy) of n_tokens tokens over every target layer of
    the translation workload."""
    import numpy as np

    import oracle
    import synth
    tc = synth.TR_BENCH
    Ks, Vs = synth.source_cache(tc, n_tokens)
    Kn, Vn = Ks.float().numpy().astype(np.float64), Vs.float().numpy().astype(np.float64)
    E = oracle.relative_depth_sources(tc.n_src, tc.n_tgt, tc.nu)
    layers = []
    for l, e in enumerate(E):
        Tk, Tv, _, _ = synth.translator_maps(tc, l)
        layers.append((Kn[:, e[0]:e[0] + tc.nu].reshape(n_tokens, -1), Vn[:, e[0]:e[0] + tc.nu].reshape(n_tokens, -1),
                       Tk.float().numpy().astype(np.float64).T, Tv.float().numpy().astype(np.float64).T, None, None))
    t0 = time.perf_counter()
    oracle.translate(0, n_tokens, 0, layers, tc.n_kv_heads, tc.head_dim, tc.rope_base)
    return n_tokens / (time.perf_counter() - t0)


def cpu_baseline(cfg, n_tokens: int, n_fit_rows: int):
    """Time the oracle (fp64 NumPy) on a bounded sample of the same workload."""
    import numpy as np
    import torch

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    cores = len(os.sched_getaffinity(0))
    X = synth.hidden_states(cfg, n_tokens, "prompt").float().numpy().astype(np.float64)
    layers = []
    for l in cfg.filled_layers:
        w = synth.layer_weights(cfg, l, maps="law")
        f = lambda t: t.float().numpy().astype(np.float64)
        layers.append((f(w.W_map).T, f(w.b_map), f(w.gamma), f(w.W_k).T, f(w.W_v).T))
    t0 = time.perf_counter()
    oracle.fill(X, 0, n_tokens, 0, layers, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.rope_base)
    t_fill = time.perf_counter() - t0
    Xc = synth.hidden_states(cfg, n_fit_rows, "calib").float().numpy().astype(np.float64)
    Ys = [synth.late_layer_inputs(cfg, torch.from_numpy(Xc).to(torch.bfloat16), l).float().numpy().astype(np.float64)
          for l in cfg.filled_layers]
    t0 = time.perf_counter()
    oracle.gram_sums(Xc, Ys)
    t_gram = time.perf_counter() - t0
    return {
        "value": n_tokens / t_fill, "unit": "filled tokens/s", "cores": min(cores, threads), "kind": "oracle",
        "sample": f"fill of {n_tokens} prompt tokens x {len(cfg.filled_layers)} layers (d={cfg.d}), fp64 NumPy, "
                  f"{t_fill:.1f} s; fit rows/s from the one-pass sums of {n_fit_rows} calibration rows "
                  f"({t_gram:.1f} s)",
        "fit_rows_per_s": n_fit_rows / t_gram,
        "blas_threads": threads,
    }


def streamed_leg(steps: int, stream, dev, cfg, fw, Xp, cache, filler, ring_slots=2, layers_per_slot=2, w32=None):
    """The same fill with its maps streamed from page-locked host memory (rf_fill_streamed),
    alternated with the resident fill so both see the same clock and power state.  With the
    fp32 maps ``w32`` also the weight-only int8 maps (rf_quantize_map), resident and streamed."""
    import dataclasses

    import torch

    from linear_kv_cache_amd.runner import Filler, StreamedFiller, pinned_copy, quantize_map

    T, L = cfg.fill_tokens, cfg.n_targets
    host = [pinned_copy(W.cpu()) for W in fw.W_map]
    sw = dataclasses.replace(fw, W_map=host)
    sf = StreamedFiller(sw, cfg.rope_base, T, T, dev, ring_slots=ring_slots, layers_per_slot=layers_per_slot)

    def timed(f):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        f.fill(Xp, 0, T, 0, cache, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    timed(sf)
    res_ms, str_ms = [], []
    for _ in range(steps):
        res_ms.append(timed(filler))
        str_ms.append(timed(sf))
    rm, sm = statistics.median(res_ms), statistics.median(str_ms)
    map_bytes = L * cfg.d * cfg.d * 2
    out = {"what": "rf_fill with the maps in page-locked host memory, streamed through a device ring; "
                   "alternated with the resident fill", "ring_slots": ring_slots, "layers_per_slot": layers_per_slot,
           "ring_MiB": round(ring_slots * layers_per_slot * cfg.d * cfg.d * 2 / 2 ** 20, 1),
           "resident_maps_MiB": round(map_bytes / 2 ** 20, 1),
           "ms_median": round(sm, 3), "resident_ms_median": round(rm, 3),
           "tokens_per_s": round(T / (sm / 1e3), 1), "vs_resident": round(rm / sm, 4),
           "host_to_device_GBps": round(map_bytes / (sm / 1e3) / 1e9, 1)}
    if w32 is not None:
        qs = [quantize_map(W) for W in w32]
        qw = dataclasses.replace(fw, W_map=[q for q, _ in qs], map_scale=[s_ for _, s_ in qs])
        qf = Filler(qw, cfg.rope_base, T, T, dev, ws_slots=8)
        qsf = StreamedFiller(dataclasses.replace(qw, W_map=[pinned_copy(q.cpu()) for q, _ in qs]), cfg.rope_base, T,
                             T, dev, ring_slots=ring_slots, layers_per_slot=layers_per_slot)
        timed(qf)
        timed(qsf)
        bf_ms, qr_ms, qs_ms = [], [], []
        for _ in range(steps):
            bf_ms.append(timed(filler))
            qr_ms.append(timed(qf))
            qs_ms.append(timed(qsf))
        bm, qrm, qsm = statistics.median(bf_ms), statistics.median(qr_ms), statistics.median(qs_ms)
        qbytes = L * cfg.d * cfg.d
        # what the int8 codes change: the caches of both fills of the last layer, K and V, their
        # largest and RMS difference relative to the RMS of the bf16-map caches (a property of
        # the quantisation, outside the parity bar, which holds against the dequantised codes)
        from linear_kv_cache_amd.runner import alloc_cache
        c2 = alloc_cache(L, cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, dev)
        filler.fill(Xp, 0, T, 0, cache, stream)
        qf.fill(Xp, 0, T, 0, c2, stream)
        torch.cuda.synchronize()
        dev_max, dev_rms = 0.0, 0.0
        for a, b_ in ((cache.k[L - 1], c2.k[L - 1]), (cache.v[L - 1], c2.v[L - 1])):
            a, b_ = a.float(), b_.float()   # contiguous pools of exactly the T filled tokens
            r = float(a.pow(2).mean().sqrt())
            dev_max = max(dev_max, float((a - b_).abs().max()) / r)
            dev_rms = max(dev_rms, float((a - b_).pow(2).mean().sqrt()) / r)
        del c2
        out["int8_maps"] = {
            "what": "weight-only int8 maps (rf_quantize_map: row-wise symmetric codes and fp32 row scales), "
                    "resident and streamed, alternated with the bf16 resident fill",
            "maps_MiB": round(qbytes / 2 ** 20, 1), "resident_ms_median": round(qrm, 3),
            "streamed_ms_median": round(qsm, 3), "bf16_resident_ms_median": round(bm, 3),
            "streamed_tokens_per_s": round(T / (qsm / 1e3), 1), "streamed_vs_int8_resident": round(qrm / qsm, 4),
            "streamed_vs_bf16_resident": round(bm / qsm, 4), "resident_vs_bf16_resident": round(bm / qrm, 4),
            "host_to_device_GBps": round(qbytes / (qsm / 1e3) / 1e9, 1),
            "kv_vs_bf16_maps_max_rel_rms": round(dev_max, 4), "kv_vs_bf16_maps_rms_rel_rms": round(dev_rms, 4)}
    return out


def translate_leg(steps: int, stream, dev, tc=None):
    """Time rf_translate over every target layer of the translation workload, in one call."""
    import torch

    import linear_kv_cache_amd as rf
    import synth
    from linear_kv_cache_amd.runner import Translator, alloc_cache, translate_weights

    tc = tc or synth.TR_BENCH
    T = tc.t1 - tc.t0
    log(f"translate workload {tc.name}: {tc.n_src} -> {tc.n_tgt} layers, nu={tc.nu}, T={T}")
    E = rf.rf_relative_depth_sources(tc.n_src, tc.n_tgt, tc.nu)
    Ks, Vs = synth.source_cache(tc, T, device=dev)
    maps = [synth.translator_maps(tc, l, device=dev) for l in range(tc.n_tgt)]
    tw = translate_weights(tc.d_in, tc.n_kv_heads, tc.head_dim, tc.torch_dtype, [m[0] for m in maps],
                           [m[1] for m in maps], headwise=tc.maps == "headwise")
    del maps
    cache = alloc_cache(tc.n_tgt, tc.n_kv_heads, tc.head_dim, T, tc.torch_dtype, dev)
    tr = Translator(tw, tc.rope_base, T, dev)
    src_k = [Ks[0, e[0]] for e in E]
    src_v = [Vs[0, e[0]] for e in E]
    ld = tc.n_src * tc.d_src

    def call():
        tr.translate(src_k, src_v, ld, tc.t0, tc.t1, 0, cache, stream)

    call()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = statistics.median(ms)
    flop = T * tc.n_tgt * tc.flop_per_token_layer()
    # algorithmic bytes: the nu source layers' K and V rows read, the target K and V rows written
    nbytes = T * tc.n_tgt * (2 * tc.d_in + 2 * tc.kv_width) * 2
    tflops = flop / (med / 1e3) / 1e12
    gbps = nbytes / (med / 1e3) / 1e9
    return {"workload": tc.name, "n_src": tc.n_src, "n_tgt": tc.n_tgt, "nu": tc.nu, "d_in": tc.d_in,
            "kv_width": tc.kv_width, "tokens": T, "maps": tc.maps,
            "ms": round(statistics.mean(ms), 3), "ms_median": round(med, 3),
            "tokens_per_s": round(T / (med / 1e3), 1),
            "flop_per_token_layer": tc.flop_per_token_layer(), "tflops": round(tflops, 1),
            "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
            "bytes_per_token_layer": (2 * tc.d_in + 2 * tc.kv_width) * 2, "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def gdn_leg(steps: int, stream, dev, n_layers=12, n_heads=16, d_k=128, d_v=128, T=16384):
    """Time rf_gdn_state (the Gated DeltaNet state update of filled hybrid layers) over a
    16384-token prompt: 12 layers (the linear-attention three quarters of 16 filled layers) of
    16 heads with 128 x 128 states, bf16 keys and values, unit-length keys."""
    import torch

    import linear_kv_cache_amd as rf
    import synth
    log(f"gated deltanet state update: {n_layers} layers x {n_heads} heads x ({d_v} x {d_k}), T={T}")
    ins = [synth.gdn_inputs(11, l, T, n_heads, d_k, d_v, torch.bfloat16, device=dev) for l in range(n_layers)]
    S = [torch.zeros(n_heads, d_v, d_k, dtype=torch.float32, device=dev) for _ in range(n_layers)]
    desc = rf.gdn_desc(n_heads, d_k, d_v, torch.bfloat16, True)

    def call():
        for s in S:
            s.zero_()
        rf.rf_gdn_state(desc, [x[0] for x in ins], [x[1] for x in ins], [x[2] for x in ins], [x[3] for x in ins], S,
                        stream=stream)

    (ms,) = alternate(stream, [call], steps)
    # per token, head and state element: the row's dot product (2 FLOP) and the update
    # a s + c k (3 FLOP)
    flop = 5 * T * n_layers * n_heads * d_k * d_v
    return {"workload": f"gdn-{n_layers}x{n_heads}h-{d_v}x{d_k}-T{T}", "ms_median": round(ms, 3),
            "tokens_per_s": round(T / (ms / 1e3), 1), "tflops_fp32": round(flop / (ms / 1e3) / 1e12, 2),
            "frac_fp32_vector_peak": round(flop / (ms / 1e3) / 1e12 / FP32_PEAK_TFLOPS, 4),
            "bound": "vector ALU issue: each head's state advances one token after the other, so the "
                     "update runs on the vector units (no packed fp32: half the published fp32 peak)"}


def fill_only(cfg, steps: int, warmup: int, streamed: bool = False):
    """``--fill-only``: time rf_fill alone over a configuration's whole filled range, in its own
    chunks (the 27B-shaped and long-context workloads have no calibration set: their maps are
    the random-init law), and print one JSON line for it.  Not the benchmark's headline line."""
    import torch

    import synth
    from linear_kv_cache_amd.runner import ComposedFiller, Filler, alloc_cache, fill_weights

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    layers = cfg.filled_layers
    T = cfg.prompt_tokens
    log(f"fill-only workload {cfg.name}: d={cfg.d} layers={len(layers)} fill [{cfg.fill_t0}, {cfg.fill_t1}) "
        f"in chunks of {cfg.fill_chunk}{' (paged)' if cfg.paged else ''}")
    ws = [synth.layer_weights(cfg, l, device=dev) for l in layers]
    fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                      [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    del ws
    X = synth.hidden_states(cfg, cfg.fill_tokens, "prompt", device=dev)
    table = synth.block_table(cfg, T, device=dev) if cfg.paged else None
    cache = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, dev, paged=cfg.paged,
                        block_size=cfg.block_size, block_table=table,
                        n_blocks=(int(table.max()) + 1) if table is not None else None)
    direct = Filler(fw, cfg.rope_base, T, cfg.fill_chunk, dev, ws_slots=8)
    composed = ComposedFiller(fw, cfg.rope_base, T, cfg.fill_chunk, dev)

    def runner(filler):
        def run():
            for c0 in range(cfg.fill_t0, cfg.fill_t1, cfg.fill_chunk):
                c1 = min(cfg.fill_t1, c0 + cfg.fill_chunk)
                filler.fill(X[c0 - cfg.fill_t0:c1 - cfg.fill_t0], c0, c1, 0, cache, stream)
        return run

    fns = [runner(composed), runner(direct)]
    if streamed:
        # the maps in page-locked host memory, one call over the whole range: each map crosses
        # the host link once, the range is filled in steps of the workload's chunk inside each
        # ring slot (rf_fill_streamed with rows_per_fill)
        import dataclasses

        from linear_kv_cache_amd.runner import StreamedFiller, pinned_copy
        sw = dataclasses.replace(fw, W_map=[pinned_copy(W.cpu()) for W in fw.W_map])
        sf = StreamedFiller(sw, cfg.rope_base, T, cfg.fill_chunk, dev, ring_slots=2, layers_per_slot=2,
                            rows_per_fill=cfg.fill_chunk)
        fns.append(lambda: sf.fill(X, cfg.fill_t0, cfg.fill_t1, 0, cache, stream))
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    meds = alternate(stream, fns, steps)
    med, med_direct = meds[0], meds[1]
    alg = cfg.fill_tokens * len(layers) * cfg.fill_flop_per_token_layer()
    exe = cfg.fill_tokens * len(layers) * composed_flop_per_token_layer(cfg.d, cfg.kv_width)
    print(json.dumps({"metric": "filled tokens/sec (all filled layers) + % bf16 MFMA peak, fill only",
                      "config": {"workload": cfg.name, "d": cfg.d, "filled_layers": len(layers),
                                 "fill_tokens": cfg.fill_tokens, "fill_chunk": cfg.fill_chunk, "paged": cfg.paged},
                      "steps": steps, "warmup": warmup, "path": "composed (rf_fill_composed)",
                      "ms_median": round(med, 3), "tokens_per_s": round(cfg.fill_tokens / (med / 1e3), 1),
                      "frac_bf16_peak": round(alg / (med / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                      "flop_per_token_layer": cfg.fill_flop_per_token_layer(),
                      "executed_flop_per_token_layer": composed_flop_per_token_layer(cfg.d, cfg.kv_width),
                      "executed_frac_bf16_peak": round(exe / (med / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                      "cache_write_GBps": round(cfg.fill_tokens * len(layers) * 4 * cfg.kv_width / (med / 1e3) / 1e9,
                                                1),
                      "direct": {"ms_median": round(med_direct, 3),
                                 "tokens_per_s": round(cfg.fill_tokens / (med_direct / 1e3), 1),
                                 "frac_bf16_peak": round(alg / (med_direct / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
                      **({"streamed": {"what": "rf_fill_streamed, one call, maps in page-locked host memory "
                                               "(2 slots x 2 layers), steps of the workload's chunk",
                                       "ms_median": round(meds[2], 3),
                                       "tokens_per_s": round(cfg.fill_tokens / (meds[2] / 1e3), 1),
                                       "vs_resident_direct": round(med_direct / meds[2], 4)}} if streamed else {})}),
          flush=True)


def fit_only(cfg, steps: int, warmup: int):
    """``--fit-only``: time the fit alone on a configuration (e.g. the fit-heavy C4: every
    calibration chunk through rf_gram_accumulate, then one rf_solve per lambda of the
    configuration on the shared state) and print one JSON line for it."""
    import torch

    import linear_kv_cache_amd as rf
    import synth
    from linear_kv_cache_amd.runner import GramState, device_bytes

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    L, d = cfg.n_targets, cfg.d
    layers = [cfg.split + l for l in range(L)]
    n_chunks = cfg.calib_rows // cfg.calib_chunk
    log(f"fit-only workload {cfg.name}: d={d} targets={L} N={cfg.calib_rows} in {n_chunks} chunks, "
        f"lambdas={cfg.lambdas}; drawing inputs on the GPU")
    Xc = [synth.hidden_states(cfg, cfg.calib_chunk, "calib", chunk=c, device=dev) for c in range(n_chunks)]
    Yc = [[synth.late_layer_inputs(cfg, Xc[c], l, chunk=c) for l in layers] for c in range(n_chunks)]
    state = GramState(d, L, cfg.torch_dtype, dev)
    nl = len(cfg.lambdas)
    ws = device_bytes(rf.rf_solve_workspace_bytes(state.desc, L, nl), dev)
    W_lp = torch.empty(nl, L, d, d, dtype=torch.bfloat16, device=dev)
    b = torch.empty(nl, L, d, dtype=torch.float32, device=dev)
    info = torch.empty(nl, dtype=torch.int32, device=dev)
    cond = torch.empty(nl, dtype=torch.float64, device=dev)

    def step():
        # every lambda of the workload in one rf_solve call on the shared state
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        rf.rf_gram_init(state.desc, state.buf, stream)
        for c in range(n_chunks):
            rf.rf_gram_accumulate(state.desc, state.buf, Xc[c], Yc[c], stream=stream)
        ev[1].record(stream)
        rf.rf_solve(state.desc, state.buf, list(cfg.lambdas), rf.RF_LAMBDA_ABSOLUTE, list(range(L)), None, W_lp, b,
                    info, ws, stream, cond=cond)
        ev[2].record(stream)
        return ev

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if rf.rf_info_status(info.cpu().tolist()) != rf.RF_OK:
        raise SystemExit(f"solve reported a non-positive pivot: {rf.rf_last_error()}")
    recs = []
    for _ in range(steps):
        recs.append(step())
        torch.cuda.synchronize()
    gram = statistics.median(r[0].elapsed_time(r[1]) for r in recs)
    solves = [statistics.median(r[1].elapsed_time(r[2]) for r in recs)]
    # the batched call against one lambda alone, alternated on the same state
    ws1 = device_bytes(rf.rf_solve_workspace_bytes(state.desc, L, 1), dev)
    mid = cfg.lambdas[len(cfg.lambdas) // 2]
    one, alln = alternate(stream, [
        lambda: rf.rf_solve(state.desc, state.buf, mid, rf.RF_LAMBDA_ABSOLUTE, list(range(L)), None, W_lp[0], b[0],
                            info[:1], ws1, stream),
        lambda: rf.rf_solve(state.desc, state.buf, list(cfg.lambdas), rf.RF_LAMBDA_ABSOLUTE, list(range(L)), None,
                            W_lp, b, info, ws, stream)], max(steps, 3))
    del ws1
    tflops = cfg.calib_rows * cfg.fit_flop_per_row() / (gram / 1e3) / 1e12
    print(json.dumps({"metric": "ridge-fit rows/sec, fit only",
                      "config": {"workload": cfg.name, "d": d, "targets": L, "calib_rows": cfg.calib_rows,
                                 "calib_chunk": cfg.calib_chunk, "lambdas": list(cfg.lambdas)},
                      "steps": steps, "warmup": warmup, "gram_ms_median": round(gram, 3),
                      "rows_per_s": round(cfg.calib_rows / (gram / 1e3), 1), "gram_tflops": round(tflops, 1),
                      "gram_frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
                      "solve_ms_median_all_lambdas": round(solves[0], 3),
                      "solve_alternated": {"one_lambda_ms": round(one, 3), "all_lambdas_ms": round(alln, 3),
                                           "ratio": round(alln / one, 3), "lambda_alone": mid},
                      "equilibrated_inverse_max": [round(float(x), 4) for x in cond.cpu().tolist()],
                      "rows_per_s_incl_solves": round(cfg.calib_rows / ((gram + sum(solves)) / 1e3), 1),
                      "flop_per_row": cfg.fit_flop_per_row()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16384)
    ap.add_argument("--cpu-fit-rows", type=int, default=8192)
    ap.add_argument("--cpu-translate-tokens", type=int, default=4096)
    ap.add_argument("--library-reference", action="store_true",
                    help="also time the fill's two products per layer as plain torch.matmul (hipBLASLt) "
                         "GEMMs on the same maps, projections and prompt states")
    ap.add_argument("--no-translate", action="store_true", help="skip the cache-translator leg")
    ap.add_argument("--no-streamed", action="store_true", help="skip the streamed-maps leg")
    ap.add_argument("--no-gdn", action="store_true", help="skip the Gated DeltaNet state-update leg")
    ap.add_argument("--streamed", action="store_true",
                    help="with --fill-only: also time the fill with streamed maps over the whole range in one call")
    ap.add_argument("--fill-only", action="store_true",
                    help="time the fill alone over --config's filled range (e.g. C3, C5) and print its own line")
    ap.add_argument("--fit-only", action="store_true",
                    help="time the fit alone on --config (e.g. C4: all chunks, one solve per lambda) and print "
                         "its own line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one 1 GiB device-to-device copy before the steps, a known-size reference "
                         "for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the fit and fill run on a single MI355X; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_kv_cache_amd as rf
    import synth
    from linear_kv_cache_amd.runner import (ComposedFiller, Filler, GramState, alloc_cache, compose_weights,
                                            device_bytes, pack_weights)

    cfg = synth.CONFIGS[args.config]
    if args.fill_only:
        fill_only(cfg, args.steps, args.warmup, streamed=args.streamed)
        return
    if args.fit_only:
        fit_only(cfg, args.steps, args.warmup)
        return
    if cfg.calib_rows == 0 or cfg.fill_tokens == 0 or cfg.dtype != "bf16":
        raise SystemExit(f"{args.config} is a parity-test configuration, not a bench workload "
                         "(the bench times the bf16 fit-then-fill pipeline)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    d, L, T = cfg.d, cfg.n_targets, cfg.fill_tokens
    n_chunks = cfg.calib_rows // cfg.calib_chunk
    log(f"workload {cfg.name}: d={d} layers={L} N={cfg.calib_rows} T={T}; drawing inputs on the GPU")
    Xc = [synth.hidden_states(cfg, cfg.calib_chunk, "calib", chunk=c, device=dev) for c in range(n_chunks)]
    Yc = [[synth.late_layer_inputs(cfg, Xc[c], l, chunk=c) for l in cfg.filled_layers] for c in range(n_chunks)]
    Xp = synth.hidden_states(cfg, T, "prompt", device=dev)
    kv = [synth.kv_weights(cfg, l, device=dev) for l in cfg.filled_layers]
    state = GramState(d, L, cfg.torch_dtype, dev)
    solve_ws = device_bytes(rf.rf_solve_workspace_bytes(state.desc, L), dev)
    W_lp = torch.empty(L, d, d, dtype=torch.bfloat16, device=dev)
    b = torch.empty(L, d, dtype=torch.float32, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    cache = alloc_cache(L, cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, dev)
    # the K/V projections are model weights: packed once at load (rf_solve writes W_lp packed)
    fw = rf.FillWeights(d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [W_lp[i] for i in range(L)],
                        [b[i] for i in range(L)], [g for (_, _, g) in kv],
                        [pack_weights(k, cfg.head_dim) for (k, _, _) in kv],
                        [pack_weights(v, cfg.head_dim) for (_, v, _) in kv])
    filler = Filler(fw, cfg.rope_base, T, T, dev, ws_slots=8)   # 8 layers per fill launch (1 GiB of H)
    # the composed weights' buffers; rf_fill_compose rewrites them from each step's maps
    cw = compose_weights(fw, slots=L)
    compose_ws = device_bytes(rf.rf_fill_compose_workspace_bytes(fw) * L, dev)
    cfiller = ComposedFiller(fw, cfg.rope_base, T, T, dev, composed=cw)
    lam = cfg.lambdas[0]
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: 1 GiB device-to-device copy (1048576 KiB read, 1048576 KiB written)")
        del src, dst
    torch.cuda.synchronize()

    def step():
        ev = {k: torch.cuda.Event(enable_timing=True) for k in ("start", "gram", "solve", "compose", "fill")}
        gram_ev = []
        ev["start"].record(stream)
        rf.rf_gram_init(state.desc, state.buf, stream)
        for c in range(n_chunks):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rf.rf_gram_accumulate(state.desc, state.buf, Xc[c], Yc[c], stream=stream)
            e1.record(stream)
            gram_ev.append((e0, e1))
        ev["gram"].record(stream)
        rf.rf_solve(state.desc, state.buf, lam, rf.RF_LAMBDA_ABSOLUTE, list(range(L)), None, W_lp, b, info,
                    solve_ws, stream)
        ev["solve"].record(stream)
        rf.rf_fill_compose(fw, cw, compose_ws, stream)
        ev["compose"].record(stream)
        cfiller.fill(Xp, 0, T, 0, cache, stream)
        ev["fill"].record(stream)
        return ev, gram_ev

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    if int(info.item()) != 0:
        raise SystemExit(f"solve reported a non-positive pivot: {int(info.item())}")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")

    gram_ms = [r[0]["start"].elapsed_time(r[0]["gram"]) for r in recs]
    solve_ms = [r[0]["gram"].elapsed_time(r[0]["solve"]) for r in recs]
    compose_ms = [r[0]["solve"].elapsed_time(r[0]["compose"]) for r in recs]
    fill_ms = [r[0]["compose"].elapsed_time(r[0]["fill"]) for r in recs]
    launch_ms = [e0.elapsed_time(e1) for r in recs for (e0, e1) in r[1]]
    fill_flop = T * L * cfg.fill_flop_per_token_layer()
    gram_flop_per_launch = cfg.calib_chunk * cfg.fit_flop_per_row()
    fill_s = sum(fill_ms) / 1e3
    tok_s = T * args.steps / fill_s
    fill_tflops = fill_flop * args.steps / fill_s / 1e12
    exe_flop_tl = composed_flop_per_token_layer(d, cfg.kv_width)
    exe_tflops = T * L * exe_flop_tl * args.steps / fill_s / 1e12
    gram_launch_ms = statistics.mean(launch_ms)
    gram_tflops = gram_flop_per_launch / (gram_launch_ms / 1e3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "filled tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "d": d, "filled_layers": L, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "fill_tokens": T, "calib_rows": cfg.calib_rows,
                   "calib_chunk": cfg.calib_chunk, "lambda": lam},
        "fill": {"path": "composed maps (rf_fill_composed); algorithmic FLOP as the method's two products",
                 "ms": round(statistics.mean(fill_ms), 3), "ms_median": round(statistics.median(fill_ms), 3),
                 "tokens_per_s": round(tok_s, 1),
                 "tflops": round(fill_tflops, 1), "frac_bf16_peak": round(fill_tflops / BF16_PEAK_TFLOPS, 4),
                 "flop_per_token_layer": cfg.fill_flop_per_token_layer(),
                 "executed_flop_per_token_layer": exe_flop_tl, "executed_tflops": round(exe_tflops, 1),
                 "executed_frac_bf16_peak": round(exe_tflops / BF16_PEAK_TFLOPS, 4),
                 # bf16 K and V rows written to the caches: 2 * H_kv * d_h * 2 B per token-layer
                 "cache_write_GBps": round(T * L * 4 * cfg.n_kv_heads * cfg.head_dim * args.steps / fill_s / 1e9, 1)},
        "fit": {"rows_per_s": round(cfg.calib_rows / (statistics.mean(gram_ms) / 1e3), 1),
                "gram_ms": round(statistics.mean(gram_ms), 3), "solve_ms": round(statistics.mean(solve_ms), 3),
                "compose_ms": round(statistics.mean(compose_ms), 3),
                "gram_ms_median": round(statistics.median(gram_ms), 3),
                "solve_ms_median": round(statistics.median(solve_ms), 3),
                "rows_per_s_incl_solve": round(cfg.calib_rows / ((statistics.mean(gram_ms) +
                                                                   statistics.mean(solve_ms)) / 1e3), 1),
                "flop_per_row": cfg.fit_flop_per_row()},
        "roofline": {"bound": "mfma",
                     "kernel": f"rf_gram_accumulate of {cfg.calib_chunk} rows x {L} targets "
                               f"(k_gram_pipe, column sums in its last work-groups)",
                     "achieved": round(gram_tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gram_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": gram_traffic() if args.config == "C2" else None,
                     "launch_ms": round(gram_launch_ms, 4), "flop_per_launch": gram_flop_per_launch},
    }
    if args.library_reference:
        # the same maps in plain layout: the solve's fp32 output rounded to bf16, as its packed
        # bf16 output is; the same unpacked projections and prompt states
        W32 = torch.empty(L, d, d, dtype=torch.float32, device=dev)
        rf.rf_solve(state.desc, state.buf, lam, rf.RF_LAMBDA_ABSOLUTE, list(range(L)), W32, None, b, info,
                    solve_ws, stream)
        Wt = [W32[i].to(torch.bfloat16).t().contiguous() for i in range(L)]
        del W32
        Wkv = [torch.cat([k, v]).t().contiguous() for (k, v, _) in kv]
        H = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
        KV = torch.empty(T, Wkv[0].shape[1], dtype=torch.bfloat16, device=dev)

        def library_fill():
            for i in range(L):
                torch.matmul(Xp, Wt[i], out=H)
                torch.matmul(H, Wkv[i], out=KV)

        def timed(fn):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        library_fill()
        torch.cuda.synchronize()
        # alternate the two so both see the same clock and power state
        lib_ms, fused_ms = [], []
        for _ in range(args.steps):
            fused_ms.append(timed(lambda: filler.fill(Xp, 0, T, 0, cache, stream)))
            lib_ms.append(timed(library_fill))
        ms, fms = statistics.median(lib_ms), statistics.median(fused_ms)
        out["library_reference"] = {
            "what": "torch.matmul (hipBLASLt) of the fill's map and K/V products per layer, no norm, RoPE or "
                    "cache write, same data; alternated with the fused fill",
            "ms_median": round(ms, 3), "tflops": round(fill_flop / (ms / 1e3) / 1e12, 1),
            "frac_bf16_peak": round(fill_flop / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "fused_fill_ms_median": round(fms, 3),
            "fused_fill_frac_bf16_peak": round(fill_flop / (fms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del Wt, Wkv, H, KV
        # the Gram's products as one library GEMM on the same chunk: [X | Y_1 .. Y_L]^T X, the
        # shape of a linear layer's weight gradient (both operands row-major over the rows, the
        # left one read through a transposed view), full square, bf16 output
        XY = torch.cat([Xc[0]] + list(Yc[0]), dim=1)
        G = torch.empty(d, XY.shape[1], dtype=torch.bfloat16, device=dev)
        lib_gram_flop = 2 * cfg.calib_chunk * d * XY.shape[1]

        def library_gram():
            torch.matmul(Xc[0].t(), XY, out=G)

        library_gram()
        torch.cuda.synchronize()
        lib_g, ours_g = [], []
        for _ in range(args.steps):
            ours_g.append(timed(lambda: rf.rf_gram_accumulate(state.desc, state.buf, Xc[0], Yc[0],
                                                              stream=stream)))
            lib_g.append(timed(library_gram))
        gms, oms = statistics.median(lib_g), statistics.median(ours_g)
        out["library_reference"]["gram"] = {
            "what": f"torch.matmul (hipBLASLt) of X^T [X | Y] over one {cfg.calib_chunk}-row chunk, full square, "
                    "bf16 output, no fp32 accumulation into a state or column sums; alternated with "
                    "rf_gram_accumulate on the same chunk",
            "ms_median": round(gms, 3), "tflops": round(lib_gram_flop / (gms / 1e3) / 1e12, 1),
            "frac_bf16_peak": round(lib_gram_flop / (gms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "ours_ms_median": round(oms, 3),
            "ours_frac_bf16_peak": round(gram_flop_per_launch / (oms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del XY, G
    # the direct fill on the same maps, alternated with the composed one
    log("direct fill (rf_fill) alternated with the composed fill")
    cms, dms = alternate(stream, [lambda: cfiller.fill(Xp, 0, T, 0, cache, stream),
                                  lambda: filler.fill(Xp, 0, T, 0, cache, stream)], args.steps)
    out["fill_direct"] = {"what": "rf_fill (map product, RMSNorm, K/V product, RoPE, cache write) on the same maps, "
                                  "alternated with rf_fill_composed",
                          "ms_median": round(dms, 3), "tokens_per_s": round(T / (dms / 1e3), 1),
                          "frac_bf16_peak": round(fill_flop / (dms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                          "composed_ms_median": round(cms, 3), "composed_speedup": round(dms / cms, 4)}
    # the solve's accuracy on this workload: the largest entry of the equilibrated inverse and
    # the fp64 stationarity residual of the fp32 maps (one extra call, outside the timed steps)
    _, _, _, info_r, cond_r, resid_r = state.solve_many([lam], rf.RF_LAMBDA_ABSOLUTE, list(range(L)), want_bf16=False,
                                                        want_resid=True)
    torch.cuda.synchronize()
    out["fit"]["equilibrated_inverse_max"] = round(float(cond_r[0].item()), 4)
    out["fit"]["product_route"] = "fp64" if float(cond_r[0].item()) > rf.RF_SPLIT_COND_MAX else "split bf16"
    out["fit"]["stationarity_residual_max"] = float(resid_r.max().item())
    del cond_r, resid_r
    if not args.no_streamed:
        log("streamed maps: the fill with its maps in page-locked host memory (bf16, then int8)")
        # the fp32 maps of one more solve (outside the timed steps) feed the int8 quantiser
        W32 = torch.empty(L, d, d, dtype=torch.float32, device=dev)
        rf.rf_solve(state.desc, state.buf, lam, rf.RF_LAMBDA_ABSOLUTE, list(range(L)), W32, None, b, info,
                    solve_ws, stream)
        out["fill_streamed"] = streamed_leg(args.steps, stream, dev, cfg, fw, Xp, cache, filler,
                                            w32=[W32[i] for i in range(L)])
        del W32
    if not args.no_translate:
        del Xc, Yc
        out["translate"] = translate_leg(args.steps, stream, dev)
        out["translate_headwise"] = translate_leg(args.steps, stream, dev,
                                                  synth.scaled(synth.TR_BENCH, maps="headwise",
                                                               name=synth.TR_BENCH.name + "-headwise"))
    if not args.no_gdn:
        out["gdn_state"] = gdn_leg(args.steps, stream, dev)
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_tokens} tokens and {args.cpu_fit_rows} calibration rows")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens, args.cpu_fit_rows)
        if not args.no_translate:
            log(f"timing the CPU oracle's translation of {args.cpu_translate_tokens} tokens")
            out["cpu_baseline"]["translate_tokens_per_s"] = cpu_translate_baseline(args.cpu_translate_tokens)
            out["cpu_baseline"]["sample"] += (f"; translate tokens/s from {args.cpu_translate_tokens} tokens x "
                                              f"{synth.TR_BENCH.n_tgt} target layers")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
