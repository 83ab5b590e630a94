#!/usr/bin/env python3
"""Benchmark: top-k block-sparse decode on one MI355X.

One step = one layer's decode step of the 70B-shaped 128K workload: the
query heads of layer l attend to their selected blocks, and the indexer
vectors of layer l score layer l+1's compressed keys and pick its blocks
(top-k), both in one sda_decode_step call: a scoring launch leaves per-chunk
candidate lists, and the decode launch merges them into layer l+1's block
sets (--step separate: sda_score_select then sda_sparse_decode).  Steps
walk a ring of distinct layers whose K/V, compressed keys and vectors are
all resident in HBM, so every step reads cold data as a real layer stack
does (the ring of 8 layers touches 0.86 GB per pass, well beyond the L2 and
Infinity caches together).

Prints one JSON line.  `value` is whole-job queries/s over the timed steps
(one query = one sequence's decode token); `roofline` prices the step's one
launch against the 8 TB/s HBM peak on its algorithmic bytes (layer l's
selected K/V blocks plus layer l+1's compressed keys), `roofline_decode`
the decode launch alone (sda_sparse_decode, selected K/V bytes); `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload; `rows` measures the other
rows of the hot path (compressed-key build and per-token refresh, the G-head
comparator, grouped verification decode, offloaded gather) at their own
workloads, each against its roofline with the oracle timed beside it.

  python bench.py [--steps K] [--warmup W] [--config 3] [--layers L]
  python bench.py --copy-calibration     (plain copy of known size, for counter scaling)
"""
import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_attention_pool_amd as sda  # noqa: E402
import synth  # noqa: E402
from synth import inputs  # noqa: E402

METRIC = "sparse-decode queries/s + achieved HBM GB/s (% of peak) at 128K ctx"
HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "decode_c3_counters.json")
# sources of the measured kernels: counters taken on other sources are stale
KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_pool_amd", "csrc", f)
               for f in ("k_attention.hip", "sda_select_dev.hpp", "sda_internal.h", "sda_device.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build_layers(cfg, n_layers, dev):
    """K, V, compressed keys, indexer vectors and queries for a ring of layers."""
    layers = []
    for l in range(n_layers):
        t0 = time.time()
        # the 8B-shaped workload biases 5 % of each row's blocks along the
        # direction of the indexer vectors that select them (the previous
        # layer's in the ring: layer l-1's vectors score layer l's keys)
        dirs = (inputs.bias_directions(inputs.indexer_vectors(cfg, (l - 1) % n_layers)) if cfg.bias_frac > 0
                else None)
        K, V, _ = inputs.kv_layer(cfg, l, device=dev, bias_dirs=dirs)
        kt = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
        lo = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
        hi = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=dev)
        sda.sda_update_compressed_keys(K, kt, lo, hi, cfg.T)
        F = inputs.to_bf16(inputs.indexer_vectors(cfg, l), dev)
        Q = inputs.to_bf16(inputs.attention_queries(cfg, l), dev)
        torch.cuda.synchronize()
        layers.append(dict(K=K, V=V, kt=kt, F=F, Q=Q))
        log(f"layer {l}: K/V {2 * K.numel() * 2 / 1e9:.2f} GB drawn, compressed keys built "
            f"({time.time() - t0:.1f} s)")
    return layers


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Worker threads for the CPU baseline: the cores this process may run
    on, capped at the GPU's host CPU share (16)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


_CPU_ROW = {}


def _cpu_row_init(cid, b, g, n_layers):
    """Worker set-up (untimed): one (batch, KV head) row of the workload with
    its keys and values drawn on the host (N(0,1), rounded to bf16: the
    workload's distributions; the GPU run's device draws are not reproduced
    here), the oracle's compressed keys of it, and the row's indexer vectors
    of every ring layer and its query heads (the same host draws the GPU run uses)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        _CPU_ROW["limiter"] = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    torch.set_num_threads(1)
    cfg = synth.get_config(cid)
    rng = np.random.Generator(np.random.PCG64(inputs.derive_seed(cid, "cpu_baseline_kv", b, g)))
    kv = [O.bf16_to_f64(inputs.bf16_bits(inputs.to_bf16(rng.standard_normal((cfg.T, cfg.d), dtype=np.float32))))
          for _ in range(2)]
    _CPU_ROW.update(cfg=cfg, k=kv[0], v=kv[1], kt=O.store_bf16(O.compressed_keys(kv[0], cfg.T)),
                    f=[O.bf16_to_f64(inputs.bf16_bits(inputs.to_bf16(inputs.indexer_vectors(cfg, l)[b, 0, g])))
                       for l in range(n_layers)],
                    q=O.bf16_to_f64(inputs.bf16_bits(inputs.to_bf16(
                        inputs.attention_queries(cfg, 1)[b, 0, g * cfg.G:(g + 1) * cfg.G]))))


def _cpu_row_run(budget_s):
    """Repeat the oracle's per-step work on this worker's row (scores, top-k,
    block set, attention of the row's query heads), one ring layer's indexer
    vector after another, for about budget_s seconds; returns (row-steps, seconds)."""
    import oracle as O
    r = _CPU_ROW
    cfg = r["cfg"]
    scale = 1.0 / math.sqrt(cfg.d)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        blocks, _ = O.select_row(r["f"][done % len(r["f"])], r["kt"], cfg.n_init, cfg.n_local, cfg.top_k)
        O.decode_row(r["q"], r["k"], r["v"], blocks, cfg.T, scale)
        done += 1
    return done, time.perf_counter() - t0


def cpu_baseline(cfg, n_layers, budget_s=12.0):
    """Time the CPU oracle's per-step work on a sample of the workload: one
    (batch, KV head) row per worker process, all workers at once for about
    budget_s seconds.  Called before the process touches the GPU, so the
    workers are plain forks of a process without GPU state."""
    import multiprocessing as mp
    nthr = cpu_threads()
    rows = [(b, g) for b in range(cfg.B) for g in range(cfg.H_kv)][:nthr]
    ctx = mp.get_context("fork")
    pools = [ctx.Pool(1, initializer=_cpu_row_init, initargs=(cfg.cid, b, g, n_layers)) for (b, g) in rows]
    try:
        for p in pools:                                    # set-up finished everywhere before timing
            p.apply(time.time)
        t0 = time.perf_counter()
        res = [p.apply_async(_cpu_row_run, (budget_s,)) for p in pools]
        got = [r.get() for r in res]
        wall = time.perf_counter() - t0
    finally:
        for p in pools:
            p.terminate()
    done = sum(d for d, _ in got)
    return {
        "value": done / wall / cfg.H_kv,
        "unit": "queries/s",
        "cores": len(rows),
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": f"{len(rows)} (batch, KV head) rows of the {cfg.T // 1024}K workload, one per worker process "
                  f"({len(rows)} of the {len(os.sched_getaffinity(0))} cores the process may use, capped at the "
                  f"GPU's 16-core host share), {done} row-steps in {wall:.1f} s of wall time; float64 NumPy, one "
                  f"BLAS thread per worker; per row-step: scores, top-k, block set, attention of {cfg.G} heads "
                  f"(indexer vectors of each ring layer in turn); keys and values drawn on the host with the "
                  f"workload's distributions; a query = one sequence's {cfg.H_kv} KV heads",
    }


# ---------------------------------------------------------------------------
# the other rows of the hot path, each at its own workload
# ---------------------------------------------------------------------------

def graph_time(fn, reps=30, copies=8):
    """Mean device seconds per call of fn (which must not allocate), from a
    graph of `copies` calls replayed `reps` times between two HIP events."""
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        fn()
    torch.cuda.current_stream().wait_stream(warm)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(copies):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * copies)


def eager_time(fn, reps=10):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def oracle_time(fn, budget_s=1.5):
    """Seconds per call of an oracle function (one thread), repeated for about budget_s."""
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    n, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        fn()
        t += time.perf_counter() - t0
        n += 1
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    return t / n


def hbm(nbytes, sec):
    gbs = nbytes / sec / 1e9
    return {"achieved_gbs": gbs, "peak_gbs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
            "algorithmic_bytes": int(nbytes)}


ROW_NAMES = ("a1", "a7", "c2", "prefill", "pooled", "grouped", "chain", "offload")


def measure_rows(cfg, layers, only=None):
    """The other rows of the hot path, each timed on the GPU against its
    roofline with the CPU oracle timed beside it on a small sample (`only`:
    a subset of ROW_NAMES)."""
    import oracle as O
    dev = "cuda"
    rows = {}
    want = set(only or ROW_NAMES)
    T, d, G = cfg.T, cfg.d, cfg.G
    scale = 1.0 / math.sqrt(d)
    ln = layers[1 % len(layers)]

    # a1: compressed keys of one 128K layer (bulk build) and the per-token refresh
    kt = torch.zeros_like(ln["kt"])
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    full = torch.full((cfg.B,), T, dtype=torch.int32, device=dev)
    prev = torch.full((cfg.B,), T - 1, dtype=torch.int32, device=dev)
    kk = O.bf16_to_f64(inputs.bf16_bits(ln["K"][0, 0]))
    nrow = cfg.B * cfg.H_kv
    if "a1" in want:
        t_build = eager_time(lambda: sda.sda_update_compressed_keys(ln["K"], kt, zero, full, T), reps=5)
        t_tok = graph_time(lambda: sda.sda_update_compressed_keys(ln["K"], kt, prev, full, 1))
        t_or = oracle_time(lambda: O.store_bf16(O.compressed_keys(kk, T)))
        rows["a1_compressed_keys"] = {
            "workload": f"{cfg.name}: K~ of {nrow} (batch, KV head) rows x {cfg.NB} blocks",
            "build_us": t_build * 1e6, "build_roofline": hbm(cfg.B * cfg.H_kv * T * d * 2 + cfg.ktilde_bytes(), t_build),
            "per_token_update_us": t_tok * 1e6,
            "per_token_update_roofline": hbm(nrow * (64 * d * 2 + d * 2), t_tok),
            "oracle_rows_per_s": 1.0 / t_or, "gpu_rows_per_s": nrow / t_build,
        }

    if "a7" in want:
        # a7: the G-head comparator selector on the same layer
        nsm = cfg.n_init + cfg.n_local + cfg.top_k
        bi = torch.empty((cfg.B, 1, cfg.H_kv, nsm), dtype=torch.int32, device=dev)
        ns = torch.empty((cfg.B, 1, cfg.H_kv), dtype=torch.int32, device=dev)
        wsm = torch.zeros(sda.lib().sda_score_select_multihead_workspace(cfg.B, 1, cfg.H_q, cfg.H_kv, cfg.NB,
                                                                        cfg.top_k), dtype=torch.uint8, device=dev)
        tau = math.sqrt(d)
        # one call per resident layer in turn (8 x 33.5 MB of compressed keys: the
        # working set exceeds the 256 MB Infinity Cache, so every call reads HBM)
        L = len(layers)
        turn = [0]

        def mh_call():
            lay = layers[turn[0] % L]
            turn[0] += 1
            sda.sda_score_select_multihead(lay["Q"], lay["kt"], full, cfg.n_init, cfg.n_local, cfg.top_k, tau,
                                           block_idx=bi, n_sel=ns, ws=wsm)
        t_mh = graph_time(mh_call, copies=L)
        Qd = O.bf16_to_f64(inputs.bf16_bits(ln["Q"][0, 0, :G]))
        ktd = O.store_bf16(O.compressed_keys(kk, T))
        t_or = oracle_time(lambda: O.select_row_multihead(Qd, ktd, cfg.n_init, cfg.n_local, cfg.top_k, tau))
        wss = torch.zeros(sda.lib().sda_score_select_workspace(cfg.B, 1, cfg.H_kv, cfg.NB, cfg.top_k),
                          dtype=torch.uint8, device=dev)
        turn[0] = 0

        def sel_call():
            lay = layers[turn[0] % L]
            turn[0] += 1
            sda.sda_score_select(lay["F"], lay["kt"], full, cfg.n_init, cfg.n_local, cfg.top_k, block_idx=bi,
                                 n_sel=ns, ws=wss)
        t_fc = graph_time(sel_call, copies=L)
        rows["a7_comparator"] = {
            "workload": f"{cfg.name}: G = {G} heads per KV group, tau = sqrt(d)",
            "us": t_mh * 1e6, "roofline": hbm(cfg.ktilde_bytes(), t_mh),
            "forecast_select_us": t_fc * 1e6, "g_head_over_forecast": t_mh / t_fc,
            "oracle_rows_per_s": 1.0 / t_or, "gpu_rows_per_s": nrow / t_mh,
        }
    if "c2" in want:
        rows["c2_step"] = measure_step_config(2)
    if "prefill" in want:
        rows["n2_prefill"] = measure_prefill(2)
    if "pooled" in want:
        rows["n1_pooled_select"] = measure_pooled(cfg, layers, O, full, prev)
    if "grouped" in want:
        rows["a5_grouped"] = measure_grouped(O)
    if "chain" in want:
        rows["n3_refresh_reuse"] = measure_chain()
    if "offload" in want:
        rows["a6_offload"] = measure_offload(O)
    return rows


def measure_step_config(cid, n_layers=8):
    """The decode step (sda_decode_step: layer l's decode and layer l+1's
    scoring and selection in one launch) at another workload, over a ring of
    resident layers like the headline, and the two calls it replaces."""
    cfg = synth.get_config(cid)
    dev = "cuda"
    layers = build_layers(cfg, n_layers, dev)
    L = len(layers)
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=dev)
    nsm = cfg.n_init + cfg.n_local + cfg.top_k
    bi = [torch.empty((cfg.B, 1, cfg.H_kv, nsm), dtype=torch.int32, device=dev) for _ in range(L)]
    ns = [torch.empty((cfg.B, 1, cfg.H_kv), dtype=torch.int32, device=dev) for _ in range(L)]
    for i in range(L):
        sda.sda_score_select(layers[(i - 1) % L]["F"], layers[i]["kt"], seq, cfg.n_init, cfg.n_local, cfg.top_k,
                             block_idx=bi[i], n_sel=ns[i])
    out = torch.empty((cfg.B, 1, cfg.H_q, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, 1, cfg.H_q), dtype=torch.float32, device=dev)
    ws = torch.zeros(sda.lib().sda_decode_step_workspace(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, nsm, 0, cfg.NB,
                                                         cfg.top_k), dtype=torch.uint8, device=dev)
    ws_sel = torch.zeros(sda.lib().sda_score_select_workspace(cfg.B, 1, cfg.H_kv, cfg.NB, cfg.top_k),
                         dtype=torch.uint8, device=dev)
    ws_dec = torch.zeros(max(16, sda.lib().sda_sparse_decode_workspace(cfg.B, 1, cfg.H_q, cfg.H_kv, nsm, cfg.d, 0)),
                         dtype=torch.uint8, device=dev)
    steps, sels, decs = [], [], []
    for i in range(L):
        lc, ln = layers[i], layers[(i + 1) % L]
        pc, _ = sda.prepare(sda.sda_decode_step, lc["Q"], lc["K"], lc["V"], seq, bi[i], ns[i], lc["F"], ln["kt"],
                            seq, cfg.n_init, cfg.n_local, cfg.top_k, block_idx_next=bi[(i + 1) % L],
                            n_sel_next=ns[(i + 1) % L], out=out, lse=lse, ws=ws)
        steps.append(pc)
        sc, _ = sda.prepare(sda.sda_score_select, lc["F"], ln["kt"], seq, cfg.n_init, cfg.n_local, cfg.top_k,
                            block_idx=bi[(i + 1) % L], n_sel=ns[(i + 1) % L], ws=ws_sel)
        dc, _ = sda.prepare(sda.sda_sparse_decode, lc["Q"], lc["K"], lc["V"], seq, bi[i], ns[i], out=out, lse=lse,
                            ws=ws_dec)
        sels.append(sc)
        decs.append(dc)
    t_step = call_time(steps, 30)
    t_sel = call_time(sels, 30)
    t_dec = call_time(decs, 30)
    step_bytes = cfg.selected_kv_bytes() + cfg.ktilde_bytes()
    res = {
        "workload": f"{cfg.name}: B={cfg.B}, H_q={cfg.H_q}, H_kv={cfg.H_kv}, d={cfg.d}, T={cfg.T}, "
                    f"{cfg.n_init} init + {cfg.n_local} local + top-{cfg.top_k}, 5 % of blocks biased along "
                    f"the indexer direction, ring of {L} resident layers",
        "step_us": t_step * 1e6, "step_roofline": hbm(step_bytes, t_step),
        "queries_per_s": cfg.B / t_step,
        "score_select_us": t_sel * 1e6, "score_select_roofline": hbm(cfg.ktilde_bytes(), t_sel),
        "sparse_decode_us": t_dec * 1e6, "sparse_decode_roofline": hbm(cfg.selected_kv_bytes(), t_dec),
    }
    del layers
    torch.cuda.empty_cache()
    return res


def measure_prefill(cid=2):
    """Prefill of a whole 32K sequence at the 8B-shaped layer (B 8, H_q 32,
    H_kv 8, d 128, 1 init + 2 local + top-16 per query position): the bulk
    build of the compressed keys, per-token selection and causal
    block-sparse attention, each timed, the attention priced against the
    bf16 MFMA peak on eq. (15)'s work (4 d flops per query head and visible
    key token of its blocks, counted from the lists) and against HBM on the
    bytes any prefill must move (the layer's K and V once, Q in, out)."""
    cfg = dataclasses.replace(synth.get_config(cid), bias_frac=0.0, bias_beta=0.0)
    dev = "cuda"
    T, G = cfg.T, cfg.G
    K, V, _ = inputs.kv_layer(cfg, 0, device=dev)
    F = inputs.to_bf16(inputs.prefill_indexer_vectors(cfg, 0, T), dev)
    Q = inputs.prefill_queries(cfg, 0, T, device=dev)
    seq = torch.full((cfg.B,), T, dtype=torch.int32, device=dev)
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    kt = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
    nsm = cfg.n_init + cfg.n_local + cfg.top_k
    bi = torch.empty((cfg.B, T, cfg.H_kv, nsm), dtype=torch.int32, device=dev)
    ns = torch.empty((cfg.B, T, cfg.H_kv), dtype=torch.int32, device=dev)
    out = torch.empty((cfg.B, T, cfg.H_q, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, T, cfg.H_q), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(16, sda.lib().sda_prefill_attention_workspace(cfg.B, T, cfg.H_q, cfg.H_kv, nsm, cfg.d,
                                                                        cfg.NB)), dtype=torch.uint8, device=dev)
    sel = (cfg.n_init, cfg.n_local, cfg.top_k)
    t_keys = eager_time(lambda: sda.sda_update_compressed_keys(K, kt, zero, seq, T), reps=5)
    t_sel = eager_time(lambda: sda.sda_prefill_select(F, kt, seq, 0, *sel, block_idx=bi, n_sel=ns), reps=5)
    t_att = eager_time(lambda: sda.sda_prefill_attention(Q, K, V, seq, bi, ns, 0, out=out, lse=lse, ws=ws), reps=3)
    # work: each query head times the visible tokens of its blocks (causal: a
    # block at or past the query's own block counts only its first tokens)
    bi_h = bi.cpu().numpy()
    ns_h = ns.cpu().numpy()
    pos = np.arange(T)[None, :, None, None]
    valid = np.arange(nsm)[None, None, None, :] < ns_h[..., None]
    vis = np.clip(pos + 1 - bi_h.astype(np.int64) * 64, 0, 64) * valid
    tokens = int(vis.sum())                            # (query, KV head, visible key) triples
    att_flops = tokens * G * 4 * cfg.d
    sel_flops = int(sum(2 * cfg.d * (p // 64 + 1) for p in range(T))) * cfg.B * cfg.H_kv
    kv_bytes = 2 * cfg.B * cfg.H_kv * T * cfg.d * 2
    q_bytes = cfg.B * T * cfg.H_q * cfg.d * 2
    out_bytes = cfg.B * T * cfg.H_q * (cfg.d + 1) * 4
    min_bytes = kv_bytes + q_bytes + out_bytes + int(bi.numel()) * 4
    tf = att_flops / t_att / 1e12
    # adjacent positions' top-k overlap near the end of the sequence (the
    # correlation of consecutive indexer vectors); the lists there hold
    # init, top-k and local blocks in ascending order
    tail = bi_h[:, T - 1025:, :, :]
    ov = []
    for b in range(cfg.B):
        for g in range(cfg.H_kv):
            for i in range(0, 1024, 16):
                a0, a1 = tail[b, i, g], tail[b, i + 1, g]
                top0 = set(a0) - set(range(cfg.n_init)) - set(range((T - 1025 + i) // 64 - 1, (T - 1025 + i) // 64 + 1))
                top1 = set(a1) - set(range(cfg.n_init)) - set(range((T - 1024 + i) // 64 - 1, (T - 1024 + i) // 64 + 1))
                ov.append(len(top0 & top1) / max(1, len(top0)))
    ov = float(np.mean(ov))
    # blocks the attention loads: the union of each tile's lists (tiles of
    # min(32, 128 / G) consecutive positions, one fetch per block and tile)
    C = max(1, min(32, 128 // G))
    grp = bi_h.reshape(cfg.B, T // C, C, cfg.H_kv, nsm).transpose(0, 1, 3, 2, 4).reshape(cfg.B, T // C, cfg.H_kv, -1)
    grp = np.sort(grp, axis=-1)
    loads = int(((np.diff(grp, axis=-1) != 0) & (grp[..., 1:] >= 0)).sum() + (grp[..., 0] >= 0).sum())
    loaded_bytes = loads * 64 * cfg.d * 2 * 2
    res = {
        "workload": f"prefill of {T} tokens at the 8B-shaped layer: B={cfg.B}, H_q={cfg.H_q}, H_kv={cfg.H_kv}, "
                    f"d={cfg.d}, {cfg.n_init} init + {cfg.n_local} local + top-{cfg.top_k} per query position, "
                    f"indexer vectors of consecutive positions correlated {inputs.PREFILL_RHO} (adjacent "
                    f"top-{cfg.top_k} overlap {ov:.2f})",
        "compressed_keys_us": t_keys * 1e6,
        "select_us": t_sel * 1e6,
        "select_roofline": {"bound": "mfma", "achieved_tflops": sel_flops / t_sel / 1e12, "peak_tflops": 2500.0,
                            "frac": sel_flops / t_sel / 1e12 / 2500.0, "flops": sel_flops},
        "attention_us": t_att * 1e6,
        "attention_roofline": {"bound": "mfma", "achieved_tflops": tf, "peak_tflops": 2500.0, "frac": tf / 2500.0,
                               "flops": att_flops},
        "attention_hbm": hbm(min_bytes, t_att),
        "attention_blocks_loaded": loads,
        "attention_loaded_roofline": hbm(loaded_bytes, t_att),
        "tokens_per_s": cfg.B * T / (t_keys + t_sel + t_att),
    }
    del K, V, F, Q, kt, bi, ns, out, lse, ws
    torch.cuda.empty_cache()
    return res


def measure_pooled(cfg, layers, O, full, prev, window=32, stride=16):
    """InfLLM-V2's inference compression (kernel 32, stride 16) on the 128K
    layer: the bulk build and per-token refresh of the overlapping compressed
    keys, and the pooled score/select (compressed scores max-pooled onto the
    64-token blocks, then top-k), one call per resident layer in turn."""
    dev = "cuda"
    T, d = cfg.T, cfg.d
    nc = -(-T // stride)
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    kts = []
    for lay in layers:
        kt = torch.zeros((cfg.B, cfg.H_kv, nc, d), dtype=torch.bfloat16, device=dev)
        sda.sda_update_compressed_keys_strided(lay["K"], kt, zero, full, T, window, stride)
        kts.append(kt)
    K0 = layers[0]["K"]
    t_build = eager_time(lambda: sda.sda_update_compressed_keys_strided(K0, kts[0], zero, full, T, window, stride),
                         reps=5)
    t_tok = graph_time(lambda: sda.sda_update_compressed_keys_strided(K0, kts[0], prev, full, 1, window, stride))
    nrow = cfg.B * cfg.H_kv
    kt_bytes = nrow * nc * d * 2
    # the refresh for token T-1 recomputes every window holding it (keys up to T)
    touched = [j for j in range(nc) if j * stride <= T - 1 < j * stride + window]
    tok_bytes = sum(min(window, T - j * stride) * d * 2 + d * 2 for j in touched)
    nsm = cfg.n_init + cfg.n_local + cfg.top_k
    bi = torch.empty((cfg.B, 1, cfg.H_kv, nsm), dtype=torch.int32, device=dev)
    ns = torch.empty((cfg.B, 1, cfg.H_kv), dtype=torch.int32, device=dev)
    ws = torch.zeros(sda.lib().sda_score_select_pooled_workspace(cfg.B, 1, cfg.H_kv, nc, stride, cfg.top_k),
                     dtype=torch.uint8, device=dev)
    L = len(layers)
    turn = [0]

    def pooled_call():
        i = turn[0] % L
        turn[0] += 1
        sda.sda_score_select_pooled(layers[i]["F"], kts[(i + 1) % L], full, window, stride, cfg.n_init,
                                    cfg.n_local, cfg.top_k, block_idx=bi, n_sel=ns, ws=ws)
    t_sel = graph_time(pooled_call, copies=L)
    # InfLLM-V2's own selector in the same setting: the G query heads of the
    # next layer, per-head softmax over the compressed entries, sum, max-pool
    wsm = torch.zeros(sda.lib().sda_score_select_multihead_pooled_workspace(cfg.B, 1, cfg.H_q, cfg.H_kv, nc, stride,
                                                                           cfg.top_k), dtype=torch.uint8, device=dev)
    tau = math.sqrt(d)
    turn[0] = 0

    def mh_pooled_call():
        i = turn[0] % L
        turn[0] += 1
        sda.sda_score_select_multihead_pooled(layers[(i + 1) % L]["Q"], kts[(i + 1) % L], full, window, stride,
                                              cfg.n_init, cfg.n_local, cfg.top_k, tau, block_idx=bi, n_sel=ns, ws=wsm)
    t_mh = graph_time(mh_pooled_call, copies=L)
    # oracle: one row's window means, scores, pool and selection
    kk = O.bf16_to_f64(inputs.bf16_bits(K0[0, 0]))
    f0 = O.bf16_to_f64(inputs.bf16_bits(layers[0]["F"][0, 0, 0]))
    t_or_keys = oracle_time(lambda: O.store_bf16(O.compressed_keys_strided(kk, T, window, stride)))
    ktc = O.store_bf16(O.compressed_keys_strided(kk, T, window, stride))
    t_or_sel = oracle_time(lambda: O.select_row_pooled(f0, ktc, T, window, stride, cfg.n_init, cfg.n_local,
                                                       cfg.top_k))
    res = {
        "workload": f"{cfg.name}: kernel {window} / stride {stride} compression ({nc} compressed keys per row, "
                    f"{nrow} rows), block score = max over the overlapping windows, 1 init + 2 local + top-{cfg.top_k}",
        "build_us": t_build * 1e6,
        "build_roofline": hbm(nrow * T * d * 2 + kt_bytes, t_build),
        "per_token_update_us": t_tok * 1e6,
        "per_token_update_roofline": hbm(nrow * tok_bytes, t_tok),
        "select_us": t_sel * 1e6,
        "select_roofline": hbm(kt_bytes, t_sel),
        "g_head_select_us": t_mh * 1e6,
        "g_head_select_roofline": hbm(kt_bytes, t_mh),
        "g_head_over_forecast": t_mh / t_sel,
        "oracle_rows_per_s_keys": 1.0 / t_or_keys,
        "oracle_rows_per_s_select": 1.0 / t_or_sel,
        "gpu_rows_per_s_select": nrow / t_sel,
    }
    del kts
    torch.cuda.empty_cache()
    return res


def adjacent_overlap(bi_np, C):
    """Mean share of a query's blocks that the next query of its group also
    selects (lists [B, NQ, H_kv, n], full rows)."""
    B, NQ, H, n = bi_np.shape
    vals = []
    for b in range(B):
        for g in range(H):
            for q0 in range(0, NQ, C):
                for c in range(q0, min(q0 + C, NQ) - 1):
                    vals.append(len(np.intersect1d(bi_np[b, c, g], bi_np[b, c + 1, g])) / n)
    return float(np.mean(vals))


def distinct_blocks(bi_np, C=None):
    """Distinct (batch, KV head, block) tiles among the lists; with C, only
    each group's first list (the shared representative)."""
    B, NQ, H, n = bi_np.shape
    tot = 0
    for b in range(B):
        for g in range(H):
            rows = bi_np[b, ::C, g] if C else bi_np[b, :, g]
            tot += np.unique(rows).size
    return tot


def tile_union_blocks(bi_np, C, G):
    """Blocks the exact grouped launch loads: the union of each verification
    tile's lists, a tile holding as many whole groups of C queries as fit in
    128 rows of G heads and 32 queries (the library's tiling)."""
    B, NQ, H, n = bi_np.shape
    cq = min((min(32, 128 // G) // C) * C, -(-NQ // C) * C)
    tot = 0
    for b in range(B):
        for g in range(H):
            for q0 in range(0, NQ, cq):
                v = bi_np[b, q0:q0 + cq, g]
                tot += np.unique(v[v >= 0]).size
    return tot


def grouped_lists(cfg, kt, seq, gamma, n_sets):
    """Draft-query block lists of the verification workload whose adjacent
    queries share about gamma of their blocks: sigma (the draft noise of the
    indexer vectors) bisected on the library's own selections, then n_sets
    independent list sets at that sigma."""
    dev = "cuda"

    def select(sigma, layer):
        F = inputs.to_bf16(inputs.indexer_vectors(cfg, layer, sigma=sigma), dev)
        bi, _ = sda.sda_score_select(F, kt, seq, 0, 0, cfg.top_k)
        return bi
    lo, hi = 0.0, 4.0
    for _ in range(16):
        mid = 0.5 * (lo + hi)
        ov = adjacent_overlap(select(mid, 0).cpu().numpy(), cfg.group_C)
        lo, hi = (mid, hi) if ov > gamma else (lo, mid)
    sigma = 0.5 * (lo + hi)
    return sigma, [select(sigma, s) for s in range(n_sets)]


def profile_grouped(reps=4):
    """Eager launches for hardware-counter runs at the verification workload
    (gamma = 0.75): the per-query decode, mode A, mode B, NSA's three
    branches and exact verification of all 16 draft queries as one group,
    `reps` launches each in that order, on independent list sets."""
    cfg = synth.get_config(4)
    dev = "cuda"
    K, V, _ = inputs.kv_layer(cfg, 0, device=dev)
    n, C = cfg.top_k, cfg.group_C
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=dev)
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    kt = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kt)
    sda.sda_update_compressed_keys(K, kt, zero, seq, cfg.T)
    sda.sda_update_compressed_keys(V, vc, zero, seq, cfg.T)
    sigma, bis = grouped_lists(cfg, kt, seq, 0.75, reps)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0, sigma=sigma), dev)
    ns = torch.full((cfg.B, cfg.NQ, cfg.H_kv), n, dtype=torch.int32, device=dev)
    gates = torch.rand((cfg.B, cfg.NQ, cfg.H_q, 3), generator=torch.Generator(device=dev).manual_seed(5),
                       device=dev, dtype=torch.float32)
    wss = {}
    torch.cuda.synchronize()
    log(f"profile_grouped: sigma {sigma:.4f}; launches in order: per-query x{reps}, mode A x{reps}, "
        f"mode B x{reps}, NSA x{reps}, one group of {cfg.NQ} x{reps}")
    for i in range(reps):
        sda.sda_sparse_decode(Q, K, V, seq, bis[i], ns)
    for mode in (sda.SDA_GROUP_EXACT, sda.SDA_GROUP_SHARED_REP):
        for i in range(reps):
            sda.sda_grouped_decode(Q, K, V, seq, bis[i], ns, C, mode=mode)
    for i in range(reps):
        sda.sda_nsa_decode(Q, K, V, kt, vc, seq, bis[i], ns, gates, 64, 512, group_C=C, mode=sda.SDA_GROUP_EXACT)
    ws16 = torch.zeros(max(16, sda.lib().sda_grouped_decode_workspace(cfg.B, cfg.NQ, cfg.H_q, cfg.H_kv, n, cfg.d,
                                                                      cfg.NB, cfg.NQ, sda.SDA_GROUP_EXACT, 0)),
                       dtype=torch.uint8, device=dev)
    for i in range(reps):
        sda.sda_grouped_decode(Q, K, V, seq, bis[i], ns, cfg.NQ, mode=sda.SDA_GROUP_EXACT, ws=ws16)
    torch.cuda.synchronize()
    blk = 64 * cfg.d * 2 * 2
    bnp = [b.cpu().numpy() for b in bis]
    print(json.dumps({"profile": "grouped", "gamma": 0.75, "sigma": sigma, "reps": reps,
                      "distinct_bytes_per_query_or_mode_A": float(np.mean([distinct_blocks(b) for b in bnp])) * blk,
                      "distinct_bytes_mode_B": float(np.mean([distinct_blocks(b, C) for b in bnp])) * blk}))


def measure_grouped(O):
    """a5 at the draft-verification workload (64K, 16 draft queries per
    sequence in groups of C = 4): the queries' block lists come from the
    library's own selection on draft indexer vectors f_c = f0 + sigma eps_c,
    with sigma bisected so that adjacent queries of a group share gamma of
    their top-16 blocks, gamma in {0.5, 0.75, 0.9}.  Per gamma: mode A (each
    union block loaded once per group), mode B (the first query's list), the
    per-query decode of the same lists, the blocks each launch loads and the
    distinct (batch, KV head, block) tiles it touches (repeats across the
    groups of a KV head are cache hits, so rooflines use distinct bytes), and
    mode B's error against the exact per-query result (mode A)."""
    cfg = synth.get_config(4)
    dev = "cuda"
    K, V, _ = inputs.kv_layer(cfg, 0, device=dev)
    n, C = cfg.top_k, cfg.group_C
    kt = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=dev)
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    sda.sda_update_compressed_keys(K, kt, zero, seq, cfg.T)
    blk = 64 * cfg.d * 2 * 2
    n_sets = 6                 # independent list sets, used in turn: together they exceed the Infinity Cache
    ns = torch.full((cfg.B, cfg.NQ, cfg.H_kv), n, dtype=torch.int32, device=dev)
    out = torch.empty((cfg.B, cfg.NQ, cfg.H_q, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.NQ, cfg.H_q), dtype=torch.float32, device=dev)
    uc_shape = (cfg.B, cfg.NQ // C, cfg.H_kv)

    res = {"workload": f"{cfg.name}: B={cfg.B}, NQ={cfg.NQ}, C={C}, H_q={cfg.H_q}, H_kv={cfg.H_kv}, T={cfg.T}, "
                       f"top-{n} per query from the library's selection on draft indexer vectors; adjacent "
                       f"overlap gamma tuned by bisection on the draft noise", "gammas": {}}
    groups = cfg.B * (cfg.NQ // C) * cfg.H_kv
    for gamma in cfg.gammas:
        sigma, bis = grouped_lists(cfg, kt, seq, gamma, n_sets)
        bnp = [b.cpu().numpy() for b in bis]
        measured = float(np.mean([adjacent_overlap(b, C) for b in bnp]))
        Q = inputs.to_bf16(inputs.attention_queries(cfg, 0, sigma=sigma), dev)
        row = {"sigma": sigma, "measured_gamma": measured}
        per_q_blocks = cfg.B * cfg.NQ * cfg.H_kv * n
        dist_all = float(np.mean([distinct_blocks(b) for b in bnp]))
        dist_rep = float(np.mean([distinct_blocks(b, C) for b in bnp]))
        outs = {}
        for mode, name in ((sda.SDA_GROUP_EXACT, "mode_A"), (sda.SDA_GROUP_SHARED_REP, "mode_B")):
            ws = torch.zeros(sda.lib().sda_grouped_decode_workspace(cfg.B, cfg.NQ, cfg.H_q, cfg.H_kv, n, cfg.d,
                                                                    cfg.NB, C, mode, 0), dtype=torch.uint8,
                             device=dev)
            ucs = [torch.empty(uc_shape, dtype=torch.int32, device=dev) for _ in range(n_sets)]
            turn = [0]

            def grouped_call():
                i = turn[0] % n_sets
                turn[0] += 1
                sda.sda_grouped_decode(Q, K, V, seq, bis[i], ns, C, mode=mode, out=out, lse=lse,
                                       union_count=ucs[i], ws=ws)
            t = graph_time(grouped_call, copies=n_sets)
            group_unions = sum(int(u.sum().item()) for u in ucs) / n_sets
            if mode == sda.SDA_GROUP_EXACT:
                # exact mode walks the union of each tile of whole groups once
                loaded = float(np.mean([tile_union_blocks(b.cpu().numpy(), C, cfg.G) for b in bis]))
                dist = dist_all
            else:
                loaded = group_unions                     # each group walks its representative's list
                dist = dist_rep
            row[name] = {"us": t * 1e6, "blocks_loaded": loaded, "group_union_blocks": group_unions,
                         "distinct_blocks": dist, "roofline": hbm(dist * blk, t),
                         "roofline_loaded": hbm(loaded * blk, t)}
            o, _, _ = sda.sda_grouped_decode(Q, K, V, seq, bis[0], ns, C, mode=mode, ws=ws)
            outs[name] = o
        # exact verification with all NQ draft queries of a sequence as one
        # group (NQ * G = 64 rows at G = 4: the row-tiled engine, its union split among
        # workgroups): each distinct block is fetched once per (batch, KV head)
        CA = cfg.NQ
        ws = torch.zeros(max(16, sda.lib().sda_grouped_decode_workspace(cfg.B, cfg.NQ, cfg.H_q, cfg.H_kv, n, cfg.d,
                                                                        cfg.NB, CA, sda.SDA_GROUP_EXACT, 0)),
                         dtype=torch.uint8, device=dev)
        ucs = [torch.empty((cfg.B, 1, cfg.H_kv), dtype=torch.int32, device=dev) for _ in range(n_sets)]
        turn = [0]

        def tiled_call():
            i = turn[0] % n_sets
            turn[0] += 1
            sda.sda_grouped_decode(Q, K, V, seq, bis[i], ns, CA, mode=sda.SDA_GROUP_EXACT, out=out, lse=lse,
                                   union_count=ucs[i], ws=ws)
        t = graph_time(tiled_call, copies=n_sets)
        loaded = sum(int(u.sum().item()) for u in ucs) / n_sets
        o16, _, _ = sda.sda_grouped_decode(Q, K, V, seq, bis[0], ns, CA, mode=sda.SDA_GROUP_EXACT, ws=ws)
        row["exact_one_group_of_16"] = {"us": t * 1e6, "blocks_loaded": loaded, "distinct_blocks": dist_all,
                                        "roofline": hbm(dist_all * blk, t), "roofline_loaded": hbm(loaded * blk, t),
                                        "max_abs_diff_vs_mode_A": (o16 - outs["mode_A"]).abs().max().item()}
        ws = torch.zeros(sda.lib().sda_sparse_decode_workspace(cfg.B, cfg.NQ, cfg.H_q, cfg.H_kv, n, cfg.d, 0),
                         dtype=torch.uint8, device=dev)
        turn = [0]

        def per_query_call():
            i = turn[0] % n_sets
            turn[0] += 1
            sda.sda_sparse_decode(Q, K, V, seq, bis[i], ns, out=out, lse=lse, ws=ws)
        t = graph_time(per_query_call, copies=n_sets)
        row["per_query"] = {"us": t * 1e6, "blocks_loaded": per_q_blocks, "distinct_blocks": dist_all,
                            "roofline": hbm(dist_all * blk, t), "roofline_loaded": hbm(per_q_blocks * blk, t)}
        row["measured_saving_mode_A"] = 1.0 - row["mode_A"]["group_union_blocks"] / per_q_blocks
        row["formula_saving"] = 1.0 - O.union_size_formula(n, C, measured) / (n * C)
        row["speedup_mode_A_vs_per_query"] = row["per_query"]["us"] / row["mode_A"]["us"]
        row["speedup_one_group_vs_per_query"] = row["per_query"]["us"] / row["exact_one_group_of_16"]["us"]
        # mode B approximates: its error against the exact per-query result
        dB = (outs["mode_B"] - outs["mode_A"]).abs()
        row["mode_B_error_vs_exact"] = {"max_abs": dB.max().item(), "mean_abs": dB.mean().item(),
                                        "rows_exact": float((dB.amax(dim=-1) == 0).float().mean().item())}
        res["gammas"][f"{gamma:g}"] = row
        log(f"grouped gamma {gamma}: sigma {sigma:.4f} measured {measured:.3f}; mode A {row['mode_A']['us']:.1f} us, "
            f"mode B {row['mode_B']['us']:.1f} us, per-query {row['per_query']['us']:.1f} us, one group of 16 "
            f"{row['exact_one_group_of_16']['us']:.1f} us; mode B max err "
            f"{row['mode_B_error_vs_exact']['max_abs']:.3e}")
        if gamma == 0.75:
            sets75, Q75, dist75 = bis, Q, dist_all
    # NSA's three branches in one launch at gamma = 0.75 (exact merge for the
    # listed blocks, a 512-token window, 64/64 compressed keys and values,
    # random gates)
    window = 512
    kc = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    sda.sda_update_compressed_keys(K, kc, zero, seq, cfg.T)
    sda.sda_update_compressed_keys(V, vc, zero, seq, cfg.T)
    gates = torch.rand((cfg.B, cfg.NQ, cfg.H_q, 3), generator=torch.Generator(device=dev).manual_seed(5),
                       device=dev, dtype=torch.float32)
    nsa_ws = torch.zeros(max(sda.lib().sda_nsa_decode_workspace(cfg.B, cfg.NQ, cfg.H_q, cfg.H_kv, n, cfg.d, cfg.T,
                                                                cfg.NB, window, C, m)
                             for m in (sda.SDA_GROUP_EXACT, sda.SDA_GROUP_SHARED_REP)),
                         dtype=torch.uint8, device=dev)
    nsa_lse = torch.empty((cfg.B, cfg.NQ, cfg.H_q, 3), dtype=torch.float32, device=dev)
    ucs_n = [torch.empty(uc_shape, dtype=torch.int32, device=dev) for _ in range(n_sets)]
    turn = [0]

    def nsa_call():
        i = turn[0] % n_sets
        turn[0] += 1
        sda.sda_nsa_decode(Q75, K, V, kc, vc, seq, sets75[i], ns, gates, 64, window, group_C=C,
                           mode=sda.SDA_GROUP_EXACT, out=out, lse=nsa_lse, union_count=ucs_n[i], ws=nsa_ws)
    t = graph_time(nsa_call, copies=n_sets)
    # loaded: a row tile holds the 16 queries of one (batch, KV head) (64
    # rows) and loads the union of their lists, the window's blocks and the
    # compressed keys and values once
    kv_rows = cfg.B * cfg.H_kv
    sel_blocks = dist75
    win_blocks = kv_rows * (window // 64)
    cmp_loaded = kv_rows * cfg.NB * cfg.d * 2 * 2
    # distinct: the window's last 8 blocks and the compressed keys and values
    # once per (batch, KV head); window blocks also selected counted once
    win_dist = 0
    for bnp in (sets75[0].cpu().numpy(),):
        for b in range(cfg.B):
            for g in range(cfg.H_kv):
                sel = np.unique(bnp[b, :, g])
                win_dist += np.setdiff1d(np.arange(cfg.NB - window // 64, cfg.NB), sel).size
    dist_bytes = (dist75 + win_dist) * blk + kv_rows * cfg.NB * cfg.d * 2 * 2
    res["nsa_three_branch_gamma_0.75"] = {
        "us": t * 1e6, "window": window, "compressed_keys_per_row": cfg.NB,
        "selected_blocks_loaded": sel_blocks, "window_blocks_loaded": win_blocks,
        "distinct_bytes": int(dist_bytes), "roofline": hbm(dist_bytes, t),
        "roofline_loaded": hbm((sel_blocks + win_blocks) * blk + cmp_loaded, t),
        "extra_us_over_mode_A": t * 1e6 - res["gammas"]["0.75"]["mode_A"]["us"],
    }
    # the same three branches in shared-representative mode (every query takes
    # its group's first list)
    turn[0] = 0

    def nsa_call_b():
        i = turn[0] % n_sets
        turn[0] += 1
        sda.sda_nsa_decode(Q75, K, V, kc, vc, seq, sets75[i], ns, gates, 64, window, group_C=C,
                           mode=sda.SDA_GROUP_SHARED_REP, out=out, lse=nsa_lse, union_count=ucs_n[i], ws=nsa_ws)
    tb = graph_time(nsa_call_b, copies=n_sets)
    res["nsa_three_branch_gamma_0.75"]["mode_B_us"] = tb * 1e6
    log(f"NSA three branches at gamma 0.75: exact {t * 1e6:.1f} us, shared representative {tb * 1e6:.1f} us")
    # oracle: one group (C queries x G heads) of one (batch, KV head), mode A
    kk = O.bf16_to_f64(inputs.bf16_bits(K[0, 0, :cfg.T]))
    vv = O.bf16_to_f64(inputs.bf16_bits(V[0, 0, :cfg.T]))
    qd = O.bf16_to_f64(inputs.bf16_bits(Q75[0, :C, :cfg.G])).reshape(C, cfg.G, cfg.d)
    b0 = sets75[0].cpu().numpy()
    lists = [b0[0, c, 0] for c in range(C)]
    t_or = oracle_time(lambda: O.grouped_row(qd, kk, vv, lists, cfg.T, 1.0 / math.sqrt(cfg.d), O.MODE_EXACT))
    res["oracle_groups_per_s"] = 1.0 / t_or
    res["gpu_groups_per_s_gamma_0.75"] = groups / (res["gammas"]["0.75"]["mode_A"]["us"] * 1e-6)
    del K, V, kc, vc
    torch.cuda.empty_cache()
    return res


def measure_chain(L=15, schedules=(1, 3, 5), window=512):
    """NEXT 3 at the verification workload (64K, 16 draft queries per
    sequence in groups of 4, top-16, 512-token window, 64/64 compressed keys
    and values): a chain of L NSA layers where every r-th layer routes and
    caches its block lists and the others reuse them (sda_nsa_chain), for
    r in `schedules`; T_refresh (routing + the three-branch launch) and
    T_reuse (the launch alone) per layer, and T_total against R T_refresh +
    (L - R) T_reuse."""
    cfg = synth.get_config(4)
    dev = "cuda"
    n, C = cfg.top_k, cfg.group_C
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=dev)
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    # the draft noise of the gamma = 0.75 workload, bisected on layer 0
    K0, _, _ = inputs.kv_layer(cfg, 0, device=dev)
    kt0 = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
    sda.sda_update_compressed_keys(K0, kt0, zero, seq, cfg.T)
    sigma, _ = grouped_lists(cfg, kt0, seq, 0.75, 1)
    del K0, kt0
    layers = []
    for j in range(L):
        K, V, _ = inputs.kv_layer(cfg, j, device=dev)
        kc = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        sda.sda_update_compressed_keys(K, kc, zero, seq, cfg.T)
        sda.sda_update_compressed_keys(V, vc, zero, seq, cfg.T)
        gates = torch.rand((cfg.B, cfg.NQ, cfg.H_q, 3), generator=torch.Generator(device=dev).manual_seed(j),
                           device=dev, dtype=torch.float32)
        layers.append(dict(q=inputs.to_bf16(inputs.attention_queries(cfg, j, sigma=sigma), dev), k=K, v=V, k_cmp=kc,
                           v_cmp=vc, k_route=kc, f_route=inputs.to_bf16(inputs.indexer_vectors(cfg, j, sigma=sigma),
                                                                        dev), gates=gates))
    res = {"workload": f"{cfg.name}: chain of {L} NSA verification layers (B={cfg.B}, NQ={cfg.NQ}, C={C}, "
                       f"H_q={cfg.H_q}, H_kv={cfg.H_kv}, T={cfg.T}, top-{n}, window {window}, 64/64 compressed "
                       f"keys and values), draft routing vectors at the gamma = 0.75 noise", "schedules": {}}
    bic = torch.empty((cfg.B, cfg.NQ, cfg.H_kv, n), dtype=torch.int32, device=dev)
    nsc = torch.empty((cfg.B, cfg.NQ, cfg.H_kv), dtype=torch.int32, device=dev)
    ws = torch.zeros(sda.lib().sda_nsa_chain_workspace(cfg.B, cfg.NQ, cfg.H_q, cfg.H_kv, cfg.d, cfg.T, cfg.NB, window,
                                                       n, C, sda.SDA_GROUP_EXACT), dtype=torch.uint8, device=dev)
    times = {}
    for r in schedules:
        sched = [j % r == 0 for j in range(L)]
        call, _ = sda.sda_nsa_chain(layers, sched, seq, n, 64, window, group_C=C, block_idx_cache=bic,
                                    n_sel_cache=nsc, ws=ws, _prepare=True)
        times[r] = call_time([call], 20, copies=2)
    # one layer of each kind: a chain of L reuse layers after one refresh is
    # what r = L gives; single-layer timings come from the r = 1 and r = L chains
    t_refresh = times[1] / L if 1 in times else float("nan")
    callL, _ = sda.sda_nsa_chain(layers, [j == 0 for j in range(L)], seq, n, 64, window, group_C=C,
                                 block_idx_cache=bic, n_sel_cache=nsc, ws=ws, _prepare=True)
    t_L = call_time([callL], 20, copies=2)
    t_reuse = (t_L - t_refresh) / (L - 1)
    for r in schedules:
        sched = [j % r == 0 for j in range(L)]
        R = sum(sched)
        res["schedules"][f"r={r}"] = {"refresh_layers": R, "reuse_layers": L - R, "T_total_us": times[r] * 1e6,
                                      "formula_us": (R * t_refresh + (L - R) * t_reuse) * 1e6,
                                      "saving_vs_all_refresh": 1.0 - times[r] / times[1] if 1 in times else None}
    res["T_refresh_us"] = t_refresh * 1e6
    res["T_reuse_us"] = t_reuse * 1e6
    del layers
    torch.cuda.empty_cache()
    return res


def measure_offload(O, chain=8, pool_sizes=(16, 32, 64, 128)):
    """a6 and NEXT 4 at the offload workload (256K, B 4, H_q 32, H_kv 8, 1 + 2 +
    top-32 per layer, 8 layers): the K/V of every layer in pinned host memory
    (8 distinct layers, 34 GB, unless pinning that much is refused), the
    compressed keys, queries and indexer vectors on the GPU.  Timed: one
    layer's gather alone against a plain pinned copy of the same bytes; the
    decode from the stage; the chain with the persistent prefetch pool
    (sda_offload_chain; the lookahead selection of layer l+1 inside the loop)
    for several pool sizes; the same chain with one gather launch per layer
    on a side stream.  overlap = (sum of the chain's parts run one after the
    other) / chain time: above 1 when transfers hide behind compute."""
    cfg = synth.get_config(5)
    dev = "cuda"
    T = cfg.T
    nsm = cfg.n_init + cfg.n_local + cfg.top_k
    seq = torch.full((cfg.B,), T, dtype=torch.int32, device=dev)
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    host, kts, note = [], [], ""
    for l in range(chain):
        K, V, _ = inputs.kv_layer(cfg, l, device=dev)
        kt = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=dev)
        sda.sda_update_compressed_keys(K, kt, zero, seq, T)
        kts.append(kt)
        try:
            Kh = torch.empty(K.shape, dtype=torch.bfloat16, pin_memory=True)
            Vh = torch.empty(V.shape, dtype=torch.bfloat16, pin_memory=True)
        except RuntimeError as e:                      # pinning refused: reuse the layers pinned so far
            note = f"pinning layer {l} refused ({e}); host layers cycle over {len(host)}"
            log(note)
            del K, V
            break
        Kh.copy_(K)
        Vh.copy_(V)
        host.append((Kh, Vh))
        if l == 0:
            kk = O.bf16_to_f64(inputs.bf16_bits(K[0, 0, :T]))
            vv = O.bf16_to_f64(inputs.bf16_bits(V[0, 0, :T]))
        del K, V
        torch.cuda.empty_cache()
    for l in range(len(kts), chain):                   # compressed keys of the cycled layers
        kts.append(kts[l % len(host)])
    nh = len(host)
    Qs = [inputs.to_bf16(inputs.attention_queries(cfg, l), dev) for l in range(chain)]
    Fs = [inputs.to_bf16(inputs.indexer_vectors(cfg, l), dev) for l in range(chain)]
    f_first = inputs.to_bf16(inputs.indexer_vectors(cfg, 1000), dev)
    layers = [dict(k_host=host[l % nh][0], v_host=host[l % nh][1], k_tilde=kts[l], q=Qs[l], f=Fs[l])
              for l in range(chain)]
    side = torch.cuda.Stream()
    res_pool = {}
    ws = None
    bi_chain = torch.empty((chain, cfg.B, 1, cfg.H_kv, nsm), dtype=torch.int32, device=dev)
    for wgs in pool_sizes:
        outs, _, ws = sda.sda_offload_chain(layers, seq, cfg.n_init, cfg.n_local, cfg.top_k, f_first,
                                            prefetch_workgroups=wgs, block_idx=bi_chain, ws=ws, side_stream=side)
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            sda.sda_offload_chain(layers, seq, cfg.n_init, cfg.n_local, cfg.top_k, f_first, prefetch_workgroups=wgs,
                                  block_idx=bi_chain, ws=ws, side_stream=side)
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        err = int(ws[8:12].view(torch.int32).item())
        res_pool[str(wgs)] = {"chain_ms": min(ts) * 1e3, "error_word": err}
    # parts, each alone: a layer's selection, gather (one launch) and decode from the stage
    bi = torch.empty((cfg.B, 1, cfg.H_kv, nsm), dtype=torch.int32, device=dev)
    ns = torch.empty((cfg.B, 1, cfg.H_kv), dtype=torch.int32, device=dev)
    wsel = torch.zeros(sda.lib().sda_score_select_workspace(cfg.B, 1, cfg.H_kv, cfg.NB, cfg.top_k),
                       dtype=torch.uint8, device=dev)
    t_sel = eager_time(lambda: sda.sda_score_select(Fs[0], kts[1], seq, cfg.n_init, cfg.n_local, cfg.top_k,
                                                    block_idx=bi, n_sel=ns, ws=wsel), reps=5)
    stage_shape = (cfg.B, cfg.H_kv, nsm * 64, cfg.d)
    stages = [(torch.empty(stage_shape, dtype=torch.bfloat16, device=dev),
               torch.empty(stage_shape, dtype=torch.bfloat16, device=dev),
               torch.empty((cfg.B, 1, cfg.H_kv, nsm), dtype=torch.int32, device=dev)) for _ in range(2)]
    bis = [torch.empty_like(bi) for _ in range(chain)]
    nss = [torch.empty_like(ns) for _ in range(chain)]
    out = torch.empty((cfg.B, 1, cfg.H_q, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, 1, cfg.H_q), dtype=torch.float32, device=dev)
    wdec = torch.zeros(sda.lib().sda_sparse_decode_workspace(cfg.B, 1, cfg.H_q, cfg.H_kv, nsm, cfg.d, 0),
                       dtype=torch.uint8, device=dev)

    def select(l):                      # layer l's blocks: its own vectors at l = 0, else layer l-1's
        sda.sda_score_select(f_first if l == 0 else Fs[l - 1], kts[l], seq, cfg.n_init, cfg.n_local, cfg.top_k,
                             block_idx=bis[l], n_sel=nss[l], ws=wsel)

    def gather(l):
        st = stages[l % 2]
        sda.sda_gather_blocks(host[l % nh][0], host[l % nh][1], bis[l], nss[l], k_stage=st[0], v_stage=st[1],
                              slot=st[2], max_workgroups=128)

    def decode(l):
        st = stages[l % 2]
        sda.sda_sparse_decode(Qs[l], st[0], st[1], seq, bis[l], nss[l], slot=st[2], out=out, lse=lse, ws=wdec)

    select(0)
    t_gather = eager_time(lambda: gather(0), reps=5)
    gather(0)
    t_dec = eager_time(lambda: decode(0), reps=10)
    # the per-layer-launch chain: the side stream gathers layer l+1 while the
    # stream decodes layer l, the selection of l+1 inside the loop
    main = torch.cuda.current_stream()

    def launch_chain_ordered():
        select(0)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            gather(0)
        done = [None] * chain
        done[0] = torch.cuda.Event()
        done[0].record(side)
        for l in range(chain):
            if l + 1 < chain:
                select(l + 1)
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    gather(l + 1)
                done[l + 1] = torch.cuda.Event()
                done[l + 1].record(side)
            main.wait_event(done[l])
            decode(l)
    launch_chain_ordered()
    torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        launch_chain_ordered()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    t_launch_chain = min(ts)
    # host-link reference: a plain pinned -> device copy of the same size
    nbytes = cfg.selected_kv_bytes()
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, pin_memory=True)
    dst = torch.empty_like(src, device=dev)
    t_copy = eager_time(lambda: dst.copy_(src, non_blocking=True), reps=5)
    link = nbytes / t_copy / 1e9
    gbs = nbytes / t_gather / 1e9
    parts = chain * (t_sel + t_gather + t_dec)
    best = min(res_pool.items(), key=lambda kv: kv[1]["chain_ms"])
    for v in res_pool.values():
        v["overlap"] = parts / (v["chain_ms"] * 1e-3)
        v["host_link_gbs"] = chain * nbytes / (v["chain_ms"] * 1e-3) / 1e9
    t_or = oracle_time(lambda: O.decode_row(O.bf16_to_f64(inputs.bf16_bits(Qs[0][0, 0, :cfg.G].cpu())), kk, vv,
                                            bis[0][0, 0, 0].cpu().numpy(), T, 1.0 / math.sqrt(cfg.d)))
    res = {
        "workload": f"{cfg.name}: B={cfg.B}, H_q={cfg.H_q}, H_kv={cfg.H_kv}, T={T}, {nsm} blocks per row and layer "
                    f"from pinned host memory, {nh} distinct host layers ({2 * nh * cfg.B * cfg.H_kv * T * cfg.d * 2 / 1e9:.1f}"
                    f" GB pinned), chain of {chain}" + (f"; {note}" if note else ""),
        "gather_us": t_gather * 1e6,
        "gather_roofline": {"bound": "host link", "achieved_gbs": gbs, "peak_gbs": link,
                            "peak_kind": "measured pinned host -> device copy of the same size",
                            "frac": gbs / link, "algorithmic_bytes": int(nbytes)},
        "select_us": t_sel * 1e6,
        "decode_from_stage_us": t_dec * 1e6,
        "sum_of_parts_ms": parts * 1e3,
        "persistent_pool": res_pool,
        "persistent_pool_best": {"workgroups": int(best[0]), **best[1]},
        "per_layer_gather_launches": {"chain_ms": t_launch_chain * 1e3, "overlap": parts / t_launch_chain,
                                      "host_link_gbs": chain * nbytes / t_launch_chain / 1e9},
        "transfer_bound_ms": chain * nbytes / (link * 1e9) * 1e3,
        "oracle_rows_per_s": 1.0 / t_or, "gpu_rows_per_s": cfg.B * cfg.H_kv / t_dec,
    }
    del layers, host, kts
    torch.cuda.empty_cache()
    return res


def copy_calibration(nbytes=1 << 30):
    dev = "cuda"
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}))


def timed_graph(step, L, steps, per_graph=80):
    """Time exactly `steps` steps as HIP graph replays between synchronisations:
    one graph holds `per_graph` consecutive steps (a decode token through an
    80-layer stack, cycling the L resident layers), a second one the remainder;
    returns (wall seconds, steps)."""
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for i in range(L):
            step(i)
    torch.cuda.current_stream().wait_stream(warm)
    per_graph = max(L, per_graph // L * L)          # whole passes over the ring keep the lists chained

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(i)
        return g
    replays, rest = divmod(steps, per_graph)
    full = capture(per_graph) if replays else None
    tail = capture(rest) if rest else None
    torch.cuda.synchronize()
    for g in (full, tail):                           # one untimed replay of each
        if g is not None:
            g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        full.replay()
    if tail is not None:
        tail.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, steps


def call_time(prepared, reps, copies=8):
    """Mean device seconds per launch of the prepared calls, from `reps` replays
    of one graph holding `copies` passes over them, between two HIP events."""
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for c in prepared:
            c.run()
    torch.cuda.current_stream().wait_stream(warm)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(copies):
            for c in prepared:
                c.run()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * copies * len(prepared))


def launch_distribution(prepared, n=60):
    """Per-launch device time of a call: n eager launches cycling over the
    prepared calls (the resident layers), each bracketed by HIP events on the
    stream it runs on; median, p10 and p90 in us.  Each interval also holds
    the dispatch of its launch, so these sit a little above the graph means."""
    for c in prepared:
        c.run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        prepared[i % len(prepared)].run()
        evs[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)), "p90": float(np.percentile(t, 90)),
            "launches": n}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the other hot-path rows")
    ap.add_argument("--rows", help="comma-separated subset of the other rows: " + ",".join(ROW_NAMES))
    ap.add_argument("--no-graph", action="store_true", help="time eager prepared calls (for counter runs)")
    ap.add_argument("--overlap", action="store_true",
                    help="run layer l+1's selection on a side stream beside layer l's decode "
                         "(slower on this GPU: the two kernels contend for the same bandwidth and CUs)")
    ap.add_argument("--step", choices=("fused", "separate"), default="fused",
                    help="fused: one sda_decode_step call per layer (the decode launch finishes the next "
                         "layer's selection); separate: sda_score_select then sda_sparse_decode")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--step-refresh", action="store_true",
                    help="the step launch also refreshes the decoded layer's compressed keys for its newest token")
    ap.add_argument("--call-reps", type=int, default=50, help="graph replays per per-call timing")
    ap.add_argument("--profile", choices=("grouped",),
                    help="only run eager launches of one row for hardware-counter runs, then exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode path has no multi-GPU mode "
              "(sharding is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)
    # counting devices does not initialise the GPU: the CPU baseline below
    # forks its workers before anything does
    if torch.cuda.device_count() < 1:
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cfg = synth.get_config(args.config)
    cpu = None
    if not (args.no_cpu_baseline or args.copy_calibration or args.profile):
        cpu = cpu_baseline(cfg, args.layers)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.profile == "grouped":
        sda.lib()
        profile_grouped()
        return

    dev = "cuda"
    sda.lib()
    log(f"config {cfg.cid}: {cfg.name}; ring of {args.layers} layers")
    layers = build_layers(cfg, args.layers, dev)
    L = len(layers)
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=dev)
    n_sel_max = cfg.n_init + cfg.n_local + cfg.top_k
    bi = [torch.empty((cfg.B, 1, cfg.H_kv, n_sel_max), dtype=torch.int32, device=dev) for _ in range(L)]
    ns = [torch.empty((cfg.B, 1, cfg.H_kv), dtype=torch.int32, device=dev) for _ in range(L)]
    out = torch.empty((cfg.B, 1, cfg.H_q, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, 1, cfg.H_q), dtype=torch.float32, device=dev)
    ws_sel = torch.empty(sda.lib().sda_score_select_workspace(cfg.B, 1, cfg.H_kv, cfg.NB, cfg.top_k),
                         dtype=torch.uint8, device=dev)
    nb_dec = sda.lib().sda_sparse_decode_workspace(cfg.B, 1, cfg.H_q, cfg.H_kv, n_sel_max, cfg.d, args.split_k)
    ws_dec = torch.zeros(max(nb_dec, 16), dtype=torch.uint8, device=dev)   # counters start at zero
    # prepared calls: one (score_select, sparse_decode) pair per ring position;
    # layer i's indexer vectors score layer i+1's compressed keys
    calls = []
    for i in range(L):
        lc, ln = layers[(i - 1) % L], layers[i]
        sc, _ = sda.prepare(sda.sda_score_select, lc["F"], ln["kt"], seq, cfg.n_init, cfg.n_local, cfg.top_k,
                            block_idx=bi[i], n_sel=ns[i], ws=ws_sel)
        dc, _ = sda.prepare(sda.sda_sparse_decode, ln["Q"], ln["K"], ln["V"], seq, bi[i], ns[i], out=out,
                            lse=lse, split_k=args.split_k, ws=ws_dec)
        calls.append((sc, dc))
    # the step entry point: position i decodes layer i with bi[i] and selects
    # layer i+1's blocks (layer i's indexer vectors, layer i+1's compressed
    # keys); --step-refresh also refreshes layer i's compressed keys for its
    # newest token in the same launch (not part of the metric's step)
    ws_step = torch.zeros(sda.lib().sda_decode_step_workspace(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, n_sel_max,
                                                              args.split_k, cfg.NB, cfg.top_k),
                          dtype=torch.uint8, device=dev)
    seq_prev = seq - 1
    step_calls = []
    for i in range(L):
        lc, ln = layers[i], layers[(i + 1) % L]
        pc, _ = sda.prepare(sda.sda_decode_step, lc["Q"], lc["K"], lc["V"], seq, bi[i], ns[i], lc["F"], ln["kt"],
                            seq, cfg.n_init, cfg.n_local, cfg.top_k, block_idx_next=bi[(i + 1) % L],
                            n_sel_next=ns[(i + 1) % L], out=out, lse=lse, split_k=args.split_k,
                            k_tilde_cur=lc["kt"] if args.step_refresh else None, len_old_cur=seq_prev,
                            max_new_tokens_cur=1, ws=ws_step)
        step_calls.append(pc)

    def fused_step(i, ev=None):
        if ev is not None:
            ev[0].record()
            ev[1].record()
        step_calls[i % L].run()
        if ev is not None:
            ev[2].record()

    def step(i, ev=None):
        if args.step == "fused" and not args.overlap:
            return fused_step(i, ev)
        sc, dc = calls[i % L]
        if ev is not None:
            ev[0].record()
        sc.run()
        if ev is not None:
            ev[1].record()
        dc.run()
        if ev is not None:
            ev[2].record()

    # The selection for layer i+1 needs only layer i's indexer vectors and layer
    # i+1's compressed keys, so it runs on a side stream beside layer i's decode
    # (the lookahead overlap); the step joins both before layer i+1.
    side = torch.cuda.Stream()

    def pipelined_step(i):
        sc = calls[(i + 1) % L][0]
        dc = calls[i % L][1]
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            sc.run()
        dc.run()
        main.wait_stream(side)

    for i in range(max(args.warmup, L)):
        step(i)
    torch.cuda.synchronize()

    run_step = pipelined_step if args.overlap else step
    if args.no_graph:
        # eager: events on the launch stream around each call (the host
        # enqueues ahead of the GPU, so each interval also holds the dispatch)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        steps_timed = args.steps
        t_sel = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
        t_dec = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
        t_step = float((t_sel + t_dec).mean())
    else:
        wall, steps_timed = timed_graph(run_step, L, args.steps)
        # per-launch device time of each call: a graph of the ring's launches of
        # that call alone, replayed back to back between two HIP events on the
        # stream the graph runs on (inter-kernel gaps included)
        t_sel = np.array([call_time([c[0] for c in calls], args.call_reps)])
        t_dec = np.array([call_time([c[1] for c in calls], args.call_reps)])
        t_step = call_time(step_calls, args.call_reps)

    queries = cfg.B * cfg.NQ
    value = queries * steps_timed / wall
    dec_bytes = cfg.selected_kv_bytes()
    sel_bytes = cfg.ktilde_bytes()
    dec_gbs = dec_bytes / t_dec.mean() / 1e9
    step_fused = args.step == "fused" and not args.overlap
    # the dominant kernel of the timed step: the step launch (decode of layer l
    # plus scoring and selection of layer l+1), else the decode launch
    rl_key = "decode_step" if step_fused else "sparse_decode"
    # the step also refreshes the block of layer l's compressed keys that holds
    # the newest token: 64 keys read and one compressed key written per row
    ref_bytes = cfg.B * cfg.H_kv * (64 * cfg.d * 2 + cfg.d * 2) if args.step_refresh else 0
    rl_bytes = dec_bytes + sel_bytes + ref_bytes if step_fused else dec_bytes
    rl_gbs = rl_bytes / (t_step if step_fused else t_dec.mean()) / 1e9

    def counters_for(key):
        if not os.path.exists(PROFILE_COUNTERS):
            return None
        try:
            pc = json.load(open(PROFILE_COUNTERS))
            if pc.get("kernel_hash") == kernel_hash() and pc.get("config") == cfg.cid:
                return pc.get(key, {}).get("hbm_bytes_per_launch")
        except Exception:
            return None
        return None
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": wall / steps_timed * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B}, H_q={cfg.H_q}, H_kv={cfg.H_kv}, d={cfg.d}, T={cfg.T}, "
                        f"64-token blocks, {cfg.n_init} init + {cfg.n_local} local + top-{cfg.top_k}, "
                        f"F(layer l) . K~(layer l+1), ring of {L} resident layers",
            "global_batch": cfg.B,
            "seq_len": cfg.T,
            "parallelism": "single GPU",
            "config_id": cfg.cid,
            "launch": ("eager prepared calls" if args.no_graph else
                       f"HIP graphs of 80 consecutive steps (a token through an 80-layer stack over the {L} "
                       "resident layers), replayed")
                      + (", layer l+1's score_select beside layer l's sparse_decode (two streams)"
                         if args.overlap else
                         ", one sda_decode_step per layer (one launch: layer l's decode workgroups, then "
                         "workgroups that score layer l+1's compressed keys and select its block sets"
                         + (", then workgroups that refresh layer l's compressed keys for the newest token)"
                            if args.step_refresh else ")")
                         if args.step == "fused" else ", score_select then sparse_decode per layer"),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": rl_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": rl_gbs / HBM_PEAK_GBS,
            "traffic": counters_for(rl_key),
            "kernel": ("attn_kernel<128, 1, true> (sda_decode_step: layer l's decode and layer l+1's scoring "
                       "and selection in one launch" + (", with the refresh of layer l's compressed keys)"
                                                        if args.step_refresh else ")") if step_fused else
                       "attn_kernel<128, 1, false> (sda_sparse_decode; splits merged by the last workgroup of "
                       "each row)"),
            "algorithmic_bytes_per_launch": rl_bytes,
        },
        # the decode launch alone (sda_sparse_decode), against the same peak
        "roofline_decode": {
            "bound": "hbm",
            "achieved": dec_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS,
            "traffic": counters_for("sparse_decode"),
            "algorithmic_bytes_per_launch": dec_bytes,
        },
        "kernels_us": {
            "score_select": t_sel.mean() * 1e6,
            "sparse_decode": t_dec.mean() * 1e6,
            "decode_step": t_step * 1e6,
            "timing": ("eager: events around each call" if args.no_graph else
                       f"graph of {8 * L} back-to-back launches of the call, {args.call_reps} replays "
                       "between two HIP events"),
        },
        "score_select_gbs": sel_bytes / t_sel.mean() / 1e9,
        "queries_per_s_from_kernels": queries / (t_sel.mean() + t_dec.mean()),
        # one query = one sequence's token through all query heads of the layer
        "head_queries_per_s": value * cfg.H_q,
    }
    if not args.no_graph:
        res["kernels_us_per_launch"] = {
            "score_select": launch_distribution([c[0] for c in calls]),
            "sparse_decode": launch_distribution([c[1] for c in calls]),
            "decode_step": launch_distribution(step_calls),
            "timing": "eager launches cycling over the resident layers, HIP events around each on its stream",
        }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    if not args.no_rows:
        res["rows"] = measure_rows(cfg, layers, args.rows.split(",") if args.rows else None)
        # the pages' selection-cost comparison: the G-head selector's time over
        # the one-head indexer's on the same compressed keys
        ratio = {}
        if "a7_comparator" in res["rows"]:
            ratio["64/64 blocks"] = res["rows"]["a7_comparator"]["g_head_over_forecast"]
        if "n1_pooled_select" in res["rows"]:
            ratio["32/16 compressed keys, max-pooled"] = res["rows"]["n1_pooled_select"]["g_head_over_forecast"]
        if ratio:
            res["selection_cost_ratio_g_head_over_forecast"] = ratio
    print(json.dumps(res))


if __name__ == "__main__":
    main()
