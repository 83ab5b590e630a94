#!/usr/bin/env python3
"""Benchmark: top-k block-sparse decode on one MI355X.

One step = one layer's decode step of the 70B-shaped 128K workload: the
indexer vectors of layer l score layer l+1's compressed keys, top-k picks
the blocks (sda_score_select), and the query heads of layer l+1 attend to
them (sda_sparse_decode).  Steps walk a ring of distinct layers whose K/V,
compressed keys and vectors are all resident in HBM, so every step reads
cold data as a real layer stack does (the ring is larger than the L2 and
Infinity caches together).

Prints one JSON line.  `value` is whole-job queries/s over the timed steps
(one query = one sequence's decode token); `roofline` prices the decode
call (attention kernel + split combine) against the 8 TB/s HBM peak on its
algorithmic bytes (the selected K/V blocks); `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--config 3] [--layers L]
  python bench.py --copy-calibration     (plain copy of known size, for counter scaling)
"""
import argparse
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
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "sparse_decode_c3_counters.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_pool_amd", "csrc", "k_attention.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash():
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def build_layers(cfg, n_layers, dev):
    """K, V, compressed keys, indexer vectors and queries for a ring of layers."""
    layers = []
    for l in range(n_layers):
        t0 = time.time()
        K, V, _ = inputs.kv_layer(cfg, l, device=dev)
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


def cpu_baseline(cfg, layers, budget_s=12.0, n_rows=16):
    """Time the CPU oracle's per-step work (scores, top-k, block set,
    attention) on a sample of the same workload: the first n_rows (batch, KV
    head) rows of layer 1, scored by the indexer vectors of every layer of
    the ring in turn, until about budget_s seconds of timed work.  Building
    the oracle's compressed keys is setup, not timed."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    L = len(layers)
    ln = layers[1 % L]
    G, T = cfg.G, cfg.T
    scale = 1.0 / math.sqrt(cfg.d)
    rows = [(b, g) for b in range(cfg.B) for g in range(cfg.H_kv)][:n_rows]
    Qd = O.bf16_to_f64(inputs.bf16_bits(ln["Q"]))
    Fds = [O.bf16_to_f64(inputs.bf16_bits(l["F"])) for l in layers]
    data = {}
    for (b, g) in rows:
        kk = O.bf16_to_f64(inputs.bf16_bits(ln["K"][b, g]))
        vv = O.bf16_to_f64(inputs.bf16_bits(ln["V"][b, g]))
        data[(b, g)] = (kk, vv, O.store_bf16(O.compressed_keys(kk, T)))
    timed, done, passes = 0.0, 0, 0
    while timed < budget_s:
        Fd = Fds[passes % L]
        for (b, g) in rows:
            kk, vv, kt = data[(b, g)]
            t0 = time.perf_counter()
            blocks, _ = O.select_row(Fd[b, 0, g], kt, cfg.n_init, cfg.n_local, cfg.top_k)
            O.decode_row(Qd[b, 0, g * G:(g + 1) * G], kk, vv, blocks, T, scale)
            timed += time.perf_counter() - t0
            done += 1
        passes += 1
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    return {
        "value": done / timed / cfg.H_kv,
        "unit": "queries/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(rows)} (batch, KV head) rows of the 128K workload x {passes} passes "
                  f"(indexer vectors of each ring layer in turn) = {done} row-steps, {timed:.1f} s timed; "
                  f"float64 NumPy on one thread; per row: scores, top-k, block set, attention of "
                  f"{cfg.G} heads; a query = one sequence's {cfg.H_kv} KV heads",
    }


def copy_calibration(nbytes=1 << 30):
    dev = "cuda"
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}))


def timed_graph(step, L, steps):
    """Capture the L-step layer ring as one HIP graph, replay it for exactly
    `steps` steps (the remainder eagerly) between synchronisations; returns
    (wall seconds, steps)."""
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for i in range(L):
            step(i)
    torch.cuda.current_stream().wait_stream(warm)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(L):
            step(i)
    torch.cuda.synchronize()
    replays, rest = divmod(steps, L)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        graph.replay()
    for i in range(rest):
        step(i)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager prepared calls (for counter runs)")
    ap.add_argument("--overlap", action="store_true",
                    help="run layer l+1's selection on a side stream beside layer l's decode "
                         "(slower on this GPU: the two kernels contend for the same bandwidth and CUs)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--call-reps", type=int, default=50, help="graph replays per per-call timing")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode path has no multi-GPU mode "
              "(sharding is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    cfg = synth.get_config(args.config)
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

    def step(i, ev=None):
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
    else:
        wall, steps_timed = timed_graph(run_step, L, args.steps)
        # per-launch device time of each call: a graph of the ring's launches of
        # that call alone, replayed back to back between two HIP events on the
        # stream the graph runs on (inter-kernel gaps included)
        t_sel = np.array([call_time([c[0] for c in calls], args.call_reps)])
        t_dec = np.array([call_time([c[1] for c in calls], args.call_reps)])

    queries = cfg.B * cfg.NQ
    value = queries * steps_timed / wall
    dec_bytes = cfg.selected_kv_bytes()
    sel_bytes = cfg.ktilde_bytes()
    dec_gbs = dec_bytes / t_dec.mean() / 1e9
    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        try:
            pc = json.load(open(PROFILE_COUNTERS))
            if pc.get("kernel_hash") == kernel_hash() and pc.get("config") == cfg.cid:
                traffic = pc.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None
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
            "launch": ("eager prepared calls" if args.no_graph else f"HIP graph of the {L}-layer ring, replayed")
                      + (", layer l+1's score_select beside layer l's sparse_decode (two streams)"
                         if args.overlap else ", score_select then sparse_decode per layer"),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": dec_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": "sda_sparse_decode (attn_kernel; splits merged by the last workgroup of each row)",
            "algorithmic_bytes_per_launch": dec_bytes,
        },
        "kernels_us": {
            "score_select": t_sel.mean() * 1e6,
            "sparse_decode": t_dec.mean() * 1e6,
            "timing": ("eager: events around each call" if args.no_graph else
                       f"graph of {8 * L} back-to-back launches of the call, {args.call_reps} replays "
                       "between two HIP events"),
        },
        "score_select_gbs": sel_bytes / t_sel.mean() / 1e9,
        "queries_per_s_from_kernels": queries / (t_sel.mean() + t_dec.mean()),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, layers)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
