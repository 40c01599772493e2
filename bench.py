"""Decode-attention benchmark of the sparse-sketch path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config multi_agent_250k]

One step = one decode-attention layer for the whole batch: the APPEND key
sketch of the rows' own tokens, the query sketch, scoring every far token,
top-k selection and the gathered merged-softmax attention (all calls of the
C ABI on one stream).  Inputs are seeded synthetic caches resident in HBM
before timing starts.  `--replicas` distinct copies of the cache (standing in
for consecutive layers) are visited round-robin so that no step finds the
previous step's data in the last-level cache.

The steps run with SKS_STEP_NO_SCORES (the scores buffer is scratch), so
that long far regions take the candidate mode, which stores no scores;
--keep-scores stores them.

Prints ONE JSON line with steps/s, the roofline of the dominant kernel (the
score pass, HBM-bound) measured with HIP events on the launch stream, and the
CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "score_kernel_{workload}_hbm_counters.txt")
SCORE_SOURCES = ("k_score.hip", "sks_internal.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--lib", default=None,
                    help="load this build of the library instead of libsks.so (e.g. "
                         "libsks_attn_valu.so from `build --attn-valu`)")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="multi_agent_250k")
    ap.add_argument("--kv", choices=("bf16", "int8", "int4"), default=None,
                    help="store the workload's KV cache in another format (default: its own)")
    ap.add_argument("--context", type=int, default=None,
                    help="override the workload's context length (e.g. a short chat)")
    ap.add_argument("--dense", action="store_true",
                    help="time the dense step (no scoring or selection: each row attends its "
                         "last window + topk tokens), the switch's choice for short rows")
    ap.add_argument("--host-kv", action="store_true",
                    help="keep the full K/V in pinned host memory (read over PCIe for the "
                         "selected rows) with the window in a device ring")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--parts", type=int, default=1,
                    help="sub-batches per step (scheduled on --streams streams)")
    ap.add_argument("--streams", type=int, default=1)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying "
                    "a captured HIP graph")
    ap.add_argument("--steps-per-graph", type=int, default=0,
                    help="consecutive steps (one per cache replica) captured in one graph; "
                         "0 = all replicas")
    ap.add_argument("--five-calls", action="store_true",
                    help="issue each step as the five individual C-ABI calls instead of the one "
                         "sks_decode_step call")
    ap.add_argument("--keep-scores", action="store_true",
                    help="store the int32 scores in every step (no candidate mode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def algorithmic_bytes(cfg):
    """Bytes the method must move per step (per the row geometry of row 0..R-1).

    sketch: 64 B per far token/block per (b, KV head), one pass for all rows;
    gathered: one K and one V row per attended entry per (b, row, KV head);
    plus q in, out and idx out.
    """
    B, R, Hkv, Hq = cfg.B, cfg.R, cfg.Hkv, cfg.Hq
    row_bytes = cfg.kv_row_bytes + (0 if cfg.kv_dtype == 0 else 2)     # codes carry an fp16 scale
    n_far_max = cfg.n_far(R - 1)
    sketch = B * Hkv * n_far_max * 64
    gathered = sum(B * Hkv * cfg.n_attended(i) * 2 * row_bytes for i in range(R))
    small = B * R * Hq * 128 * 2 + B * R * Hq * 128 * 4 + B * R * Hkv * cfg.topk * 4
    return sketch, gathered, small


def counted_traffic(workload, mode):
    """HBM bytes per score launch (mode "candidates" or "stores") from the
    committed FETCH_SIZE / WRITE_SIZE counter summary (scaled by the
    copy-kernel calibration it records), or None when there is none for this
    workload and mode or the score kernel's sources have changed since the
    counters were taken."""
    import hashlib
    path = COUNTERS.format(workload=workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for ln in open(path):
        k, sep, v = ln.partition(":")
        if sep:
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(ROOT, "long_context_sparse_sketch_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if (fields.get("workload") != workload or fields.get("mode", "stores") != mode
            or fields.get("score_sources_sha256") != h.hexdigest()):
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(cfg, case, seconds):
    """Time the oracle's per-step functions on sequence 0 (a bounded sample),
    with NumPy's BLAS on every host core available to this process: three
    timed runs of about seconds / 3 each, the median reported."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import sks_oracle as orc

    g = cfg.g
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    with threadpool_limits(limits=cores):
        pools = [{k: p.get(k) for k in ("internal_api", "num_threads", "version")}
                 for p in threadpool_info()]
        qf = orc.bf16_to_f64(case.q)
        prep = []
        for h in range(cfg.Hkv):             # bulk key sketch: outside the timed region
            Kf, Vf = orc.cache_rows(case.K, case.V, case.K_scale, case.V_scale, 0, h,
                                    cfg.kv_dtype)
            Kp, Vp = orc.pool_mean(Kf, cfg.pool), orc.pool_mean(Vf, cfg.pool)
            _, kc = orc.key_sketch(Kp, case.basis, float(case.key_scale[h]))
            prep.append((Kf, Vf, Kp, Vp, kc))

        def one_sequence():
            for h in range(cfg.Hkv):
                Kf, Vf, Kp, Vp, kc = prep[h]
                for i in range(cfg.R):
                    Li = int(case.seq_len[0]) + i
                    n_far, ws = orc.row_geometry(Li, cfg.window, cfg.pool)
                    qc, _, _ = orc.query_sketch(qf[0, i, h * g:(h + 1) * g], case.basis)
                    sc = orc.scores(qc, kc[:n_far])
                    sel = orc.select_topk(sc, cfg.topk)
                    orc.attend(qf[0, i, h * g:(h + 1) * g],
                               np.concatenate([Kp[sel], Kf[ws:Li]]),
                               np.concatenate([Vp[sel], Vf[ws:Li]]), 1.0 / np.sqrt(128.0))

        runs = []
        for _ in range(3):
            reps, t0 = 0, time.perf_counter()
            while True:
                one_sequence()
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds / 3:
                    break
            runs.append((el / reps, reps, el))
    per_seq, _, _ = sorted(runs)[1]
    return {"value": 1.0 / (per_seq * cfg.B), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"sequence 0 of {cfg.B} ({cfg.Hkv} KV heads x {cfg.R} rows); median of 3 "
                      f"runs ({', '.join(f'{r} reps in {e:.1f} s' for _, r, e in runs)}); "
                      f"steps/s = 1 / ({cfg.B} x time per sequence); bulk key sketch excluded "
                      "as on the GPU",
            "os_cpu_count": os.cpu_count(), "threadpools": pools}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the sparse-sketch path here has no multi-GPU "
              "mode (each (sequence, KV head) pair would shard without communication).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from long_context_sparse_sketch_amd import binding as sks
    if args.lib:
        sks.LIB_PATH = os.path.abspath(args.lib)
    from long_context_sparse_sketch_amd import configs as C
    from long_context_sparse_sketch_amd.runtime import (SparseDecodeLayer, StepRunner,
                                                        capture_steps, to_device)
    from long_context_sparse_sketch_amd.synth import make_case

    cfg = C.BY_NAME[args.config]
    if args.kv is not None:
        cfg = C.with_kv(cfg, {v: k for k, v in C.KV_NAMES.items()}[args.kv])
    if args.context is not None:
        cfg = cfg.scaled(name=f"{cfg.name}_ctx{args.context}", L=args.context)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sks.lib()
    t_gen = time.perf_counter()
    case = make_case(cfg)
    print(f"[bench] generated {cfg.name} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)

    i8 = cfg.kv_dtype != C.KV_BF16          # int8 codes or packed int4 bytes, with row scales
    K0 = torch.from_numpy(case.K).to(dev) if i8 else to_device(case.K, dev, bf16=True)
    V0 = torch.from_numpy(case.V).to(dev) if i8 else to_device(case.V, dev, bf16=True)
    Ks0 = to_device(case.K_scale, dev) if i8 else None
    Vs0 = to_device(case.V_scale, dev) if i8 else None
    q = to_device(case.q, dev, bf16=True)
    sl = torch.from_numpy(case.seq_len.copy()).to(dev)
    basis = torch.from_numpy(case.basis).to(dev)
    kscale = torch.from_numpy(case.key_scale).to(dev)

    W_hot = cfg.window + cfg.R
    if args.host_kv:
        # full cache in pinned host memory; the window (and the rows' own
        # tokens) in a device ring of W_hot slots, position p in slot p % W_hot
        if cfg.pool > 1:
            raise SystemExit("--host-kv needs an unpooled workload")
        def ring_of(t):
            if t is None:
                return None
            end = int(case.seq_len[0]) + cfg.R - 1       # equal lengths in the workloads
            pos = torch.arange(max(0, end - W_hot), end, device=dev)
            r = torch.zeros((t.shape[0], t.shape[1], W_hot) + tuple(t.shape[3:]), dtype=t.dtype,
                            device=dev)
            r[:, :, pos % W_hot] = t[:, :, pos]
            return r
        hot0 = tuple(ring_of(t) for t in (K0, V0, Ks0, Vs0))
        K0, V0, Ks0, Vs0 = (None if t is None else t.cpu().pin_memory() for t in (K0, V0, Ks0, Vs0))
        torch.cuda.synchronize()
    copy = (lambda t: t.clone().pin_memory()) if args.host_kv else (lambda t: t.clone())

    layers = []
    for r in range(args.replicas):
        K = K0 if r == 0 else copy(K0)
        V = V0 if r == 0 else copy(V0)
        Ks = Ks0 if (r == 0 or Ks0 is None) else copy(Ks0)
        Vs = Vs0 if (r == 0 or Vs0 is None) else copy(Vs0)
        hot = None
        if args.host_kv:
            hot = tuple(None if t is None else (t if r == 0 else t.clone()) for t in hot0)
        cache = sks.Cache(K, V, sl, Ks, Vs, hot=hot)
        lay = SparseDecodeLayer(cfg.B, cfg.R, cfg.Hq, cfg.Hkv, cfg.T_max, cfg.window, cfg.topk,
                                cfg.pool, cfg.kv_dtype, dev).bind(cache, basis, kscale)
        lay.build_sketch(0, cfg.T_max)
        layers.append(lay)
    torch.cuda.synchronize()
    print(f"[bench] {args.replicas} cache replicas resident, sketches built", file=sys.stderr,
          flush=True)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    stream = torch.cuda.current_stream()
    runners = [StepRunner(lay, parts=args.parts, streams=args.streams, fused=not args.five_calls,
                          dense=args.dense, keep_scores=args.keep_scores)
               for lay in layers]
    # the step's own rule (sks.h, SKS_STEP_NO_SCORES): candidate mode for rows
    # of more than 8,192 far entries, with at most 65,536 far entries per row,
    # or one row per sequence and at least 2^20 far entries in all
    max_far = max(0, cfg.T_max - cfg.window) // cfg.pool
    cand = (not args.keep_scores and not args.dense and not args.five_calls and max_far > 8192
            and (max_far <= 65536 or (cfg.R == 1 and cfg.B * cfg.Hkv * max_far >= 1 << 20)))
    R_ = len(runners)
    spg = args.steps_per_graph or R_
    if R_ % spg:
        raise SystemExit("--replicas must be a multiple of --steps-per-graph")
    # graphs of spg consecutive layers, plus one single-step graph per layer for
    # step counts that do not fill a whole multi-step graph
    multi = [] if args.no_graph else [capture_steps(runners[i:i + spg], q)
                                      for i in range(0, R_, spg)]
    single = [] if args.no_graph or spg == 1 else [capture_steps([r], q) for r in runners]

    def run_steps(k0, n):
        """Steps k0 .. k0+n-1 (layer k % replicas), as eager launches or graph replays."""
        k = k0
        while k < k0 + n:
            if args.no_graph:
                runners[k % R_].step(q)
                k += 1
            elif (k % R_) % spg == 0 and k + spg <= k0 + n:
                multi[(k % R_) // spg].replay()
                k += spg
            else:
                (single[k % R_] if single else multi[k % R_]).replay()
                k += 1

    run_steps(0, args.warmup)
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # timed region: exactly K whole steps, nothing else on the stream
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    run_steps(args.warmup, args.steps)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)

    # spread: each multi-step graph replay timed on its own (per-step time =
    # replay time / steps per graph)
    spread = None
    if not args.no_graph:
        per = []
        for k in range(max(8, args.steps // spg)):
            a, b = ev(), ev()
            a.record(stream)
            multi[k % len(multi)].replay()
            b.record(stream)
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) / spg)
        spread = {f"p{p}": float(np.percentile(per, p)) for p in (10, 50, 90)}

    def launch_avg_ms(call):
        """Average duration of call(layer) over about K back-to-back launches,
        rotating the replicas, between two events on the launch stream.  The
        launches are one graph (one launch per replica) replayed K / replicas
        times, so that the host's launch rate does not bound short kernels;
        eager launches with --no-graph."""
        n = len(layers)
        a, b = ev(), ev()
        if args.no_graph:
            a.record(stream)
            for k in range(args.steps):
                call(layers[k % n])
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / args.steps
        for lay in layers:                   # warm up outside the capture
            call(lay)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for lay in layers:
                call(lay)
        torch.cuda.synchronize()
        reps = max(1, args.steps // n)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * n)

    # dominant kernel: its average launch duration -- in candidate mode the
    # score pass alone, on the estimates the steps left in each workspace
    stores_avg_ms = launch_avg_ms(lambda lay: lay.score())
    if cand:
        # the sample pass's estimates in the workspace timed here (the steps
        # ran through a view with a workspace of its own)
        for lay in layers:
            lay.score_candidates()
        score_avg_ms = launch_avg_ms(lambda lay: lay.score_candidates(flags=sks.CAND_KEEP_ESTIMATE))
    else:
        score_avg_ms = stores_avg_ms
    for lay in layers:                       # the extra histograms: back to zero at rest
        sks.workspace_init(lay.ws)
    # attention (gather + merged softmax) the same way, on each layer's last selection
    attn_avg_ms = launch_avg_ms(lambda lay: lay.attend(q))

    # standalone gather/pack of the same rows into packed buffers
    Cn = cfg.topk + cfg.window + cfg.pool - 1
    kdt = {C.KV_BF16: torch.bfloat16, C.KV_I8: torch.int8, C.KV_I4: torch.uint8}[cfg.kv_dtype]
    Ko = torch.empty((cfg.B, cfg.R, cfg.Hkv, Cn, case.K.shape[-1]), dtype=kdt, device=dev)
    Vo = torch.empty_like(Ko)
    Kso = torch.empty((cfg.B, cfg.R, cfg.Hkv, Cn), dtype=torch.int16, device=dev) if i8 else None
    Vso = torch.empty_like(Kso) if i8 else None
    n_out = torch.empty((cfg.B, cfg.R, cfg.Hkv), dtype=torch.int32, device=dev)
    gather_avg_ms = launch_avg_ms(lambda lay: sks.gather_pack(lay.cache, lay.p, lay.idx, Ko, Vo, n_out,
                                                              lay.Kp, lay.Vp, Kso, Vso))
    del Ko, Vo, Kso, Vso

    # basis refit over every cached key (off the per-step path; bf16 caches):
    # Gram matrix, eigenvectors, key scale, each timed on its own (median of 3)
    refit = None
    if cfg.kv_dtype == C.KV_BF16:
        lay = layers[0]
        rws = torch.empty(sks.refit_workspace_bytes(lay.cache, 0, cfg.T_max), dtype=torch.uint8,
                          device=dev)
        G = torch.empty((cfg.Hkv, 128, 128), dtype=torch.float64, device=dev)
        Pn = torch.empty((cfg.Hkv, 64, 128), dtype=torch.float32, device=dev)
        ksn = torch.empty(cfg.Hkv, dtype=torch.float32, device=dev)
        calls = {"gram": lambda: sks.refit_gram(lay.cache, 0, cfg.T_max, G, rws),
                 "basis": lambda: sks.refit_basis(G, Pn, rws),
                 "key_scale": lambda: sks.refit_key_scale(lay.cache, 0, cfg.T_max, Pn, ksn, rws)}
        refit = {}
        for name, fn in calls.items():
            ts = []
            for _ in range(3):
                a, b = ev(), ev()
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            refit[name + "_ms"] = float(np.median(ts))
        key_bytes = cfg.B * cfg.Hkv * cfg.L * cfg.kv_row_bytes
        refit["gram_GBps"] = key_bytes / (refit["gram_ms"] * 1e-3) / 1e9
        refit["key_scale_GBps"] = key_bytes / (refit["key_scale_ms"] * 1e-3) / 1e9
        del rws, G, Pn, ksn

    # per-phase breakdown (events between the calls of each step; includes
    # the events' own small overhead)
    names = ("append_sketch", "query_sketch", "score", "topk", "attention")
    evs = [[ev() for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        lay = layers[k % len(layers)]
        e = evs[k]
        e[0].record(stream)
        lay.build_sketch(sks.APPEND, 0)
        e[1].record(stream)
        lay.query_sketch(q)
        e[2].record(stream)
        if cand:
            lay.score_candidates()
        else:
            lay.score()
        e[3].record(stream)
        if cand:
            lay.select_candidates()
        else:
            lay.select()
        e[4].record(stream)
        lay.attend(q)
        e[5].record(stream)
    torch.cuda.synchronize()
    phase_ms = {n: float(np.median([evs[k][j].elapsed_time(evs[k][j + 1])
                                     for k in range(args.steps)])) for j, n in enumerate(names)}

    ms_per_step = total_ms / args.steps
    sketch_b, gather_b, small_b = algorithmic_bytes(cfg)
    # bytes of the selected far rows (K and V, with their scales): what crosses
    # PCIe with a host tier
    row_b = cfg.kv_row_bytes + (0 if cfg.kv_dtype == C.KV_BF16 else 2)
    selected_b = sum(cfg.B * cfg.Hkv * min(cfg.topk, cfg.n_far(i)) * 2 * row_b for i in range(cfg.R))
    achieved = sketch_b / (score_avg_ms * 1e-3) / 1e9
    line = {
        "metric": "decode-attn steps/s and achieved HBM GB/s (% peak) at 250K ctx, top-k 2048",
        "value": 1000.0 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"i8 sketch / {C.KV_NAMES[cfg.kv_dtype]} KV / f32 accumulate",
        "data": "synthetic (seeded N(0,1) caches with planted needles)",
        "config": {"workload": cfg.name + ("+host_kv" if args.host_kv else "")
                               + ("+dense" if args.dense else ""), "batch": cfg.B,
                   "context": cfg.L, "rows": cfg.R,
                   "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "window": cfg.window,
                   "topk": cfg.topk, "pool": cfg.pool, "replicas": args.replicas,
                   "schedule": ("five C-ABI calls" if args.five_calls else
                                "sks_decode_step" + (" (dense)" if args.dense else "")
                                + (" (candidate mode: scores not stored)" if cand else ""))
                               + f", {args.parts} sub-batches on {args.streams} streams, "
                               + ("eager launches" if args.no_graph else
                                  f"HIP graph replay ({spg} steps per graph)")
                               + (f", library {os.path.basename(args.lib)}" if args.lib else "")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counted_traffic(cfg.name, "candidates" if cand else "stores"),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                     "kernel": ("score pass in candidate mode (sks_score_candidates, "
                                "SKS_CAND_KEEP_ESTIMATE)" if cand else "sketch_score"),
                     "algorithmic_bytes": sketch_b,
                     "avg_ms": score_avg_ms,
                     "avg_ms_timing": ("HIP events around back-to-back launches, "
                                       + ("eager" if args.no_graph else
                                          "as graph replays (one launch per replica)"))},
        "detail": {
            "algorithmic_bytes_per_step": sketch_b + gather_b + small_b,
            "gathered_kv_bytes": gather_b,
            "score_with_stores_avg_ms": stores_avg_ms,
            "attn_avg_ms": attn_avg_ms,
            "attn_GBps": gather_b / (attn_avg_ms * 1e-3) / 1e9,
            "gather_pack_avg_ms": gather_avg_ms,
            "kv_tier": (f"host (pinned host K/V, device ring of {W_hot} slots)" if args.host_kv
                        else "device"),
            "host_selected_bytes": selected_b if args.host_kv else None,
            "attn_host_GBps": (selected_b / (attn_avg_ms * 1e-3) / 1e9 if args.host_kv else None),
            "gather_pack_GBps": 2 * gather_b / (gather_avg_ms * 1e-3) / 1e9,
            "step_ms_spread": spread,
            "refit": refit,
            "score_plus_attn_GBps": (sketch_b + gather_b) / ((score_avg_ms + attn_avg_ms) * 1e-3) / 1e9,
            "step_GBps": (sketch_b + gather_b + small_b) / (ms_per_step * 1e-3) / 1e9,
            "phase_ms_median": phase_ms,
        },
    }
    line["detail"]["score_plus_attn_frac"] = line["detail"]["score_plus_attn_GBps"] / HBM_PEAK_GBPS
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, case, args.cpu_seconds)
        # the oracle's rate over the step's algorithmic bytes, as for the GPU
        line["cpu_baseline"]["GBps"] = (line["cpu_baseline"]["value"]
                                        * line["detail"]["algorithmic_bytes_per_step"] / 1e9)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
