"""Throughput of the eviction hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-others]

A step is one pass of the whole path over one batch of synthetic input, with
the inputs already resident in HBM.  The default workload is the largest one
that fits one GPU: KV² chunked scoring at the Qwen3-8B shape (36 layers, 32
query / 8 KV heads, d=128, bf16, N=131,072 in 32 chunks of 4,096 after 4
sinks, 410 reconstruction queries per chunk, keep 2% per (layer, KV head)).
Its step is one compression call: both scoring passes, the per-head top-k and
the compaction of K and V.  For the block-loop workload (EpiCache-style block
prefill, Llama-3.2-3B shape) a step is the whole 8-block loop, 6 compressions
of a 6,144-row cache back to 4,096 rows.

Prints one JSON line: the metric (scored cache tokens per second, i.e.
layers x KV heads x N summed over the scoring calls, per second), the roofline
of the dominant kernel from HIP events recorded around its launches inside the
timed region, the per-kernel averages, the float64 CPU oracle timed on a
bounded sample of the same workload, and (under "other_workloads") the same
figures for every other workload, measured in the same process.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
METRIC = "scored cache tokens/sec (Σ layers×kv_heads×N) + % peak MFMA; compact GB/s"
WORKLOADS = ["kv2_131k", "epicache_block_loop", "kv2_32k", "episodic", "tiny"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="kv2_131k", choices=WORKLOADS)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true",
                    help="time without per-launch events (for profiler runs)")
    ap.add_argument("--no-others", action="store_true",
                    help="measure the named workload only")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the next rows (query selection, global eviction, ...)")
    ap.add_argument("--other-steps", type=int, default=10,
                    help="timed steps of each other workload")
    ap.add_argument("--overlap-v", action="store_true",
                    help="block loop: gather V on a second stream beside the next step's scoring")
    return ap.parse_args()


def build_step(K, drivers, gen, torch, w, dev, overlap_v=False):
    """Inputs in HBM and the step function of workload w."""
    s = w.shape
    env = {}
    if w.kind == "block_loop":
        x = gen.block_loop_inputs(w, device=dev)
        loop = drivers.BlockLoop(s.layers, s.q_heads, s.kv_heads, s.head_dim, torch.bfloat16,
                                 w.block_len, w.budget_m, s.n_sinks, s.q_per_chunk, device=dev,
                                 overlap_v=overlap_v)
        calls = []
        n = 0
        for b in range(w.n_blocks):
            n += w.block_len
            if n > w.budget_m:
                calls.append(n)
                n = w.budget_m
        kl = [w.budget_m] * s.layers

        def step():
            loop.run(x["k_tokens"], x["v_tokens"], x["q_steps"])
        env["loop"] = loop
    else:
        if w.kind == "episodic":
            x = gen.episodic_inputs(w, device=dev)
            qs = x["q_episodes"]
            kl = [int(v) for v in K.kvs_layer_budgets(s.layers, w.total_budget, x["sens"], w.alpha,
                                                      s.n_cache, s.n_sinks)]
            total, sens, alpha = w.total_budget, x["sens"], w.alpha
        else:
            x = gen.single_inputs(w, device=dev)
            qs = x["q"][None]
            keep = w.keep_per_layer()
            kl = [keep] * s.layers
            total, sens, alpha = keep * s.layers, None, 0.0
        calls = [s.n_cache] * qs.shape[0]
        p = K.make_problem(s.layers, s.q_heads, s.kv_heads, s.head_dim, s.n_cache, s.n_sinks,
                           s.chunk_size, s.q_per_chunk, x["k"].dtype)
        rows = s.kv_heads * int(sum(kl))
        scores = torch.empty(s.layers * s.kv_heads * s.n_cache, device=dev)
        kept = torch.empty(rows, dtype=torch.int32, device=dev)
        ko = torch.empty(rows, s.head_dim, dtype=x["k"].dtype, device=dev)
        vo = torch.empty(rows, s.head_dim, dtype=x["k"].dtype, device=dev)
        ws = K.workspace(p, dev)

        def step():
            for e in range(qs.shape[0]):
                K.kvs_compress_block(p, qs[e], x["k"], x["v"], total, sens, alpha, scores, kept,
                                     ko, vo, 0, ws=ws)
        env.update(p=p, scores=scores, ws=ws)
    env.update(x=x, calls=calls, kl=kl)
    return step, env


def time_step(K, torch, step, steps, warmup, p1_name, trace):
    """Wall time per step over `steps` timed steps (events only around pass 1
    inside the timed region), then a per-kernel breakdown from a few more
    steps with every launch traced."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    K.kvs_trace_summary()  # drop anything recorded so far
    # Inside the timed region only the dominant kernel is bracketed by events
    # (two event records per launch of every kernel would add to the step).
    K.kvs_trace_only(p1_name)
    K.kvs_trace_enable(trace)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    K.kvs_trace_enable(False)
    timed_trace = K.kvs_trace_summary()
    ms_step = (t1 - t0) * 1e3 / steps
    breakdown, bd_steps = {}, max(1, min(steps, 5))
    if trace:
        K.kvs_trace_only(None)
        K.kvs_trace_enable(True)
        for _ in range(bd_steps):
            step()
        torch.cuda.synchronize()
        K.kvs_trace_enable(False)
        breakdown = K.kvs_trace_summary()
    return ms_step, timed_trace, breakdown, bd_steps


def figures(w, env, ms_step, timed_trace, trace, bd_steps):
    """Throughput and roofline figures of one workload's step."""
    s = w.shape
    calls, kl = env["calls"], env["kl"]
    L, Hq, Hkv, d = s.layers, s.q_heads, s.kv_heads, s.head_dim
    eb = s.elem_bytes()
    p1_name = "score_pass1_bf16" if s.dtype == "bf16" else "score_pass1_f32"
    p2_name = "score_pass2_bf16" if s.dtype == "bf16" else "score_pass2_f32"
    tokens = sum(L * Hkv * n for n in calls)
    shp = [s.__class__(L, Hq, Hkv, d, n, s.n_sinks,
                       (n - s.n_sinks) if w.kind == "block_loop" else s.chunk_size,
                       s.q_per_chunk, s.dtype) for n in calls]
    p1_flops = [2 * d * sh.pass1_pairs() for sh in shp]
    all_flops = sum(sh.counted_flops() for sh in shp)
    kept_rows = [Hkv * int(sum(kl))] * len(calls)
    sel_bytes = sum(4 * L * Hkv * n + 4 * r for n, r in zip(calls, kept_rows))
    cmp_bytes = sum(r * (2 * d * eb * 2 + 4) for r in kept_rows)

    def avg(name, tr):
        e = tr.get(name)
        return e["avg_ms"] if e else None

    def tot(name):
        e = trace.get(name)
        return e["total_ms"] / bd_steps if e else 0.0

    peak = PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_FP32_TFLOPS
    roofline = None
    if avg(p1_name, timed_trace):
        # per launch: the pass-1 flops of one scoring call (all calls of a step
        # share a shape); launch duration from the events recorded in the timed
        # region, on the stream the kernel is launched on
        per_launch = p1_flops[0]
        achieved = per_launch / (avg(p1_name, timed_trace) * 1e-3) / 1e12
        roofline = {"kernel": p1_name, "bound": "mfma" if s.dtype == "bf16" else "alu",
                    "achieved": round(achieved, 2),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": profiled_traffic(w.name, p1_name), "flops_per_launch": per_launch,
                    "avg_launch_ms": round(avg(p1_name, timed_trace), 5)}
    score_ms = tot(p1_name) + tot("score_merge_splits") + tot(p2_name)
    # the per-head selects are "select" (LDS-resident) and "select_*" (one
    # workgroup streaming, multi-workgroup)
    sel_ms = sum(tot(k) for k in trace if k == "select" or k.startswith("select_"))
    sc_ms = sel_ms + tot("compact")
    kernels = {k: {"avg_ms": round(v["avg_ms"], 5), "count_per_step": v["count"] / bd_steps}
               for k, v in trace.items()}
    return {
        "tokens": tokens, "value": tokens / (ms_step * 1e-3), "ms_per_step": round(ms_step, 4),
        "roofline": roofline,
        "score_mfma_frac": round(all_flops / (score_ms * 1e-3) / 1e12 / peak, 4) if score_ms else None,
        "select_compact_GBps": round((sel_bytes + cmp_bytes) / (sc_ms * 1e-3) / 1e9, 1) if sc_ms else None,
        "select_compact_hbm_frac": round((sel_bytes + cmp_bytes) / (sc_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
        if sc_ms else None,
        "select_GBps": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1) if sel_ms else None,
        "kernels": kernels,
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the eviction path is measured per GPU; see DESIGN.md for how it would shard.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_compression_kvs_amd as K
    from kv_cache_compression_kvs_amd import drivers
    from workloads import FULL, gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(K.LIB_PATH):
        from kv_cache_compression_kvs_amd import build as _b
        _b.build()
    dev = torch.device("cuda:0")
    w = FULL[args.workload]
    s = w.shape
    t_gen = time.perf_counter()
    step, env = build_step(K, drivers, gen, torch, w, dev, args.overlap_v)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    x, calls, kl = env["x"], env["calls"], env["kl"]

    # One plain copy of known size (224 slabs x 2048 rows x 256 B = 114,688 KiB),
    # outside the timed region: the scale for the FETCH_SIZE / WRITE_SIZE
    # counters of a rocprofv3 run of this script.
    csrc = torch.empty(224, 2048, 128, dtype=torch.bfloat16, device=dev)
    cdst = torch.empty_like(csrc)
    K.kvs_append_rows(224, 128, torch.bfloat16, csrc, 2048, 0, 2048, cdst, 2048, 0)
    torch.cuda.synchronize()
    del csrc, cdst

    # ---- timed region -----------------------------------------------------------
    p1_name = "score_pass1_bf16" if s.dtype == "bf16" else "score_pass1_f32"
    ms_step, timed_trace, trace, bd_steps = time_step(K, torch, step, args.steps, args.warmup,
                                                      p1_name, not args.no_trace)
    fig = figures(w, env, ms_step, timed_trace, trace, bd_steps)
    L, Hkv, d = s.layers, s.kv_heads, s.head_dim
    eb = s.elem_bytes()

    rec = {
        "metric": METRIC,
        "value": fig["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fig["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "q_heads": s.q_heads, "kv_heads": Hkv,
                   "head_dim": d, "n_cache_per_call": calls[0], "chunk_size": s.chunk_size,
                   "queries_per_chunk": s.q_per_chunk, "scoring_calls_per_step": len(calls),
                   "scored_tokens_per_step": fig["tokens"],
                   "keep_per_layer": kl[0] if kl else None,
                   "parallelism": "single GPU",
                   "v_gather": "second stream" if (w.kind == "block_loop" and args.overlap_v)
                   else "same stream"},
        "roofline": fig["roofline"],
        "score_mfma_frac": fig["score_mfma_frac"],
        "select_compact_GBps": fig["select_compact_GBps"],
        "select_compact_hbm_frac": fig["select_compact_hbm_frac"],
        "kernels": fig["kernels"],
        "input_generation_s": round(t_gen, 2),
    }
    next_rows = not (args.no_trace or args.no_next)
    p, scores, ws = env.get("p"), env.get("scores"), env.get("ws")

    # ---- stage-1 query selection on the final scores (KV² refinement pass) -------
    # Outside the timed step: the chunked workloads' stage-2 scores choose the
    # next pass's reconstruction queries (rho = 10%, as in their configs).
    if w.kind != "block_loop" and s.n_chunks > 1 and next_rows:
        rho = 0.1
        qcounts = K.kvs_query_counts(p, rho)
        qtotal = int(qcounts.sum())
        qpos = torch.empty(qtotal, dtype=torch.int32, device=dev)
        qws = torch.empty(max(K.kvs_query_workspace_bytes(p), 256), dtype=torch.uint8, device=dev)
        for _ in range(2):
            K.kvs_query_select(p, scores, rho, qpos, qws)
        torch.cuda.synchronize()
        K.kvs_trace_summary()
        K.kvs_trace_only(None)
        K.kvs_trace_enable(True)
        reps = 10
        for _ in range(reps):
            K.kvs_query_select(p, scores, rho, qpos, qws)
        torch.cuda.synchronize()
        K.kvs_trace_enable(False)
        qtr = K.kvs_trace_summary()
        q_ms = sum(v["total_ms"] for v in qtr.values()) / reps
        nc = s.n_cache - min(s.n_sinks, s.n_cache)
        q_bytes = 4 * L * Hkv * s.n_cache + 2 * 4 * nc + 4 * qtotal
        rec["next_rows"] = {"f1_query_select": {
            "rho": rho, "queries": qtotal, "ms_per_call": round(q_ms, 5),
            "algorithmic_bytes": q_bytes,
            "GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "kernels": {k: round(v["avg_ms"], 5) for k, v in qtr.items()}}}

    # ---- global eviction, ragged compaction and decode (KV² global budget) ------
    # Outside the timed step: the same scores evicted under one budget over
    # every (layer, KV head) (the per-layer total), the kept rows gathered into
    # a ragged cache, and one decode token attending it.
    if w.kind != "block_loop" and next_rows:
        rec["next_rows"] = rec.get("next_rows", {})
        rec["next_rows"]["f2_global"] = global_row(K, torch, p, s, x, scores, int(sum(kl)) * Hkv,
                                                   ws, dev)

    # ---- layer-sensitivity calibration over the cache's keys (EpiCache) --------
    # Outside the timed step: the similarity kernel streams two key tensors of
    # the workload's shape (here the cache's K and V stand in for the full- and
    # block-prefill keys; the arithmetic and traffic do not depend on values).
    if w.kind != "block_loop" and next_rows:
        sim = torch.empty(s.layers, dtype=torch.float64, device=dev)
        sws = torch.empty(max(K.kvs_similarity_workspace_bytes(p), 256), dtype=torch.uint8,
                          device=dev)
        for _ in range(2):
            K.kvs_key_similarity(p, x["k"], x["v"], sim, sws)
        torch.cuda.synchronize()
        K.kvs_trace_summary()
        K.kvs_trace_only(None)
        K.kvs_trace_enable(True)
        reps = 5
        for _ in range(reps):
            K.kvs_key_similarity(p, x["k"], x["v"], sim, sws)
        torch.cuda.synchronize()
        K.kvs_trace_enable(False)
        ctr = K.kvs_trace_summary()
        c_ms = sum(v["total_ms"] for v in ctr.values()) / reps
        c_bytes = 2 * L * Hkv * s.n_cache * d * eb
        rec["next_rows"] = rec.get("next_rows", {})
        rec["next_rows"]["f3_similarity"] = {
            "ms_per_call": round(c_ms, 5), "algorithmic_bytes": c_bytes,
            "GBps": round(c_bytes / (c_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(c_bytes / (c_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "kernels": {k: round(v["avg_ms"], 5) for k, v in ctr.items()}}

    # ---- episode clustering and matching (EpiCache) ------------------------------
    # Outside the timed step: 2048 unit-norm segment embeddings of width 1024
    # (a 90K-token history in segments of about 45 tokens) clustered into 4
    # episodes by 10 Lloyd rounds, the medoid of each episode, and 64 questions
    # matched to episodes.
    if next_rows and w.kind != "block_loop":
        rec["next_rows"] = rec.get("next_rows", {})
        rec["next_rows"]["f4_episodes"] = episode_row(K, torch, gen, FULL["episodic"].episodes, dev)

    # ---- float64 oracle on a bounded sample of the same workload ---------------
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds, kl)
        if "next_rows" in rec:
            oracle_rows(w, x, scores, rec["next_rows"], gen)

    # ---- every other workload, same process, same figures -----------------------
    if not args.no_others:
        del step, env, x, p, scores, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        others = {}
        for name in WORKLOADS:
            if name == w.name:
                continue
            wo = FULL[name]
            so = wo.shape
            t = time.perf_counter()
            ostep, oenv = build_step(K, drivers, gen, torch, wo, dev)
            torch.cuda.synchronize()
            tg = time.perf_counter() - t
            pn = "score_pass1_bf16" if so.dtype == "bf16" else "score_pass1_f32"
            ms_o, ttr_o, tr_o, bd_o = time_step(K, torch, ostep, args.other_steps, 2, pn,
                                                not args.no_trace)
            fo = figures(wo, oenv, ms_o, ttr_o, tr_o, bd_o)
            others[name] = {
                "ms_per_step": fo["ms_per_step"], "tokens_per_s": fo["value"],
                "scored_tokens_per_step": fo["tokens"], "steps": args.other_steps,
                "dtype": so.dtype,
                "pass1_frac": fo["roofline"]["frac"] if fo["roofline"] else None,
                "score_mfma_frac": fo["score_mfma_frac"],
                "select_compact_GBps": fo["select_compact_GBps"],
                "select_compact_hbm_frac": fo["select_compact_hbm_frac"],
                "select_GBps": fo["select_GBps"],
                "kernels": {k: v["avg_ms"] for k, v in fo["kernels"].items()},
                "input_generation_s": round(tg, 2)}
            print(f"[bench] {name}: {fo['ms_per_step']:.3f} ms per step", file=sys.stderr,
                  flush=True)
            del ostep, oenv
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        rec["other_workloads"] = others
    print(json.dumps(rec), flush=True)


def global_row(K, torch, p, s, x, scores, total, ws, dev):
    """Times kvs_select_global, kvs_compact_ragged and kvs_decode_ragged on the
    workload's final scores, with the algorithmic bytes of each."""
    L, Hq, Hkv, d, N = s.layers, s.q_heads, s.kv_heads, s.head_dim, s.n_cache
    eb = s.elem_bytes()
    U = L * Hkv
    kept = torch.empty(total, dtype=torch.int32, device=dev)
    offsets = torch.empty(U + 1, dtype=torch.int64, device=dev)
    ko = torch.empty(total, d, dtype=x["k"].dtype, device=dev)
    vo = torch.empty(total, d, dtype=x["k"].dtype, device=dev)
    q1 = torch.randn(L, Hq, d, device=dev).to(x["k"].dtype)
    out = torch.empty(L, Hq, d, device=dev)
    dws = torch.empty(max(K.kvs_decode_workspace_bytes(p, total), 256), dtype=torch.uint8,
                      device=dev)

    def once():
        K.kvs_select_global(p, scores, total, kept, offsets, ws)
        K.kvs_compact_ragged(p, x["k"], x["v"], kept, offsets, total, ko, vo)
        K.kvs_decode_ragged(p, q1, ko, vo, offsets, total, out, dws)

    for _ in range(2):
        once()
    torch.cuda.synchronize()
    K.kvs_trace_summary()
    K.kvs_trace_only(None)
    K.kvs_trace_enable(True)
    reps = 10
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    K.kvs_trace_enable(False)
    tr = K.kvs_trace_summary()
    counts = (offsets[1:] - offsets[:-1]).cpu()

    def ms(pred):
        return sum(v["total_ms"] for k, v in tr.items() if pred(k)) / reps

    sel_ms = ms(lambda k: k.startswith("select_"))
    cmp_ms = ms(lambda k: k == "compact_ragged")
    dec_ms = ms(lambda k: k.startswith("decode_"))
    sel_b = 4 * U * N + 4 * total + 8 * (U + 1)
    cmp_b = total * (2 * d * eb * 2 + 4)
    dec_b = total * 2 * d * eb + L * Hq * d * (eb + 4)

    def r(b, t):
        return {"ms": round(t, 5), "algorithmic_bytes": b, "GBps": round(b / (t * 1e-3) / 1e9, 1),
                "hbm_frac": round(b / (t * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}

    return {"total_budget": total, "head_rows_min": int(counts.min()),
            "head_rows_max": int(counts.max()),
            "select_global": r(sel_b, sel_ms), "compact_ragged": r(cmp_b, cmp_ms),
            "select_compact": r(sel_b + cmp_b, sel_ms + cmp_ms), "decode_ragged": r(dec_b, dec_ms),
            "kernels": {k: round(v["avg_ms"], 5) for k, v in tr.items()}}


def episode_row(K, torch, gen, E, dev):
    n, dim, rounds = 2048, 1024, 10
    emb = gen.episode_embeddings(n, dim, E, seed=0)
    x = emb["x"].to(dev)
    init = emb["x"][emb["init_index"]].contiguous().to(dev)
    q = emb["q"].to(dev)
    cent = torch.empty_like(init)
    assign = torch.empty(n, dtype=torch.int32, device=dev)
    med = torch.empty(E, dtype=torch.int32, device=dev)
    totals = torch.empty(n, device=dev)
    ep = torch.empty(q.shape[0], dtype=torch.int32, device=dev)

    def once():
        K.kvs_kmeans(x, init, rounds, cent, assign)
        K.kvs_medoids(x, assign, E, med, totals)
        K.kvs_match_episodes(q, cent, ep)

    for _ in range(2):
        once()
    torch.cuda.synchronize()
    K.kvs_trace_summary()
    K.kvs_trace_only(None)
    K.kvs_trace_enable(True)
    reps = 5
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    K.kvs_trace_enable(False)
    tr = K.kvs_trace_summary()
    a = assign.cpu()
    sizes = torch.bincount(a.long(), minlength=E)
    same_pairs = int((sizes.double() * (sizes.double() - 1) / 2).sum())
    # algorithmic: each distinct same-cluster pair once (a distance serves both
    # points), a subtract and a fused multiply-add per element; executed: the
    # 32 x 32 tile pairs (I <= J) of the cluster-sorted order whose cluster
    # ranges overlap, each formed whole
    tile = 32
    key = torch.sort(a.long()).values
    tiles = (n + tile - 1) // tile
    first = key[torch.arange(tiles) * tile]
    last = key[torch.clamp(torch.arange(tiles) * tile + tile - 1, max=n - 1)]
    formed = sum(int((last[i] >= first[i:]).sum()) for i in range(tiles))
    medoid_flops = 3 * dim * same_pairs
    executed_flops = 3 * dim * formed * tile * tile
    med_ms = tr["medoid_tile"]["avg_ms"] if "medoid_tile" in tr else None
    return {"segments": n, "dim": dim, "episodes": E, "lloyd_rounds": rounds,
            "ms_total": round(sum(v["total_ms"] for v in tr.values()) / reps, 5),
            "medoid_tile_ms": round(med_ms, 5) if med_ms else None,
            "medoid_TFLOPs": round(medoid_flops / (med_ms * 1e-3) / 1e12, 2) if med_ms else None,
            "medoid_fp32_frac": round(medoid_flops / (med_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)
            if med_ms else None,
            "medoid_executed_TFLOPs": round(executed_flops / (med_ms * 1e-3) / 1e12, 2)
            if med_ms else None,
            "labels_recovered": bool(torch.equal(a.long(), emb["labels"])),
            "kernels": {k: {"avg_ms": round(v["avg_ms"], 5), "count_per_call": v["count"] / reps}
                        for k, v in tr.items()}}


def profiled_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, calibrated against a plain copy), or
    None if there is none or the kernel source changed since it was taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        m = re.match(r"kernel=(\S+) traffic_bytes_per_launch=(\d+) source=(\S+) sha256_16=([0-9a-f]+)",
                     line.strip())
        if m and m.group(1) == kernel:
            src = os.path.join(ROOT, m.group(3))
            if not os.path.exists(src):
                return None
            h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
            return int(m.group(2)) if h == m.group(4) else None
    return None


def oracle_rows(w, x, scores, rows, gen):
    """The oracle beside each next row, on a bounded sample of the row's own
    input, in the row's unit: algorithmic GB/s of the sample (ms per call for
    the clustering, which is timed whole)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import oracle as O

    s = w.shape
    L, Hq, Hkv, d, N, S = s.layers, s.q_heads, s.kv_heads, s.head_dim, s.n_cache, s.n_sinks
    G, eb, U = s.group, s.elem_bytes(), s.layers * s.kv_heads
    threads = int(max((p.get("num_threads", 1) for p in threadpool_info()), default=1))

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    def base(value, unit, sample):
        return {"value": round(value, 3), "unit": unit, "cores": threads, "kind": "oracle",
                "sample": sample}

    def timed(fn):
        """Seconds per call of fn, repeated until half a second has passed (at most
        50 calls), and the last call's result."""
        n, t0 = 0, time.perf_counter()
        while True:
            out = fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= 0.5 or n >= 50:
                return dt / n, out

    sc = scores.view(L, Hkv, N).cpu().numpy()
    if "f1_query_select" in rows:
        r = rows["f1_query_select"]
        dt, _ = timed(lambda: O.select_queries(O.token_scores(sc), N, S, s.chunk_size, r["rho"]))
        r["cpu_baseline"] = base(r["algorithmic_bytes"] / dt / 1e9, "GB/s",
                                 f"the whole row: float64 token means of {U} units x {N} and the selection "
                                 f"of every chunk, {dt:.3f} s per call")
    if "f2_global" in rows:
        r = rows["f2_global"]
        us = 8  # the first 8 units (layer 0), the budget scaled to them
        need = (r["total_budget"] - U * S) * us // U
        tot = need + us * S
        s8 = sc[:1, :us].astype(np.float64)
        t_sel, kept = timed(lambda: O.select_global(s8, tot, S))
        k0, v0 = f64(x["k"][:1, :us]), f64(x["v"][:1, :us])
        t_cmp, (ko, vo) = timed(lambda: O.compact_ragged(k0, v0, kept))
        _, off = O.pack_ragged(kept)
        q1 = np.random.default_rng(0).standard_normal((1, us * G, d))
        t_dec, _ = timed(lambda: O.decode_attention(q1, ko, vo, off, us))
        sel_b, cmp_b = 4 * us * N + 4 * tot, tot * (2 * d * eb * 2 + 4)
        dec_b = tot * 2 * d * eb + us * G * d * (eb + 4)
        what = f"{us} of {U} units (layer 0), budget {tot} scaled to them"
        r["select_compact"]["cpu_baseline"] = base((sel_b + cmp_b) / (t_sel + t_cmp) / 1e9, "GB/s",
                                                   f"{what}, {t_sel + t_cmp:.3f} s per call")
        r["decode_ragged"]["cpu_baseline"] = base(dec_b / t_dec / 1e9, "GB/s",
                                                  f"{what}: {us * G} query heads, "
                                                  f"{t_dec:.4f} s per call")
    if "f3_similarity" in rows:
        r = rows["f3_similarity"]
        kf, kb = f64(x["k"][:1, :2]), f64(x["v"][:1, :2])
        dt, _ = timed(lambda: O.key_similarity(kf, kb))
        r["cpu_baseline"] = base(2 * 2 * N * d * eb / dt / 1e9, "GB/s",
                                 f"layer 0, 2 of {Hkv} KV heads x {N} positions, "
                                 f"{dt:.3f} s per call")
    if "f4_episodes" in rows:
        r = rows["f4_episodes"]
        emb = gen.episode_embeddings(r["segments"], r["dim"], r["episodes"], seed=0)
        xe = emb["x"].double().numpy()
        init, qe = xe[emb["init_index"].numpy()], emb["q"].double().numpy()

        def row():
            cent, assign = O.kmeans(xe, init, r["lloyd_rounds"])
            O.medoids(xe, assign, r["episodes"])
            return O.nearest_centroid(qe, cent)
        dt, _ = timed(row)
        r["cpu_baseline"] = base(dt * 1e3, "ms per call", f"the whole row, {dt:.2f} s per call")


def cpu_baseline(w, x, budget_s, kl):
    """The oracle, as it is, on a bounded sample of the workload until about
    budget_s seconds have been spent; reported in the metric's unit (scored
    positions per second).  For the block loop a sampled unit is carried
    through the oracle's own block loop (every scoring step); a one-chunk
    workload scores and selects whole (layer, KV head) units; a chunked one
    scores whole chunks of successive units (a chunk's scores need every one
    of its queries over the whole cache, which is where the time goes; the
    selection, which needs the whole unit, is left out)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import oracle as O

    s = w.shape
    G = s.group

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    done_tokens, spent, units, pieces = 0, 0.0, 0, 0
    chunked = w.kind != "block_loop" and s.n_chunks > 1
    for l in range(s.layers):
        for g in range(s.kv_heads):
            if w.kind == "block_loop":
                kt = f64(x["k_tokens"][l:l + 1, g:g + 1])
                vt = f64(x["v_tokens"][l:l + 1, g:g + 1])
                qs = f64(x["q_steps"][:, l:l + 1, g * G:(g + 1) * G])
                t = time.perf_counter()
                recs = O.block_loop(kt, vt, qs, w.block_len, w.budget_m, s.n_sinks)
                spent += time.perf_counter() - t
                done_tokens += sum(r["n_cache"] for r in recs if "kept" in r)
            elif chunked:
                qg = f64(x["q"][l, g * G:(g + 1) * G])
                kg = f64(x["k"][l, g])
                for r, (a, b) in enumerate(O.chunk_bounds(s.n_cache, s.n_sinks, s.chunk_size)):
                    t = time.perf_counter()
                    O.chunk_scores(qg, kg, r, s.n_sinks, s.chunk_size, s.q_per_chunk)
                    spent += time.perf_counter() - t
                    done_tokens += b - a
                    pieces += 1
                    if spent >= budget_s:
                        break
            else:
                q_all = x["q_episodes"][0] if w.kind == "episodic" else x["q"]
                qg = f64(q_all[l, g * G:(g + 1) * G])
                kg = f64(x["k"][l, g])
                t = time.perf_counter()
                sc = O.unit_scores(qg, kg, s.n_sinks, s.chunk_size, s.q_per_chunk)
                O.select_unit(sc, int(kl[l]), s.n_sinks)
                spent += time.perf_counter() - t
                done_tokens += s.n_cache
            units += 1
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    if w.kind == "block_loop":
        what = (f"{units} of {s.layers * s.kv_heads} (layer, KV head) units of {w.name}: the "
                f"oracle's block loop (every scoring step, selection and compaction)")
    elif chunked:
        what = (f"{pieces} chunks ({done_tokens} positions, every query of each chunk over all "
                f"{s.n_cache} cached keys) of {units} of {s.layers * s.kv_heads} (layer, KV head) "
                f"units of {w.name}: float64 chunk scores")
    else:
        what = (f"{units} of {s.layers * s.kv_heads} (layer, KV head) units of {w.name}: float64 "
                f"scores and selection of one scoring call")
    return {"value": done_tokens / spent, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{what}, {spent:.1f} s",
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
