"""Benchmark: µs per decode step per layer of the PRR path (select + speculate + repair) on one MI355X, and the
achieved HBM bandwidth of the dominant kernel against the 8 TB/s peak.

A "step" is one decode step of one attention layer: score_select, speculate over the predicted blocks, repair and
merge, and the EMA prediction for the next step (the whole hot path), on synthetic inputs resident in HBM. So that
consecutive steps do not run out of the 256 MB Infinity Cache, the timed loop rotates over L layers (copies of the
KV cache, distinct memory, like the layers of a model), with L chosen so that the bytes one step touches times L
exceed 512 MiB (at most 32 layers and 48 GiB); the reported time is per (step, layer).

Prints ONE JSON line. `python bench.py --gpus N` with N > 1 exits: the benchmark runs on one GPU only.
"""
from __future__ import annotations

import argparse
import copy
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per decode step per layer (select+speculate+repair); KV GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0
# HIP kernels behind each traced launch
HIP_KERNELS = {("prr_fused", "score"): "score_kernel (the scores alone; the EMA is updated by the selection "
                                       "launch, except under a per-row budget below 128 rows)",
               ("prr_fused", "select_topk"): "the selection launch(es) by shape: select_spec_kernel (true top-K, "
                                             "next top-K', speculation over P_t), seg_spec_kernel + merge2_kernel "
                                             "(rows of more than 8192 blocks), select_missed_kernel (K <= 32, also "
                                             "the missed blocks), topk_pair_kernel (>= 128 rows; the speculation "
                                             "has its own launch)",
               ("prr_fused", "repair"): "repair_kernel + finalize_kernel (repair_kernel alone where one workgroup "
                                        "per row writes the output)",
               ("prr_fused", "finalize"): "merge_hits_kernel or finalize_kernel",
               ("prr_fused", "speculate"): "speculate_kernel",
               ("serialized", "repair"): "repair_kernel (+ finalize_kernel)",
               ("prr_1stream", "repair"): "repair_kernel (+ finalize_kernel)",
               ("prr_2stream", "repair"): "repair_kernel (+ finalize_kernel)"}


def parse():
    from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="paged_b32_64k", choices=list(WORKLOADS),
                    help="workload (default: the batched paged-KV layer, the largest that one GPU holds)")
    ap.add_argument("--kspec", type=int, default=None, help="speculation budget (default: the workload's largest)")
    ap.add_argument("--layers", type=int, default=0, help="KV copies to rotate over (0 = auto)")
    ap.add_argument("--mode", default="prr_fused",
                    choices=["prr_fused", "prr_2stream", "prr_1stream", "serialized", "serialized_fused"])
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--detail-out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--calibrate-mib", type=int, default=0,
                    help="before timing, stream-read and then stream-write a buffer of this many MiB once each (a "
                         "known byte count for scaling hardware traffic counters)")
    ap.add_argument("--budget-profile", action="store_true",
                    help="instead of the step benchmark: measure the selection time over a grid of block counts and "
                         "the speculation time over a grid of budgets K', and print the profiled budget K'*")
    ap.add_argument("--scorer", default="quest", choices=["quest", "mean"], help="block scorer")
    ap.add_argument("--sink", type=int, default=0, help="attention-sink blocks forced into every selection")
    ap.add_argument("--local", type=int, default=0, help="local-window blocks (the last ones) forced likewise")
    ap.add_argument("--budget", default="fixed", choices=["fixed", "misses", "confidence"],
                    help="per-row size of the predicted set (at most --kspec): fixed, K + ceil(beta * missed), or "
                         "the blocks whose optimistic score e + c|s - e| reaches the K-th EMA entry")
    ap.add_argument("--budget-beta", type=float, default=1.0, help="misses budget: blocks added per missed block")
    ap.add_argument("--budget-c", type=float, default=0.5, help="confidence budget: weight of |s - e|")
    ap.add_argument("--budget-kmin", type=int, default=0, help="smallest per-row budget (0: K, capped at --kspec)")
    ap.add_argument("--no-kspec-sweep", action="store_true",
                    help="skip the workload's speculation-budget sweep (e.g. for counter passes of one K')")
    ap.add_argument("--other-modes", default="all",
                    help="comma list of further modes to time beside --mode ('all' or 'none')")
    ap.add_argument("--no-budget-profile", action="store_true",
                    help="skip the profiled speculation budget K'* reported beside the fixed K'")
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path is not sharded across GPUs.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from dynamic_sparse_attention_decode_amd import _lib as L
    from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS
    from dynamic_sparse_attention_decode_amd.runtime import PRRLayer

    L.lib()   # fail loudly without the native library
    if a.calibrate_mib:
        buf = torch.empty((a.calibrate_mib << 20,), dtype=torch.uint8, device="cuda:0")
        sink = torch.zeros((65536,), dtype=torch.float32, device="cuda:0")
        L.flush_write(buf)          # first touch, not counted
        torch.cuda.synchronize()
        L.stream_read(buf, sink)
        L.flush_write(buf)
        torch.cuda.synchronize()
        del buf, sink
    w = WORKLOADS[a.workload]
    if a.sink or a.local or a.scorer != "quest":
        w = w.replace(sink_blocks=a.sink, local_blocks=a.local, scorer=a.scorer)
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp, gap_info = workload_inputs(w, dev)
    if a.budget_profile:
        print(json.dumps({"budget_profile": budget_profile(w, inp)}), flush=True)
        return
    kspec = max(w.k_spec) if a.kspec is None else a.kspec
    shape = L.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.page_size, w.n_blocks,
                         {"f32": L.F32, "bf16": L.BF16, "f16": L.F16}[w.dtype], w.scale,
                         ctx_len=w.ctx if w.ctx % w.block_size else 0, sink_blocks=w.sink_blocks,
                         local_blocks=w.local_blocks, scorer=L.SCORER_MEAN if w.scorer == "mean" else L.SCORER_QUEST)
    e = w.elem_bytes
    kv_layer = 2 * w.n_pages * w.n_kv_heads * w.page_size * w.head_dim * e
    summ_layer = w.batch * w.n_kv_heads * w.n_blocks * 2 * w.head_dim * e
    # Layers to rotate over: a real model visits every other layer between two visits of one layer, so the bytes one
    # step touches (summaries, scores and EMA, the true set's and the predicted set's KV) times the layers rotated
    # must exceed twice the 256 MB Infinity Cache, or later steps would read this layer's data from it. Capped at
    # 32 layers and 48 GiB of KV (the tiny workload stays cache-resident whatever the count).
    touched = (w.batch * w.n_kv_heads * (w.n_blocks * (2 * w.head_dim * e + 12)
                                         + (w.top_k + max(w.k_spec)) * w.block_size * 2 * w.head_dim * e))
    n_layers = a.layers or int(min(32, max(1, 48 * 2 ** 30 // (kv_layer + summ_layer)),
                                   max(1, math.ceil(512 * 2 ** 20 / touched))))
    kvs = [(inp.k_cache, inp.v_cache)] + [(inp.k_cache.clone(), inp.v_cache.clone()) for _ in range(n_layers - 1)]
    streams = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))
    qs = [inp.q[t].contiguous() for t in range(w.steps)]

    budget_cfg = None
    if a.budget != "fixed":
        budget_cfg = {"policy": a.budget, "beta": a.budget_beta, "c": a.budget_c,
                      "k_min": a.budget_kmin or min(w.top_k, kspec)}

    def make_layers(mode, k_spec=None, n_kv=None):
        ls = []
        kp = kspec if k_spec is None else k_spec
        for k, v in kvs[:n_kv]:
            bud = budget_cfg if kp > 0 else None
            if bud is not None and bud["k_min"] > kp:
                bud = dict(bud, k_min=kp)
            lay = PRRLayer(shape, w.top_k, kp, w.alpha, mode=mode, device=dev, streams=streams, budget=bud)
            lay.build(k, v, inp.table)
            ls.append(lay)
        torch.cuda.synchronize()
        return ls

    def run(layers, n):
        for _ in range(n):
            for lay in layers:
                lay.enqueue(qs[lay.t % w.steps])

    # bytes each kernel must move per launch (algorithmic: what the method reads and writes; partial-state records
    # are implementation overhead and not counted)
    rows = w.batch * w.n_kv_heads
    blk_kv = w.block_size * 2 * w.head_dim * e
    summ_b = rows * w.n_blocks * 2 * w.head_dim * e
    row_f32 = rows * w.n_blocks * 4

    # ---- statistics pass: overlap, missed blocks (untimed, per-step syncs) ---------------------------------------
    # The drifting workload moves its hot blocks as the workload defines it (the stored query draws keep the gap on
    # the drifted keys): on a copy of the keys, with the summaries of the moved blocks rebuilt before each such step.
    # The timed passes replay the steps on fixed keys; the rebuild is timed on its own (summary_rebuild_us).
    stat_inp = inp
    if w.drift_every:
        stat_inp = copy.copy(inp)
        stat_inp.k_cache, stat_inp.hot, stat_inp.saved = inp.k_cache.clone(), inp.hot.copy(), dict(inp.saved)
    stat = PRRLayer(shape, w.top_k, kspec, w.alpha, mode=a.mode, device=dev, streams=streams,
                    budget=budget_cfg if kspec > 0 else None)
    stat.build(stat_inp.k_cache, inp.v_cache, inp.table)
    missed, missed_max, overlap, pred_size = [], 0, [], []
    banded, instances = 0, 0
    for i in range(min(w.steps, 32)):
        ids = stat_inp.drift(stat.t) if w.drift_every else ()
        if len(ids):
            stat.rebuild_blocks(torch.as_tensor(ids, device=dev))
        stat.step(qs[stat.t % w.steps])
        stat.sync_spec()
        torch.cuda.synchronize()
        if stat.t > 1 and stat.k_spec:
            nm = stat.n_missed.cpu().numpy()
            missed.append(float(nm.mean()))
            missed_max = max(missed_max, int(nm.max()))
            overlap.append(float(1.0 - nm.mean() / w.top_k))
        if stat.k_spec:
            pred_size.append(float((stat.pred_next >= 0).sum(-1).float().mean()))
        if w.top_k < w.n_blocks:   # rows whose relative gap at the K-th score is within 1e-4 (several valid sets)
            srt = np.sort(stat.scores_last.cpu().numpy().reshape(-1, w.n_blocks), axis=1)[:, ::-1]
            sk, sk1 = srt[:, w.top_k - 1].astype(np.float64), srt[:, w.top_k].astype(np.float64)
            gap = (sk - sk1) / np.maximum(np.abs(sk), 1e-30)
            banded += int((gap <= 1e-4).sum())
            instances += len(gap)
    stat.close()
    mean_missed = float(np.mean(missed)) if missed else float(w.top_k)
    mean_pred = float(np.mean(pred_size)) if pred_size else float(kspec)   # filled slots of a predicted set
    prr_mode = not a.mode.startswith("serialized")

    # the fused step's many-row path (speculation in its own launch, a selection launch of top-K workgroups) serves
    # batches whose rows alone fill the chip
    many_row = rows >= 128
    # below 128 rows with a fixed budget, the fused step's selection launch updates the EMA (the workgroups that
    # predict P_{t+1}); under a per-row budget the scoring pass does
    sel_ema = not many_row and a.budget == "fixed"

    def alg_bytes(mode):
        """Algorithmic bytes per launch of each traced kernel in `mode`."""
        spec = rows * mean_pred * blk_kv
        rep = rows * (w.top_k if mode.startswith("serialized") else mean_missed) * blk_kv
        if mode == "prr_fused" and many_row:
            # speculation over P_t in its own launch; scores; the selection launch (T from the scores; P_{t+1} from
            # the EMA, which its workgroups update from the scores); the spread-out repair (its merge launch traced
            # as "finalize")
            return {"speculate": spec, "score": summ_b + row_f32, "select_topk": 4 * row_f32, "repair": rep}
        if mode == "prr_fused" and w.top_k <= 32:
            # the selection launch reads the scores (and the EMA, which its prediction workgroups update from them
            # under a fixed budget, else the scoring pass does), speculates over P_t and attends the missed blocks;
            # the merge launch (traced as "finalize") only reads partial records
            if sel_ema:
                return {"score": summ_b + row_f32, "select_topk": 4 * row_f32 + spec + rep}
            return {"score": summ_b + 3 * row_f32, "select_topk": 2 * row_f32 + spec + rep}
        if mode == "prr_fused" and sel_ema:
            # scores alone; the selection launch reads the scores for T, updates the EMA from them in the workgroups
            # that predict P_{t+1} (scores and EMA read, EMA written) and speculates over P_t; then the repair
            return {"score": summ_b + row_f32, "select_topk": 4 * row_f32 + spec, "repair": rep}
        if mode == "prr_fused":
            # per-row budget: scoring also updates the EMA; the selection launch reads scores and EMA and
            # speculates; then the repair
            return {"score": summ_b + 3 * row_f32, "select_topk": 2 * row_f32 + spec, "repair": rep}
        if mode == "serialized_fused" and rows >= 128:
            # two launches: scores, then selection with the row-wise attention and merge
            return {"score": summ_b + row_f32, "repair": row_f32 + rep}
        d = {"score": summ_b + row_f32, "select_topk": row_f32, "repair": rep}
        if mode != "serialized":
            d.update({"speculate": spec, "ema_topk": 3 * row_f32})
        return d

    alg = alg_bytes(a.mode)
    kern = list(alg) + ["finalize"]

    def measure(mode, trace_kernels=None, k_spec=None, n_kv=None):
        """Warm up eagerly, capture exactly a.steps steps (x layers) in a HIP graph, replay once untimed and once
        timed. Returns (us per step, per-kernel launch durations from the timed replay)."""
        ls = make_layers(mode, k_spec, n_kv)
        run(ls, a.warmup)
        torch.cuda.synchronize()
        tr = None
        if trace_kernels:
            tr = L.Trace(min(4096, a.steps * len(ls) + 8))
            tr.enable(trace_kernels)
        if a.eager:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run(ls, a.steps)
            torch.cuda.synchronize()
            us_ = (time.perf_counter() - t0) / (a.steps * len(ls)) * 1e6
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=streams[0]):
                for i in range(a.steps):
                    for li, lay in enumerate(ls):
                        lay.enqueue(qs[lay.t % w.steps], join=(i == a.steps - 1 and li == len(ls) - 1))
            if tr:
                tr.disable()
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            us_ = (time.perf_counter() - t0) / (a.steps * len(ls)) * 1e6
            del g   # a graph captured while tracing refers to the trace's events: release it before the trace
        durs = {}
        if tr:
            tr.disable()
            try:
                for k in trace_kernels:
                    d = tr.read(k)
                    if d:
                        durs[k] = float(np.mean(d)) * 1e3
            except L.PRRError as ex:
                print(f"[bench] kernel trace unavailable in this run: {ex}", file=sys.stderr, flush=True)
                durs = {}
            tr.close()
        for lay in ls:
            lay.close()
        return us_, durs

    def step_percentiles(mode):
        """Spread of the step time: the same warm-up and steps as measure(), each step (every layer once) captured as
        a graph of its own, the graphs replayed in order, each between two HIP events on the stream it runs on.
        Returns p10 / p50 / p90 of µs per layer-step (a graph launch per step adds its own start-up to each
        sample, so p50 sits a little above the one-graph average)."""
        ls = make_layers(mode)
        run(ls, a.warmup)
        torch.cuda.synchronize()
        graphs = []
        for i in range(a.steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=streams[0]):
                for li, lay in enumerate(ls):
                    lay.enqueue(qs[lay.t % w.steps], join=(li == len(ls) - 1))
            graphs.append(g)
        cur = torch.cuda.current_stream(dev)   # replay() launches a graph on the current stream
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in graphs]
        for g, (e0, e1) in zip(graphs, ev):
            e0.record(cur)
            g.replay()
            e1.record(cur)
        torch.cuda.synchronize()
        t = np.array([e0.elapsed_time(e1) * 1e3 / len(ls) for e0, e1 in ev])
        del graphs
        for lay in ls:
            lay.close()
        return {"p10": float(np.percentile(t, 10)), "p50": float(np.percentile(t, 50)),
                "p90": float(np.percentile(t, 90)), "samples": len(t),
                "how": "one graph per step (all layers), replayed in order between HIP events"}

    def isolated(mode, kernel):
        """Average duration (µs) of `kernel` alone: a HIP graph of a.steps x layers back-to-back launches of the one
        entry point that runs it, each with its layer's state after the warm-up steps, timed with HIP events on the
        stream the graph runs on. None when no entry point launches that kernel alone."""
        if mode == "serialized_fused" and rows >= 128:   # its repair launch is the selection launch too
            return None
        ls = make_layers(mode)
        run(ls, a.warmup)
        torch.cuda.synchronize()
        calls = []
        K = w.top_k
        for lay in ls:
            par, nxt = lay.t % 2, (lay.t + 1) % 2
            q = qs[lay.t % w.steps]
            kc = lay.k_spec if lay.t > 0 else 0
            if kernel == "score":
                # as the step scores: the EMA update rides in the scoring pass only under a per-row budget
                e = lay.ema.clone() if mode == "prr_fused" and not many_row and not sel_ema else None
                calls.append(lambda lay=lay, q=q, e=e, par=par: L.score(
                    shape, q, lay.summaries, lay.scores[par], e, w.alpha, False, stream=streams[0]))
            elif kernel == "select_topk" and mode == "prr_fused" and "repair" in alg:   # the select_spec launch
                kc = 0 if "speculate" in alg else kc   # many rows: the speculation has its own launch
                calls.append(lambda lay=lay, q=q, par=par, nxt=nxt, kc=kc: L.select_speculate(
                    shape, lay.scores[par], K, lay.sel_idx, lay.ema, lay.k_spec, lay.pred[nxt], q, lay.k_cache,
                    lay.v_cache, lay.table, lay.pred[par], kc, lay.partials[par], workspace=lay.workspace,
                    stream=streams[0], budget=lay.budgets[par] if lay.budgets else None))
            elif kernel == "speculate" and lay.k_spec:
                calls.append(lambda lay=lay, q=q, par=par: L.speculate(
                    shape, q, lay.k_cache, lay.v_cache, lay.table, lay.pred[par], lay.k_spec, lay.partials[par],
                    stream=streams[0]))
            elif kernel == "repair":   # the repair launch and its merge launch (one entry point)
                calls.append(lambda lay=lay, q=q, par=par, kc=kc: L.repair_merge(
                    shape, q, lay.k_cache, lay.v_cache, lay.table, lay.sel_idx, K, lay.pred[par] if kc else None, kc,
                    lay.partials[par] if kc else None, lay.out[par], lay.n_missed, lay.workspace, stream=streams[0]))
            else:
                break
        us_ = None
        if len(calls) == len(ls):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=streams[0]):
                for _ in range(a.steps):
                    for c in calls:
                        c()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            cur = torch.cuda.current_stream()   # replay() launches the graph on the current stream
            e0.record(cur)
            g.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            us_ = e0.elapsed_time(e1) * 1e3 / (a.steps * len(calls))
        for lay in ls:
            lay.close()
        return us_

    # per-kernel breakdown: HIP events around every launch in an eager pass of the same steps (PyTorch's HIP runtime
    # does not record timing events inside a captured graph); then the headline timed replay; then the dominant
    # kernel alone in a graph of back-to-back launches
    eager_flag, a.eager = a.eager, True
    _, per_kernel = measure(a.mode, kern)
    a.eager = eager_flag
    dominant = max((k for k in per_kernel if k in alg), key=lambda k: per_kernel[k])
    us, _ = measure(a.mode)
    iso = isolated(a.mode, dominant)
    if iso is not None:
        dom = {dominant: iso}
        dom_where = ("graph of back-to-back launches of its entry point" +
                     (" (repair and merge launches)" if dominant == "repair" else ""))
    else:
        dom = {dominant: per_kernel[dominant]}
        dom_where = "events around each launch in an eager pass of the same steps"
    dom_us = dom.get(dominant, float("nan"))
    dom_bytes = alg[dominant]
    if iso is not None and a.mode == "prr_fused" and dominant == "select_topk" and sel_ema:
        dom_bytes -= 2 * row_f32   # the selection entry point replayed alone reads the EMA without updating it
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    other = {}
    others = ("prr_fused", "prr_2stream", "prr_1stream", "serialized", "serialized_fused") \
        if a.other_modes == "all" else \
        tuple(m for m in a.other_modes.split(",") if m and m != "none")
    for mode in others:
        if mode != a.mode:
            other[mode] = measure(mode)[0]

    # selected-KV attention path: speculation + repair in the PRR modes, attend(T) (the repair launch with an empty
    # prediction) in the serialized mode; the fused mode speculates inside the selection launch, so its path time is
    # the whole selection launch
    if a.mode == "prr_fused" and "speculate" in alg:   # speculation in its own launch, then the repair
        attn_us = (per_kernel.get("speculate", 0.0) + per_kernel.get("repair", 0.0) + per_kernel.get("finalize", 0.0))
        attn_bytes = alg["speculate"] + alg["repair"]
    elif a.mode == "prr_fused" and "repair" not in alg:   # speculation and missed blocks in the selection launch
        attn_us = per_kernel.get("select_topk", 0.0) + per_kernel.get("finalize", 0.0)
        attn_bytes = rows * mean_pred * blk_kv + rows * mean_missed * blk_kv
    elif a.mode == "prr_fused":   # speculation in the selection launch, then the repair launch
        attn_us = per_kernel.get("select_topk", 0.0) + per_kernel.get("repair", 0.0)
        attn_bytes = rows * mean_pred * blk_kv + alg["repair"]
    elif a.mode == "serialized_fused" and rows >= 128:   # the repair launch also selects
        attn_us = per_kernel.get("repair", 0.0)
        attn_bytes = alg["repair"]
    else:
        attn_us = per_kernel.get("speculate", 0.0) + per_kernel.get("repair", 0.0)
        attn_bytes = alg.get("speculate", 0) + alg["repair"]
    detail = {
        "us_per_step": {a.mode: us, **other},
        "timing": "eager" if a.eager else "hip graph of all timed steps",
        "dominant_kernel_timed_in": dom_where,
        "kernel_us": per_kernel,
        "attention_path_GBps": attn_bytes / (attn_us * 1e-6) / 1e9 if attn_us else None,
        "attention_path_frac": (attn_bytes / (attn_us * 1e-6) / 1e9) / HBM_PEAK_GBS if attn_us else None,
        "step_alg_bytes": summ_b + attn_bytes,
        "predictor_overlap": float(np.mean(overlap)) if overlap else None,
        "budget": {"policy": a.budget, **({k: budget_cfg[k] for k in ("beta", "c", "k_min")} if budget_cfg else {}),
                   "k_spec_cap": kspec, "predicted_blocks_mean": mean_pred},
        "repaired_blocks_mean": mean_missed,
        "repaired_blocks_max": missed_max if missed else w.top_k,
        "banded_instances": {"count": banded, "of": instances,
                             "rule": "relative gap at the K-th score <= 1e-4 (from the device's scores)"},
        "gap_draws": gap_info,
        "layers_rotated": n_layers,
        "touched_MiB_per_step": touched / 2 ** 20,
        "working_set_MiB": n_layers * (kv_layer + summ_layer) / 2 ** 20,
    }
    detail["step_GBps"] = detail["step_alg_bytes"] / (us * 1e-6) / 1e9
    # the achievable streaming-read bandwidth of this GPU (2 GiB, beyond the Infinity Cache), for a second fraction
    rd = torch.empty((2 << 30,), dtype=torch.uint8, device=dev)
    rd_sink = torch.zeros((65536,), dtype=torch.float32, device=dev)
    L.flush_write(rd)
    L.stream_read(rd, rd_sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        L.stream_read(rd, rd_sink)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 5 * rd.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del rd, rd_sink
    detail["hbm_read_GBps_measured"] = read_gbs
    if not a.no_budget_profile:   # the profiled budget K'* beside the fixed K' of the line
        detail["budget_profile"] = budget_profile(w, inp, kvs, qs, steps=min(a.steps, 32))
    detail["attention_path_frac_of_measured"] = (detail["attention_path_GBps"] / read_gbs
                                                 if detail["attention_path_GBps"] else None)
    if not a.eager:
        detail["us_per_step_percentiles"] = step_percentiles(a.mode)
    if n_layers > 1:   # the same step with one layer only: its data stays in the Infinity Cache between steps
        detail["us_per_step_one_layer_cache_warm"] = measure(a.mode, n_kv=1)[0]
    if len(w.k_spec) > 1 and a.mode != "serialized" and not a.no_kspec_sweep:   # the workload sweeps its budget
        detail["us_per_step_by_kspec"] = {str(k): measure(a.mode, k_spec=k)[0] for k in w.k_spec}
    if w.drift_every:   # rebuilding the summaries of the blocks whose keys changed (not part of the step)
        lay = make_layers(a.mode)[0]
        ids = torch.as_tensor(inp.drift(w.drift_every), device=dev)
        lay.rebuild_blocks(ids)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            lay.rebuild_blocks(ids)
        e1.record()
        torch.cuda.synchronize()
        detail["summary_rebuild_us"] = {"blocks": int(ids.numel()), "us": e0.elapsed_time(e1) * 1e3 / 20}
        lay.close()
    # decode-time append (the step before selection in a decoder; not part of the timed step): one new token per
    # (sequence, KV head) written at the last slot of the sequences and its block's summary updated, as a graph of
    # 200 launches timed with HIP events on the stream the graph runs on (last, since it rewrites that slot)
    lay = make_layers(a.mode, n_kv=1)[0]
    gk = torch.Generator(device=dev).manual_seed(w.seed + 7)
    kn = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=gk, device=dev).to(w.torch_dtype)
    vn = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=gk, device=dev).to(w.torch_dtype)
    s_app = L.Shape.from_buffer_copy(shape)
    s_app.ctx_len = w.n_blocks * w.block_size
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=streams[0]):
        for _ in range(200):
            L.append_kv(s_app, kn, vn, lay.k_cache, lay.v_cache, lay.table, lay.summaries, stream=streams[0])
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gr.replay()
    e1.record()
    torch.cuda.synchronize()
    detail["append_us"] = e0.elapsed_time(e1) * 1e3 / 200
    lay.close()
    print(f"[bench] {json.dumps(detail)}", file=sys.stderr, flush=True)

    cpu = None if a.no_cpu else cpu_baseline(w, inp, kspec, a.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(us, 3), "unit": "us/step", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": us / 1e3, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "ctx": w.ctx, "block_size": w.block_size, "page_size": w.page_size,
                   "top_k": w.top_k, "k_spec": kspec, "alpha": w.alpha, "mode": a.mode,
                   "sink_blocks": w.sink_blocks, "local_blocks": w.local_blocks, "scorer": w.scorer,
                   "budget": a.budget, "layers_rotated": n_layers, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": dominant,
                     "hip_kernels": HIP_KERNELS.get((a.mode, dominant), dominant),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name, a.mode, dominant),
                     "alg_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3)},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    s = json.dumps(line)
    print(s, flush=True)
    if a.detail_out:
        with open(a.detail_out, "a") as f:
            f.write(s + "\n")


def workload_inputs(w, dev):
    """The workload's inputs with the stored gap-keeping query draws (tests/golden/gap_attempts/<workload>.json,
    written by a script that uses the oracle): on every (step, sequence, KV head) the oracle's relative score gap at
    the K-th boundary exceeds 1e-4, so the selection has one correct answer. A workload changed by the command line
    (forced blocks, another scorer) has no stored table and uses the first draws."""
    from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS, load_attempts, make_inputs

    path = os.path.join(ROOT, "tests", "golden", "gap_attempts", f"{w.name}.json")
    full = WORKLOADS.get(w.name)
    info = {"table": None}
    attempts = None
    if full is not None and full.key() == w.key() and os.path.exists(path):
        attempts = load_attempts(path, w)
        meta = json.load(open(path))
        info = {"table": os.path.relpath(path, ROOT), "banded": meta["banded"], "instances": meta["instances"],
                "mean_attempt": round(meta["mean_attempt"], 3)}
    return make_inputs(w, device=dev, attempts=attempts), info


def budget_profile(w, inp, kvs=None, qs=None, steps=20):
    """The profiling-guided speculation budget of the workload (dynamic_sparse_attention_decode_amd.profiling): the
    two-stream rule's tables (selection over a grid of block counts, speculation over a grid of budgets) and the
    fused step's table (whole steps at each grid budget, rotated over the same layers as the timed step), with K'*
    from each."""
    import torch

    from dynamic_sparse_attention_decode_amd import _lib as L
    from dynamic_sparse_attention_decode_amd import profiling as P

    dev = inp.k_cache.device
    dt = {"f32": L.F32, "bf16": L.BF16, "f16": L.F16}[w.dtype]
    shape = L.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.page_size, w.n_blocks, dt,
                         w.scale, ctx_len=w.ctx if w.ctx % w.block_size else 0, sink_blocks=w.sink_blocks,
                         local_blocks=w.local_blocks,
                         scorer=L.SCORER_MEAN if w.scorer == "mean" else L.SCORER_QUEST)
    k_grid = P.default_k_grid(w.top_k, w.n_blocks, w.k_spec)
    qs = qs or [inp.q[t].contiguous() for t in range(w.steps)]
    two = P.two_stream_tables(shape, w.top_k, qs[1 % len(qs)], inp.k_cache, inp.v_cache, inp.table, k_grid=k_grid,
                              seed=w.seed)
    fused = P.fused_step_table(shape, w.top_k, w.alpha, kvs or [(inp.k_cache, inp.v_cache)], inp.table, qs, k_grid,
                               steps=steps)
    torch.cuda.synchronize(dev)
    r2 = lambda xs: [round(x, 2) for x in xs]
    return {"workload": w.name, "n_target": w.n_blocks, "kspec_grid": k_grid,
            "two_stream": {"n_grid": two["n_grid"], "t_sel_us": r2(two["t_sel_us"]),
                           "t_sel_fit_us": round(two["t_sel_fit_us"], 2), "t_spec_us": r2(two["t_spec_us"]),
                           "kspec_star": two["kspec_star"]},
            "fused": {"t_step_us": r2(fused["t_step_us"]), "kspec_star": fused["kspec_star"]},
            "kspec_star_two_stream": two["kspec_star"], "kspec_star_fused": fused["kspec_star"]}


def source_digest() -> str:
    """sha256 over the HIP sources and the C header with comments and whitespace removed: a recorded counter value
    is valid only for the same kernels."""
    import hashlib
    import re

    def code(path):
        src = open(path).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        return " ".join(src.split()).encode()

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_decode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        h.update(name.encode() + b"\0" + code(os.path.join(csrc, name)))
    h.update(code(os.path.join(ROOT, "include", "prr.h")))
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, mode: str, kernel: str):
    """HBM bytes per launch of `kernel` from profiles/pmc_traffic.txt (FETCH_SIZE + WRITE_SIZE per dispatch, each
    scaled by the same counter's reading for a copy kernel of known size), or None when no entry matches the current
    kernel sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = source_digest()
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 5 and not line.startswith("#") and parts[:4] == [workload, mode, kernel, digest]:
                return float(parts[4])
    return None


def cpu_baseline(w, inp, kspec, seconds):
    """Time the fp64 oracle's decode step (scores from precomputed summaries, top-K, speculation partials and repair
    over the true set, EMA update and prediction) on a bounded sample of the same workload's rows, on the host's
    cores: the sampled (sequence, KV head) rows are independent, so each runs its own decode steps in its own thread
    (BLAS single-threaded inside each), until the time is up. The oracle itself is unchanged."""
    import threading
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import prr_oracle as O

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(16, cores))
    rows_all = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    per_row = 2 * w.ctx * w.head_dim * 8 + 2 * w.n_blocks * w.head_dim * 8
    n_rows = max(1, min(len(rows_all), 2 * cores, (8 << 30) // per_row))
    rng = np.random.default_rng(w.seed)
    rows = [rows_all[i] for i in sorted(rng.choice(len(rows_all), n_rows, replace=False))]
    print(f"[bench] cpu baseline: gathering {len(rows)} of {len(rows_all)} rows", file=sys.stderr, flush=True)
    data = {}
    for (b, g) in rows:
        pages = torch.as_tensor(inp.table_np[b], device=inp.k_cache.device, dtype=torch.long)
        k = inp.k_cache[pages, g].float().cpu().numpy().reshape(-1, w.head_dim)[:w.ctx].astype(np.float64)
        v = inp.v_cache[pages, g].float().cpu().numpy().reshape(-1, w.head_dim)[:w.ctx].astype(np.float64)
        kmin, kmax = O.block_summaries(k, w.block_size)
        data[(b, g)] = (k, v, kmin, kmax)
    G = w.group
    q = inp.q.float().cpu().numpy().astype(np.float64)
    done = {r: 0 for r in rows}
    stop = threading.Event()

    def run_row(r):
        b, g = r
        k, v, kmin, kmax = data[r]
        ema, pred = None, np.zeros((0,), dtype=np.int64)
        t = 0
        while not stop.is_set():
            qg = q[t % w.steps, b, g * G:(g + 1) * G]
            s_ = O.quest_scores(qg, kmin, kmax)
            T = O.top_k(s_, w.top_k)
            O.prr_output(qg, k, v, T, pred if t % w.steps else [], w.block_size, w.scale)
            ema = O.ema_update(ema, s_, w.alpha, t % w.steps == 0)
            pred = O.predict(ema, kspec) if kspec else np.zeros((0,), dtype=np.int64)
            t += 1
            done[r] = t

    with threadpool_limits(limits=1), ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        futs = [ex.submit(run_row, r) for r in rows]
        time.sleep(seconds)
        stop.set()
        for f in futs:
            f.result()
        el = time.perf_counter() - t0
    row_steps = sum(done.values())
    us = el / row_steps * 1e6 * len(rows_all)   # one step of every row at the measured aggregate rate
    return {"value": round(us, 1), "unit": "us/step", "cores": min(cores, len(rows)), "kind": "oracle",
            "sample": f"{row_steps} (sequence, KV head) decode steps over {len(rows)} of {len(rows_all)} rows in "
                      f"{min(cores, len(rows))} threads for {el:.1f} s, scaled to a step of all rows; fp64 numpy "
                      f"oracle as it stands (BLAS one thread per worker)"}


if __name__ == "__main__":
    main()
