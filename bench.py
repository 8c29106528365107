"""Benchmark: µs per decode step per layer of the PRR path (select + speculate + repair) on one MI355X, and the
achieved HBM bandwidth of the dominant kernel against the 8 TB/s peak.

A "step" is one decode step of one attention layer: score_select, speculate over the predicted blocks, repair and
merge, and the EMA prediction for the next step (the whole hot path), on synthetic inputs resident in HBM. So that
consecutive steps do not run out of the 256 MB Infinity Cache, the timed loop rotates over L copies of the layer's
KV cache (distinct memory, like the layers of a model), with L (at most 8) chosen so the working set exceeds
512 MiB where 8 copies suffice; the reported time is per (step, layer).

Prints ONE JSON line. `python bench.py --gpus N` with N > 1 exits: this build runs on one GPU only.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per decode step per layer (select+speculate+repair); KV GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--kspec", type=int, default=None, help="speculation budget (default: the workload's largest)")
    ap.add_argument("--layers", type=int, default=0, help="KV copies to rotate over (0 = auto)")
    ap.add_argument("--mode", default="prr_fused",
                    choices=["prr_fused", "prr_2stream", "prr_1stream", "serialized", "serialized_fused"])
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--detail-out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--other-modes", default="all",
                    help="comma list of further modes to time beside --mode ('all' or 'none')")
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
    from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS, make_inputs
    from dynamic_sparse_attention_decode_amd.runtime import PRRLayer

    L.lib()   # fail loudly without the native library
    w = WORKLOADS[a.workload]
    kspec = max(w.k_spec) if a.kspec is None else a.kspec
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = make_inputs(w, device=dev)
    shape = L.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.page_size, w.n_blocks,
                         {"f32": L.F32, "bf16": L.BF16, "f16": L.F16}[w.dtype], w.scale)
    e = w.elem_bytes
    kv_layer = 2 * w.n_pages * w.n_kv_heads * w.page_size * w.head_dim * e
    summ_layer = w.batch * w.n_kv_heads * w.n_blocks * 2 * w.head_dim * e
    n_layers = a.layers or min(8, max(1, math.ceil(512 * 2 ** 20 / (kv_layer + summ_layer))))
    kvs = [(inp.k_cache, inp.v_cache)] + [(inp.k_cache.clone(), inp.v_cache.clone()) for _ in range(n_layers - 1)]
    streams = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))
    qs = [inp.q[t].contiguous() for t in range(w.steps)]

    def make_layers(mode):
        ls = []
        for k, v in kvs:
            lay = PRRLayer(shape, w.top_k, kspec, w.alpha, mode=mode, device=dev, streams=streams)
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
    stat = make_layers(a.mode)[0]
    missed, overlap = [], []
    for i in range(min(w.steps, 32)):
        stat.step(qs[stat.t % w.steps])
        torch.cuda.synchronize()
        if stat.t > 1 and stat.k_spec:
            nm = stat.n_missed.cpu().numpy()
            missed.append(float(nm.mean()))
            overlap.append(float(1.0 - nm.mean() / w.top_k))
    stat.close()
    mean_missed = float(np.mean(missed)) if missed else float(w.top_k)
    prr_mode = not a.mode.startswith("serialized")

    def alg_bytes(mode):
        """Algorithmic bytes per launch of each traced kernel in `mode`."""
        spec = rows * kspec * blk_kv
        rep = rows * (w.top_k if mode.startswith("serialized") else mean_missed) * blk_kv
        if mode == "prr_fused":
            # two launches: scores + EMA update + speculation, then selection (true and next predicted sets) with the
            # row-wise repair and merge
            return {"score": summ_b + 3 * row_f32 + spec, "repair": 2 * row_f32 + rep}
        if mode == "serialized_fused":
            return {"score": summ_b + row_f32, "repair": row_f32 + rep}
        d = {"score": summ_b + row_f32, "select_topk": row_f32, "repair": rep}
        if mode != "serialized":
            d.update({"speculate": spec, "ema_topk": 3 * row_f32})
        return d

    alg = alg_bytes(a.mode)
    kern = list(alg) + ["finalize"]

    def measure(mode, trace_kernels=None):
        """Warm up eagerly, capture exactly a.steps steps (x layers) in a HIP graph, replay once untimed and once
        timed. Returns (us per step, per-kernel launch durations from the timed replay)."""
        ls = make_layers(mode)
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

    # per-kernel breakdown (traced), then the headline timed replay with only the dominant kernel traced
    _, per_kernel = measure(a.mode, kern)
    if not per_kernel:
        eager_flag, a.eager = a.eager, True
        _, per_kernel = measure(a.mode, kern)
        a.eager = eager_flag
    dominant = max((k for k in per_kernel if k in alg), key=lambda k: per_kernel[k])
    us, dom = measure(a.mode, [dominant])
    dom_where = "timed region"
    if dominant not in dom:   # events could not be recorded inside the graph: time that kernel in an eager pass
        eager_flag, a.eager = a.eager, True
        _, dom = measure(a.mode, [dominant])
        a.eager = eager_flag
        dom_where = "eager pass of the same steps"
    dom_us = dom.get(dominant, float("nan"))
    achieved = alg[dominant] / (dom_us * 1e-6) / 1e9
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
    if a.mode in ("prr_fused", "serialized_fused"):   # the repair launch also selects; speculation is in "score"
        attn_us = per_kernel.get("repair", 0.0)
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
        "repaired_blocks_mean": mean_missed,
        "layers_rotated": n_layers,
        "working_set_MiB": n_layers * (kv_layer + summ_layer) / 2 ** 20,
    }
    detail["step_GBps"] = detail["step_alg_bytes"] / (us * 1e-6) / 1e9
    print(f"[bench] {json.dumps(detail)}", file=sys.stderr, flush=True)

    cpu = None if a.no_cpu else cpu_baseline(w, inp, kspec, a.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(us, 3), "unit": "us/step", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": us / 1e3, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "ctx": w.ctx, "block_size": w.block_size, "page_size": w.page_size,
                   "top_k": w.top_k, "k_spec": kspec, "alpha": w.alpha, "mode": a.mode,
                   "layers_rotated": n_layers, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "alg_bytes_per_launch": alg[dominant], "avg_launch_us": round(dom_us, 3)},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    s = json.dumps(line)
    print(s, flush=True)
    if a.detail_out:
        with open(a.detail_out, "a") as f:
            f.write(s + "\n")


def cpu_baseline(w, inp, kspec, seconds):
    """Time the fp64 oracle's decode step (scores from precomputed summaries, top-K, speculation partials and repair
    over the true set, EMA update and prediction) on a bounded sample of the same workload's rows."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import prr_oracle as O

    rows_all = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    budget_bytes = 2 * 2 ** 30
    per_row = 2 * w.ctx * w.head_dim * 8
    rows = rows_all[:max(1, min(len(rows_all), budget_bytes // per_row))]
    print(f"[bench] cpu baseline: gathering {len(rows)} of {len(rows_all)} rows", file=sys.stderr, flush=True)
    data = {}
    for (b, g) in rows:
        import torch
        pages = torch.as_tensor(inp.table_np[b], device=inp.k_cache.device, dtype=torch.long)
        k = inp.k_cache[pages, g].float().cpu().numpy().reshape(w.ctx, w.head_dim).astype(np.float64)
        v = inp.v_cache[pages, g].float().cpu().numpy().reshape(w.ctx, w.head_dim).astype(np.float64)
        kmin, kmax = O.block_summaries(k, w.block_size)
        data[(b, g)] = (k, v, kmin, kmax)
    G = w.group
    q = inp.q.float().cpu().numpy().astype(np.float64)
    ema = {r: None for r in rows}
    pred = {r: np.zeros((0,), dtype=np.int64) for r in rows}
    steps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            t = steps % w.steps
            for (b, g) in rows:
                k, v, kmin, kmax = data[(b, g)]
                qg = q[t, b, g * G:(g + 1) * G]
                s = O.quest_scores(qg, kmin, kmax)
                T = O.top_k(s, w.top_k)
                O.prr_output(qg, k, v, T, pred[(b, g)] if t else [], w.block_size, w.scale)
                ema[(b, g)] = O.ema_update(ema[(b, g)], s, w.alpha, t == 0)
                pred[(b, g)] = O.predict(ema[(b, g)], kspec) if kspec else np.zeros((0,), dtype=np.int64)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    us = el / steps * 1e6 * len(rows_all) / len(rows)
    return {"value": round(us, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
            "sample": f"{steps} decode steps over {len(rows)} of {len(rows_all)} (sequence, KV head) rows, "
                      f"scaled to all rows; fp64 numpy, one thread ({el:.1f} s)"}


if __name__ == "__main__":
    main()
