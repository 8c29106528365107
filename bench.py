"""Benchmark: µs per decode step per layer of the PRR path (select + speculate + repair) on one MI355X, and the
achieved HBM bandwidth of the dominant kernel against the 8 TB/s peak.

A "step" is one decode step of one attention layer: score_select, speculate over the predicted blocks, repair and
merge, and the EMA prediction for the next step (the whole hot path), on synthetic inputs resident in HBM. So that
consecutive steps do not run out of the 256 MB Infinity Cache, the timed loop rotates over L copies of the layer's
KV cache (distinct memory, like the layers of a model), with L chosen so the working set exceeds 512 MiB; the
reported time is per (step, layer).

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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--kspec", type=int, default=None, help="speculation budget (default: the workload's largest)")
    ap.add_argument("--layers", type=int, default=0, help="KV copies to rotate over (0 = auto)")
    ap.add_argument("--mode", default="prr_2stream", choices=["prr_2stream", "prr_1stream", "serialized"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--detail-out", default=None, help="also append the JSON line to this file")
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
    n_layers = a.layers or max(1, math.ceil(512 * 2 ** 20 / (kv_layer + summ_layer)))
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

    def timed(layers, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(layers, n)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (n * len(layers)) * 1e6

    # bytes each kernel must move per launch
    rows = w.batch * w.n_kv_heads
    blk_kv = w.block_size * 2 * w.head_dim * e
    alg = {"score": rows * w.n_blocks * 2 * w.head_dim * e,
           "select_topk": rows * w.n_blocks * 4,
           "ema_topk": rows * w.n_blocks * 12,
           "speculate": rows * kspec * blk_kv}

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
    alg["repair"] = rows * mean_missed * blk_kv if a.mode != "serialized" else rows * w.top_k * blk_kv

    # ---- per-kernel breakdown (traced pass) ------------------------------------------------------------------------
    layers = make_layers(a.mode)
    run(layers, a.warmup)
    cap = 64 * n_layers
    tr = L.Trace(cap)
    kern = ["score", "select_topk", "speculate", "repair", "finalize", "ema_topk"]
    tr.enable(kern)
    run(layers, 32)
    torch.cuda.synchronize()
    tr.disable()
    per_kernel = {}
    for k in kern:
        d = tr.read(k)
        if d:
            per_kernel[k] = float(np.mean(d[len(d) // 4:]) * 1e3)
    dominant = max((k for k in per_kernel if k in alg), key=lambda k: per_kernel[k])

    # ---- timed loop (headline mode), dominant kernel traced live on its own stream ---------------------------------
    tr.close()
    tr = L.Trace(a.steps * n_layers + 8)
    tr.enable([dominant])
    us = timed(layers, a.steps)
    tr.disable()
    d = tr.read(dominant)
    tr.close()
    dom_ms = float(np.mean(d)) if d else float("nan")
    achieved = alg[dominant] / (dom_ms * 1e-3) / 1e9
    for lay in layers:
        lay.close()

    # ---- the other modes for comparison ------------------------------------------------------------------------
    other = {}
    for mode in ("prr_2stream", "prr_1stream", "serialized"):
        if mode == a.mode:
            continue
        ls = make_layers(mode)
        run(ls, a.warmup)
        other[mode] = timed(ls, a.steps)
        for lay in ls:
            lay.close()

    attn_ms = (per_kernel.get("speculate", 0.0) + per_kernel.get("repair", 0.0)) * 1e-3
    attn_bytes = alg["speculate"] + alg["repair"] if a.mode != "serialized" else alg["repair"]
    detail = {
        "us_per_step": {a.mode: us, **other},
        "kernel_us": per_kernel,
        "attention_path_GBps": attn_bytes / (attn_ms * 1e-3) / 1e9 if attn_ms else None,
        "attention_path_frac": (attn_bytes / (attn_ms * 1e-3) / 1e9) / HBM_PEAK_GBS if attn_ms else None,
        "step_alg_bytes": alg["score"] + attn_bytes,
        "step_GBps": (alg["score"] + attn_bytes) / (us * 1e-6) / 1e9,
        "predictor_overlap": float(np.mean(overlap)) if overlap else None,
        "repaired_blocks_mean": mean_missed,
        "layers_rotated": n_layers,
        "working_set_MiB": n_layers * (kv_layer + summ_layer) / 2 ** 20,
    }
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
                     "alg_bytes_per_launch": alg[dominant], "avg_launch_us": round(dom_ms * 1e3, 3)},
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
