"""Latency tables for the profiling-guided speculation budget, measured on the device.

PRR abstract: the speculation budget is chosen from profiled latencies so that speculative work stays off the
critical path; PRR summary page, Limitations: the overheads come from profiled grids, with polynomial regression for
context lengths outside them. Two windows are profiled:

* two-stream step (speculation on its own stream beside the selection): t_sel(N), the time of the whole selection
  (scores and top-K) on a grid of block counts N, and t_spec(K'), the time of the speculation launch alone on a grid
  of budgets; K'* = the largest K' with t_spec(K') <= t_sel at the layer's N (prr_choose_budget, a degree-2
  least-squares polynomial in N off the grid; the grid leaves out the layer's own N so the fit is exercised, except
  at the top-K kernels' largest N, where the fit would have to extrapolate).
* fused single-stream step (speculation inside the selection launch): t_step(K'), the time of whole decode steps of
  the layer at each grid budget, predicted sets from the layer's own EMA; K'* = the largest K' whose step is no
  slower than the step without speculation (prr_choose_budget_fused).

Every launch goes through the C ABI; PyTorch supplies device memory, streams and timing events. Each time is a graph
of back-to-back calls, replayed once untimed and once between HIP events on the stream the graph runs on.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L
from .runtime import PRRLayer


def graph_us(fn, reps: int, device) -> float:
    """µs per call of fn(stream): ``reps`` calls captured in one graph, the second replay timed."""
    fn(None)
    torch.cuda.synchronize(device)
    s = torch.cuda.Stream(device=device)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            fn(s)
    g.replay()
    torch.cuda.synchronize(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream(device)   # replay() launches the graph on the current stream
    e0.record(cur)
    g.replay()
    e1.record(cur)
    torch.cuda.synchronize(device)
    return e0.elapsed_time(e1) * 1e3 / reps


def default_n_grid(n_blocks: int) -> list:
    """Block counts around the layer's, within the top-K kernels' range. The layer's own N is left out, so the
    off-grid fit is used, where the range reaches past it; at the range's end the grid holds the layer's N itself,
    since a fit could only extrapolate there (a quadratic through concave points turns down past the last one)."""
    grid = {n for n in (n_blocks // 8, n_blocks // 4, n_blocks // 2, n_blocks * 2, n_blocks * 4) if 64 <= n <= 32768}
    if any(n > n_blocks for n in grid):
        return sorted(grid - {n_blocks})
    return sorted(grid | {n_blocks})


def default_k_grid(top_k: int, n_blocks: int, extra=()) -> list:
    return [k for k in sorted({0, top_k // 4, top_k // 2, top_k, (3 * top_k) // 2, 2 * top_k} | set(extra))
            if k <= n_blocks]


def two_stream_tables(shape: L.Shape, top_k: int, q: torch.Tensor, k_cache, v_cache, table, n_grid=None,
                      k_grid=None, reps: int = 50, seed: int = 0) -> dict:
    """t_sel(N) on random summaries of the layer's batch and heads for each N of the grid, and t_spec(K') of the
    speculation launch over random predicted sets of the layer itself."""
    dev = q.device
    B, Hq, Hkv, D, N0 = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_blocks
    n_grid = default_n_grid(N0) if n_grid is None else list(n_grid)
    k_grid = default_k_grid(top_k, N0) if k_grid is None else list(k_grid)
    gen = torch.Generator(device=dev).manual_seed(seed)
    t_sel = []
    for n in n_grid:
        s = L.make_shape(B, Hq, Hkv, D, shape.block_size, shape.page_size, n, shape.dtype, shape.softmax_scale)
        summ = torch.randn((B, Hkv, n, 2, D), generator=gen, device=dev).to(shape.torch_dtype)
        qn = torch.randn((B, Hq, D), generator=gen, device=dev).to(shape.torch_dtype)
        sc = torch.zeros((B, Hkv, n), dtype=torch.float32, device=dev)
        kk = min(top_k, n)
        sel = torch.zeros((B, Hkv, kk), dtype=torch.int32, device=dev)
        ws = torch.zeros((L.workspace_bytes(s, kk) // 4 + 1,), dtype=torch.float32, device=dev)
        t_sel.append(graph_us(lambda st, s=s, qn=qn, summ=summ, sc=sc, sel=sel, ws=ws, kk=kk: L.score_select(
            s, qn, summ, kk, sc, sel, workspace=ws, stream=st), reps, dev))
        del summ, sc, sel, ws
    rng = np.random.default_rng(seed)
    rows = B * Hkv
    t_spec = []
    for k in k_grid:
        if k == 0:
            t_spec.append(0.0)
            continue
        pred = torch.as_tensor(np.stack([np.sort(rng.choice(N0, k, replace=False)) for _ in range(rows)])
                               .reshape(B, Hkv, k).astype(np.int32), device=dev)
        part = torch.zeros((L.partials_bytes(shape, k) // 4,), dtype=torch.float32, device=dev)
        t_spec.append(graph_us(lambda st, pred=pred, part=part, k=k: L.speculate(
            shape, q, k_cache, v_cache, table, pred, k, part, stream=st), reps, dev))
    k_star = L.choose_budget(n_grid, t_sel, k_grid, t_spec, float(N0), 2)
    fit = float(np.polyval(np.polyfit(n_grid, t_sel, min(2, len(n_grid) - 1)), N0)) if n_grid else None
    return {"n_grid": n_grid, "t_sel_us": t_sel, "t_sel_fit_us": fit, "kspec_grid": k_grid, "t_spec_us": t_spec,
            "kspec_star": k_star}


def fused_step_table(shape: L.Shape, top_k: int, alpha: float, kvs, table, queries, k_grid, steps: int = 20,
                     warmup: int = 5) -> dict:
    """t_step(K') of whole fused decode steps (PRR_MODE_FUSED; K' = 0 is the step without speculation) over the
    layers in ``kvs`` (a list of (k_cache, v_cache) rotated through, as a model's layers are), queries cycled."""
    dev = queries[0].device
    streams = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))
    t_step = []
    for k in k_grid:
        layers = []
        for kc, vc in kvs:
            lay = PRRLayer(shape, top_k, k, alpha, mode="prr_fused", device=dev, streams=streams)
            lay.build(kc, vc, table)
            layers.append(lay)
        for _ in range(warmup):
            for lay in layers:
                lay.enqueue(queries[lay.t % len(queries)])
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=streams[0]):
            for _ in range(steps):
                for lay in layers:
                    lay.enqueue(queries[lay.t % len(queries)])
        g.replay()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream(dev)
        e0.record(cur)
        g.replay()
        e1.record(cur)
        torch.cuda.synchronize(dev)
        t_step.append(e0.elapsed_time(e1) * 1e3 / (steps * len(layers)))
        for lay in layers:
            lay.close()
        del g, layers
    return {"kspec_grid": list(k_grid), "t_step_us": t_step,
            "kspec_star": L.choose_budget_fused(list(k_grid), t_step)}
