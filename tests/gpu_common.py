"""Shared helpers of the GPU parity tests: reduced workloads, oracle views of the generated inputs."""
from __future__ import annotations

import functools
import os

import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd import _lib as L
from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS, Workload, load_attempts, make_inputs

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def small(name: str) -> Workload:
    """Reduced versions of the five workloads: the oracle finishes them in seconds, yet they span several tiles of
    every kernel and end on ragged tails (block counts, K and K' that are not multiples of the tile sizes)."""
    w = WORKLOADS[name]
    if name == "tiny_f32_4k":
        return w
    if name == "llama3_8b_32k":
        return w.replace(ctx=w.block_size * 250, top_k=30, k_spec=(37,), steps=10, hot_blocks=12)
    if name == "long_ctx_131k_b4":
        return w.replace(batch=2, ctx=w.block_size * 130, top_k=14, k_spec=(19,), steps=10, hot_blocks=10)
    if name == "paged_b32_64k":
        return w.replace(batch=3, ctx=w.block_size * 300, top_k=33, k_spec=(33,), steps=8)
    if name == "million_token":
        return w.replace(ctx=w.block_size * 2100, top_k=61, k_spec=(0, 29, 61, 93), steps=8, hot_blocks=40)
    raise KeyError(name)


SMALL = ["tiny_f32_4k", "llama3_8b_32k", "long_ctx_131k_b4", "paged_b32_64k", "million_token"]


def wide_paged(**kw) -> Workload:
    """136 rows (17 sequences x 8 KV heads) of the reduced paged workload, with a partly filled last block: enough
    rows for the fused step's many-row path (speculation in its own launch, a selection launch of top-K workgroups
    only, then the spread-out repair)."""
    args = dict(batch=17, ctx=16 * 70 - 3, top_k=12, k_spec=(12,), steps=5)
    args.update(kw)
    return small("paged_b32_64k").replace(**args)


def shape_of(w: Workload) -> L.Shape:
    return L.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.page_size, w.n_blocks,
                        {"f32": L.F32, "bf16": L.BF16, "f16": L.F16}[w.dtype], w.scale,
                        ctx_len=w.ctx if w.ctx % w.block_size else 0, sink_blocks=w.sink_blocks,
                        local_blocks=w.local_blocks, scorer=L.SCORER_MEAN if w.scorer == "mean" else L.SCORER_QUEST)


def oracle_scores(w: Workload, q_group, keys):
    """The oracle's block scores of one (sequence, KV head) under the workload's scorer."""
    from oracle import prr_oracle as O
    if w.scorer == "mean":
        return O.mean_key_scores(q_group, keys, w.block_size)
    kmin, kmax = O.block_summaries(keys, w.block_size)
    return O.quest_scores(q_group, kmin, kmax)


def ragged(w: Workload, short: int) -> Workload:
    """The workload with its sequences ending `short` tokens before the end of the last block."""
    return w.replace(name=w.name + f"_short{short}", ctx=w.ctx - short)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class OracleView:
    """fp64 host copies of one (b, g) row's logical keys/values, gathered through the page table by the oracle."""

    def __init__(self, inp):
        self.inp = inp
        self.w = inp.w
        self.table = inp.table_np
        self._k = {}
        self._v = {}

    def _cache_row(self, cache: torch.Tensor, b: int, g: int) -> np.ndarray:
        from oracle import prr_oracle as O
        pages = torch.as_tensor(self.table[b], device=cache.device, dtype=torch.long)
        sub = cache[pages, g].float().cpu().numpy()            # [pps, page, D] (plain page copy)
        local_table = np.arange(len(self.table[b]), dtype=np.int64)[None, :]
        return O.logical_tokens(sub[:, None], local_table, 0, 0, self.w.ctx)

    def keys(self, b: int, g: int) -> np.ndarray:
        if (b, g) not in self._k:
            self._k[(b, g)] = self._cache_row(self.inp.k_cache, b, g)
        return self._k[(b, g)]

    def values(self, b: int, g: int) -> np.ndarray:
        if (b, g) not in self._v:
            self._v[(b, g)] = self._cache_row(self.inp.v_cache, b, g)
        return self._v[(b, g)]

    def invalidate_keys(self):
        self._k.clear()

    def q_group(self, t: int, b: int, g: int) -> np.ndarray:
        G = self.w.group
        return np64(self.inp.q[t, b, g * G:(g + 1) * G])


GAP_TABLES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gap_attempts")


@functools.lru_cache(maxsize=64)
def _searched_attempts(w: Workload, steps: int) -> np.ndarray:
    from tests.gap_search import search
    return search(w, steps)[0]


def gap_attempts(w: Workload, steps: int | None = None) -> np.ndarray:
    """Query-draw attempts that keep the selection's relative score gap above 1e-4 on every (step, row): the stored
    table of a full-size workload, else a search with the oracle (reduced workloads take seconds)."""
    steps = w.steps if steps is None else steps
    full = WORKLOADS.get(w.name)
    if full is not None and full.key() == w.key():
        return load_attempts(os.path.join(GAP_TABLES, f"{w.name}.json"), w, steps)
    return _searched_attempts(w, steps)


def gap_inputs(w: Workload, device="cuda", steps: int | None = None) -> "object":
    """make_inputs with the gap-keeping query draws (so the selection is checked for exact equality everywhere)."""
    steps = w.steps if steps is None else steps
    return make_inputs(w, device=device, steps=steps, attempts=gap_attempts(w, steps))
