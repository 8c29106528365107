"""Search of the query draws that keep the selection's score gap above 1e-4 (test infrastructure: uses the oracle).

The selection must equal the oracle's exactly wherever the relative gap (s_(K) - s_(K+1)) / |s_(K)| of the oracle's
block scores exceeds 1e-4; the inputs are drawn so that it does. For every (sequence b, KV head g) and every step t
in order, the group's query draw of that step (q_0 at t = 0, the AR(1) innovation after) is tried with attempt
0, 1, ... until the oracle's plain Quest scores (or mean-key scores) of the stored bytes give a gap above 1e-4; the
first such attempt is kept and the next step builds on the accepted query. A row that reaches ``cap`` attempts keeps
its widest-gap attempt and counts as banded.

The bytes are exactly those the device reads: keys and queries are cast to the storage dtype (round to nearest
even) by the input generator's own functions, the hot-block bias follows the accepted q_0, and the hot-block drift
is replayed. Rows are independent, so they are searched in parallel threads.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from dynamic_sparse_attention_decode_amd import inputs as I
from oracle import prr_oracle as O

REL_GAP = 1e-4


def _as_stored(x: np.ndarray, dtype: str) -> np.ndarray:
    """The values the device reads for fp32 data x: cast to the storage dtype, widened (exactly) to fp32."""
    return I.to_storage(np.asarray(x, dtype=np.float32), dtype).float().numpy()


def _stored_query(qg: np.ndarray, dtype: str) -> np.ndarray:
    """A query group as stored (fp64 -> fp32 -> storage dtype), widened to fp64."""
    t = torch.as_tensor(np.asarray(qg), dtype=torch.float32)
    return (t if dtype == "f32" else t.to({"bf16": torch.bfloat16, "f16": torch.float16}[dtype])).double().numpy()


class _Row:
    """The stored keys' block statistics of one (b, g) row, kept up to date with the planted and drifting bias."""

    def __init__(self, w: I.Workload, b: int, g: int):
        self.w = w
        bs, D = w.block_size, w.head_dim
        self.keys32 = I.key_row(w, b, g)                        # unbiased fp32 draw, [capacity, D]
        self.base = _as_stored(self.keys32, w.dtype)            # unbiased stored keys (device bytes), [capacity, D]
        self.hot = I.hot_sets(w)[b, g].copy()
        self.n_tok = [min(bs, w.ctx - n * bs) for n in range(w.n_blocks)]
        if w.scorer == "mean":
            self.cur = self.base[:w.ctx].copy()                 # current stored keys, logical order
        else:
            # min and max are exact in the stored values' own (fp32) form; widened once for the fp64 scores
            kmin, kmax = O.block_summaries(self.base[:w.ctx], bs)
            self.kmin, self.kmax = kmin.astype(np.float64), kmax.astype(np.float64)
        self.bias = np.zeros(D, dtype=np.float32)

    def _block(self, n: int, keys_stored: np.ndarray) -> None:
        """Record block n's stored keys (its first n_tok[n] rows count)."""
        bs = self.w.block_size
        kb = keys_stored[: self.n_tok[n]]
        if self.w.scorer == "mean":
            self.cur[n * bs: n * bs + self.n_tok[n]] = kb
        else:
            mn, mx = O.block_summaries(kb, self.n_tok[n])
            self.kmin[n], self.kmax[n] = mn[0], mx[0]

    def plant(self, q0_group: np.ndarray) -> None:
        """The initial bias from the group's first query on every hot block (fp32 add, then the cast)."""
        w, bs = self.w, self.w.block_size
        if not w.hot_blocks:
            return
        self.bias = w.hot_bias * I.qhat_group(q0_group)
        for n in self.hot:
            n = int(n)
            self._block(n, _as_stored(self.keys32[n * bs:(n + 1) * bs] + self.bias, w.dtype))

    def drift(self, t: int, b: int, g: int) -> None:
        """The drift before step t: the old block gets back its unbiased stored keys, the new block becomes
        cast(stored keys + bias)."""
        w, bs = self.w, self.w.block_size
        i_old, n_new = I.drift_choice(w, t, b, g, self.hot)
        n_old = int(self.hot[i_old])
        self._block(n_old, self.base[n_old * bs:(n_old + 1) * bs])
        self._block(n_new, _as_stored(self.base[n_new * bs:(n_new + 1) * bs] + self.bias, w.dtype))
        self.hot[i_old] = n_new

    def scores(self, q_stored: np.ndarray, fast: bool) -> np.ndarray:
        w = self.w
        if w.scorer == "mean":
            return O.mean_key_scores(q_stored, self.cur, w.block_size)
        if fast:
            return O.quest_scores_signsplit(q_stored, self.kmin, self.kmax)
        return O.quest_scores(q_stored, self.kmin, self.kmax)


def selection_gap(w: I.Workload, s: np.ndarray) -> float:
    """The relative gap that decides exactness: at the K-th boundary of the unforced blocks when blocks are forced."""
    n = len(s)
    forced = np.array([i < w.sink_blocks or i >= n - w.local_blocks for i in range(n)]) \
        if (w.sink_blocks or w.local_blocks) else np.zeros(n, dtype=bool)
    k = w.top_k - int(forced.sum())
    if k <= 0:
        return math.inf
    return O.boundary_gap(s[~forced], k)[2]


def search_row(w: I.Workload, b: int, g: int, steps: int, cap: int = 1024):
    """(attempts [steps], gaps [steps]) of row (b, g)."""
    row = _Row(w, b, g)
    attempts = np.zeros(steps, dtype=np.int64)
    gaps = np.zeros(steps, dtype=np.float64)
    prev = None
    for t in range(steps):
        if t > 0 and I.drifts_at(w, t):
            row.drift(t, b, g)
        best = (-math.inf, 0, None)
        last = -1
        for a in range(cap):
            last = a
            qg = I.query_group(w, t, b, g, prev, a)
            if t == 0:
                row.plant(qg)
            qs = _stored_query(qg, w.dtype)
            if w.scorer == "quest" and selection_gap(w, row.scores(qs, True)) <= 0.5 * REL_GAP:
                gap = -1.0          # far inside the band by the fast exact form: no need for the plain one
            else:
                gap = selection_gap(w, row.scores(qs, False))
            if gap > best[0]:
                best = (gap, a, qg)
            if gap > REL_GAP:
                break
        gap, a, qg = best
        if t == 0 and a != last:
            row.plant(qg)        # the kept draw's bias (the loop left the last attempt's)
        attempts[t], gaps[t], prev = a, gap, qg
    return attempts, gaps


def search(w: I.Workload, steps: int | None = None, cap: int = 1024, threads: int | None = None):
    """attempts int64 [steps, B, Hkv] and the accepted gaps fp64 [steps, B, Hkv] of workload w."""
    steps = w.steps if steps is None else steps
    rows = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    attempts = np.zeros((steps, w.batch, w.n_kv_heads), dtype=np.int64)
    gaps = np.zeros((steps, w.batch, w.n_kv_heads), dtype=np.float64)
    from threadpoolctl import threadpool_limits
    prev_torch = torch.get_num_threads()
    torch.set_num_threads(1)   # one thread per row: no nested BLAS or torch thread pools
    try:
        with threadpool_limits(limits=1), ThreadPoolExecutor(threads or I.default_threads()) as ex:
            for (b, g), (a, gp) in zip(rows, ex.map(lambda bg: search_row(w, bg[0], bg[1], steps, cap), rows)):
                attempts[:, b, g] = a
                gaps[:, b, g] = gp
    finally:
        torch.set_num_threads(prev_torch)
    return attempts, gaps
