"""Seeded synthetic inputs for one attention layer's sparse decode.

This module is shared by the HIP path and by the fp64 oracle's tests, so it holds none of the method's arithmetic:
only random keys, values and queries, the planted "hot" block bias, the query AR(1) process, the paged layout and
page-table permutation, and the hot-block drift schedule.

The workloads are the five shapes the method is measured on here (named by what they are, with their sizes). The
pages evaluate on long-context benchmarks that are not available; these synthetic streams stand in for them:
temporal locality (the property the method exploits, "Predict, Reuse, and Repair", arxivlens summary) comes from the
slowly varying AR(1) queries and the hot blocks whose keys lean towards the first query of their KV group.

Recipe (per workload, master seed ``seed``):

* K, V ~ N(0, 1) per element, drawn in fp32 on the host and cast to the storage dtype with round-to-nearest-even.
  Every (sequence b, KV head g) row is drawn in chunks of ``CHUNK_TOKENS`` tokens, each from its own counter-based
  Philox stream keyed by (seed, purpose, b, g, chunk): the bytes do not depend on the device, the thread count or the
  order of generation, so a CPU process can rebuild exactly the keys a GPU run reads.
* Queries per (b, g) group of G query heads: q_0 ~ N(0, I) and q_t = rho * q_{t-1} + sqrt(1 - rho^2) * eps_t, run in
  fp64 and cast per step. q_0 and eps_t are drawn from streams keyed by (seed, purpose, [t,] b, g, attempt), where
  ``attempt`` comes from a per-(t, b, g) table (0 when none is given). A redraw changes only that group's step.
* For each (b, g): ``hot_blocks`` distinct block ids; every key of a hot block gets ``+hot_bias * qhat[b, g]``
  (fp32, before the cast), qhat = unit vector of the sum of the group's q_0.
* Drift (``drift_every`` > 0): before the selection of step t (t > 0, t % drift_every == 0), for each (b, g) the bias
  moves from one uniformly chosen hot block to one uniformly chosen non-hot block: the old block gets back its
  unbiased stored keys, the new block becomes cast(stored keys widened to fp32 + bias).
* Paged KV: ``page_size`` tokens per page; the page table is the identity, or a seeded permutation of all pages of
  the batch when ``shuffle_pages`` is set.
* A context that ends inside a block (``ctx`` not a multiple of ``block_size``): the cache holds whole blocks, and
  the slots past the end hold poison (keys +50, values 1e4), which no result may depend on.

The attempt table is how the inputs keep a relative score gap above 1e-4 at the K-th/(K+1)-th selection boundary:
a script beside the tests searches, step by step, the first attempt of each group's draw whose boundary gap (by the
oracle's plain block scores on these exact bytes) exceeds 1e-4, and stores the attempts; this module only draws by
them.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

# purpose codes for the seed sequence
_P_K, _P_V, _P_Q0, _P_EPS, _P_HOT, _P_PAGES, _P_DRIFT = range(7)
CHUNK_TOKENS = 8192            # tokens per independently keyed K/V draw


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx: int
    block_size: int
    page_size: int
    top_k: int
    k_spec: tuple
    alpha: float
    rho: float
    steps: int
    hot_blocks: int
    drift_every: int = 0
    shuffle_pages: bool = False
    dtype: str = "bf16"          # storage dtype of q, K, V and the block summaries: "f32" | "bf16" | "f16"
    hot_bias: float = 2.0
    seed: int = 20261203
    sink_blocks: int = 0         # forced blocks of every selection: the first sink_blocks and the last local_blocks
    local_blocks: int = 0
    scorer: str = "quest"        # block scorer: "quest" (key min/max bound) or "mean" (mean key)

    # ---- derived sizes -------------------------------------------------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_blocks(self) -> int:
        return -(-self.ctx // self.block_size)   # the last block may be partly filled

    @property
    def capacity(self) -> int:
        """Token slots per sequence in the paged cache (whole blocks)."""
        return self.n_blocks * self.block_size

    @property
    def pages_per_seq(self) -> int:
        return self.capacity // self.page_size

    @property
    def n_pages(self) -> int:
        return self.batch * self.pages_per_seq

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self):
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def validate(self) -> None:
        assert self.n_q_heads % self.n_kv_heads == 0
        assert self.ctx >= 1 and self.block_size % self.page_size == 0
        assert 1 <= self.top_k <= self.n_blocks
        assert all(0 <= k <= self.n_blocks for k in self.k_spec)
        assert 0 <= self.hot_blocks <= self.n_blocks
        if self.drift_every:
            assert 0 < self.hot_blocks < self.n_blocks

    def key(self) -> dict:
        """Every field that decides the generated bytes (for checking a stored attempt table against a workload)."""
        d = dataclasses.asdict(self)
        d.pop("steps")
        d["k_spec"] = list(d["k_spec"])
        return d


# The five workloads. Shapes, budgets, EMA weights and query processes as specified for this path; where a value was
# left open (page size of the unpaged workloads, hot-block count of the batched paged workload) the plain reading is
# used: one page per selection block, and no planted blocks.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_4k", 1, 4, 1, 64, 4096, 32, 32, 16, (16,), 0.9, 0.95, 8, 8, dtype="f32",
                 seed=20261203 + 1),
        Workload("llama3_8b_32k", 1, 32, 8, 128, 32768, 16, 16, 128, (160,), 0.9, 0.95, 64, 32,
                 seed=20261203 + 2),
        Workload("long_ctx_131k_b4", 4, 32, 8, 128, 131072, 64, 64, 64, (80,), 0.8, 0.9, 64, 48, drift_every=4,
                 seed=20261203 + 3),
        Workload("paged_b32_64k", 32, 32, 8, 128, 65536, 16, 16, 128, (128,), 0.7, 0.5, 32, 0,
                 shuffle_pages=True, seed=20261203 + 4),
        Workload("million_token", 1, 64, 8, 128, 1048576, 32, 32, 256, (0, 128, 256, 384), 0.9, 0.95, 32, 128,
                 seed=20261203 + 5),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


def _subseed(seed: int, purpose: int, *idx: int) -> int:
    ss = np.random.SeedSequence([seed & 0xFFFFFFFF, purpose, *[int(i) for i in idx]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)


def _np_rng(seed: int, purpose: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(_subseed(seed, purpose, *idx)))


def default_threads() -> int:
    """Host threads for the bulk K/V draws: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # not on Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---- keys and values -----------------------------------------------------------------------------------------------


def _normal_row(w: Workload, purpose: int, b: int, g: int) -> np.ndarray:
    """fp32 [capacity, D] of N(0, 1), chunk by chunk from independently keyed streams."""
    out = np.empty((w.capacity, w.head_dim), dtype=np.float32)
    for c0 in range(0, w.capacity, CHUNK_TOKENS):
        c1 = min(w.capacity, c0 + CHUNK_TOKENS)
        _np_rng(w.seed, purpose, b, g, c0 // CHUNK_TOKENS).standard_normal(out=out[c0:c1], dtype=np.float32)
    return out


def key_row(w: Workload, b: int, g: int) -> np.ndarray:
    """Unbiased keys of sequence b, KV head g in logical token order: fp32 [capacity, D]; slots past ctx hold +50."""
    k = _normal_row(w, _P_K, b, g)
    k[w.ctx:] = 50.0
    return k


def value_row(w: Workload, b: int, g: int) -> np.ndarray:
    """Values of sequence b, KV head g in logical token order: fp32 [capacity, D]; slots past ctx hold 1e4."""
    v = _normal_row(w, _P_V, b, g)
    v[w.ctx:] = 1e4
    return v


def to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 host array -> CPU tensor of the storage dtype, rounded to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if dtype == "f32" else t.to({"bf16": torch.bfloat16, "f16": torch.float16}[dtype])


def plant_hot(keys_f32: np.ndarray, hot_ids, bias: np.ndarray, block_size: int) -> None:
    """Adds the fp32 bias to every key of the hot blocks, in place."""
    kb = keys_f32[: (len(keys_f32) // block_size) * block_size].reshape(-1, block_size, keys_f32.shape[1])
    kb[np.asarray(hot_ids, dtype=np.int64)] += bias.astype(np.float32)


# ---- queries -------------------------------------------------------------------------------------------------------


def query_group(w: Workload, t: int, b: int, g: int, prev, attempt: int = 0) -> np.ndarray:
    """fp64 [G, D] queries of group (b, g) at step t: the first draw at t = 0, else the AR(1) step from ``prev``.
    ``attempt`` selects the draw's stream (redraws of one group's step)."""
    shp = (w.group, w.head_dim)
    if t == 0:
        return _np_rng(w.seed, _P_Q0, b, g, attempt).standard_normal(shp)
    c = math.sqrt(max(0.0, 1.0 - w.rho * w.rho))
    eps = _np_rng(w.seed, _P_EPS, t, b, g, attempt).standard_normal(shp)
    return w.rho * np.asarray(prev, dtype=np.float64) + c * eps


def query_stream(w: Workload, steps: int | None = None, attempts=None) -> np.ndarray:
    """fp64 queries [steps, B, Hq, D] of the AR(1) process (before the storage cast); attempts [>= steps, B, Hkv] or
    None (all 0)."""
    steps = w.steps if steps is None else steps
    G = w.group
    q = np.empty((steps, w.batch, w.n_q_heads, w.head_dim), dtype=np.float64)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            prev = None
            for t in range(steps):
                a = 0 if attempts is None else int(attempts[t, b, g])
                prev = query_group(w, t, b, g, prev, a)
                q[t, b, g * G:(g + 1) * G] = prev
    return q


def qhat_group(q0_group: np.ndarray) -> np.ndarray:
    """fp32 [D] unit vector of the group-summed first query (direction of the hot-block bias)."""
    s = np.asarray(q0_group, dtype=np.float64).sum(axis=0)
    n = np.linalg.norm(s)
    return (s / (n if n > 0 else 1.0)).astype(np.float32)


def qhat(w: Workload, q0: np.ndarray) -> np.ndarray:
    """fp32 [B, Hkv, D]: qhat_group of every group of q0 [B, Hq, D]."""
    G = w.group
    return np.stack([np.stack([qhat_group(q0[b, g * G:(g + 1) * G]) for g in range(w.n_kv_heads)])
                     for b in range(w.batch)])


# ---- layout, hot sets, drift ----------------------------------------------------------------------------------------


def block_table(w: Workload) -> np.ndarray:
    """int32 [B, pages_per_seq] logical page -> physical page id."""
    if w.shuffle_pages:
        perm = _np_rng(w.seed, _P_PAGES).permutation(w.n_pages)
    else:
        perm = np.arange(w.n_pages)
    return perm.reshape(w.batch, w.pages_per_seq).astype(np.int32)


def hot_sets(w: Workload) -> np.ndarray:
    """int64 [B, Hkv, H] initial hot block ids (distinct per row)."""
    out = np.zeros((w.batch, w.n_kv_heads, w.hot_blocks), dtype=np.int64)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            if w.hot_blocks:
                out[b, g] = _np_rng(w.seed, _P_HOT, b, g).choice(w.n_blocks, w.hot_blocks, replace=False)
    return out


def drifts_at(w: Workload, t: int) -> bool:
    return bool(w.drift_every) and t > 0 and t % w.drift_every == 0


def drift_choice(w: Workload, t: int, b: int, g: int, hot_row: np.ndarray):
    """(position in the hot list, new block id) of row (b, g)'s drift before step t."""
    rng = _np_rng(w.seed, _P_DRIFT, t, b, g)
    i_old = int(rng.integers(w.hot_blocks))
    mask = np.ones(w.n_blocks, dtype=bool)
    mask[hot_row] = False
    cold = np.flatnonzero(mask)
    return i_old, int(cold[rng.integers(len(cold))])


# ---- stored attempt tables -------------------------------------------------------------------------------------------


def load_attempts(path: str, w: Workload, steps: int | None = None) -> np.ndarray:
    """int64 [steps, B, Hkv] attempts from a stored table, checked against the workload's generating fields."""
    steps = w.steps if steps is None else steps
    with open(path) as f:
        d = json.load(f)
    if d["workload"] != w.key():
        raise ValueError(f"{path}: the table was made for other workload fields")
    a = np.asarray(d["attempts"], dtype=np.int64).reshape(d["shape"])
    if a.shape[0] < steps:
        raise ValueError(f"{path}: table covers {a.shape[0]} steps, {steps} asked for")
    return a[:steps]


@dataclass
class DecodeInputs:
    """Device-resident inputs of one layer's decode run."""

    w: Workload
    device: torch.device
    k_cache: torch.Tensor          # [n_pages, Hkv, page, D] storage dtype
    v_cache: torch.Tensor          # [n_pages, Hkv, page, D]
    table: torch.Tensor            # int32 [B, pages_per_seq] on device
    table_np: np.ndarray           # same, host copy
    q: torch.Tensor                # [steps, B, Hq, D] storage dtype (device)
    hot: np.ndarray                # [B, Hkv, H] current hot block ids
    qhat: np.ndarray               # [B, Hkv, D] fp32
    saved: dict = field(default_factory=dict)   # (b, g, n) -> unbiased keys [bs, D] of a biased block
    attempts: np.ndarray | None = None          # [steps, B, Hkv] draws used for the queries (None: all 0)

    # ---- paged-layout helpers (input plumbing) ------------------------------------------------------------------
    def _pages_of_block(self, b: int, n: int) -> np.ndarray:
        w = self.w
        ppb = w.block_size // w.page_size
        return self.table_np[b, n * ppb:(n + 1) * ppb]

    def block_keys(self, b: int, g: int, n: int) -> torch.Tensor:
        pages = torch.as_tensor(self._pages_of_block(b, n), device=self.device, dtype=torch.long)
        return self.k_cache[pages, g].reshape(self.w.block_size, self.w.head_dim)

    def set_block_keys(self, b: int, g: int, n: int, keys: torch.Tensor) -> None:
        pages = torch.as_tensor(self._pages_of_block(b, n), device=self.device, dtype=torch.long)
        self.k_cache[pages, g] = keys.reshape(len(pages), self.w.page_size, self.w.head_dim).to(self.k_cache.dtype)

    def _bias(self, b: int, g: int) -> torch.Tensor:
        return torch.as_tensor(self.w.hot_bias * self.qhat[b, g], device=self.device, dtype=torch.float32)

    # ---- drift ---------------------------------------------------------------------------------------------------
    def drift(self, t: int) -> np.ndarray:
        """Apply the hot-block drift scheduled before step t's selection.

        Returns int32 flat block ids ``(b * Hkv + g) * N + n`` of every block whose keys changed (empty if none)."""
        w = self.w
        if not drifts_at(w, t):
            return np.zeros((0,), dtype=np.int32)
        changed = []
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                hot = self.hot[b, g]
                i_old, n_new = drift_choice(w, t, b, g, hot)
                n_old = int(hot[i_old])
                # remove the bias from the old block: restore its unbiased keys
                self.set_block_keys(b, g, n_old, self.saved.pop((b, g, n_old)))
                # plant it on the new block
                cur = self.block_keys(b, g, n_new).clone()
                self.saved[(b, g, n_new)] = cur
                self.set_block_keys(b, g, n_new, cur.float() + self._bias(b, g))
                hot[i_old] = n_new
                base = (b * w.n_kv_heads + g) * w.n_blocks
                changed += [base + n_old, base + n_new]
        return np.asarray(sorted(changed), dtype=np.int32)


def make_inputs(w: Workload, device="cpu", steps: int | None = None, attempts=None,
                threads: int | None = None) -> DecodeInputs:
    """Generate one layer's paged K/V cache, page table and query stream on ``device``.

    attempts: int [>= steps, B, Hkv] per-group draw attempts of the queries (None: the first draw everywhere)."""
    w.validate()
    device = torch.device(device)
    steps = w.steps if steps is None else steps
    if attempts is not None:
        attempts = np.asarray(attempts, dtype=np.int64)[:steps]
        assert attempts.shape == (steps, w.batch, w.n_kv_heads), attempts.shape
    dt = w.torch_dtype
    B, Hkv, D, page = w.batch, w.n_kv_heads, w.head_dim, w.page_size
    pps = w.pages_per_seq
    table_np = block_table(w)
    q64 = query_stream(w, steps, attempts)
    qh = qhat(w, q64[0])
    hot = hot_sets(w)

    def row(bg):
        b, g = bg
        k = key_row(w, b, g)
        base = None
        if w.hot_blocks:
            if w.drift_every:   # the unbiased stored keys of the hot blocks, for moving the bias later
                kb = k[:w.capacity].reshape(w.n_blocks, w.block_size, D)
                base = to_storage(kb[hot[b, g]], w.dtype)
            plant_hot(k, hot[b, g], w.hot_bias * qh[b, g], w.block_size)
        return b, g, to_storage(k, w.dtype), to_storage(value_row(w, b, g), w.dtype), base

    k_cache = torch.empty((w.n_pages, Hkv, page, D), dtype=dt, device=device)
    v_cache = torch.empty_like(k_cache)
    saved = {}
    rows = [(b, g) for b in range(B) for g in range(Hkv)]
    nthr = threads or default_threads()
    prev_torch = torch.get_num_threads()
    torch.set_num_threads(1)   # the rows run in parallel threads: no nested torch thread pools for the casts
    try:
        with ThreadPoolExecutor(nthr) as ex:
            for i0 in range(0, len(rows), 2 * nthr):   # bounded host memory: a few rows in flight
                for b, g, kc, vc, base in ex.map(row, rows[i0:i0 + 2 * nthr]):
                    phys = torch.as_tensor(table_np[b], device=device, dtype=torch.long)
                    k_cache[phys, g] = kc.view(pps, page, D).to(device)
                    v_cache[phys, g] = vc.view(pps, page, D).to(device)
                    if base is not None:
                        for j, n in enumerate(hot[b, g]):
                            saved[(b, g, int(n))] = base[j].to(device)
    finally:
        torch.set_num_threads(prev_torch)
    q = torch.as_tensor(q64, dtype=torch.float32).to(dt).to(device)
    table = torch.as_tensor(table_np, device=device)
    return DecodeInputs(w, device, k_cache, v_cache, table, table_np, q, hot, qh, saved, attempts)
