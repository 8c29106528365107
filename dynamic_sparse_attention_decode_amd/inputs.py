"""Seeded synthetic inputs for one attention layer's sparse decode.

This module is shared by the HIP path and by the fp64 oracle's tests, so it holds none of the method's arithmetic:
only random keys, values and queries, the planted "hot" block bias, the query AR(1) process, the paged layout and
page-table permutation, and the hot-block drift schedule.

The workloads are the five shapes the method is measured on here (named by what they are, with their sizes). The
pages evaluate on long-context benchmarks that are not available; these synthetic streams stand in for them:
temporal locality (the property the method exploits, "Predict, Reuse, and Repair", arxivlens summary) comes from the
slowly varying AR(1) queries and the hot blocks whose keys lean towards the first query of their KV group.

Recipe (per workload, master seed ``seed``):

* K, V ~ N(0, 1) per element, drawn in fp32 and cast to the storage dtype with round-to-nearest-even.
* q_0[b, h] ~ N(0, I_D); q_t = rho * q_{t-1} + sqrt(1 - rho^2) * eps_t, run in fp64 and cast per step.
* For each (sequence b, KV head g): ``hot_blocks`` distinct block ids; every key of a hot block gets
  ``+hot_bias * qhat[b, g]`` (fp32, before the cast), qhat = unit vector of the sum of the group's q_0.
* Drift (``drift_every`` > 0): before the selection of step t (t > 0, t % drift_every == 0), for each (b, g) the bias
  moves from one uniformly chosen hot block to one uniformly chosen non-hot block.
* Paged KV: ``page_size`` tokens per page; the page table is the identity, or a seeded permutation of all pages of
  the batch when ``shuffle_pages`` is set.
* A context that ends inside a block (``ctx`` not a multiple of ``block_size``): the cache holds whole blocks, and
  the slots past the end hold poison (keys +50, values 1e4), which no result may depend on.

Every random draw is keyed by (seed, purpose, indices) through numpy's SeedSequence, so any part can be regenerated
independently. Bulk K/V draws use torch's generator on the target device; within one device the bytes are
reproducible for a given seed.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np
import torch

# purpose codes for the seed sequence
_P_K, _P_V, _P_Q0, _P_EPS, _P_HOT, _P_PAGES, _P_DRIFT = range(7)


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


def _torch_gen(device, seed: int, purpose: int, *idx: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_subseed(seed, purpose, *idx))
    return g


def query_stream(w: Workload, steps: int | None = None) -> np.ndarray:
    """fp64 queries [steps, B, Hq, D] of the AR(1) process (before the storage cast)."""
    steps = w.steps if steps is None else steps
    q = np.empty((steps, w.batch, w.n_q_heads, w.head_dim), dtype=np.float64)
    q[0] = _np_rng(w.seed, _P_Q0).standard_normal(q.shape[1:])
    c = math.sqrt(max(0.0, 1.0 - w.rho * w.rho))
    for t in range(1, steps):
        eps = _np_rng(w.seed, _P_EPS, t).standard_normal(q.shape[1:])
        q[t] = w.rho * q[t - 1] + c * eps
    return q


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


def qhat(w: Workload, q0: np.ndarray) -> np.ndarray:
    """fp32 [B, Hkv, D] unit vector of the group-summed first query (direction of the hot-block bias)."""
    G = w.group
    s = q0.reshape(w.batch, w.n_kv_heads, G, w.head_dim).sum(axis=2)
    n = np.linalg.norm(s, axis=-1, keepdims=True)
    n[n == 0] = 1.0
    return (s / n).astype(np.float32)


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
        if not w.drift_every or t == 0 or t % w.drift_every:
            return np.zeros((0,), dtype=np.int32)
        changed = []
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                rng = _np_rng(w.seed, _P_DRIFT, t, b, g)
                hot = self.hot[b, g]
                i_old = int(rng.integers(w.hot_blocks))
                mask = np.ones(w.n_blocks, dtype=bool)
                mask[hot] = False
                cold = np.flatnonzero(mask)
                n_new = int(cold[rng.integers(len(cold))])
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


def make_inputs(w: Workload, device="cpu", steps: int | None = None) -> DecodeInputs:
    """Generate one layer's paged K/V cache, page table and query stream on ``device``."""
    w.validate()
    device = torch.device(device)
    dt = w.torch_dtype
    B, Hkv, D, ctx, page = w.batch, w.n_kv_heads, w.head_dim, w.ctx, w.page_size
    pps = w.pages_per_seq
    table_np = block_table(w)
    q64 = query_stream(w, steps)
    qh = qhat(w, q64[0])
    hot = hot_sets(w)

    k_cache = torch.empty((w.n_pages, Hkv, page, D), dtype=dt, device=device)
    v_cache = torch.empty_like(k_cache)
    saved = {}
    cap = w.capacity
    for b in range(B):
        phys = torch.as_tensor(table_np[b], device=device, dtype=torch.long)
        for g in range(Hkv):
            k = torch.randn((cap, D), generator=_torch_gen(device, w.seed, _P_K, b, g), device=device,
                            dtype=torch.float32)
            v = torch.randn((cap, D), generator=_torch_gen(device, w.seed, _P_V, b, g), device=device,
                            dtype=torch.float32)
            k[ctx:] = 50.0   # slots past the end of the sequence
            v[ctx:] = 1e4
            if w.hot_blocks:
                kb = k.view(w.n_blocks, w.block_size, D)
                idx = torch.as_tensor(hot[b, g], device=device, dtype=torch.long)
                if w.drift_every:
                    base = kb[idx].to(dt)
                    for j, n in enumerate(hot[b, g]):
                        saved[(b, g, int(n))] = base[j].clone()
                kb[idx] += torch.as_tensor(w.hot_bias * qh[b, g], device=device)
            k_cache[phys, g] = k.to(dt).view(pps, page, D)
            v_cache[phys, g] = v.to(dt).view(pps, page, D)
            del k, v
    q = torch.as_tensor(q64, dtype=torch.float32).to(dt).to(device)
    table = torch.as_tensor(table_np, device=device)
    return DecodeInputs(w, device, k_cache, v_cache, table, table_np, q, hot, qh, saved)
