"""Per-layer PRR decode state and the step driver.

PRRLayer owns one attention layer's decode buffers (summaries, scores, EMA, predicted-set and partial double
buffers, repair workspace) as PyTorch device tensors, and two HIP streams (default priority). ``step(q)`` enqueues
one decode step through the library's ``prr_decode_step``; in the two-stream mode, with one fork and one join:

  stream_sel:  [fork] score_select(t) -> [join: wait speculation] -> repair_merge(t) -> ema_predict(t)
  stream_spec: [wait fork] speculate(P_t)

giving out_t and P_{t+1}. The other modes run on stream_sel alone (``prr_fused``: the same steps in fewer launches,
speculation inside the selection launch or in a launch of its own).

A per-row budget (prr_budget) may size each row's predicted set below k_spec; its rows then end in -1 slots.

PRR abstract: speculation over the predicted blocks runs while selection is in flight; the missed blocks are
repaired once the true set is known. Step 0 has no prediction (full repair). Buffers that the two streams share
across steps alternate by step parity, so step t+1's speculation never overwrites what step t's repair reads.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L

MODES = {"serialized": L.MODE_SERIALIZED, "prr_1stream": L.MODE_ONE_STREAM, "prr_2stream": L.MODE_TWO_STREAM,
         "prr_fused": L.MODE_FUSED, "serialized_fused": L.MODE_SERIALIZED_FUSED}


BUDGETS = {"fixed": L.BUDGET_FIXED, "misses": L.BUDGET_MISSES, "confidence": L.BUDGET_CONFIDENCE}


class PRRLayer:
    def __init__(self, shape: L.Shape, top_k: int, k_spec: int, alpha: float, mode: str = "prr_2stream",
                 device="cuda", streams=None, budget: dict | None = None, static_workspace: bool = False):
        """budget: None (every row predicts k_spec blocks) or {"policy": "misses" | "confidence", "k_min": int,
        "beta": float, "c": float}: per-row sizes of the predicted set, at most k_spec (prr_budget); the missed
        counts that the misses policy reads are double-buffered here. static_workspace: step through
        prr_decode_step_noalloc (the library's scratch; no workspace buffer here)."""
        if mode not in MODES:
            raise ValueError(f"mode must be one of {list(MODES)}")
        self.shape = L.Shape.from_buffer_copy(shape)   # own copy: append() advances its ctx_len
        shape = self.shape
        self.top_k = int(top_k)
        self.k_spec = int(k_spec) if mode not in ("serialized", "serialized_fused") else 0
        self.alpha = float(alpha)
        self.mode = mode
        self.device = torch.device(device)
        B, Hkv, N, D = shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim
        dt = shape.torch_dtype
        dev = self.device
        self.summaries = torch.empty((B, Hkv, N, 2, D), dtype=dt, device=dev)
        self.scores = [torch.zeros((B, Hkv, N), dtype=torch.float32, device=dev) for _ in range(2)]
        self.ema = torch.zeros((B, Hkv, N), dtype=torch.float32, device=dev)
        self.sel_idx = torch.zeros((B, Hkv, self.top_k), dtype=torch.int32, device=dev)
        kp = max(self.k_spec, 1)
        self.pred = [torch.zeros((B, Hkv, kp), dtype=torch.int32, device=dev) for _ in range(2)]
        pb = max(L.partials_bytes(shape, kp), 16)
        self.partials = [torch.zeros((pb // 4,), dtype=torch.float32, device=dev) for _ in range(2)]
        self.out = [torch.zeros((B, shape.n_q_heads, D), dtype=torch.float32, device=dev) for _ in range(2)]
        self.missed = [torch.zeros((B, Hkv), dtype=torch.int32, device=dev) for _ in range(2)]   # by step parity
        self.budgets = None
        if budget is not None and BUDGETS[budget.get("policy", "fixed")] != L.BUDGET_FIXED and self.k_spec > 0:
            pol = BUDGETS[budget["policy"]]
            # step t writes P_{t+1} under the budget whose missed counts are step t-1's (the other parity)
            self.budgets = [L.make_budget(pol, self.top_k, int(budget.get("k_min", 1)), float(budget.get("beta", 0.0)),
                                          float(budget.get("c", 0.0)), self.missed[1 - par]) for par in range(2)]
        self.static_workspace = bool(static_workspace)
        self.workspace = None if self.static_workspace else torch.zeros(
            (L.workspace_bytes(shape, self.top_k) // 4 + 1,), dtype=torch.float32, device=dev)
        if streams is None:
            streams = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))
        self.s_sel, self.s_spec = streams
        self.ctx = L.step_ctx_create()
        self.t = 0
        self.k_cache = self.v_cache = self.table = None

    def close(self):
        if self.ctx is not None:
            torch.cuda.synchronize(self.device)
            L.step_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- KV cache ------------------------------------------------------------------------------------------------
    def build(self, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor) -> None:
        """Attach the paged KV cache and build every block summary (on the selection stream)."""
        self.k_cache, self.v_cache, self.table = k_cache, v_cache, block_table
        cur = torch.cuda.current_stream(self.device)
        self.s_sel.wait_stream(cur)
        L.build_summaries(self.shape, k_cache, block_table, self.summaries, stream=self.s_sel)
        cur.wait_stream(self.s_sel)

    def rebuild_blocks(self, flat_ids: torch.Tensor) -> None:
        """Rebuild the summaries of the listed blocks ((b * Hkv + g) * N + n), e.g. after their keys changed."""
        if flat_ids.numel() == 0:
            return
        cur = torch.cuda.current_stream(self.device)
        self.s_sel.wait_stream(cur)
        L.build_summaries(self.shape, self.k_cache, self.table, self.summaries, block_ids=flat_ids,
                          stream=self.s_sel)
        cur.wait_stream(self.s_sel)

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        """Decode-time append of one token per sequence (k_new, v_new: [B, Hkv, D]) at the end of the layer's
        sequences, on the selection stream, ahead of the next step; the last block must have room for it."""
        s = self.shape
        n_tok = s.ctx_len or s.n_blocks * s.block_size
        if n_tok >= s.n_blocks * s.block_size:
            raise L.PRRError("append: the last block is full (the block count is fixed for this layer)")
        s.ctx_len = n_tok + 1
        cur = torch.cuda.current_stream(self.device)
        self.s_sel.wait_stream(cur)
        L.append_kv(s, k_new, v_new, self.k_cache, self.v_cache, self.table, self.summaries, stream=self.s_sel)
        cur.wait_stream(self.s_sel)

    def reset(self) -> None:
        """Forget the prediction state: the next step is a first step (no speculation, no missed counts)."""
        self.t = 0
        for m in self.missed:
            m.zero_()

    # ---- one decode step -----------------------------------------------------------------------------------------
    def _args(self, q: torch.Tensor) -> L.StepArgs:
        t = self.t
        par, nxt = t % 2, (t + 1) % 2
        kc = self.k_spec if t > 0 else 0
        vp = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
        bud = ctypes.addressof(self.budgets[par]) if self.budgets else None
        return L.StepArgs(vp(q), vp(self.k_cache), vp(self.v_cache), vp(self.table), vp(self.summaries),
                          vp(self.scores[par]), vp(self.sel_idx), vp(self.ema), vp(self.pred[par]),
                          vp(self.pred[nxt]), vp(self.partials[par]), vp(self.out[par]), vp(self.missed[par]),
                          vp(self.workspace), self.top_k, kc, self.k_spec, int(t == 0), self.alpha, bud)

    def enqueue(self, q: torch.Tensor, join: bool = False) -> torch.Tensor:
        """Enqueue one step on the layer's streams without touching the caller's stream (for timing loops and graph
        capture). Returns the output buffer (valid once stream_sel reaches this point; reused two steps later)."""
        if q.dtype != self.shape.torch_dtype or not q.is_contiguous() or not q.is_cuda:
            raise L.PRRError("q must be a contiguous device tensor of the layer's dtype")
        if tuple(q.shape) != (self.shape.batch, self.shape.n_q_heads, self.shape.head_dim):
            raise L.PRRError(f"q has shape {tuple(q.shape)}")
        out = self.out[self.t % 2]
        step = L.decode_step_noalloc if self.static_workspace else L.decode_step
        step(self.ctx, self.shape, self._args(q), MODES[self.mode], join, self.s_sel, self.s_spec)
        self.t += 1
        return out

    def step(self, q: torch.Tensor) -> torch.Tensor:
        """One decode step for queries q [B, Hq, D]; returns out [B, Hq, D] fp32, ordered on the current stream."""
        cur = torch.cuda.current_stream(self.device)
        self.s_sel.wait_stream(cur)
        out = self.enqueue(q)
        cur.wait_stream(self.s_sel)
        return out

    def sync_spec(self) -> None:
        """Make the current stream wait for the speculation stream (its last speculation launch)."""
        torch.cuda.current_stream(self.device).wait_stream(self.s_spec)

    @property
    def pred_current(self) -> torch.Tensor:
        """Predicted set that the last step used (valid after step >= 1)."""
        return self.pred[(self.t - 1) % 2][..., :self.k_spec]

    @property
    def pred_next(self) -> torch.Tensor:
        return self.pred[self.t % 2][..., :self.k_spec]

    @property
    def n_missed(self) -> torch.Tensor:
        """Missed blocks per row of the last step (|T minus P|; all of T when nothing was predicted)."""
        return self.missed[(self.t - 1) % 2]

    @property
    def scores_last(self) -> torch.Tensor:
        return self.scores[(self.t - 1) % 2]
