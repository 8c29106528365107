"""Plain, slow fp64 CPU oracle for one decode step of PRR's dynamic sparse attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may import this
module. The HIP library never uses it, and it shares no code with the HIP library: it reads plain numpy arrays and
computes every quantity from its definition in float64.

Sources (the pages describing "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context
LLM Decoding", arXiv 2606.30389):
  * PRR abstract: decoding attends only to the top-K KV blocks relevant to each query; an EMA-based predictor
    forecasts the blocks; attention is speculated over them while selection runs; missed blocks are folded into the
    partial attention state with online-softmax statistics once the true set is known.
  * PRR summary page (arxivlens), Summary / Key findings / Contributions: the repair covers exactly the missed
    blocks and the result keeps standard DSA accuracy (full top-K coverage); Limitations: the budget comes from
    profiled latency grids plus polynomial regression off the grid.
  * PRR reference list: Quest (query-aware block scores from per-block elementwise key min/max), FlashAttention-2
    (online softmax), PagedAttention (paged KV cache with a block table).

Readings where the pages are silent (each is listed in the design notes):
  * score: Quest's per-head upper bound sum_d max(q_d * kmin_d, q_d * kmax_d), summed over the query heads of the
    KV group (one selection per sequence and KV head);
  * top-K ties go to the lower block index; index lists are reported in ascending order; optional forced blocks
    (the first n_sink and last n_local) rank first;
  * the EMA averages block scores: e_0 = s_0, e_t = alpha * e_{t-1} + (1 - alpha) * s_t; step 0 has no prediction;
    the prediction for step t is the top-K' of e_{t-1} with the same tie rule;
  * softmax scale 1/sqrt(D);
  * budget: K'* is the largest profiled K' whose speculation time does not exceed the selection time predicted for
    the target block count (a least-squares polynomial in the block count when that count is off the grid).

Layouts: K/V caches [n_pages, Hkv, page, D]; block table int32 [B, pages_per_seq]; logical token i of sequence b sits
in physical page table[b, i // page] at row i % page.
"""
from __future__ import annotations

import math
from itertools import combinations

import numpy as np

# ------------------------------------------------------------------------------------------------------------------
# paged KV cache (PagedAttention, in the PRR reference list)
# ------------------------------------------------------------------------------------------------------------------


def logical_tokens(cache: np.ndarray, table: np.ndarray, b: int, g: int, n_tokens: int) -> np.ndarray:
    """Keys (or values) of sequence b, KV head g in logical token order, as float64 [n_tokens, D]."""
    page = cache.shape[2]
    i = np.arange(n_tokens)
    return np.asarray(cache[table[b, i // page], g, i % page], dtype=np.float64)


# ------------------------------------------------------------------------------------------------------------------
# Quest block summaries and scores (Quest, in the PRR reference list)
# ------------------------------------------------------------------------------------------------------------------


def block_summaries(keys: np.ndarray, block_size: int):
    """Elementwise min and max of the keys of each block: kmin, kmax [N, D] (exact: comparisons only). Block n holds
    tokens [n * block_size, (n + 1) * block_size) of the sequence; when the sequence ends inside a block (decode
    appends one token at a time), the last block's summary covers the tokens it holds."""
    n_tok, d = keys.shape
    if n_tok % block_size == 0:   # whole blocks: the same min and max, vectorised
        kb = keys.reshape(n_tok // block_size, block_size, d)
        return kb.min(axis=1), kb.max(axis=1)
    n_blk = -(-n_tok // block_size)
    kmin = np.empty((n_blk, d), dtype=keys.dtype)
    kmax = np.empty((n_blk, d), dtype=keys.dtype)
    for n in range(n_blk):
        blk = keys[n * block_size:(n + 1) * block_size]
        kmin[n] = blk.min(axis=0)
        kmax[n] = blk.max(axis=0)
    return kmin, kmax


def quest_scores(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """s[n] = sum over the group's heads h and dims d of max(q_hd * kmin_nd, q_hd * kmax_nd)  (plain max form).

    For one head this bounds max_i q . k_i over the block's tokens from above."""
    s = np.zeros(kmin.shape[0], dtype=np.float64)
    for h in range(q_group.shape[0]):
        q = q_group[h].astype(np.float64)
        s += np.maximum(kmin * q, kmax * q).sum(axis=1)
    return s


def quest_scores_signsplit(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Same value as quest_scores via max(q*a, q*b) = max(q,0)*b + min(q,0)*a for a <= b (faster; used for large
    sampled checks; pinned against the plain form)."""
    qp = np.maximum(q_group, 0.0).sum(axis=0)
    qn = np.minimum(q_group, 0.0).sum(axis=0)
    return kmax @ qp + kmin @ qn


def block_means(keys: np.ndarray, block_size: int) -> np.ndarray:
    """Mean key of each block over the tokens it holds: [N, D] (float64)."""
    n_tok = len(keys)
    n_blk = -(-n_tok // block_size)
    return np.stack([np.asarray(keys[n * block_size:(n + 1) * block_size], dtype=np.float64).mean(axis=0)
                     for n in range(n_blk)])


def mean_key_scores(q_group: np.ndarray, keys: np.ndarray, block_size: int) -> np.ndarray:
    """A second scorer (representative-key block scores; the PRR abstract speaks of representative DSA methods):
    s[n] = sum over the group's heads h of q_h . mean of the block's keys, i.e. the block's average group-summed
    logit before scaling."""
    means = block_means(keys, block_size)
    return means @ np.asarray(q_group, dtype=np.float64).sum(axis=0)


# ------------------------------------------------------------------------------------------------------------------
# top-K block selection (PRR abstract: attend only to the top-K blocks)
# ------------------------------------------------------------------------------------------------------------------


def top_k(values: np.ndarray, k: int, n_sink: int = 0, n_local: int = 0) -> np.ndarray:
    """Indices of the k largest values, ties to the lower index; returned ascending (int64).

    Forced blocks (attention sinks and a local window; StreamingLLM in the PRR reference list): the first n_sink and
    the last n_local blocks rank above every other block, among themselves by index, so they are always selected
    when k covers them."""
    n = len(values)
    idx = np.arange(n)
    forced = (idx < n_sink) | (idx >= n - n_local)
    rank_value = np.where(forced, 0.0, -np.asarray(values, dtype=np.float64))   # forced: by index alone
    order = np.lexsort((idx, rank_value, ~forced))
    return np.sort(order[:k])


def boundary_gap(values: np.ndarray, k: int):
    """(v_(k), v_(k+1), relative gap (v_(k) - v_(k+1)) / |v_(k)|), v_(i) the i-th largest value.

    gap = inf when k == n (nothing is left out). When v_(k) = 0 the relative gap is inf if v_(k+1) < 0 and 0 if the
    two are equal. A positive gap means the top-k set is the only k-set of largest sum."""
    v = np.sort(np.asarray(values, dtype=np.float64))[::-1]
    if k >= len(v):
        return float(v[k - 1]), -math.inf, math.inf
    a, b = float(v[k - 1]), float(v[k])
    return a, b, (a - b) / abs(a) if a != 0 else (math.inf if a > b else 0.0)


# ------------------------------------------------------------------------------------------------------------------
# attention over a block set: the definition of the output (standard DSA over the true top-K set)
# ------------------------------------------------------------------------------------------------------------------


def block_tokens(blocks, block_size: int, n_tokens: int) -> np.ndarray:
    """Token indices of ``blocks`` in a sequence of n_tokens tokens (a last, partly filled block holds fewer)."""
    parts = [np.arange(n * block_size, min((n + 1) * block_size, n_tokens)) for n in blocks]
    return np.concatenate(parts) if parts else np.zeros((0,), dtype=np.int64)


def attention_over_blocks(q_group, keys, values, blocks, block_size: int, scale: float) -> np.ndarray:
    """o[h] = softmax(scale * q_h . k_i) weighted sum of v_i over the tokens of ``blocks`` (keys and values hold the
    sequence's tokens); two-pass softmax (max first, then the sum), float64. Returns [G, D]."""
    idx = block_tokens(blocks, block_size, len(keys))
    k = keys[idx]
    v = values[idx]
    out = np.empty((q_group.shape[0], keys.shape[1]), dtype=np.float64)
    for h in range(q_group.shape[0]):
        z = scale * (k @ q_group[h].astype(np.float64))
        zmax = z.max()
        w = np.exp(z - zmax)
        out[h] = (w @ v) / w.sum()
    return out


# ------------------------------------------------------------------------------------------------------------------
# online-softmax partial states and their merge (FlashAttention-2 in the reference list; PRR abstract: the repair
# folds missed blocks into the partial attention state using online-softmax statistics)
# ------------------------------------------------------------------------------------------------------------------


def block_partial(q_h, k_blk, v_blk, scale: float):
    """(m, l, O) of one head over one block: m = max z, l = sum exp(z - m), O = sum exp(z - m) v."""
    z = scale * (k_blk @ np.asarray(q_h, dtype=np.float64))
    m = z.max()
    p = np.exp(z - m)
    return float(m), float(p.sum()), p @ v_blk


def merge(a, b):
    """Online-softmax merge of two partial states over disjoint token sets."""
    (m1, l1, o1), (m2, l2, o2) = a, b
    m = max(m1, m2)
    c1, c2 = math.exp(m1 - m), math.exp(m2 - m)
    return m, l1 * c1 + l2 * c2, o1 * c1 + o2 * c2


def finalize(state) -> np.ndarray:
    m, l, o = state
    return o / l


def prr_output(q_group, keys, values, true_set, pred_set, block_size: int, scale: float):
    """Reference speculate-reuse-repair pipeline for one (sequence, KV head).

    Speculation leaves one partial per predicted block; repair computes partials for the missed blocks M = T \\ P;
    the output merges, in ascending block order, the speculated partials of T n P and the repaired partials of M.
    Predicted blocks outside T never enter. Returns (o [G, D], missed ascending, wasted ascending)."""
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    T = [int(n) for n in true_set]
    P = {int(n) for n in pred_set}
    spec = {}
    for n in P:                                   # speculation over every predicted block
        sl = slice(n * block_size, (n + 1) * block_size)
        spec[n] = [block_partial(q_group[h], keys[sl], values[sl], scale) for h in range(q_group.shape[0])]
    missed = [n for n in T if n not in P]
    out = np.empty((q_group.shape[0], keys.shape[1]), dtype=np.float64)
    for h in range(q_group.shape[0]):
        state = None
        for n in sorted(T):
            if n in P:
                part = spec[n][h]
            else:                                 # repair: a missed block
                sl = slice(n * block_size, (n + 1) * block_size)
                part = block_partial(q_group[h], keys[sl], values[sl], scale)
            state = part if state is None else merge(state, part)
        out[h] = finalize(state)
    wasted = sorted(P - set(T))
    return out, np.asarray(missed, dtype=np.int64), np.asarray(wasted, dtype=np.int64)


# ------------------------------------------------------------------------------------------------------------------
# decode-time append: the sequence gains one token per step (its key and value); the summaries and every later
# quantity are the definitions above applied to the longer sequence
# ------------------------------------------------------------------------------------------------------------------


def append_token(keys: np.ndarray, values: np.ndarray, k_new, v_new):
    """The sequence's keys and values after one decode step appends (k_new, v_new): [n + 1, D] each."""
    return (np.concatenate([keys, np.asarray(k_new, dtype=np.float64)[None]]),
            np.concatenate([values, np.asarray(v_new, dtype=np.float64)[None]]))


# ------------------------------------------------------------------------------------------------------------------
# EMA score predictor (PRR abstract: a light predictor built on an exponential moving average; summary page: it
# forecasts the top-K blocks)
# ------------------------------------------------------------------------------------------------------------------


def ema_update(ema_prev, scores, alpha: float, first: bool) -> np.ndarray:
    s = np.asarray(scores, dtype=np.float64)
    if first:
        return s.copy()
    return alpha * np.asarray(ema_prev, dtype=np.float64) + (1.0 - alpha) * s


def predict(ema, k_spec: int, n_sink: int = 0, n_local: int = 0) -> np.ndarray:
    """Predicted set for the next step: top-K' of the EMA with the selection's tie rule and forced blocks
    (ascending)."""
    return top_k(ema, k_spec, n_sink, n_local)


# ------------------------------------------------------------------------------------------------------------------
# per-row budgets of the predicted set (PRR summary page: speculative work is held to a dynamic budget; Future work:
# adaptive budgeting, and confidence measures for the EMA predictor). The pages give no formula for either; both
# rules below are readings. The device takes their integer decisions in fp32, so these functions do too.
# ------------------------------------------------------------------------------------------------------------------


def budget_from_misses(missed_prev, k_top: int, k_cap: int, beta: float, k_min: int) -> np.ndarray:
    """Size of each row's next predicted set from the blocks the row missed at its last completed step:
    k = K + ceil(beta * m), clamped to [k_min, k_cap]. A row whose prediction missed more blocks speculates more.
    beta * m is an fp32 product."""
    m = np.asarray(missed_prev).astype(np.float32)
    grow = np.minimum(np.ceil(np.float32(beta) * m), np.float32(k_cap))   # k_cap bounds k anyway; keeps the cast exact
    return np.minimum(np.maximum(k_top + grow.astype(np.int64), k_min), k_cap)


def confidence_bound(scores, ema, c: float) -> np.ndarray:
    """u = e + c * |s - e| per block, every operation rounded to fp32: the EMA raised by c times its disagreement
    with the step's score, an optimistic score for blocks whose scores move."""
    s = np.asarray(scores, dtype=np.float32)
    e = np.asarray(ema, dtype=np.float32)
    return e + np.float32(c) * np.abs(s - e)


def budget_from_confidence(scores, ema, k_top: int, k_cap: int, c: float, k_min: int, n_sink: int = 0,
                           n_local: int = 0):
    """(k, u): k counts the blocks whose optimistic score u reaches the K-th entry of the EMA in the selection order
    (forced blocks first, then larger value, then lower index), clamped to [k_min, k_cap]. A forced block reaches
    every value; when the K-th entry is itself forced, only forced blocks reach it."""
    e = np.asarray(ema, dtype=np.float32)
    u = confidence_bound(scores, e, c)
    n = len(e)
    idx = np.arange(n)
    forced = (idx < n_sink) | (idx >= n - n_local)
    order = np.lexsort((idx, -e.astype(np.float64), ~forced))   # the selection order of the EMA
    kth = order[k_top - 1]
    if forced[kth]:
        count = int(forced.sum())
    else:
        count = int(forced.sum()) + int(np.count_nonzero(~forced & (u >= e[kth])))
    return int(min(max(count, k_min), k_cap)), u


def predict_confident(scores, ema, k_top: int, k_cap: int, c: float, k_min: int, n_sink: int = 0,
                      n_local: int = 0) -> np.ndarray:
    """Confidence-aware prediction: the k blocks with the largest optimistic scores u (forced first, ties to the
    lower index), k from budget_from_confidence; ascending."""
    k, u = budget_from_confidence(scores, ema, k_top, k_cap, c, k_min, n_sink, n_local)
    return top_k(u, k, n_sink, n_local)


# ------------------------------------------------------------------------------------------------------------------
# profiling-guided speculation budget (PRR abstract; summary page, Limitations: polynomial regression off the grid)
# ------------------------------------------------------------------------------------------------------------------


def choose_budget(n_grid, t_sel, kspec_grid, t_spec, n_target: float, degree: int = 2) -> int:
    """Largest profiled K' whose measured speculation time is at most the selection time at n_target blocks.

    The selection time at n_target is the measured one when n_target is on the grid, else a least-squares polynomial
    of ``degree`` in the block count. K' = 0 is always admissible."""
    n_grid = np.asarray(n_grid, dtype=np.float64)
    t_sel = np.asarray(t_sel, dtype=np.float64)
    hit = np.flatnonzero(n_grid == n_target)
    if len(hit):
        t_target = float(t_sel[hit[0]])
    else:
        coef = np.polyfit(n_grid, t_sel, min(degree, len(n_grid) - 1))
        t_target = float(np.polyval(coef, n_target))
    best = 0
    for k, t in zip(kspec_grid, t_spec):
        if t <= t_target and k > best:
            best = int(k)
    return best


def choose_budget_fused(kspec_grid, t_step) -> int:
    """Budget of the fused single-stream step, where the speculation shares the selection launch: both its cost (the
    launch grows) and its saving (fewer missed blocks to repair) show only in the step's own time, so the profile
    measures the step at each grid budget (the grid holds 0, the step without speculation). K'* is the largest
    profiled K' whose step time is at most the step time without speculation: the largest budget that keeps the
    speculative work off the step's critical path."""
    ks = [int(k) for k in kspec_grid]
    t0 = float(t_step[ks.index(0)])
    best = 0
    for k, t in zip(ks, t_step):
        if float(t) <= t0 and k > best:
            best = k
    return best


# ------------------------------------------------------------------------------------------------------------------
# brute force (tiny inputs only): used by the pins
# ------------------------------------------------------------------------------------------------------------------


def brute_force_top_k(values, k: int, forced=()):
    """Among all k-subsets that contain the forced blocks (or, when k is smaller than their number, that lie inside
    them), the one with the largest sum; ties to the lexicographically smallest ascending tuple."""
    forced = set(forced)
    best, best_sum = None, -math.inf
    for c in combinations(range(len(values)), k):
        cs = set(c)
        if (len(forced) <= k and not forced <= cs) or (len(forced) > k and not cs <= forced):
            continue
        s = float(sum(values[i] for i in c)) if len(forced) <= k else -float(sum(c))
        if s > best_sum or (s == best_sum and c < best):
            best, best_sum = c, s
    return np.asarray(best, dtype=np.int64)
