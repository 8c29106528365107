"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle module ``o`` disagrees with:
  * a library special case (all blocks selected = dense attention, checked against torch's
    scaled_dot_product_attention in float64 on the CPU),
  * brute force on tiny inputs (every K-subset),
  * closed forms (zero query, constant values, one-token blocks, EMA of a linear ramp, linear latency tables),
  * invariants stated by the pages (repair covers exactly the missed blocks and the output equals standard DSA over
    the true set, whatever was predicted: PRR summary page, Summary and Key findings),
  * the hand-worked example in tests/golden.
They take the module as an argument so that tests/test_oracle_mutants.py can show that planted mistakes fail them.
"""
from __future__ import annotations

import json
import math
import os

from itertools import combinations

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, n_blocks=6, bs=3, d=5, g=2):
    keys = rng.standard_normal((n_blocks * bs, d))
    values = rng.standard_normal((n_blocks * bs, d))
    q = rng.standard_normal((g, d))
    return q, keys, values


def pin_dense_equivalence(o):
    """K = N: attention over every block equals dense softmax attention (torch SDPA, fp64, CPU)."""
    rng = np.random.default_rng(11)
    for (nb, bs, d, g) in [(4, 8, 16, 4), (7, 3, 5, 1), (16, 32, 64, 4)]:
        q, k, v = _rand_problem(rng, nb, bs, d, g)
        scale = 1.0 / math.sqrt(d)
        got = o.attention_over_blocks(q, k, v, np.arange(nb), bs, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, g, -1, -1),
            torch.from_numpy(v)[None, None].expand(1, g, -1, -1), scale=scale)[0, :, 0, :].numpy()
        assert np.allclose(got, ref, rtol=0, atol=1e-13), np.abs(got - ref).max()
        # the speculate-reuse-repair pipeline with an arbitrary prediction gives the same dense result
        pred = rng.choice(nb, size=max(1, nb // 2), replace=False)
        got2, _, _ = o.prr_output(q, k, v, np.arange(nb), pred, bs, scale)
        assert np.allclose(got2, ref, rtol=0, atol=1e-13)


def pin_brute_force_selection(o):
    """Tiny inputs: the selected set maximises the summed score over all K-subsets (ties: lowest indices)."""
    rng = np.random.default_rng(12)
    for trial in range(60):
        nb = int(rng.integers(2, 9))
        bs = int(rng.integers(1, 5))
        d = int(rng.integers(1, 9))
        g = int(rng.integers(1, 3))
        k = int(rng.integers(1, nb + 1))
        q, keys, _ = _rand_problem(rng, nb, bs, d, g)
        if trial % 3 == 0:   # integer-valued data: exact ties in the scores
            q = np.round(q * 2)
            keys = np.round(keys)
        kmin, kmax = o.block_summaries(keys, bs)
        # summaries against a per-token scan
        for n in range(nb):
            blk = keys[n * bs:(n + 1) * bs]
            for dd in range(d):
                assert kmin[n, dd] == min(blk[:, dd]) and kmax[n, dd] == max(blk[:, dd])
        s = o.quest_scores(q, kmin, kmax)
        # score against its element-by-element definition
        for n in range(nb):
            ref = sum(max(q[h, dd] * kmin[n, dd], q[h, dd] * kmax[n, dd]) for h in range(g) for dd in range(d))
            assert abs(s[n] - ref) <= 1e-12 * max(1.0, abs(ref))
        got = o.top_k(s, k)
        ref = o.brute_force_top_k(list(s), k)
        assert list(got) == list(ref), (s, got, ref)


def pin_quest_upper_bound(o):
    """Per head, the block score bounds the largest exact q.k over the block's tokens from above; with one token per
    block it equals the exact dot product (summed over the group's heads)."""
    rng = np.random.default_rng(13)
    for _ in range(20):
        q, keys, _ = _rand_problem(rng, 8, 4, 16, 1)
        kmin, kmax = o.block_summaries(keys, 4)
        s = o.quest_scores(q, kmin, kmax)
        exact = (keys @ q[0]).reshape(8, 4).max(axis=1)
        assert np.all(s >= exact - 1e-12)
        qg, keys1, _ = _rand_problem(rng, 10, 1, 16, 4)
        kmin, kmax = o.block_summaries(keys1, 1)
        s1 = o.quest_scores(qg, kmin, kmax)
        assert np.allclose(s1, keys1 @ qg.sum(axis=0), rtol=0, atol=1e-12)


def pin_signsplit(o):
    rng = np.random.default_rng(14)
    q, keys, _ = _rand_problem(rng, 64, 8, 32, 4)
    kmin, kmax = o.block_summaries(keys, 8)
    a = o.quest_scores(q, kmin, kmax)
    b = o.quest_scores_signsplit(q, kmin, kmax)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def pin_merge_order_free(o):
    """Merging per-block partials in any order and bracketing equals the two-pass softmax over their union."""
    rng = np.random.default_rng(15)
    q, k, v = _rand_problem(rng, 9, 5, 8, 1)
    k = k * 3.0   # spread the logits so the rescaling matters
    scale = 0.7
    parts = [o.block_partial(q[0], k[n * 5:(n + 1) * 5], v[n * 5:(n + 1) * 5], scale) for n in range(9)]
    ref = o.attention_over_blocks(q, k, v, np.arange(9), 5, scale)[0]
    for trial in range(20):
        order = rng.permutation(9)
        pool = [parts[i] for i in order]
        while len(pool) > 1:   # random bracketing
            i = int(rng.integers(len(pool) - 1))
            pool[i:i + 2] = [o.merge(pool[i], pool[i + 1])]
        got = o.finalize(pool[0])
        assert np.allclose(got, ref, rtol=0, atol=1e-13), np.abs(got - ref).max()
    # a partial's own fields against their definitions; the merged m is the running maximum of every logit
    m, l, O = parts[0]
    z = scale * (k[:5] @ q[0])
    assert abs(m - z.max()) < 1e-15 and abs(l - np.exp(z - z.max()).sum()) < 1e-13
    zall = scale * (k @ q[0])
    m_all = o.merge(o.merge(parts[3], parts[0]), parts[7])[0]
    assert m_all == max(zall[15:20].max(), zall[0:5].max(), zall[35:40].max())
    # logits hundreds apart: the merge must not overflow (weights relative to the running maximum)
    big = [o.block_partial(q[0], 400.0 * n * np.tile(q[0], (5, 1)) / (q[0] @ q[0]), v[n * 5:(n + 1) * 5], 1.0)
           for n in range(3)]
    st = o.merge(o.merge(big[2], big[0]), big[1])
    assert np.all(np.isfinite(o.finalize(st))) and np.allclose(o.finalize(st), v[10:15].mean(axis=0), atol=1e-12)


def pin_repair_invariants(o):
    """P = T needs no repair; P = {} repairs everything; any P (random, disjoint, poisoned) gives the same output."""
    rng = np.random.default_rng(16)
    nb, bs, d, g, K = 12, 4, 8, 2, 5
    q, keys, vals = _rand_problem(rng, nb, bs, d, g)
    kmin, kmax = o.block_summaries(keys, bs)
    T = o.top_k(o.quest_scores(q, kmin, kmax), K)
    scale = 1 / math.sqrt(d)
    ref = o.attention_over_blocks(q, keys, vals, T, bs, scale)
    out, missed, wasted = o.prr_output(q, keys, vals, T, T, bs, scale)
    assert len(missed) == 0 and len(wasted) == 0 and np.allclose(out, ref, rtol=0, atol=1e-13)
    out, missed, wasted = o.prr_output(q, keys, vals, T, [], bs, scale)
    assert list(missed) == list(T) and len(wasted) == 0 and np.allclose(out, ref, rtol=0, atol=1e-13)
    outside = [n for n in range(nb) if n not in set(T)]
    for P in [rng.choice(nb, 7, replace=False), outside, list(T[:2]) + outside[:3]]:
        out, missed, wasted = o.prr_output(q, keys, vals, T, P, bs, scale)
        assert sorted(set(missed) | (set(T) & set(P))) == sorted(T)
        assert sorted(wasted) == sorted(set(P) - set(T))
        assert np.allclose(out, ref, rtol=0, atol=1e-13)
    # a poison block (keys aligned with every query, huge logits) that is predicted but not selected must not leak
    pk = keys.copy()
    pois = outside[0]
    pk[pois * bs:(pois + 1) * bs] = 100.0 * q.sum(axis=0) / np.linalg.norm(q.sum(axis=0))
    ref_p = o.attention_over_blocks(q, pk, vals, T, bs, scale)
    out, _, wasted = o.prr_output(q, pk, vals, T, [pois] + list(T), bs, scale)
    assert list(wasted) == [pois] and np.allclose(out, ref_p, rtol=0, atol=1e-13)
    assert np.allclose(ref_p, ref)


def pin_closed_forms(o):
    rng = np.random.default_rng(17)
    nb, bs, d, g, K = 10, 4, 6, 3, 4
    _, keys, vals = _rand_problem(rng, nb, bs, d, g)
    # q = 0: all scores 0, T = first K blocks, uniform weights -> mean of V over T
    q0 = np.zeros((g, d))
    kmin, kmax = o.block_summaries(keys, bs)
    s = o.quest_scores(q0, kmin, kmax)
    T = o.top_k(s, K)
    assert list(T) == list(range(K))
    out = o.attention_over_blocks(q0, keys, vals, T, bs, 0.5)
    assert np.allclose(out, vals[:K * bs].mean(axis=0)[None], rtol=0, atol=1e-14)
    # constant V: the output is that constant
    q = rng.standard_normal((g, d))
    c = rng.standard_normal(d)
    out = o.attention_over_blocks(q, keys, np.tile(c, (nb * bs, 1)), [1, 4, 7], bs, 0.3)
    assert np.allclose(out, c[None], rtol=0, atol=1e-14)
    # one-token blocks, K = 1: the output is v of the token with the largest group-summed dot product
    k1 = rng.standard_normal((nb, d))
    v1 = rng.standard_normal((nb, d))
    q1 = rng.standard_normal((1, d))
    kmin, kmax = o.block_summaries(k1, 1)
    T = o.top_k(o.quest_scores(q1, kmin, kmax), 1)
    assert T[0] == int(np.argmax(k1 @ q1[0]))
    assert np.allclose(o.attention_over_blocks(q1, k1, v1, T, 1, 0.125)[0], v1[T[0]], rtol=0, atol=1e-15)


def pin_hand_example(o):
    ex = json.load(open(os.path.join(GOLDEN, "hand_worked_example.json")))
    q = np.asarray(ex["q"], dtype=np.float64)
    keys = np.asarray(ex["keys"], dtype=np.float64)
    vals = np.asarray(ex["values"], dtype=np.float64)
    bs, K = ex["block_size"], ex["top_k"]
    kmin, kmax = o.block_summaries(keys, bs)
    assert kmin.tolist() == ex["kmin"] and kmax.tolist() == ex["kmax"]
    s = o.quest_scores(q, kmin, kmax)
    assert s.tolist() == ex["scores"]
    T = o.top_k(s, K)
    assert T.tolist() == ex["selected"]
    out = o.attention_over_blocks(q, keys, vals, T, bs, math.log(2.0))
    assert np.allclose(out[0] * 12.0, ex["out_numerator_over_12"], rtol=0, atol=1e-12)
    out2, missed, wasted = o.prr_output(q, keys, vals, T, ex["pred"], bs, math.log(2.0))
    assert missed.tolist() == ex["missed"] and wasted.tolist() == ex["wasted"]
    assert np.allclose(out2, out, rtol=0, atol=1e-13)


def pin_ema_closed_form(o):
    """EMA of a linear ramp s_t = (t0 + t) c started at e_0 = s_0: the constant t0 c passes through unchanged and the
    ramp part gives e_t = (t0 + t - a/(1-a) + a^(t+1)/(1-a)) c."""
    t0 = 5.0
    for a in (0.9, 0.7, 0.5):
        c = np.array([1.0, -2.0, 0.5])
        e = None
        for t in range(30):
            e = o.ema_update(e, (t0 + t) * c, a, first=(t == 0))
            ref = (t0 + t - a / (1 - a) + a ** (t + 1) / (1 - a)) * c
            assert np.allclose(e, ref, rtol=0, atol=1e-12), (t, e, ref)
    # prediction uses the same tie rule as selection
    assert o.predict(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), 2).tolist() == [1, 2]


def pin_budget_closed_form(o):
    """Linear latency tables: t_sel(N) = 2 + 0.01 N, t_spec(K') = 1 + 0.05 K'. At N = 1000 (off the grid),
    t_sel = 12, so the largest admissible K' on the grid {0, 64, ..., 384} is the largest with 1 + 0.05 K' <= 12,
    i.e. K' <= 220 -> 192. At N = 4096 (on the grid) t_sel = 42.96 -> K' <= 839.2 -> 384."""
    n_grid = [256, 512, 2048, 4096, 8192]
    t_sel = [2 + 0.01 * n for n in n_grid]
    ks = [0, 64, 128, 192, 256, 320, 384]
    t_spec = [1 + 0.05 * k for k in ks]
    assert o.choose_budget(n_grid, t_sel, ks, t_spec, 1000) == 192
    assert o.choose_budget(n_grid, t_sel, ks, t_spec, 4096) == 384
    assert o.choose_budget(n_grid, t_sel, ks, [100.0] * len(ks), 1000) == 0
    # a quadratic table is reproduced exactly off the grid: t_sel = 1 + N^2 / 1e6 -> at 3000: 10 -> K' <= 180 -> 128
    t_q = [1 + n * n / 1e6 for n in n_grid]
    assert o.choose_budget(n_grid, t_q, ks, t_spec, 3000) == 128


def pin_paged_gather(o):
    """Logical token order through a permuted page table, against a hand-built cache: page p of sequence b holds
    tokens [p * page, (p + 1) * page), so entry (phys, g, r) of the cache is token table[b].index(phys) * page + r."""
    B, Hkv, page, D, pps = 2, 3, 4, 2, 5
    table = np.array([[7, 2, 9, 0, 4], [1, 8, 3, 6, 5]], dtype=np.int32)
    cache = np.zeros((B * pps, Hkv, page, D))
    for b in range(B):
        for p in range(pps):
            for g in range(Hkv):
                for r in range(page):
                    tok = p * page + r
                    cache[table[b, p], g, r] = [1000 * b + 100 * g + tok, -tok]
    for b in range(B):
        for g in range(Hkv):
            got = o.logical_tokens(cache, table, b, g, pps * page)
            ref = np.array([[1000 * b + 100 * g + i, -i] for i in range(pps * page)], dtype=np.float64)
            assert np.array_equal(got, ref)


def pin_partial_last_block(o):
    """A sequence that ends inside a block (decode appends one token at a time): with every block selected the output
    is dense attention over the tokens that exist (torch SDPA, fp64), through the speculate-reuse-repair pipeline
    too; a one-token last block's summary is that token's key; the Quest score of the partial block bounds the exact
    largest q.k over its tokens; appending tokens one by one gives, at every length, the summaries of that prefix
    and dense attention over it."""
    rng = np.random.default_rng(19)
    for (n_tok, bs, d, g) in [(13, 4, 6, 2), (17, 8, 5, 1), (33, 32, 16, 4), (9, 3, 4, 3)]:
        q = rng.standard_normal((g, d))
        k = rng.standard_normal((n_tok, d))
        v = rng.standard_normal((n_tok, d))
        scale = 1.0 / math.sqrt(d)
        nb = -(-n_tok // bs)
        kmin, kmax = o.block_summaries(k, bs)
        assert kmin.shape == (nb, d) and kmax.shape == (nb, d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, g, -1, -1),
            torch.from_numpy(v)[None, None].expand(1, g, -1, -1), scale=scale)[0, :, 0, :].numpy()
        got = o.attention_over_blocks(q, k, v, np.arange(nb), bs, scale)
        assert np.allclose(got, ref, rtol=0, atol=1e-13), np.abs(got - ref).max()
        got2, missed, _ = o.prr_output(q, k, v, np.arange(nb), [nb - 1, 0], bs, scale)
        assert np.allclose(got2, ref, rtol=0, atol=1e-13) and nb - 1 not in set(missed)
        s = o.quest_scores(q[:1], kmin, kmax)
        last = k[(nb - 1) * bs:]
        assert s[nb - 1] >= (last @ q[0]).max() - 1e-12
    # one-token last block
    k = rng.standard_normal((9, 4))
    kmin, kmax = o.block_summaries(k, 4)
    assert np.array_equal(kmin[2], k[8]) and np.array_equal(kmax[2], k[8])
    # appending one token at a time
    bs, d, g = 4, 5, 2
    q = rng.standard_normal((g, d))
    k = rng.standard_normal((6, d))
    v = rng.standard_normal((6, d))
    for step in range(9):
        k_new, v_new = rng.standard_normal(d), rng.standard_normal(d)
        k, v = o.append_token(k, v, k_new, v_new)
        assert len(k) == 7 + step and np.array_equal(k[-1], k_new) and np.array_equal(v[-1], v_new)
        kmin, kmax = o.block_summaries(k, bs)
        n_last = (len(k) - 1) // bs
        assert np.array_equal(kmax[n_last], np.max(k[n_last * bs:], axis=0))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, g, -1, -1),
            torch.from_numpy(v)[None, None].expand(1, g, -1, -1), scale=0.5)[0, :, 0, :].numpy()
        got = o.attention_over_blocks(q, k, v, np.arange(n_last + 1), bs, 0.5)
        assert np.allclose(got, ref, rtol=0, atol=1e-13)


def pin_forced_blocks(o):
    """Forced blocks (attention sinks and a local window): against brute force over every K-subset that contains
    them (or lies inside them when K is smaller), with integer ties included; no forced blocks is the plain top-K;
    K equal to their number selects exactly them, even when they hold the lowest scores; the prediction forces them
    too."""
    rng = np.random.default_rng(21)
    for trial in range(80):
        nb = int(rng.integers(3, 10))
        sink = int(rng.integers(0, 3))
        local = int(rng.integers(0, 3))
        if sink + local > nb:
            continue
        k = int(rng.integers(1, nb + 1))
        vals = rng.standard_normal(nb)
        if trial % 3 == 0:
            vals = np.round(vals * 2)
        forced = [i for i in range(nb) if i < sink or i >= nb - local]
        got = o.top_k(vals, k, sink, local)
        ref = o.brute_force_top_k(list(vals), k, forced)
        assert list(got) == list(ref), (vals, k, sink, local, got, ref)
        assert list(o.top_k(vals, k, 0, 0)) == list(o.brute_force_top_k(list(vals), k))
    vals = np.array([-5.0, 3.0, 2.0, 9.0, 1.0, -7.0, -6.0])
    assert o.top_k(vals, 3, 1, 2).tolist() == [0, 5, 6]
    assert o.top_k(vals, 4, 1, 2).tolist() == [0, 3, 5, 6]
    assert o.predict(vals, 2, 1, 2).tolist() == [0, 5]


def pin_mean_key_scores(o):
    """The mean-key scorer: equal to the average over each block's tokens of the group-summed exact logits q . k
    (per token, a different order of summation); constant keys give that key's dot product; one-token blocks give
    the exact dot product; a partial last block averages over the tokens it holds; the Quest bound is never below
    it (a mean of dot products cannot exceed their maximum, which the bound covers)."""
    rng = np.random.default_rng(23)
    for (n_tok, bs, d, g) in [(24, 4, 6, 2), (19, 8, 5, 3), (7, 1, 4, 1)]:
        q = rng.standard_normal((g, d))
        k = rng.standard_normal((n_tok, d))
        s = o.mean_key_scores(q, k, bs)
        per_tok = np.array([sum(float(q[h] @ k[i]) for h in range(g)) for i in range(n_tok)])
        nb = -(-n_tok // bs)
        ref = np.array([per_tok[n * bs:(n + 1) * bs].mean() for n in range(nb)])
        assert np.allclose(s, ref, rtol=0, atol=1e-12)
        kmin, kmax = o.block_summaries(k, bs)
        assert np.all(o.quest_scores(q, kmin, kmax) >= s - 1e-12)
    c = rng.standard_normal(5)
    q = rng.standard_normal((2, 5))
    s = o.mean_key_scores(q, np.tile(c, (12, 1)), 4)
    assert np.allclose(s, q.sum(axis=0) @ c, rtol=0, atol=1e-13)


def pin_adaptive_budgets(o):
    """Per-row budgets of the predicted set (two readings of the pages' adaptive budget and confidence measures).
    Misses: worked values of K + ceil(beta * m) with clamping, no growth at beta = 0 or m = 0, and an fp32 decision
    where fp64 would round the other way (0.3f * 50 is 15.000001 in fp32 but 15.0 in fp64; 1.1f * 50 is 55.0 in
    fp32 but 55.00000000000001 in fp64). Confidence: against a
    plain loop over every block in fp32 plus brute force over every k-subset on tiny rows (forced blocks and integer
    ties included); c = 0 on distinct values is the plain top-K of the EMA; a huge c fills the cap."""
    assert o.budget_from_misses([0, 3, 10, 100], 8, 20, 0.5, 4).tolist() == [8, 10, 13, 20]
    assert o.budget_from_misses([0, 5], 8, 20, 0.0, 4).tolist() == [8, 8]
    assert o.budget_from_misses([0, 1], 3, 20, 0.5, 6).tolist() == [6, 6]     # k_min lifts small budgets
    assert o.budget_from_misses([50], 4, 64, 0.3, 1).tolist() == [20]          # fp32: 0.3f * 50 = 15.000001
    assert o.budget_from_misses([50], 4, 64, 1.1, 1).tolist() == [59]          # fp32: 1.1f * 50 = 55.0
    assert o.budget_from_misses([1], 4, 64, 0.25, 1).tolist() == [5]           # ceil(0.25) = 1
    assert o.budget_from_misses([5, 0], 8, 20, 1e30, 1).tolist() == [20, 8]    # a huge product stays at the cap

    # worked by hand: e = [2, 4, 3, 1, 7, 3, 1], s = [1, 5, 3, 2, 8, 0.5, 4], c = 1 gives u = e + |s - e| =
    # [3, 5, 3, 2, 8, 5.5, 4]; the 2nd largest EMA entry is 4 (block 1), four blocks have u >= 4 (1, 4, 5, 6)
    s_h = np.array([1, 5, 3, 2, 8, 0.5, 4], dtype=np.float32)
    e_h = np.array([2, 4, 3, 1, 7, 3, 1], dtype=np.float32)
    k_h, u_h = o.budget_from_confidence(s_h, e_h, 2, 6, 1.0, 1)
    assert k_h == 4 and u_h.tolist() == [3, 5, 3, 2, 8, 5.5, 4]
    assert o.predict_confident(s_h, e_h, 2, 6, 1.0, 1).tolist() == [1, 4, 5, 6]
    assert o.predict_confident(s_h, e_h, 2, 3, 1.0, 1).tolist() == [1, 4, 5]          # capped at 3
    assert o.predict_confident(s_h, e_h, 2, 6, 1.0, 5).tolist() == [0, 1, 4, 5, 6]    # k_min 5: next is block 0
    f32 = np.float32
    rng = np.random.default_rng(29)
    for trial in range(120):
        n = int(rng.integers(3, 9))
        sink = int(rng.integers(0, 2)) if trial % 2 else 0
        local = int(rng.integers(0, 2)) if trial % 3 == 0 else 0
        if sink + local >= n:
            continue
        kt = int(rng.integers(1, n + 1))
        cap = int(rng.integers(kt, n + 1))
        kmin = int(rng.integers(1, cap + 1))
        c = float(rng.choice([0.0, 0.5, 1.0, 3.0]))
        s = rng.standard_normal(n).astype(np.float32)
        e = rng.standard_normal(n).astype(np.float32)
        if trial % 4 == 0:
            s, e = np.round(s * 2).astype(np.float32), np.round(e * 2).astype(np.float32)
        forced = [i < sink or i >= n - local for i in range(n)]
        u = [f32(e[i]) + f32(c) * f32(abs(f32(s[i]) - f32(e[i]))) for i in range(n)]
        rank = sorted(range(n), key=lambda i: (not forced[i], -float(e[i]), i))
        kth = rank[kt - 1]
        if forced[kth]:
            count = sum(forced)
        else:
            count = sum(1 for i in range(n) if forced[i] or u[i] >= e[kth])
        k = min(max(count, kmin), cap)
        got_k, got_u = o.budget_from_confidence(s, e, kt, cap, c, kmin, sink, local)
        assert got_k == k, (trial, got_k, k)
        assert np.array_equal(np.asarray(got_u, dtype=np.float32), np.asarray(u, dtype=np.float32))
        ref = o.brute_force_top_k([float(x) for x in u], k, [i for i in range(n) if forced[i]])
        got = o.predict_confident(s, e, kt, cap, c, kmin, sink, local)
        assert list(got) == list(ref), (trial, got, ref)
    e = rng.permutation(40).astype(np.float32)
    s = e + rng.standard_normal(40).astype(np.float32)
    assert o.predict_confident(s, e, 7, 20, 0.0, 1).tolist() == o.top_k(e, 7).tolist()
    assert len(o.predict_confident(s, e, 7, 20, 1e30, 1)) == 20


def _maximising_k_sets(values, k):
    """Number of k-subsets whose summed value is the largest (brute force)."""
    sums = [sum(values[i] for i in c) for c in combinations(range(len(values)), k)]
    best = max(sums)
    return sum(1 for x in sums if x == best)


def pin_boundary_gap(o):
    """The relative gap at the K-th/(K+1)-th boundary on hand-worked vectors (distinct values, an exact tie, k = n,
    a negative K-th value, a zero K-th value above and equal to the next), and what it means: on integer-valued
    vectors a positive gap leaves exactly one k-set of largest sum, a zero gap at least two (brute force)."""
    inf = math.inf
    cases = [
        ([5.0, 3.0, 9.0, 1.0], 2, 5.0, 3.0, 0.4),          # sorted 9 5 | 3 1: (5 - 3) / 5
        ([4.0, 1.0, 3.0, 2.0], 1, 4.0, 3.0, 0.25),
        ([4.0, 1.0, 3.0, 2.0], 3, 2.0, 1.0, 0.5),
        ([2.0, 7.0, 2.0, 1.0], 2, 2.0, 2.0, 0.0),          # exact tie at the boundary
        ([1.0, 2.0, 3.0], 3, 1.0, -inf, inf),             # k = n: nothing left out
        ([-1.0, -4.0, -2.0, -8.0], 2, -2.0, -4.0, 1.0),    # negative K-th value: (-2 - -4) / |-2|
        ([-3.0, -3.5, 10.0], 2, -3.0, -3.5, 0.5 / 3.0),
        ([3.0, 0.0, -1.0], 2, 0.0, -1.0, inf),            # K-th value 0 above the next
        ([0.0, 5.0, 0.0], 2, 0.0, 0.0, 0.0),              # K-th and next both 0
        ([10.0, 9.999, 1.0], 1, 10.0, 9.999, 1e-4),
    ]
    for vals, k, a, b, gap in cases:
        ga, gb, gg = o.boundary_gap(np.asarray(vals), k)
        assert ga == a and gb == b, (vals, k, ga, gb)
        if math.isinf(gap):
            assert math.isinf(gg) and gg > 0, (vals, k, gg)
        else:
            assert math.isclose(gg, gap, rel_tol=1e-9, abs_tol=0.0), (vals, k, gg, gap)
    rng = np.random.default_rng(21)
    for _ in range(80):
        n = int(rng.integers(2, 8))
        vals = [float(x) for x in rng.integers(-4, 5, size=n)]
        k = int(rng.integers(1, n))
        gap = o.boundary_gap(np.asarray(vals), k)[2]
        count = _maximising_k_sets(vals, k)
        assert (count == 1) == (gap > 0), (vals, k, gap, count)


def pin_budget_fused_closed_form(o):
    """The fused-step budget on hand-made step-time tables: the largest K' whose step time is at most the time
    without speculation (a tie with it qualifies), whatever the order of the grid; 0 when every budget lengthens the
    step; the grid's largest K' when speculation never costs more."""
    ks = [0, 32, 64, 128, 192]
    assert o.choose_budget_fused(ks, [20.0, 19.0, 19.5, 20.0, 21.0]) == 128     # 128 ties t(0)
    assert o.choose_budget_fused(ks, [20.0, 19.0, 20.5, 19.9, 24.0]) == 128     # not monotone: 64 fails, 128 fits
    assert o.choose_budget_fused(ks, [20.0, 20.1, 21.0, 22.0, 25.0]) == 0
    assert o.choose_budget_fused(ks, [20.0, 18.0, 17.0, 16.0, 15.0]) == 192
    assert o.choose_budget_fused([64, 0, 128, 32], [19.0, 20.0, 19.5, 25.0]) == 128   # grid in any order


ALL_PINS = [pin_dense_equivalence, pin_brute_force_selection, pin_quest_upper_bound, pin_signsplit,
            pin_merge_order_free, pin_repair_invariants, pin_closed_forms, pin_hand_example, pin_ema_closed_form,
            pin_budget_closed_form, pin_paged_gather, pin_partial_last_block, pin_forced_blocks,
            pin_mean_key_scores, pin_adaptive_budgets, pin_boundary_gap,
            pin_budget_fused_closed_form]
