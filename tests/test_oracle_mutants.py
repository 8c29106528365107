"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant replaces one oracle function with a plausible wrong version (a dropped term, a wrong sign or index, a
transposed operand, a wrong tie rule); the test asserts that running all pins against the mutated oracle raises."""
import math

import numpy as np
import pytest

from oracle import prr_oracle as O
from tests import checker as C
from tests.checker_cases import ALL_CASES
from tests.oracle_pins import ALL_PINS


def _quest_drop_kmin(q_group, kmin, kmax):
    return sum((kmax * q_group[h]).sum(axis=1) for h in range(q_group.shape[0]))


def _quest_min_not_max(q_group, kmin, kmax):
    return sum(np.minimum(kmin * q_group[h], kmax * q_group[h]).sum(axis=1) for h in range(q_group.shape[0]))


def _quest_first_head_only(q_group, kmin, kmax):
    q = q_group[0]
    return np.maximum(kmin * q, kmax * q).sum(axis=1)


def _signsplit_swapped(q_group, kmin, kmax):
    qp = np.maximum(q_group, 0.0).sum(axis=0)
    qn = np.minimum(q_group, 0.0).sum(axis=0)
    return kmin @ qp + kmax @ qn


def _summaries_swapped(keys, bs):
    kb = keys.reshape(-1, bs, keys.shape[1])
    return kb.max(axis=1), kb.min(axis=1)


def _summaries_last_window(keys, bs):
    """Partial last block summarised over the last bs tokens of the sequence (reaching into the previous block)."""
    n_tok = len(keys)
    kmin, kmax = _orig["block_summaries"](keys, bs)
    if n_tok % bs:
        tail = keys[max(0, n_tok - bs):]
        kmin[-1], kmax[-1] = tail.min(axis=0), tail.max(axis=0)
    return kmin, kmax


def _attn_whole_last_block(q_group, keys, values, blocks, block_size, scale):
    """Attention that drops the tokens of a partial last block (only whole blocks attended)."""
    n_whole = len(keys) // block_size
    blocks = [n for n in blocks if n < n_whole] or list(blocks)
    return _orig["attention_over_blocks"](q_group, keys, values, blocks, block_size, scale)


def _topk_ignores_forced(values, k, n_sink=0, n_local=0):
    return _orig["top_k"](values, k)


def _topk_local_off_by_one(values, k, n_sink=0, n_local=0):
    n = len(values)
    idx = np.arange(n)
    forced = (idx < n_sink) | (idx > n - n_local)
    rank_value = np.where(forced, 0.0, -np.asarray(values, dtype=np.float64))
    return np.sort(np.lexsort((idx, rank_value, ~forced))[:k])


def _mean_scores_first_head(q_group, keys, block_size):
    return _orig["mean_key_scores"](q_group[:1], keys, block_size)


def _mean_scores_sum_not_mean(q_group, keys, block_size):
    return _orig["mean_key_scores"](q_group, keys, block_size) * block_size


def _topk_high_ties(values, k):
    n = len(values)
    order = np.lexsort((-np.arange(n), -np.asarray(values, dtype=np.float64)))
    return np.sort(order[:k])


def _topk_off_by_one(values, k):
    n = len(values)
    order = np.lexsort((np.arange(n), -np.asarray(values, dtype=np.float64)))
    return np.sort(order[1:k + 1]) if k < n else np.sort(order[:k])


def _topk_unsorted(values, k):
    n = len(values)
    return np.lexsort((np.arange(n), -np.asarray(values, dtype=np.float64)))[:k]


def _attn_no_scale(q_group, keys, values, blocks, block_size, scale):
    return _orig["attention_over_blocks"](q_group, keys, values, blocks, block_size, 1.0)


def _attn_keys_as_values(q_group, keys, values, blocks, block_size, scale):
    return _orig["attention_over_blocks"](q_group, keys, keys, blocks, block_size, scale)


def _attn_block_index_shift(q_group, keys, values, blocks, block_size, scale):
    idx = np.concatenate([np.arange(n * block_size + 1, (n + 1) * block_size + 1) % len(keys) for n in blocks])
    k, v = keys[idx], values[idx]
    out = np.empty((q_group.shape[0], keys.shape[1]))
    for h in range(q_group.shape[0]):
        z = scale * (k @ q_group[h])
        w = np.exp(z - z.max())
        out[h] = (w @ v) / w.sum()
    return out


def _merge_no_rescale_l(a, b):
    (m1, l1, o1), (m2, l2, o2) = a, b
    m = max(m1, m2)
    c1, c2 = math.exp(m1 - m), math.exp(m2 - m)
    return m, l1 * c1 + l2, o1 * c1 + o2 * c2


def _merge_min(a, b):
    (m1, l1, o1), (m2, l2, o2) = a, b
    m = min(m1, m2)
    c1, c2 = math.exp(m1 - m), math.exp(m2 - m)
    return m, l1 * c1 + l2 * c2, o1 * c1 + o2 * c2


def _partial_unshifted(q_h, k_blk, v_blk, scale):
    z = scale * (k_blk @ q_h)
    p = np.exp(z)
    return float(z.max()), float(p.sum()), p @ v_blk


def _prr_keeps_wasted(q_group, keys, values, true_set, pred_set, block_size, scale):
    allb = sorted(set(int(n) for n in true_set) | set(int(n) for n in pred_set))
    out = _orig["attention_over_blocks"](q_group, keys, values, allb, block_size, scale)
    _, missed, wasted = _orig["prr_output"](q_group, keys, values, true_set, pred_set, block_size, scale)
    return out, missed, wasted


def _prr_skips_repair(q_group, keys, values, true_set, pred_set, block_size, scale):
    hit = [n for n in true_set if n in set(int(p) for p in pred_set)]
    _, missed, wasted = _orig["prr_output"](q_group, keys, values, true_set, pred_set, block_size, scale)
    if not hit:
        hit = list(true_set[:1])
    return _orig["attention_over_blocks"](q_group, keys, values, hit, block_size, scale), missed, wasted


def _ema_swapped(ema_prev, scores, alpha, first):
    return _orig["ema_update"](ema_prev, scores, 1.0 - alpha, first)


def _ema_no_init(ema_prev, scores, alpha, first):
    prev = np.zeros_like(np.asarray(scores, dtype=np.float64)) if first else ema_prev
    return alpha * prev + (1 - alpha) * np.asarray(scores, dtype=np.float64)


def _budget_strict(n_grid, t_sel, kspec_grid, t_spec, n_target, degree=2):
    return _orig["choose_budget"](n_grid, t_sel, kspec_grid, [t * 1.0000001 + 1e-9 for t in t_spec], n_target,
                                  degree) if False else _budget_linear(n_grid, t_sel, kspec_grid, t_spec, n_target)


def _budget_linear(n_grid, t_sel, kspec_grid, t_spec, n_target, degree=2):
    return _orig["choose_budget"](n_grid, t_sel, kspec_grid, t_spec, n_target, 1)


def _budget_smallest(n_grid, t_sel, kspec_grid, t_spec, n_target, degree=2):
    best = _orig["choose_budget"](n_grid, t_sel, kspec_grid, t_spec, n_target, degree)
    ok = [k for k in kspec_grid if 0 < k <= best]
    return min(ok) if ok else 0


def _gather_identity(cache, table, b, g, n_tokens):
    page = cache.shape[2]
    i = np.arange(n_tokens)
    return np.asarray(cache[b * table.shape[1] + i // page, g, i % page], dtype=np.float64)


def _budget_misses_floor(missed_prev, k_top, k_cap, beta, k_min):
    m = np.asarray(missed_prev).astype(np.float32)
    return np.minimum(np.maximum(k_top + np.floor(np.float32(beta) * m).astype(np.int64), k_min), k_cap)


def _budget_misses_fp64(missed_prev, k_top, k_cap, beta, k_min):
    m = np.asarray(missed_prev).astype(np.float64)
    return np.minimum(np.maximum(k_top + np.ceil(beta * m).astype(np.int64), k_min), k_cap)


def _bound_minus(scores, ema, c):
    s = np.asarray(scores, dtype=np.float32)
    e = np.asarray(ema, dtype=np.float32)
    return e - np.float32(c) * np.abs(s - e)


def _confidence_theta_from_u(scores, ema, k_top, k_cap, c, k_min, n_sink=0, n_local=0):
    u = O.confidence_bound(scores, ema, c)
    return _orig["budget_from_confidence"](scores, u, k_top, k_cap, 0.0, k_min, n_sink, n_local)[0], u


def _predict_confident_by_ema(scores, ema, k_top, k_cap, c, k_min, n_sink=0, n_local=0):
    k, _ = O.budget_from_confidence(scores, ema, k_top, k_cap, c, k_min, n_sink, n_local)
    return O.top_k(np.asarray(ema, dtype=np.float32), k, n_sink, n_local)


def _gap_off_by_one(values, k):
    v = np.sort(np.asarray(values, dtype=np.float64))[::-1]
    if k + 1 >= len(v):
        return float(v[-1]), -math.inf, math.inf
    a, b = float(v[k]), float(v[k + 1])
    return a, b, (a - b) / abs(a) if a != 0 else (math.inf if a > b else 0.0)


def _gap_sign(values, k):
    a, b, _ = _orig["boundary_gap"](values, k)
    if math.isinf(b):
        return a, b, math.inf
    return a, b, (b - a) / abs(a) if a != 0 else (math.inf if a > b else 0.0)


def _gap_zero_branch(values, k):
    a, b, g = _orig["boundary_gap"](values, k)
    return a, b, 0.0 if a == 0 else g


def _gap_over_next(values, k):
    a, b, g = _orig["boundary_gap"](values, k)
    if math.isinf(b) or a == 0 or b == 0:
        return a, b, g
    return a, b, (a - b) / abs(b)


def _gap_ascending(values, k):
    v = np.sort(np.asarray(values, dtype=np.float64))
    if k >= len(v):
        return float(v[k - 1]), -math.inf, math.inf
    a, b = float(v[k - 1]), float(v[k])
    return a, b, abs(a - b) / abs(a) if a != 0 else math.inf


def _fused_strict(kspec_grid, t_step):
    ks = list(kspec_grid)
    t0 = t_step[ks.index(0)]
    return max([0] + [k for k, t in zip(ks, t_step) if t < t0])


def _fused_argmin(kspec_grid, t_step):
    return int(list(kspec_grid)[int(np.argmin(t_step))])


def _fused_smallest(kspec_grid, t_step):
    best = _orig["choose_budget_fused"](kspec_grid, t_step)
    ok = [k for k, t in zip(kspec_grid, t_step) if 0 < k and t <= t_step[list(kspec_grid).index(0)]]
    return min(ok) if ok else best


def _fused_first_entry(kspec_grid, t_step):
    """Compares with the grid's first entry instead of the step without speculation."""
    return max([0] + [k for k, t in zip(kspec_grid, t_step) if t <= t_step[0]])


_orig = {k: getattr(O, k) for k in ["attention_over_blocks", "prr_output", "ema_update", "choose_budget",
                                    "block_summaries", "top_k", "mean_key_scores", "budget_from_confidence",
                                    "boundary_gap", "choose_budget_fused"]}

MUTANTS = {
    "quest_drop_kmin": ("quest_scores", _quest_drop_kmin),
    "quest_min_not_max": ("quest_scores", _quest_min_not_max),
    "quest_first_head_only": ("quest_scores", _quest_first_head_only),
    "signsplit_swapped": ("quest_scores_signsplit", _signsplit_swapped),
    "summaries_swapped": ("block_summaries", _summaries_swapped),
    "summaries_last_window": ("block_summaries", _summaries_last_window),
    "attn_drops_partial_block": ("attention_over_blocks", _attn_whole_last_block),
    "topk_high_ties": ("top_k", _topk_high_ties),
    "topk_ignores_forced": ("top_k", _topk_ignores_forced),
    "mean_scores_first_head": ("mean_key_scores", _mean_scores_first_head),
    "mean_scores_sum_not_mean": ("mean_key_scores", _mean_scores_sum_not_mean),
    "topk_local_off_by_one": ("top_k", _topk_local_off_by_one),
    "topk_off_by_one": ("top_k", _topk_off_by_one),
    "topk_unsorted": ("top_k", _topk_unsorted),
    "attn_no_scale": ("attention_over_blocks", _attn_no_scale),
    "attn_keys_as_values": ("attention_over_blocks", _attn_keys_as_values),
    "attn_block_index_shift": ("attention_over_blocks", _attn_block_index_shift),
    "merge_no_rescale_l": ("merge", _merge_no_rescale_l),
    "merge_min": ("merge", _merge_min),
    "partial_unshifted": ("block_partial", _partial_unshifted),
    "prr_keeps_wasted": ("prr_output", _prr_keeps_wasted),
    "prr_skips_repair": ("prr_output", _prr_skips_repair),
    "ema_swapped_alpha": ("ema_update", _ema_swapped),
    "ema_no_init": ("ema_update", _ema_no_init),
    "budget_linear_fit": ("choose_budget", _budget_linear),
    "budget_smallest": ("choose_budget", _budget_smallest),
    "gather_ignores_table": ("logical_tokens", _gather_identity),
    "budget_misses_floor": ("budget_from_misses", _budget_misses_floor),
    "budget_misses_fp64": ("budget_from_misses", _budget_misses_fp64),
    "confidence_bound_minus": ("confidence_bound", _bound_minus),
    "confidence_theta_from_u": ("budget_from_confidence", _confidence_theta_from_u),
    "predict_confident_by_ema": ("predict_confident", _predict_confident_by_ema),
    "gap_off_by_one": ("boundary_gap", _gap_off_by_one),
    "gap_sign": ("boundary_gap", _gap_sign),
    "gap_zero_branch": ("boundary_gap", _gap_zero_branch),
    "gap_over_next": ("boundary_gap", _gap_over_next),
    "gap_ascending": ("boundary_gap", _gap_ascending),
    "fused_strict": ("choose_budget_fused", _fused_strict),
    "fused_argmin": ("choose_budget_fused", _fused_argmin),
    "fused_smallest": ("choose_budget_fused", _fused_smallest),
    "fused_first_entry": ("choose_budget_fused", _fused_first_entry),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            failures += 1
        except Exception:   # a crash inside a pin also counts as caught
            failures += 1
    assert failures > 0, f"mutant {name} passed every pin"


# ---- planted mistakes in the comparison rules (tests/checker.py), caught by tests/checker_cases.py -----------------
_check_selection = C.check_selection
_check_output = C.check_output


def _band(g, s, k, eps):
    mask = np.zeros(len(s), dtype=bool)
    mask[g] = True
    outside = s[~mask].max() if (~mask).any() else -np.inf
    assert s[mask].min() >= outside - eps


def _sel_eps_absolute(gpu_idx, oracle_scores, k, rel=C.REL_GAP, n_sink=0, n_local=0):
    """The band taken as an absolute 1e-4 instead of relative to |s_(K)|."""
    if n_sink or n_local:
        return _check_selection(gpu_idx, oracle_scores, k, rel, n_sink, n_local)
    g, s = np.asarray(gpu_idx), np.asarray(oracle_scores, dtype=np.float64)
    assert g.shape == (k,) and np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < len(s)
    if O.boundary_gap(s, k)[2] > rel:
        assert np.array_equal(g, O.top_k(s, k))
        return True
    _band(g, s, k, rel)
    return False


def _sel_threshold_inverted(gpu_idx, oracle_scores, k, rel=C.REL_GAP, n_sink=0, n_local=0):
    """Exactness demanded where the gap is small (and the band used where it is large)."""
    if n_sink or n_local:
        return _check_selection(gpu_idx, oracle_scores, k, rel, n_sink, n_local)
    g, s = np.asarray(gpu_idx), np.asarray(oracle_scores, dtype=np.float64)
    assert g.shape == (k,) and np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < len(s)
    if O.boundary_gap(s, k)[2] <= rel:
        assert np.array_equal(g, O.top_k(s, k))
        return True
    _band(g, s, k, rel * abs(O.boundary_gap(s, k)[0]))
    return False


def _sel_band_wrong_side(gpu_idx, oracle_scores, k, rel=C.REL_GAP, n_sink=0, n_local=0):
    """The band added on the wrong side (inside minimum >= outside maximum + eps)."""
    if n_sink or n_local:
        return _check_selection(gpu_idx, oracle_scores, k, rel, n_sink, n_local)
    g, s = np.asarray(gpu_idx), np.asarray(oracle_scores, dtype=np.float64)
    assert g.shape == (k,) and np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < len(s)
    if O.boundary_gap(s, k)[2] > rel:
        assert np.array_equal(g, O.top_k(s, k))
        return True
    _band(g, s, k, -rel * abs(O.boundary_gap(s, k)[0]))
    return False


def _sel_no_order_check(gpu_idx, oracle_scores, k, rel=C.REL_GAP, n_sink=0, n_local=0):
    """Ids compared as a set: an unsorted or repeated list passes."""
    g = np.unique(np.asarray(gpu_idx))
    if len(g) != k:
        g = np.sort(np.asarray(gpu_idx))
        return True
    return _check_selection(g, oracle_scores, k, rel, n_sink, n_local)


def _sel_forced_last(gpu_idx, oracle_scores, k, rel=C.REL_GAP, n_sink=0, n_local=0):
    """K below the number of forced blocks compared with the last K of them."""
    n = len(oracle_scores)
    f_idx = [i for i in range(n) if i < n_sink or i >= n - n_local]
    if (n_sink or n_local) and k <= len(f_idx):
        assert np.array_equal(np.asarray(gpu_idx), np.asarray(f_idx[-k:]))
        return True
    return _check_selection(gpu_idx, oracle_scores, k, rel, n_sink, n_local)


def _out_mean_abs(got, ref, dtype):
    err = float(np.mean(np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))))
    assert not np.isnan(err) and err <= C.TOL[dtype]
    return err


def _out_bf16_tol(got, ref, dtype):
    return _check_output(got, ref, "bf16")


CHECKER_MUTANTS = {
    "sel_eps_absolute": ("check_selection", _sel_eps_absolute),
    "sel_threshold_inverted": ("check_selection", _sel_threshold_inverted),
    "sel_band_wrong_side": ("check_selection", _sel_band_wrong_side),
    "sel_no_order_check": ("check_selection", _sel_no_order_check),
    "sel_forced_last": ("check_selection", _sel_forced_last),
    "out_mean_abs": ("check_output", _out_mean_abs),
    "out_bf16_tolerance_for_f32": ("check_output", _out_bf16_tol),
}


@pytest.mark.parametrize("name", sorted(CHECKER_MUTANTS))
def test_checker_mutant_is_caught(name, monkeypatch):
    attr, fn = CHECKER_MUTANTS[name]
    monkeypatch.setattr(C, attr, fn)
    failures = 0
    for case in ALL_CASES:
        try:
            case(C)
        except Exception:   # AssertionError or a crash inside a case
            failures += 1
    assert failures > 0, f"checker mutant {name} passed every case"
