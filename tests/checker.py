"""Comparison rules between the HIP path and the fp64 oracle.

Selection (several answers can be correct at near-ties): a GPU set T_g of K distinct ascending ids is valid when its
smallest oracle score is at least the largest excluded oracle score minus eps = rel * |s_(K)|. Where the oracle's
relative gap at the K-th/(K+1)-th boundary exceeds rel, the only valid set is the oracle's own, so validity is then
bit-exact equality. The GPU computes scores in fp32 (relative error ~1e-6), far inside rel = 1e-4.

Outputs are compared with the oracle's attention over the GPU's own (validated) set, element by element, with the
stated max-abs tolerance: 1e-5 for fp32 storage, 2e-2 for bf16/fp16 storage.
"""
from __future__ import annotations

import numpy as np

from oracle import prr_oracle as O

REL_GAP = 1e-4
TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}


def check_selection(gpu_idx, oracle_scores, k: int, rel: float = REL_GAP, n_sink: int = 0, n_local: int = 0):
    """Returns whether exact equality was required. Raises AssertionError if the GPU set is invalid. Forced blocks
    (the first n_sink and last n_local) must all be in the set (or, when k is smaller, the set is the first k of
    them); the rest of the set is judged among the other blocks by the rule above."""
    g = np.asarray(gpu_idx, dtype=np.int64)
    s = np.asarray(oracle_scores, dtype=np.float64)
    assert g.shape == (k,), g.shape
    assert np.all(np.diff(g) > 0), "indices not strictly ascending"
    assert g.min() >= 0 and g.max() < len(s), "index out of range"
    if n_sink or n_local:
        n = len(s)
        forced = np.array([i < n_sink or i >= n - n_local for i in range(n)])
        f_idx = np.flatnonzero(forced)
        if k <= len(f_idx):
            assert np.array_equal(g, f_idx[:k]), (g, f_idx[:k])
            return True
        assert set(f_idx) <= set(g.tolist()), "a forced block is missing"
        rest = np.flatnonzero(~forced)
        pos = {int(b): i for i, b in enumerate(rest)}
        g_rest = np.asarray([pos[int(b)] for b in g if not forced[b]], dtype=np.int64)
        return check_selection(g_rest, s[rest], k - len(f_idx), rel)
    ref = O.top_k(s, k)
    _, _, gap = O.boundary_gap(s, k)
    if gap > rel:
        assert np.array_equal(g, ref), f"selection differs where the gap {gap:.3e} > {rel}: {set(g) ^ set(ref)}"
        return True
    eps = rel * abs(O.boundary_gap(s, k)[0])
    mask = np.zeros(len(s), dtype=bool)
    mask[g] = True
    inside_min = s[mask].min()
    outside_max = s[~mask].max() if (~mask).any() else -np.inf
    assert inside_min >= outside_max - eps, (inside_min, outside_max, eps)
    return False


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def check_output(got, ref, dtype: str) -> float:
    """Element-by-element comparison of an output with the oracle's: raises AssertionError when any element differs
    by more than the storage dtype's max-abs tolerance. Returns the largest difference."""
    a = np.asarray(got, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite output"
    err = max_abs(a, b)
    assert err <= TOL[dtype], f"max |gpu - oracle| = {err:.3e} > {TOL[dtype]:.0e} ({dtype})"
    return err
