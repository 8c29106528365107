"""Cases the comparison rules of tests/checker.py must meet, written from the rules' statement, not from the code.

Each case takes a namespace ``c`` with ``check_selection`` and ``check_output`` and raises AssertionError when the
rules misbehave; tests/test_checker.py runs them on the real checker and tests/test_oracle_mutants.py shows that
planted mistakes in the checker fail at least one of them.

The rules: a GPU selection of K distinct ascending ids is valid when its smallest oracle score is at least the
largest excluded score minus 1e-4 * |s_(K)|; where the relative gap at the boundary exceeds 1e-4 that is the oracle's
set alone. Forced blocks must all be in the set (or, for K below their number, the set is the first K of them).
Outputs must lie within the dtype's max-abs tolerance (1e-5 fp32, 2e-2 bf16 and fp16) element by element.
"""
from __future__ import annotations

from itertools import combinations

import numpy as np

from oracle import prr_oracle as O


def _rejects(fn, *args, **kw) -> bool:
    try:
        fn(*args, **kw)
    except AssertionError:
        return True
    return False


def case_accepts_oracle(c):
    """The oracle's own selection is always accepted: random scores, integer ties, every K, forced blocks."""
    rng = np.random.default_rng(31)
    for trial in range(40):
        n = int(rng.integers(2, 40))
        s = rng.standard_normal(n) * 100.0
        if trial % 4 == 0:
            s = np.round(s / 50.0)          # exact ties
        for k in range(1, n + 1):
            sink = int(rng.integers(0, 3)) if trial % 3 == 0 else 0
            local = int(rng.integers(0, 3)) if trial % 3 == 0 else 0
            if sink + local > n:
                sink = local = 0
            c.check_selection(O.top_k(s, k, sink, local), s, k, n_sink=sink, n_local=local)


def case_exact_where_gap_large(c):
    """Where the relative gap exceeds 1e-4 every one-block swap across the boundary is rejected, however close."""
    s = np.array([10.0, 9.0, 8.0, 7.0, 6.0])
    assert c.check_selection(np.array([0, 1]), s, 2) is True
    assert _rejects(c.check_selection, np.array([0, 2]), s, 2)
    # gap 1.5e-4: the swapped set would be within 1.5e-4 relative, still not allowed
    s = np.array([1000.0, 999.85, 5.0, 1.0])
    assert _rejects(c.check_selection, np.array([1, 2]), s, 1) and _rejects(c.check_selection, np.array([1]), s, 1)
    rng = np.random.default_rng(32)
    for _ in range(30):
        n = int(rng.integers(3, 30))
        s = rng.standard_normal(n) * 50.0 + 200.0
        k = int(rng.integers(1, n))
        if O.boundary_gap(s, k)[2] <= 1e-4:
            continue
        T = O.top_k(s, k)
        out = np.setdiff1d(np.arange(n), T)
        for i in T:
            for j in out:
                swapped = np.sort(np.concatenate([T[T != i], [j]]))
                assert _rejects(c.check_selection, swapped, s, k), (s, k, i, j)


def case_band_where_gap_small(c):
    """Where the gap is at most 1e-4 the band applies: a swap within 1e-4 * |s_(K)| is accepted, one beyond it is
    not; the band is relative to |s_(K)|, also for negative scores."""
    s = np.array([1000.0, 999.95, 999.93, 999.0, 1.0])        # gap (999.95 - 999.93) / 999.95 = 2e-5
    assert c.check_selection(np.array([0, 1]), s, 2) is False  # banded: exactness not required
    assert c.check_selection(np.array([0, 2]), s, 2) is False  # within 0.1 of the largest excluded
    assert _rejects(c.check_selection, np.array([0, 3]), s, 2)  # 999.0 is 0.95 below: outside the band
    assert _rejects(c.check_selection, np.array([0, 4]), s, 2)
    s = -np.array([999.0, 999.93, 999.95, 1000.5])            # negative: top-2 {0, 1}, band 1e-4 * 999.93
    assert c.check_selection(np.array([0, 2]), s, 2) is False
    assert _rejects(c.check_selection, np.array([0, 3]), s, 2)  # -1000.5 is 0.57 below -999.93
    s = np.array([5.0, 3.0, 3.0, 1.0])                          # an exact tie: either tied block is valid
    assert c.check_selection(np.array([0, 1]), s, 2) is False and c.check_selection(np.array([0, 2]), s, 2) is False
    # the rule over all K-sets of a small banded vector: accepted exactly when the band condition holds
    s = np.array([100.0, 99.995, 99.994, 99.0, 98.0])
    for k in (2, 3):
        eps = 1e-4 * abs(np.sort(s)[::-1][k - 1])
        for cset in combinations(range(len(s)), k):
            g = np.array(cset)
            inside = s[g].min()
            outside = np.delete(s, g).max()
            ok = inside >= outside - eps
            assert (not _rejects(c.check_selection, g, s, k)) == ok, (k, cset)


def case_rejects_malformed(c):
    """Wrong length, unsorted, repeated or out-of-range ids are rejected."""
    s = np.array([4.0, 3.0, 2.0, 1.0])
    assert _rejects(c.check_selection, np.array([0]), s, 2)
    assert _rejects(c.check_selection, np.array([1, 0]), s, 2)
    assert _rejects(c.check_selection, np.array([0, 0]), s, 2)
    assert _rejects(c.check_selection, np.array([0, 4]), s, 2)
    assert _rejects(c.check_selection, np.array([-1, 0]), s, 2)


def case_forced_blocks(c):
    """Forced blocks: each must be in the set, whatever its score; K below their number takes the first K of them
    by index; the rest of the set is judged among the unforced blocks."""
    s = np.array([0.0, 50.0, 40.0, 30.0, 20.0, -5.0])          # block 0 a sink, block 5 in the local window
    assert c.check_selection(np.array([0, 1, 5]), s, 3, n_sink=1, n_local=1)
    assert _rejects(c.check_selection, np.array([0, 1, 2]), s, 3, n_sink=1, n_local=1)   # local block missing
    assert _rejects(c.check_selection, np.array([0, 2, 5]), s, 3, n_sink=1, n_local=1)   # 2 instead of 1
    assert c.check_selection(np.array([0, 1, 2, 5]), s, 4, n_sink=1, n_local=1)
    s = np.array([9.0, 8.0, 7.0, 100.0, 100.0])                 # three sinks, K = 2: the first two of them
    assert c.check_selection(np.array([0, 1]), s, 2, n_sink=3)
    assert _rejects(c.check_selection, np.array([1, 2]), s, 2, n_sink=3)
    assert _rejects(c.check_selection, np.array([3, 4]), s, 2, n_sink=3)


def case_output_tolerance(c):
    """+2e-5 on one fp32 element is rejected and +5e-6 accepted; bf16 allows 2e-2 but not 3e-2; NaN is rejected."""
    ref = np.random.default_rng(33).standard_normal((4, 8, 64))
    got = ref.copy()
    got[2, 5, 17] += 2e-5
    assert _rejects(c.check_output, got, ref, "f32")
    got = ref.copy()
    got[1, 0, 3] -= 5e-6
    c.check_output(got, ref, "f32")
    got = ref.copy()
    got[3, 7, 63] += 1.5e-2
    c.check_output(got, ref, "bf16")
    got[3, 7, 63] += 1.5e-2
    assert _rejects(c.check_output, got, ref, "bf16")
    got = ref.copy()
    got[0, 0, 0] = np.nan
    assert _rejects(c.check_output, got, ref, "f32")


ALL_CASES = [case_accepts_oracle, case_exact_where_gap_large, case_band_where_gap_small, case_rejects_malformed,
             case_forced_blocks, case_output_tolerance]
