"""The gap-keeping query draws (tests/gap_search.py) against the generated inputs, and the stored attempt tables
against the search (CPU).

For reduced versions of the five workloads (and ragged, forced-block and mean-key variants), the gap of every
(step, sequence, KV head) is recomputed from the generated cache itself (the oracle's page-table gather, summaries
and plain scores of the stored query, with the generator's own drift applied before each step) and must equal the
search's and exceed 1e-4. The stored full-size tables must load for their workloads, and sampled rows must equal a
fresh search."""
import json
import os

import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS, load_attempts, make_inputs
from oracle import prr_oracle as O
from tests.gap_search import REL_GAP, search, search_row, selection_gap
from tests.gpu_common import small

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gap_attempts")


def _case(name):
    if name == "llama_ragged_forced":
        return small("llama3_8b_32k").replace(ctx=16 * 250 - 5, sink_blocks=1, local_blocks=2, steps=5)
    if name == "paged_mean":
        return small("paged_b32_64k").replace(scorer="mean", steps=4)
    if name == "long_ctx_drift":
        return small("long_ctx_131k_b4").replace(steps=9)
    return small(name).replace(steps=min(small(name).steps, 6))


CASES = ["tiny_f32_4k", "llama3_8b_32k", "long_ctx_drift", "paged_b32_64k", "million_token", "llama_ragged_forced",
         "paged_mean"]


@pytest.mark.parametrize("name", CASES)
def test_gap_holds_on_generated_bytes(name):
    w = _case(name)
    att, gaps = search(w)
    inp = make_inputs(w, attempts=att)
    kc = inp.k_cache.float().numpy()
    G = w.group
    for t in range(w.steps):
        if len(inp.drift(t)):
            kc = inp.k_cache.float().numpy()
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                keys = O.logical_tokens(kc, inp.table_np, b, g, w.ctx)
                qg = inp.q[t, b, g * G:(g + 1) * G].double().numpy()
                if w.scorer == "mean":
                    s = O.mean_key_scores(qg, keys, w.block_size)
                else:
                    kmin, kmax = O.block_summaries(keys, w.block_size)
                    s = O.quest_scores(qg, kmin, kmax)
                gap = selection_gap(w, s)
                assert gap == gaps[t, b, g], (t, b, g, gap, gaps[t, b, g])
                assert gap > REL_GAP, (t, b, g, gap, att[t, b, g])
    # the literal draws (attempt 0 everywhere) leave banded instances on most of these workloads
    print(f"[result] {name}: mean attempt {att.mean():.2f}, max {att.max()}")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_stored_table_matches_a_fresh_search(name):
    path = os.path.join(GOLDEN, f"{name}.json")
    w = WORKLOADS[name]
    att = load_attempts(path, w)
    meta = json.load(open(path))
    assert att.shape == (w.steps, w.batch, w.n_kv_heads)
    assert meta["banded"] == 0, meta["banded"]
    # sampled rows (all of them on the small workloads), over a prefix of the steps, equal a fresh search
    rows = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    rng = np.random.default_rng(0)
    pick = rows if len(rows) <= 8 else [rows[i] for i in rng.choice(len(rows), 2, replace=False)]
    steps = w.steps if name == "tiny_f32_4k" else (5 if name == "long_ctx_131k_b4" else 2)
    if name == "million_token":
        pick = pick[:1]
    for b, g in pick:
        a, gp = search_row(w, b, g, steps)
        assert np.array_equal(a, att[:steps, b, g]), (b, g, a, att[:steps, b, g])
        assert np.all(gp > REL_GAP)
