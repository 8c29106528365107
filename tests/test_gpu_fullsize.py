"""Parity at the full workload sizes, in the launch configuration the benchmark times (fused single-stream PRR step
with the workload's largest speculation budget): a few decode steps through libprr, and for sampled (sequence, KV
head) rows the fp64 oracle recomputes that row alone (summaries, scores, selection, attention over the selected
blocks, EMA and the predicted set) and the GPU's row is checked against it with the same rules as the reduced tests.
"""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS
from dynamic_sparse_attention_decode_amd.runtime import PRRLayer
from oracle import prr_oracle as O
from tests.checker import TOL, check_selection, max_abs
from tests.gpu_common import OracleView, gap_inputs, np64, requires_gpu, shape_of

pytestmark = [pytest.mark.gpu, requires_gpu]

STEPS = 3


# every workload in the benchmark's mode and in the serialized step; the million-token row (32768 blocks, selected
# by segments) in the two-stream step too
CASES = ([(n, "prr_fused") for n in WORKLOADS] + [(n, "serialized") for n in WORKLOADS]
         + [("million_token", "prr_2stream")])


@pytest.mark.parametrize("name,mode", CASES)
def test_full_size_sampled_rows(name, mode):
    w = WORKLOADS[name]
    k_spec = max(w.k_spec)
    rng = np.random.default_rng(5)
    rows = sorted({(0, 0), (w.batch - 1, w.n_kv_heads - 1),
                   (int(rng.integers(w.batch)), int(rng.integers(w.n_kv_heads)))})
    print(f"[case] full-size {name} {mode} K={w.top_k} K'={k_spec} rows {rows}", flush=True)
    inp = gap_inputs(w, steps=STEPS)
    ov = OracleView(inp)
    layer = PRRLayer(shape_of(w), w.top_k, k_spec, w.alpha, mode=mode)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    ema = {}
    G = w.group
    worst = 0.0
    for t in range(STEPS):
        ids = inp.drift(t)
        if len(ids):
            layer.rebuild_blocks(torch.as_tensor(ids, device="cuda"))
            ov.invalidate_keys()
        out = layer.step(inp.q[t].contiguous())
        torch.cuda.synchronize()
        out_h, sel, nm = np64(out), layer.sel_idx.cpu().numpy(), layer.n_missed.cpu().numpy()
        kp = layer.k_spec
        pred = layer.pred_current.cpu().numpy() if t > 0 and kp > 0 else None
        for (b, g) in rows:
            qg = ov.q_group(t, b, g)
            keys = ov.keys(b, g)
            kmin, kmax = O.block_summaries(keys, w.block_size)
            s = O.quest_scores_signsplit(qg, kmin, kmax)
            # the stored draws keep the relative gap above 1e-4 on every row and step: exact equality is required
            assert check_selection(sel[b, g], s, w.top_k), (t, b, g)
            ref = O.attention_over_blocks(qg, keys, ov.values(b, g), sel[b, g], w.block_size, w.scale)
            e = max_abs(out_h[b, g * G:(g + 1) * G], ref)
            worst = max(worst, e)
            assert e <= TOL[w.dtype], (t, b, g, e)
            if pred is not None:
                check_selection(pred[b, g], ema[(b, g)], kp)
                assert nm[b, g] == len(set(sel[b, g]) - set(pred[b, g])), (t, b, g)
            else:
                assert nm[b, g] == w.top_k
            ema[(b, g)] = O.ema_update(ema.get((b, g)), s, w.alpha, t == 0)
    layer.close()
    print(f"[result] full-size {name}: worst output error {worst:.3e}", flush=True)


@pytest.mark.parametrize("name,policy", [("million_token", "misses"), ("million_token", "confidence"),
                                         ("llama3_8b_32k", "confidence")])
def test_full_size_budget_sampled_rows(name, policy):
    """A per-row budget at full size in the benchmark's step (the million-token rows predict by segments through the
    workspace's candidate regions): sampled rows' outputs against the oracle, missed counts against the filled part
    of the predicted set, and each sampled row's next predicted set equal to the oracle's budgeted prediction from
    the device's scores and EMA and the row's previous missed count."""
    w = WORKLOADS[name]
    k_spec = max(w.k_spec)
    cfg = {"policy": policy, "k_min": w.top_k, "beta": 1.0, "c": 0.5}
    rng = np.random.default_rng(6)
    rows = sorted({(0, 0), (w.batch - 1, w.n_kv_heads - 1),
                   (int(rng.integers(w.batch)), int(rng.integers(w.n_kv_heads)))})
    print(f"[case] full-size budget {name} {policy} K={w.top_k} K'={k_spec} rows {rows}", flush=True)
    inp = gap_inputs(w, steps=STEPS)
    ov = OracleView(inp)
    layer = PRRLayer(shape_of(w), w.top_k, k_spec, w.alpha, mode="prr_fused", budget=cfg)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    G = w.group
    prev_nm = np.zeros((w.batch, w.n_kv_heads), dtype=np.int64)
    pred_t = None
    for t in range(STEPS):
        out = layer.step(inp.q[t].contiguous())
        torch.cuda.synchronize()
        out_h, sel, nm = np64(out), layer.sel_idx.cpu().numpy(), layer.n_missed.cpu().numpy()
        s_gpu, e_gpu, p_next = (layer.scores_last.cpu().numpy(), layer.ema.cpu().numpy(),
                                layer.pred_next.cpu().numpy())
        for (b, g) in rows:
            qg = ov.q_group(t, b, g)
            keys = ov.keys(b, g)
            kmin, kmax = O.block_summaries(keys, w.block_size)
            assert check_selection(sel[b, g], O.quest_scores_signsplit(qg, kmin, kmax), w.top_k), (t, b, g)
            ref = O.attention_over_blocks(qg, keys, ov.values(b, g), sel[b, g], w.block_size, w.scale)
            assert max_abs(out_h[b, g * G:(g + 1) * G], ref) <= TOL[w.dtype], (t, b, g)
            filled = pred_t[b, g][pred_t[b, g] >= 0] if pred_t is not None else np.zeros(0, dtype=np.int64)
            assert nm[b, g] == (len(set(sel[b, g]) - set(filled)) if pred_t is not None else w.top_k)
            if policy == "misses":
                k = int(O.budget_from_misses([prev_nm[b, g]], w.top_k, k_spec, 1.0, w.top_k)[0])
                ids = O.top_k(e_gpu[b, g].astype(np.float64), k)
            else:
                ids = O.predict_confident(s_gpu[b, g], e_gpu[b, g], w.top_k, k_spec, 0.5, w.top_k)
            exp = np.full(k_spec, -1, dtype=np.int64)
            exp[:len(ids)] = ids
            assert np.array_equal(p_next[b, g], exp), (t, b, g)
        prev_nm = nm.astype(np.int64)
        pred_t = p_next.copy()
    layer.close()
