"""Parity at the full workload sizes, in the launch configuration the benchmark times (fused single-stream PRR step
with the workload's largest speculation budget): a few decode steps through libprr, and for sampled (sequence, KV
head) rows the fp64 oracle recomputes that row alone (summaries, scores, selection, attention over the selected
blocks, EMA and the predicted set) and the GPU's row is checked against it with the same rules as the reduced tests.

Every other row of the same steps is checked through properties that hold at any size, evaluated on the device in
fp32 with plain tensor operations (no part of the HIP path): the scores equal the Quest bound of the block's key
minima and maxima (the group's heads summed, within fp32 rounding of its magnitude), the selected set is exactly the
top-K of the device's own scores under the tie rule (lower index first), the output is softmax attention over the
selected blocks (to the dtype's tolerance), the EMA follows its recurrence, the next predicted set is exactly the
top-K' of that EMA, and the missed count is |T minus P|.
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


def _topk_mask(v: torch.Tensor, k: int) -> torch.Tensor:
    """Mask of the k largest values along the last axis, equal values to the lower index (the selection's rule)."""
    vk = v.sort(dim=-1, descending=True).values[..., k - 1:k]
    gt, eq = v > vk, v == vk
    need = k - gt.sum(-1, keepdim=True)
    return gt | (eq & (eq.cumsum(-1) <= need))


def _set_mask(idx: torch.Tensor, n: int) -> torch.Tensor:
    """Mask of a row-wise index list after checking that every list is strictly ascending and within [0, n)."""
    assert bool((idx >= 0).all()) and bool((idx < n).all()), "index out of range"
    if idx.shape[-1] > 1:
        assert bool((idx[..., 1:] > idx[..., :-1]).all()), "indices not strictly ascending"
    m = torch.zeros(idx.shape[:-1] + (n,), dtype=torch.bool, device=idx.device)
    return m.scatter_(-1, idx.long(), True)


def _check_all_rows(w, inp, layer, t, out, ema_prev, pred_t):
    """The properties above on every (sequence, KV head) row of step t. ema_prev: the EMA before the step (None at
    the first step); pred_t: the predicted set the step used (None when nothing was predicted)."""
    B, Hkv, G, D, N, bs, page = w.batch, w.n_kv_heads, w.group, w.head_dim, w.n_blocks, w.block_size, w.page_size
    assert w.ctx == N * bs and bs % page == 0 and not (w.sink_blocks or w.local_blocks) and w.scorer == "quest"
    ppb = bs // page
    tab = inp.table.long()                                                      # [B, pages per sequence]
    # block key minima / maxima through the page table: per page, then over a block's pages
    pmin, pmax = inp.k_cache.amin(2), inp.k_cache.amax(2)                       # [pages, Hkv, D]
    kmin = pmin[tab].view(B, N, ppb, Hkv, D).amin(2).permute(0, 2, 1, 3).float()   # [B, Hkv, N, D]
    kmax = pmax[tab].view(B, N, ppb, Hkv, D).amax(2).permute(0, 2, 1, 3).float()
    q = inp.q[t].float().view(B, Hkv, G, D)
    qp, qn = q.clamp(min=0).sum(2), q.clamp(max=0).sum(2)                       # [B, Hkv, D]
    # sum over heads of max(q kmin, q kmax) = kmax . sum max(q, 0) + kmin . sum min(q, 0), since kmin <= kmax
    s_ref = (kmax * qp[:, :, None]).sum(-1) + (kmin * qn[:, :, None]).sum(-1)
    mag = (kmax.abs() * qp[:, :, None]).sum(-1) - (kmin.abs() * qn[:, :, None]).sum(-1)
    s_dev = layer.scores_last
    err = ((s_dev - s_ref).abs() / (mag + 1e-30)).max().item()
    assert err <= 1e-5, f"scores: worst error {err:.3e} of the bound's magnitude"
    # T is the top-K of the device's scores, ties to the lower index
    sel = layer.sel_idx
    sel_mask = _set_mask(sel, N)
    assert torch.equal(sel_mask, _topk_mask(s_dev, w.top_k)), "selection is not the top-K of the scores"
    # the output is softmax attention over the selected blocks' tokens
    j = torch.arange(ppb, device=sel.device)
    cols = (sel.long()[..., None] * ppb + j).reshape(B, Hkv * w.top_k * ppb)
    pids = tab.gather(1, cols).view(B, Hkv, w.top_k * ppb)
    heads = torch.arange(Hkv, device=sel.device)[None, :, None].expand_as(pids)
    ks = inp.k_cache[pids, heads].reshape(B, Hkv, w.top_k * bs, D).float()
    vs = inp.v_cache[pids, heads].reshape(B, Hkv, w.top_k * bs, D).float()
    p = torch.softmax(torch.matmul(q, ks.transpose(-1, -2).contiguous()) * w.scale, dim=-1)
    ref = torch.matmul(p, vs).reshape(B, Hkv * G, D)
    e_out = (out - ref).abs().max().item()
    assert e_out <= TOL[w.dtype], f"output: worst error {e_out:.3e}"
    # missed counts
    nm = layer.n_missed.long()
    if pred_t is None:
        assert bool((nm == w.top_k).all())
    else:
        pm = _set_mask(pred_t, N)
        assert torch.equal(nm, (sel_mask & ~pm).sum(-1)), "missed count is not |T minus P|"
    # the EMA recurrence and the next predicted set
    if layer.k_spec > 0:
        ema = layer.ema
        if ema_prev is None:
            assert torch.equal(ema, s_dev), "first-step EMA differs from the scores"
        else:
            a = w.alpha
            e_ref = a * ema_prev + (1.0 - a) * s_dev
            bound = 1e-6 * (a * ema_prev.abs() + (1.0 - a) * s_dev.abs()) + 1e-30
            assert bool(((ema - e_ref).abs() <= bound).all()), "EMA does not follow its recurrence"
        assert torch.equal(_set_mask(layer.pred_next, N), _topk_mask(ema, layer.k_spec)), \
            "next predicted set is not the top-K' of the EMA"
    return err, e_out


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
    ema_dev = None
    for t in range(STEPS):
        ids = inp.drift(t)
        if len(ids):
            layer.rebuild_blocks(torch.as_tensor(ids, device="cuda"))
            ov.invalidate_keys()
        out = layer.step(inp.q[t].contiguous())
        torch.cuda.synchronize()
        kp = layer.k_spec
        e_s, e_o = _check_all_rows(w, inp, layer, t, out, ema_dev, layer.pred_current if t > 0 and kp > 0 else None)
        print(f"[rows] step {t}: all {w.batch * w.n_kv_heads} rows hold; scores {e_s:.1e} of magnitude, "
              f"output {e_o:.1e}", flush=True)
        ema_dev = layer.ema.clone() if kp > 0 else None
        out_h, sel, nm = np64(out), layer.sel_idx.cpu().numpy(), layer.n_missed.cpu().numpy()
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
