"""Per-row budgets of the predicted set (prr_budget: the misses rule and the confidence rule) against the oracle.

The budgets are integer decisions taken in fp32 from fp32 inputs, so the device must match the oracle exactly once
both start from the same fp32 values: the tests hand the oracle the device's own EMA (itself checked against the
oracle's update within fp32 rounding) and the scores the device read. Each row's set is its first k_r entries
(ascending block ids) followed by -1 up to the capacity; speculation skips the -1 slots and repair never matches
them, so the step's output stays the oracle's attention over the true set."""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd import _lib as L
from dynamic_sparse_attention_decode_amd.runtime import PRRLayer
from oracle import prr_oracle as O
from tests.checker import TOL, check_selection, max_abs
from tests.gpu_common import (OracleView, gap_inputs, np64, oracle_scores, requires_gpu, shape_of, small,
                              wide_paged)

pytestmark = [pytest.mark.gpu, requires_gpu]

POLICIES = {"misses": L.BUDGET_MISSES, "confidence": L.BUDGET_CONFIDENCE}


def _expected_row(policy, s_row, e_row, m, K, cap, k_min, beta, c, sink, local):
    """The oracle's predicted set of one row (ascending ids, then -1 up to cap)."""
    if policy == "misses":
        k = int(O.budget_from_misses([m], K, cap, beta, k_min)[0])
        ids = O.top_k(e_row.astype(np.float64), k, sink, local)
    else:
        ids = O.predict_confident(s_row, e_row, K, cap, c, k_min, sink, local)
    out = np.full(cap, -1, dtype=np.int64)
    out[:len(ids)] = ids
    return out


def _rows(rng, rows, N, kind):
    if kind == "normal":
        s = rng.standard_normal((rows, N)) * 3 + 20
        e = s + rng.standard_normal((rows, N)) * 2
    else:   # many equal values: ties resolved by index on both sides
        s = np.round(rng.standard_normal((rows, N)) * 2)
        e = np.round(s + rng.standard_normal((rows, N)))
    return s.astype(np.float32), e.astype(np.float32)


@pytest.mark.parametrize("policy", ["misses", "confidence"])
@pytest.mark.parametrize("n_blocks", [129, 2048, 4096, 6000, 20001])
def test_ema_predict_budget(policy, n_blocks):
    """prr_ema_predict with a budget: the EMA update, each row's size and set (forced blocks included) against the
    oracle, for row lengths across the workgroup shapes (512 threads up to 4096 blocks, 1024 beyond), random and
    tie-heavy values, first and later steps."""
    rng = np.random.default_rng(n_blocks)
    rows, N = 6, n_blocks
    K = min(N, 40)
    cap = min(N, 90)
    for kind in ("normal", "ties"):
        for first in (False, True):
            for (sink, local) in ((0, 0), (1, 3)):
                print(f"[case] ema_predict budget {policy} N={N} {kind} first={first} sink={sink} local={local}",
                      flush=True)
                s = L.make_shape(1, 4 * rows, rows, 128, 16, 16, N, L.BF16, sink_blocks=sink, local_blocks=local)
                s32, e32 = _rows(rng, rows, N, kind)
                m = rng.integers(0, K + 1, size=rows).astype(np.int32)
                k_min = int(rng.integers(1, K + 1))
                beta, c = 0.7, 0.4
                scores = torch.as_tensor(s32[None], device="cuda").contiguous()
                ema = torch.as_tensor(e32[None], device="cuda").contiguous()
                missed = torch.as_tensor(m[None], device="cuda").contiguous()
                pred = torch.full((1, rows, cap), -7, dtype=torch.int32, device="cuda")
                bud = L.make_budget(POLICIES[policy], K, k_min, beta, c, missed)
                L.ema_predict(s, scores, ema, 0.8, first, cap, pred, budget=bud)
                torch.cuda.synchronize()
                e_gpu = ema.cpu().numpy()[0]
                ref_e = np.stack([O.ema_update(e32[r], s32[r], 0.8, first) for r in range(rows)])
                assert np.allclose(e_gpu, ref_e, rtol=1e-6, atol=1e-5)
                got = pred.cpu().numpy()[0]
                for r in range(rows):
                    ref = _expected_row(policy, s32[r], e_gpu[r], int(m[r]), K, cap, k_min, beta, c, sink, local)
                    assert np.array_equal(got[r], ref), (r, got[r][:12], ref[:12])


@pytest.mark.parametrize("forced", [(0, 0), (2, 3)])
@pytest.mark.parametrize("with_ws", [True, False])
@pytest.mark.parametrize("policy", ["misses", "confidence"])
@pytest.mark.parametrize("n_blocks", [2048, 20001])
def test_select_speculate_budget(policy, n_blocks, with_ws, forced):
    """prr_select_speculate with a budget: T as without one; P_{t+1} from the already updated EMA by the budget
    (in the selection launch up to 8192 blocks; beyond, by segments whose candidates the merge launch budgets when a
    workspace is given, else in a launch of its own), forced blocks included; speculation over a padded P_t writes
    the records of its filled slots as prr_speculate does and leaves the -1 slots untouched."""
    rng = np.random.default_rng(7 + n_blocks)
    N = n_blocks
    sink, local = forced
    s = L.make_shape(1, 32, 8, 128, 16, 16, N, L.BF16, sink_blocks=sink, local_blocks=local)
    rows, K, cap = 8, 30, 45
    inp_k = torch.randn((N, 8, 16, 128), device="cuda").to(torch.bfloat16)
    inp_v = torch.randn((N, 8, 16, 128), device="cuda").to(torch.bfloat16)
    table = torch.arange(N, dtype=torch.int32, device="cuda")[None].contiguous()
    q = torch.randn((1, 32, 128), device="cuda").to(torch.bfloat16)
    s32, e32 = _rows(rng, rows, N, "normal")
    scores = torch.as_tensor(s32[None], device="cuda").contiguous()
    ema = torch.as_tensor(e32[None], device="cuda").contiguous()
    m = rng.integers(0, K + 1, size=rows).astype(np.int32)
    missed = torch.as_tensor(m[None], device="cuda").contiguous()
    # P_t: filled prefixes of various lengths, then -1
    p_cur = np.full((rows, cap), -1, dtype=np.int32)
    for r in range(rows):
        n_fill = int(rng.integers(0, cap + 1))
        p_cur[r, :n_fill] = np.sort(rng.choice(N, size=n_fill, replace=False))
    pred_cur = torch.as_tensor(p_cur[None], device="cuda").contiguous()
    pb = L.partials_bytes(s, cap) // 4
    part = torch.full((pb,), 12345.0, dtype=torch.float32, device="cuda")
    part_ref = torch.full((pb,), 12345.0, dtype=torch.float32, device="cuda")
    sel = torch.zeros((1, rows, K), dtype=torch.int32, device="cuda")
    pred_next = torch.full((1, rows, cap), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros((L.workspace_bytes(s, K) // 4 + 1,), dtype=torch.float32, device="cuda")
    bud = L.make_budget(POLICIES[policy], K, 5, 0.7, 0.4, missed)
    print(f"[case] select_speculate budget {policy} N={N} workspace={with_ws} sink={sink} local={local}", flush=True)
    L.select_speculate(s, scores, K, sel, ema, cap, pred_next, q, inp_k, inp_v, table, pred_cur, cap, part,
                       workspace=ws if with_ws else None, budget=bud)
    L.speculate(s, q, inp_k, inp_v, table, pred_cur, cap, part_ref)
    torch.cuda.synchronize()
    got_sel = sel.cpu().numpy()[0]
    for r in range(rows):
        assert np.array_equal(got_sel[r], O.top_k(s32[r].astype(np.float64), K, sink, local))
    got_p = pred_next.cpu().numpy()[0]
    for r in range(rows):
        ref = _expected_row(policy, s32[r], e32[r], int(m[r]), K, cap, 5, 0.7, 0.4, sink, local)
        assert np.array_equal(got_p[r], ref), (r, got_p[r][:12], ref[:12])
    # the records (m[G], l[G] fp32 padded to 4 floats, then O / l [G][D] in fp16; G = 4, D = 128): equal to the
    # standalone speculation's where filled (O / l within one fp16 rounding); untouched where empty
    words = (8 * 4 + 4 * 128 * 2) // 4
    a = part.cpu().numpy().view(np.uint32)[:rows * cap * words].reshape(rows, cap, words)
    b = part_ref.cpu().numpy().view(np.uint32)[:rows * cap * words].reshape(rows, cap, words)
    filled = p_cur >= 0
    ml_a, ml_b = a[filled][:, :8].view(np.float32), b[filled][:, :8].view(np.float32)
    assert np.allclose(ml_a, ml_b, rtol=1e-6, atol=1e-6)
    o_a = a[filled][:, 8:].copy().view(np.float16).astype(np.float64)
    o_b = b[filled][:, 8:].copy().view(np.float16).astype(np.float64)
    assert np.all(np.abs(o_a - o_b) <= 2.0 ** -10 * np.abs(o_b) + 1e-7)
    fill = np.float32(12345.0).view(np.uint32)
    assert np.all(a[~filled] == fill) and np.all(b[~filled] == fill)


@pytest.mark.parametrize("mode", ["prr_fused", "prr_1stream", "prr_2stream"])
@pytest.mark.parametrize("policy", ["misses", "confidence"])
@pytest.mark.parametrize("name", ["tiny_f32_4k", "llama3_8b_32k", "paged_b32_64k", "million_token", "paged_wide",
                                  "paged_512"])
def test_decode_with_budget(name, policy, mode):
    """Whole decode runs with a budget: every step's selection and output against the oracle (the output is
    attention over the true set whatever was predicted), the missed count = |T minus the filled part of P_t|, and
    P_{t+1} equal to the oracle's budgeted prediction from the step's scores and EMA and the previous step's missed
    counts; the sets' sizes vary by row within [k_min, k_spec]."""
    if name == "paged_wide":   # 136 rows: the fused step's many-row path
        w = wide_paged()
    elif name == "paged_512":   # 512 rows, K = 64: one repair workgroup per row, with -1-padded predicted sets
        w = wide_paged(batch=64, top_k=64, ctx=16 * 100 - 3, k_spec=(96,))
    else:
        w = small(name)
    kp = min(w.n_blocks, max(max(w.k_spec), w.top_k + w.top_k // 2))   # room above K for the sizes to vary
    k_min = max(1, w.top_k // 2)
    cfg = {"policy": policy, "k_min": k_min, "beta": 0.5, "c": 0.3}
    print(f"[case] decode budget {name} {policy} {mode} K'={kp}", flush=True)
    inp = gap_inputs(w)
    ov = OracleView(inp)
    layer = PRRLayer(shape_of(w), w.top_k, kp, w.alpha, mode=mode, budget=cfg)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    G = w.group
    prev_missed = np.zeros((w.batch, w.n_kv_heads), dtype=np.int64)
    pred_t = None
    sizes = []
    for t in range(w.steps):
        ids = inp.drift(t)
        if len(ids):
            layer.rebuild_blocks(torch.as_tensor(ids, device="cuda"))
            ov.invalidate_keys()
        out = layer.step(inp.q[t].contiguous())
        layer.sync_spec()
        torch.cuda.synchronize()
        out_h, sel = np64(out), layer.sel_idx.cpu().numpy()
        nm = layer.n_missed.cpu().numpy()
        s_gpu = layer.scores_last.cpu().numpy()
        e_gpu = layer.ema.cpu().numpy()
        p_next = layer.pred_next.cpu().numpy()
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                qg = ov.q_group(t, b, g)
                keys = ov.keys(b, g)
                assert check_selection(sel[b, g], oracle_scores(w, qg, keys), w.top_k, n_sink=w.sink_blocks,
                                       n_local=w.local_blocks), (t, b, g)
                ref = O.attention_over_blocks(qg, keys, ov.values(b, g), sel[b, g], w.block_size, w.scale)
                assert max_abs(out_h[b, g * G:(g + 1) * G], ref) <= TOL[w.dtype], (t, b, g)
                if pred_t is None:
                    assert nm[b, g] == w.top_k
                else:
                    filled = pred_t[b, g][pred_t[b, g] >= 0]
                    assert nm[b, g] == len(set(sel[b, g]) - set(filled))
                exp = _expected_row(policy, s_gpu[b, g], e_gpu[b, g], int(prev_missed[b, g]), w.top_k, kp, k_min,
                                    0.5, 0.3, w.sink_blocks, w.local_blocks)
                assert np.array_equal(p_next[b, g], exp), (t, b, g, p_next[b, g][:10], exp[:10])
                sizes.append(int((p_next[b, g] >= 0).sum()))
        prev_missed = nm.astype(np.int64)
        pred_t = p_next.copy()
    layer.close()
    assert min(sizes) >= min(k_min, kp) and max(sizes) <= kp
    print(f"[result] {name} {policy} {mode}: predicted-set sizes {min(sizes)}..{max(sizes)} "
          f"(mean {np.mean(sizes):.1f}, cap {kp})")


@pytest.mark.parametrize("rows,mode,policy", [("short", "prr_fused", "misses"), ("short", "prr_fused", "confidence"),
                                              ("short", "prr_2stream", "misses"),
                                              ("long", "prr_fused", "confidence"), ("long", "prr_fused", "misses")])
def test_budget_graph_replay_matches_eager(rows, mode, policy):
    """Budgeted steps captured in a HIP graph and replayed several times (eager work and synchronisation between the
    replays) give the same outputs, selections, missed counts and predicted sets as the same steps run eagerly: the
    budgets read their missed counts through device pointers, so a captured graph keeps adapting. Long rows (12000
    blocks) select and predict by segments through the workspace's three candidate regions."""
    if rows == "short":
        w = small("llama3_8b_32k")
    else:
        w = small("million_token").replace(ctx=32 * 12000 - 7, top_k=61, k_spec=(93,), steps=6)
    kp = min(w.n_blocks, max(max(w.k_spec), w.top_k + w.top_k // 2))
    cfg = {"policy": policy, "k_min": max(1, w.top_k // 2), "beta": 0.5, "c": 0.3}
    print(f"[case] budget graph replay {rows} rows N={w.n_blocks} {mode} {policy}", flush=True)
    inp = gap_inputs(w)
    qs = [inp.q[t].contiguous() for t in range(w.steps)]
    seq = [0] + [1, 2, 3, 4] * 3
    eager = PRRLayer(shape_of(w), w.top_k, kp, w.alpha, mode=mode, budget=cfg)
    eager.build(inp.k_cache, inp.v_cache, inp.table)
    ref = []
    for t in seq:
        out = eager.step(qs[t])
        eager.sync_spec()
        torch.cuda.synchronize()
        ref.append((np64(out), eager.sel_idx.cpu().numpy().copy(), eager.n_missed.cpu().numpy().copy(),
                    eager.pred_next.cpu().numpy().copy()))
    eager.close()
    lay = PRRLayer(shape_of(w), w.top_k, kp, w.alpha, mode=mode, budget=cfg)
    lay.build(inp.k_cache, inp.v_cache, inp.table)
    lay.step(qs[0])
    lay.sync_spec()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=lay.s_sel):
        outs = [lay.enqueue(qs[t], join=(t == 4)) for t in (1, 2, 3, 4)]
    sizes = set()
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 16, device="cuda").sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        base = 1 + 4 * r
        for i in (2, 3):   # the two output buffers hold the last two steps of the replay
            assert np.array_equal(np64(outs[i]), ref[base + i][0]), (r, i)
        assert np.array_equal(lay.sel_idx.cpu().numpy(), ref[base + 3][1])
        assert np.array_equal(lay.n_missed.cpu().numpy(), ref[base + 3][2])
        p = lay.pred_next.cpu().numpy()
        assert np.array_equal(p, ref[base + 3][3])
        sizes.update((p >= 0).sum(-1).ravel().tolist())
        del scratch
    lay.close()
    print(f"[result] predicted-set sizes seen after replays: {sorted(sizes)}")


@pytest.mark.parametrize("policy", ["misses", "confidence"])
def test_budget_edge_parameters(policy):
    """Budget parameters at their edges, against the oracle: a cap below K (every row at the cap), k_min equal to the
    cap, beta = 0 and c = 0 (the plain top-K of the EMA, with ties), a huge beta or c (every row at the cap), missed
    counts of 0 and above K, K = 1 and K = N."""
    rng = np.random.default_rng(77)
    rows, N = 5, 700
    s32, e32 = _rows(rng, rows, N, "ties")
    cases = [(40, 30, 1, 0.5, 0.5), (40, 90, 90, 0.5, 0.5), (40, 90, 1, 0.0, 0.0), (40, 90, 1, 1e30, 1e30),
             (1, 90, 1, 2.0, 1.0), (N, N, 1, 1.0, 1.0), (40, N, 40, 3.0, 0.25)]
    for (K, cap, k_min, beta, c) in cases:
        print(f"[case] budget edges {policy} K={K} cap={cap} k_min={k_min} beta={beta} c={c}", flush=True)
        s = L.make_shape(1, 4 * rows, rows, 128, 16, 16, N, L.BF16)
        m = np.array([0, K, 3 * K + 5, 1, 2], dtype=np.int32)
        scores = torch.as_tensor(s32[None], device="cuda").contiguous()
        ema = torch.as_tensor(e32[None], device="cuda").contiguous()
        missed = torch.as_tensor(m[None], device="cuda").contiguous()
        pred = torch.full((1, rows, cap), -7, dtype=torch.int32, device="cuda")
        bud = L.make_budget(POLICIES[policy], K, k_min, beta, c, missed)
        L.ema_predict(s, scores, ema, 0.5, False, cap, pred, budget=bud)
        torch.cuda.synchronize()
        e_gpu = ema.cpu().numpy()[0]
        got = pred.cpu().numpy()[0]
        for r in range(rows):
            ref = _expected_row(policy, s32[r], e_gpu[r], int(m[r]), K, cap, k_min, beta, c, 0, 0)
            assert np.array_equal(got[r], ref), (K, cap, r, got[r][:12], ref[:12])


@pytest.mark.parametrize("name", ["llama3_8b_32k", "million_token"])
def test_budget_chooser_on_profiled_tables(name):
    """The profiling-guided budget on tables measured here (PRR abstract; PRR summary page, Limitations): the
    library's two choosers give the oracle's K'* on the same measured tables (the two-stream rule with its off-grid
    polynomial fit, and the fused step's rule), and the fused K'* is a budget whose measured step is no slower than
    the step without speculation while every larger grid budget is slower."""
    from dynamic_sparse_attention_decode_amd import profiling as P
    w = small(name)
    print(f"[case] budget profile {name} N={w.n_blocks} K={w.top_k}", flush=True)
    inp = gap_inputs(w)
    s = shape_of(w)
    qs = [inp.q[t].contiguous() for t in range(w.steps)]
    k_grid = P.default_k_grid(w.top_k, w.n_blocks, w.k_spec)
    two = P.two_stream_tables(s, w.top_k, qs[1], inp.k_cache, inp.v_cache, inp.table, k_grid=k_grid, reps=20,
                              seed=w.seed)
    fused = P.fused_step_table(s, w.top_k, w.alpha, [(inp.k_cache, inp.v_cache)], inp.table, qs, k_grid, steps=8,
                               warmup=3)
    print(f"[result] {name}: t_sel {np.round(two['t_sel_us'], 2)} t_spec {np.round(two['t_spec_us'], 2)} "
          f"t_step {np.round(fused['t_step_us'], 2)} K'* two-stream {two['kspec_star']} fused {fused['kspec_star']}")
    assert all(t > 0 for t in two["t_sel_us"]) and all(t > 0 for t in fused["t_step_us"])
    ref = O.choose_budget(two["n_grid"], two["t_sel_us"], k_grid, two["t_spec_us"], float(w.n_blocks), 2)
    if two["kspec_star"] != ref:   # only a near-tie between the fitted selection time and a table entry may differ
        tt = np.polyval(np.polyfit(two["n_grid"], two["t_sel_us"], 2), w.n_blocks)
        k = max(two["kspec_star"], ref)
        assert abs(two["t_spec_us"][k_grid.index(k)] - tt) < 1e-9 * max(1.0, abs(tt)), (two["kspec_star"], ref)
    assert fused["kspec_star"] == O.choose_budget_fused(k_grid, fused["t_step_us"])
    t0 = fused["t_step_us"][k_grid.index(0)]
    ks = fused["kspec_star"]
    assert fused["t_step_us"][k_grid.index(ks)] <= t0
    assert all(t > t0 for k, t in zip(k_grid, fused["t_step_us"]) if k > ks)
