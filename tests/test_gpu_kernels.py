"""Kernel-by-kernel parity of the HIP path (through the C ABI) against the fp64 oracle, on reduced workloads.

Every call goes through libprr's C entry points; nothing here computes the method on the device with torch."""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd import _lib as L
from oracle import prr_oracle as O
from tests.checker import TOL, check_selection, max_abs
from tests.gpu_common import SMALL, OracleView, gap_inputs, np64, ragged, requires_gpu, shape_of, small

pytestmark = [pytest.mark.gpu, requires_gpu]


def _setup(name, seed_shift=0):
    if name == "paged_wide":   # a wide batch of short rows
        w = small("paged_b32_64k")
        w = w.replace(batch=17, ctx=w.block_size * 70, top_k=12, k_spec=(12,), steps=4)
    elif name == "paged_many":   # 512 rows: the spread-out repair takes 8 entries of T per wave (a ragged last one)
        w = small("paged_b32_64k")
        w = w.replace(batch=64, ctx=w.block_size * 160, top_k=61, k_spec=(61,), steps=4)
    else:
        w = small(name)
    if seed_shift:
        w = w.replace(seed=w.seed + seed_shift)
    print(f"[case] {name} B={w.batch} N={w.n_blocks} K={w.top_k} K'={w.k_spec}", flush=True)
    inp = gap_inputs(w)
    s = shape_of(w)
    summ = torch.zeros((w.batch, w.n_kv_heads, w.n_blocks, 2, w.head_dim), dtype=w.torch_dtype, device="cuda")
    L.build_summaries(s, inp.k_cache, inp.table, summ)
    torch.cuda.synchronize()
    return w, inp, s, summ, OracleView(inp)


@pytest.mark.parametrize("name", SMALL)
def test_summaries_exact(name):
    w, inp, s, summ, ov = _setup(name)
    got = np64(summ)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            kmin, kmax = O.block_summaries(ov.keys(b, g), w.block_size)
            assert np.array_equal(got[b, g, :, 0], kmin), (b, g)
            assert np.array_equal(got[b, g, :, 1], kmax), (b, g)


def test_summaries_block_ids_after_drift():
    w, inp, s, summ, ov = _setup("long_ctx_131k_b4")
    changed = inp.drift(4)
    assert len(changed)
    ids = torch.as_tensor(changed, device="cuda")
    L.build_summaries(s, inp.k_cache, inp.table, summ, block_ids=ids)
    full = torch.zeros_like(summ)
    L.build_summaries(s, inp.k_cache, inp.table, full)
    torch.cuda.synchronize()
    assert torch.equal(summ.view(torch.int16), full.view(torch.int16))


@pytest.mark.parametrize("name", SMALL)
def test_score_select(name):
    w, inp, s, summ, ov = _setup(name)
    B, Hkv, N, K = w.batch, w.n_kv_heads, w.n_blocks, w.top_k
    scores = torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda")
    sel = torch.full((B, Hkv, K), -1, dtype=torch.int32, device="cuda")
    exact = banded = 0
    for t in range(min(w.steps, 4)):
        L.score_select(s, inp.q[t].contiguous(), summ, K, scores, sel)
        torch.cuda.synchronize()
        gs, gi = np64(scores), sel.cpu().numpy()
        for b in range(B):
            for g in range(Hkv):
                kmin, kmax = O.block_summaries(ov.keys(b, g), w.block_size)
                ref = O.quest_scores(ov.q_group(t, b, g), kmin, kmax)
                err = np.max(np.abs(gs[b, g] - ref)) / max(1.0, np.max(np.abs(ref)))
                assert err < 2e-6, (t, b, g, err)
                if check_selection(gi[b, g], ref, K):
                    exact += 1
                else:
                    banded += 1
    print(f"[result] {name}: exact {exact} banded {banded}")
    assert banded == 0   # the inputs keep the relative gap above 1e-4 at every step


@pytest.mark.parametrize("name", ["llama3_8b_32k", "million_token", "tiny_f32_4k"])
def test_topk_ties_and_extremes(name):
    """Exact ties, constant rows, K = 1, K = N, negative values: the selection equals the oracle's tie rule."""
    w, inp, s, summ, ov = _setup(name)
    B, Hkv, N = w.batch, w.n_kv_heads, w.n_blocks
    rng = np.random.default_rng(3)
    cases = [
        np.round(rng.standard_normal((B, Hkv, N)) * 2),          # many exact ties
        np.zeros((B, Hkv, N)),                                   # all equal
        -np.abs(rng.standard_normal((B, Hkv, N))) * 1e3,         # negative
        rng.standard_normal((B, Hkv, N)) * 1e-30,                # tiny
    ]
    ema = torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda")
    for vals in cases:
        v32 = vals.astype(np.float32)
        for k in sorted({1, 2, 7, N // 3, N - 1, N}):
            out = torch.full((B, Hkv, k), -1, dtype=torch.int32, device="cuda")
            L.ema_predict(s, torch.as_tensor(v32, device="cuda"), ema, 0.5, True, k, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for b in range(B):
                for g in range(Hkv):
                    ref = O.top_k(v32[b, g].astype(np.float64), k)
                    assert np.array_equal(got[b, g], ref), (k, b, g)
            assert np.array_equal(ema.cpu().numpy(), v32)       # first step: ema = scores


def test_ema_update_matches_oracle():
    w, inp, s, summ, ov = _setup("llama3_8b_32k")
    B, Hkv, N, Kp = w.batch, w.n_kv_heads, w.n_blocks, w.k_spec[0]
    rng = np.random.default_rng(4)
    ema = torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda")
    pred = torch.zeros((B, Hkv, Kp), dtype=torch.int32, device="cuda")
    e_ref = None
    for t in range(6):
        sc = (rng.standard_normal((B, Hkv, N)) * 50 + 500).astype(np.float32)
        L.ema_predict(s, torch.as_tensor(sc, device="cuda"), ema, w.alpha, t == 0, Kp, pred)
        torch.cuda.synchronize()
        e_ref = O.ema_update(e_ref, sc.astype(np.float64), w.alpha, t == 0)
        got = np64(ema)
        assert np.max(np.abs(got - e_ref) / np.abs(e_ref)) < 1e-6
        for b in range(B):
            for g in range(Hkv):
                check_selection(pred.cpu().numpy()[b, g], e_ref[b, g], Kp)


def _records(part, w, k_spec):
    """(m, l, O) of every speculation record: m and l fp32; O in fp32 for fp32 storage; for 16-bit storage the
    record holds O / l in fp16, so O = that times l."""
    G, D = w.group, w.head_dim
    ml = (2 * G + 3) // 4 * 4
    ob = 4 if w.dtype == "f32" else 2
    rb = ml * 4 + G * D * ob
    raw = part.cpu().numpy().view(np.uint8)[:w.batch * w.n_kv_heads * k_spec * rb]
    raw = raw.reshape(w.batch, w.n_kv_heads, k_spec, rb)
    mlv = raw[..., :ml * 4].copy().view(np.float32).astype(np.float64)
    m, l = mlv[..., :G], mlv[..., G:2 * G]
    if ob == 4:
        o = raw[..., ml * 4:].copy().view(np.float32).astype(np.float64).reshape(w.batch, w.n_kv_heads, k_spec, G, D)
    else:
        o = raw[..., ml * 4:].copy().view(np.float16).astype(np.float64).reshape(w.batch, w.n_kv_heads, k_spec, G, D)
        o = o * l[..., None]
    return m, l, o


@pytest.mark.parametrize("name", SMALL)
def test_speculate_partials(name):
    w, inp, s, summ, ov = _setup(name)
    B, Hkv, N = w.batch, w.n_kv_heads, w.n_blocks
    Kp = max(w.k_spec)
    rng = np.random.default_rng(7)
    pred_np = np.stack([np.stack([np.sort(rng.choice(N, Kp, replace=False)) for _ in range(Hkv)])
                        for _ in range(B)]).astype(np.int32)
    pred = torch.as_tensor(pred_np, device="cuda")
    part = torch.zeros((L.partials_bytes(s, Kp) // 4,), dtype=torch.float32, device="cuda")
    t = 1
    L.speculate(s, inp.q[t].contiguous(), inp.k_cache, inp.v_cache, inp.table, pred, Kp, part)
    torch.cuda.synchronize()
    m, l, o = _records(part, w, Kp)
    bs = w.block_size
    worst = 0.0
    for b in range(B):
        for g in range(Hkv):
            qg = ov.q_group(t, b, g)
            k, v = ov.keys(b, g), ov.values(b, g)
            for j in range(0, Kp, max(1, Kp // 7)):
                n = pred_np[b, g, j]
                for h in range(w.group):
                    rm, rl, ro = O.block_partial(qg[h], k[n * bs:(n + 1) * bs], v[n * bs:(n + 1) * bs], w.scale)
                    assert abs(m[b, g, j, h] * np.log(2.0) - rm) < 1e-5 * max(1, abs(rm))
                    assert abs(l[b, g, j, h] - rl) < 1e-5 * rl
                    e = max_abs(o[b, g, j, h] / l[b, g, j, h], ro / rl)
                    # 16-bit storage keeps O / l in fp16: each element rounded to nearest (2^-11 relative)
                    tol = 1e-5 if w.dtype == "f32" else 1e-5 + 2.0 ** -11 * np.abs(ro).max() / rl
                    assert e <= tol, (b, g, j, h, e, tol)
                    worst = max(worst, e)
    print(f"[result] {name}: worst partial O/l error {worst:.3e}")


def _forced_sets(rng, T, N, Kp_list):
    T = list(T)
    outside = [n for n in range(N) if n not in set(T)]
    sets = {"empty": [], "equal": T, "random": sorted(rng.choice(N, min(N, len(T) + 5), replace=False).tolist()),
            "disjoint": sorted(rng.choice(outside, min(len(outside), len(T)), replace=False).tolist()),
            "superset": sorted(set(T) | set(rng.choice(outside, 7, replace=False).tolist())),
            "half": sorted(T[::2] + rng.choice(outside, 3, replace=False).tolist()),
            "unsorted": list(rng.permutation(T[::2] + rng.choice(outside, 3, replace=False).tolist()))}
    return sets


@pytest.mark.parametrize("name", SMALL + ["paged_wide", "paged_many"])
def test_repair_merge_forced_predictions(name):
    """Whatever the predicted set (empty, equal, random, disjoint, superset, partial, unsorted), the repaired output
    equals attention over the true set and the missed count is |T \\ P| (PRR summary page, Key findings); also on a
    wide batch of 17 sequences (136 rows) with short rows, and on 512 rows, where each repair wave takes several
    entries of the true set."""
    w, inp, s, summ, ov = _setup(name)
    B, Hkv, N, K, G = w.batch, w.n_kv_heads, w.n_blocks, w.top_k, w.group
    t = 2
    q = inp.q[t].contiguous()
    scores = torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda")
    sel = torch.zeros((B, Hkv, K), dtype=torch.int32, device="cuda")
    L.score_select(s, q, summ, K, scores, sel)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    rng = np.random.default_rng(9)
    ref = {}
    for b in range(B):
        for g in range(Hkv):
            ref[(b, g)] = O.attention_over_blocks(ov.q_group(t, b, g), ov.keys(b, g), ov.values(b, g),
                                                  sel_np[b, g], w.block_size, w.scale)
    ws = torch.zeros((L.workspace_bytes(s, K) // 4 + 1,), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    nm = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    kinds = list(_forced_sets(rng, sel_np[0, 0], N, None))
    worst = 0.0
    for kind in kinds:
        sets = [[_forced_sets(np.random.default_rng(100 * b + g), sel_np[b, g], N, None)[kind] for g in range(Hkv)]
                for b in range(B)]
        kp = max(1, max(len(x) for row in sets for x in row))
        if kind == "empty":
            kp = 0
        # pad each list to kp entries with blocks outside T (extra wrongly predicted blocks)
        pred_np = np.zeros((B, Hkv, max(kp, 1)), dtype=np.int32)
        for b in range(B):
            for g in range(Hkv):
                p = list(sets[b][g])
                pool = [n for n in range(N) if n not in set(p) and n not in set(sel_np[b, g])]
                while len(p) < kp:
                    p.append(pool.pop())
                pred_np[b, g, :kp] = p if kind == "unsorted" else np.sort(p)
        pred = torch.as_tensor(pred_np, device="cuda")
        part = torch.zeros((max(L.partials_bytes(s, kp), 16) // 4,), dtype=torch.float32, device="cuda")
        L.speculate(s, q, inp.k_cache, inp.v_cache, inp.table, pred, kp, part)
        L.repair_merge(s, q, inp.k_cache, inp.v_cache, inp.table, sel, K, pred if kp else None, kp,
                       part if kp else None, out, nm, ws)
        torch.cuda.synchronize()
        # the same repair inside the selection launch (two-launch step)
        out2 = torch.zeros_like(out)
        nm2 = torch.full_like(nm, -1)
        sel2 = torch.zeros_like(sel)
        L.select_repair(s, scores, K, sel2, q, inp.k_cache, inp.v_cache, inp.table, out2, nm2, ws,
                        pred_idx=pred if kp else None, k_spec=kp, partials=part if kp else None)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel2)
        for got, nmn in ((np64(out), nm.cpu().numpy()), (np64(out2), nm2.cpu().numpy())):
            for b in range(B):
                for g in range(Hkv):
                    e = max_abs(got[b, g * G:(g + 1) * G], ref[(b, g)])
                    worst = max(worst, e)
                    assert e <= TOL[w.dtype], (kind, b, g, e)
                    missed = len(set(sel_np[b, g]) - set(pred_np[b, g, :kp]))
                    assert nmn[b, g] == missed, (kind, b, g, nmn[b, g], missed)
    print(f"[result] {name}: worst forced-P output error {worst:.3e}")


@pytest.mark.parametrize("name", ["llama3_8b_32k", "paged_wide"])
def test_repair_empty_slot_inside_prediction(name):
    """A predicted set with an empty (-1) slot before valid ids: ids after the first empty slot are never matched
    (speculation may have skipped them), so their blocks of T are repaired. The output is attention over T and the
    missed count is |T minus the ids before the empty slot|, in the spread-out and the row-wise repair alike."""
    w, inp, s, summ, ov = _setup(name)
    B, Hkv, N, K, G = w.batch, w.n_kv_heads, w.n_blocks, w.top_k, w.group
    t = 1
    q = inp.q[t].contiguous()
    scores = torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda")
    sel = torch.zeros((B, Hkv, K), dtype=torch.int32, device="cuda")
    L.score_select(s, q, summ, K, scores, sel)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    cut = K // 2
    pred_np = np.sort(sel_np, axis=-1).astype(np.int32)
    pred_np[:, :, cut] = -1                      # T with one empty slot in the middle: the ids after it are in T too
    pred = torch.as_tensor(pred_np, device="cuda")
    part = torch.zeros((L.partials_bytes(s, K) // 4,), dtype=torch.float32, device="cuda")
    L.speculate(s, q, inp.k_cache, inp.v_cache, inp.table, pred, K, part)
    ws = torch.zeros((L.workspace_bytes(s, K) // 4 + 1,), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    nm = torch.full((B, Hkv), -1, dtype=torch.int32, device="cuda")
    L.repair_merge(s, q, inp.k_cache, inp.v_cache, inp.table, sel, K, pred, K, part, out, nm, ws)
    out2 = torch.zeros_like(out)
    nm2 = torch.full_like(nm, -1)
    sel2 = torch.zeros_like(sel)
    L.select_repair(s, scores, K, sel2, q, inp.k_cache, inp.v_cache, inp.table, out2, nm2, ws, pred_idx=pred,
                    k_spec=K, partials=part)
    torch.cuda.synchronize()
    for got, nmn in ((np64(out), nm.cpu().numpy()), (np64(out2), nm2.cpu().numpy())):
        for b in range(B):
            for g in range(Hkv):
                ref = O.attention_over_blocks(ov.q_group(t, b, g), ov.keys(b, g), ov.values(b, g), sel_np[b, g],
                                              w.block_size, w.scale)
                e = max_abs(got[b, g * G:(g + 1) * G], ref)
                assert e <= TOL[w.dtype], (b, g, e)
                assert nmn[b, g] == K - cut, (b, g, nmn[b, g], K - cut)


def test_poison_block_excluded():
    """A predicted block outside the true set whose keys align with the queries (logits far above every selected
    token) must not leak into the output."""
    w, inp, s, summ, ov = _setup("llama3_8b_32k")
    B, Hkv, N, K, G = w.batch, w.n_kv_heads, w.n_blocks, w.top_k, w.group
    t = 1
    q = inp.q[t].contiguous()
    scores = torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda")
    sel = torch.zeros((B, Hkv, K), dtype=torch.int32, device="cuda")
    L.score_select(s, q, summ, K, scores, sel)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    pred_np = np.zeros((B, Hkv, K + 1), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            outside = [n for n in range(N) if n not in set(sel_np[b, g])]
            pois = outside[len(outside) // 2]
            qs = ov.q_group(t, b, g).sum(axis=0)
            keys = torch.as_tensor(np.tile(40.0 * qs / np.linalg.norm(qs), (w.block_size, 1)), dtype=torch.float32)
            inp.set_block_keys(b, g, pois, keys.cuda())
            pred_np[b, g] = np.sort(np.append(sel_np[b, g], pois))
    ov.invalidate_keys()
    pred = torch.as_tensor(pred_np, device="cuda")
    part = torch.zeros((L.partials_bytes(s, K + 1) // 4,), dtype=torch.float32, device="cuda")
    ws = torch.zeros((L.workspace_bytes(s, K) // 4 + 1,), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    nm = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    L.speculate(s, q, inp.k_cache, inp.v_cache, inp.table, pred, K + 1, part)
    L.repair_merge(s, q, inp.k_cache, inp.v_cache, inp.table, sel, K, pred, K + 1, part, out, nm, ws)
    torch.cuda.synchronize()
    got = np64(out)
    for b in range(B):
        for g in range(Hkv):
            ref = O.attention_over_blocks(ov.q_group(t, b, g), ov.keys(b, g), ov.values(b, g), sel_np[b, g],
                                          w.block_size, w.scale)
            assert max_abs(got[b, g * G:(g + 1) * G], ref) <= TOL[w.dtype]
    assert int(nm.sum()) == 0


@pytest.mark.parametrize("n_blocks", [32768, 5000, 4096, 3000, 2048, 1000, 129])
def test_topk_large_rows(n_blocks):
    """Rows up to 32768 values (the largest row the top-K kernels take), across the workgroup shapes (512 threads
    with 1 to 8 values each up to 4096 values, 1024 threads beyond, full and ragged): random values, massive ties,
    constant rows, a few distinct levels, and rows whose evenly spaced entries hold the extremes. For every K the
    selection equals the oracle's tie rule (lowest index first among equal values, ascending output)."""
    s = L.make_shape(1, 16, 2, 128, 16, 16, n_blocks, L.BF16)
    N, rows = n_blocks, 2
    rng = np.random.default_rng(21)
    stride = max(1, N // 1024)
    cases = {
        "normal": rng.standard_normal((rows, N)),
        "constant": np.full((rows, N), 3.5),
        "few_levels": rng.integers(0, 3, size=(rows, N)).astype(np.float64),
        "rounded": np.round(rng.standard_normal((rows, N)) * 4),
    }
    hi = rng.standard_normal((rows, N))
    hi[:, ::stride] = 100.0 + rng.random((rows, len(range(0, N, stride))))
    cases["strided_high"] = hi
    lo = rng.standard_normal((rows, N)) + 50.0
    lo[:, ::stride] = -100.0
    cases["strided_low"] = lo
    ema = torch.zeros((1, rows, N), dtype=torch.float32, device="cuda")
    for name, vals in cases.items():
        v32 = vals.astype(np.float32)
        for k in sorted({k for k in (1, 64, 256, 2000, N) if k <= N}):
            out = torch.full((1, rows, k), -1, dtype=torch.int32, device="cuda")
            L.ema_predict(s, torch.as_tensor(v32[None], device="cuda").contiguous(), ema, 0.5, True, k, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()[0]
            for r in range(rows):
                ref = O.top_k(v32[r].astype(np.float64), k)
                assert np.array_equal(got[r], ref), (name, k, r)


def _tie_cases(rng, rows, N):
    stride = max(1, N // 1024)
    cases = {
        "normal": rng.standard_normal((rows, N)),
        "constant": np.full((rows, N), 3.5),
        "few_levels": rng.integers(0, 3, size=(rows, N)).astype(np.float64),
        "rounded": np.round(rng.standard_normal((rows, N)) * 4),
        "signed_zeros": np.where(rng.random((rows, N)) < 0.5, -0.0, 0.0),
    }
    hi = rng.standard_normal((rows, N))
    hi[:, ::stride] = 100.0 + rng.random((rows, len(range(0, N, stride))))
    cases["strided_high"] = hi
    # the largest values all in the last (short) segment, then all in the first
    tail = rng.standard_normal((rows, N))
    tail[:, -min(N, 3000):] += 50.0
    cases["tail_high"] = tail
    cases["head_high"] = tail[:, ::-1].copy()
    return cases


def _ref_top_k(v32, k):
    """The oracle's selection over the fp32 values (larger value first, then lower index; -0.0 equals +0.0)."""
    return O.top_k(v32.astype(np.float64), k).astype(np.int32)


@pytest.mark.parametrize("n_blocks", [8193, 20001, 32768])
def test_topk_split_rows(n_blocks):
    """Long rows with a workspace: prr_ema_predict and prr_score_select's top-K run by segments of 4096 values and a
    merge. The selection equals the tie rule on every case (ties, constant rows, signed zeros, the largest values in
    the short last segment or in the first), for K up to the largest split size and beyond it (one workgroup per
    row), and equals the call without a workspace; the EMA written is the same bits."""
    s = L.make_shape(1, 16, 2, 128, 16, 16, n_blocks, L.BF16)
    N, rows = n_blocks, 2
    print(f"[case] split top-K N={N}", flush=True)
    rng = np.random.default_rng(23)
    ws = torch.zeros((L.workspace_bytes(s, 64) // 4 + 1,), dtype=torch.float32, device="cuda")
    for name, vals in _tie_cases(rng, rows, N).items():
        v32 = vals.astype(np.float32)
        vd = torch.as_tensor(v32[None], device="cuda").contiguous()
        for k in sorted({1, 64, 256, 1000, 2048, min(N, 3000)}):
            out_a = torch.full((1, rows, k), -1, dtype=torch.int32, device="cuda")
            out_b = torch.full((1, rows, k), -1, dtype=torch.int32, device="cuda")
            em_a = torch.as_tensor(np.float32(0.25) * v32[None], device="cuda").contiguous()
            em_b = em_a.clone()
            L.ema_predict(s, vd, em_a, 0.5, False, k, out_a, workspace=ws)
            L.ema_predict(s, vd, em_b, 0.5, False, k, out_b)
            torch.cuda.synchronize()
            assert torch.equal(em_a.view(torch.int32), em_b.view(torch.int32)), (name, k)
            assert torch.equal(out_a, out_b), (name, k)
            e32 = em_a.cpu().numpy()[0]
            got = out_a.cpu().numpy()[0]
            for r in range(rows):
                assert np.array_equal(got[r], _ref_top_k(e32[r], k)), (name, k, r)
            if name == "rounded":
                # first step: ema = values, so the selection is the values' own top-K
                L.ema_predict(s, vd, em_a, 0.5, True, k, out_a, workspace=ws)
                torch.cuda.synchronize()
                for r in range(rows):
                    assert np.array_equal(out_a.cpu().numpy()[0][r], O.top_k(v32[r].astype(np.float64), k)), (k, r)


@pytest.mark.parametrize("n_blocks", [20001, 32768])
def test_select_speculate_split_rows(n_blocks):
    """prr_select_speculate on long rows with a workspace (selection by segments of 2048 values inside the
    speculation launch, then the merge launch) writes the same true set, predicted set and partial records, bit for
    bit, as without it, and the sets follow the tie rule, for K and K' on both sides of the segments' candidate
    count."""
    s = L.make_shape(1, 8, 2, 128, 16, 16, n_blocks, L.BF16)
    N, B, Hkv, bs = n_blocks, 1, 2, 16
    print(f"[case] split select_speculate N={N}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(31)
    n_pages = N + 17
    kc = torch.randn((n_pages, Hkv, bs, 128), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((n_pages, Hkv, bs, 128), generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(37)
    table = torch.as_tensor(rng.permutation(n_pages)[:N].astype(np.int32)[None], device="cuda").contiguous()
    q = torch.randn((B, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
    ws = torch.zeros((L.workspace_bytes(s, 64) // 4 + 1,), dtype=torch.float32, device="cuda")
    for name, vals in list(_tie_cases(rng, B * Hkv, N).items())[:6]:
        sc = torch.as_tensor(vals.astype(np.float32).reshape(B, Hkv, N), device="cuda").contiguous()
        em = torch.as_tensor(np.round(rng.standard_normal((B, Hkv, N)) * 3).astype(np.float32), device="cuda")
        for K, Kp, kspec in [(256, 384, 300), (1024, 64, 0), (7, 1024, 64)]:
            cur = torch.as_tensor(np.stack([np.sort(rng.choice(N, max(kspec, 1), replace=False))
                                            for _ in range(B * Hkv)]).reshape(B, Hkv, -1).astype(np.int32),
                                  device="cuda")
            res = []
            for w_ in (ws, None):
                sel = torch.full((B, Hkv, K), -1, dtype=torch.int32, device="cuda")
                pn = torch.full((B, Hkv, Kp), -1, dtype=torch.int32, device="cuda")
                pa = torch.zeros((max(L.partials_bytes(s, kspec), 4) // 4,), dtype=torch.float32, device="cuda")
                L.select_speculate(s, sc, K, sel, em, Kp, pn, q, kc, vc, table, cur, kspec, pa, workspace=w_)
                torch.cuda.synchronize()
                res.append((sel, pn, pa))
            (sel_a, pn_a, pa_a), (sel_b, pn_b, pa_b) = res
            assert torch.equal(sel_a, sel_b) and torch.equal(pn_a, pn_b), (name, K, Kp)
            assert torch.equal(pa_a.view(torch.int32), pa_b.view(torch.int32)), (name, K, Kp)
            s32, e32 = sc.cpu().numpy().reshape(-1, N), em.cpu().numpy().reshape(-1, N)
            for r in range(B * Hkv):
                assert np.array_equal(sel_a.cpu().numpy().reshape(-1, K)[r], _ref_top_k(s32[r], K)), (name, K, r)
                assert np.array_equal(pn_a.cpu().numpy().reshape(-1, Kp)[r], _ref_top_k(e32[r], Kp)), (name, Kp, r)


@pytest.mark.parametrize("name", SMALL)
def test_fused_launches_match_separate(name):
    """prr_score (with the EMA update) followed by prr_select_speculate produce, bit for bit, the scores, EMA, true
    set, next predicted set and speculation partials of the separate calls (score_select, ema_predict, speculate)."""
    w, inp, s, summ, ov = _setup(name)
    B, Hkv, N, K = w.batch, w.n_kv_heads, w.n_blocks, w.top_k
    Kp = max(w.k_spec) or K
    dev = "cuda"
    sc_a, sc_b = (torch.zeros((B, Hkv, N), dtype=torch.float32, device=dev) for _ in range(2))
    em_a, em_b = (torch.zeros((B, Hkv, N), dtype=torch.float32, device=dev) for _ in range(2))
    sel_a, sel_b = (torch.full((B, Hkv, K), -1, dtype=torch.int32, device=dev) for _ in range(2))
    pn_a, pn_b = (torch.full((B, Hkv, Kp), -1, dtype=torch.int32, device=dev) for _ in range(2))
    pb = L.partials_bytes(s, Kp) // 4
    pa_a, pa_b = (torch.zeros((pb,), dtype=torch.float32, device=dev) for _ in range(2))
    rng = np.random.default_rng(11)
    em_prev = None
    for t in range(3):
        q = inp.q[t].contiguous()
        cur = torch.as_tensor(np.stack([np.sort(rng.choice(N, Kp, replace=False)) for _ in range(B * Hkv)])
                              .reshape(B, Hkv, Kp).astype(np.int32), device=dev)
        L.score_select(s, q, summ, K, sc_a, sel_a)
        L.ema_predict(s, sc_a, em_a, w.alpha, t == 0, Kp, pn_a)
        L.speculate(s, q, inp.k_cache, inp.v_cache, inp.table, cur, Kp, pa_a)
        L.score(s, q, summ, sc_b, em_b, w.alpha, t == 0)
        L.select_speculate(s, sc_b, K, sel_b, em_b, Kp, pn_b, q, inp.k_cache, inp.v_cache, inp.table, cur, Kp, pa_b)
        torch.cuda.synchronize()
        assert torch.equal(sc_a, sc_b), t
        assert torch.equal(em_a.view(torch.int32), em_b.view(torch.int32)), t
        assert torch.equal(sel_a, sel_b), t
        assert torch.equal(pn_a, pn_b), t
        assert torch.equal(pa_a.view(torch.int32), pa_b.view(torch.int32)), t
        # scores + EMA + speculation in one launch: the same bits again
        sc_c, em_c = torch.zeros_like(sc_a), em_b.clone()
        pa_c = torch.zeros_like(pa_a)
        if t > 0:
            em_c.copy_(em_prev)
        L.score_speculate(s, q, summ, sc_c, em_c, w.alpha, t == 0, inp.k_cache, inp.v_cache, inp.table, cur, Kp,
                          pa_c)
        torch.cuda.synchronize()
        assert torch.equal(sc_a, sc_c) and torch.equal(em_a.view(torch.int32), em_c.view(torch.int32)), t
        assert torch.equal(pa_a.view(torch.int32), pa_c.view(torch.int32)), t
        em_prev = em_a.clone()


@pytest.mark.parametrize("name,short", [("tiny_f32_4k", 31), ("llama3_8b_32k", 5), ("paged_b32_64k", 15),
                                        ("long_ctx_131k_b4", 40), ("million_token", 3)])
def test_partial_last_block_summaries_and_append(name, short):
    """Sequences that end inside their last block: the summaries cover the tokens that exist (the slots past the end
    hold poison that must never enter). Then tokens are appended one at a time through prr_append_kv (when the last
    block holds a single token, the first append rewrites it and so opens the block): the cache rows written equal the
    appended tokens, and after every append each summary equals the oracle's over the longer sequence, exactly."""
    w = ragged(small(name), short)
    print(f"[case] partial last block {w.name} ctx={w.ctx} N={w.n_blocks}", flush=True)
    inp = gap_inputs(w)
    s = shape_of(w)
    B, Hkv, N, D, bs, page = w.batch, w.n_kv_heads, w.n_blocks, w.head_dim, w.block_size, w.page_size
    summ = torch.zeros((B, Hkv, N, 2, D), dtype=w.torch_dtype, device="cuda")
    L.build_summaries(s, inp.k_cache, inp.table, summ)
    torch.cuda.synchronize()
    ov = OracleView(inp)
    keys = {(b, g): ov.keys(b, g) for b in range(B) for g in range(Hkv)}
    vals = {(b, g): ov.values(b, g) for b in range(B) for g in range(Hkv)}

    def check_summaries(tag):
        got = np64(summ)
        for (b, g), k in keys.items():
            kmin, kmax = O.block_summaries(k, bs)
            assert np.array_equal(got[b, g, :, 0], kmin) and np.array_equal(got[b, g, :, 1], kmax), (tag, b, g)

    check_summaries("built")
    rng = np.random.default_rng(41)
    n_tok = w.ctx
    if (n_tok - 1) % bs == 0:   # rewrite the last block's only token: the append opens the block
        n_tok -= 1
        for key in keys:
            keys[key], vals[key] = keys[key][:-1], vals[key][:-1]
    for i in range(min(6, w.n_blocks * bs - n_tok)):
        kn = torch.as_tensor(rng.standard_normal((B, Hkv, D)), dtype=torch.float32).to(w.torch_dtype)
        vn = torch.as_tensor(rng.standard_normal((B, Hkv, D)), dtype=torch.float32).to(w.torch_dtype)
        n_tok += 1
        s.ctx_len = n_tok
        L.append_kv(s, kn.cuda(), vn.cuda(), inp.k_cache, inp.v_cache, inp.table, summ)
        torch.cuda.synchronize()
        pos = n_tok - 1
        for (b, g) in keys:
            keys[(b, g)], vals[(b, g)] = O.append_token(keys[(b, g)], vals[(b, g)], kn[b, g].double().numpy(),
                                                         vn[b, g].double().numpy())
            phys = int(inp.table_np[b, pos // page])
            assert torch.equal(inp.k_cache[phys, g, pos % page].cpu(), kn[b, g]), (i, b, g)
            assert torch.equal(inp.v_cache[phys, g, pos % page].cpu(), vn[b, g]), (i, b, g)
        check_summaries(f"append {i}")


@pytest.mark.parametrize("n_blocks", [300, 20001])
def test_topk_forced_blocks(n_blocks):
    """Forced blocks (the first sink_blocks and last local_blocks) in every top-K launch: prr_ema_predict and
    prr_select_speculate (one workgroup per row, and by segments on long rows with a workspace), for K below, at and
    above the number of forced blocks, on values with many ties: equal to the oracle's rule."""
    N, rows = n_blocks, 2
    rng = np.random.default_rng(47)
    print(f"[case] forced blocks N={N}", flush=True)
    for sink, local in [(1, 0), (0, 3), (2, 5)]:
        s = L.make_shape(1, 8, rows, 128, 16, 16, N, L.BF16, sink_blocks=sink, local_blocks=local)
        ws = torch.zeros((L.workspace_bytes(s, 64) // 4 + 1,), dtype=torch.float32, device="cuda")
        vals = (np.round(rng.standard_normal((rows, N)) * 4) + 0.25).astype(np.float32)
        vd = torch.as_tensor(vals[None], device="cuda").contiguous()
        em = torch.zeros_like(vd)
        for k in sorted({1, sink + local, sink + local + 1, 64, 300}):
            if k < 1 or k > N:
                continue
            ref = np.stack([O.top_k(vals[r].astype(np.float64), k, sink, local) for r in range(rows)])
            for w_ in (None, ws):
                out = torch.full((1, rows, k), -1, dtype=torch.int32, device="cuda")
                L.ema_predict(s, vd, em, 0.5, True, k, out, workspace=w_)
                sel = torch.full((1, rows, k), -1, dtype=torch.int32, device="cuda")
                pn = torch.full((1, rows, k), -1, dtype=torch.int32, device="cuda")
                L.select_speculate(s, vd, k, sel, em, k, pn, workspace=w_)
                torch.cuda.synchronize()
                for name, got in (("ema_predict", out), ("select T", sel), ("select P", pn)):
                    assert np.array_equal(got.cpu().numpy()[0], ref), (name, sink, local, k, w_ is not None)


@pytest.mark.parametrize("name,short", [("tiny_f32_4k", 9), ("llama3_8b_32k", 0), ("paged_b32_64k", 15),
                                        ("million_token", 5)])
def test_mean_scorer_summaries_scores_append(name, short):
    """The mean-key scorer: each block's fp32 mean key (a partial last block over the tokens it holds), the scores
    against the oracle's mean-key scores, and the running mean after appends against the mean recomputed over the
    longer sequence; all within fp32 rounding of the fp64 values."""
    from tests.gpu_common import oracle_scores
    w = small(name).replace(scorer="mean")
    if short:
        w = ragged(w, short)
    print(f"[case] mean scorer {w.name} ctx={w.ctx}", flush=True)
    inp = gap_inputs(w)
    s = shape_of(w)
    B, Hkv, N, D, bs = w.batch, w.n_kv_heads, w.n_blocks, w.head_dim, w.block_size
    summ = torch.zeros((B, Hkv, N, 2, D), dtype=w.torch_dtype, device="cuda")
    L.build_summaries(s, inp.k_cache, inp.table, summ)
    ov = OracleView(inp)
    keys = {(b, g): ov.keys(b, g) for b in range(B) for g in range(Hkv)}

    def means_gpu():
        raw = summ.view(torch.uint8).reshape(B, Hkv, N, -1)[..., :D * 4].contiguous().view(torch.float32)
        return raw.cpu().numpy().astype(np.float64)

    def check_means(tag):
        got = means_gpu()
        for (b, g), k in keys.items():
            ref = O.block_means(k, bs)
            assert np.allclose(got[b, g], ref, rtol=0, atol=2e-6 * max(1.0, np.abs(k).max())), (tag, b, g)

    torch.cuda.synchronize()
    check_means("built")
    scores = torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda")
    q = inp.q[1].contiguous()
    L.score(s, q, summ, scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy().astype(np.float64)
    for (b, g), k in keys.items():
        ref = oracle_scores(w, ov.q_group(1, b, g), k)
        assert np.allclose(sc[b, g], ref, rtol=0, atol=1e-5 * max(1.0, np.abs(ref).max())), (b, g)
    rng = np.random.default_rng(53)
    n_tok = w.ctx
    for i in range(min(4, w.n_blocks * bs - n_tok)):
        kn = torch.as_tensor(rng.standard_normal((B, Hkv, D)), dtype=torch.float32).to(w.torch_dtype)
        vn = torch.as_tensor(rng.standard_normal((B, Hkv, D)), dtype=torch.float32).to(w.torch_dtype)
        n_tok += 1
        s.ctx_len = n_tok
        L.append_kv(s, kn.cuda(), vn.cuda(), inp.k_cache, inp.v_cache, inp.table, summ)
        torch.cuda.synchronize()
        for (b, g) in keys:
            keys[(b, g)] = np.concatenate([keys[(b, g)], kn[b, g].double().numpy()[None]])
        check_means(f"append {i}")
