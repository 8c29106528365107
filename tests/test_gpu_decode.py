"""Whole decode runs through the two-stream step (libprr's prr_decode_step) against the fp64 oracle, on reduced
workloads: every step's selection (tie-band rule), output (stated tolerance), missed count, and the predictor's
sets; the three modes; EMA save and restore."""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd import _lib as L
from dynamic_sparse_attention_decode_amd.runtime import PRRLayer
from oracle import prr_oracle as O
from tests.checker import TOL, check_selection, max_abs
from tests.gpu_common import (OracleView, SMALL, gap_inputs, np64, oracle_scores, ragged, requires_gpu, shape_of,
                              small, wide_paged)

pytestmark = [pytest.mark.gpu, requires_gpu]


def run_layer(w, inp, k_spec, mode, steps=None, check=True, ov=None):
    """Run the layer over the steps; returns per-step (out, sel, pred, n_missed) host copies and stats."""
    steps = w.steps if steps is None else steps
    layer = PRRLayer(shape_of(w), w.top_k, k_spec, w.alpha, mode=mode)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    hist = []
    ema_ref = {}
    for t in range(steps):
        ids = inp.drift(t)
        if len(ids):
            layer.rebuild_blocks(torch.as_tensor(ids, device="cuda"))
            if ov is not None:
                ov.invalidate_keys()
        out = layer.step(inp.q[t].contiguous())
        torch.cuda.synchronize()
        hist.append(dict(out=np64(out), sel=layer.sel_idx.cpu().numpy().copy(),
                         pred=None if (t == 0 or layer.k_spec == 0) else layer.pred_current.cpu().numpy().copy(),
                         nm=layer.n_missed.cpu().numpy().copy(), ema=np64(layer.ema)))
        if check:
            _check_step(w, ov, t, hist[-1], layer.k_spec, ema_ref)
    layer.close()
    return hist


def _check_step(w, ov, t, h, k_spec, ema_ref):
    G = w.group
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            qg = ov.q_group(t, b, g)
            keys = ov.keys(b, g)
            s = oracle_scores(w, qg, keys)
            exact = check_selection(h["sel"][b, g], s, w.top_k, n_sink=w.sink_blocks, n_local=w.local_blocks)
            # the inputs keep the oracle's relative gap above 1e-4 at every step, so the set must be the oracle's
            assert exact, (t, b, g, "banded instance: the inputs did not keep the gap")
            ref = O.attention_over_blocks(qg, keys, ov.values(b, g), h["sel"][b, g], w.block_size, w.scale)
            e = max_abs(h["out"][b, g * G:(g + 1) * G], ref)
            assert e <= TOL[w.dtype], (t, b, g, e)
            # oracle EMA over the oracle's scores; the GPU's predicted set must be valid for it
            prev = ema_ref.get((b, g)) if t > 0 else None
            if t > 0 and k_spec:
                check_selection(h["pred"][b, g], prev, k_spec, n_sink=w.sink_blocks, n_local=w.local_blocks)
                missed = len(set(h["sel"][b, g]) - set(h["pred"][b, g]))
                assert h["nm"][b, g] == missed
            elif t == 0 or not k_spec:
                assert h["nm"][b, g] == w.top_k
            ema_ref[(b, g)] = O.ema_update(prev, s, w.alpha, t == 0)


@pytest.mark.parametrize("mode", ["prr_2stream", "prr_fused", "serialized_fused"])
@pytest.mark.parametrize("name", SMALL)
def test_decode_vs_oracle(name, mode):
    w = small(name)
    for kp in (w.k_spec if mode != "serialized_fused" else (0,)):
        print(f"[case] decode {name} {mode} K'={kp}", flush=True)
        inp = gap_inputs(w)
        ov = OracleView(inp)
        hist = run_layer(w, inp, kp, mode, ov=ov)
        if kp:
            ov_steps = [len(set(h["sel"][b, g]) & set(h["pred"][b, g])) / w.top_k
                        for h in hist[1:] for b in range(w.batch) for g in range(w.n_kv_heads)]
            print(f"[result] {name} K'={kp}: mean overlap {np.mean(ov_steps):.3f}, "
                  f"mean missed {np.mean([h['nm'].mean() for h in hist[1:]]):.2f}")


def _run_unsynced(w, inp, k_spec, mode, delays=None):
    """All steps enqueued without a host synchronisation between them; each step's results are copied on the
    caller's stream (ordered after the step's stream_sel work)."""
    layer = PRRLayer(shape_of(w), w.top_k, k_spec, w.alpha, mode=mode)
    if delays:
        L.step_ctx_set_delays(layer.ctx, *delays)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    qs = [inp.q[t].contiguous() for t in range(w.steps)]
    res = []
    for t in range(w.steps):
        out = layer.step(qs[t])
        res.append((out.clone(), layer.sel_idx.clone(), layer.n_missed.clone(), layer.pred_next.clone()))
    torch.cuda.synchronize()
    layer.close()
    return [tuple(x.cpu().numpy() for x in r) for r in res]


@pytest.mark.parametrize("name", ["llama3_8b_32k", "paged_b32_64k", "million_token"])
def test_two_stream_delays_do_not_change_results(name):
    """Race check: a bounded sleep kernel (about 100 us) on stream_spec before the speculation, on stream_sel before
    the repair, or on both, leaves every step's output, selection, missed count and next predicted set bitwise equal
    to the one-stream run: the two streams are ordered by their fork and join, not by timing."""
    w = small(name)
    kp = max(w.k_spec)
    inp = gap_inputs(w)
    ref = _run_unsynced(w, inp, kp, "prr_1stream")
    for delays in ((0, 30), (30, 0), (30, 30)):
        print(f"[case] two-stream delays {name} (sel, spec) = {delays}", flush=True)
        got = _run_unsynced(w, inp, kp, "prr_2stream", delays)
        for t, (a, b) in enumerate(zip(ref, got)):
            for x, y, what in zip(a, b, ("out", "sel_idx", "n_missed", "pred_next")):
                assert np.array_equal(x, y), (delays, t, what)


@pytest.mark.parametrize("k_spec,extra", [(12, {}), (20, {}), (20, {"sink_blocks": 1, "local_blocks": 3}),
                                          (20, {"scorer": "mean"}),
                                          (20, {"batch": 64, "top_k": 64, "ctx": 16 * 100 - 3})])
def test_decode_many_rows_vs_oracle(k_spec, extra):
    """A batch of 136 rows (17 sequences x 8 KV heads, a partly filled last block): the fused step's many-row path
    (speculation in its own launch, then the scores, the selection of T and of P_{t+1} with the EMA update, the
    repair), also with forced sink and local blocks and with the mean-key scorer; and 512 rows with K = 64, where one
    repair workgroup per row writes the output itself; every step against the oracle."""
    w = wide_paged(k_spec=(k_spec,), **extra)
    print(f"[case] decode many rows B={w.batch} K'={k_spec} {extra}", flush=True)
    inp = gap_inputs(w)
    run_layer(w, inp, k_spec, "prr_fused", ov=OracleView(inp))


def test_decode_wide_selection_launch_vs_oracle():
    """32 rows of 64-token blocks (drifting hot blocks) with K' = 80: the fused step's selection launch holds 64 top-K
    workgroups and 2560 speculation waves, more than one 512-thread workgroup per CU can hold at once, so it runs as
    256-thread workgroups, and each block's four chunks share one page lookup; every step against the oracle, and the
    EMA, the selected and predicted sets and the missed counts bitwise equal to the one-stream step."""
    w = small("long_ctx_131k_b4").replace(batch=4, top_k=20, k_spec=(80,), steps=6)
    print(f"[case] decode wide selection launch B={w.batch} N={w.n_blocks} K={w.top_k} K'=80", flush=True)
    inp = gap_inputs(w)
    got = run_layer(w, inp, 80, "prr_fused", ov=OracleView(inp))
    ref = run_layer(w, gap_inputs(w), 80, "prr_1stream", check=False)
    for t, (a, b) in enumerate(zip(ref, got)):
        assert np.array_equal(a["ema"], b["ema"]), t
        assert np.array_equal(a["sel"], b["sel"]) and np.array_equal(a["nm"], b["nm"]), t
        if a["pred"] is not None:
            assert np.array_equal(a["pred"], b["pred"]), t


@pytest.mark.parametrize("name", ["llama3_8b_32k", "paged_b32_64k", "tiny_f32_4k", "million_token"])
def test_modes_agree(name):
    """Two-stream and one-stream runs are bitwise identical (same kernels, same order). The two-launch fused run
    selects the same true and predicted sets and misses the same blocks; its output (merged in another order) and
    the serialized runs' outputs match within the output tolerance."""
    w = small(name)
    kp = max(w.k_spec)
    runs = {}
    for mode in ("prr_2stream", "prr_fused", "prr_1stream", "serialized", "serialized_fused"):
        inp = gap_inputs(w)
        runs[mode] = run_layer(w, inp, kp, mode, check=False)
    for a, b in zip(runs["prr_2stream"], runs["prr_1stream"]):
        assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["sel"], b["sel"])
        assert np.array_equal(a["nm"], b["nm"])
        if a["pred"] is not None:
            assert np.array_equal(a["pred"], b["pred"])
    for a, b in zip(runs["prr_2stream"], runs["prr_fused"]):
        assert np.array_equal(a["sel"], b["sel"]) and np.array_equal(a["nm"], b["nm"])
        if a["pred"] is not None:
            assert np.array_equal(a["pred"], b["pred"])
        assert max_abs(a["out"], b["out"]) <= TOL[w.dtype]
    for ser in ("serialized", "serialized_fused"):
        for a, b in zip(runs["prr_2stream"], runs[ser]):
            assert np.array_equal(a["sel"], b["sel"])
            assert max_abs(a["out"], b["out"]) <= TOL[w.dtype]
            assert np.all(b["nm"] == w.top_k)


@pytest.mark.parametrize("name", ["paged_wide", "llama3_8b_32k", "million_token", "tiny_f32_4k", "million_long"])
def test_ema_identical_in_every_mode(name):
    """The EMA update runs in the scoring pass, in the selection launch's prediction workgroups (many rows), in the
    EMA-segment workgroups of the segment launch (long rows) or in a prediction launch of its own (one and two
    streams), always as e = fma(alpha, e, (1 - alpha) s): after every
    step the EMA, the selected and predicted sets and the missed counts are bitwise the same in each mode."""
    if name == "paged_wide":
        w = wide_paged()
    elif name == "million_long":   # 12000 blocks per row: selection by segments and a merge
        w = small("million_token").replace(ctx=32 * 12000 - 7, top_k=61, k_spec=(93,), steps=6)
    else:
        w = small(name)
    kp = max(w.k_spec) or w.top_k
    print(f"[case] EMA across modes {name} N={w.n_blocks} K'={kp}", flush=True)
    ref = run_layer(w, gap_inputs(w), kp, "prr_1stream", check=False)
    for mode in ("prr_fused", "prr_2stream"):
        got = run_layer(w, gap_inputs(w), kp, mode, check=False)
        for t, (a, b) in enumerate(zip(ref, got)):
            assert np.array_equal(a["ema"], b["ema"]), (mode, t)
            assert np.array_equal(a["sel"], b["sel"]) and np.array_equal(a["nm"], b["nm"]), (mode, t)
            if a["pred"] is not None:
                assert np.array_equal(a["pred"], b["pred"]), (mode, t)


def test_ema_state_save_restore():
    """The EMA vector and the next predicted set are the only cross-step state: restoring them into a fresh layer
    reproduces the remaining predicted sets and outputs exactly."""
    w = small("llama3_8b_32k")
    kp = w.k_spec[0]
    inp = gap_inputs(w)
    full = run_layer(w, inp, kp, "prr_2stream", check=False)
    inp = gap_inputs(w)
    layer = PRRLayer(shape_of(w), w.top_k, kp, w.alpha)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    cut = 4
    for t in range(cut):
        layer.step(inp.q[t].contiguous())
    torch.cuda.synchronize()
    saved = dict(ema=layer.ema.cpu().clone(), pred=layer.pred_next.cpu().clone(), t=layer.t)
    layer.close()
    fresh = PRRLayer(shape_of(w), w.top_k, kp, w.alpha)
    fresh.build(inp.k_cache, inp.v_cache, inp.table)
    fresh.ema.copy_(saved["ema"].cuda())
    fresh.t = saved["t"]
    fresh.pred[fresh.t % 2][..., :kp].copy_(saved["pred"].cuda())
    for t in range(cut, w.steps):
        out = fresh.step(inp.q[t].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(np64(out), full[t]["out"])
        assert np.array_equal(fresh.pred_current.cpu().numpy(), full[t]["pred"])
    fresh.close()


@pytest.mark.parametrize("rows,mode", [("short", "prr_2stream"), ("short", "prr_fused"), ("long", "prr_fused"),
                                       ("long", "serialized"), ("long", "prr_2stream")])
def test_graph_replay_matches_eager(rows, mode):
    """Steps captured in a HIP graph and replayed several times (with eager work and synchronisation between the
    replays) give the same outputs, selections and missed counts as the same steps run eagerly; also with rows of
    12000 blocks, which select by segments through the workspace's candidate regions (the last block partly
    filled)."""
    if rows == "short":
        w = small("llama3_8b_32k")
        kp = w.k_spec[0]
    else:
        w = small("million_token").replace(ctx=32 * 12000 - 7, top_k=61, k_spec=(93,), steps=6)
        kp = 93
    print(f"[case] graph replay {rows} rows N={w.n_blocks} {mode}", flush=True)
    inp = gap_inputs(w)
    qs = [inp.q[t].contiguous() for t in range(w.steps)]
    seq = [0] + [1, 2, 3, 4] * 3
    eager = PRRLayer(shape_of(w), w.top_k, kp, w.alpha, mode=mode)
    eager.build(inp.k_cache, inp.v_cache, inp.table)
    ref = []
    for t in seq:
        out = eager.step(qs[t])
        torch.cuda.synchronize()
        ref.append((np64(out), eager.sel_idx.cpu().numpy().copy(), eager.n_missed.cpu().numpy().copy()))
    eager.close()
    lay = PRRLayer(shape_of(w), w.top_k, kp, w.alpha, mode=mode)
    lay.build(inp.k_cache, inp.v_cache, inp.table)
    lay.step(qs[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=lay.s_sel):
        outs = [lay.enqueue(qs[t], join=(t == 4)) for t in (1, 2, 3, 4)]
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
        del scratch
    lay.close()


def _variant(dtype, G, page, k):
    """A small layer of the given storage dtype and group size (two KV heads, two sequences), with pages shuffled."""
    from dynamic_sparse_attention_decode_amd.inputs import Workload
    D = 64 if dtype == "f32" else 128
    return Workload(f"variant_{dtype}_g{G}_p{page}", 2, 2 * G, 2, D, 32 * 70, 32, page, k, (k + 5,), 0.8, 0.9, 4, 6,
                    shuffle_pages=True, dtype=dtype, seed=20261203 + 17 * G + page)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_dtypes_and_group_sizes(dtype, G):
    """Every storage dtype and group size the library supports, through the fused PRR step (page-aligned chunks)
    and the serialized step on 8-token pages (chunks straddling pages), against the oracle at every step."""
    for page, mode, k in ((16, "prr_fused", 13), (8, "serialized", 11), (16, "prr_fused", 40), (8, "prr_fused", 13)):
        w = _variant(dtype, G, page, k)
        print(f"[case] {w.name} {mode} K={k}", flush=True)
        inp = gap_inputs(w)
        ov = OracleView(inp)
        run_layer(w, inp, max(w.k_spec), mode, ov=ov)


@pytest.mark.parametrize("dtype,G", [("f32", 4), ("f16", 8), ("bf16", 1)])
def test_row_workgroup_repair_dtypes_and_groups(dtype, G):
    """256 rows with K = 124 of 140 blocks: the repair takes one 8-wave workgroup per row that splits T into hits and
    missed blocks and writes the output itself; other storage dtypes and group sizes than the paged batch's, in the
    fused PRR step and the serialized one, against the oracle at every step."""
    from dynamic_sparse_attention_decode_amd.inputs import Workload
    D = 64 if dtype == "f32" else 128
    w = Workload(f"rows256_{dtype}_g{G}", 128, 2 * G, 2, D, 16 * 140 - 5, 16, 16, 124, (130,), 0.8, 0.9, 3, 6,
                 shuffle_pages=True, dtype=dtype, seed=20261203 + 29 * G)
    inp = gap_inputs(w)
    for mode in ("prr_fused", "serialized"):
        print(f"[case] {w.name} {mode}", flush=True)
        run_layer(w, inp, 130, mode, ov=OracleView(inp))


def test_all_blocks_selected_is_dense_attention():
    """K = N (every block selected) equals dense attention over the whole context, in the fused PRR step."""
    w = small("tiny_f32_4k").replace(top_k=128, k_spec=(128,), steps=3)
    inp = gap_inputs(w)
    ov = OracleView(inp)
    hist = run_layer(w, inp, 128, "prr_fused", ov=ov)
    G = w.group
    for t, h in enumerate(hist):
        qg = ov.q_group(t, 0, 0)
        ref = O.attention_over_blocks(qg, ov.keys(0, 0), ov.values(0, 0), np.arange(128), w.block_size, w.scale)
        assert max_abs(h["out"][0, :G], ref) <= TOL[w.dtype]
        assert list(h["sel"][0, 0]) == list(range(128))


PARTIAL = [("tiny_f32_4k", 31, "prr_fused"), ("llama3_8b_32k", 5, "prr_fused"), ("llama3_8b_32k", 9, "serialized"),
           ("long_ctx_131k_b4", 40, "prr_2stream"), ("paged_b32_64k", 15, "prr_fused"),
           ("paged_b32_64k", 7, "serialized_fused"), ("million_token", 3, "prr_fused"),
           ("million_token", 20, "prr_1stream")]


@pytest.mark.parametrize("name,short,mode", PARTIAL)
def test_partial_last_block_decode(name, short, mode):
    """Sequences that end inside their last block (the slots past the end hold poison): every step's selection,
    output, missed count and predicted set against the oracle over the tokens that exist."""
    w = ragged(small(name), short).replace(steps=4)
    print(f"[case] partial decode {w.name} ctx={w.ctx} {mode}", flush=True)
    inp = gap_inputs(w)
    ov = OracleView(inp)
    kp = max(w.k_spec) or w.top_k
    run_layer(w, inp, kp, mode, ov=ov)


class _Grown:
    """Oracle view of sequences that grow by one appended token per step (host copies of what was appended)."""

    def __init__(self, ov):
        self.ov = ov
        self.k = {}
        self.v = {}

    def keys(self, b, g):
        return self.k.setdefault((b, g), self.ov.keys(b, g))

    def values(self, b, g):
        return self.v.setdefault((b, g), self.ov.values(b, g))

    def append(self, b, g, kn, vn):
        self.k[(b, g)], self.v[(b, g)] = O.append_token(self.keys(b, g), self.values(b, g), kn, vn)

    def q_group(self, t, b, g):
        return self.ov.q_group(t, b, g)


@pytest.mark.parametrize("name,mode", [("llama3_8b_32k", "prr_fused"), ("paged_b32_64k", "prr_2stream"),
                                       ("tiny_f32_4k", "serialized"), ("million_token", "prr_fused"),
                                       ("paged_wide", "prr_fused")])
def test_decode_with_appends(name, mode):
    """A decoder's loop: before every step after the first, one new token per sequence is appended (prr_append_kv
    through PRRLayer.append); the step then selects, speculates and repairs over the longer sequences. Checked at
    every step against the oracle over the sequences with the same appended tokens."""
    w = ragged(wide_paged() if name == "paged_wide" else small(name), 7).replace(steps=6)
    print(f"[case] decode with appends {w.name} {mode}", flush=True)
    inp = gap_inputs(w)
    view = _Grown(OracleView(inp))
    kp = max(w.k_spec) or w.top_k
    layer = PRRLayer(shape_of(w), w.top_k, kp, w.alpha, mode=mode)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    rng = np.random.default_rng(43)
    ema_ref = {}
    for t in range(w.steps):
        if t > 0:
            kn = torch.as_tensor(rng.standard_normal((w.batch, w.n_kv_heads, w.head_dim)),
                                 dtype=torch.float32).to(w.torch_dtype)
            vn = torch.as_tensor(rng.standard_normal((w.batch, w.n_kv_heads, w.head_dim)),
                                 dtype=torch.float32).to(w.torch_dtype)
            layer.append(kn.cuda(), vn.cuda())
            for b in range(w.batch):
                for g in range(w.n_kv_heads):
                    view.append(b, g, kn[b, g].double().numpy(), vn[b, g].double().numpy())
        out = layer.step(inp.q[t].contiguous())
        torch.cuda.synchronize()
        h = dict(out=np64(out), sel=layer.sel_idx.cpu().numpy().copy(),
                 pred=None if (t == 0 or layer.k_spec == 0) else layer.pred_current.cpu().numpy().copy(),
                 nm=layer.n_missed.cpu().numpy().copy())
        _check_step(w, view, t, h, layer.k_spec, ema_ref)
    assert layer.shape.ctx_len == w.ctx + w.steps - 1
    layer.close()


@pytest.mark.parametrize("name,mode", [("tiny_f32_4k", "prr_fused"), ("llama3_8b_32k", "prr_2stream"),
                                       ("paged_b32_64k", "prr_fused"), ("million_token", "serialized"),
                                       ("long_ctx_131k_b4", "prr_1stream")])
def test_forced_blocks_decode(name, mode):
    """Attention sinks and a local window (one sink block, three local blocks) forced into every selection and
    prediction: each step against the oracle with the same forced blocks."""
    w = small(name).replace(sink_blocks=1, local_blocks=3, steps=4)
    print(f"[case] forced blocks decode {name} {mode}", flush=True)
    inp = gap_inputs(w)
    kp = max(w.k_spec) or w.top_k
    run_layer(w, inp, kp, mode, ov=OracleView(inp))


@pytest.mark.parametrize("name,mode,extra", [("tiny_f32_4k", "prr_fused", {}), ("llama3_8b_32k", "serialized", {}),
                                             ("llama3_8b_32k", "prr_2stream", {"sink_blocks": 1, "local_blocks": 2}),
                                             ("paged_b32_64k", "prr_fused", {}),
                                             ("million_token", "prr_fused", {"ctx_short": 11})])
def test_mean_scorer_decode(name, mode, extra):
    """The whole decode with the mean-key scorer (with forced blocks, and with a partly filled last block): every
    step against the oracle's mean-key selection and attention."""
    extra = dict(extra)
    short = extra.pop("ctx_short", 0)
    w = small(name).replace(scorer="mean", steps=4, **extra)
    if short:
        w = ragged(w, short)
    print(f"[case] mean scorer decode {w.name} {mode} {extra}", flush=True)
    inp = gap_inputs(w)
    kp = max(w.k_spec) or w.top_k
    run_layer(w, inp, kp, mode, ov=OracleView(inp))


@pytest.mark.parametrize("mode", ["prr_fused", "serialized", "prr_2stream"])
@pytest.mark.parametrize("ctx,bs,page,k,kp", [(5, 32, 32, 1, 1), (32, 32, 32, 1, 1), (40, 16, 16, 2, 3),
                                               (17, 16, 8, 1, 2), (3, 16, 16, 1, 1), (5100, 256, 256, 4, 6),
                                               (200, 4, 4, 5, 7), (301, 12, 4, 6, 8), (1000, 128, 32, 3, 5)])
def test_degenerate_contexts(ctx, bs, page, k, kp, mode):
    """The smallest layers and the block-size extremes: one block (partly or wholly filled), a few blocks with K and
    K' near N, pages smaller than a 16-token chunk, blocks of 4 and 12 tokens, blocks of 128 and 256 tokens (chunks
    beyond one pipelined call); every step against the oracle (selection, output, missed count, predicted set)."""
    from dynamic_sparse_attention_decode_amd.inputs import Workload
    w = Workload(f"degenerate_{ctx}_{bs}_{page}", 2, 8, 2, 128, ctx, bs, page, k, (kp,), 0.8, 0.9, 4, 0,
                 shuffle_pages=True, seed=20261203 + ctx + bs + page)
    print(f"[case] degenerate ctx={ctx} bs={bs} page={page} N={w.n_blocks} K={k} K'={kp} {mode}", flush=True)
    inp = gap_inputs(w)
    ov = OracleView(inp)
    run_layer(w, inp, kp if mode != "serialized" else 0, mode, ov=ov)


def test_kernel_trace_lifecycle():
    """The per-kernel trace as the benchmark uses it: enabled around eager steps, read (one positive duration per
    traced launch), disabled and destroyed, three traces in a row; steps after the last one is destroyed run
    untraced (the library drops a destroyed trace)."""
    w = small("llama3_8b_32k")
    inp = gap_inputs(w)
    lay = PRRLayer(shape_of(w), w.top_k, w.k_spec[0], w.alpha, mode="prr_1stream")
    lay.build(inp.k_cache, inp.v_cache, inp.table)
    qs = [inp.q[t].contiguous() for t in range(w.steps)]
    for rep in range(3):
        tr = L.Trace(16)
        tr.enable(["score", "repair", "speculate"])
        for t in range(4):
            lay.step(qs[t])
        torch.cuda.synchronize()
        tr.disable()
        for k, n in (("score", 4), ("repair", 4), ("speculate", 3)):   # step 0 of each run has nothing predicted
            d = tr.read(k)
            assert len(d) == n and all(x > 0 for x in d), (rep, k, d)
        tr.close()
        lay.reset()
    lay.step(qs[0])
    torch.cuda.synchronize()
    lay.close()
