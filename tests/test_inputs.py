"""The seeded input generator: determinism, hot-block planting, drift, paging (CPU)."""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS, make_inputs, query_stream, block_table


def _small(name, **kw):
    w = WORKLOADS[name]
    base = dict(ctx=w.block_size * 64, steps=9, hot_blocks=min(w.hot_blocks, 8) if w.hot_blocks else 0,
                top_k=min(w.top_k, 16), k_spec=tuple(min(k, 20) for k in w.k_spec))
    base.update(kw)
    return w.replace(**base)


def test_workload_shapes():
    for w in WORKLOADS.values():
        w.validate()
    w = WORKLOADS["million_token"]
    assert w.n_blocks == 32768 and w.group == 8 and w.k_spec == (0, 128, 256, 384)
    w = WORKLOADS["paged_b32_64k"]
    assert w.n_blocks == 4096 and w.shuffle_pages and w.page_size == 16


def test_determinism_same_bytes():
    w = _small("llama3_8b_32k", batch=2)
    a = make_inputs(w)
    b = make_inputs(w)
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    assert torch.equal(a.v_cache.view(torch.int16), b.v_cache.view(torch.int16))
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    c = make_inputs(w.replace(seed=w.seed + 1))
    assert not torch.equal(a.k_cache.view(torch.int16), c.k_cache.view(torch.int16))


def test_query_ar1_process():
    w = WORKLOADS["paged_b32_64k"].replace(steps=4000, batch=1, n_q_heads=8, n_kv_heads=2)
    q = query_stream(w)
    # stationary unit variance and lag-1 correlation rho
    x = q[100:].reshape(q.shape[0] - 100, -1)
    assert abs(x.var() - 1.0) < 0.05
    r = (x[1:] * x[:-1]).mean() / x.var()
    assert abs(r - w.rho) < 0.03


def test_hot_blocks_planted():
    w = _small("llama3_8b_32k", batch=1, n_q_heads=8, n_kv_heads=2)
    inp = make_inputs(w)
    G = w.group
    for g in range(w.n_kv_heads):
        for n in inp.hot[0, g]:
            k = inp.block_keys(0, g, int(n)).float()
            # the bias direction dominates the mean key of a hot block
            mean = k.mean(dim=0).numpy()
            assert mean @ inp.qhat[0, g] > 1.0   # bias 2, noise std 0.25
    # qhat is the unit group-summed first query
    q0 = inp.q[0, 0].float().numpy()
    s = q0[:G].sum(axis=0)
    assert np.allclose(inp.qhat[0, 0], s / np.linalg.norm(s), atol=2e-2)


def test_page_table_permutation():
    w = _small("paged_b32_64k", batch=3)
    t = block_table(w)
    assert t.shape == (3, w.pages_per_seq)
    assert sorted(t.ravel().tolist()) == list(range(w.n_pages))
    assert not np.array_equal(t.ravel(), np.arange(w.n_pages))
    w2 = _small("llama3_8b_32k", batch=2)
    assert np.array_equal(block_table(w2).ravel(), np.arange(w2.n_pages))


def test_bf16_cast_is_round_to_nearest_even():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=torch.float32)
    y = x.to(torch.bfloat16).float()
    assert y.tolist() == [1.0, 1.0 + 2 ** -6, -1.0]


def test_drift_moves_one_block_per_row():
    w = _small("long_ctx_131k_b4", batch=2)
    inp = make_inputs(w)
    before_hot = inp.hot.copy()
    k_before = inp.k_cache.clone()
    assert len(inp.drift(3)) == 0
    changed = inp.drift(4)
    assert len(changed) == 2 * w.batch * w.n_kv_heads
    after = inp.hot
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            assert len(set(before_hot[b, g]) ^ set(after[b, g])) == 2
    # only the keys of the changed blocks moved
    N = w.n_blocks
    moved = set()
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            for n in range(N):
                if not torch.equal(inp.block_keys(b, g, n), _keys(k_before, inp, b, g, n)):
                    moved.add((b * w.n_kv_heads + g) * N + n)
    assert moved == set(changed.tolist())
    # a block that loses the bias gets back exactly its unbiased keys: moving it back and forth is lossless
    inp2 = make_inputs(w)
    for t in (4, 8, 12):
        inp2.drift(t)
    assert len(inp2.saved) == w.batch * w.n_kv_heads * w.hot_blocks


def _keys(cache, inp, b, g, n):
    pages = torch.as_tensor(inp._pages_of_block(b, n), dtype=torch.long)
    return cache[pages, g].reshape(inp.w.block_size, inp.w.head_dim)


def test_bytes_do_not_depend_on_thread_count():
    w = _small("paged_b32_64k", batch=3)
    a = make_inputs(w, threads=1)
    b = make_inputs(w, threads=5)
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    assert torch.equal(a.v_cache.view(torch.int16), b.v_cache.view(torch.int16))


def test_cache_rows_follow_the_host_recipe():
    """Through the page table, each row of the cache is the host draw (bias planted on the hot blocks) cast to the
    storage dtype; slots past the context hold the poison values."""
    from dynamic_sparse_attention_decode_amd import inputs as I
    w = _small("paged_b32_64k", batch=2, hot_blocks=5, ctx=16 * 64 - 7)
    inp = make_inputs(w)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            pages = torch.as_tensor(inp.table_np[b], dtype=torch.long)
            k = inp.k_cache[pages, g].reshape(w.capacity, w.head_dim)
            v = inp.v_cache[pages, g].reshape(w.capacity, w.head_dim)
            kr = I.key_row(w, b, g)
            I.plant_hot(kr, inp.hot[b, g], w.hot_bias * inp.qhat[b, g], w.block_size)
            assert torch.equal(k.view(torch.int16), I.to_storage(kr, w.dtype).view(torch.int16))
            assert torch.equal(v.view(torch.int16), I.to_storage(I.value_row(w, b, g), w.dtype).view(torch.int16))
            # poison past the end (a hot last block carries the bias there too)
            assert torch.all(k[w.ctx:].float() > 45.0) and torch.all(v[w.ctx:].float() > 9000.0)


def test_attempts_redraw_only_their_group_step():
    w = _small("llama3_8b_32k", batch=2, steps=6)
    base = query_stream(w)
    att = np.zeros((w.steps, w.batch, w.n_kv_heads), dtype=np.int64)
    att[3, 1, 5] = 2
    q = query_stream(w, attempts=att)
    G = w.group
    diff = np.argwhere(np.any(q != base, axis=-1))
    assert len(diff) > 0
    for t, b, h in diff:
        assert t >= 3 and b == 1 and h // G == 5, (t, b, h)
    assert np.all(np.any(q[3:, 1, 5 * G:6 * G] != base[3:, 1, 5 * G:6 * G], axis=-1))
    att0 = att.copy()
    att0[0, 0, 2] = 1   # a redrawn first query moves that group's hot-block bias direction too
    inp_a = make_inputs(w.replace(steps=2), attempts=att0[:2])
    inp_b = make_inputs(w.replace(steps=2))
    assert not np.array_equal(inp_a.qhat[0, 2], inp_b.qhat[0, 2])
    assert np.array_equal(inp_a.qhat[0, 1], inp_b.qhat[0, 1])


def test_load_attempts_checks_the_workload(tmp_path):
    import json
    from dynamic_sparse_attention_decode_amd.inputs import load_attempts
    w = _small("tiny_f32_4k", steps=3)
    a = np.arange(3 * w.batch * w.n_kv_heads).reshape(3, w.batch, w.n_kv_heads)
    p = tmp_path / "t.json"
    p.write_text(json.dumps({"workload": w.key(), "shape": list(a.shape), "attempts": a.ravel().tolist()}))
    assert np.array_equal(load_attempts(str(p), w), a)
    assert np.array_equal(load_attempts(str(p), w, steps=2), a[:2])
    with pytest.raises(ValueError):
        load_attempts(str(p), w.replace(seed=1))
    with pytest.raises(ValueError):
        load_attempts(str(p), w.replace(steps=4))
