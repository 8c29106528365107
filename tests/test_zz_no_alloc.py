"""The allocation-free decode step (prr_decode_step_noalloc, the library's static scratch in place of a caller
workspace) against prr_decode_step with a workspace.

GPU: whole decode runs through the C ABI in three modes give the same outputs, selections, predicted sets and
missed counts, bit for bit, as the same runs with a workspace. Three layers run one after the other on the GPU, each
smaller than the one before (the scratch keeps the previous run's contents): rows of 12000 blocks (the scratch's
top-K candidate regions and repair part), a batch of 384 rows (the row-wise repair's part), then a short layer.
Host: a non-NULL workspace and a shape whose workspace exceeds the scratch are rejected before any device call."""
import ctypes

import numpy as np
import pytest
import torch

from dynamic_sparse_attention_decode_amd import _lib as L
from dynamic_sparse_attention_decode_amd.runtime import PRRLayer
from tests.gpu_common import gap_inputs, np64, requires_gpu, shape_of, small


def _layers():
    long_rows = small("million_token").replace(ctx=32 * 12000 - 7, top_k=61, k_spec=(93,), steps=4)
    many_rows = small("paged_b32_64k").replace(batch=48, steps=4)
    short = small("llama3_8b_32k").replace(steps=5)
    return [long_rows, many_rows, short]


def _run(w, inp, mode, static):
    layer = PRRLayer(shape_of(w), w.top_k, max(w.k_spec), w.alpha, mode=mode, static_workspace=static)
    layer.build(inp.k_cache, inp.v_cache, inp.table)
    hist = []
    for t in range(w.steps):
        out = layer.step(inp.q[t].contiguous())
        layer.sync_spec()
        torch.cuda.synchronize()
        hist.append((np64(out), layer.sel_idx.cpu().numpy().copy(), layer.n_missed.cpu().numpy().copy(),
                     layer.pred_next.cpu().numpy().copy() if layer.k_spec else None))
    layer.close()
    return hist


@pytest.mark.gpu
@requires_gpu
@pytest.mark.parametrize("mode", ["prr_fused", "prr_2stream", "serialized"])
def test_noalloc_step_equals_workspace_step(mode):
    for w in _layers():
        print(f"[case] noalloc {mode} B={w.batch} N={w.n_blocks} K={w.top_k} K'={max(w.k_spec)} "
              f"workspace {L.workspace_bytes(shape_of(w), w.top_k)} B", flush=True)
        assert L.workspace_bytes(shape_of(w), w.top_k) <= L.SCRATCH_MAX_BYTES
        inp = gap_inputs(w)
        ref = _run(w, inp, mode, static=False)
        got = _run(w, inp, mode, static=True)
        for t, (a, b) in enumerate(zip(ref, got)):
            assert np.array_equal(a[0], b[0]), (t, np.abs(a[0] - b[0]).max())
            assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]), t
            if a[3] is not None:
                assert np.array_equal(a[3], b[3]), t


def test_noalloc_rejects_before_any_device_call():
    lib = L.lib()
    ptrs = [ctypes.c_void_p(256 * (i + 1)) for i in range(14)]
    s = L.make_shape(1, 32, 8, 128, 16, 16, 2048, L.BF16)
    args = L.StepArgs(*ptrs, 8, 8, 8, 0, 0.9, None)   # a workspace pointer is given: rejected
    assert lib.prr_decode_step_noalloc(None, ctypes.byref(s), ctypes.byref(args), L.MODE_FUSED, 0, None, None) == -1
    big = L.make_shape(16, 64, 8, 128, 32, 32, 32768, L.BF16)   # about 62 MiB of workspace
    assert L.workspace_bytes(big, 256) > L.SCRATCH_MAX_BYTES
    no_ws = list(ptrs)
    no_ws[13] = None
    args = L.StepArgs(*no_ws, 256, 256, 256, 0, 0.9, None)
    assert lib.prr_decode_step_noalloc(None, ctypes.byref(big), ctypes.byref(args), L.MODE_FUSED, 0, None,
                                       None) == -1
    assert b"scratch" in lib.prr_last_error()
    args = L.StepArgs(*no_ws, 0, 8, 8, 0, 0.9, None)   # top_k out of range
    assert lib.prr_decode_step_noalloc(None, ctypes.byref(s), ctypes.byref(args), L.MODE_FUSED, 0, None, None) == -1
