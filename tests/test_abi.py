"""The C-ABI library loads, exports every entry point that include/prr.h declares, and validates arguments on the host
(no device call is made: these run without a GPU)."""
import ctypes
import os
import re

import pytest

from dynamic_sparse_attention_decode_amd import _lib as L
from oracle import prr_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "prr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(prr_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    declared = _declared()
    assert set(declared) == set(L.EXPORTS), (set(declared) ^ set(L.EXPORTS))
    for name in declared:
        assert hasattr(lib, name), name
    assert L.version().startswith("libprr")


def _shape(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=16, page_size=16, n_blocks=2048,
                dtype=L.BF16)
    base.update(kw)
    return L.make_shape(**base)


def _status(fn, *args):
    return fn(*args)


@pytest.mark.parametrize("bad,code", [
    (dict(n_q_heads=30), L.lib and -1),           # Hq % Hkv != 0
    (dict(n_q_heads=24, n_kv_heads=2), -2),       # G = 12 unsupported
    (dict(head_dim=64), -2),                      # bf16 x 64 unsupported
    (dict(dtype=L.F32), -2),                      # f32 x 128 unsupported
    (dict(dtype=7), -1),                          # unknown dtype
    (dict(block_size=18, page_size=2), -2),       # block_size % 4 != 0
    (dict(block_size=16, page_size=32), -1),      # block_size % page_size != 0
    (dict(n_blocks=0), -1),
    (dict(n_blocks=40000), -2),                   # top-K kernels support N <= 32768
    (dict(ctx_len=2047 * 16), -1),                # ctx_len must end inside the last block
    (dict(ctx_len=2048 * 16 + 1), -1),
])
def test_shape_validation(bad, code):
    lib = L.lib()
    s = _shape(**bad)
    nz = ctypes.c_void_p(16)
    st = lib.prr_score_select(ctypes.byref(s), nz, nz, 8, nz, nz, None, None)
    assert st == code, (bad, st, lib.prr_last_error())
    assert lib.prr_last_error()


def test_append_validation_without_launch():
    lib = L.lib()
    nz = ctypes.c_void_p(16)
    s = _shape(ctx_len=2047 * 16 + 5)
    assert lib.prr_append_kv(ctypes.byref(s), None, nz, nz, nz, nz, nz, None) == -1       # null k_new
    assert lib.prr_append_kv(ctypes.byref(s), nz, nz, nz, nz, nz, None, None) == -1       # null summaries
    bad = _shape(ctx_len=2047 * 16)
    assert lib.prr_append_kv(ctypes.byref(bad), nz, nz, nz, nz, nz, nz, None) == -1       # ctx_len out of range


def test_argument_validation_without_launch():
    lib = L.lib()
    s = _shape()
    nz = ctypes.c_void_p(16)
    assert lib.prr_score_select(ctypes.byref(s), None, nz, 8, nz, nz, None, None) == -1          # null q
    assert lib.prr_score_select(ctypes.byref(s), nz, nz, 0, nz, nz, None, None) == -1            # K < 1
    assert lib.prr_score_select(ctypes.byref(s), nz, nz, 2049, nz, nz, None, None) == -1         # K > N
    assert lib.prr_score(ctypes.byref(s), nz, None, nz, None, 0.5, 0, None) == -1         # null summaries
    assert lib.prr_score(ctypes.byref(s), nz, nz, nz, nz, -0.5, 0, None) == -1            # alpha < 0 with an EMA
    # select_speculate: prediction needs the EMA; speculation needs its buffers; P_t and P_{t+1} buffers differ
    assert lib.prr_select_speculate(ctypes.byref(s), nz, 8, nz, None, 8, nz, None, None, None, None, None, 0, None,
                                    None, None, None) == -1
    assert lib.prr_select_speculate(ctypes.byref(s), nz, 8, nz, None, 0, None, nz, None, nz, nz, nz, 4, nz,
                                    None, None, None) == -1
    assert lib.prr_select_speculate(ctypes.byref(s), nz, 8, nz, nz, 8, nz, nz, nz, nz, nz, nz, 8, nz, None, None,
                                    None) == -1
    # select_repair: argument checks, then the supported-shape rule (page size multiple of 16, K <= 2048)
    assert lib.prr_select_repair(ctypes.byref(s), nz, 8, nz, None, 0, None, nz, nz, nz, nz, None, 4, None, nz, nz,
                                 nz, None) == -1                                              # k_spec > 0, no P
    assert lib.prr_select_repair(ctypes.byref(s), nz, 8, nz, None, 0, None, nz, nz, nz, nz, None, 0, None, nz, nz,
                                 None, None) == -1                                            # no workspace
    s8 = _shape(block_size=16, page_size=8, n_blocks=2048)
    assert lib.prr_select_repair(ctypes.byref(s8), nz, 8, nz, None, 0, None, nz, nz, nz, nz, None, 0, None, nz, nz,
                                 nz, None) == -2                                              # page 8: unsupported
    s4 = _shape(n_blocks=4096)
    assert lib.prr_select_repair(ctypes.byref(s4), nz, 2049, nz, None, 0, None, nz, nz, nz, nz, None, 0, None, nz,
                                 nz, nz, None) == -2                                          # K > 2048
    assert lib.prr_score_speculate(ctypes.byref(s), nz, nz, nz, None, 0.5, 0, None, None, None, None, 4, None,
                                   None) == -1                                                # k_spec > 0, no KV
    assert lib.prr_ema_predict(ctypes.byref(s), nz, nz, 0.9, 0, 0, nz, None, None, None) == -1   # K' < 1
    assert lib.prr_ema_predict(ctypes.byref(s), nz, nz, 1.5, 0, 8, nz, None, None, None) == -1   # alpha > 1
    # per-row budgets: policy, K, k_min, beta / c and the missed counts are checked before any launch
    for bad in (L.Budget(7, 8, 1, 0.5, 0.0, 16), L.Budget(L.BUDGET_MISSES, 0, 1, 0.5, 0.0, 16),
                L.Budget(L.BUDGET_MISSES, 8, 0, 0.5, 0.0, 16), L.Budget(L.BUDGET_MISSES, 8, 9, 0.5, 0.0, 16),
                L.Budget(L.BUDGET_MISSES, 8, 1, -0.5, 0.0, 16), L.Budget(L.BUDGET_MISSES, 8, 1, float("nan"), 0.0, 16),
                L.Budget(L.BUDGET_MISSES, 8, 1, 0.5, 0.0, None), L.Budget(L.BUDGET_CONFIDENCE, 8, 1, 0.0, -1.0, None),
                L.Budget(L.BUDGET_CONFIDENCE, 8, 1, 0.0, float("inf"), None),
                L.Budget(L.BUDGET_CONFIDENCE, s.n_blocks + 1, 1, 0.0, 1.0, None)):
        assert lib.prr_ema_predict(ctypes.byref(s), nz, nz, 0.9, 0, 8, nz, ctypes.byref(bad), None, None) == -1, bad
        assert lib.prr_select_speculate(ctypes.byref(s), nz, 8, nz, nz, 8, nz, None, None, None, None, None, 0, None,
                                        ctypes.byref(bad), None, None) == -1, bad
    assert lib.prr_speculate(ctypes.byref(s), nz, nz, nz, nz, nz, -1, nz, None) == -1      # K' < 0
    assert lib.prr_speculate(ctypes.byref(s), None, None, None, None, None, 0, None, None) == 0   # K' = 0: no-op
    assert lib.prr_repair_merge(ctypes.byref(s), nz, nz, nz, nz, nz, 8, None, 4, None, nz, nz, nz, None) == -1
    assert lib.prr_build_summaries(None, nz, nz, None, 0, nz, None) == -1
    assert lib.prr_decode_step(None, ctypes.byref(s), None, 2, 0, None, None) == -1
    # a decode step checks its budget before any launch (also on the two-launch path), and its K against the step's
    for bad in (L.Budget(L.BUDGET_MISSES, 8, 0, 0.5, 0.0, 16), L.Budget(L.BUDGET_MISSES, 8, 1, 0.5, 0.0, None),
                L.Budget(L.BUDGET_CONFIDENCE, 9, 1, 0.0, 1.0, None)):
        args = L.StepArgs(nz, nz, nz, nz, nz, nz, nz, nz, nz, nz, nz, nz, nz, nz, 8, 8, 8, 0, 0.9,
                          ctypes.addressof(bad))
        for mode in (L.MODE_FUSED, L.MODE_ONE_STREAM):
            assert lib.prr_decode_step(None, ctypes.byref(s), ctypes.byref(args), mode, 0, None, None) == -1, bad
    # top_k and the budgets of P_t and P_{t+1} are checked before any launch in every mode, including the fused
    # two-launch path (B * Hkv >= 128): a rejected call has enqueued nothing, so the EMA is left as it was. Distinct
    # non-null pointers, so that only the value under test is wrong (no call here may reach a launch).
    ptrs = [ctypes.c_void_p(256 * (i + 1)) for i in range(14)]
    s_many = _shape(batch=16, n_blocks=2048)
    for shp in (s, s_many):
        n = shp.n_blocks
        for top_k, kc, kn in ((0, 8, 8), (-1, 8, 8), (n + 1, 8, 8), (8, n + 1, 8), (8, 8, n + 1), (8, -1, 8)):
            args = L.StepArgs(*ptrs, top_k, kc, kn, 0, 0.9, None)
            bad_k = top_k < 1 or top_k > n
            for mode in (L.MODE_FUSED, L.MODE_ONE_STREAM, L.MODE_SERIALIZED, L.MODE_SERIALIZED_FUSED):
                if not bad_k and mode in (L.MODE_SERIALIZED, L.MODE_SERIALIZED_FUSED):
                    continue   # the serialized modes ignore both budgets: this call would be valid
                st = lib.prr_decode_step(None, ctypes.byref(shp), ctypes.byref(args), mode, 0, None, None)
                assert st == -1, (shp.batch, top_k, kc, kn, mode, st, lib.prr_last_error())
    # each null buffer, equal P_t and P_{t+1} buffers, and alpha outside [0, 1] are rejected before the scoring launch
    for i in range(14):
        bad = list(ptrs)
        bad[i] = None
        args = L.StepArgs(*bad, 8, 8, 8, 0, 0.9, None)
        assert lib.prr_decode_step(None, ctypes.byref(s_many), ctypes.byref(args), L.MODE_FUSED, 0, None,
                                   None) == -1, i
    same = list(ptrs)
    same[9] = same[8]   # pred_next = pred_cur
    args = L.StepArgs(*same, 8, 8, 8, 0, 0.9, None)
    assert lib.prr_decode_step(None, ctypes.byref(s_many), ctypes.byref(args), L.MODE_FUSED, 0, None, None) == -1
    args = L.StepArgs(*ptrs, 8, 8, 8, 0, 1.5, None)
    assert lib.prr_decode_step(None, ctypes.byref(s_many), ctypes.byref(args), L.MODE_FUSED, 0, None, None) == -1
    assert lib.prr_flush_write(nz, 17, None) == -1
    assert b"null" in lib.prr_status_string(-1).lower() or lib.prr_status_string(-1)


def test_buffer_sizes():
    """Speculation records: m[G] and l[G] fp32 padded to 16 bytes, then O[G][D] in bf16 for 16-bit storage and in
    fp32 for fp32 storage."""
    s = _shape()
    G, D = 4, 128
    ml = (2 * G + 3) // 4 * 4
    assert L.partials_bytes(s, 160) == 1 * 8 * 160 * (ml * 4 + G * D * 2)
    assert L.partials_bytes(s, 0) == 0
    assert L.workspace_bytes(s, 128) > 0
    s1 = _shape(n_q_heads=8, n_kv_heads=8)   # G = 1: m and l padded to 16 bytes
    assert L.partials_bytes(s1, 3) == 8 * 3 * (16 + 128 * 2)
    s2 = _shape(n_q_heads=4, n_kv_heads=1, head_dim=64, dtype=L.F32, block_size=32, page_size=32, n_blocks=128)
    assert L.partials_bytes(s2, 16) == 16 * (ml * 4 + 4 * 64 * 4)


def test_budget_chooser_matches_oracle_and_closed_forms():
    n_grid = [256, 512, 2048, 4096, 8192]
    ks = [0, 64, 128, 192, 256, 320, 384]
    t_spec = [1 + 0.05 * k for k in ks]
    t_lin = [2 + 0.01 * n for n in n_grid]
    t_quad = [1 + n * n / 1e6 for n in n_grid]
    assert L.choose_budget(n_grid, t_lin, ks, t_spec, 1000) == 192
    assert L.choose_budget(n_grid, t_lin, ks, t_spec, 4096) == 384
    assert L.choose_budget(n_grid, t_quad, ks, t_spec, 3000) == 128
    assert L.choose_budget(n_grid, t_lin, ks, [100.0] * len(ks), 1000) == 0
    import numpy as np
    rng = np.random.default_rng(5)
    for _ in range(50):
        ts = sorted(rng.uniform(1, 50, size=5))
        tp = sorted(rng.uniform(0, 60, size=len(ks)))
        nt = float(rng.uniform(100, 9000))
        for deg in (1, 2, 3):
            a = L.choose_budget(n_grid, ts, ks, tp, nt, deg)
            b = O.choose_budget(n_grid, ts, ks, tp, nt, deg)
            if a != b:   # only a near-tie between fitted time and a table entry may differ
                tt = np.polyval(np.polyfit(n_grid, ts, deg), nt)
                k = max(a, b)
                assert abs(tp[ks.index(k)] - tt) < 1e-9 * max(1, abs(tt))


def test_fused_budget_chooser_matches_oracle():
    ks = [0, 32, 64, 128, 192]
    assert L.choose_budget_fused(ks, [20.0, 19.0, 19.5, 20.0, 21.0]) == 128
    assert L.choose_budget_fused(ks, [20.0, 20.1, 21.0, 22.0, 25.0]) == 0
    import numpy as np
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        grid = sorted(set([0] + [int(x) for x in rng.integers(1, 512, size=n)]))
        rng.shuffle(grid)
        t = [float(x) for x in np.round(rng.uniform(10, 20, size=len(grid)), 1)]   # rounded: exact ties occur
        assert L.choose_budget_fused(grid, t) == O.choose_budget_fused(grid, t), (grid, t)
    lib = L.lib()
    D = ctypes.c_double
    assert lib.prr_choose_budget_fused((D * 2)(32, 64), (D * 2)(1.0, 2.0), 2) == -1            # no zero entry
    assert lib.prr_choose_budget_fused((D * 2)(0, 64), (D * 2)(1.0, float("nan")), 2) == -1     # non-finite time
    assert lib.prr_choose_budget_fused(None, None, 0) == -1


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of prr_shape, prr_budget and prr_step_args have the C header's size and field offsets
    (a C program built with the host compiler against include/prr.h prints them)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"prr_shape": L.Shape, "prr_budget": L.Budget, "prr_step_args": L.StepArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "prr.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            parts = line.split()
            got[tuple(parts[:-1])] = int(parts[-1])
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)
