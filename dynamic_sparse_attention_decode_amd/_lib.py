"""ctypes binding of libprr (argument marshalling only; every step of the path runs in the library's kernels).

Each function takes torch tensors (device memory owned by PyTorch), checks device, dtype and contiguity, and passes
raw pointers and the HIP stream handle to the C ABI declared in include/prr.h. Errors raise PRRError with the
library's message. There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libprr.so")

F32, BF16, F16 = 0, 1, 2
SCORER_QUEST, SCORER_MEAN = 0, 1
MODE_SERIALIZED, MODE_ONE_STREAM, MODE_TWO_STREAM, MODE_FUSED, MODE_SERIALIZED_FUSED = 0, 1, 2, 3, 4
_DT_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}

# every entry point of include/prr.h
EXPORTS = ["prr_build_summaries", "prr_append_kv", "prr_score_select", "prr_ema_predict", "prr_speculate", "prr_repair_merge",
           "prr_score", "prr_select_speculate", "prr_score_speculate", "prr_select_repair",
           "prr_partials_bytes", "prr_workspace_bytes", "prr_step_ctx_create", "prr_step_ctx_destroy",
           "prr_step_ctx_set_delays",
           "prr_decode_step", "prr_decode_step_noalloc", "prr_choose_budget", "prr_choose_budget_fused", "prr_trace_create", "prr_trace_destroy", "prr_trace_enable",
           "prr_trace_read", "prr_flush_write", "prr_stream_read", "prr_status_string", "prr_last_error",
           "prr_version"]

KERNELS = {"summaries": 0, "score": 1, "select_topk": 2, "ema_topk": 3, "speculate": 4, "repair": 5, "finalize": 6}


class PRRError(RuntimeError):
    pass


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("n_blocks", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("ctx_len", ctypes.c_int32), ("sink_blocks", ctypes.c_int32),
                ("local_blocks", ctypes.c_int32), ("scorer", ctypes.c_int32)]

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self):
        return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[self.dtype]


BUDGET_FIXED, BUDGET_MISSES, BUDGET_CONFIDENCE = 0, 1, 2


class Budget(ctypes.Structure):
    """prr_budget: a per-row budget of the predicted set (policy BUDGET_MISSES or BUDGET_CONFIDENCE)."""
    _fields_ = [("policy", ctypes.c_int32), ("top_k", ctypes.c_int32), ("k_min", ctypes.c_int32),
                ("beta", ctypes.c_float), ("c", ctypes.c_float), ("missed_prev", ctypes.c_void_p)]


def make_budget(policy: int, top_k: int, k_min: int = 1, beta: float = 0.0, c: float = 0.0, missed_prev=None):
    """A Budget; missed_prev (int32 [B, Hkv] on the device) for BUDGET_MISSES. Keep the returned object (and the
    tensor) alive while calls that use it are pending."""
    mp = _p(missed_prev, torch.int32, "missed_prev")
    b = Budget(policy, top_k, k_min, beta, c, mp.value if mp is not None else None)
    b._keep = missed_prev
    return b


def _b(budget):
    return ctypes.byref(budget) if budget is not None else None


class StepArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("summaries", ctypes.c_void_p), ("scores", ctypes.c_void_p),
                ("sel_idx", ctypes.c_void_p), ("ema", ctypes.c_void_p), ("pred_cur", ctypes.c_void_p),
                ("pred_next", ctypes.c_void_p), ("partials", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("n_missed", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("top_k", ctypes.c_int32),
                ("k_spec_cur", ctypes.c_int32), ("k_spec_next", ctypes.c_int32), ("first_step", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("budget", ctypes.c_void_p)]


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, block_size, page_size, n_blocks, dtype,
               softmax_scale=None, ctx_len=0, sink_blocks=0, local_blocks=0, scorer=0) -> Shape:
    """ctx_len: tokens per sequence when the last block is partly filled (0: n_blocks * block_size); sink_blocks,
    local_blocks: blocks every selection keeps (the first and the last of each sequence); scorer: SCORER_QUEST or
    SCORER_MEAN."""
    if isinstance(dtype, torch.dtype):
        dtype = _DT_CODE[dtype]
    pps = n_blocks * block_size // page_size
    scale = head_dim ** -0.5 if softmax_scale is None else softmax_scale
    return Shape(batch, n_q_heads, n_kv_heads, head_dim, block_size, page_size, n_blocks, pps, dtype, scale, ctx_len,
                 sink_blocks, local_blocks, scorer)


_lib = None


def lib():
    """Load libprr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise PRRError(f"{LIB_PATH} is missing: build it with `python -m dynamic_sparse_attention_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sp = ctypes.POINTER(Shape)
    bp = ctypes.POINTER(Budget)
    sig = {
        "prr_build_summaries": (i32, [sp, vp, vp, vp, i32, vp, vp]),
        "prr_append_kv": (i32, [sp, vp, vp, vp, vp, vp, vp, vp]),
        "prr_score_select": (i32, [sp, vp, vp, i32, vp, vp, vp, vp]),
        "prr_ema_predict": (i32, [sp, vp, vp, f32, i32, i32, vp, bp, vp, vp]),
        "prr_speculate": (i32, [sp, vp, vp, vp, vp, vp, i32, vp, vp]),
        "prr_repair_merge": (i32, [sp, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp]),
        "prr_score": (i32, [sp, vp, vp, vp, vp, f32, i32, vp]),
        "prr_select_speculate": (i32, [sp, vp, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, bp, vp, vp]),
        "prr_score_speculate": (i32, [sp, vp, vp, vp, vp, f32, i32, vp, vp, vp, vp, i32, vp, vp]),
        "prr_select_repair": (i32, [sp, vp, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
        "prr_partials_bytes": (sz, [sp, i32]),
        "prr_workspace_bytes": (sz, [sp, i32]),
        "prr_step_ctx_create": (i32, [ctypes.POINTER(vp)]),
        "prr_step_ctx_destroy": (None, [vp]),
        "prr_step_ctx_set_delays": (i32, [vp, i32, i32]),
        "prr_decode_step": (i32, [vp, sp, ctypes.POINTER(StepArgs), i32, i32, vp, vp]),
        "prr_decode_step_noalloc": (i32, [vp, sp, ctypes.POINTER(StepArgs), i32, i32, vp, vp]),
        "prr_choose_budget": (i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), i32,
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), i32,
                                    ctypes.c_double, i32]),
        "prr_choose_budget_fused": (i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), i32]),
        "prr_trace_create": (i32, [ctypes.POINTER(vp), i32]),
        "prr_trace_destroy": (None, [vp]),
        "prr_trace_enable": (i32, [vp, ctypes.c_uint32]),
        "prr_trace_read": (i32, [vp, i32, ctypes.POINTER(ctypes.c_float), i32]),
        "prr_flush_write": (i32, [vp, sz, vp]),
        "prr_stream_read": (i32, [vp, sz, vp, vp]),
        "prr_status_string": (ctypes.c_char_p, [i32]),
        "prr_last_error": (ctypes.c_char_p, []),
        "prr_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise PRRError(f"{what}: {L.prr_status_string(status).decode()}: {L.prr_last_error().decode()}")


def _p(t: torch.Tensor | None, dtype=None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise PRRError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise PRRError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PRRError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _s(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def build_summaries(shape: Shape, k_cache, block_table, summaries, block_ids=None, stream=None) -> None:
    dt = shape.torch_dtype
    n_ids = 0 if block_ids is None else block_ids.numel()
    _check(lib().prr_build_summaries(ctypes.byref(shape), _p(k_cache, dt, "k_cache"),
                                     _p(block_table, torch.int32, "block_table"),
                                     _p(block_ids, torch.int32, "block_ids"), n_ids, _p(summaries, dt, "summaries"),
                                     _s(stream)), "build_summaries")


def append_kv(shape: Shape, k_new, v_new, k_cache, v_cache, block_table, summaries, stream=None) -> None:
    """Write the token at position shape.ctx_len - 1 (k_new, v_new: [B, Hkv, D]) and update its block's summary."""
    dt = shape.torch_dtype
    _check(lib().prr_append_kv(ctypes.byref(shape), _p(k_new, dt, "k_new"), _p(v_new, dt, "v_new"),
                               _p(k_cache, dt, "k_cache"), _p(v_cache, dt, "v_cache"),
                               _p(block_table, torch.int32, "block_table"), _p(summaries, dt, "summaries"),
                               _s(stream)), "append_kv")


def score_select(shape: Shape, q, summaries, top_k: int, scores, sel_idx, workspace=None, stream=None) -> None:
    dt = shape.torch_dtype
    _check(lib().prr_score_select(ctypes.byref(shape), _p(q, dt, "q"), _p(summaries, dt, "summaries"), top_k,
                                  _p(scores, torch.float32, "scores"), _p(sel_idx, torch.int32, "sel_idx"),
                                  _p(workspace, None, "workspace"), _s(stream)), "score_select")


def ema_predict(shape: Shape, scores, ema, alpha: float, first_step: bool, k_spec: int, pred_idx_next,
                workspace=None, stream=None, budget: Budget | None = None) -> None:
    _check(lib().prr_ema_predict(ctypes.byref(shape), _p(scores, torch.float32, "scores"),
                                 _p(ema, torch.float32, "ema"), alpha, int(bool(first_step)), k_spec,
                                 _p(pred_idx_next, torch.int32, "pred_idx_next"), _b(budget),
                                 _p(workspace, None, "workspace"), _s(stream)), "ema_predict")


def speculate(shape: Shape, q, k_cache, v_cache, block_table, pred_idx, k_spec: int, partials, stream=None) -> None:
    dt = shape.torch_dtype
    _check(lib().prr_speculate(ctypes.byref(shape), _p(q, dt, "q"), _p(k_cache, dt, "k_cache"),
                               _p(v_cache, dt, "v_cache"), _p(block_table, torch.int32, "block_table"),
                               _p(pred_idx, torch.int32, "pred_idx"), k_spec,
                               _p(partials, torch.float32, "partials"), _s(stream)), "speculate")


def repair_merge(shape: Shape, q, k_cache, v_cache, block_table, sel_idx, top_k: int, pred_idx, k_spec: int,
                 partials, out, n_missed, workspace, stream=None) -> None:
    dt = shape.torch_dtype
    _check(lib().prr_repair_merge(ctypes.byref(shape), _p(q, dt, "q"), _p(k_cache, dt, "k_cache"),
                                  _p(v_cache, dt, "v_cache"), _p(block_table, torch.int32, "block_table"),
                                  _p(sel_idx, torch.int32, "sel_idx"), top_k,
                                  _p(pred_idx, torch.int32, "pred_idx"), k_spec,
                                  _p(partials, torch.float32, "partials"), _p(out, torch.float32, "out"),
                                  _p(n_missed, torch.int32, "n_missed"), _p(workspace, None, "workspace"),
                                  _s(stream)), "repair_merge")


def score(shape: Shape, q, summaries, scores, ema=None, alpha: float = 0.0, first_step=False, stream=None) -> None:
    dt = shape.torch_dtype
    _check(lib().prr_score(ctypes.byref(shape), _p(q, dt, "q"), _p(summaries, dt, "summaries"),
                           _p(scores, torch.float32, "scores"), _p(ema, torch.float32, "ema"), alpha,
                           int(bool(first_step)), _s(stream)), "score")


def select_speculate(shape: Shape, scores, top_k: int, sel_idx, ema=None, k_spec_next: int = 0, pred_idx_next=None,
                     q=None, k_cache=None, v_cache=None, block_table=None, pred_idx=None, k_spec: int = 0,
                     partials=None, workspace=None, stream=None, budget: Budget | None = None) -> None:
    dt = shape.torch_dtype
    _check(lib().prr_select_speculate(ctypes.byref(shape), _p(scores, torch.float32, "scores"), top_k,
                                      _p(sel_idx, torch.int32, "sel_idx"), _p(ema, torch.float32, "ema"), k_spec_next,
                                      _p(pred_idx_next, torch.int32, "pred_idx_next"), _p(q, dt, "q"),
                                      _p(k_cache, dt, "k_cache"), _p(v_cache, dt, "v_cache"),
                                      _p(block_table, torch.int32, "block_table"), _p(pred_idx, torch.int32, "pred_idx"),
                                      k_spec, _p(partials, torch.float32, "partials"), _b(budget),
                                      _p(workspace, None, "workspace"), _s(stream)), "select_speculate")


def score_speculate(shape: Shape, q, summaries, scores, ema=None, alpha: float = 0.0, first_step=False,
                    k_cache=None, v_cache=None, block_table=None, pred_idx=None, k_spec: int = 0, partials=None,
                    stream=None) -> None:
    dt = shape.torch_dtype
    _check(lib().prr_score_speculate(ctypes.byref(shape), _p(q, dt, "q"), _p(summaries, dt, "summaries"),
                                     _p(scores, torch.float32, "scores"), _p(ema, torch.float32, "ema"), alpha,
                                     int(bool(first_step)), _p(k_cache, dt, "k_cache"), _p(v_cache, dt, "v_cache"),
                                     _p(block_table, torch.int32, "block_table"), _p(pred_idx, torch.int32, "pred_idx"),
                                     k_spec, _p(partials, torch.float32, "partials"), _s(stream)), "score_speculate")


def select_repair(shape: Shape, scores, top_k: int, sel_idx, q, k_cache, v_cache, block_table, out, n_missed,
                  workspace, ema=None, k_spec_next: int = 0, pred_idx_next=None, pred_idx=None, k_spec: int = 0,
                  partials=None, stream=None) -> None:
    dt = shape.torch_dtype
    _check(lib().prr_select_repair(ctypes.byref(shape), _p(scores, torch.float32, "scores"), top_k,
                                   _p(sel_idx, torch.int32, "sel_idx"), _p(ema, torch.float32, "ema"), k_spec_next,
                                   _p(pred_idx_next, torch.int32, "pred_idx_next"), _p(q, dt, "q"),
                                   _p(k_cache, dt, "k_cache"), _p(v_cache, dt, "v_cache"),
                                   _p(block_table, torch.int32, "block_table"), _p(pred_idx, torch.int32, "pred_idx"),
                                   k_spec, _p(partials, torch.float32, "partials"), _p(out, torch.float32, "out"),
                                   _p(n_missed, torch.int32, "n_missed"), _p(workspace, None, "workspace"),
                                   _s(stream)), "select_repair")


def partials_bytes(shape: Shape, k_spec: int) -> int:
    return int(lib().prr_partials_bytes(ctypes.byref(shape), k_spec))


def workspace_bytes(shape: Shape, top_k: int) -> int:
    return int(lib().prr_workspace_bytes(ctypes.byref(shape), top_k))


def step_ctx_create() -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().prr_step_ctx_create(ctypes.byref(h)), "step_ctx_create")
    return h


def step_ctx_destroy(h) -> None:
    lib().prr_step_ctx_destroy(h)


def decode_step(ctx, shape: Shape, args: StepArgs, mode: int, join: bool, stream_sel, stream_spec) -> None:
    _check(lib().prr_decode_step(ctx, ctypes.byref(shape), ctypes.byref(args), mode, int(bool(join)),
                                 _s(stream_sel), _s(stream_spec)), "decode_step")


def step_ctx_set_delays(ctx, delay_sel: int, delay_spec: int) -> None:
    """Race check: sleep iterations before the repair (stream_sel) and before the speculation (stream_spec)."""
    _check(lib().prr_step_ctx_set_delays(ctx, int(delay_sel), int(delay_spec)), "step_ctx_set_delays")


def decode_step_noalloc(ctx, shape: Shape, args: StepArgs, mode: int, join: bool, stream_sel, stream_spec) -> None:
    """prr_decode_step with the library's static scratch as the workspace (args.workspace must be None)."""
    _check(lib().prr_decode_step_noalloc(ctx, ctypes.byref(shape), ctypes.byref(args), mode, int(bool(join)),
                                         _s(stream_sel), _s(stream_spec)), "decode_step_noalloc")


SCRATCH_MAX_BYTES = 32 << 20   # PRR_SCRATCH_MAX_BYTES in include/prr.h


def choose_budget_fused(kspec_grid, t_step) -> int:
    """The fused step's budget from measured step times at each grid budget (the grid holds 0)."""
    D = ctypes.c_double
    if len(kspec_grid) != len(t_step):
        raise PRRError("choose_budget_fused: kspec_grid and t_step differ in length")
    r = lib().prr_choose_budget_fused((D * len(kspec_grid))(*kspec_grid), (D * len(t_step))(*t_step),
                                      len(kspec_grid))
    if r < 0:
        raise PRRError("choose_budget_fused: invalid arguments (the grid must hold 0; times must be finite)")
    return r


def choose_budget(n_grid, t_sel, kspec_grid, t_spec, n_target: float, degree: int = 2) -> int:
    D = ctypes.c_double
    a = (D * len(n_grid))(*n_grid)
    b = (D * len(t_sel))(*t_sel)
    c = (D * len(kspec_grid))(*kspec_grid)
    d = (D * len(t_spec))(*t_spec)
    r = lib().prr_choose_budget(a, b, len(n_grid), c, d, len(kspec_grid), float(n_target), degree)
    if r < 0:
        raise PRRError("choose_budget: invalid arguments")
    return int(r)


class Trace:
    """Per-kernel launch timing (HIP events on each kernel's own stream); see prr_trace_* in include/prr.h."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.h = ctypes.c_void_p()
        _check(lib().prr_trace_create(ctypes.byref(self.h), capacity), "trace_create")

    def enable(self, kernels) -> None:
        mask = 0
        for k in kernels:
            mask |= 1 << KERNELS[k]
        _check(lib().prr_trace_enable(self.h, mask), "trace_enable")

    def disable(self) -> None:
        lib().prr_trace_enable(None, 0)

    def read(self, kernel: str) -> list:
        buf = (ctypes.c_float * self.capacity)()
        n = lib().prr_trace_read(self.h, KERNELS[kernel], buf, self.capacity)
        if n < 0:
            _check(n, "trace_read")
        return [float(buf[i]) for i in range(n)]

    def close(self) -> None:
        if self.h:
            lib().prr_trace_destroy(self.h)
            self.h = ctypes.c_void_p()


def flush_write(buf, stream=None) -> None:
    _check(lib().prr_flush_write(_p(buf, None, "buf"), buf.numel() * buf.element_size(), _s(stream)), "flush_write")


def stream_read(buf, sink, stream=None) -> None:
    _check(lib().prr_stream_read(_p(buf, None, "buf"), buf.numel() * buf.element_size(),
                                 _p(sink, torch.float32, "sink"), _s(stream)), "stream_read")


def version() -> str:
    return lib().prr_version().decode()
