// C ABI of libprr: argument validation, launch configuration, the two-stream decode step, and status strings.
// Every check happens on the host before any launch; nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <new>

#include "prr_device.h"
#include "prr_launch.h"

namespace prr {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

prr_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return PRR_ELAUNCH;
  }
  return PRR_OK;
}

// ---- kernel tracing ------------------------------------------------------------------------------------------------

}  // namespace prr

struct prr_trace {
  int32_t capacity = 0;
  uint32_t mask = 0;
  char failure[256] = "";   // first failed record (tracing never changes the status of a launch)
  int32_t count[PRR_KERNEL_COUNT] = {};
  hipEvent_t* ev0[PRR_KERNEL_COUNT] = {};
  hipEvent_t* ev1[PRR_KERNEL_COUNT] = {};
};

namespace prr {

static std::atomic<prr_trace*> g_trace{nullptr};

// Under stream capture the record becomes an external event node of the graph, so every replay records it. A
// failed record is noted on the trace and cleared from HIP's last-error state.
static void record(prr_trace* t, hipEvent_t e, hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t err = hipStreamIsCapturing(stream, &cs);
  if (err == hipSuccess)
    err = cs == hipStreamCaptureStatusActive ? hipEventRecordWithFlags(e, stream, hipEventRecordExternal)
                                             : hipEventRecord(e, stream);
  if (err != hipSuccess) {
    if (!t->failure[0])
      snprintf(t->failure, sizeof(t->failure), "event record failed (capture status %d): %s", (int)cs,
               hipGetErrorString(err));
    (void)hipGetLastError();
  }
}

void trace_begin(int kid, hipStream_t stream) {
  prr_trace* t = g_trace.load(std::memory_order_acquire);
  if (!t || !(t->mask & (1u << kid)) || t->count[kid] >= t->capacity) return;
  record(t, t->ev0[kid][t->count[kid]], stream);
}

void trace_end(int kid, hipStream_t stream) {
  prr_trace* t = g_trace.load(std::memory_order_acquire);
  if (!t || !(t->mask & (1u << kid)) || t->count[kid] >= t->capacity) return;
  record(t, t->ev1[kid][t->count[kid]], stream);
  ++t->count[kid];
}

// ---- benchmark helper kernels ------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void flush_kernel(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, (uint32_t)i, 0u, 0u);
}

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                          float* __restrict__ sink) {
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = __uint_as_float(red[0] & 0x007fffffu);   // finite value
}

prr_status launch_flush(void* buf, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return PRR_OK;
  const int64_t blocks = (n16 + 255) / 256;
  flush_kernel<<<dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0, stream>>>(static_cast<uint4*>(buf),
                                                                                            n16);
  return check_launch("flush_write");
}

prr_status launch_stream_read(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return PRR_OK;
  const int64_t blocks = (n16 + 255) / 256;
  stream_read_kernel<<<dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(buf), n16, sink);
  return check_launch("stream_read");
}

// ---- validation ------------------------------------------------------------------------------------------------------

static prr_status check_shape(const prr_shape* s) {
  if (!s) { set_error("shape is NULL"); return PRR_EINVAL; }
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->head_dim < 1 || s->block_size < 1 ||
      s->page_size < 1 || s->n_blocks < 1 || s->pages_per_seq < 1) {
    set_error("shape has a non-positive size");
    return PRR_EINVAL;
  }
  if (s->n_q_heads % s->n_kv_heads) { set_error("n_q_heads %% n_kv_heads != 0"); return PRR_EINVAL; }
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) { set_error("group size %d not in {1,2,4,8}", G); return PRR_EUNSUPPORTED; }
  if (s->dtype != kF32 && s->dtype != kBF16 && s->dtype != kF16) { set_error("unknown dtype %d", s->dtype); return PRR_EINVAL; }
  const bool row256 = (s->dtype == kF32 && s->head_dim == 64) || (s->dtype != kF32 && s->head_dim == 128);
  if (!row256) {
    set_error("unsupported dtype/head_dim combination (%d, %d): need f32 x 64 or bf16/f16 x 128", s->dtype,
              s->head_dim);
    return PRR_EUNSUPPORTED;
  }
  if (s->block_size % 4) { set_error("block_size %% 4 != 0"); return PRR_EUNSUPPORTED; }
  if (s->block_size % s->page_size) { set_error("block_size %% page_size != 0"); return PRR_EINVAL; }
  if ((int64_t)s->pages_per_seq * s->page_size != (int64_t)s->n_blocks * s->block_size) {
    set_error("pages_per_seq * page_size != n_blocks * block_size");
    return PRR_EINVAL;
  }
  if (s->n_blocks > 65536) { set_error("n_blocks > 65536"); return PRR_EUNSUPPORTED; }
  if (s->ctx_len != 0 && ((int64_t)s->ctx_len <= (int64_t)(s->n_blocks - 1) * s->block_size ||
                           (int64_t)s->ctx_len > (int64_t)s->n_blocks * s->block_size)) {
    set_error("ctx_len %d not in ((n_blocks - 1) * block_size, n_blocks * block_size]", s->ctx_len);
    return PRR_EINVAL;
  }
  if (s->scorer != 0 && s->scorer != 1) { set_error("unknown scorer %d", s->scorer); return PRR_EINVAL; }
  if (s->sink_blocks < 0 || s->local_blocks < 0 || (int64_t)s->sink_blocks + s->local_blocks > s->n_blocks) {
    set_error("sink_blocks %d, local_blocks %d: need both >= 0 and their sum <= n_blocks", s->sink_blocks,
              s->local_blocks);
    return PRR_EINVAL;
  }
  if (!(s->softmax_scale > 0.f) || !isfinite(s->softmax_scale)) {
    set_error("softmax_scale must be finite and > 0");
    return PRR_EINVAL;
  }
  return PRR_OK;
}

#define PRR_REQUIRE(cond, ...)            \
  do {                                    \
    if (!(cond)) {                        \
      set_error(__VA_ARGS__);             \
      return PRR_EINVAL;                  \
    }                                     \
  } while (0)

#define PRR_TRY(expr)                  \
  do {                                 \
    const prr_status st_ = (expr);     \
    if (st_ != PRR_OK) return st_;     \
  } while (0)

static prr_status check_topk_n(const prr_shape* s) {
  if (s->n_blocks > 32768) { set_error("n_blocks > 32768 is not supported by the top-K kernels"); return PRR_EUNSUPPORTED; }
  return PRR_OK;
}

static inline hipStream_t as_stream(void* p) { return static_cast<hipStream_t>(p); }

// A budget for a predicted set of k_spec slots (NULL or PRR_BUDGET_FIXED: nothing to check).
static prr_status check_budget(const prr_shape* s, const prr_budget* b, int k_spec, const char* who) {
  if (!b || b->policy == PRR_BUDGET_FIXED) return PRR_OK;
  PRR_REQUIRE(b->policy == PRR_BUDGET_MISSES || b->policy == PRR_BUDGET_CONFIDENCE, "%s: unknown budget policy %d",
              who, b->policy);
  PRR_REQUIRE(b->top_k >= 1 && b->top_k <= s->n_blocks, "%s: budget top_k %d not in [1, %d]", who, b->top_k,
              s->n_blocks);
  PRR_REQUIRE(b->k_min >= 1 && b->k_min <= k_spec, "%s: budget k_min %d not in [1, %d]", who, b->k_min, k_spec);
  if (b->policy == PRR_BUDGET_MISSES) {
    PRR_REQUIRE(std::isfinite(b->beta) && b->beta >= 0.f, "%s: budget beta must be finite and >= 0", who);
    PRR_REQUIRE(b->missed_prev, "%s: the misses budget needs missed_prev", who);
  } else {
    PRR_REQUIRE(std::isfinite(b->c) && b->c >= 0.f, "%s: budget c must be finite and >= 0", who);
  }
  return PRR_OK;
}

}  // namespace prr

using namespace prr;

struct prr_step_ctx {
  hipEvent_t q_ready, spec_done;   // the fork and the join of the two-stream step
  int32_t delay_sel = 0, delay_spec = 0;   // race check: sleep iterations before the repair / the speculation
};

// A bounded sleep of `iters` s_sleep(127) instructions (about 8000 shader clocks each) by one wave: a kernel that
// only takes time, for checking that results do not depend on the timing of the two streams.
__global__ __launch_bounds__(64) void delay_kernel(int32_t iters) {
  for (int32_t i = 0; i < iters; ++i) __builtin_amdgcn_s_sleep(127);
}

static prr_status launch_delay(int32_t iters, hipStream_t st) {
  delay_kernel<<<dim3(1), dim3(64), 0, st>>>(iters);
  return check_launch("step delay");
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- the allocation-free step's scratch ------------------------------------------------------------------------------
// A file-scope device array stands in for the caller's workspace in prr_decode_step_noalloc. Each GPU the library
// runs on holds its own copy (module-load time, until the process ends). In host code its name is only a host-side
// stand-in: the device address comes from hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever passed to kernels. The workspace needs no initialisation, so nothing is cleared.
constexpr size_t kScratchBytes = (size_t)PRR_SCRATCH_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mu;

// The scratch's device address for the device of `stream` (the null stream: the current device), which must be the
// current device.
static prr_status scratch_of_stream(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) {
    set_error("decode_step_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    (void)hipGetLastError();
    return PRR_ELAUNCH;
  }
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) {
      set_error("decode_step_noalloc: hipStreamGetDevice: %s", hipGetErrorString(e));
      (void)hipGetLastError();
      return PRR_ELAUNCH;
    }
  }
  PRR_REQUIRE(dev == cur, "decode_step_noalloc: the stream is on device %d, make it current (device %d is)", dev, cur);
  PRR_REQUIRE(dev >= 0 && dev < kMaxDevices, "decode_step_noalloc: device %d out of range", dev);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        set_error("decode_step_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        (void)hipGetLastError();
        return PRR_ELAUNCH;
      }
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PRR_OK;
}

static prr_status decode_step_impl(prr_step_ctx* ctx, const prr_shape* shape, const prr_step_args* a, int32_t mode,
                                   int32_t join, void* stream_sel, void* stream_spec);

// The workspace: three top-K candidate regions for long rows (the true set's, the predicted set's, and the
// optimistic scores' of a confidence budget), then the repair's part (spread-out or row-wise repair). The parts are
// disjoint, so the true-set selection, the predicted-set selection and the repair may run at once.
static size_t cand_part_bytes(const prr_shape& s) { return round256(topk_cand_bytes(s)); }

static void* cand_region(const prr_shape& s, void* ws, int which) {
  if (!ws || topk_cand_bytes(s) == 0) return nullptr;
  return static_cast<char*>(ws) + (size_t)which * cand_part_bytes(s);
}

static void* repair_ws(const prr_shape& s, void* ws) { return static_cast<char*>(ws) + 3 * cand_part_bytes(s); }

extern "C" {

prr_status prr_build_summaries(const prr_shape* shape, const void* k_cache, const int32_t* block_table,
                               const int32_t* block_ids, int32_t n_block_ids, void* summaries, void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(k_cache && block_table && summaries, "build_summaries: null pointer");
  int64_t jobs = (int64_t)shape->batch * shape->n_kv_heads * shape->n_blocks;
  if (block_ids) {
    PRR_REQUIRE(n_block_ids >= 0, "build_summaries: n_block_ids < 0");
    jobs = n_block_ids;
  }
  return launch_summaries(*shape, k_cache, block_table, block_ids, jobs, summaries, as_stream(stream));
}

prr_status prr_append_kv(const prr_shape* shape, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* block_table, void* summaries, void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(k_new && v_new && k_cache && v_cache && block_table && summaries, "append_kv: null pointer");
  return launch_append(*shape, k_new, v_new, k_cache, v_cache, block_table, summaries, as_stream(stream));
}

prr_status prr_score_select(const prr_shape* shape, const void* q, const void* summaries, int32_t top_k,
                            float* scores, int32_t* sel_idx, void* workspace, void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_TRY(check_topk_n(shape));
  PRR_REQUIRE(q && summaries && scores && sel_idx, "score_select: null pointer");
  PRR_REQUIRE(top_k >= 1 && top_k <= shape->n_blocks, "score_select: top_k %d not in [1, %d]", top_k,
              shape->n_blocks);
  PRR_TRY(launch_score(*shape, q, summaries, scores, nullptr, 0.f, 0, as_stream(stream)));
  return launch_topk(*shape, scores, nullptr, 0.f, 0, top_k, sel_idx, as_stream(stream),
                     cand_region(*shape, workspace, 0));
}

prr_status prr_ema_predict(const prr_shape* shape, const float* scores, float* ema, float alpha, int32_t first_step,
                           int32_t k_spec, int32_t* pred_idx_next, const prr_budget* budget, void* workspace,
                           void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_TRY(check_topk_n(shape));
  PRR_REQUIRE(scores && ema && pred_idx_next, "ema_predict: null pointer");
  PRR_REQUIRE(k_spec >= 1 && k_spec <= shape->n_blocks, "ema_predict: k_spec %d not in [1, %d]", k_spec,
              shape->n_blocks);
  PRR_REQUIRE(alpha >= 0.f && alpha <= 1.f, "ema_predict: alpha not in [0, 1]");
  PRR_TRY(check_budget(shape, budget, k_spec, "ema_predict"));
  const BudgetDev bp = budget_dev(budget);
  if (bp.policy != 0)
    return launch_predict_budget(*shape, scores, ema, alpha, first_step ? 1 : 0, k_spec, bp, pred_idx_next, true,
                                 as_stream(stream));
  return launch_topk(*shape, scores, ema, alpha, first_step ? 1 : 0, k_spec, pred_idx_next, as_stream(stream),
                     cand_region(*shape, workspace, 1));
}

prr_status prr_speculate(const prr_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* pred_idx, int32_t k_spec, float* partials,
                         void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(k_spec >= 0 && k_spec <= shape->n_blocks, "speculate: k_spec %d not in [0, %d]", k_spec,
              shape->n_blocks);
  if (k_spec == 0) return PRR_OK;
  PRR_REQUIRE(q && k_cache && v_cache && block_table && pred_idx && partials, "speculate: null pointer");
  return launch_speculate(*shape, q, k_cache, v_cache, block_table, pred_idx, k_spec, partials, as_stream(stream));
}

prr_status prr_repair_merge(const prr_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* sel_idx, int32_t top_k,
                            const int32_t* pred_idx, int32_t k_spec, const float* partials, float* out,
                            int32_t* n_missed, void* workspace, void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(q && k_cache && v_cache && block_table && sel_idx && out && n_missed && workspace,
              "repair_merge: null pointer");
  PRR_REQUIRE(top_k >= 1 && top_k <= shape->n_blocks, "repair_merge: top_k %d not in [1, %d]", top_k,
              shape->n_blocks);
  PRR_REQUIRE(k_spec >= 0 && k_spec <= shape->n_blocks, "repair_merge: k_spec %d not in [0, %d]", k_spec,
              shape->n_blocks);
  if (k_spec > 0) PRR_REQUIRE(pred_idx && partials, "repair_merge: k_spec > 0 needs pred_idx and partials");
  return launch_repair(*shape, q, k_cache, v_cache, block_table, sel_idx, top_k, k_spec ? pred_idx : nullptr,
                       k_spec, k_spec ? partials : nullptr, out, n_missed, repair_ws(*shape, workspace),
                       as_stream(stream));
}

prr_status prr_score(const prr_shape* shape, const void* q, const void* summaries, float* scores, float* ema,
                     float alpha, int32_t first_step, void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(q && summaries && scores, "score: null pointer");
  if (ema) PRR_REQUIRE(alpha >= 0.f && alpha <= 1.f, "score: alpha not in [0, 1]");
  return launch_score(*shape, q, summaries, scores, ema, alpha, first_step ? 1 : 0, as_stream(stream));
}

prr_status prr_select_speculate(const prr_shape* shape, const float* scores, int32_t top_k, int32_t* sel_idx,
                                const float* ema, int32_t k_spec_next, int32_t* pred_idx_next, const void* q,
                                const void* k_cache, const void* v_cache, const int32_t* block_table,
                                const int32_t* pred_idx, int32_t k_spec, float* partials, const prr_budget* budget,
                                void* workspace, void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_TRY(check_topk_n(shape));
  PRR_REQUIRE(scores && sel_idx, "select_speculate: null pointer");
  PRR_REQUIRE(top_k >= 1 && top_k <= shape->n_blocks, "select_speculate: top_k %d not in [1, %d]", top_k,
              shape->n_blocks);
  PRR_REQUIRE(k_spec_next >= 0 && k_spec_next <= shape->n_blocks, "select_speculate: k_spec_next %d not in [0, %d]",
              k_spec_next, shape->n_blocks);
  PRR_REQUIRE(k_spec >= 0 && k_spec <= shape->n_blocks, "select_speculate: k_spec %d not in [0, %d]", k_spec,
              shape->n_blocks);
  if (k_spec_next > 0) PRR_REQUIRE(ema && pred_idx_next, "select_speculate: k_spec_next > 0 needs ema and pred_idx_next");
  if (k_spec > 0)
    PRR_REQUIRE(q && k_cache && v_cache && block_table && pred_idx && partials, "select_speculate: null pointer");
  if (k_spec > 0 && k_spec_next > 0 && pred_idx == pred_idx_next) {
    set_error("select_speculate: pred_idx and pred_idx_next must be different buffers");
    return PRR_EINVAL;
  }
  if (k_spec_next > 0) PRR_TRY(check_budget(shape, budget, k_spec_next, "select_speculate"));
  return launch_select_spec(*shape, scores, top_k, sel_idx, ema, k_spec_next, pred_idx_next, q, k_cache, v_cache,
                            block_table, pred_idx, k_spec, partials, as_stream(stream),
                            cand_region(*shape, workspace, 0), cand_region(*shape, workspace, 1),
                            cand_region(*shape, workspace, 2),
                            k_spec_next > 0 ? budget_dev(budget) : BudgetDev{});
}

prr_status prr_score_speculate(const prr_shape* shape, const void* q, const void* summaries, float* scores, float* ema,
                               float alpha, int32_t first_step, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* pred_idx, int32_t k_spec, float* partials,
                               void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(q && summaries && scores, "score_speculate: null pointer");
  if (ema) PRR_REQUIRE(alpha >= 0.f && alpha <= 1.f, "score_speculate: alpha not in [0, 1]");
  PRR_REQUIRE(k_spec >= 0 && k_spec <= shape->n_blocks, "score_speculate: k_spec %d not in [0, %d]", k_spec,
              shape->n_blocks);
  if (k_spec > 0)
    PRR_REQUIRE(k_cache && v_cache && block_table && pred_idx && partials, "score_speculate: null pointer");
  return launch_score_spec(*shape, q, summaries, scores, ema, alpha, first_step ? 1 : 0, k_cache, v_cache,
                           block_table, pred_idx, k_spec, partials, as_stream(stream));
}

prr_status prr_select_repair(const prr_shape* shape, const float* scores, int32_t top_k, int32_t* sel_idx,
                             const float* ema, int32_t k_spec_next, int32_t* pred_idx_next, const void* q,
                             const void* k_cache, const void* v_cache, const int32_t* block_table,
                             const int32_t* pred_idx, int32_t k_spec, const float* partials, float* out,
                             int32_t* n_missed, void* workspace, void* stream) {
  PRR_TRY(check_shape(shape));
  PRR_TRY(check_topk_n(shape));
  PRR_REQUIRE(scores && sel_idx && q && k_cache && v_cache && block_table && out && n_missed && workspace,
              "select_repair: null pointer");
  PRR_REQUIRE(top_k >= 1 && top_k <= shape->n_blocks, "select_repair: top_k %d not in [1, %d]", top_k,
              shape->n_blocks);
  PRR_REQUIRE(k_spec >= 0 && k_spec <= shape->n_blocks, "select_repair: k_spec %d not in [0, %d]", k_spec,
              shape->n_blocks);
  PRR_REQUIRE(k_spec_next >= 0 && k_spec_next <= shape->n_blocks, "select_repair: k_spec_next %d not in [0, %d]",
              k_spec_next, shape->n_blocks);
  if (k_spec > 0) PRR_REQUIRE(pred_idx && partials, "select_repair: k_spec > 0 needs pred_idx and partials");
  if (k_spec_next > 0) PRR_REQUIRE(ema && pred_idx_next, "select_repair: k_spec_next > 0 needs ema and pred_idx_next");
  if (k_spec > 0 && k_spec_next > 0 && pred_idx == pred_idx_next) {
    set_error("select_repair: pred_idx and pred_idx_next must be different buffers");
    return PRR_EINVAL;
  }
  if (!two_launch_supported(*shape, top_k, k_spec, k_spec_next)) {
    set_error("select_repair: needs page_size %% 16 == 0, block_size <= 128 and top_k, k_spec, k_spec_next <= 2048");
    return PRR_EUNSUPPORTED;
  }
  return launch_select_missed(*shape, scores, top_k, sel_idx, ema, k_spec_next, pred_idx_next, q, k_cache, v_cache,
                              block_table, k_spec ? pred_idx : nullptr, k_spec, k_spec ? const_cast<float*>(partials)
                              : nullptr, false, out, n_missed, repair_ws(*shape, workspace), as_stream(stream));
}

size_t prr_partials_bytes(const prr_shape* shape, int32_t k_spec) {
  if (check_shape(shape) != PRR_OK || k_spec <= 0) return 0;
  const int G = shape->n_q_heads / shape->n_kv_heads;
  return (size_t)shape->batch * shape->n_kv_heads * (size_t)k_spec *
         (size_t)spec_rec_bytes(shape->dtype, G, shape->head_dim);
}

size_t prr_workspace_bytes(const prr_shape* shape, int32_t top_k) {
  if (check_shape(shape) != PRR_OK || top_k <= 0) return 0;
  const size_t a = repair_workspace_bytes(*shape, top_k), b = select_missed_ws_bytes(*shape, top_k);
  return 3 * cand_part_bytes(*shape) + (a > b ? a : b);
}

prr_status prr_step_ctx_create(prr_step_ctx** out) {
  if (!out) { set_error("step_ctx_create: null pointer"); return PRR_EINVAL; }
  auto* c = new (std::nothrow) prr_step_ctx{};
  if (!c) { set_error("step_ctx_create: out of host memory"); return PRR_EINVAL; }
  hipEvent_t* ev[2] = {&c->q_ready, &c->spec_done};
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(ev[i], hipEventDisableTiming) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(*ev[j]);
      delete c;
      set_error("step_ctx_create: hipEventCreateWithFlags failed");
      return PRR_ELAUNCH;
    }
  }
  *out = c;
  return PRR_OK;
}

prr_status prr_step_ctx_set_delays(prr_step_ctx* ctx, int32_t delay_sel, int32_t delay_spec) {
  PRR_REQUIRE(ctx, "step_ctx_set_delays: null context");
  PRR_REQUIRE(delay_sel >= 0 && delay_sel <= 100000 && delay_spec >= 0 && delay_spec <= 100000,
              "step_ctx_set_delays: delays must be in [0, 100000] sleep iterations");
  ctx->delay_sel = delay_sel;
  ctx->delay_spec = delay_spec;
  return PRR_OK;
}

void prr_step_ctx_destroy(prr_step_ctx* ctx) {
  if (!ctx) return;
  (void)hipEventDestroy(ctx->q_ready);
  (void)hipEventDestroy(ctx->spec_done);
  delete ctx;
}

static prr_status hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return PRR_ELAUNCH;
  }
  return PRR_OK;
}

prr_status prr_decode_step(prr_step_ctx* ctx, const prr_shape* shape, const prr_step_args* a, int32_t mode,
                           int32_t join, void* stream_sel, void* stream_spec) {
  return decode_step_impl(ctx, shape, a, mode, join, stream_sel, stream_spec);
}

prr_status prr_decode_step_noalloc(prr_step_ctx* ctx, const prr_shape* shape, const prr_step_args* a, int32_t mode,
                                   int32_t join, void* stream_sel, void* stream_spec) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(a, "decode_step_noalloc: args is NULL");
  PRR_REQUIRE(!a->workspace, "decode_step_noalloc: args->workspace must be NULL (the library's scratch is used)");
  PRR_REQUIRE(a->top_k >= 1 && a->top_k <= shape->n_blocks, "decode_step_noalloc: top_k %d not in [1, %d]",
              a->top_k, shape->n_blocks);
  const size_t need = prr_workspace_bytes(shape, a->top_k);
  PRR_REQUIRE(need <= kScratchBytes, "decode_step_noalloc: this shape needs %zu bytes of workspace, more than the "
              "library's %zu-byte scratch (use prr_decode_step with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  PRR_TRY(scratch_of_stream(as_stream(stream_sel), &ws));
  if (mode == PRR_MODE_TWO_STREAM) {   // both streams must be on the scratch's device
    void* ws2 = nullptr;
    PRR_TRY(scratch_of_stream(as_stream(stream_spec), &ws2));
  }
  prr_step_args with_ws = *a;
  with_ws.workspace = ws;
  return decode_step_impl(ctx, shape, &with_ws, mode, join, stream_sel, stream_spec);
}

}  // extern "C"

static prr_status decode_step_impl(prr_step_ctx* ctx, const prr_shape* shape, const prr_step_args* a, int32_t mode,
                                   int32_t join, void* stream_sel, void* stream_spec) {
  PRR_TRY(check_shape(shape));
  PRR_REQUIRE(a, "decode_step: args is NULL");
  PRR_REQUIRE(mode >= PRR_MODE_SERIALIZED && mode <= PRR_MODE_SERIALIZED_FUSED, "decode_step: unknown mode %d", mode);
  PRR_REQUIRE(mode != PRR_MODE_TWO_STREAM || ctx, "decode_step: two-stream mode needs a step context");
  const hipStream_t s1 = as_stream(stream_sel);
  const hipStream_t s2 = as_stream(stream_spec);
  const bool serial = mode == PRR_MODE_SERIALIZED || mode == PRR_MODE_SERIALIZED_FUSED;
  const int kc = serial ? 0 : a->k_spec_cur;
  const int kn = serial ? 0 : a->k_spec_next;
  const int N = shape->n_blocks;
  // every argument of every mode is checked here, before the first launch: a rejected call enqueues nothing (and so
  // leaves the EMA and every other buffer as it was)
  PRR_TRY(check_topk_n(shape));
  PRR_REQUIRE(a->top_k >= 1 && a->top_k <= N, "decode_step: top_k %d not in [1, %d]", a->top_k, N);
  PRR_REQUIRE(kc >= 0 && kc <= N && kn >= 0 && kn <= N, "decode_step: k_spec_cur %d, k_spec_next %d not in [0, %d]",
              kc, kn, N);
  PRR_REQUIRE(a->q && a->k_cache && a->v_cache && a->block_table && a->summaries && a->scores && a->sel_idx &&
              a->out && a->n_missed && a->workspace, "decode_step: null pointer");
  if (kc > 0) PRR_REQUIRE(a->pred_cur && a->partials, "decode_step: k_spec_cur > 0 needs pred_cur and partials");
  if (kn > 0) {
    PRR_REQUIRE(a->ema && a->pred_next, "decode_step: k_spec_next > 0 needs ema and pred_next");
    PRR_REQUIRE(kc == 0 || a->pred_next != a->pred_cur, "decode_step: pred_cur and pred_next must differ");
    PRR_REQUIRE(a->alpha >= 0.f && a->alpha <= 1.f, "decode_step: alpha not in [0, 1]");
  }

  const int64_t rows = (int64_t)shape->batch * shape->n_kv_heads;
  const prr_budget* budget = kn > 0 ? a->budget : nullptr;
  const bool budgeted = budget && budget->policy != PRR_BUDGET_FIXED;
  if (budgeted) {
    PRR_TRY(check_budget(shape, budget, kn, "decode_step"));
    PRR_REQUIRE(budget->top_k == a->top_k, "decode_step: the budget's top_k %d differs from the step's %d",
                budget->top_k, a->top_k);
  }

  // select-then-attend in two launches pays off only when the rows alone fill the chip (one workgroup per row
  // attends over the row's whole true set); otherwise the spread-out attention launches are faster
  if (mode == PRR_MODE_SERIALIZED_FUSED) {
    if (two_launch_supported(*shape, a->top_k, 0, 0) && (int64_t)shape->batch * shape->n_kv_heads >= 128) {
      PRR_TRY(prr_score(shape, a->q, a->summaries, a->scores, nullptr, 0.f, 0, s1));
      return prr_select_repair(shape, a->scores, a->top_k, a->sel_idx, nullptr, 0, nullptr, a->q, a->k_cache,
                               a->v_cache, a->block_table, nullptr, 0, nullptr, a->out, a->n_missed, a->workspace,
                               s1);
    }
    mode = PRR_MODE_SERIALIZED;
  }
  // budgeted predictions are written by the selection launches (one workgroup per row up to 8192 blocks)
  // (with nothing predicted or to predict the fused step runs the serialized launches, below)
  if (mode == PRR_MODE_FUSED && (kc > 0 || kn > 0) && two_launch_supported(*shape, a->top_k, kc, kn) &&
      a->top_k <= 32 && rows < 128 && !(budgeted && shape->n_blocks > 8192)) {
    // short true sets: scores; then selection of T and of P_{t+1} (whose workgroups update the EMA first, under a
    // fixed budget), speculation over P_t and the few missed blocks T \ P_t in one launch (one workgroup per row
    // attends its row's missed blocks right after its selection); then the merge of the missed-block record with the
    // speculated records of T ∩ P_t
    const bool sel_ema = kn > 0 && !budgeted;
    PRR_TRY(prr_score(shape, a->q, a->summaries, a->scores, kn > 0 && !sel_ema ? a->ema : nullptr, a->alpha,
                      a->first_step, s1));
    return launch_select_missed(*shape, a->scores, a->top_k, a->sel_idx, a->ema, kn, a->pred_next, a->q, a->k_cache,
                                a->v_cache, a->block_table, kc ? a->pred_cur : nullptr, kc,
                                kc ? a->partials : nullptr, true, a->out, a->n_missed,
                                repair_ws(*shape, a->workspace), s1, budget_dev(budget), sel_ema, a->alpha,
                                a->first_step ? 1 : 0);
  }
  if (mode == PRR_MODE_FUSED && rows >= 128) {
    // When the rows alone fill the chip every phase is bound by bandwidth. The speculation over P_t takes its own
    // launch (several slots per wave, pipelined), which moves the gathered blocks faster than speculation roles
    // beside the selection would; the selection launch then holds only top-K workgroups (T and P_{t+1}), all
    // resident at once, and the workgroups that select P_{t+1} also update the EMA, which they read anyway (the
    // bandwidth-bound scoring pass then writes the scores alone); the spread-out repair merges the hits' records
    // and attends the missed blocks.
    if (kc > 0)
      PRR_TRY(prr_speculate(shape, a->q, a->k_cache, a->v_cache, a->block_table, a->pred_cur, kc, a->partials, s1));
    if (kn > 0 && N <= kTopkSplitMinN) {
      PRR_TRY(prr_score(shape, a->q, a->summaries, a->scores, nullptr, 0.f, 0, s1));
      PRR_TRY(launch_topk_pair(*shape, a->scores, a->top_k, a->sel_idx, a->ema, kn, a->pred_next, budget_dev(budget),
                               s1, true, a->alpha, a->first_step ? 1 : 0));
    } else {   // long rows select by segments, whose EMA-segment workgroups update the EMA (as below 128 rows)
      const bool sel_ema = kn > 0 && !budgeted;
      PRR_TRY(prr_score(shape, a->q, a->summaries, a->scores, kn > 0 && !sel_ema ? a->ema : nullptr, a->alpha,
                        a->first_step, s1));
      PRR_TRY(launch_select_spec(*shape, a->scores, a->top_k, a->sel_idx, a->ema, kn, a->pred_next, a->q,
                                 a->k_cache, a->v_cache, a->block_table, nullptr, 0, nullptr, s1,
                                 cand_region(*shape, a->workspace, 0), cand_region(*shape, a->workspace, 1),
                                 cand_region(*shape, a->workspace, 2), kn > 0 ? budget_dev(budget) : BudgetDev{},
                                 sel_ema, a->alpha, a->first_step ? 1 : 0));
    }
    return prr_repair_merge(shape, a->q, a->k_cache, a->v_cache, a->block_table, a->sel_idx, a->top_k, a->pred_cur,
                            kc, a->partials, a->out, a->n_missed, a->workspace, s1);
  }
  if (mode == PRR_MODE_FUSED) {
    // Otherwise the speculation rides in the latency-bound selection launch (long rows select in two launches,
    // segments then a merge, through the workspace's candidate regions), then the spread-out repair. The workgroups
    // that predict P_{t+1} (or rank the EMA's segments) update the EMA, which they read anyway, so the scoring pass
    // writes the scores alone (same-box A/B over two runs: million-token layer 66.1 -> 65.3 us at K' = 384, 59.7 ->
    // 58.2 us at K' = 128, with the update in the segment launch). Under a per-row budget the scoring pass keeps
    // the update: the confidence rule reads the EMA beside the prediction, and the budgeted prediction roles would
    // take more registers.
    const bool sel_ema = kn > 0 && !budgeted;
    PRR_TRY(prr_score(shape, a->q, a->summaries, a->scores, kn > 0 && !sel_ema ? a->ema : nullptr, a->alpha,
                      a->first_step, s1));
    PRR_TRY(launch_select_spec(*shape, a->scores, a->top_k, a->sel_idx, a->ema, kn, a->pred_next, a->q, a->k_cache,
                               a->v_cache, a->block_table, kc ? a->pred_cur : nullptr, kc,
                               kc ? a->partials : nullptr, s1, cand_region(*shape, a->workspace, 0),
                               cand_region(*shape, a->workspace, 1), cand_region(*shape, a->workspace, 2),
                               kn > 0 ? budget_dev(budget) : BudgetDev{}, sel_ema, a->alpha, a->first_step ? 1 : 0));
    return prr_repair_merge(shape, a->q, a->k_cache, a->v_cache, a->block_table, a->sel_idx, a->top_k, a->pred_cur,
                            kc, a->partials, a->out, a->n_missed, a->workspace, s1);
  }
  auto score_select = [&](hipStream_t st) {
    return prr_score_select(shape, a->q, a->summaries, a->top_k, a->scores, a->sel_idx, a->workspace, st);
  };
  auto ema_predict = [&](hipStream_t st) {
    return prr_ema_predict(shape, a->scores, a->ema, a->alpha, a->first_step, kn, a->pred_next, budget, a->workspace,
                           st);
  };
  if (mode != PRR_MODE_TWO_STREAM) {
    if (kc > 0) PRR_TRY(prr_speculate(shape, a->q, a->k_cache, a->v_cache, a->block_table, a->pred_cur, kc,
                                      a->partials, s1));
    PRR_TRY(score_select(s1));
    PRR_TRY(prr_repair_merge(shape, a->q, a->k_cache, a->v_cache, a->block_table, a->sel_idx, a->top_k, a->pred_cur,
                             kc, a->partials, a->out, a->n_missed, a->workspace, s1));
    if (kn > 0) PRR_TRY(ema_predict(s1));
    return PRR_OK;
  }
  // One fork and one join per step: speculation over P_t runs on stream_spec while stream_sel scores and selects;
  // the repair waits for it; the next prediction follows the repair on stream_sel, so the next step's fork (recorded
  // after it) orders the next speculation after P_{t+1}. Every edge between the streams costs an idle gap when a
  // graph runs the two branches on different hardware queues, so the step keeps only these two.
  (void)join;   // stream_spec's work always ends in the join below
  PRR_TRY(hip_ok(hipEventRecord(ctx->q_ready, s1), "decode_step: record fork"));
  PRR_TRY(hip_ok(hipStreamWaitEvent(s2, ctx->q_ready, 0), "decode_step: wait fork"));
  if (ctx->delay_spec > 0) PRR_TRY(launch_delay(ctx->delay_spec, s2));
  if (kc > 0) PRR_TRY(prr_speculate(shape, a->q, a->k_cache, a->v_cache, a->block_table, a->pred_cur, kc,
                                    a->partials, s2));
  PRR_TRY(hip_ok(hipEventRecord(ctx->spec_done, s2), "decode_step: record join"));
  PRR_TRY(score_select(s1));
  PRR_TRY(hip_ok(hipStreamWaitEvent(s1, ctx->spec_done, 0), "decode_step: wait join"));
  if (ctx->delay_sel > 0) PRR_TRY(launch_delay(ctx->delay_sel, s1));
  PRR_TRY(prr_repair_merge(shape, a->q, a->k_cache, a->v_cache, a->block_table, a->sel_idx, a->top_k, a->pred_cur,
                           kc, a->partials, a->out, a->n_missed, a->workspace, s1));
  if (kn > 0) PRR_TRY(ema_predict(s1));
  return PRR_OK;
}

extern "C" {

prr_status prr_trace_create(prr_trace** out, int32_t capacity) {
  if (!out || capacity < 1) { set_error("trace_create: null pointer or capacity < 1"); return PRR_EINVAL; }
  auto* t = new (std::nothrow) prr_trace{};
  if (!t) { set_error("trace_create: out of host memory"); return PRR_EINVAL; }
  t->capacity = capacity;
  for (int k = 0; k < PRR_KERNEL_COUNT; ++k) {
    t->ev0[k] = new (std::nothrow) hipEvent_t[capacity]();
    t->ev1[k] = new (std::nothrow) hipEvent_t[capacity]();
    if (!t->ev0[k] || !t->ev1[k]) { prr_trace_destroy(t); set_error("trace_create: out of host memory"); return PRR_EINVAL; }
    for (int i = 0; i < capacity; ++i) {
      if (hipEventCreate(&t->ev0[k][i]) != hipSuccess || hipEventCreate(&t->ev1[k][i]) != hipSuccess) {
        prr_trace_destroy(t);
        set_error("trace_create: hipEventCreate failed");
        return PRR_ELAUNCH;
      }
    }
  }
  *out = t;
  return PRR_OK;
}

void prr_trace_destroy(prr_trace* t) {
  if (!t) return;
  prr_trace* expected = t;
  g_trace.compare_exchange_strong(expected, nullptr);
  for (int k = 0; k < PRR_KERNEL_COUNT; ++k) {
    for (int i = 0; i < t->capacity; ++i) {
      if (t->ev0[k] && t->ev0[k][i]) (void)hipEventDestroy(t->ev0[k][i]);
      if (t->ev1[k] && t->ev1[k][i]) (void)hipEventDestroy(t->ev1[k][i]);
    }
    delete[] t->ev0[k];
    delete[] t->ev1[k];
  }
  delete t;
}

prr_status prr_trace_enable(prr_trace* t, uint32_t mask) {
  if (!t || mask == 0) { g_trace.store(nullptr, std::memory_order_release); return PRR_OK; }
  t->mask = mask;
  t->failure[0] = 0;
  for (int k = 0; k < PRR_KERNEL_COUNT; ++k) t->count[k] = 0;
  g_trace.store(t, std::memory_order_release);
  return PRR_OK;
}

int32_t prr_trace_read(prr_trace* t, int32_t kernel, float* ms_out, int32_t cap) {
  if (!t || kernel < 0 || kernel >= PRR_KERNEL_COUNT || (cap > 0 && !ms_out)) {
    set_error("trace_read: invalid argument");
    return PRR_EINVAL;
  }
  if (t->failure[0]) {
    set_error("trace_read: %s", t->failure);
    return PRR_ELAUNCH;
  }
  const int n = t->count[kernel] < cap ? t->count[kernel] : cap;
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(t->ev1[kernel][i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms_out[i], t->ev0[kernel][i], t->ev1[kernel][i]);
    if (e != hipSuccess) {
      set_error("trace_read: event query failed: %s", hipGetErrorString(e));
      (void)hipGetLastError();
      return PRR_ELAUNCH;
    }
  }
  return n;
}

prr_status prr_flush_write(void* buf, size_t bytes, void* stream) {
  PRR_REQUIRE(buf && bytes % 16 == 0, "flush_write: null buffer or size not a multiple of 16");
  return launch_flush(buf, bytes, as_stream(stream));
}

prr_status prr_stream_read(const void* buf, size_t bytes, float* sink, void* stream) {
  PRR_REQUIRE(buf && sink && bytes % 16 == 0, "stream_read: null pointer or size not a multiple of 16");
  return launch_stream_read(buf, bytes, sink, as_stream(stream));
}

const char* prr_status_string(prr_status s) {
  switch (s) {
    case PRR_OK: return "PRR_OK";
    case PRR_EINVAL: return "PRR_EINVAL: invalid argument";
    case PRR_EUNSUPPORTED: return "PRR_EUNSUPPORTED: unsupported shape or dtype";
    case PRR_ELAUNCH: return "PRR_ELAUNCH: HIP runtime error";
  }
  return "unknown prr_status";
}

const char* prr_last_error(void) { return g_err; }

const char* prr_version(void) { return "libprr 0.1 (gfx950)"; }

}  // extern "C"
