// C-ABI host layer of libssa: argument validation, geometry, kernel launch.
// All validation happens before anything touches the HIP runtime, so invalid
// calls fail the same way on machines without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/ssa.h"
#include "ssa_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

ssa_status_t fail(ssa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

ssa_status_t hip_fail(hipError_t e, const char* where) {
  return fail(SSA_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validate the shape and fill the kernel geometry.  `want_empty` is set when
// there is nothing to compute.
ssa_status_t make_geometry(const ssa_shape_t* s, ssa::Geometry* g, bool* empty, const char* fn) {
  if (!s) return fail(SSA_ERR_INVALID_ARG, "%s: shape is NULL", fn);
  if (s->batch < 0 || s->seq_q < 0 || s->seq_kv < 0 || s->q_offset < 0)
    return fail(SSA_ERR_INVALID_ARG, "%s: negative batch/seq_q/seq_kv/q_offset", fn);
  if (s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads != 0)
    return fail(SSA_ERR_INVALID_ARG, "%s: n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                fn, s->n_q_heads, s->n_kv_heads);
  if (s->head_dim < 1 || s->block < 1 || s->topk < 1)
    return fail(SSA_ERR_INVALID_ARG, "%s: head_dim, block and topk must be >= 1", fn);
  if ((int64_t)s->q_offset + s->seq_q != s->seq_kv)
    return fail(SSA_ERR_INVALID_ARG, "%s: seq_kv (%d) must equal q_offset (%d) + seq_q (%d)", fn,
                s->seq_kv, s->q_offset, s->seq_q);
  if (s->seq_q > 1 && s->q_offset % s->block != 0)
    return fail(SSA_ERR_INVALID_ARG, "%s: a multi-row query chunk must start on a block boundary", fn);
  if (!isfinite(s->scale)) return fail(SSA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (s->scale < 0.f) return fail(SSA_ERR_UNSUPPORTED, "%s: negative scale", fn);
  if (s->causal != 1) return fail(SSA_ERR_UNSUPPORTED, "%s: only causal attention is implemented", fn);
  if (s->head_dim != ssa::kHeadDim)
    return fail(SSA_ERR_UNSUPPORTED, "%s: head_dim %d (supported: %d)", fn, s->head_dim, ssa::kHeadDim);
  if (s->block != ssa::kBlock)
    return fail(SSA_ERR_UNSUPPORTED, "%s: block %d (supported: %d)", fn, s->block, ssa::kBlock);
  if (s->topk > ssa::kMaxTopk)
    return fail(SSA_ERR_UNSUPPORTED, "%s: topk %d (supported: <= %d)", fn, s->topk, ssa::kMaxTopk);
  const int64_t rows_q = (int64_t)s->batch * s->n_q_heads * s->seq_q * s->head_dim;
  const int64_t rows_kv = (int64_t)s->batch * s->n_kv_heads * s->seq_kv * s->head_dim;
  const int64_t nkb = (s->seq_kv + s->block - 1) / s->block;
  const int64_t nqb = (s->seq_q + s->block - 1) / s->block;
  const int64_t nscores = (int64_t)s->batch * s->n_q_heads * nqb * nkb;
  const int64_t limit = (int64_t)1 << 40;
  if (rows_q > limit || rows_kv > limit || nscores > limit || s->batch * (int64_t)s->n_q_heads * nqb > INT32_MAX)
    return fail(SSA_ERR_UNSUPPORTED, "%s: problem too large", fn);
  g->batch = s->batch;
  g->hq = s->n_q_heads;
  g->hkv = s->n_kv_heads;
  g->group = s->n_q_heads / s->n_kv_heads;
  g->seq_q = s->seq_q;
  g->seq_kv = s->seq_kv;
  g->q_offset = s->q_offset;
  g->topk = s->topk;
  g->nqb = (int)nqb;
  g->nkb = (int)nkb;
  const double scale = s->scale != 0.f ? (double)s->scale : 1.0 / sqrt((double)s->head_dim);
  g->scale = (float)scale;
  g->scale_log2 = (float)((double)g->scale * 1.4426950408889634);
  *empty = (s->batch == 0 || s->seq_q == 0);
  g_last_error[0] = '\0';
  return SSA_OK;
}

#define CHECK_PTR(p, align, fn)                                                              \
  do {                                                                                       \
    if (!(p)) return fail(SSA_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);                    \
    if (!aligned((p), (align))) return fail(SSA_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", fn, #p, (int)(align)); \
  } while (0)

// Workspace bytes past the work queue hold per-workgroup timing records.
void set_trace(ssa::AttnArgs* a, void* workspace, size_t workspace_bytes) {
  const size_t rec = (workspace_bytes - ssa::kQueueBytes) / (ssa::kTraceWords * sizeof(uint32_t));
  if (rec == 0) return;
  a->trace = (uint32_t*)((uint8_t*)workspace + ssa::kQueueBytes);
  a->trace_cap = rec > (size_t)INT32_MAX ? INT32_MAX : (int)rec;
}

// Scratch of ssa_block_sparse_attn_fwd_noalloc: one static array per GPU, held
// until the process ends.  The first kScratchQueueBytes are the prefill work
// queue (zero between calls: every completed launch leaves its counters zero);
// the rest holds the decode partials (written before they are read).
constexpr size_t kScratchQueueBytes = 1024;
constexpr size_t kScratchPartialBytes = (size_t)8 << 20;
constexpr size_t kScratchBytes = kScratchQueueBytes + kScratchPartialBytes;
static_assert(kScratchQueueBytes >= ssa::kQueueBytes, "queue region too small");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_zeroed[kMaxDevices] = {};

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of the current device's scratch array (looked up once per
// device).  Until one clearing of the queue region has run outside stream
// capture, every call enqueues it first (inside a capture it becomes part of
// the graph).
ssa_status_t scratch_base(hipStream_t stream, uint8_t** base, const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(SSA_ERR_UNSUPPORTED, "%s: device %d (at most %d)", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, fn);
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  if (!g_scratch_zeroed[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, fn);
    const int words = (int)(kScratchQueueBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       (uint32_t*)g_scratch_ptr[dev], words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, fn);
    if (cs == hipStreamCaptureStatusNone) g_scratch_zeroed[dev] = true;
  }
  *base = g_scratch_ptr[dev];
  return SSA_OK;
}

}  // namespace

extern "C" {

ssa_status_t ssa_block_summaries(const ssa_shape_t* shape, const void* k, float* k_summary,
                                 hipStream_t stream) {
  const char* fn = "ssa_block_summaries";
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (g.batch == 0 || g.seq_kv == 0) return SSA_OK;
  CHECK_PTR(k, 16, fn);
  CHECK_PTR(k_summary, 16, fn);
  hipError_t e = ssa::launch_block_summaries((const uint16_t*)k, k_summary, g, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

ssa_status_t ssa_block_summaries_learned(const ssa_shape_t* shape, const void* k, const float* qbar,
                                         float* k_summary, hipStream_t stream) {
  const char* fn = "ssa_block_summaries_learned";
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (g.batch == 0 || g.seq_kv == 0) return SSA_OK;
  CHECK_PTR(k, 16, fn);
  CHECK_PTR(qbar, 4, fn);
  CHECK_PTR(k_summary, 16, fn);
  hipError_t e = ssa::launch_learned_summaries((const uint16_t*)k, qbar, k_summary, g, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

ssa_status_t ssa_entmax_route(const ssa_shape_t* shape, const float* scores, float alpha, float gamma, float sigma,
                              int32_t* block_idx, float* block_bias, float* weights, hipStream_t stream) {
  const char* fn = "ssa_entmax_route";
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (!(alpha > 1.f && alpha <= 2.f))
    return fail(alpha == alpha ? SSA_ERR_UNSUPPORTED : SSA_ERR_INVALID_ARG, "%s: alpha must be in (1, 2] (got %g)", fn,
                (double)alpha);
  if (!(gamma >= 0.f) || !isfinite(gamma) || !(sigma >= 0.f) || !isfinite(sigma))
    return fail(SSA_ERR_INVALID_ARG, "%s: gamma and sigma must be finite and >= 0", fn);
  if (g.nkb > 1024) return fail(SSA_ERR_UNSUPPORTED, "%s: more than 1024 key blocks", fn);
  if (empty) return SSA_OK;
  CHECK_PTR(scores, 4, fn);
  CHECK_PTR(block_idx, 4, fn);
  CHECK_PTR(block_bias, 4, fn);
  if (weights) CHECK_PTR(weights, 4, fn);
  hipError_t e = ssa::launch_entmax_route(scores, alpha, gamma, sigma, block_idx, block_bias, weights, g, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

ssa_status_t ssa_block_scores(const ssa_shape_t* shape, const void* q, const void* k, float* k_summary,
                              int summary_is_input, float* scores, hipStream_t stream) {
  const char* fn = "ssa_block_scores";
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (empty) return SSA_OK;
  CHECK_PTR(q, 16, fn);
  CHECK_PTR(k_summary, 16, fn);
  CHECK_PTR(scores, 4, fn);
  if (!summary_is_input) CHECK_PTR(k, 16, fn);
  if (g.seq_q == 1 && g.group > 64)
    return fail(SSA_ERR_UNSUPPORTED, "%s: decode with more than 64 query heads per KV head", fn);
  hipError_t e = hipSuccess;
  if (!summary_is_input) e = ssa::launch_block_summaries((const uint16_t*)k, k_summary, g, stream);
  if (e == hipSuccess) {
    if (g.seq_q == 1)
      e = ssa::launch_decode_scores((const uint16_t*)q, k_summary, scores, g, stream);
    else
      e = ssa::launch_prefill_scores((const uint16_t*)q, k_summary, scores, g, stream);
  }
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

ssa_status_t ssa_decode_scores_select(const ssa_shape_t* shape, const void* q, const float* k_summary, float* scores,
                                      int32_t* block_idx, int32_t shared, hipStream_t stream) {
  const char* fn = "ssa_decode_scores_select";
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (g.seq_q != 1) return fail(SSA_ERR_INVALID_ARG, "%s: decode only (seq_q == 1), got seq_q %d", fn, g.seq_q);
  if (empty) return SSA_OK;
  CHECK_PTR(q, 16, fn);
  CHECK_PTR(k_summary, 16, fn);
  CHECK_PTR(block_idx, 4, fn);
  if (scores) CHECK_PTR(scores, 4, fn);
  if (!ssa::decode_select_fits(g, shared != 0))
    return fail(SSA_ERR_UNSUPPORTED,
                "%s: %d query heads per KV head x %d key blocks do not fit one workgroup; "
                "use ssa_block_scores and ssa_select_topk",
                fn, g.group, g.nkb);
  hipError_t e = ssa::launch_decode_select((const uint16_t*)q, k_summary, scores, block_idx, g, shared != 0, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

}  // extern "C"

namespace {

ssa_status_t select_topk_impl(const ssa_shape_t* shape, const float* scores, int32_t* block_idx, bool shared,
                              hipStream_t stream, const char* fn) {
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (empty) return SSA_OK;
  CHECK_PTR(scores, 4, fn);
  CHECK_PTR(block_idx, 4, fn);
  hipError_t e = ssa::launch_select_topk(scores, block_idx, g, shared, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

ssa_status_t sparse_fwd_impl(const ssa_shape_t* shape, const void* q, const void* k, const void* v,
                             const int32_t* block_idx, bool shared, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, const char* fn,
                             const float* block_bias = nullptr, bool biased = false, bool use_scratch = false) {
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (empty) return SSA_OK;
  if (biased) CHECK_PTR(block_bias, 4, fn);
  CHECK_PTR(q, 16, fn);
  CHECK_PTR(k, 16, fn);
  CHECK_PTR(v, 16, fn);
  CHECK_PTR(block_idx, 4, fn);
  CHECK_PTR(out, 16, fn);
  CHECK_PTR(lse, 4, fn);
  ssa::AttnArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.idx = block_idx;
  a.idx_shared = shared ? 1 : 0;
  a.bias = biased ? block_bias : nullptr;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.qb_begin = 0;
  a.qb_count = g.nqb;
  a.rows_out = g.seq_q;
  hipError_t e;
  if (g.seq_q == 1) {
    if (g.group > 32)
      return fail(SSA_ERR_UNSUPPORTED, "%s: decode with more than 32 query heads per KV head", fn);
    if ((int64_t)g.group * g.topk > ssa::kDecodeMaxList || g.nkb > ssa::kDecodeMaxBlocks)
      return fail(SSA_ERR_UNSUPPORTED, "%s: decode needs (query heads per KV head) x topk <= %d and <= %d key blocks",
                  fn, ssa::kDecodeMaxList, ssa::kDecodeMaxBlocks);
    const size_t need = ssa::decode_workspace_bytes(g.batch, g.hq, g.hkv);
    if (use_scratch) {
      if (need > kScratchPartialBytes)
        return fail(SSA_ERR_WORKSPACE, "%s: %zu bytes of scratch needed, the static array holds %zu", fn, need,
                    kScratchPartialBytes);
      uint8_t* base = nullptr;
      st = scratch_base(stream, &base, fn);
      if (st != SSA_OK) return st;
      workspace = base + kScratchQueueBytes;
      workspace_bytes = kScratchPartialBytes;
    }
    if (workspace_bytes < need)
      return fail(SSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
    CHECK_PTR(workspace, 16, fn);
    e = ssa::launch_attn_decode(a, (float*)workspace, g, stream);
  } else {
    if (use_scratch) {
      uint8_t* base = nullptr;
      st = scratch_base(stream, &base, fn);
      if (st != SSA_OK) return st;
      workspace = base;
      workspace_bytes = kScratchQueueBytes;
    }
    // an optional zeroed workspace of kQueueBytes makes the launch persistent
    if (workspace && workspace_bytes >= ssa::kQueueBytes) {
      CHECK_PTR(workspace, 16, fn);
      a.queue = (int32_t*)workspace;
      set_trace(&a, workspace, workspace_bytes);
    }
    e = ssa::launch_attn_prefill(a, false, g, stream);
  }
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

ssa_status_t full_impl(const ssa_shape_t* shape, const void* q, const void* k, const void* v,
                       const int32_t* block_idx, bool shared, int32_t q_block_begin, int32_t q_block_count,
                       void* out_full, float* lse_full, float* dropped_mass, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, const char* fn) {
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (q_block_begin < 0 || q_block_count < 0 || (int64_t)q_block_begin + q_block_count > g.nqb)
    return fail(SSA_ERR_INVALID_ARG, "%s: query block range [%d, %d) outside [0, %d)", fn, q_block_begin,
                q_block_begin + q_block_count, g.nqb);
  if (empty || q_block_count == 0) return SSA_OK;
  CHECK_PTR(q, 16, fn);
  CHECK_PTR(k, 16, fn);
  CHECK_PTR(v, 16, fn);
  CHECK_PTR(block_idx, 4, fn);
  CHECK_PTR(out_full, 16, fn);
  CHECK_PTR(lse_full, 4, fn);
  CHECK_PTR(dropped_mass, 4, fn);
  ssa::AttnArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.idx = block_idx;
  a.idx_shared = shared ? 1 : 0;
  a.out = (uint16_t*)out_full;
  a.lse = lse_full;
  a.dropped = dropped_mass;
  a.qb_begin = q_block_begin;
  a.qb_count = q_block_count;
  const int64_t end_row = (int64_t)(q_block_begin + q_block_count) * ssa::kBlock;
  a.rows_out = (int)((end_row < g.seq_q ? end_row : g.seq_q) - (int64_t)q_block_begin * ssa::kBlock);
  if (workspace && workspace_bytes >= ssa::kQueueBytes) {
    CHECK_PTR(workspace, 16, fn);
    a.queue = (int32_t*)workspace;
    set_trace(&a, workspace, workspace_bytes);
  }
  hipError_t e = ssa::launch_attn_prefill(a, true, g, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

ssa_status_t bwd_impl(const ssa_shape_t* shape, const void* q, const void* k, const void* v,
                      const int32_t* block_idx, bool shared, bool full, int32_t q_block_begin, int32_t q_block_count,
                      const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, const char* fn) {
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (!full) {
    q_block_begin = 0;
    q_block_count = g.nqb;
  }
  if (q_block_begin < 0 || q_block_count < 0 || (int64_t)q_block_begin + q_block_count > g.nqb)
    return fail(SSA_ERR_INVALID_ARG, "%s: query block range [%d, %d) outside [0, %d)", fn, q_block_begin,
                q_block_begin + q_block_count, g.nqb);
  if (!full && g.group > 32)
    return fail(SSA_ERR_UNSUPPORTED, "%s: more than 32 query heads per KV head", fn);
  if (empty || q_block_count == 0) return SSA_OK;
  CHECK_PTR(q, 16, fn);
  CHECK_PTR(k, 16, fn);
  CHECK_PTR(v, 16, fn);
  if (!full) CHECK_PTR(block_idx, 4, fn);
  CHECK_PTR(out, 16, fn);
  CHECK_PTR(lse, 4, fn);
  CHECK_PTR(dout, 16, fn);
  CHECK_PTR(dq, 16, fn);
  CHECK_PTR(dk, 16, fn);
  CHECK_PTR(dv, 16, fn);
  ssa::BwdPlan plan;
  size_t off[6], need;
  ssa::bwd_plan(g, full, q_block_begin, q_block_count, &plan, off, &need);
  const uint64_t grid = (uint64_t)g.batch * g.hkv * (uint64_t)plan.slots;
  if (grid > 0x7fffffffull || plan.max_pairs > 0x7fffffffll)
    return fail(SSA_ERR_UNSUPPORTED, "%s: problem too large", fn);
  if (workspace_bytes < need)
    return fail(SSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  CHECK_PTR(workspace, 256, fn);
  ssa::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)out;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.idx = block_idx;
  a.idx_shared = shared ? 1 : 0;
  a.full = full ? 1 : 0;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  uint8_t* ws = (uint8_t*)workspace;
  a.lse2 = (float*)(ws + off[0]);
  a.delta = (float*)(ws + off[1]);
  a.mask = full ? nullptr : (uint32_t*)(ws + off[2]);
  a.pairs = full ? nullptr : (int*)(ws + off[3]);
  a.pair_base = (int*)(ws + off[4]);
  a.part = (float*)(ws + off[5]);
  a.qb_begin = q_block_begin;
  a.qb_count = q_block_count;
  const int64_t end_row = (int64_t)(q_block_begin + q_block_count) * ssa::kBlock;
  a.rows_out = (int)((end_row < g.seq_q ? end_row : g.seq_q) - (int64_t)q_block_begin * ssa::kBlock);
  a.plan = plan;
  hipError_t e = ssa::launch_attn_backward(a, g, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

}  // namespace

extern "C" {

ssa_status_t ssa_block_sparse_attn_bwd(const ssa_shape_t* shape, const void* q, const void* k, const void* v,
                                       const int32_t* block_idx, const void* out, const float* lse,
                                       const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(shape, q, k, v, block_idx, false, false, 0, 0, out, lse, dout, dq, dk, dv, workspace,
                  workspace_bytes, stream, "ssa_block_sparse_attn_bwd");
}

ssa_status_t ssa_block_sparse_attn_bwd_shared(const ssa_shape_t* shape, const void* q, const void* k,
                                              const void* v, const int32_t* block_idx, const void* out,
                                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(shape, q, k, v, block_idx, true, false, 0, 0, out, lse, dout, dq, dk, dv, workspace,
                  workspace_bytes, stream, "ssa_block_sparse_attn_bwd_shared");
}

ssa_status_t ssa_full_attn_bwd(const ssa_shape_t* shape, const void* q, const void* k, const void* v,
                               int32_t q_block_begin, int32_t q_block_count, const void* out_full,
                               const float* lse_full, const void* dout_full, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(shape, q, k, v, nullptr, false, true, q_block_begin, q_block_count, out_full, lse_full, dout_full,
                  dq, dk, dv, workspace, workspace_bytes, stream, "ssa_full_attn_bwd");
}

ssa_status_t ssa_select_topk(const ssa_shape_t* shape, const float* scores, int32_t* block_idx,
                             hipStream_t stream) {
  return select_topk_impl(shape, scores, block_idx, false, stream, "ssa_select_topk");
}

ssa_status_t ssa_select_topk_shared(const ssa_shape_t* shape, const float* scores, int32_t* block_idx,
                                    hipStream_t stream) {
  return select_topk_impl(shape, scores, block_idx, true, stream, "ssa_select_topk_shared");
}

ssa_status_t ssa_block_sparse_attn_fwd(const ssa_shape_t* shape, const void* q, const void* k,
                                       const void* v, const int32_t* block_idx, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sparse_fwd_impl(shape, q, k, v, block_idx, false, out, lse, workspace, workspace_bytes, stream,
                         "ssa_block_sparse_attn_fwd");
}

ssa_status_t ssa_block_sparse_attn_fwd_noalloc(const ssa_shape_t* shape, const void* q, const void* k,
                                               const void* v, const int32_t* block_idx, void* out, float* lse,
                                               hipStream_t stream) {
  return sparse_fwd_impl(shape, q, k, v, block_idx, false, out, lse, nullptr, 0, stream,
                         "ssa_block_sparse_attn_fwd_noalloc", nullptr, false, true);
}

ssa_status_t ssa_block_sparse_attn_fwd_shared(const ssa_shape_t* shape, const void* q, const void* k,
                                              const void* v, const int32_t* block_idx, void* out, float* lse,
                                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sparse_fwd_impl(shape, q, k, v, block_idx, true, out, lse, workspace, workspace_bytes, stream,
                         "ssa_block_sparse_attn_fwd_shared");
}

ssa_status_t ssa_block_sparse_attn_fwd_biased(const ssa_shape_t* shape, const void* q, const void* k,
                                              const void* v, const int32_t* block_idx, const float* block_bias,
                                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  return sparse_fwd_impl(shape, q, k, v, block_idx, true, out, lse, workspace, workspace_bytes, stream,
                         "ssa_block_sparse_attn_fwd_biased", block_bias, true);
}

ssa_status_t ssa_full_attn_fwd_dropped_mass(const ssa_shape_t* shape, const void* q, const void* k,
                                            const void* v, const int32_t* block_idx, int32_t q_block_begin,
                                            int32_t q_block_count, void* out_full, float* lse_full,
                                            float* dropped_mass, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  return full_impl(shape, q, k, v, block_idx, false, q_block_begin, q_block_count, out_full, lse_full,
                   dropped_mass, workspace, workspace_bytes, stream, "ssa_full_attn_fwd_dropped_mass");
}

ssa_status_t ssa_full_attn_fwd_dropped_mass_shared(const ssa_shape_t* shape, const void* q, const void* k,
                                                   const void* v, const int32_t* block_idx,
                                                   int32_t q_block_begin, int32_t q_block_count, void* out_full,
                                                   float* lse_full, float* dropped_mass, void* workspace,
                                                   size_t workspace_bytes, hipStream_t stream) {
  return full_impl(shape, q, k, v, block_idx, true, q_block_begin, q_block_count, out_full, lse_full,
                   dropped_mass, workspace, workspace_bytes, stream, "ssa_full_attn_fwd_dropped_mass_shared");
}

ssa_status_t ssa_block_sparse_attn_fwd_early_stop(const ssa_shape_t* shape, const void* q, const void* k,
                                                  const void* v, const float* scores, const int32_t* block_idx,
                                                  float tau, void* out, float* lse, int32_t* blocks_used,
                                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  const char* fn = "ssa_block_sparse_attn_fwd_early_stop";
  ssa::Geometry g;
  bool empty;
  ssa_status_t st = make_geometry(shape, &g, &empty, fn);
  if (st != SSA_OK) return st;
  if (!(tau >= 0.f)) return fail(SSA_ERR_INVALID_ARG, "%s: tau must be >= 0 (got %g)", fn, (double)tau);
  if (empty) return SSA_OK;
  CHECK_PTR(q, 16, fn);
  CHECK_PTR(k, 16, fn);
  CHECK_PTR(v, 16, fn);
  CHECK_PTR(scores, 4, fn);
  CHECK_PTR(block_idx, 4, fn);
  CHECK_PTR(out, 16, fn);
  CHECK_PTR(lse, 4, fn);
  CHECK_PTR(blocks_used, 4, fn);
  ssa::AttnArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.idx = block_idx;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.qb_begin = 0;
  a.qb_count = g.nqb;
  a.rows_out = g.seq_q;
  hipError_t e = ssa::launch_attn_early_stop(a, scores, tau, blocks_used, g, stream);
  return e == hipSuccess ? SSA_OK : hip_fail(e, fn);
}

size_t ssa_workspace_bytes(const ssa_shape_t* shape, ssa_op_t op) {
  ssa::Geometry g;
  bool empty;
  if (make_geometry(shape, &g, &empty, "ssa_workspace_bytes") != SSA_OK) return SIZE_MAX;
  if (empty) return 0;
  if (op == SSA_OP_SPARSE_FWD && g.seq_q == 1) return ssa::decode_workspace_bytes(g.batch, g.hq, g.hkv);
  if (op == SSA_OP_SPARSE_FWD || op == SSA_OP_FULL_FWD) return ssa::kQueueBytes;
  if (op == SSA_OP_SPARSE_BWD || op == SSA_OP_FULL_BWD) {
    ssa::BwdPlan plan;
    size_t off[6], need;
    ssa::bwd_plan(g, op == SSA_OP_FULL_BWD, 0, g.nqb, &plan, off, &need);
    return need;
  }
  return 0;
}

const char* ssa_status_string(ssa_status_t status) {
  switch (status) {
    case SSA_OK: return "ok";
    case SSA_ERR_INVALID_ARG: return "invalid argument";
    case SSA_ERR_UNSUPPORTED: return "unsupported shape or option";
    case SSA_ERR_HIP: return "HIP runtime error";
    case SSA_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* ssa_last_error(void) { return g_last_error; }

int32_t ssa_version(void) { return 10000; }

}  // extern "C"
