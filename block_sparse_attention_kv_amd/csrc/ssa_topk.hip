// Top-k block selection with the diagonal (most recent) block always kept (gfx950).
//
// One wavefront per (b, h, query block).  Each earlier block j < jd gets a
// 32-bit key that orders scores (larger score -> larger key; -0 == +0; NaN
// below -inf; empty slots 0).  The (k-1)-th largest key T is found by a
// most-significant-bit-first binary search: each of the 32 steps counts the
// candidates at or above a trial value with compares whose results are
// wave-wide bitmasks (popcounted on the scalar unit), so no data moves between
// lanes.  Blocks above T are kept, plus the lowest-index blocks equal to T
// until k-1 are kept ("higher score, then lower index"); a ballot scan writes
// them in ascending order and the diagonal goes last.
// With group-shared selection one row per (b, KV head, query block) ranks the
// mean of the group's per-head scores.
// Method: SSA guide (mauroscia.it), "Block-sparse attention e Receptive
// Field" (fixed top-k block budget); DashAttention summary, "Etapa 2"
// (near-diagonal chunk kept by its own branch) and "Etapa 1" (routing of the
// query heads sharing a KV head averaged into one shared selection).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"
#include "ssa_select.hpp"

namespace ssa {
namespace {

constexpr int kRowsPerWg = 4;

// Rows are (b, query head, query block), or (b, KV head, query block) for the
// group-shared selection (then each wavefront also averages its row).
template <int NPER, bool SHARED>
__global__ __launch_bounds__(256) void select_topk_kernel(const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, Geometry geo, int nrows) {
  __shared__ uint32_t sCb[kRowsPerWg][64];  // per-wave gather buffer of the narrowed search
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerWg + wave;
  if (row >= nrows) return;  // whole wavefront leaves together; no block barriers below
  const int i = row % geo.nqb;
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  const int k = geo.topk;
  RowScores srow;
  if (SHARED) {
    const int bg = row / geo.nqb;  // b * Hkv + g
    const int b = bg / geo.hkv, g = bg - b * geo.hkv;
    srow.s0 = scores + ((size_t)(b * geo.hq + g * geo.group) * geo.nqb + i) * geo.nkb;
    srow.hstride = (size_t)geo.nqb * geo.nkb;
    srow.heads = geo.group;
  } else {
    srow.s0 = scores + (size_t)row * geo.nkb;
    srow.hstride = 0;
    srow.heads = 1;
  }
  int32_t* orow = idx + (size_t)row * k;
  if (jd + 1 <= k) {
    for (int e = lane; e < k; e += 64) orow[e] = e <= jd ? e : -1;
    return;
  }
  if (NPER > 0)
    select_rows<(NPER > 0 ? NPER : 1)>(srow, orow, jd, k - 1, lane, sCb[wave]);
  else
    select_rows_long(srow, orow, jd, k - 1, lane);
  if (lane == 0) orow[k - 1] = jd;
}

// Group-shared selection with the averaging spread over a workgroup: one
// workgroup per (b, KV head, query block) row; its 256 threads average the
// candidates' scores into LDS, then one wavefront selects.
constexpr int kSharedMaxBlocks = 16384;  // LDS row of averaged scores (64 KB)
template <int NPER>
__global__ __launch_bounds__(256) void select_topk_shared_kernel(const float* __restrict__ scores,
                                                                 int32_t* __restrict__ idx, Geometry geo) {
  extern __shared__ float smean[];  // [jd]: averaged scores of the candidates
  __shared__ uint32_t sCb[64];       // gather buffer of the narrowed search
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int row = blockIdx.x;
  const int i = row % geo.nqb;
  const int bg = row / geo.nqb;
  const int b = bg / geo.hkv, g = bg - b * geo.hkv;
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  const int k = geo.topk;
  int32_t* orow = idx + (size_t)row * k;
  if (jd + 1 <= k) {
    if (wave == 0)
      for (int e = lane; e < k; e += 64) orow[e] = e <= jd ? e : -1;
    return;  // the whole workgroup leaves: no barrier is reached
  }
  RowScores src;
  src.s0 = scores + ((size_t)(b * geo.hq + g * geo.group) * geo.nqb + i) * geo.nkb;
  src.hstride = (size_t)geo.nqb * geo.nkb;
  src.heads = geo.group;
  for (int j = tid; j < jd; j += 256) smean[j] = src(j);
  __syncthreads();
  if (wave != 0) return;
  RowScores srow;
  srow.s0 = smean;
  srow.hstride = 0;
  srow.heads = 1;
  if (NPER > 0)
    select_rows<(NPER > 0 ? NPER : 1)>(srow, orow, jd, k - 1, lane, sCb);
  else
    select_rows_long(srow, orow, jd, k - 1, lane);
  if (lane == 0) orow[k - 1] = jd;
}

}  // namespace

hipError_t launch_select_topk(const float* scores, int32_t* idx, const Geometry& g, bool shared,
                              hipStream_t stream) {
  const size_t nrows = (size_t)g.batch * (shared ? g.hkv : g.hq) * g.nqb;
  if (nrows == 0) return hipSuccess;
  if (shared && g.nkb <= kSharedMaxBlocks) {
    const int maxjd_s = (g.q_offset + (g.nqb - 1) * kBlock) / kBlock;
    const size_t lds = (size_t)(maxjd_s > 0 ? maxjd_s : 1) * sizeof(float);
    if (maxjd_s <= 128)
      hipLaunchKernelGGL(select_topk_shared_kernel<2>, dim3((unsigned)nrows), dim3(256), lds, stream, scores, idx, g);
    else if (maxjd_s <= 512)
      hipLaunchKernelGGL(select_topk_shared_kernel<8>, dim3((unsigned)nrows), dim3(256), lds, stream, scores, idx, g);
    else
      hipLaunchKernelGGL(select_topk_shared_kernel<0>, dim3((unsigned)nrows), dim3(256), lds, stream, scores, idx, g);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((nrows + kRowsPerWg - 1) / kRowsPerWg)), block(256);
  const int maxjd = (g.q_offset + (g.nqb - 1) * kBlock) / kBlock;  // largest candidate count
  if (shared)  // rows longer than the LDS row of the workgroup variant
    hipLaunchKernelGGL((select_topk_kernel<0, true>), grid, block, 0, stream, scores, idx, g, (int)nrows);
  else if (maxjd <= 128)
    hipLaunchKernelGGL((select_topk_kernel<2, false>), grid, block, 0, stream, scores, idx, g, (int)nrows);
  else if (maxjd <= 512)
    hipLaunchKernelGGL((select_topk_kernel<8, false>), grid, block, 0, stream, scores, idx, g, (int)nrows);
  else
    hipLaunchKernelGGL((select_topk_kernel<0, false>), grid, block, 0, stream, scores, idx, g, (int)nrows);
  return hipGetLastError();
}

}  // namespace ssa
