// Top-k block selection with the diagonal (most recent) block always kept (gfx950).
//
// One wavefront per (b, h, query block).  Each earlier block j < jd gets a
// unique 64-bit key (orderable fp32 score, then ~j), so "higher score, then
// lower index" is plain unsigned order.  The (k-1)-th largest key is found by
// k-1 rounds of "largest key below the previous one" (a wave max-reduction per
// round; no state besides the previous key), then the kept blocks are
// compacted in ascending order with a ballot scan and the diagonal appended.
// Method: SSA guide (mauroscia.it), "Block-sparse attention e Receptive
// Field" (fixed top-k block budget); DashAttention summary, "Etapa 2"
// (near-diagonal chunk kept by its own branch).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kRowsPerWg = 4;
constexpr int kRegCands = 8;  // candidates held in registers per lane (jd <= 512)

__device__ __forceinline__ uint64_t cand_key(float s, int j) {
  return ((uint64_t)orderable_score(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__global__ __launch_bounds__(256) void select_topk_kernel(const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, Geometry geo,
                                                          int nrows) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerWg + wave;
  if (row >= nrows) return;  // whole wavefront leaves together; no block barriers below
  const int i = row % geo.nqb;
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  const int k = geo.topk;
  const float* srow = scores + (size_t)row * geo.nkb;
  int32_t* orow = idx + (size_t)row * k;

  if (jd + 1 <= k) {
    for (int e = lane; e < k; e += 64) orow[e] = e <= jd ? e : -1;
    return;
  }

  uint64_t thresh = ~0ull;  // after the loop: the (k-1)-th largest key
  if (jd <= kRegCands * 64) {
    uint64_t key[kRegCands];
#pragma unroll
    for (int c = 0; c < kRegCands; ++c) {
      const int j = lane + 64 * c;
      key[c] = j < jd ? cand_key(srow[j], j) : 0ull;
    }
    for (int it = 0; it < k - 1; ++it) {
      uint64_t best = 0ull;
#pragma unroll
      for (int c = 0; c < kRegCands; ++c) best = (key[c] < thresh && key[c] > best) ? key[c] : best;
      thresh = wave_max_u64(best);
    }
  } else {
    for (int it = 0; it < k - 1; ++it) {
      uint64_t best = 0ull;
      for (int j = lane; j < jd; j += 64) {
        const uint64_t kk = cand_key(srow[j], j);
        best = (kk < thresh && kk > best) ? kk : best;
      }
      thresh = wave_max_u64(best);
    }
  }

  // Ascending compaction of {j < jd : key(j) >= thresh}; exactly k-1 of them.
  int count = 0;
  for (int jb = 0; jb < jd; jb += 64) {
    const int j = jb + lane;
    const bool keep = j < jd && cand_key(srow[j], j) >= thresh;
    const uint64_t m = __ballot(keep);
    const int pos = count + (int)__popcll(m & ((1ull << lane) - 1ull));
    if (keep) orow[pos] = j;
    count += (int)__popcll(m);
  }
  if (lane == 0) orow[k - 1] = jd;
}

}  // namespace

hipError_t launch_select_topk(const float* scores, int32_t* idx, const Geometry& g,
                              hipStream_t stream) {
  const size_t nrows = (size_t)g.batch * g.hq * g.nqb;
  if (nrows == 0) return hipSuccess;
  const size_t nwg = (nrows + kRowsPerWg - 1) / kRowsPerWg;
  hipLaunchKernelGGL(select_topk_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, scores, idx,
                     g, (int)nrows);
  return hipGetLastError();
}

}  // namespace ssa
