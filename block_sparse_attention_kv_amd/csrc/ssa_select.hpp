// Top-k selection of one row by one wavefront (ranking keys, the per-row
// score reader and the selection itself), shared by the selection kernels and
// the fused decode scoring + selection.
#pragma once
#include "ssa_common.hpp"

namespace ssa {

// 0 = empty slot; NaN = 1 (below every number); numbers keep their order above.
__device__ __forceinline__ uint32_t cand_key(float s) {
  const uint32_t o = orderable_score(s);
  return o == 0u ? 1u : o;
}

__device__ __forceinline__ int wave_count(bool pred) {
  return (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(pred));
}

// Score of candidate j of one row: the row's own score, or (group-shared
// selection) the mean of the group's per-head scores, summed in head order in
// fp64, divided by the group size and rounded once to fp32.
struct RowScores {
  const float* s0;  // the row (first head of the group when shared)
  size_t hstride;   // distance between the heads' rows
  int heads;        // 1, or the group size when shared
  __device__ __forceinline__ float operator()(int j) const {
    if (heads == 1) return s0[j];
    double acc = 0.0;
    for (int h0 = 0; h0 < heads; h0 += 16) {
      // 16 unconditional loads (past the last head: the last head again), all
      // in flight before the first is summed; then the sum in head order
      float v[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) v[x] = s0[(size_t)min(h0 + x, heads - 1) * hstride + j];
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (h0 + x < heads) acc += (double)v[x];
    }
    return (float)(acc / heads);
  }
};

// Keys of candidates j = lane + 64*c, c < NPER, held in registers.
// With NPER >= 4 and a 64-word LDS buffer `cbuf` for this wavefront, the
// search narrows after its first 12 bits: the keys that share those bits with
// the threshold (at most 64 of them, else the search simply goes on) are
// gathered one per lane, so the remaining 20 steps compare one register
// instead of NPER (the keys above that prefix are counted once).  The result
// is the same threshold.
template <int NPER>
__device__ __forceinline__ void select_rows(const RowScores& srow, int32_t* __restrict__ orow, int jd,
                                            int need, int lane, uint32_t* cbuf = nullptr) {
  // every score is requested before the first is used (rows past the
  // candidates read candidate 0 and are dropped)
  float sv[NPER];
#pragma unroll
  for (int c = 0; c < NPER; ++c) {
    const int j = lane + 64 * c;
    sv[c] = srow(j < jd ? j : 0);
  }
  uint32_t key[NPER];
#pragma unroll
  for (int c = 0; c < NPER; ++c) key[c] = lane + 64 * c < jd ? cand_key(sv[c]) : 0u;
  uint32_t t = 0u;
  int bit = 31;
  if (NPER >= 4 && cbuf) {
    constexpr int kHi = 12;
    for (; bit >= 32 - kHi; --bit) {
      const uint32_t trial = t | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < NPER; ++c) cnt += wave_count(key[c] >= trial);
      if (cnt >= need) t = trial;
    }
    constexpr uint32_t kLow = (1u << (32 - kHi)) - 1u;
    const uint32_t hi_next = t + (kLow + 1u);  // 0 when the prefix is all ones
    int above = 0, live = 0;
#pragma unroll
    for (int c = 0; c < NPER; ++c) {
      if (hi_next != 0u) above += wave_count(key[c] >= hi_next);
      live += wave_count((key[c] & ~kLow) == t);
    }
    if (live <= 64) {
      int base = 0;
#pragma unroll
      for (int c = 0; c < NPER; ++c) {
        const bool lv = (key[c] & ~kLow) == t;
        const uint64_t m = __builtin_amdgcn_ballot_w64(lv);
        if (lv) cbuf[base + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull))] = key[c];
        base += (int)__builtin_popcountll(m);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint32_t lk = lane < live ? cbuf[lane] : 0u;
      const int need2 = need - above;
      for (; bit >= 0; --bit) {
        const uint32_t trial = t | (1u << bit);
        if (wave_count(lk >= trial) >= need2) t = trial;
      }
      __builtin_amdgcn_wave_barrier();  // the buffer's reads are done before it is written again
    }
  }
  for (; bit >= 0; --bit) {
    const uint32_t trial = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < NPER; ++c) cnt += wave_count(key[c] >= trial);
    if (cnt >= need) t = trial;
  }
  int greater = 0;
#pragma unroll
  for (int c = 0; c < NPER; ++c) greater += wave_count(key[c] > t);
  const int ties = need - greater;  // blocks equal to t to keep, lowest index first
  int count = 0, tie_seen = 0;
#pragma unroll
  for (int c = 0; c < NPER; ++c) {
    const uint64_t lt = (1ull << lane) - 1ull;
    const uint64_t tm = __builtin_amdgcn_ballot_w64(key[c] == t);
    const int tie_rank = tie_seen + (int)__builtin_popcountll(tm & lt);
    const bool keep = key[c] > t || (key[c] == t && tie_rank < ties);
    const uint64_t km = __builtin_amdgcn_ballot_w64(keep);
    if (keep) orow[count + (int)__builtin_popcountll(km & lt)] = lane + 64 * c;
    count += (int)__builtin_popcountll(km);
    tie_seen += (int)__builtin_popcountll(tm);
  }
}

// Same selection for long rows: keys recomputed from the (cached) score rows.
__device__ __forceinline__ void select_rows_long(const RowScores& srow, int32_t* __restrict__ orow, int jd,
                                                 int need, int lane) {
  uint32_t t = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial = t | (1u << bit);
    int cnt = 0;
    for (int jb = 0; jb < jd; jb += 64) {
      const int j = jb + lane;
      cnt += wave_count(j < jd && cand_key(srow(j)) >= trial);
    }
    if (cnt >= need) t = trial;
  }
  int greater = 0;
  for (int jb = 0; jb < jd; jb += 64) {
    const int j = jb + lane;
    greater += wave_count(j < jd && cand_key(srow(j)) > t);
  }
  const int ties = need - greater;
  int count = 0, tie_seen = 0;
  for (int jb = 0; jb < jd; jb += 64) {
    const int j = jb + lane;
    const uint32_t k = j < jd ? cand_key(srow(j)) : 0u;
    const uint64_t lt = (1ull << lane) - 1ull;
    const uint64_t tm = __builtin_amdgcn_ballot_w64(k == t && j < jd);
    const int tie_rank = tie_seen + (int)__builtin_popcountll(tm & lt);
    const bool keep = j < jd && (k > t || (k == t && tie_rank < ties));
    const uint64_t km = __builtin_amdgcn_ballot_w64(keep);
    if (keep) orow[count + (int)__builtin_popcountll(km & lt)] = j;
    count += (int)__builtin_popcountll(km);
    tie_seen += (int)__builtin_popcountll(tm);
  }
}

}  // namespace ssa
