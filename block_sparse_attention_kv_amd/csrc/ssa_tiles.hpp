// LDS tile helpers shared by the attention kernels (gfx950): 64x64 bf16 tiles
// stored as 64 rows x 128 B with 16-byte chunks XOR-swizzled by row, filled by
// direct-to-LDS loads, and the explicit waits that order those loads.
//
// Swizzles.  The LDS has 64 four-byte banks (256 bytes per cycle): two rows of
// a tile share a bank set when they have the same parity, so for each read
// pattern the chunk permutation must separate same-parity rows:
//   * MFMA K operand (16-byte reads): 16 consecutive rows, one chunk -> the
//     eight rows of each parity need eight different chunk positions;
//   * transposing V reads of the prefill kernels: rows 4m..4m+3, four aligned
//     chunks -> rows 4m and 4m+2 need disjoint aligned chunk quads;
//   * transposing V reads of the decode kernel: rows 16m..16m+7, two aligned
//     chunks -> rows 16m, +2, +4, +6 need disjoint aligned chunk pairs.
// With u = (row >> 1) & 7, swizzle kind 0 XORs the chunk with rot(u) =
// ((u & 1) << 2) | (u >> 1), kind 1 with ((u & 3) << 1) | (u >> 2); both are
// bijections of u, which serves the K reads.
#pragma once

#include "ssa_common.hpp"

namespace ssa {

constexpr int kTileBytes = kBlock * kHeadDim * 2;  // 8 KB: 64 rows x 128 B
constexpr float kRescaleSlack = 8.f;               // log2 headroom before the reference max moves

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_cvoid;

// Chunk XOR of row `row` under swizzle kind S.
template <int S>
__device__ __forceinline__ int swz_x(int row) {
  const int u = (row >> 1) & 7;
  return S == 0 ? (((u & 1) << 2) | (u >> 1)) : (((u & 3) << 1) | (u >> 2));
}

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` under swizzle kind S.
template <int S>
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ swz_x<S>(row)) << 4));
}

__device__ __forceinline__ lds_void* to_lds(void* p) { return (lds_void*)p; }

// The direct-to-LDS loads are not ordered against later LDS reads by the
// compiler, so the pipeline waits explicitly: vmcnt(N) = at most the N most
// recent vector-memory instructions still in flight (in-order completion for
// loads).  The empty asm and scheduling barriers keep every LDS access on its
// side of the wait.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// All LDS reads of this wave have returned (before a DMA overwrites their buffer).
__device__ __forceinline__ void wait_lds_reads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// One unit's index row into registers: lane e holds entries e + 64c (c < 4),
// -1 past topk.
__device__ __forceinline__ void load_index_row(const int32_t* __restrict__ irow, int topk, int lane, int iv[4]) {
#pragma unroll
  for (int c = 0; c < kMaxTopk / 64; ++c) {
    const int e = lane + 64 * c;
    iv[c] = e < topk ? irow[e] : -1;
  }
}

// A per-entry fp32 row laid out like load_index_row's (0 past topk).
__device__ __forceinline__ void load_value_row(const float* __restrict__ vrow, int topk, int lane, float v[4]) {
#pragma unroll
  for (int c = 0; c < kMaxTopk / 64; ++c) {
    const int e = lane + 64 * c;
    v[c] = e < topk ? vrow[e] : 0.f;
  }
}

// LDS writes of this wave are visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Canonical form of an index row (as loaded by load_index_row) in LDS: the
// distinct blocks j with 0 <= j <= jd, ascending.  A -1 or any other entry
// outside [0, jd] is skipped wherever it stands, and a block listed twice is
// kept once, so the row is read as the set it names.  With VAL each kept block
// carries the value (bv, loaded like iv) of its first listing into vlst.  A row
// that is already strictly ascending is only compacted; any other row is
// ranked entry by entry against a copy in tmp (n^2/64 LDS broadcast reads per
// lane).  Returns the count.  Whole-wave operation; lst, vlst and tmp have
// room for kMaxTopk entries (vlst only with VAL).
template <bool VAL>
__device__ __forceinline__ int canonical_index_row(const int iv[4], const float bv[4], int topk, int jd, int* lst,
                                                   float* vlst, int* tmp, int lane) {
  int n = 0;
#pragma unroll
  for (int c = 0; c < kMaxTopk / 64; ++c) {
    const int e = lane + 64 * c;
    const int j = iv[c];
    const bool keep = e < topk && j >= 0 && j <= jd;
    const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
    if (keep) {
      const int pos = n + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull));
      lst[pos] = j;
      if (VAL) vlst[pos] = bv[c];
    }
    n += (int)__builtin_popcountll(m);
  }
  wave_lds_sync();
  bool unordered = false;
  for (int e = lane + 1; e < n; e += 64) unordered |= lst[e] <= lst[e - 1];
  if (__builtin_amdgcn_ballot_w64(unordered) == 0ull) return n;

  // General row.  tmp: the listing with later listings of a block replaced
  // by a sentinel; each first listing then goes to its rank among the
  // distinct blocks (the values are read before lst and vlst are rewritten).
  for (int e = lane; e < n; e += 64) {
    const int j = lst[e];
    bool first = true;
    for (int f = 0; f < e; ++f) first = first && lst[f] != j;
    tmp[e] = first ? j : 0x7fffffff;
  }
  float vv[kMaxTopk / 64];
#pragma unroll
  for (int c = 0; c < kMaxTopk / 64; ++c) vv[c] = (VAL && lane + 64 * c < n) ? vlst[lane + 64 * c] : 0.f;
  wave_lds_sync();
  int cnt = 0;
#pragma unroll
  for (int c = 0; c < kMaxTopk / 64; ++c) {
    const int e = lane + 64 * c;
    if (64 * c >= n) break;
    const int j = e < n ? tmp[e] : 0x7fffffff;
    int rank = 0;
    for (int f = 0; f < n; ++f) rank += tmp[f] < j ? 1 : 0;
    const bool first = j != 0x7fffffff;
    cnt += (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(first));
    if (first) {
      lst[rank] = j;
      if (VAL) vlst[rank] = vv[c];
    }
  }
  wave_lds_sync();
  return cnt;
}

// One direct-to-LDS load: every lane fetches the 16 bytes at gtile + voff and
// the wave's 1 KB lands at LDS byte address lds_base + 16 * lane.  Issued from
// inline asm so the compiler does not track it; each use is ordered by the
// explicit waits of the pipeline (it has no register outputs: the address
// registers are read at issue).
// NT: the non-temporal cache policy, for data read once (streamed past the
// caches rather than kept in them).
template <bool NT = false>
__device__ __forceinline__ void dma_1k(const uint16_t* gtile, uint32_t voff, uint32_t lds_base) {
  if (NT)
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(gtile), "s"(lds_base)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(gtile), "s"(lds_base)
        : "memory", "m0");
}

// Same load for the partial last tile of a sequence.  The asm text differs so
// the compiler keeps it on its own (rare) path instead of merging the two
// paths into per-load selects.
template <bool NT = false>
__device__ __forceinline__ void dma_1k_ragged(const uint16_t* gtile, uint32_t voff, uint32_t lds_base) {
  if (NT)
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1 nt ; partial tile"
        :
        : "v"(voff), "s"(gtile), "s"(lds_base)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1 ; partial tile"
        :
        : "v"(voff), "s"(gtile), "s"(lds_base)
        : "memory", "m0");
}

// A wave-uniform global pointer, placed in scalar registers (the DMA
// instructions take their base address from an SGPR pair).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const T*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)p);
}

// Transposed MFMA operand from a swizzle-kind-0 tile (64 rows x 64 bf16):
// lane l receives column 32*cb + l%32 of the tile rows
//   row0 + 8*(t/4) + 4*(l/32) + t%4,   t = 0..7 (its 8 k-slots),
// i.e. the row order of the accumulator registers 8*ap .. 8*ap+7 when
// row0 = 32*kb + 16*ap.  Two transposing reads (4 rows x 16 columns per
// 16-lane group each).
__device__ __forceinline__ bf16x8 read_tile_tr(const uint8_t* tile, int row0, int cb, int lane) {
  const int grp = lane >> 4, s16 = lane & 15;
  const int tq = s16 >> 2, qq = s16 & 3;
  const int hh = grp >> 1, gd = grp & 1;
  uint32_t w[4];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = row0 + 8 * rr + 4 * hh + tq;
    const int chunk = 4 * cb + 2 * gd + (qq >> 1);
    const uint32_t off = swz<0>(row, chunk) + 8 * (qq & 1);
    const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)to_lds((void*)(tile + off)));
    const u32x2 tw = __builtin_bit_cast(u32x2, t);
    w[2 * rr] = tw[0];
    w[2 * rr + 1] = tw[1];
  }
  u32x4 va;
  va[0] = w[0]; va[1] = w[1]; va[2] = w[2]; va[3] = w[3];
  return as_bf16x8(va);
}

// Per-lane byte offset (within a tile) of the 16 bytes this lane fetches for
// slice c (rows 8c..8c+7): chunk q of row r is stored at swz(r, q).  Rows at or
// past `nvalid` re-read row 0 of the tile (always present); their contents
// never reach an output (causal mask / unwritten rows).
template <int S>
__device__ __forceinline__ uint32_t slice_offset(int c, int lane, int nvalid) {
  const int row = 8 * c + (lane >> 3);
  // this lane fills LDS slot (row, lane & 7), which holds chunk (lane & 7) ^ x(row)
  const int chunk = (lane & 7) ^ swz_x<S>(row);
  return (uint32_t)((row < nvalid ? row * kHeadDim : 0) + chunk * 8) * 2u;
}

// The offsets of the slices first, first+STEP, ... of a full tile that this
// wavefront requests, computed once (indexed by a compile-time slot).
template <int STEP, int S>
struct TileOffsets {
  static constexpr int kN = 8 / STEP;
  int first;
  uint32_t v[kN];
  __device__ __forceinline__ void init(int lane, int first_slice) {
    first = first_slice;
#pragma unroll
    for (int k = 0; k < kN; ++k) v[k] = slice_offset<S>(first_slice + k * STEP, lane, kBlock);
  }
};

// Request this wavefront's slices of one tile into LDS at `lds`.  Full tiles
// use the precomputed offsets; a partial last tile clamps rows.  NT: tiles
// read once (the non-temporal policy).
template <bool NT = false, int STEP, int S>
__device__ __forceinline__ void tile_load(const uint16_t* gtile, int nvalid, const uint8_t* lds, int lane,
                                          const TileOffsets<STEP, S>& off) {
  const uint32_t base = lds_addr(lds);
  if (nvalid >= kBlock) {
#pragma unroll
    for (int k = 0; k < TileOffsets<STEP, S>::kN; ++k)
      dma_1k<NT>(gtile, off.v[k], __builtin_amdgcn_readfirstlane(base + (off.first + k * STEP) * 1024));
  } else {
    // The lane index passes through an opaque copy here, so that the partial
    // path's offsets are computed on that (rare) path instead of being hoisted
    // out of the tile loop into registers the full path needs.
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int k = 0; k < TileOffsets<STEP, S>::kN; ++k) {
      const int c = off.first + k * STEP;
      dma_1k_ragged<NT>(gtile, slice_offset<S>(c, l, nvalid), __builtin_amdgcn_readfirstlane(base + c * 1024));
    }
  }
}

}  // namespace ssa
