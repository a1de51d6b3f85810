// Backward kernels (gfx950) of the block-sparse forward and of the full causal
// counterpart: given dO, O and the forward's LSE, the gradients dQ, dK, dV of
// the attention output.
//
// With P = exp(scale * Q K^T - LSE) on the keys a row attends to (0 elsewhere)
// and D = rowsum(dO * O):
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//   dQ = scale * dS K,   dK = scale * dS^T Q.
// Method: SSA summary (gist.science 2511.20102), 1 "Planteamiento del
// Problema" (the sparse stream gives keys outside the selected blocks no
// gradient and normalises over the selected subset) and 2 "Mecanismo Central"
// (the full stream passes gradient to every token); the formulas are the chain
// rule through the softmax.
//
// Work is split two ways, so that no gradient is accumulated with atomics and
// the result is bitwise reproducible:
//   * dQ kernel: one workgroup (2 waves, 32 query rows each) per unit
//     (b, query head, query block), walking the unit's key blocks like the
//     forward; it also writes the per-row LSE (log2 units) and D that the
//     key-side kernel reads.  Per tile, transposed as in the forward (a lane
//     owns one query column):  S^T = K Q^T,  dP^T = V dO^T  (Q, dO in
//     registers), then dQ^T += K^T dS^T with K^T read transposed from LDS.
//   * dK/dV kernel: the (query head, query block) pairs of each (batch, KV
//     head) group, numbered key block by key block and in (query block,
//     head) order within one -- the pairs whose list holds key block j
//     (block-sparse: 2 waves of 32 keys on block j), or every pair of key
//     block j (full: 4 waves on blocks j and j+1, which share each pair's
//     tiles; block j+1 skips the pairs wholly in its future) -- are cut into
//     equal contiguous ranges, one per workgroup, so that every workgroup
//     does the same number of pairs whatever the selection.  Per pair,
//     untransposed (a lane owns one key column): S = Q K^T,  dP = dO V^T
//     (K, V in registers), then dV += P^T dO and dK += dS^T Q with dO, Q read
//     transposed from LDS.  A range writes one fp32 partial per key block it
//     touches; a reduce kernel sums the partials of a key block in range
//     order and rounds to bf16.
// The tile loops stream through rings of LDS buffers.  The dQ loop and the
// block-sparse dK/dV loop use two: the next step's tiles are requested while
// a step is computed, and the smaller LDS footprint lets more workgroups
// share a CU.  The full dK/dV loop uses three (requests two steps ahead).
// The pairs of a key block come from a bitmask mask[b, g, j, i] (bit hh: head
// g*G+hh lists j for query block i) built from the index rows with atomic
// ORs (order-independent); the pairs of each key block are then counted from
// the bits, so the range boundaries do not depend on timing.
#include <algorithm>
#include <type_traits>

#include "ssa_common.hpp"
#include "ssa_internal.hpp"
#include "ssa_tiles.hpp"

namespace ssa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSparsePairs = 64;   // pair-list entries per step of a block-sparse range
constexpr int kFullPairs = 1 << 30;  // full ranges need no list: one step per key unit
// dK/dV workgroups in flight at once on a 256-CU device (per CU: four of the
// block-sparse kernel, two of the full one); a launch of this many, split
// over the groups, runs in one round
constexpr int kSparseDkvWorkgroups = 1024;
constexpr int kFullDkvWorkgroups = 512;
constexpr int kRing = 3;           // tile buffers per loop (full dK/dV)
constexpr int kDqRing = 2;         // K/V tile buffers of the dQ loop

// ---------------------------------------------------------------------------- index inversion

__global__ __launch_bounds__(256) void bwd_fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) p[e] = 0u;
}

// One wavefront per index row (b, query head or KV group, query block i): the
// row's entries that name a causal block 0 <= j <= diag(i) set the bits of
// their query heads in mask[b, g, j, i].
__global__ __launch_bounds__(64) void bwd_mask_kernel(const int32_t* __restrict__ idx, uint32_t* __restrict__ mask,
                                                      Geometry geo, int shared) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // (b, head or group, i)
  const int i = row % geo.nqb;
  const int bh = row / geo.nqb;
  const int G = geo.group;
  int gi, bits;
  if (shared) {
    gi = bh;
    bits = G >= 32 ? -1 : (int)((1u << G) - 1u);
  } else {
    const int b = bh / geo.hq, h = bh - b * geo.hq;
    gi = b * geo.hkv + h / G;
    bits = (int)(1u << (h % G));
  }
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  int iv[kMaxTopk / 64];
  load_index_row(idx + (size_t)row * geo.topk, geo.topk, lane, iv);
  // the row is read as the set it names: a -1 or out-of-range entry is
  // skipped wherever it stands, and a repeated block sets the same bit
#pragma unroll
  for (int c = 0; c < kMaxTopk / 64; ++c) {
    const int e = lane + 64 * c;
    const int j = iv[c];
    if (e < geo.topk && j >= 0 && j <= jd)
      atomicOr(mask + ((size_t)gi * geo.nkb + j) * geo.nqb + i, (uint32_t)bits);
  }
}

// ---------------------------------------------------------------------------- dQ

// Four 16-byte pieces of one bf16 row as MFMA operand k-slots: piece ks holds
// columns 16*ks + 8*hl .. +7 (zeros for a row that does not exist).
__device__ __forceinline__ void load_row_op(const uint16_t* rowp, bool valid, int hl, bf16x8 op[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (valid) v = *reinterpret_cast<const u32x4*>(rowp + 16 * ks + 8 * hl);
    op[ks] = as_bf16x8(v);
  }
}

__device__ __forceinline__ float dot_row_ops(const bf16x8 a[4], const bf16x8 b[4]) {
  float acc = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = fmaf((float)a[ks][t], (float)b[ks][t], acc);
  return acc;
}

// Workgroup id -> (KV group gi = b*Hkv + g, unit index within the group, 0 =
// heaviest), dealt so that a KV group's units stay on a fixed subset of the 8
// XCDs when the counts allow (its K and V then stay in that L2).
__device__ __forceinline__ void map_unit_bwd(int w, int n_groups, int per_group, int& gi, int& u) {
  const int n = n_groups * per_group;
  if ((n & 7) == 0 && n_groups <= 8 && (8 % n_groups) == 0) {
    const int x = w & 7, k = w >> 3, xpg = 8 / n_groups;
    gi = x / xpg;
    u = k * xpg + (x - gi * xpg);
  } else if ((n & 7) == 0 && (n_groups & 7) == 0) {
    const int x = w & 7, k = w >> 3, gpx = n_groups >> 3;
    gi = x + 8 * (k % gpx);
    u = k / gpx;
  } else {
    gi = w % n_groups;
    u = w / n_groups;
  }
}

// R: K/V tile buffers in the ring (3: the tile after next is requested while a
// tile is computed; 2: the next one, for less LDS and more workgroups per CU).
// NH: query heads of one KV group per workgroup (two waves each); with NH = 2
// (full backward, or one list per KV group) each K/V tile serves both heads.
template <int R, int NH>
__global__ __launch_bounds__(128 * NH, 2) void attn_bwd_dq_kernel(BwdArgs a, Geometry geo) {
  constexpr int kTileReq = 8 / NH;  // requests per wave per tile (its K and V slices)
  __shared__ __attribute__((aligned(1024))) uint8_t sK[R][kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[R][kTileBytes];
  __shared__ int sList[2 * NH][kMaxTopk];
  __shared__ int sTmp[2 * NH][kMaxTopk];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = geo.group;
  int gi, u;
  const int GU = G / NH;  // workgroups per (KV group, query block)
  map_unit_bwd(blockIdx.x, geo.batch * geo.hkv, GU * a.qb_count, gi, u);
  const int i = a.qb_begin + a.qb_count - 1 - u / GU;  // longest rows first
  const int b = gi / geo.hkv, g = gi - b * geo.hkv;
  const int h = g * G + (u - (u / GU) * GU) * NH + (wave >> 1);
  const int bh = b * geo.hq + h;
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  const size_t kvoff = (size_t)gi * geo.seq_kv * kHeadDim;
  const uint16_t* kbase = a.k + kvoff;
  const uint16_t* vbase = a.v + kvoff;

  const int row = i * kBlock + 32 * (wave & 1) + l32;  // this lane's query row
  const bool vrow = row < geo.seq_q;
  const int orow = row - a.qb_begin * kBlock;    // its row in the slice-shaped tensors
  int nt = jd + 1;
  if (!a.full) {
    const int irow = a.idx_shared ? gi : bh;
    int iv[kMaxTopk / 64];
    load_index_row(a.idx + ((size_t)irow * geo.nqb + i) * geo.topk, geo.topk, lane, iv);
    nt = canonical_index_row<false>(iv, nullptr, geo.topk, jd, sList[wave], nullptr, sTmp[wave], lane);
  }
  bf16x8 qop[4], dop[4], oop[4];
  load_row_op(a.q + ((size_t)bh * geo.seq_q + (vrow ? row : 0)) * kHeadDim, vrow, hl, qop);
  const size_t srow = (size_t)bh * a.rows_out + (vrow ? orow : 0);
  load_row_op(a.dout + srow * kHeadDim, vrow, hl, dop);
  load_row_op(a.o + srow * kHeadDim, vrow, hl, oop);
  const float lse = vrow ? a.lse[srow] : 0.f;
  auto tile_block = [&](int t) { return a.full ? t : __builtin_amdgcn_readfirstlane(sList[wave][t]); };
  TileOffsets<2 * NH, 0> toff;
  toff.init(lane, wave);
  // requests of tile t into ring buffer BUF (a compile-time index, so that
  // every LDS address below is a fixed per-lane offset plus an immediate)
  auto issue = [&](auto BUF, int t) {
    constexpr int buf = decltype(BUF)::value;
    const int jn = tile_block(t);
    const size_t off = (size_t)jn * kBlock * kHeadDim;
    const int nv = geo.seq_kv - jn * kBlock;
    tile_load(kbase + off, nv, sK[buf], lane, toff);
    tile_load(vbase + off, nv, sV[buf], lane, toff);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  static_assert(R == 2 || R == 3, "the tile loop is unrolled over a two- or three-buffer ring");
  if (nt > 0) issue(B0{}, 0);
  if (R == 3 && nt > 1) issue(B1{}, 1);
  // per-row constants: LSE in log2 units (+inf where the row has no keys or
  // does not exist, so that every P is 0) and D = dO . O
  const float dsum = sum_xor32(dot_row_ops(dop, oop));
  const float lse2 = (vrow && lse > -__builtin_inff()) ? lse * kLog2e : __builtin_inff();
  if (hl == 0) {
    const size_t prow = (size_t)bh * (a.qb_count * kBlock) + (row - a.qb_begin * kBlock);
    a.lse2[prow] = lse2;
    a.delta[prow] = vrow ? dsum : 0.f;
  }
  f32x16 dq[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;
  const float c = geo.scale_log2;
  const int pos = geo.q_offset + row;
  auto step = [&](auto BUF, int t) {
    constexpr int buf = decltype(BUF)::value;
    const int j = tile_block(t);
    // this wave's share of tile t landed (with three buffers tile t+1's
    // requests may still be in flight)
    if (R == 3 && t + 1 < nt)
      wait_vmem<kTileReq>();
    else
      wait_vmem<0>();
    __syncthreads();  // every wave's share; every wave is done with tile t-1
    if (t + R - 1 < nt) issue(std::integral_constant<int, (buf + R - 1) % R>{}, t + R - 1);
    const uint8_t* tK = sK[buf];
    const uint8_t* tV = sV[buf];
    const bool diag = j == jd;
    int qrel = pos - j * kBlock;  // query position relative to the tile's first key
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 ka[4], va[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ka[ks] = *reinterpret_cast<const bf16x8*>(tK + swz<0>(32 * kb + l32, 2 * ks + hl));
        va[ks] = *reinterpret_cast<const bf16x8*>(tV + swz<0>(32 * kb + l32, 2 * ks + hl));
      }
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = mfma32(ka[ks], qop[ks], s);    // S^T: rows keys, columns queries
        dp = mfma32(va[ks], dop[ks], dp);  // dP^T
      }
      if (diag) {
        // the tile holding the rows' own positions: a key after the query gets -inf
        asm volatile("" : "+v"(qrel));  // keep the mask inside this branch
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          const uint32_t neg_inf_if_future = (uint32_t)((qrel - kr) >> 31) & 0xFF800000u;
          s[r] += __uint_as_float(neg_inf_if_future);
        }
      }
      // dS^T = P^T * (dP^T - D), P^T = exp2(S^T * c - LSE2)
      u32x4 pds[2];
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float d2[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int r = 8 * ap + 2 * e + x;
            const float p = fast_exp2(fmaf(s[r], c, -lse2));
            d2[x] = p * (dp[r] - dsum);
          }
          pds[ap][e] = pack_bf16x2(d2[0], d2[1]);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
#pragma unroll
        for (int db = 0; db < 2; ++db)
          dq[db] = mfma32(read_tile_tr(tK, 32 * kb + 16 * ap, db, lane), as_bf16x8(pds[ap]), dq[db]);
    }
  };
  for (int t0 = 0; t0 < nt; t0 += R) {
    step(B0{}, t0);
    if (t0 + 1 < nt) step(B1{}, t0 + 1);
    if (R == 3 && t0 + 2 < nt) step(std::integral_constant<int, 2 % R>{}, t0 + 2);
  }
  if (vrow) {
    uint16_t* qp = a.dq + ((size_t)bh * a.rows_out + orow) * kHeadDim;
    const float sc = geo.scale;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 w;
        w[0] = pack_bf16x2(dq[db][4 * rg] * sc, dq[db][4 * rg + 1] * sc);
        w[1] = pack_bf16x2(dq[db][4 * rg + 2] * sc, dq[db][4 * rg + 3] * sc);
        *reinterpret_cast<u32x2*>(qp + 32 * db + 8 * rg + 4 * hl) = w;
      }
  }
}

// ---------------------------------------------------------------------------- dK / dV

// One dword per lane of a 64-float row, direct to LDS.
__device__ __forceinline__ void dma_row64(const float* g, uint32_t lds_base, int lane) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"((uint32_t)lane * 4u), "s"(g), "s"(lds_base)
      : "memory", "m0");
}

// pairs[gi, j] = number of head bits of key block j over its query blocks
// (one wavefront per (group, key block)).
__global__ __launch_bounds__(64) void bwd_count_kernel(BwdArgs a, Geometry geo) {
  const int lane = threadIdx.x;
  const int gi = blockIdx.x / geo.nkb, j = blockIdx.x - gi * geo.nkb;
  const BwdPlan pl = a.plan;
  const uint32_t* m = a.mask + ((size_t)gi * geo.nkb + j) * geo.nqb;
  int cnt = 0;
  for (int i = pl.first_block(j) + lane; i < pl.hi; i += 64) cnt += __builtin_popcount(m[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) a.pairs[blockIdx.x] = cnt;
}

// Exclusive scan over key units of each group's pair counts:
// pair_base[gi, u] = first pair of key unit u, pair_base[gi, nku] = the
// group's pairs.
__global__ __launch_bounds__(256) void bwd_pair_scan_kernel(BwdArgs a, Geometry geo) {
  __shared__ int sTot[256];
  const int gi = blockIdx.x, tid = threadIdx.x;
  const BwdPlan pl = a.plan;
  const int nku = pl.n_units(geo.nkb);
  const int per = (nku + 255) / 256;
  const int u0 = min(nku, tid * per), u1 = min(nku, u0 + per);
  auto pairs = [&](int u) {
    const int j = u * pl.kpb;  // the unit's first key block: its pairs are the unit's
    return a.full ? geo.group * pl.n_blocks(j) : a.pairs[(size_t)gi * geo.nkb + j];
  };
  int tot = 0;
  for (int u = u0; u < u1; ++u) tot += pairs(u);
  sTot[tid] = tot;
  __syncthreads();
  int base = 0;
  for (int t = 0; t < tid; ++t) base += sTot[t];
  int* pb = a.pair_base + (size_t)gi * (geo.nkb + 1);
  for (int u = u0; u < u1; ++u) {
    pb[u] = base;
    base += pairs(u);
  }
  if (tid == 255) pb[nku] = base;
}

// Workgroups a group's pairs are cut into (at most one pair each), and the
// first pair of range s: floor(s * n / slots).
__device__ __forceinline__ int range_slots(const BwdPlan& pl, int n) { return min(pl.slots, n); }
__device__ __forceinline__ int range_begin(int s, int n, int slots) {
  return (int)(((long long)s * n) / slots);
}
// The range that holds pair x (ranges are non-empty as slots <= n).
__device__ __forceinline__ int range_of(int x, int n, int slots) {
  return (int)((((long long)x + 1) * slots - 1) / n);
}

// KPB key blocks per key unit (1: block-sparse, 2: full), two waves of 32
// keys per block; the waves share every pair's Q and dO tiles.  Workgroup
// (s, group) walks range s of the group's pairs, key unit by key unit, P
// pairs per step.
// R: pair buffers in the ring (3: the pair after next is requested while a
// pair is computed; 2: the next one, for less LDS and more workgroups per CU).
template <int KPB, int R = kRing>
__global__ __launch_bounds__(128 * KPB, 2) void attn_bwd_dkv_kernel(BwdArgs a, Geometry geo) {
  constexpr int NW = 2 * KPB;                      // waves
  constexpr int kLoadsPerPair = 2 * (8 / NW) + 1;  // per wave: its Q and dO tile slices and one row
  __shared__ __attribute__((aligned(1024))) uint8_t sQ[R][kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sO[R][kTileBytes];  // dO tiles
  __shared__ __attribute__((aligned(256))) float sL[R][kBlock];          // LSE (log2 units)
  __shared__ __attribute__((aligned(256))) float sD[R][kBlock];          // D
  __shared__ int sPairs[kSparsePairs];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = geo.group;
  const BwdPlan pl = a.plan;
  // workgroup -> (group, range): the dispatcher deals workgroups to the 8 XCDs
  // round-robin, so each XCD gets a contiguous run of ranges (a span of key
  // blocks, whose pairs share more of their Q/dO tiles in that XCD's L2):
  // 2-3% faster than ranges dealt across the XCDs
  const int nb = gridDim.x;
  const int lin = (nb & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3));
  const int gi = lin / pl.slots;
  const int rs = lin - gi * pl.slots;  // this workgroup's range
  const int* pb = a.pair_base + (size_t)gi * (geo.nkb + 1);
  const int nku = pl.n_units(geo.nkb);
  const int npg = __builtin_amdgcn_readfirstlane(pb[nku]);  // the group's pairs
  const int nrs = range_slots(pl, npg);
  if (rs >= nrs) return;  // the whole workgroup: no barrier is passed before this
  const int x_end = range_begin(rs + 1, npg, nrs);
  const int b = gi / geo.hkv, g = gi - b * geo.hkv;
  const int kblk = wave >> 1, kw = wave & 1;  // this wave's key block within the unit, and 32-key half
  TileOffsets<NW, 0> toff;
  toff.init(lane, wave);
  const size_t rows_pad = (size_t)a.qb_count * kBlock;
  const float c = geo.scale_log2;
  // the key unit that holds the range's first pair: the last u with pb[u] <= x
  int x = range_begin(rs, npg, nrs);
  int ku = 0;
  for (int lo = 0, hi = nku; lo < hi;) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(pb[mid]) <= x)
      lo = mid;
    else
      hi = mid - 1;
    ku = lo;
  }
  for (; x < x_end; ++ku) {
  const int ub = __builtin_amdgcn_readfirstlane(pb[ku]);
  const int ue = __builtin_amdgcn_readfirstlane(pb[ku + 1]);
  if (ue <= x) continue;  // a key unit with no pairs
  const int j0 = ku * KPB;        // the unit's first key block: its pairs are the unit's
  const int j = j0 + kblk;        // this wave's key block
  const bool kvalid = j < geo.nkb;
  const int ifirst = pl.first_block(j0);
  const int p_end = min(x_end, ue) - ub;  // the range's pairs of this unit: x - ub .. p_end - 1

  // this wave's 32 keys as MFMA B operands (rows past seq_kv re-read a valid
  // row; such keys lie in the future of every query and are masked)
  const int key = j * kBlock + 32 * kw + l32;
  const int krow = min(key, geo.seq_kv - 1);
  bf16x8 kop[4], vop[4];
  load_row_op(a.k + ((size_t)gi * geo.seq_kv + krow) * kHeadDim, true, hl, kop);
  load_row_op(a.v + ((size_t)gi * geo.seq_kv + krow) * kHeadDim, true, hl, vop);
  // The operands are consumed here, so the compiler waits for them once,
  // before the pair loop.  Left to the first MFMA that reads them, its waits
  // stay inside the loop, where the vector-memory counter also holds the next
  // pairs' tile requests (issued by inline asm, which it does not track), and
  // each step would wait for those to land.
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(kop[ks]), "+v"(vop[ks]));
  f32x16 dk[2], dv[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  for (int p_lo = x - ub, npairs; p_lo < p_end; p_lo += npairs) {
  npairs = __builtin_amdgcn_readfirstlane(min(pl.P, p_end - p_lo));
  __syncthreads();  // every wave is done with the previous step's buffers and pair list

  if (!a.full) {
    // this step's pairs: numbers p_lo .. p_lo + npairs - 1 of key block j, in
    // (query block, head) order, from the head bits of query blocks ifirst..
    if (wave == 0) {
      int before = 0;  // pairs of the query blocks already passed
      for (int i0 = ifirst; i0 < pl.hi && before < p_lo + npairs; i0 += 64) {
        const int ii = i0 + lane;
        const uint32_t bits = ii < pl.hi ? a.mask[((size_t)gi * geo.nkb + j0) * geo.nqb + ii] : 0u;
        const int cnt = __builtin_popcount(bits);
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (lane >= o) incl += y;
        }
        int pos = before + incl - cnt;
        uint32_t m = bits;
        while (m) {
          const int hh = __builtin_ctz(m);
          m &= m - 1u;
          if (pos >= p_lo && pos < p_lo + npairs) sPairs[pos - p_lo] = (ii << 8) | hh;
          ++pos;
        }
        before += __shfl(incl, 63, 64);
      }
    }
    __syncthreads();
  }
  auto pair_of = [&](int p, int& ii, int& hh) {
    if (a.full) {
      const int q = p_lo + p;
      ii = ifirst + q / G;
      hh = q - (q / G) * G;
    } else {
      const int e = __builtin_amdgcn_readfirstlane(sPairs[p]);
      ii = e >> 8;
      hh = e & 255;
    }
  };

  // requests of pair p into ring buffer BUF (a compile-time index, so that
  // every LDS address below is a fixed per-lane offset plus an immediate)
  auto issue = [&](auto BUF, int p) {
    constexpr int buf = decltype(BUF)::value;
    int ii, hh;
    pair_of(p, ii, hh);
    const int bh = b * geo.hq + g * G + hh;
    const int nv = geo.seq_q - ii * kBlock;
    tile_load(a.q + ((size_t)bh * geo.seq_q + (size_t)ii * kBlock) * kHeadDim, nv, sQ[buf], lane, toff);
    const int orow0 = (ii - a.qb_begin) * kBlock;
    tile_load(a.dout + ((size_t)bh * a.rows_out + orow0) * kHeadDim, a.rows_out - orow0, sO[buf], lane, toff);
    const size_t prow = (size_t)bh * rows_pad + orow0;
    // every wave requests one row (with four waves each row twice, same bytes),
    // so that all waves count the same loads per pair
    if (kw == 0)
      dma_row64(a.lse2 + prow, lds_addr(sL[buf]), lane);
    else
      dma_row64(a.delta + prow, lds_addr(sD[buf]), lane);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  static_assert(R == 2 || R == 3, "the pair loop is unrolled over a two- or three-buffer ring");
  if (npairs > 0) issue(B0{}, 0);
  if (R == 3 && npairs > 1) issue(B1{}, 1);

  auto step = [&](auto BUF, int p) {
    constexpr int buf = decltype(BUF)::value;
    int ii, hh;
    pair_of(p, ii, hh);
    // this wave's share of pair p landed (with three buffers pair p+1's
    // requests may still be in flight)
    if (R == 3 && p + 1 < npairs)
      wait_vmem<kLoadsPerPair>();
    else
      wait_vmem<0>();
    __syncthreads();  // every wave's share; every wave is done with pair p-1
    if (p + R - 1 < npairs) issue(std::integral_constant<int, (buf + R - 1) % R>{}, p + R - 1);
    const uint8_t* tQ = sQ[buf];
    const uint8_t* tO = sO[buf];
    const float* tL = sL[buf];
    const float* tD = sD[buf];
    const int dblk = (geo.q_offset + ii * kBlock) / kBlock;  // the query block's diagonal key block
    // a later block of the unit may lie wholly in this query block's future
    if (!kvalid || j > dblk) return;
    const bool diag = j == dblk;
    int kpos = key - (geo.q_offset + ii * kBlock);  // key position relative to the block's first row
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      bf16x8 qa[4], oa[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qa[ks] = *reinterpret_cast<const bf16x8*>(tQ + swz<0>(32 * qb + l32, 2 * ks + hl));
        oa[ks] = *reinterpret_cast<const bf16x8*>(tO + swz<0>(32 * qb + l32, 2 * ks + hl));
      }
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = mfma32(qa[ks], kop[ks], s);    // S: rows queries, columns keys
        dp = mfma32(oa[ks], vop[ks], dp);  // dP
      }
      if (diag) {
        // the key-query block on the diagonal: a key after the query's position gets -inf
        asm volatile("" : "+v"(kpos));  // keep the mask inside this branch
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * qb + 8 * (r >> 2) + 4 * hl + (r & 3);
          const uint32_t neg_inf_if_future = (uint32_t)((m - kpos) >> 31) & 0xFF800000u;
          s[r] += __uint_as_float(neg_inf_if_future);
        }
      }
      u32x4 pp[2], pds[2];
#pragma unroll
      for (int ap = 0; ap < 2; ++ap) {
#pragma unroll
        for (int rg2 = 0; rg2 < 2; ++rg2) {
          const int m0 = 32 * qb + 16 * ap + 8 * rg2 + 4 * hl;  // query rows m0 .. m0+3
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(tL + m0);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(tD + m0);
          float pv[4], dv4[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 8 * ap + 4 * rg2 + x;
            const float p = fast_exp2(fmaf(s[r], c, -l4[x]));
            pv[x] = p;
            dv4[x] = p * (dp[r] - d4[x]);
          }
          pp[ap][2 * rg2] = pack_bf16x2(pv[0], pv[1]);
          pp[ap][2 * rg2 + 1] = pack_bf16x2(pv[2], pv[3]);
          pds[ap][2 * rg2] = pack_bf16x2(dv4[0], dv4[1]);
          pds[ap][2 * rg2 + 1] = pack_bf16x2(dv4[2], dv4[3]);
        }
      }
      // dV += P^T dO,  dK += dS^T Q   (contraction over this half's 32 queries)
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          dv[db] = mfma32(as_bf16x8(pp[ap]), read_tile_tr(tO, 32 * qb + 16 * ap, db, lane), dv[db]);
          dk[db] = mfma32(as_bf16x8(pds[ap]), read_tile_tr(tQ, 32 * qb + 16 * ap, db, lane), dk[db]);
        }
    }
  };
  for (int p0 = 0; p0 < npairs; p0 += R) {
    step(B0{}, p0);
    if (p0 + 1 < npairs) step(B1{}, p0 + 1);
    if (R == 3 && p0 + 2 < npairs) step(std::integral_constant<int, 2 % R>{}, p0 + 2);
  }
  }  // steps
  x = ub + p_end;
  // partial sums of block kblk over this range's pairs of the unit (piece
  // rs + ku of the group): [2][64 keys][64 d] fp32 (dK unscaled)
  if (!kvalid) continue;
  float* pk = a.part + (((size_t)gi * pl.n_pieces(geo.nkb) + rs + ku) * KPB + kblk) * (2 * kBlock * kHeadDim);
  if constexpr (KPB == 1) {
    // this lane's offset, opaque so that the 32 per-register offsets are
    // formed here rather than hoisted out of the unit loop, where they are
    // spilled (measured: 4% faster for this kernel, 3% slower for KPB = 2)
    pk = const_cast<float*>(uniform_ptr(pk));
    int lo = 4 * hl * kHeadDim + l32;
    asm volatile("" : "+v"(lo));
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = lo + (32 * kw + 8 * (r >> 2) + (r & 3)) * kHeadDim + 32 * db;
        pk[o] = dk[db][r];
        pk[kBlock * kHeadDim + o] = dv[db][r];
      }
  } else {
    float* pv = pk + kBlock * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 32 * kw + 8 * (r >> 2) + 4 * hl + (r & 3);
        pk[kr * kHeadDim + 32 * db + l32] = dk[db][r];
        pv[kr * kHeadDim + 32 * db + l32] = dv[db][r];
      }
  }
  }
}

// Sum the partials of each key block in range order: dK = scale * sum,
// dV = sum, rounded to bf16 (zero for a block no pair attends to).  One
// thread per 4 columns of a key row.
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(BwdArgs a, Geometry geo) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t per_group = (size_t)geo.seq_kv * (kHeadDim / 4);
  if (t >= (size_t)geo.batch * geo.hkv * per_group) return;
  const int gi = (int)(t / per_group);
  const int rem = (int)(t - (size_t)gi * per_group);
  const int key = rem / (kHeadDim / 4);
  const int c4 = rem - key * (kHeadDim / 4);
  const int j = key / kBlock, kr = key - j * kBlock;
  const BwdPlan pl = a.plan;
  const int kpb = pl.kpb;
  const int ku = j / kpb, kblk = j - ku * kpb;  // key unit of block j, and j's place in it
  const int* pb = a.pair_base + (size_t)gi * (geo.nkb + 1);
  const int npg = pb[pl.n_units(geo.nkb)];
  const int ub = pb[ku], ue = pb[ku + 1];
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  if (ue > ub) {
    // the ranges that hold the unit's first and last pairs, and every one between
    const int nrs = range_slots(pl, npg);
    const int s0 = range_of(ub, npg, nrs), s1 = range_of(ue - 1, npg, nrs);
    const size_t piece_floats = (size_t)kpb * 2 * kBlock * kHeadDim;
    const float* base = a.part + ((size_t)gi * pl.n_pieces(geo.nkb) + s0 + ku) * piece_floats +
                        (size_t)kblk * 2 * kBlock * kHeadDim + kr * kHeadDim + 4 * c4;
    for (int e = 0; e <= s1 - s0; ++e) {
      const float* pe = base + (size_t)e * piece_floats;
      sk += *reinterpret_cast<const f32x4*>(pe);
      sv += *reinterpret_cast<const f32x4*>(pe + kBlock * kHeadDim);
    }
  }
  const size_t o = ((size_t)gi * geo.seq_kv + key) * kHeadDim + 4 * c4;
  u32x2 wk, wv;
  wk[0] = pack_bf16x2(sk[0] * geo.scale, sk[1] * geo.scale);
  wk[1] = pack_bf16x2(sk[2] * geo.scale, sk[3] * geo.scale);
  wv[0] = pack_bf16x2(sv[0], sv[1]);
  wv[1] = pack_bf16x2(sv[2], sv[3]);
  *reinterpret_cast<u32x2*>(a.dk + o) = wk;
  *reinterpret_cast<u32x2*>(a.dv + o) = wv;
}

}  // namespace

void bwd_plan(const Geometry& g, bool full, int qb_begin, int qb_count, BwdPlan* plan, size_t off[6],
              size_t* total) {
  BwdPlan p;
  p.lo = qb_begin;
  p.hi = qb_begin + qb_count;
  p.qoffb = g.q_offset / kBlock;
  p.P = full ? kFullPairs : kSparsePairs;
  p.kpb = full ? 2 : 1;
  const long long ngroups = (long long)g.batch * g.hkv;
  const long long wgs = full ? kFullDkvWorkgroups : kSparseDkvWorkgroups;
  p.slots = (int)std::max<long long>(1, ngroups > 0 ? wgs / ngroups : 1);
  long long pairs = 0;  // every (head, query block) pair present
  for (int j = 0; j < g.nkb; j += p.kpb) pairs += (long long)g.group * p.n_blocks(j);
  if (!full) {
    // a list names at most min(topk, diag + 1) distinct blocks
    long long listed = 0;
    for (int i = p.lo; i < p.hi; ++i) listed += std::min<long long>(g.topk, (long long)p.qoffb + i + 1);
    pairs = std::min(pairs, (long long)g.group * listed);
  }
  p.max_pairs = pairs;
  // no more ranges than pairs (a range holds one pair at least)
  p.slots = (int)std::max<long long>(1, std::min<long long>(p.slots, pairs));
  *plan = p;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)g.batch * g.hq * qb_count * kBlock;
  size_t o = 0;
  off[0] = o;
  o += up(rows * sizeof(float));
  off[1] = o;
  o += up(rows * sizeof(float));
  off[2] = o;
  if (!full) o += (size_t)ngroups * g.nkb * g.nqb * sizeof(uint32_t);
  off[3] = o;
  if (!full) o += (size_t)ngroups * g.nkb * sizeof(int);
  o = up(o);
  off[4] = o;
  o += up((size_t)ngroups * (g.nkb + 1) * sizeof(int));
  off[5] = o;
  o += up((size_t)ngroups * p.n_pieces(g.nkb) * p.kpb * 2 * kBlock * kHeadDim * sizeof(float));
  *total = o;
}

hipError_t launch_attn_backward(const BwdArgs& a, const Geometry& g, hipStream_t stream) {
  const size_t units = (size_t)g.batch * g.hq * a.qb_count;
  if (units == 0) return hipSuccess;
  const size_t ngroups = (size_t)g.batch * g.hkv;
  if (!a.full) {
    const size_t words = ngroups * g.nkb * g.nqb;
    const unsigned zb = (unsigned)std::min<size_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(bwd_fill_zero_kernel, dim3(zb), dim3(256), 0, stream, a.mask, words);
    const size_t rows = (size_t)g.batch * (a.idx_shared ? g.hkv : g.hq) * g.nqb;
    hipLaunchKernelGGL(bwd_mask_kernel, dim3((unsigned)rows), dim3(64), 0, stream, a.idx, a.mask, g, a.idx_shared);
    hipLaunchKernelGGL(bwd_count_kernel, dim3((unsigned)(ngroups * g.nkb)), dim3(64), 0, stream, a, g);
  }
  hipLaunchKernelGGL(bwd_pair_scan_kernel, dim3((unsigned)ngroups), dim3(256), 0, stream, a, g);
  // heads that walk the same tiles (full, or one list per KV group) pair up
  if ((a.full || a.idx_shared) && g.group % 2 == 0)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<kDqRing, 2>), dim3((unsigned)(units / 2)), dim3(256), 0, stream, a, g);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<kDqRing, 1>), dim3((unsigned)units), dim3(128), 0, stream, a, g);
  // one workgroup per range of each group's pairs (ranges past a group's
  // pair count leave at once)
  const size_t grid = ngroups * (size_t)a.plan.slots;
  if (a.plan.kpb == 2)
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a, g);
  else
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<1, 2>), dim3((unsigned)grid), dim3(128), 0, stream, a, g);
  const size_t threads = ngroups * g.seq_kv * (kHeadDim / 4);
  if (threads > 0)
    hipLaunchKernelGGL(attn_bwd_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a, g);
  return hipGetLastError();
}

}  // namespace ssa
