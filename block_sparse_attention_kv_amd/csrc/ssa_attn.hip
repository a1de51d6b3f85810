// Prefill attention kernels (gfx950): block-sparse forward over the selected
// key blocks, and the full causal counterpart that also emits the dropped mass.
//
// A wavefront owns one unit = (b, query head, 64-row query block) and walks
// its 64-key tiles: the selected blocks (sparse) or every causal block (full).
// Per tile, computed transposed so that a lane owns query columns:
//   S^T = K Q^T      bf16 MFMA 32x32x16, fp32 accumulate; Q^T stays in registers
//   softmax          fp32 in the log2 domain; the row max is lane-local plus one
//                    swap between lane halves; the reference max only moves when
//                    a row's max grows by more than 2^8 (lazy rescale); row sums
//                    accumulate the fp32 probabilities
//   O^T += V^T P^T   bf16 MFMA; P^T comes straight from the S^T accumulators, V^T
//                    from transposing LDS reads of the row-major V tile
// Tiles move HBM/L2 -> LDS by direct-to-LDS loads (no register staging) into
// 16-byte-chunk XOR-swizzled buffers.  The sparse kernel gives each wave its
// own K and V buffers and refills K while the softmax and PV of the current
// tile run, V while the next S runs.  The full kernel runs 4 query heads of a
// KV group per workgroup; they need the same tiles, so each tile is fetched
// once into a double buffer shared by the 4 waves.  The full kernel keeps a
// second running sum over tiles that are not selected, under the same
// reference max, so dropped mass = l_dropped / l_total falls out of one pass.
//
// Method: SSA summary (gist.science 2511.20102), "Mecanismo Central" (sparse
// and full attention streams) and "Alineacion Bidireccional" (counterpart
// output, dropped mass); SSA guide (mauroscia.it), "Block-sparse attention e
// Receptive Field"; S2O summary, "Permutacion en Linea" (tiles gathered by
// index from an unchanged HBM layout).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"
#include "ssa_tiles.hpp"

namespace ssa {
namespace {

constexpr float kLog2eF = 1.4426950408889634f;

struct UnitState {
  f32x16 o[2][2];  // O^T accumulators [d block][query block]
  float m[2];      // reference max (log2 units) per owned query column
  float l[2];      // running sum (this lane's keys)
};

__device__ __forceinline__ void load_q(const uint16_t* qbase, int i, int seq_q, int l32, int hl, bf16x8 qop[2][4]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = i * kBlock + 32 * qb + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < seq_q) v = *reinterpret_cast<const u32x4*>(qbase + (size_t)row * kHeadDim + 16 * ks + 8 * hl);
      qop[qb][ks] = as_bf16x8(v);
    }
  }
}

__device__ __forceinline__ void init_state(UnitState& st) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[x][y][r] = 0.f;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    st.m[qb] = -__builtin_inff();
    st.l[qb] = 0.f;
  }
}

// S^T = K Q^T for one tile: rows = keys 32*kb + 8*(r/4) + 4*hl + r%4, columns = queries.
// All K operands are read before the MFMA burst so the LDS latency overlaps.
__device__ __forceinline__ void tile_scores(const uint8_t* sK, const bf16x8 qop[2][4], int l32, int hl,
                                            f32x16 s[2][2]) {
  bf16x8 ka[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      ka[kb][ks] = *reinterpret_cast<const bf16x8*>(sK + swz<0>(32 * kb + l32, 2 * ks + hl));
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma32(ka[kb][ks], qop[qb][ks], s[kb][qb]);
  }
  // keep the reads ahead of the products: the compiler otherwise reuses one
  // operand register set and waits for each read in turn
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
}

// p = 2^(c s + b2 - m) of a tile against the reference max m, packed to bf16
// pairs in pk, and this lane's fp32 sum per query block in rs.
template <bool BIAS>
__device__ __forceinline__ void tile_probs(const f32x16 s[2][2], const UnitState& st, u32x4 pk[2][2][2], float c,
                                           float b2, float rs[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    // a block whose bias is -inf (prior weight 0) adds nothing, whatever the reference max
    const float nm = BIAS ? (b2 == -__builtin_inff() ? -__builtin_inff() : b2 - st.m[qb]) : -st.m[qb];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[kb][qb][8 * ap + 2 * e], c, nm));
          const float p1 = fast_exp2(fmaf(s[kb][qb][8 * ap + 2 * e + 1], c, nm));
          pk[kb][ap][qb][e] = pack_bf16x2(p0, p1);
          rs0 += p0;
          rs1 += p1;
        }
    rs[qb] = rs0 + rs1;
  }
}

// Online-softmax update for one tile; leaves packed bf16 probabilities in pk.
// tile_rs (optional) receives this lane's fp32 sum of the tile's
// probabilities per query block (relative to the updated reference max).
// With BIAS, b2 (log2 units) is added to every logit of the tile.
// FULL: the running sum over unselected tiles is kept in LDS at ld[0] and
// ld[64] (one slot per lane and query block).  In registers the compiler
// spills it, and the spill's reload waits for every vector memory operation
// in flight, the next tile's K/V requests included.
template <bool FULL, bool BIAS = false>
__device__ __forceinline__ void tile_softmax(f32x16 s[2][2], UnitState& st, u32x4 pk[2][2][2], bool diag,
                                             bool selected, int key0, int pos0, int l32, int hl, float c,
                                             float* tile_rs = nullptr, float b2 = 0.f, bool first = false,
                                             float* ld = nullptr) {
  if (diag) {
    // Causal mask of the tile holding the query rows' own positions: key > pos
    // becomes -inf.  Branch-free sign arithmetic (no compare masks to keep live).
    int base = key0 - pos0 + 4 * hl - l32;  // key - pos at kb = qb = r = 0
    asm volatile("" : "+v"(base));  // opaque: the mask is built here, not hoisted out of the tile loop
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = base + 32 * (kb - qb) + 8 * (r >> 2) + (r & 3);  // key - pos
          const uint32_t neg_inf_if_future = (uint32_t)((-e) >> 31) & 0xFF800000u;
          s[kb][qb][r] += __uint_as_float(neg_inf_if_future);
        }
  }
  // Probabilities against the running reference max, without this tile's
  // own max: kept while no row's sum over this lane's 32 values exceeds
  // 32 * 2^kRescaleSlack, so no probability is more than 2^13 times the
  // reference (ample headroom for the fp32 sums).  Otherwise -- a first tile
  // (reference -inf), values far above the reference, a NaN -- the tile
  // takes the exact step: its row max, the rescale of the state, the
  // probabilities again.
  // A unit's first tile (reference -inf) goes to the exact step directly.
  float rs[2] = {0.f, 0.f};
  if (!first) tile_probs<BIAS>(s, st, pk, c, b2, rs);
  constexpr float kFastSumLimit = 32.f * (1 << (int)kRescaleSlack);
  if (first || __builtin_amdgcn_ballot_w64(!(rs[0] <= kFastSumLimit) || !(rs[1] <= kFastSumLimit)) != 0ull) {
    float mt[2];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = max_nan(s[0][qb][0], s[0][qb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = max_nan(max_nan(mx, s[0][qb][r]), s[0][qb][r + 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = max_nan(max_nan(mx, s[1][qb][r]), s[1][qb][r + 1]);
      mx = max_nan_xor32(mx);
      mt[qb] = BIAS ? fmaf(mx, c, b2) : mx * c;
      grow |= !(mt[qb] <= st.m[qb] + kRescaleSlack);
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mn = fmaxf(st.m[qb], mt[qb]);
        const float alpha = fast_exp2(st.m[qb] - mn);
        st.m[qb] = mn;
        st.l[qb] *= alpha;
        if (FULL) ld[64 * qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) st.o[db][qb][r] *= alpha;
      }
    }
    tile_probs<BIAS>(s, st, pk, c, b2, rs);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (tile_rs) tile_rs[qb] = rs[qb];
    st.l[qb] += rs[qb];
    if (FULL && !selected) ld[64 * qb] += rs[qb];
  }
}

// O^T += V^T P^T.  16-key step (kb, ap): lane half hl holds in k-slot t the key
// 32*kb + 16*ap + 8*(t/4) + 4*hl + t%4, i.e. the keys its S^T registers
// 8*ap .. 8*ap+7 hold.  The V^T operand for d block db is two transposing
// reads of 4 keys x 16 d columns per 16-lane group.
__device__ __forceinline__ void tile_pv(const uint8_t* sV, const u32x4 pk[2][2][2], UnitState& st, int lane) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // the four V^T operands of this 32-key half, read before its MFMAs
    bf16x8 vop[2][2];
#pragma unroll
    for (int ap = 0; ap < 2; ++ap)
#pragma unroll
      for (int db = 0; db < 2; ++db) vop[ap][db] = read_tile_tr(sV, 32 * kb + 16 * ap, db, lane);
#pragma unroll
    for (int ap = 0; ap < 2; ++ap)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) st.o[db][qb] = mfma32(vop[ap][db], as_bf16x8(pk[kb][ap][qb]), st.o[db][qb]);
  }
}

// Epilogue of a unit: the row sums and maxima give the normalised output
// block, its LSE and (FULL) the dropped mass.  The output block is staged in
// LDS (`stage`: 8 KB this wave may overwrite): the lane pairs that hold a row in
// the matrix-instruction layout write it there, then each lane stores 16
// contiguous bytes, so one store instruction writes eight whole 128-byte
// rows instead of sixteen bytes of each of 32 rows.  16-byte chunks are
// placed at chunk ^ (row % 8) so that neither side conflicts on LDS banks.
template <bool FULL>
__device__ __forceinline__ void unit_epilogue_staged(const UnitState& st, const AttnArgs& a, const Geometry& geo,
                                                     int bh, int i, int lane, uint8_t* stage,
                                                     const float* ld = nullptr) {
  // the lane index passes through an opaque copy, so that the staging
  // addresses are formed here rather than hoisted out of the unit loop into
  // registers the tile loop needs
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int lr = ln & 31, lh = ln >> 5;
  float inv[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = sum_xor32(st.l[qb]);
    const float dt = FULL ? sum_xor32(ld[64 * qb]) : 0.f;
    inv[qb] = 1.f / lt;
    const int row = i * kBlock + 32 * qb + lr;
    if (lh == 0 && row < geo.seq_q) {
      const size_t orow = (size_t)bh * a.rows_out + row - a.qb_begin * kBlock;
      a.lse[orow] = (st.m[qb] + fast_log2(lt)) * kLn2;
      if (FULL) a.dropped[orow] = dt * inv[qb];
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = 32 * qb + lr;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        // columns 32 db + 8 rg + 4 hl .. + 3: half of 16-byte chunk 4 db + rg
        u32x2 w;
        w[0] = pack_bf16x2(st.o[db][qb][4 * rg] * inv[qb], st.o[db][qb][4 * rg + 1] * inv[qb]);
        w[1] = pack_bf16x2(st.o[db][qb][4 * rg + 2] * inv[qb], st.o[db][qb][4 * rg + 3] * inv[qb]);
        const int chunk = (4 * db + rg) ^ (r & 7);
        *reinterpret_cast<u32x2*>(stage + r * 128 + chunk * 16 + 8 * lh) = w;
      }
  }
  wave_lds_sync();
  const int c = ln & 7;
  const size_t obase = (size_t)bh * a.rows_out + (size_t)(i - a.qb_begin) * kBlock;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = (ln >> 3) + 8 * k;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * 128 + ((c ^ (r & 7)) * 16));
    if (i * kBlock + r < geo.seq_q) *reinterpret_cast<u32x4*>(a.out + (obase + r) * kHeadDim + 8 * c) = v;
  }
}

// Optional timing record of a persistent workgroup (AttnArgs::trace): a few
// scalar counter reads per unit; written by lane 0 at the end.
struct WgTrace {
  uint64_t rt0, t0, l0;
  uint32_t loop, units, tiles;
  __device__ __forceinline__ void begin() {
    rt0 = __builtin_amdgcn_s_memrealtime();
    t0 = __builtin_amdgcn_s_memtime();
    loop = units = tiles = 0u;
  }
  __device__ __forceinline__ void loop_begin() { l0 = __builtin_amdgcn_s_memtime(); }
  __device__ __forceinline__ void loop_end(int nt) {
    loop += (uint32_t)(__builtin_amdgcn_s_memtime() - l0);
    units += 1u;
    tiles += (uint32_t)nt;
  }
  __device__ __forceinline__ void end(const AttnArgs& a, int lane) {
    if (!a.trace || (int)blockIdx.x >= a.trace_cap) return;
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t rt1 = __builtin_amdgcn_s_memrealtime();
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (lane == 0) {
      uint32_t* d = a.trace + (size_t)kTraceWords * blockIdx.x;
      d[0] = (uint32_t)rt0;
      d[1] = (uint32_t)rt1;
      d[2] = (uint32_t)(t1 - t0);
      d[3] = loop;
      d[4] = units;
      d[5] = tiles;
      d[6] = hw;
      d[7] = xcc;
    }
  }
};

// Workgroup id -> (KV group gi = b*Hkv + g, unit index within the group, 0 = heaviest).
// Workgroups are dealt to the 8 XCDs round-robin; when the counts allow, each
// KV group's units stay on a fixed subset of XCDs so its K/V stay in that L2.
__device__ __forceinline__ void map_unit(int w, int n_groups, int per_group, int& gi, int& u) {
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

// Persistent launches: workgroup b first takes unit b of the static order,
// then further units from share x = b % nx of a work queue in the caller's
// workspace: units G + x, G + x + nx, ... (G workgroups), which keeps a
// share's units on the KV groups map_unit gives XCD x when the workgroups are
// dealt to the XCDs round-robin.  Each share has its own counter; a
// workgroup's first ticket past the share's units ends it, and the share's
// last such ticket (the counter has then seen every workgroup of the share
// for the last time) returns the counter to zero.
__device__ __forceinline__ int queue_next(int32_t* q, int nx, int n_units, int lane) {
  const int G = (int)gridDim.x, b = (int)blockIdx.x, x = b % nx;
  const int share = G + x < n_units ? (n_units - G - x + nx - 1) / nx : 0;  // dynamic units of share x
  const int members = (G - x + nx - 1) / nx;                               // workgroups of share x
  int t = 0;
  if (lane == 0) {
    t = __hip_atomic_fetch_add(q + x * kQueueStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == share + members - 1) __hip_atomic_store(q + x * kQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  t = __builtin_amdgcn_readfirstlane(t);
  return t < share ? G + x + nx * t : -1;
}

// Tile loop of the block-sparse forward.  The LDS buffers arrive as distinct
// restrict pointers so that, once inlined, the compiler can tell a K read from
// an in-flight V load (and the tile list from both) and waits only for the
// buffer it reads.  The caller has requested K_0 and V_0.  Pipeline per tile t
// (K_t, V_t already requested):
//   wait K_t | S_t | request K_{t+1} | softmax_t | wait V_t | PV_t | request V_{t+1}
template <bool BIAS>
__device__ __attribute__((always_inline)) inline void sparse_tiles(
    uint8_t* __restrict__ sK, uint8_t* __restrict__ sV, const int* __restrict__ sList,
    const float* __restrict__ sBias, int nt, const uint16_t* __restrict__ kbase, const uint16_t* __restrict__ vbase,
    int seq_kv, int jd, int pos0, float c, const bf16x8 qop[2][4], UnitState& st, int lane, int l32, int hl) {
  TileOffsets<1, 0> toff;
  toff.init(lane, 0);
  for (int t = 0; t < nt; ++t) {
    // Two wavefronts share each SIMD; left to the oldest-first arbiter one of
    // them runs close to its solo speed and the other at about half, so the
    // pair finishes its units far apart.  Alternating the issue priority every
    // tile keeps the two at similar speed.
    if (t & 1)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    const int j = __builtin_amdgcn_readfirstlane(sList[t]);
    const bool more = t + 1 < nt;
    const int jn = more ? __builtin_amdgcn_readfirstlane(sList[t + 1]) : 0;
    wait_vmem<8>();  // K_t landed (V_t may still be in flight)
    f32x16 s[2][2];
    tile_scores(sK, qop, l32, hl, s);
    wait_lds_reads();
    if (more) tile_load(kbase + (size_t)jn * kBlock * kHeadDim, seq_kv - jn * kBlock, sK, lane, toff);
    u32x4 pk[2][2][2];
    const float b2 = BIAS ? sBias[t] * kLog2eF : 0.f;
    tile_softmax<false, BIAS>(s, st, pk, j == jd, true, j * kBlock, pos0, l32, hl, c, nullptr, b2, t == 0);
    if (more)
      wait_vmem<8>();  // V_t landed (K_{t+1} may still be in flight)
    else
      wait_vmem<0>();
    tile_pv(sV, pk, st, lane);
    wait_lds_reads();
    if (more) tile_load(vbase + (size_t)jn * kBlock * kHeadDim, seq_kv - jn * kBlock, sV, lane, toff);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Block-sparse forward: a wavefront per unit, private K and V buffers.  With
// a work queue the launch is persistent: each wavefront takes units until the
// queue is drained; otherwise unit = workgroup.
// BIAS: each listed block's logits are shifted by its entry of a.bias.
template <bool BIAS>
__global__ __launch_bounds__(64, 2) void attn_sparse_kernel(AttnArgs a, Geometry geo) {
  __shared__ __attribute__((aligned(1024))) uint8_t sK[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[kTileBytes];
  __shared__ int sList[kMaxTopk];
  __shared__ int sTmp[kMaxTopk];
  __shared__ float sBias[BIAS ? kMaxTopk : 1];
  const int lane = threadIdx.x, hl = lane >> 5, l32 = lane & 31;
  const int G = geo.group;
  const int n_groups = geo.batch * geo.hkv, per_group = G * a.qb_count;
  int w = (int)blockIdx.x;
  TileOffsets<1, 0> toff;
  toff.init(lane, 0);
  WgTrace tr;
  tr.begin();
  while (w >= 0) {
    int gi, u;
    map_unit(w, n_groups, per_group, gi, u);
    const int i = a.qb_begin + a.qb_count - 1 - u / G;  // longest rows first
    const int b = gi / geo.hkv, g = gi - b * geo.hkv;
    const int h = g * G + (u - (u / G) * G);
    const int bh = b * geo.hq + h;
    const int jd = (geo.q_offset + i * kBlock) / kBlock;
    const size_t kvoff = (size_t)gi * geo.seq_kv * kHeadDim;

    // The diagonal block comes first on every valid list, so its tile is
    // requested before the list is read; the index row (per query head, or
    // per KV group when shared) and Q are requested together.
    tile_load(a.k + kvoff + (size_t)jd * kBlock * kHeadDim, geo.seq_kv - jd * kBlock, sK, lane, toff);
    tile_load(a.v + kvoff + (size_t)jd * kBlock * kHeadDim, geo.seq_kv - jd * kBlock, sV, lane, toff);
    const int irow = a.idx_shared ? gi : bh;
    int iv[4];
    load_index_row(a.idx + ((size_t)irow * geo.nqb + i) * geo.topk, geo.topk, lane, iv);
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (BIAS) load_value_row(a.bias + ((size_t)irow * geo.nqb + i) * geo.topk, geo.topk, lane, bv);
    bf16x8 qop[2][4];
    load_q(a.q + (size_t)bh * geo.seq_q * kHeadDim, i, geo.seq_q, l32, hl, qop);
    const int nt = canonical_index_row<BIAS>(iv, bv, geo.topk, jd, sList, sBias, sTmp, lane);
    const bool has_diag = nt > 0 && __builtin_amdgcn_readfirstlane(sList[nt - 1]) == jd;
    if (has_diag) {
      // rotate: diagonal first, then the others in ascending order
      int jv[kMaxTopk / 64];
      float bw[kMaxTopk / 64];
#pragma unroll
      for (int cc = 0; cc < kMaxTopk / 64; ++cc) {
        const int e = lane + 64 * cc;
        jv[cc] = e < nt ? sList[(e + nt - 1) % nt] : 0;
        if (BIAS) bw[cc] = e < nt ? sBias[(e + nt - 1) % nt] : 0.f;
      }
      wave_lds_sync();
#pragma unroll
      for (int cc = 0; cc < kMaxTopk / 64; ++cc) {
        const int e = lane + 64 * cc;
        if (e < nt) {
          sList[e] = jv[cc];
          if (BIAS) sBias[e] = bw[cc];
        }
      }
    }
    UnitState st;
    init_state(st);
    wait_vmem<0>();  // Q, the list, and the diagonal tile
    wave_lds_sync();
    if (!has_diag && nt > 0) {  // a list without its diagonal: the prefetched tile is not used
      const int j0 = __builtin_amdgcn_readfirstlane(sList[0]);
      tile_load(a.k + kvoff + (size_t)j0 * kBlock * kHeadDim, geo.seq_kv - j0 * kBlock, sK, lane, toff);
      tile_load(a.v + kvoff + (size_t)j0 * kBlock * kHeadDim, geo.seq_kv - j0 * kBlock, sV, lane, toff);
      wait_vmem<0>();
      __builtin_amdgcn_wave_barrier();
    }
    tr.loop_begin();
    sparse_tiles<BIAS>(sK, sV, sList, sBias, nt, a.k + kvoff, a.v + kvoff, geo.seq_kv, jd,
                       geo.q_offset + i * kBlock, geo.scale_log2, qop, st, lane, l32, hl);
    tr.loop_end(nt);
    wait_lds_reads();  // the tiles' last reads are done: sK is the staging area
    unit_epilogue_staged<false>(st, a, geo, bh, i, lane, sK);
    if (!a.queue) break;
    wait_lds_reads();  // the next unit's tile requests overwrite sK and sV
    w = queue_next(a.queue, a.n_xcc, n_groups * per_group, lane);
  }
  tr.end(a, lane);
}

// Block-sparse forward with early stopping.  One wavefront per unit, as
// attn_sparse_kernel, but the unit's blocks are visited diagonal first and
// then by coarse score (higher first, lower index on ties, NaN last); after
// each block past the first, the unit stops if for every valid row the
// block's mass is below tau times the mass accumulated before it (the block
// is kept).  blocks_used[b,h,i] records how many blocks were visited.
// Method: S2O summary, "Regla de Parada Temprana" and "Implementacion del
// Kernel" (own segment first, then the prefix in decreasing importance).
__global__ __launch_bounds__(64, 2) void attn_sparse_early_stop_kernel(AttnArgs a, Geometry geo,
                                                                       const float* __restrict__ scores, float tau,
                                                                       int32_t* __restrict__ blocks_used) {
  __shared__ __attribute__((aligned(1024))) uint8_t sK[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[kTileBytes];
  __shared__ int sList[kMaxTopk];
  __shared__ int sOrder[kMaxTopk];
  __shared__ uint32_t sKey[kMaxTopk];
  const int lane = threadIdx.x, hl = lane >> 5, l32 = lane & 31;
  const int G = geo.group;
  int gi, u;
  map_unit(blockIdx.x, geo.batch * geo.hkv, G * a.qb_count, gi, u);
  const int i = a.qb_begin + a.qb_count - 1 - u / G;
  const int b = gi / geo.hkv, g = gi - b * geo.hkv;
  const int h = g * G + (u - (u / G) * G);
  const int bh = b * geo.hq + h;
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  const size_t kvoff = (size_t)gi * geo.seq_kv * kHeadDim;
  const uint16_t* kbase = a.k + kvoff;
  const uint16_t* vbase = a.v + kvoff;

  // the diagonal block is visited first whenever it is listed (as it is on
  // every valid list): its tile is requested before the list is read
  TileOffsets<1, 0> toff;
  toff.init(lane, 0);
  tile_load(kbase + (size_t)jd * kBlock * kHeadDim, geo.seq_kv - jd * kBlock, sK, lane, toff);
  tile_load(vbase + (size_t)jd * kBlock * kHeadDim, geo.seq_kv - jd * kBlock, sV, lane, toff);
  int iv[4];
  load_index_row(a.idx + ((size_t)bh * geo.nqb + i) * geo.topk, geo.topk, lane, iv);
  bf16x8 qop[2][4];
  load_q(a.q + (size_t)bh * geo.seq_q * kHeadDim, i, geo.seq_q, l32, hl, qop);
  const int n = canonical_index_row<false>(iv, nullptr, geo.topk, jd, sList, nullptr, sOrder, lane);
  // visiting order: the diagonal block, then the rest by (score desc, index asc)
  const float* srow = scores + ((size_t)bh * geo.nqb + i) * geo.nkb;
  int has_diag = 0;
  for (int e = lane; e < n; e += 64) {
    const int j = sList[e];
    has_diag |= j == jd;
    sKey[e] = orderable_score(srow[j]);  // each listed block's score read once
  }
  has_diag = __builtin_amdgcn_ballot_w64(has_diag != 0) != 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int e = lane; e < n; e += 64) {
    const int j = sList[e];
    if (j == jd) {
      sOrder[0] = j;
      continue;
    }
    const uint32_t kj = sKey[e];
    int rank = 0;
    for (int f = 0; f < n; ++f) {
      const int jf = sList[f];
      const uint32_t kf = sKey[f];
      rank += (jf != jd && (kf > kj || (kf == kj && jf < j))) ? 1 : 0;
    }
    sOrder[has_diag + rank] = j;
  }
  const int nt = n;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  UnitState st;
  init_state(st);
  wait_vmem<0>();  // Q, the scores and the diagonal tile
  __builtin_amdgcn_wave_barrier();
  if (!has_diag && nt > 0) {  // a list without its diagonal: its first block replaces the prefetched tile
    const int j0 = __builtin_amdgcn_readfirstlane(sOrder[0]);
    tile_load(kbase + (size_t)j0 * kBlock * kHeadDim, geo.seq_kv - j0 * kBlock, sK, lane, toff);
    tile_load(vbase + (size_t)j0 * kBlock * kHeadDim, geo.seq_kv - j0 * kBlock, sV, lane, toff);
    wait_vmem<0>();
    __builtin_amdgcn_wave_barrier();
  }
  const float c = geo.scale_log2;
  const int pos0 = geo.q_offset + i * kBlock;
  int used = 0;
  for (int t = 0; t < nt; ++t) {
    // issue priority alternates every tile, as in the block-sparse loop
    if (t & 1)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    const int j = __builtin_amdgcn_readfirstlane(sOrder[t]);
    const bool more = t + 1 < nt;
    const int jn = more ? __builtin_amdgcn_readfirstlane(sOrder[t + 1]) : 0;
    wait_vmem<8>();  // K_t landed (V_t may still be in flight)
    f32x16 s[2][2];
    tile_scores(sK, qop, l32, hl, s);
    wait_lds_reads();
    if (more) tile_load(kbase + (size_t)jn * kBlock * kHeadDim, geo.seq_kv - jn * kBlock, sK, lane, toff);
    u32x4 pk[2][2][2];
    float trs[2];
    tile_softmax<false>(s, st, pk, j == jd, true, j * kBlock, pos0, l32, hl, c, trs, 0.f, t == 0);
    // stop after this tile if every valid row gained less than tau times its earlier mass
    bool stop = false;
    if (t > 0) {
      bool keep_going = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float gain = sum_xor32(trs[qb]);
        const float before = sum_xor32(st.l[qb] - trs[qb]);
        const bool valid = i * kBlock + 32 * qb + l32 < geo.seq_q;
        keep_going |= valid && !(gain < tau * before);
      }
      stop = __builtin_amdgcn_ballot_w64(keep_going) == 0ull;
    }
    if (more && !stop)
      wait_vmem<8>();  // V_t landed (K_{t+1} may still be in flight)
    else
      wait_vmem<0>();
    tile_pv(sV, pk, st, lane);
    wait_lds_reads();
    used = t + 1;
    if (stop) break;
    if (more) tile_load(vbase + (size_t)jn * kBlock * kHeadDim, geo.seq_kv - jn * kBlock, sV, lane, toff);
  }
  __builtin_amdgcn_s_setprio(0);
  // the last K reads are done and no tile request is in flight: sK is free
  unit_epilogue_staged<false>(st, a, geo, bh, i, lane, sK);
  if (lane == 0) blocks_used[(size_t)bh * geo.nqb + i] = used;
}

// NW query heads of one KV group per workgroup (one per wave) walk the same
// tiles, fetched once into a double buffer shared by the NW waves; tile t+1 is
// requested as soon as every wave has finished tile t-1.
//   FULL:  every causal tile of the query block (the full counterpart), with
//          dropped mass from the tiles missing from each head's own list;
//   !FULL: the tiles of a group-shared selection (block-sparse forward).
// BIAS (with !FULL): each listed block's logits are shifted by its entry of
// a.bias.
template <int NW, bool FULL, bool BIAS = false>
__global__ __launch_bounds__(64 * NW, 2) void attn_group_kernel(AttnArgs a, Geometry geo) {
  __shared__ __attribute__((aligned(1024))) uint8_t sK[2][kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[2][kTileBytes];
  __shared__ int sList[NW][kMaxTopk];
  __shared__ int sTmp[NW][kMaxTopk];
  __shared__ float sBias[BIAS ? NW : 1][BIAS ? kMaxTopk : 1];
  __shared__ float sLd[FULL ? NW : 1][2][64];  // dropped-mass sums (FULL), one slot per lane and query block
  __shared__ int sUnit;
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = geo.group, GS = G / NW;
  const int n_groups = geo.batch * geo.hkv, per_group = GS * a.qb_count;
  // next unit of the workgroup: wave 0 takes it from the queue, the others read it from LDS
  auto next_unit = [&]() -> int {
    if (wave == 0) {
      const int t = queue_next(a.queue, a.n_xcc, n_groups * per_group, lane);
      if (lane == 0) sUnit = t;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(sUnit);
  };
  int w = (int)blockIdx.x;
  TileOffsets<NW, 0> toff;
  toff.init(lane, wave);
  WgTrace tr;
  tr.begin();
  while (w >= 0) {
    int gi, u;
    map_unit(w, n_groups, per_group, gi, u);
    const int i = a.qb_begin + a.qb_count - 1 - u / GS;
    const int b = gi / geo.hkv, g = gi - b * geo.hkv;
    const int h = g * G + (u - (u / GS) * GS) * NW + wave;
    const int bh = b * geo.hq + h;
    const int jd = (geo.q_offset + i * kBlock) / kBlock;
    const size_t kvoff = (size_t)gi * geo.seq_kv * kHeadDim;
    const uint16_t* kbase = a.k + kvoff;
    const uint16_t* vbase = a.v + kvoff;

    // index row (per query head, or per KV group when shared) and Q requested
    // together, so their latencies overlap
    const int irow = a.idx_shared ? gi : bh;
    int iv[4];
    load_index_row(a.idx + ((size_t)irow * geo.nqb + i) * geo.topk, geo.topk, lane, iv);
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (BIAS) load_value_row(a.bias + ((size_t)irow * geo.nqb + i) * geo.topk, geo.topk, lane, bv);
    bf16x8 qop[2][4];
    load_q(a.q + (size_t)bh * geo.seq_q * kHeadDim, i, geo.seq_q, l32, hl, qop);
    const int nsel =
        canonical_index_row<BIAS>(iv, bv, geo.topk, jd, sList[wave], sBias[BIAS ? wave : 0], sTmp[wave], lane);
    // tiles walked: 0..jd (full), or the shared list (identical in every wave)
    const int nt = FULL ? jd + 1 : nsel;
    auto tile_block = [&](int t) { return FULL ? t : __builtin_amdgcn_readfirstlane(sList[wave][t]); };
    if (nt > 0) {  // first tile requested before waiting for Q, so the two latencies overlap
      const int j0 = tile_block(0);
      tile_load(kbase + (size_t)j0 * kBlock * kHeadDim, geo.seq_kv - j0 * kBlock, sK[0], lane, toff);
      tile_load(vbase + (size_t)j0 * kBlock * kHeadDim, geo.seq_kv - j0 * kBlock, sV[0], lane, toff);
    }
    UnitState st;
    init_state(st);
    float* ld = FULL ? &sLd[FULL ? wave : 0][0][lane] : nullptr;
    if (FULL) ld[0] = ld[64] = 0.f;  // this lane's own slots: read back by this lane only
    wait_vmem<0>();
    __builtin_amdgcn_wave_barrier();
    const float c = geo.scale_log2;
    const int pos0 = geo.q_offset + i * kBlock;
    int sel_ptr = 0;
    int nxt = nsel > 0 ? __builtin_amdgcn_readfirstlane(sList[wave][0]) : -1;
    tr.loop_begin();
    for (int t = 0; t < nt; ++t) {
      // issue priority alternates every tile, as in the block-sparse loop
      if (t & 1)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
      const int j = tile_block(t);
      wait_vmem<0>();   // this wave's share of tile t landed
      __syncthreads();  // ... every wave's share; and every wave is done with tile t-1
      if (t + 1 < nt) {
        const int jn = tile_block(t + 1);
        const size_t off = (size_t)jn * kBlock * kHeadDim;
        const int nv = geo.seq_kv - jn * kBlock;
        tile_load(kbase + off, nv, sK[(t + 1) & 1], lane, toff);
        tile_load(vbase + off, nv, sV[(t + 1) & 1], lane, toff);
      }
      bool selected = true;
      if (FULL) {
        selected = (nxt == t);
        if (selected) {
          ++sel_ptr;
          nxt = sel_ptr < nsel ? __builtin_amdgcn_readfirstlane(sList[wave][sel_ptr]) : -1;
        }
      }
      f32x16 s[2][2];
      tile_scores(sK[t & 1], qop, l32, hl, s);
      u32x4 pk[2][2][2];
      const float b2 = BIAS ? sBias[BIAS ? wave : 0][BIAS ? t : 0] * kLog2eF : 0.f;
      tile_softmax<FULL, BIAS>(s, st, pk, j == jd, selected, j * kBlock, pos0, l32, hl, c, nullptr, b2, false, ld);
      tile_pv(sV[t & 1], pk, st, lane);
    }
    __builtin_amdgcn_s_setprio(0);
    tr.loop_end(nt);
    wait_lds_reads();
    __syncthreads();  // every wave is done with the tiles: each stages its outputs in a quarter of them
    unit_epilogue_staged<FULL>(st, a, geo, bh, i, lane, wave < 2 ? sK[wave] : sV[wave - 2], ld);
    if (!a.queue) break;
    wait_lds_reads();
    __syncthreads();  // every wave is done with the tiles, the lists and the unit slot
    w = next_unit();
  }
  if (wave == 0) tr.end(a, lane);
}

}  // namespace

hipError_t launch_attn_early_stop(const AttnArgs& a, const float* scores, float tau, int32_t* blocks_used,
                                  const Geometry& g, hipStream_t stream) {
  const size_t units = (size_t)g.batch * g.hq * a.qb_count;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_sparse_early_stop_kernel, dim3((unsigned)units), dim3(64), 0, stream, a, g, scores, tau,
                     blocks_used);
  return hipGetLastError();
}

// Compute units of the current device (cached per device id).
static int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

// Grid of a launch: one workgroup per unit, or with a work queue as many
// workgroups as fit on the device at once (`per_cu` per compute unit).
static unsigned prefill_grid(AttnArgs& a, size_t units_per_group, int per_cu) {
  if (!a.queue) return (unsigned)units_per_group;
  const int cus = device_cus();
  const size_t resident = (size_t)cus * per_cu;
  const unsigned grid = (unsigned)(units_per_group < resident ? units_per_group : resident);
  a.n_xcc = grid < (unsigned)kMaxXcc ? (int)grid : kMaxXcc;
  return grid;
}

hipError_t launch_attn_prefill(const AttnArgs& args, bool full, const Geometry& g, hipStream_t stream) {
  const size_t units = (size_t)g.batch * g.hq * args.qb_count;
  if (units == 0) return hipSuccess;
  AttnArgs a = args;
  const bool bias = !full && a.bias != nullptr;
  if (!full && !(a.idx_shared && g.group % 4 == 0)) {
    // per-head lists (or groups too small to share): a wavefront per unit, 8 per compute unit
    const unsigned grid = prefill_grid(a, units, 8);
    if (bias)
      hipLaunchKernelGGL(attn_sparse_kernel<true>, dim3(grid), dim3(64), 0, stream, a, g);
    else
      hipLaunchKernelGGL(attn_sparse_kernel<false>, dim3(grid), dim3(64), 0, stream, a, g);
  } else if (!full) {
    // group-shared lists: four heads of a group share every tile
    const unsigned grid = prefill_grid(a, units / 4, 2);
    if (bias)
      hipLaunchKernelGGL((attn_group_kernel<4, false, true>), dim3(grid), dim3(256), 0, stream, a, g);
    else
      hipLaunchKernelGGL((attn_group_kernel<4, false>), dim3(grid), dim3(256), 0, stream, a, g);
  } else if (g.group % 4 == 0) {
    hipLaunchKernelGGL((attn_group_kernel<4, true>), dim3(prefill_grid(a, units / 4, 2)), dim3(256), 0, stream, a, g);
  } else if (g.group % 2 == 0) {
    hipLaunchKernelGGL((attn_group_kernel<2, true>), dim3(prefill_grid(a, units / 2, 4)), dim3(128), 0, stream, a, g);
  } else {
    hipLaunchKernelGGL((attn_group_kernel<1, true>), dim3(prefill_grid(a, units, 8)), dim3(64), 0, stream, a, g);
  }
  return hipGetLastError();
}

}  // namespace ssa
