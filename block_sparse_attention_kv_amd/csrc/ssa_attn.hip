// Prefill attention kernels (gfx950): block-sparse forward over the selected
// key blocks, and the full causal counterpart that also emits the dropped mass.
//
// One wavefront owns one unit = (b, query head, 64-row query block) and walks
// its key tiles (64 keys each): the selected blocks (sparse) or every causal
// block (full).  Per tile, computed transposed so a lane owns query columns:
//   S^T = K Q^T          (bf16 MFMA 32x32x16, fp32 accumulate; Q^T stays in registers)
//   online softmax       (fp32, log2 domain; row max/sum are lane-local plus one swap)
//   O^T += V^T P^T       (bf16 MFMA; P^T comes straight from the S^T accumulators,
//                          V^T read from a transposed LDS copy in the same key order)
// The full kernel keeps a second running sum over tiles that are not selected,
// under the same running max, so dropped mass = l_dropped / l_total falls out of
// the single pass.
//
// Method: SSA summary (gist.science 2511.20102), "Mecanismo Central" (sparse
// and full attention streams) and "Alineacion Bidireccional" (counterpart
// output, dropped mass); SSA guide (mauroscia.it), "Block-sparse attention e
// Receptive Field"; S2O summary, "Permutacion en Linea" (tiles gathered by
// index from an unchanged HBM layout).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kRow = 72;  // LDS row stride in bf16 elements (144 B; 16-byte aligned rows)

template <bool FULL>
__global__ __launch_bounds__(64) void attn_prefill_kernel(AttnArgs a, Geometry geo) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBlock * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[kHeadDim * kRow];

  const int lane = threadIdx.x, hl = lane >> 5, l32 = lane & 31;
  const int nbh = geo.batch * geo.hq;
  const int i_rel = blockIdx.x / nbh;
  const int bh = blockIdx.x - i_rel * nbh;
  const int i = a.qb_begin + (a.qb_count - 1 - i_rel);  // longest rows first
  const int b = bh / geo.hq, h = bh - b * geo.hq, g = h / geo.group;
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  const uint16_t* qbase = a.q + (size_t)bh * geo.seq_q * kHeadDim;
  const size_t kvoff = (size_t)(b * geo.hkv + g) * geo.seq_kv * kHeadDim;
  const uint16_t* kbase = a.k + kvoff;
  const uint16_t* vbase = a.v + kvoff;
  const int32_t* irow = a.idx + ((size_t)bh * geo.nqb + i) * geo.topk;

  // Q^T as MFMA B operand: column = query row 32*qb + l32, k-slots = d 16*ks + 8*hl .. +8.
  bf16x8 qop[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = i * kBlock + 32 * qb + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < geo.seq_q)
        v = *reinterpret_cast<const u32x4*>(qbase + (size_t)row * kHeadDim + 16 * ks + 8 * hl);
      qop[qb][ks] = as_bf16x8(v);
    }
  }

  f32x16 o[2][2];  // O^T accumulators [d block][query block]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[x][y][r] = 0.f;
  float m[2] = {-__builtin_inff(), -__builtin_inff()};
  float l[2] = {0.f, 0.f};
  float ld[2] = {0.f, 0.f};

  const int ntiles = FULL ? jd + 1 : geo.topk;
  int sel_ptr = 0;
  for (int t = 0; t < ntiles; ++t) {
    int j = t;
    bool selected = true;
    if (FULL) {
      const int nxt = sel_ptr < geo.topk ? irow[sel_ptr] : -1;
      selected = (nxt == j);
      sel_ptr += selected ? 1 : 0;
    } else {
      j = irow[t];
      if (j < 0) break;
      if (j > jd) continue;  // not a causal block of this query block: ignored
    }

    __syncthreads();
    // Stage the tile: K row-major, V transposed (d-major) for the PV operand.
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int chunk = it * 64 + lane, row = chunk >> 3, c8 = chunk & 7;
      const int key = j * kBlock + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < geo.seq_kv) {
        kv = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * kHeadDim + c8 * 8);
        vv = *reinterpret_cast<const u32x4*>(vbase + (size_t)key * kHeadDim + c8 * 8);
      }
      *reinterpret_cast<u32x4*>(&sK[row * kRow + c8 * 8]) = kv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[(c8 * 8 + 2 * e) * kRow + row] = (uint16_t)(vv[e] & 0xffffu);
        sVt[(c8 * 8 + 2 * e + 1) * kRow + row] = (uint16_t)(vv[e] >> 16);
      }
    }
    __syncthreads();

    // S^T = K Q^T: rows = keys 32*kb + ..., columns = queries 32*qb + l32.
    f32x16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sK[(32 * kb + l32) * kRow + 16 * ks + 8 * hl]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma32(ka, qop[qb][ks], s[kb][qb]);
      }
    }

    const bool diag = (j == jd);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int pos = geo.q_offset + i * kBlock + 32 * qb + l32;
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][qb][r] * geo.scale_log2;
          if (diag) {
            const int key = j * kBlock + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key > pos) x = -__builtin_inff();
          }
          s[kb][qb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m[qb], mx);
      const float alpha = fast_exp2(m[qb] - mnew);
      m[qb] = mnew;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(s[kb][qb][r] - mnew);
          s[kb][qb][r] = p;
          rs += p;
        }
      }
      l[qb] = l[qb] * alpha + rs;
      if (FULL) ld[qb] = ld[qb] * alpha + (selected ? 0.f : rs);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
    }

    // O^T += V^T P^T over four 16-key steps (kb, ap).  Lane half hl holds, in
    // k-slot t, key 32*kb + 16*ap + 8*(t/4) + 4*hl + t%4 -- the keys its S^T
    // accumulator registers 8*ap .. 8*ap+7 already hold.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ap = 0; ap < 2; ++ap) {
        bf16x8 pop[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(s[kb][qb][8 * ap + 2 * e], s[kb][qb][8 * ap + 2 * e + 1]);
          pop[qb] = as_bf16x8(pk);
        }
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const uint16_t* vr = &sVt[(32 * db + l32) * kRow + 32 * kb + 16 * ap + 4 * hl];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
          u32x4 va;
          va[0] = lo[0]; va[1] = lo[1]; va[2] = hi[0]; va[3] = hi[1];
          const bf16x8 vop = as_bf16x8(va);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) o[db][qb] = mfma32(vop, pop[qb], o[db][qb]);
        }
      }
    }
  }

  // Epilogue: fold the two lane halves' partial sums (all lanes take part in
  // the swaps), normalise, store.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32, 64);
    const float dt = FULL ? ld[qb] + __shfl_xor(ld[qb], 32, 64) : 0.f;
    const float inv = 1.f / lt;
    const int row = i * kBlock + 32 * qb + l32;
    if (row < geo.seq_q) {
      const int orow = row - a.qb_begin * kBlock;
      uint16_t* op = a.out + ((size_t)bh * a.rows_out + orow) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 w;
          w[0] = pack_bf16x2(o[db][qb][4 * rg] * inv, o[db][qb][4 * rg + 1] * inv);
          w[1] = pack_bf16x2(o[db][qb][4 * rg + 2] * inv, o[db][qb][4 * rg + 3] * inv);
          *reinterpret_cast<u32x2*>(op + 32 * db + 8 * rg + 4 * hl) = w;
        }
      }
      if (hl == 0) {
        a.lse[(size_t)bh * a.rows_out + orow] = (m[qb] + fast_log2(lt)) * kLn2;
        if (FULL) a.dropped[(size_t)bh * a.rows_out + orow] = dt * inv;
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs& a, bool full, const Geometry& g, hipStream_t stream) {
  const size_t units = (size_t)g.batch * g.hq * a.qb_count;
  if (units == 0) return hipSuccess;
  if (full)
    hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3((unsigned)units), dim3(64), 0, stream, a, g);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3((unsigned)units), dim3(64), 0, stream, a, g);
  return hipGetLastError();
}

}  // namespace ssa
