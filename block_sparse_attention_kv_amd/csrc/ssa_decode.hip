// Decode attention (gfx950): one query token per (sequence, query head) against
// a long KV cache, over the key blocks each head selected.
//
// The wavefronts of one (sequence, KV head) group each rebuild, in LDS, the
// ascending union of the key blocks the group's query heads selected (a
// bitmap over the blocks, a popcount prefix for ranks) with the bitmask of the
// heads that chose each, and take an equal slice of it, so the work is
// balanced whatever the selection.  A wavefront streams exactly its union
// blocks from HBM through a ring of LDS slots filled by direct-to-LDS loads,
// keeping kRing-1 blocks in flight while it computes.  Each block is read once
// per call, so the loads carry the non-temporal policy (measured: the
// attention call 12-15% faster than with the default policy, which leaves
// the streamed blocks competing for the caches).
// With a group-shared list and a per-block bias (prior-biased softmax), the
// block's logits are shifted by its bias.
// Every union block is applied to all query heads of the group at once with
// bf16 MFMAs (16 heads per 16x16x32 tile): heads that did not select the block
// see it masked.  Each wavefront writes one partial online-softmax state
// (reference max, sum, unnormalised output) per head; a second kernel merges
// the slice partials.  The kernel is bound by HBM reads of the union blocks.
//
// Method: DashAttention summary, "Etapa 0" (chunk summaries cached once
// complete, no recomputation at inference) and "Resultados Experimentales"
// (memory-bound decoding); S2O summary, "Permutacion en Linea" (index-guided
// loading from an unchanged HBM layout); SSA guide (mauroscia.it),
// "Block-sparse attention e Receptive Field".
#include "ssa_common.hpp"
#include "ssa_internal.hpp"
#include "ssa_tiles.hpp"

namespace ssa {
namespace {

constexpr int kRing = kDecodeRing;  // K/V block slots per wavefront (kRing - 1 in flight while computing)
constexpr int kListChunk = 8;       // index entries per lane read at once
static_assert(kRing >= 2 && (kRing - 1) * 16 <= 63, "in-flight block loads must fit the vmcnt counter");

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wait until the DMA of the block being computed landed, leaving the `later`
// younger blocks (16 load instructions each) in flight.
__device__ __forceinline__ void wait_block(int later) {
  if (later >= 3)
    wait_vmem<48>();
  else if (later == 2)
    wait_vmem<32>();
  else if (later == 1)
    wait_vmem<16>();
  else
    wait_vmem<0>();
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Chunk ch of a group's index entries (and, with a bias row, their biases):
// entry 64 * kListChunk * ch + lane + 64 t into register t, all requested
// before any is used (entries past the end read the last one).
__device__ __forceinline__ void load_list_chunk(const int32_t* __restrict__ gidx, const float* __restrict__ brow,
                                                int cap, int ch, int lane, int (&jv)[kListChunk],
                                                float (&bv)[kListChunk]) {
#pragma unroll
  for (int t = 0; t < kListChunk; ++t) jv[t] = gidx[min(64 * kListChunk * ch + lane + 64 * t, cap - 1)];
  if (brow) {
#pragma unroll
    for (int t = 0; t < kListChunk; ++t) bv[t] = brow[min(64 * kListChunk * ch + lane + 64 * t, cap - 1)];
  }
}

// NHB: 16-head blocks per KV group, 1 (G <= 16) or 2 (G <= 32).
template <int NHB>
__global__ __launch_bounds__(64, 1) void attn_decode_partial_kernel(AttnArgs a, float* __restrict__ ws,
                                                                    Geometry geo, int npieces) {
  __shared__ __attribute__((aligned(1024))) uint8_t sKV[kRing][2][kTileBytes];
  extern __shared__ uint32_t sDyn[];  // bitmap[nw] | prefix[nw] | list[cap] | heads[cap] | bias[cap]
  const int lane = threadIdx.x;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int bg = blockIdx.x / npieces;
  const int piece = blockIdx.x - bg * npieces;
  const int b = bg / geo.hkv, g = bg - b * geo.hkv;
  const int G = geo.group;
  const int head0 = b * geo.hq + g * G;  // (b, first query head of the group)
  const int nw = (geo.nkb + 31) >> 5;
  const int cap = a.idx_shared ? geo.topk : G * geo.topk;  // index entries of the group
  uint32_t* bitmap = sDyn;
  int* prefix = reinterpret_cast<int*>(sDyn + nw);
  int* sBlk = reinterpret_cast<int*>(sDyn + 2 * nw);
  uint32_t* sHm = sDyn + 2 * nw + cap;
  float* sBias = reinterpret_cast<float*>(sDyn + 2 * nw + 2 * cap);  // group-shared lists with a bias only
  // the group's index rows: one per query head, or one shared row
  const int32_t* gidx = a.idx + (size_t)(a.idx_shared ? bg : head0) * geo.topk;
  const uint32_t all_heads = G >= 32 ? 0xffffffffu : ((1u << G) - 1u);

  // Union of the group's selected blocks: bitmap, ranks, ascending list and
  // the heads that selected each listed block.  The group's index entries are
  // read in chunks of 64 * kListChunk: entry e = 64 * kListChunk * ch +
  // lane + 64 t of chunk ch is held in register t, and a chunk's entries (and
  // their biases) are all requested before the first is used.  A list of one
  // chunk is read once for both passes.
  const int nchunk = (cap + 64 * kListChunk - 1) / (64 * kListChunk);
  const float* brow = a.bias ? a.bias + (size_t)bg * geo.topk : nullptr;  // shared rows only
  int jv[kListChunk];
  float bv[kListChunk];
  load_list_chunk(gidx, brow, cap, 0, lane, jv, bv);
  // Q^T as the B operand (requested after the index entries, so that waiting
  // for those leaves it in flight): column = head 16*hb + l16, k-slots = d 32*ks + 8*g4 .. +8.
  bf16x8 qop[NHB][2];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hh = 16 * hb + l16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hh < G) v = *reinterpret_cast<const u32x4*>(a.q + (size_t)(head0 + hh) * kHeadDim + 32 * ks + 8 * g4);
      qop[hb][ks] = as_bf16x8(v);
    }
  }
  for (int w = lane; w < nw; w += 64) bitmap[w] = 0u;
  for (int e = lane; e < cap; e += 64) sHm[e] = 0u;
  wave_sync_lds();
  for (int ch = 0; ch < nchunk; ++ch) {
    if (ch > 0) load_list_chunk(gidx, brow, cap, ch, lane, jv, bv);
#pragma unroll
    for (int t = 0; t < kListChunk; ++t) {
      const int j = jv[t];
      if (64 * kListChunk * ch + lane + 64 * t < cap && j >= 0 && j < geo.nkb)
        atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
  }
  wave_sync_lds();
  int nu = 0;
  for (int w0 = 0; w0 < nw; w0 += 64) {
    const int w = w0 + lane;
    const int cnt = w < nw ? __builtin_popcount(bitmap[w]) : 0;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (w < nw) prefix[w] = nu + incl - cnt;
    nu += __shfl(incl, 63, 64);
  }
  wave_sync_lds();
  for (int ch = 0; ch < nchunk; ++ch) {
    if (nchunk > 1) load_list_chunk(gidx, brow, cap, ch, lane, jv, bv);
#pragma unroll
    for (int t = 0; t < kListChunk; ++t) {
      const int e = 64 * kListChunk * ch + lane + 64 * t;
      const int j = jv[t];
      if (e < cap && j >= 0 && j < geo.nkb) {
        const int r = prefix[j >> 5] + __builtin_popcount(bitmap[j >> 5] & ((1u << (j & 31)) - 1u));
        sBlk[r] = j;
        atomicOr(&sHm[r], a.idx_shared ? all_heads : 1u << (e / geo.topk));
        if (brow) sBias[r] = bv[t];  // shared row: one entry per block
      }
    }
  }
  wave_sync_lds();
  const int u0 = (int)(((int64_t)nu * piece) / npieces);
  const int u1 = (int)(((int64_t)nu * (piece + 1)) / npieces);

  f32x4 o[NHB][4];
  float m[NHB], l[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    m[hb] = -__builtin_inff();
    l[hb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[hb][db][r] = 0.f;
  }
  wait_vmem<0>();  // Q and the index rows are in; from here only block loads use vmcnt
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const size_t kvoff = (size_t)bg * geo.seq_kv * kHeadDim;
  const uint16_t* kbase = uniform_ptr(a.k + kvoff);
  const uint16_t* vbase = uniform_ptr(a.v + kvoff);
  const float c = geo.scale_log2;
  const int pos = geo.q_offset;  // absolute position of the query token

  TileOffsets<1, 1> toff;
  toff.init(lane, 0);
  const int nmine = u1 - u0;
  for (int n = 0; n < kRing - 1 && n < nmine; ++n) {
    const int j = __builtin_amdgcn_readfirstlane(sBlk[u0 + n]);
    tile_load<true>(kbase + (size_t)j * kBlock * kHeadDim, geo.seq_kv - j * kBlock, sKV[n][0], lane, toff);
    tile_load<true>(vbase + (size_t)j * kBlock * kHeadDim, geo.seq_kv - j * kBlock, sKV[n][1], lane, toff);
  }
  for (int n = 0; n < nmine; ++n) {
    const int slot = n % kRing;
    // Request block n + kRing - 1 into the slot block n - 1 used (already consumed).
    const int nn = n + kRing - 1;
    if (nn < nmine) {
      wait_lds_reads();
      const int jn = __builtin_amdgcn_readfirstlane(sBlk[u0 + nn]);
      const int sn = nn % kRing;
      tile_load<true>(kbase + (size_t)jn * kBlock * kHeadDim, geo.seq_kv - jn * kBlock, sKV[sn][0], lane, toff);
      tile_load<true>(vbase + (size_t)jn * kBlock * kHeadDim, geo.seq_kv - jn * kBlock, sKV[sn][1], lane, toff);
    }
    const int j = __builtin_amdgcn_readfirstlane(sBlk[u0 + n]);
    const uint32_t hm = __builtin_amdgcn_readfirstlane(sHm[u0 + n]);
    // logit shift of this block (log2 units), 0 without a bias
    const float b2 =
        a.bias ? __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(sBias[u0 + n]))) * 1.4426950408889634f
               : 0.f;
    wait_block(min(kRing - 1, nmine - 1 - n));
    const uint8_t* sK = sKV[slot][0];
    const uint8_t* sV = sKV[slot][1];

    // S^T = K Q^T: rows = keys 16*mb + 4*g4 + r, column = head.  All K operands
    // are read before the MFMA burst.
    bf16x8 ka[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) ka[mb][ks] = *reinterpret_cast<const bf16x8*>(sK + swz<1>(16 * mb + l16, 4 * ks + g4));
    f32x4 s[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[hb][mb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) s[hb][mb] = mfma16(ka[mb][ks], qop[hb][ks], s[hb][mb]);
      }
    u32x4 pk[NHB][2];
    // Only the block holding the query position (or the cache end) needs a
    // per-key mask; a head that did not select the block gets p = 0 through
    // an exponent offset of -inf.
    const bool edge = j * kBlock + kBlock - 1 > pos || j * kBlock + kBlock > geo.seq_kv;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int hh = 16 * hb + l16;
      const bool sel = hh < G && ((hm >> hh) & 1u);
      if (edge) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = j * kBlock + 16 * mb + 4 * g4 + r;
            if (key > pos || key >= geo.seq_kv) s[hb][mb][r] = -__builtin_inff();
          }
      }
      float mx = fmaxf(fmaxf(s[hb][0][0], s[hb][0][1]), fmaxf(s[hb][0][2], s[hb][0][3]));
#pragma unroll
      for (int mb = 1; mb < 4; ++mb)
        mx = fmaxf(fmaxf(mx, fmaxf(s[hb][mb][0], s[hb][mb][1])), fmaxf(s[hb][mb][2], s[hb][mb][3]));
      mx = sel ? mx : -__builtin_inff();
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      const float mt = fmaf(mx, c, b2);  // == mx * c without a bias
      if (!(mt <= m[hb] + kRescaleSlack)) {  // per-lane: its head's reference max moves
        const float mn = fmaxf(m[hb], mt);
        const float alpha = fast_exp2(m[hb] - mn);
        m[hb] = mn;
        l[hb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[hb][db][r] *= alpha;
      }
      // unselected head, or a block whose bias is -inf (prior weight 0): p = exp2(-inf) = 0;
      // otherwise the exponent is relative to the head's reference max
      const float nm = (!sel || b2 == -__builtin_inff()) ? -__builtin_inff() : b2 - m[hb];
      float rs = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int mb = 2 * ks + half;
          const float p0 = fast_exp2(fmaf(s[hb][mb][0], c, nm));
          const float p1 = fast_exp2(fmaf(s[hb][mb][1], c, nm));
          const float p2 = fast_exp2(fmaf(s[hb][mb][2], c, nm));
          const float p3 = fast_exp2(fmaf(s[hb][mb][3], c, nm));
          rs += (p0 + p1) + (p2 + p3);
          pk[hb][ks][2 * half] = pack_bf16x2(p0, p1);
          pk[hb][ks][2 * half + 1] = pack_bf16x2(p2, p3);
        }
      }
      l[hb] += rs;
    }
    // O^T += V^T P^T: 32-key step ks, lane group g4 holds in k-slot t the key
    // 32*ks + 4*g4 + t (t < 4) or 32*ks + 16 + 4*g4 + (t - 4) -- the keys of its
    // S^T registers; V^T for d block db comes from two transposing reads.
    const int tq = l16 >> 2, qq = l16 & 3;
    bf16x8 vop[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint32_t w[4];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int row = 32 * ks + 16 * rr + 4 * g4 + tq;
          const int chunkq = 2 * db + (qq >> 1);
          const uint32_t off = swz<1>(row, chunkq) + 8 * (qq & 1);
          const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)to_lds((void*)(sV + off)));
          const u32x2 tw = __builtin_bit_cast(u32x2, t);
          w[2 * rr] = tw[0];
          w[2 * rr + 1] = tw[1];
        }
        u32x4 va;
        va[0] = w[0]; va[1] = w[1]; va[2] = w[2]; va[3] = w[3];
        vop[db][ks] = as_bf16x8(va);
      }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) o[hb][db] = mfma16(vop[db][ks], as_bf16x8(pk[hb][ks]), o[hb][db]);
  }

  // Partial state per head: reference max (log2 units), sum, unnormalised output.
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hh = 16 * hb + l16;
    const float lt = sum_xor32(sum_xor16(l[hb]));
    if (hh < G) {
      float* part = ws + ((size_t)(head0 + hh) * npieces + piece) * kPartialFloats;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        f32x4 v = o[hb][db];
        *reinterpret_cast<f32x4*>(part + 2 + 16 * db + 4 * g4) = v;
      }
      if (g4 == 0) {
        part[0] = m[hb];
        part[1] = lt;
      }
    }
  }
}

// Merge the slice partials of one (sequence, head): lane = output column.
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(const float* __restrict__ ws,
                                                                 uint16_t* __restrict__ out,
                                                                 float* __restrict__ lse, int npieces) {
  const int lane = threadIdx.x;
  const size_t bh = blockIdx.x;
  const float* part = ws + bh * npieces * kPartialFloats;
  // the first slices' outputs are requested before the maximum is formed
  constexpr int kChunk = 8;
  float ov[kChunk];
#pragma unroll
  for (int u = 0; u < kChunk; ++u) ov[u] = part[min(u, npieces - 1) * kPartialFloats + 2 + lane];
  // lane c < npieces holds slice c's reference max and sum (npieces <= 64)
  const int cl = lane < npieces ? lane : npieces - 1;
  float mc = part[cl * kPartialFloats];
  const float lc = part[cl * kPartialFloats + 1];
  if (lane >= npieces) mc = -__builtin_inff();
  float M = mc;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float fc = mc == -__builtin_inff() ? 0.f : fast_exp2(mc - M);
  // slices in order: L = sum l_c f_c, O = sum o_c f_c (empty slices weigh 0)
  float L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < npieces; c0 += kChunk) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < kChunk; ++u) ov[u] = part[min(c0 + u, npieces - 1) * kPartialFloats + 2 + lane];
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int c = c0 + u;
      if (c < npieces) {
        const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fc), c));
        L += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lc), c)) * f;
        O += ov[u] * f;
      }
    }
  }
  const float v = O / L;
  const __bf16 bv = (__bf16)v;
  out[bh * kHeadDim + lane] = __builtin_bit_cast(uint16_t, bv);
  if (lane == 0) lse[bh] = (M + fast_log2(L)) * kLn2;
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, float* workspace, const Geometry& g,
                              hipStream_t stream) {
  const int npieces = decode_pieces(g.batch, g.hkv);
  const size_t nwg = (size_t)g.batch * g.hkv * npieces;
  if (nwg == 0) return hipSuccess;
  const size_t dyn =
      (2 * (size_t)((g.nkb + 31) / 32) + 2 * (size_t)g.group * g.topk + (size_t)g.topk) * sizeof(uint32_t);
  if (g.group <= 16)
    hipLaunchKernelGGL(attn_decode_partial_kernel<1>, dim3((unsigned)nwg), dim3(64), dyn, stream, a, workspace, g,
                       npieces);
  else if (g.group <= 32)
    hipLaunchKernelGGL(attn_decode_partial_kernel<2>, dim3((unsigned)nwg), dim3(64), dyn, stream, a, workspace, g,
                       npieces);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3((unsigned)(g.batch * g.hq)), dim3(64), 0, stream,
                     workspace, a.out, a.lse, npieces);
  return hipGetLastError();
}

}  // namespace ssa
