// Decode attention (gfx950): one query token per (sequence, query head) against
// a long KV cache, over the key blocks each head selected.
//
// The key blocks of one (sequence, KV head) group are cut into chunks.  A
// workgroup owns one chunk: it forms, per block, the bitmask of the group's
// query heads that selected it, and streams every block of the chunk that any
// head selected exactly once from HBM (the union over the group), applying it
// to each selecting head.  Each workgroup writes one partial online-softmax
// state (max, sum, unnormalised output) per head; a second kernel merges the
// chunk partials.  The work is bound by HBM reads of the union of selected
// K/V blocks.
//
// Method: DashAttention summary, "Etapa 0" (chunk summaries cached once
// complete, no recomputation at inference) and "Resultados Experimentales"
// (memory-bound decoding); S2O summary, "Permutacion en Linea" (index-guided
// loading from an unchanged HBM layout); SSA guide (mauroscia.it),
// "Block-sparse attention e Receptive Field".
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kWaves = 4;
constexpr int kKRow = 66;  // LDS row stride (bf16) of the key tile: 33 dwords -> one row per lane, no conflicts

struct DecodeSmem {
  uint32_t mask[kDecodeChunk];
  union {
    struct {
      uint16_t k[kWaves][kBlock * kKRow];
      uint16_t v[kWaves][kBlock * kHeadDim];
      float p[kWaves][kBlock];
    } tile;
    float merge[kWaves][32][kPartialFloats];
  } u;
};

template <int GMAX>
__global__ __launch_bounds__(256) void attn_decode_partial_kernel(AttnArgs a, float* __restrict__ ws,
                                                                  Geometry geo, int nchunks) {
  __shared__ __attribute__((aligned(16))) DecodeSmem sm;
  __shared__ __attribute__((aligned(16))) float sQ[GMAX][kHeadDim];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bg = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - bg * nchunks;
  const int b = bg / geo.hkv, g = bg - b * geo.hkv;
  const int G = geo.group;
  const int j0 = chunk * kDecodeChunk;
  const int nj = min(kDecodeChunk, geo.nkb - j0);

  if (tid < kDecodeChunk) sm.mask[tid] = 0u;
  for (int e = tid; e < G * kHeadDim; e += 256)
    sQ[e >> 6][e & 63] = bf16_to_f32(a.q[(size_t)(b * geo.hq + g * G) * kHeadDim + e]);
  __syncthreads();
  // Which heads of the group selected each block of this chunk.
  for (int e = tid; e < G * geo.topk; e += 256) {
    const int hh = e / geo.topk;
    const int j = a.idx[(size_t)(b * geo.hq + g * G) * geo.topk + e];
    if (j >= j0 && j < j0 + nj) atomicOr(&sm.mask[j - j0], 1u << hh);
  }
  __syncthreads();

  float m[GMAX], l[GMAX], o[GMAX];
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    m[hh] = -__builtin_inff();
    l[hh] = 0.f;
    o[hh] = 0.f;
  }
  const size_t kvoff = (size_t)(b * geo.hkv + g) * geo.seq_kv * kHeadDim;
  uint16_t* sk = sm.u.tile.k[wave];
  uint16_t* sv = sm.u.tile.v[wave];
  float* sp = sm.u.tile.p[wave];
  const int pos = geo.q_offset;  // absolute position of the query token
  int rank = 0;
  for (int jj = 0; jj < nj; ++jj) {
    const uint32_t hm = sm.mask[jj];
    if (hm == 0u) continue;
    if ((rank++ & (kWaves - 1)) != wave) continue;
    const int j = j0 + jj;
    // Stage K (padded rows) and V (dense rows) of block j.
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = it * 64 + lane, row = c >> 3, c8 = c & 7;
      const int key = j * kBlock + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < geo.seq_kv) {
        kv = *reinterpret_cast<const u32x4*>(a.k + kvoff + (size_t)key * kHeadDim + c8 * 8);
        vv = *reinterpret_cast<const u32x4*>(a.v + kvoff + (size_t)key * kHeadDim + c8 * 8);
      }
      uint32_t* kd = reinterpret_cast<uint32_t*>(&sk[row * kKRow + c8 * 8]);
      kd[0] = kv[0]; kd[1] = kv[1]; kd[2] = kv[2]; kd[3] = kv[3];
      *reinterpret_cast<u32x4*>(&sv[row * kHeadDim + c8 * 8]) = vv;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // This lane's key row.
    uint32_t kr[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) kr[u] = reinterpret_cast<const uint32_t*>(&sk[lane * kKRow])[u];
    const int key = j * kBlock + lane;
    const bool visible = key <= pos && key < geo.seq_kv;
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh) {
      if (hh >= G || !((hm >> hh) & 1u)) continue;
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        s = fmaf(bf16_to_f32((uint16_t)(kr[u] & 0xffffu)), sQ[hh][2 * u], s);
        s = fmaf(bf16_to_f32((uint16_t)(kr[u] >> 16)), sQ[hh][2 * u + 1], s);
      }
      const float x = visible ? s * geo.scale_log2 : -__builtin_inff();
      const float mx = wave_max(x);
      const float mn = fmaxf(m[hh], mx);
      const float alpha = fast_exp2(m[hh] - mn);
      const float p = fast_exp2(x - mn);
      l[hh] = l[hh] * alpha + wave_sum(p);
      m[hh] = mn;
      sp[lane] = p;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float acc = 0.f;
#pragma unroll 16
      for (int t = 0; t < kBlock; ++t) acc = fmaf(sp[t], bf16_to_f32(sv[t * kHeadDim + lane]), acc);
      o[hh] = o[hh] * alpha + acc;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Merge the waves' states per head, then write this chunk's partials.
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    if (hh >= G) continue;
    sm.u.merge[wave][hh][2 + lane] = o[hh];
    if (lane == 0) {
      sm.u.merge[wave][hh][0] = m[hh];
      sm.u.merge[wave][hh][1] = l[hh];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += 256) {
    const int hh = e >> 6, d = e & 63;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.u.merge[w][hh][0]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.u.merge[w][hh][0];
        if (mw == -__builtin_inff()) continue;
        const float f = fast_exp2(mw - M);
        L += sm.u.merge[w][hh][1] * f;
        O += sm.u.merge[w][hh][2 + d] * f;
      }
    }
    float* part = ws + ((size_t)(b * geo.hq + g * G + hh) * nchunks + chunk) * kPartialFloats;
    part[2 + d] = O;
    if (d == 0) {
      part[0] = M;
      part[1] = L;
    }
  }
}

// Merge the chunk partials of one (sequence, head): lane = output column.
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(const float* __restrict__ ws,
                                                                 uint16_t* __restrict__ out,
                                                                 float* __restrict__ lse, int nchunks) {
  const int lane = threadIdx.x;
  const size_t bh = blockIdx.x;
  const float* part = ws + bh * nchunks * kPartialFloats;
  float M = -__builtin_inff();
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, part[c * kPartialFloats]);
  float L = 0.f, O = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const float mc = part[c * kPartialFloats];
    if (mc == -__builtin_inff()) continue;
    const float f = fast_exp2(mc - M);
    L += part[c * kPartialFloats + 1] * f;
    O += part[c * kPartialFloats + 2 + lane] * f;
  }
  const float v = O / L;
  const __bf16 bv = (__bf16)v;
  out[bh * kHeadDim + lane] = __builtin_bit_cast(uint16_t, bv);
  if (lane == 0) lse[bh] = (M + fast_log2(L)) * kLn2;
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, float* workspace, const Geometry& g,
                              hipStream_t stream) {
  const int nchunks = decode_chunks(g.nkb);
  const size_t nwg = (size_t)g.batch * g.hkv * nchunks;
  if (nwg == 0) return hipSuccess;
  const dim3 grid((unsigned)nwg), block(256);
  if (g.group <= 1)
    hipLaunchKernelGGL(attn_decode_partial_kernel<1>, grid, block, 0, stream, a, workspace, g, nchunks);
  else if (g.group <= 2)
    hipLaunchKernelGGL(attn_decode_partial_kernel<2>, grid, block, 0, stream, a, workspace, g, nchunks);
  else if (g.group <= 4)
    hipLaunchKernelGGL(attn_decode_partial_kernel<4>, grid, block, 0, stream, a, workspace, g, nchunks);
  else if (g.group <= 8)
    hipLaunchKernelGGL(attn_decode_partial_kernel<8>, grid, block, 0, stream, a, workspace, g, nchunks);
  else if (g.group <= 16)
    hipLaunchKernelGGL(attn_decode_partial_kernel<16>, grid, block, 0, stream, a, workspace, g, nchunks);
  else if (g.group <= 32)
    hipLaunchKernelGGL(attn_decode_partial_kernel<32>, grid, block, 0, stream, a, workspace, g, nchunks);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3((unsigned)(g.batch * g.hq)), dim3(64), 0, stream,
                     workspace, a.out, a.lse, nchunks);
  return hipGetLastError();
}

}  // namespace ssa
