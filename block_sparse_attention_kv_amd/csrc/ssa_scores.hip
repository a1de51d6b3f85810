// Block summaries and coarse block scores (gfx950).
//
// Summaries: the mean of each 64-row key block, summed exactly in fp64 and
// rounded once to fp32.  Scores: fp32 rounding of scale * qbar . kbar, with
// the dot product of exact fp64 products summed in fp64 (on the fp64 matrix
// instruction), so the top-k decision downstream is taken on fp32 scores
// that are correctly rounded except within about 2^-50 relative of a
// rounding boundary.
// Method: SSA guide (mauroscia.it), "Block-sparse attention e Receptive Field";
// DashAttention summary, "Etapa 0" (mean summary, cached once complete) and
// "Etapa 1" (query-vs-summary routing logits).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"
#include "ssa_score_ops.hpp"

namespace ssa {
namespace {

// Sum the rows [0, nrows) of a 64-wide bf16 block in fp64.  Lane layout: lane
// covers columns 8*(lane%8) .. +8 of rows lane/8, lane/8 + 8, ...; the eight
// loads (pool_load_rows) are all issued before any is used.  The eight row
// groups are then folded together (pool_sum_rows), so lanes 0..7 end with the
// column sums.
__device__ __forceinline__ void pool_load_rows(const uint16_t* __restrict__ base, int nrows, int lane,
                                               u32x4 (&v)[8]) {
  const int c8 = lane & 7, rg = lane >> 3;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = rg + 8 * k;
    v[k] = *reinterpret_cast<const u32x4*>(base + (size_t)(r < nrows ? r : 0) * kHeadDim + c8 * 8);
    if (r >= nrows) v[k] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void pool_sum_rows(const u32x4 (&v)[8], double acc[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_to_f32((uint16_t)(v[k][e] & 0xffffu));
      acc[2 * e + 1] += (double)bf16_to_f32((uint16_t)(v[k][e] >> 16));
    }
  }
#pragma unroll
  for (int o = 8; o <= 32; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }
}

__device__ __forceinline__ void pool_rows_f64(const uint16_t* __restrict__ base, int nrows, int lane,
                                              double acc[8]) {
  u32x4 v[8];
  pool_load_rows(base, nrows, lane, v);
  pool_sum_rows(v, acc);
}

__global__ __launch_bounds__(64) void block_summaries_kernel(const uint16_t* __restrict__ k,
                                                             float* __restrict__ ksum, int seq_kv,
                                                             int nkb) {
  const int lane = threadIdx.x;
  const size_t bgj = blockIdx.x;
  const size_t bg = bgj / (size_t)nkb;
  const int j = (int)(bgj - bg * (size_t)nkb);
  const int r0 = j * kBlock;
  const int nrows = min(kBlock, seq_kv - r0);
  double acc[8];
  pool_rows_f64(k + (bg * (size_t)seq_kv + r0) * kHeadDim, nrows, lane, acc);
  if (lane < 8) {
    float4 lo, hi;
    lo.x = (float)(acc[0] / nrows); lo.y = (float)(acc[1] / nrows);
    lo.z = (float)(acc[2] / nrows); lo.w = (float)(acc[3] / nrows);
    hi.x = (float)(acc[4] / nrows); hi.y = (float)(acc[5] / nrows);
    hi.z = (float)(acc[6] / nrows); hi.w = (float)(acc[7] / nrows);
    float4* dst = reinterpret_cast<float4*>(ksum + bgj * kHeadDim + lane * 8);
    dst[0] = lo;
    dst[1] = hi;
  }
}

// Chunk summaries from a learned query (one fp32 vector per KV head): the
// softmax(scale * qbar . k_c)-weighted average of the block's key rows, in
// fp64, rounded once to fp32.  One wavefront per (b, g, j): lane r scores row
// r, then lane d sums column d over the rows.  qbar = 0 reproduces the mean.
// DashAttention summary, "Etapa 0" (a learned query attends to each chunk's
// keys by local scaled dot-product attention).
__global__ __launch_bounds__(64) void learned_summaries_kernel(const uint16_t* __restrict__ k,
                                                               const float* __restrict__ qbar,
                                                               float* __restrict__ ksum, Geometry geo) {
  const int lane = threadIdx.x;
  const size_t bgj = blockIdx.x;
  const size_t bg = bgj / (size_t)geo.nkb;
  const int j = (int)(bgj - bg * (size_t)geo.nkb);
  const int g = (int)(bg % (size_t)geo.hkv);
  const int r0 = j * kBlock;
  const int nrows = min(kBlock, geo.seq_kv - r0);
  const uint16_t* base = k + (bg * (size_t)geo.seq_kv + r0) * kHeadDim;
  const float* qv = qbar + (size_t)g * kHeadDim;
  // row logits (lane = row)
  double logit = -__builtin_inf();
  if (lane < nrows) {
    double acc = 0.0;
    const u32x4* rp = reinterpret_cast<const u32x4*>(base + (size_t)lane * kHeadDim);
#pragma unroll
    for (int c = 0; c < kHeadDim / 8; ++c) {
      const u32x4 v = rp[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += (double)qv[8 * c + 2 * e] * (double)bf16_to_f32((uint16_t)(v[e] & 0xffffu));
        acc += (double)qv[8 * c + 2 * e + 1] * (double)bf16_to_f32((uint16_t)(v[e] >> 16));
      }
    }
    logit = (double)geo.scale * acc;
  }
  double mx = logit;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  const double w = lane < nrows ? exp(logit - mx) : 0.0;
  double wsum = w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
  // weighted column sums (lane = column)
  double col = 0.0;
  for (int r = 0; r < nrows; ++r) {
    const double wr = __shfl(w, r, 64);
    col += wr * (double)bf16_to_f32(base[(size_t)r * kHeadDim + lane]);
  }
  ksum[bgj * kHeadDim + lane] = (float)(col / wsum);
}

constexpr int kScoreQt = 16;    // query blocks per workgroup (prefill): the matrix row tile
constexpr int kScoreWaves = 8;  // wavefronts per workgroup (prefill)
constexpr int kScoreQStride = kHeadDim + 2;  // padded LDS row of the pooled queries (doubles)

// Prefill: one workgroup of eight wavefronts per (b, h, 16 query blocks).
// Each wavefront pools two of the query blocks into LDS (Q is read once);
// then the wavefronts take the 16-block column tiles of the summaries in
// turn (summaries are L2-resident) and write 16 x 16 scores per tile.
// Tiles wholly past the last diagonal are filled with -inf without a product.
__global__ __launch_bounds__(64 * kScoreWaves) void prefill_scores_kernel(const uint16_t* __restrict__ q,
                                                                          const float* __restrict__ ksum,
                                                                          float* __restrict__ scores,
                                                                          Geometry geo) {
  __shared__ double sQ[kScoreQt * kScoreQStride];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntile = (geo.nqb + kScoreQt - 1) / kScoreQt;
  const int bh = blockIdx.x / ntile;
  const int i0 = (blockIdx.x - bh * ntile) * kScoreQt;
  const int b = bh / geo.hq, h = bh - b * geo.hq, g = h / geo.group;
  const int nq = min(kScoreQt, geo.nqb - i0);
  // both query blocks' loads are in flight before either is summed
  constexpr int kPer = kScoreQt / kScoreWaves;
  u32x4 qv[kPer][8];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int qi = wave + kScoreWaves * u;
    const int r0 = (i0 + min(qi, nq - 1)) * kBlock;
    pool_load_rows(q + ((size_t)bh * geo.seq_q + r0) * kHeadDim, qi < nq ? min(kBlock, geo.seq_q - r0) : 0, lane,
                   qv[u]);
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int qi = wave + kScoreWaves * u;
    const int nrows = qi < nq ? min(kBlock, geo.seq_q - (i0 + qi) * kBlock) : 1;
    double acc[8];
    pool_sum_rows(qv[u], acc);
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sQ[qi * kScoreQStride + lane * 8 + e] = qi < nq ? (double)(float)(acc[e] / nrows) : 0.0;
    }
  }
  __syncthreads();

  const int col = lane & 15, ks = lane >> 4;
  double qa[16];
#pragma unroll
  for (int st = 0; st < 16; ++st) qa[st] = sQ[col * kScoreQStride + 16 * ks + st];
  const int jd0 = geo.q_offset / kBlock + i0;       // diagonal block of the first query block
  const int nt_live = (jd0 + nq - 1) / 16 + 1;      // tiles holding a block on or before a diagonal
  const int nt = (geo.nkb + 15) / 16;
  const float* kb = ksum + (size_t)(b * geo.hkv + g) * geo.nkb * kHeadDim + 16 * ks;
  float* srow = scores + ((size_t)bh * geo.nqb + i0) * geo.nkb;
  const double scale = (double)geo.scale;
  for (int t = wave; t < nt; t += kScoreWaves) {
    const int j = 16 * t + col;
    if (t < nt_live) {
      double kv[16];
      load_row16_f64(kb + (size_t)min(j, geo.nkb - 1) * kHeadDim, kv);
      const f64x4 c = mfma_dot64(qa, kv, f64x4{0.0, 0.0, 0.0, 0.0});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = ks + 4 * r;
        if (qi < nq && j < geo.nkb)
          srow[(size_t)qi * geo.nkb + j] = j <= jd0 + qi ? (float)(scale * c[r]) : -__builtin_inff();
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = ks + 4 * r;
        if (qi < nq && j < geo.nkb) srow[(size_t)qi * geo.nkb + j] = -__builtin_inff();
      }
    }
  }
}

// Decode (one query row per (b, h)): one wavefront per (b, KV head, 32 key
// blocks) scores every query head of the group, so each summary is read from
// HBM once: the group's [G x d] query rows times [d x 32] summaries, in 16-row
// tiles of heads.  No LDS: the query rows come straight from memory.
constexpr int kMaxGroupScores = 64;
constexpr int kDscTiles = 2;  // 16-block column tiles per wavefront
constexpr int kDscBlocks = 16 * kDscTiles;
__global__ __launch_bounds__(64) void decode_scores_kernel(const uint16_t* __restrict__ q,
                                                           const float* __restrict__ ksum,
                                                           float* __restrict__ scores, Geometry geo) {
  const int lane = threadIdx.x;
  const int col = lane & 15, ks = lane >> 4;
  const int npass = (geo.nkb + kDscBlocks - 1) / kDscBlocks;
  const int bg = blockIdx.x / npass;
  const int j0 = (blockIdx.x - bg * npass) * kDscBlocks;
  const int b = bg / geo.hkv, g = bg - b * geo.hkv;
  const int G = geo.group;
  const uint16_t* qg = q + (size_t)(b * geo.hq + g * G) * kHeadDim + 16 * ks;  // seq_q == 1
  // first row tile of the query heads: issued before the summaries
  uint4 qv[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  if (col < G) {
    const uint4* qr = reinterpret_cast<const uint4*>(qg + (size_t)col * kHeadDim);
    qv[0] = qr[0];
    qv[1] = qr[1];
  }
  // B operand: summaries of key blocks j0 + 16 t + col (rows past the end
  // read the last block; their scores are not stored)
  double kb[kDscTiles][16];
#pragma unroll
  for (int t = 0; t < kDscTiles; ++t)
    load_row16_f64(ksum + ((size_t)bg * geo.nkb + min(j0 + 16 * t + col, geo.nkb - 1)) * kHeadDim + 16 * ks, kb[t]);
  const int jd = geo.q_offset / kBlock;
  const double scale = (double)geo.scale;
  for (int h0 = 0; h0 < G; h0 += 16) {
    if (h0 > 0) {
      qv[0] = qv[1] = make_uint4(0, 0, 0, 0);
      if (h0 + col < G) {
        const uint4* qr = reinterpret_cast<const uint4*>(qg + (size_t)(h0 + col) * kHeadDim);
        qv[0] = qr[0];
        qv[1] = qr[1];
      }
    }
    double qa[16];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t w[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qa[8 * u + 2 * e] = (double)__uint_as_float(w[e] << 16);
        qa[8 * u + 2 * e + 1] = (double)__uint_as_float(w[e] & 0xffff0000u);
      }
    }
    f64x4 acc[kDscTiles];
#pragma unroll
    for (int t = 0; t < kDscTiles; ++t) acc[t] = mfma_dot64(qa, kb[t], f64x4{0.0, 0.0, 0.0, 0.0});
#pragma unroll
    for (int t = 0; t < kDscTiles; ++t) {
      const int j = j0 + 16 * t + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hh = h0 + ks + 4 * r;
        if (hh < G && j < geo.nkb)
          scores[(size_t)(b * geo.hq + g * G + hh) * geo.nkb + j] =
              j <= jd ? (float)(scale * acc[t][r]) : -__builtin_inff();
      }
    }
  }
}

}  // namespace

hipError_t launch_block_summaries(const uint16_t* k, float* k_summary, const Geometry& g,
                                  hipStream_t stream) {
  const size_t nblk = (size_t)g.batch * g.hkv * g.nkb;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(block_summaries_kernel, dim3((unsigned)nblk), dim3(64), 0, stream, k,
                     k_summary, g.seq_kv, g.nkb);
  return hipGetLastError();
}

hipError_t launch_learned_summaries(const uint16_t* k, const float* qbar, float* k_summary, const Geometry& g,
                                   hipStream_t stream) {
  const size_t nblk = (size_t)g.batch * g.hkv * g.nkb;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(learned_summaries_kernel, dim3((unsigned)nblk), dim3(64), 0, stream, k, qbar, k_summary, g);
  return hipGetLastError();
}

hipError_t launch_prefill_scores(const uint16_t* q, const float* k_summary, float* scores,
                                 const Geometry& g, hipStream_t stream) {
  const size_t nwg = (size_t)g.batch * g.hq * ((g.nqb + kScoreQt - 1) / kScoreQt);
  if (nwg == 0 || g.nkb == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_scores_kernel, dim3((unsigned)nwg), dim3(64 * kScoreWaves), 0, stream, q, k_summary,
                     scores, g);
  return hipGetLastError();
}

hipError_t launch_decode_scores(const uint16_t* q, const float* k_summary, float* scores,
                                const Geometry& g, hipStream_t stream) {
  if (g.group > kMaxGroupScores) return hipErrorInvalidValue;
  const size_t nwg = (size_t)g.batch * g.hkv * ((g.nkb + kDscBlocks - 1) / kDscBlocks);
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_scores_kernel, dim3((unsigned)nwg), dim3(64), 0, stream, q, k_summary, scores, g);
  return hipGetLastError();
}

}  // namespace ssa
