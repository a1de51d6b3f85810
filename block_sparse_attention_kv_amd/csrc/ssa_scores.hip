// Block summaries and coarse block scores (gfx950).
//
// Summaries: the mean of each 64-row key block, summed exactly in fp64 and
// rounded once to fp32.  Scores: fp32 rounding of scale * qbar . kbar, with
// the dot product accumulated in fp64 from the fp32 summaries, so the top-k
// decision downstream is taken on correctly rounded fp32 scores.
// Method: SSA guide (mauroscia.it), "Block-sparse attention e Receptive Field";
// DashAttention summary, "Etapa 0" (mean summary, cached once complete) and
// "Etapa 1" (query-vs-summary routing logits).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

// Sum the rows [0, nrows) of a 64-wide bf16 block in fp64.  Lane layout: lane
// covers columns 8*(lane%8) .. +8 of rows lane/8, lane/8 + 8, ...; all eight
// loads are issued before any is used.  The eight row groups are then folded
// together, so lanes 0..7 end with the column sums.
__device__ __forceinline__ void pool_rows_f64(const uint16_t* __restrict__ base, int nrows,
                                              int lane, double acc[8]) {
  const int c8 = lane & 7, rg = lane >> 3;
  u32x4 v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = rg + 8 * k;
    v[k] = *reinterpret_cast<const u32x4*>(base + (size_t)(r < nrows ? r : 0) * kHeadDim + c8 * 8);
    if (r >= nrows) v[k] = u32x4{0u, 0u, 0u, 0u};
  }
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

constexpr int kScoreQb = 4;     // query blocks per workgroup (prefill): one per wavefront
constexpr int kScoreKTile = 64;  // key blocks staged per pass (decode)
constexpr int kKbStride = 65;    // padded LDS row (floats) -> conflict-free row-per-lane reads

// One workgroup of four wavefronts per (b, h, 4 query blocks, 256 key
// blocks).  Each wavefront pools one query block (Q is read once per 256 key
// blocks: once overall up to 16k tokens); then each thread scores one key
// block's summary (read straight from global memory, L2-resident) against
// the pooled blocks.
__global__ __launch_bounds__(256) void prefill_scores_kernel(const uint16_t* __restrict__ q,
                                                             const float* __restrict__ ksum,
                                                             float* __restrict__ scores,
                                                             Geometry geo) {
  __shared__ double sQ[kScoreQb][kHeadDim];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntile = (geo.nqb + kScoreQb - 1) / kScoreQb;
  const int bh = blockIdx.x / ntile;
  const int j = blockIdx.y * 256 + tid;
  const int i0 = (blockIdx.x - bh * ntile) * kScoreQb;
  const int b = bh / geo.hq, h = bh - b * geo.hq, g = h / geo.group;
  const int nq = min(kScoreQb, geo.nqb - i0);

  const int jd0 = geo.q_offset / kBlock + i0;  // diagonal block of the first query block
  float* srow = scores + ((size_t)bh * geo.nqb + i0) * geo.nkb;
  if ((int)blockIdx.y * 256 > jd0 + nq - 1) {  // every key block here is past the diagonal
    if (j < geo.nkb)
      for (int qi = 0; qi < nq; ++qi) srow[(size_t)qi * geo.nkb + j] = -__builtin_inff();
    return;
  }
  if (wave < nq) {
    const int r0 = (i0 + wave) * kBlock;
    const int nrows = min(kBlock, geo.seq_q - r0);
    double acc[8];
    pool_rows_f64(q + ((size_t)bh * geo.seq_q + r0) * kHeadDim, nrows, lane, acc);
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sQ[wave][lane * 8 + e] = (double)(float)(acc[e] / nrows);
    }
  }
  __syncthreads();

  const float* kb = ksum + (size_t)(b * geo.hkv + g) * geo.nkb * kHeadDim;
  const double scale = (double)geo.scale;
  if (j < geo.nkb) {
    float out[kScoreQb];
#pragma unroll
    for (int qi = 0; qi < kScoreQb; ++qi) out[qi] = -__builtin_inff();
    if (j <= jd0 + nq - 1) {
      const float4* kr = reinterpret_cast<const float4*>(kb + (size_t)j * kHeadDim);
      float4 kv[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) kv[x] = kr[x];
      double acc[kScoreQb] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float kk[4] = {kv[x].x, kv[x].y, kv[x].z, kv[x].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double kd = (double)kk[e];
#pragma unroll
          for (int qi = 0; qi < kScoreQb; ++qi) acc[qi] = fma(sQ[qi][4 * x + e], kd, acc[qi]);
        }
      }
#pragma unroll
      for (int qi = 0; qi < kScoreQb; ++qi)
        if (j <= jd0 + qi) out[qi] = (float)(scale * acc[qi]);
    }
#pragma unroll
    for (int qi = 0; qi < kScoreQb; ++qi)
      if (qi < nq) srow[(size_t)qi * geo.nkb + j] = out[qi];
  }
}

// Decode (one query row per (b, h)): one workgroup per (b, KV head, pass of
// kScoreKTile key blocks) scores every query head of the group against the
// staged summaries, so each summary is read from HBM once.
constexpr int kMaxGroupScores = 64;
__global__ __launch_bounds__(256) void decode_scores_kernel(const uint16_t* __restrict__ q,
                                                            const float* __restrict__ ksum,
                                                            float* __restrict__ scores,
                                                            Geometry geo) {
  extern __shared__ float sQ[];  // [G][kHeadDim]: the group's query rows (bf16 values, exact in fp32)
  __shared__ float sKb[kScoreKTile * kKbStride];
  const int tid = threadIdx.x;
  const int npass = (geo.nkb + kScoreKTile - 1) / kScoreKTile;
  const int bg = blockIdx.x / npass;
  const int jc = (blockIdx.x - bg * npass) * kScoreKTile;
  const int b = bg / geo.hkv, g = bg - b * geo.hkv;
  const int G = geo.group;
  const int nj = min(kScoreKTile, geo.nkb - jc);
  const uint16_t* qg = q + (size_t)(b * geo.hq + g * G) * kHeadDim;  // seq_q == 1
  for (int e = tid; e < G * kHeadDim; e += 256) sQ[e] = bf16_to_f32(qg[e]);
  const float* kb = ksum + ((size_t)bg * geo.nkb + jc) * kHeadDim;
  for (int e = tid; e < nj * 16; e += 256) {
    const int jj = e >> 4, c4 = e & 15;
    const float4 v = reinterpret_cast<const float4*>(kb + (size_t)jj * kHeadDim)[c4];
    float* d = &sKb[jj * kKbStride + c4 * 4];
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __syncthreads();
  const int jd = geo.q_offset / kBlock;
  const double scale = (double)geo.scale;
  for (int e = tid; e < G * kScoreKTile; e += 256) {
    const int hh = e >> 6, jj = e & 63;
    if (jj >= nj) continue;
    const int j = jc + jj;
    float out;
    if (j > jd) {
      out = -__builtin_inff();
    } else {
      double acc = 0.0;
#pragma unroll 16
      for (int d = 0; d < kHeadDim; ++d)
        acc = fma((double)sQ[hh * kHeadDim + d], (double)sKb[jj * kKbStride + d], acc);
      out = (float)(scale * acc);
    }
    scores[(size_t)(b * geo.hq + g * G + hh) * geo.nkb + j] = out;
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
  const size_t nwg = (size_t)g.batch * g.hq * ((g.nqb + kScoreQb - 1) / kScoreQb);
  if (nwg == 0 || g.nkb == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_scores_kernel, dim3((unsigned)nwg, (unsigned)((g.nkb + 255) / 256)), dim3(256), 0,
                     stream, q, k_summary, scores, g);
  return hipGetLastError();
}

hipError_t launch_decode_scores(const uint16_t* q, const float* k_summary, float* scores,
                                const Geometry& g, hipStream_t stream) {
  if (g.group > kMaxGroupScores) return hipErrorInvalidValue;
  const size_t nwg = (size_t)g.batch * g.hkv * ((g.nkb + kScoreKTile - 1) / kScoreKTile);
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_scores_kernel, dim3((unsigned)nwg), dim3(256),
                     (size_t)g.group * kHeadDim * sizeof(float), stream, q, k_summary, scores, g);
  return hipGetLastError();
}

}  // namespace ssa
