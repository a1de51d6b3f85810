// Decode block scores and top-k selection in one launch (gfx950).
//
// One workgroup of 16 wavefronts per (sequence, KV head).  The scores of every
// query head of the group against every key block are computed as the decode
// scores kernel computes them (fp64 matrix products of the query row and the
// cached summaries, one rounding to fp32) and stay in LDS; then one wavefront
// per query head ranks its row as the selection kernel does, or, with the
// group-shared selection, one wavefront ranks the mean of the group's rows.
// The results are those of the two separate calls; the scores skip the round
// trip through memory and the selection its own launch.
// Method: SSA guide (mauroscia.it), "Block-sparse attention e Receptive
// Field" (fixed top-k block budget); DashAttention summary, "Etapa 0" (cached
// chunk summaries), "Etapa 1" (query-vs-summary routing, averaged over the
// query heads of a KV head for a shared selection) and "Etapa 2" (the most
// recent chunk kept by its own branch).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"
#include "ssa_score_ops.hpp"
#include "ssa_select.hpp"

namespace ssa {
namespace {

constexpr int kFsWaves = 16;
constexpr int kFsTiles = 2;  // 16-block column tiles a wavefront scores per step, loads in flight together
constexpr size_t kFsMaxLds = 64 * 1024;

// Ranks one row of candidates 0 .. jd-1 (jd = the most recent block, always kept).
template <int NPER>
__device__ __forceinline__ void select_one_row(const float* srow_base, int32_t* __restrict__ orow, int jd, int k,
                                               int lane, uint32_t* cbuf) {
  if (jd + 1 <= k) {
    for (int e = lane; e < k; e += 64) orow[e] = e <= jd ? e : -1;
    return;
  }
  RowScores srow;
  srow.s0 = srow_base;
  srow.hstride = 0;
  srow.heads = 1;
  if (NPER > 0)
    select_rows<(NPER > 0 ? NPER : 1)>(srow, orow, jd, k - 1, lane, cbuf);
  else
    select_rows_long(srow, orow, jd, k - 1, lane);
  if (lane == 0) orow[k - 1] = jd;
}

template <int NPER, bool SHARED>
__global__ __launch_bounds__(64 * kFsWaves) void decode_select_kernel(const uint16_t* __restrict__ q,
                                                                    const float* __restrict__ ksum,
                                                                    float* __restrict__ scores,
                                                                    int32_t* __restrict__ idx, Geometry geo) {
  extern __shared__ float sS[];  // [G][nkb] scores; with SHARED then [nkb] group mean
  __shared__ uint32_t sCb[kFsWaves][64];  // per-wave gather buffers of the narrowed search
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, ks = lane >> 4;
  const int bg = blockIdx.x;
  const int b = bg / geo.hkv, g = bg - b * geo.hkv;
  const int G = geo.group, nkb = geo.nkb;
  const int jd = geo.q_offset / kBlock;
  const double scale = (double)geo.scale;
  const uint16_t* qg = q + (size_t)(b * geo.hq + g * G) * kHeadDim + 16 * ks;  // seq_q == 1
  const float* kg = ksum + (size_t)bg * nkb * kHeadDim + 16 * ks;
  const int nbt = (nkb + 15) / 16;

  // scores: 16-head row tiles h0; a wavefront takes column tiles
  // kFsTiles * wave + 16 * kFsTiles * n .. + kFsTiles - 1
  for (int h0 = 0; h0 < G; h0 += 16) {
    uint4 qv[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    if (h0 + col < G) {
      const uint4* qr = reinterpret_cast<const uint4*>(qg + (size_t)(h0 + col) * kHeadDim);
      qv[0] = qr[0];
      qv[1] = qr[1];
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
    for (int t0 = kFsTiles * wave; t0 < nbt; t0 += kFsTiles * kFsWaves) {
      double kb[kFsTiles][16];
#pragma unroll
      for (int t = 0; t < kFsTiles; ++t)
        load_row16_f64(kg + (size_t)min(16 * (t0 + t) + col, nkb - 1) * kHeadDim, kb[t]);
#pragma unroll
      for (int t = 0; t < kFsTiles; ++t) {
        const f64x4 c = mfma_dot64(qa, kb[t], f64x4{0.0, 0.0, 0.0, 0.0});
        const int j = 16 * (t0 + t) + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hh = h0 + ks + 4 * r;
          if (hh < G && j < nkb) sS[hh * nkb + j] = j <= jd ? (float)(scale * c[r]) : -__builtin_inff();
        }
      }
    }
  }
  __syncthreads();
  if (scores) {  // the group's rows are consecutive in [b, Hq, 1, nkb]
    float* srow = scores + (size_t)(b * geo.hq + g * G) * nkb;
    for (int e = tid; e < G * nkb; e += 64 * kFsWaves) srow[e] = sS[e];
  }
  const int k = geo.topk;
  if (!SHARED) {
    for (int hh = wave; hh < G; hh += kFsWaves)
      select_one_row<NPER>(sS + hh * nkb, idx + (size_t)(b * geo.hq + g * G + hh) * k, jd, k, lane, sCb[wave]);
  } else {
    // mean of the group's scores: fp64 sum in head order, divided by the group
    // size, rounded once to fp32
    float* smean = sS + G * nkb;
    for (int j = tid; j < nkb; j += 64 * kFsWaves) {
      double acc = 0.0;
      for (int hh = 0; hh < G; ++hh) acc += (double)sS[hh * nkb + j];
      smean[j] = (float)(acc / G);
    }
    __syncthreads();
    if (wave == 0) select_one_row<NPER>(smean, idx + (size_t)bg * k, jd, k, lane, sCb[0]);
  }
}

template <bool SHARED>
hipError_t launch_fused(const uint16_t* q, const float* ksum, float* scores, int32_t* idx, const Geometry& g,
                        size_t lds, hipStream_t stream) {
  const dim3 grid((unsigned)(g.batch * g.hkv)), block(64 * kFsWaves);
  const int jd = g.q_offset / kBlock;
  if (jd <= 128)
    hipLaunchKernelGGL((decode_select_kernel<2, SHARED>), grid, block, lds, stream, q, ksum, scores, idx, g);
  else if (jd <= 512)
    hipLaunchKernelGGL((decode_select_kernel<8, SHARED>), grid, block, lds, stream, q, ksum, scores, idx, g);
  else
    hipLaunchKernelGGL((decode_select_kernel<0, SHARED>), grid, block, lds, stream, q, ksum, scores, idx, g);
  return hipGetLastError();
}

}  // namespace

size_t decode_select_lds_bytes(const Geometry& g, bool shared) {
  return ((size_t)g.group * g.nkb + (shared ? (size_t)g.nkb : 0)) * sizeof(float);
}

bool decode_select_fits(const Geometry& g, bool shared) {
  return g.group <= 32 && decode_select_lds_bytes(g, shared) <= kFsMaxLds;
}

hipError_t launch_decode_select(const uint16_t* q, const float* ksum, float* scores, int32_t* idx, const Geometry& g,
                                bool shared, hipStream_t stream) {
  if ((size_t)g.batch * g.hkv == 0 || g.nkb == 0) return hipSuccess;
  if (!decode_select_fits(g, shared)) return hipErrorInvalidValue;
  const size_t lds = decode_select_lds_bytes(g, shared);
  return shared ? launch_fused<true>(q, ksum, scores, idx, g, lds, stream)
                : launch_fused<false>(q, ksum, scores, idx, g, lds, stream);
}

}  // namespace ssa
