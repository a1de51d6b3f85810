// alpha-entmax routing (gfx950): per (b, KV head g, query block i), every
// query head h of the group turns its block scores into routing weights
//   p_h = alpha-entmax(gamma * scores[b,h,i,j]),  j < diag(i),
//   alpha-entmax(z)_j = max(0, (alpha-1) z_j - tau) ** (1/(alpha-1)),  sum_j = 1,
// the group's weights are the mean over its heads, and the block list is the
// diagonal block plus every block of positive weight (past topk blocks: the
// topk-1 largest weights, lower index on ties), ascending, with a logit bias
// sigma * ln(w) per routed block (0 for the diagonal).
// tau is found by Newton's method from max - 1 (the mass is convex and
// decreasing in tau, so the iterates rise monotonically to the root), one
// wavefront per head with DPP reductions; the weights are then normalised.
// Method: DashAttention summary, "Etapa 1" (entmax routing of the chunk
// logits; with grouped-query attention the probabilities of the heads sharing
// a KV head are averaged into one sparse support) and "Etapa 2" (prior bias
// from the routing weights added to the logits; near-diagonal chunks in their
// own branch).
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kRouteWaves = 8;
constexpr int kNewtonSteps = 32;  // cap; a handful of steps reach fp32 resolution

// Whole-wave sum / max on the VALU: DPP within rows of 16 lanes (quad
// permutes, then the half-row and row mirrors), then the 16- and 32-lane
// swaps; every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return sum_xor32(sum_xor16(x));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return max_xor32(max_xor16(x));
}

__device__ __forceinline__ float entmax_pow(float x, float inv, int kind) {
  // x >= 0; kind 2: alpha = 2 (power 1), kind 1: alpha = 1.5 (power 2), else general
  if (kind == 2) return x;
  if (kind == 1) return x * x;
  return x > 0.f ? __builtin_amdgcn_exp2f(inv * __builtin_amdgcn_logf(x)) : 0.f;
}

// d/dx of x^inv for x >= 0 (0 at x = 0).
__device__ __forceinline__ float entmax_dpow(float x, float inv, int kind) {
  if (kind == 2) return x > 0.f ? 1.f : 0.f;
  if (kind == 1) return 2.f * x;
  return x > 0.f ? inv * __builtin_amdgcn_exp2f((inv - 1.f) * __builtin_amdgcn_logf(x)) : 0.f;
}

// Dynamic LDS: per wave, the scaled scores of its current head (n floats) and
// the sum of its heads' weights (n floats).
__global__ __launch_bounds__(64 * kRouteWaves) void entmax_route_kernel(const float* __restrict__ scores, float alpha, float gamma,
                                                           float sigma, int32_t* __restrict__ idx,
                                                           float* __restrict__ bias, float* __restrict__ weights,
                                                           Geometry geo, int npad) {
  extern __shared__ float lds[];
  __shared__ int sCount;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = blockIdx.x % geo.nqb;
  const int gi = blockIdx.x / geo.nqb;
  const int b = gi / geo.hkv, g = gi - b * geo.hkv;
  const int G = geo.group;
  const int jd = (geo.q_offset + i * kBlock) / kBlock;
  const int n = jd;  // routed candidates: the blocks before the diagonal
  float* zt = lds + (size_t)wave * 2 * npad;
  float* acc = zt + npad;
  const float am1 = alpha - 1.f;
  const float inv = 1.f / am1;
  const int kind = alpha == 2.f ? 2 : (alpha == 1.5f ? 1 : 0);

  for (int j = lane; j < n; j += 64) acc[j] = 0.f;
  // heads g*G + wave*hpw .. +hpw-1 (contiguous), summed in head order per wave
  const int hpw = (G + kRouteWaves - 1) / kRouteWaves;
  for (int t = 0; t < hpw && n > 0; ++t) {
    const int hh = wave * hpw + t;
    if (hh >= G) break;
    const float* srow = scores + (((size_t)b * geo.hq + g * G + hh) * geo.nqb + i) * geo.nkb;
    float mx = -__builtin_inff();
    int nfin = 0;
    for (int j = lane; j < n; j += 64) {
      const float z = srow[j];
      const bool fin = __builtin_isfinite(z);
      const float v = fin ? am1 * (gamma * z) : -__builtin_inff();
      zt[j] = v;
      mx = fmaxf(mx, v);
      nfin += fin ? 1 : 0;
    }
    mx = wave_max_dpp(mx);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) nfin += __shfl_xor(nfin, o, 64);
    if (nfin == 0) continue;
    // Newton from below: the mass f(tau) = sum max(0, zt - tau)^inv is convex
    // and decreasing (inv >= 1), so from tau0 = max - 1 (f >= 1) each step
    // lands at or below the root; stop when tau no longer increases.
    float lo = mx - 1.f;
    for (int it = 0; it < kNewtonSteps; ++it) {
      float f = 0.f, df = 0.f;
      for (int j = lane; j < n; j += 64) {
        const float x = fmaxf(zt[j] - lo, 0.f);
        f += entmax_pow(x, inv, kind);
        df += entmax_dpow(x, inv, kind);
      }
      f = wave_sum_dpp(f);
      df = wave_sum_dpp(df);
      const float nxt = lo + (f - 1.f) / df;
      if (!(nxt > lo)) break;
      lo = nxt;
    }
    float tot = 0.f;
    for (int j = lane; j < n; j += 64) tot += entmax_pow(fmaxf(zt[j] - lo, 0.f), inv, kind);
    tot = wave_sum_dpp(tot);
    const float rs = 1.f / tot;
    for (int j = lane; j < n; j += 64) acc[j] += entmax_pow(fmaxf(zt[j] - lo, 0.f), inv, kind) * rs;
  }
  __syncthreads();
  // group mean into wave 0's accumulator: (((w0 + w1) + w2) + ...), over G
  const float rg = 1.f / (float)G;
  for (int j = tid; j < n; j += 64 * kRouteWaves) {
    float s = lds[npad + j];
    for (int w = 1; w < kRouteWaves; ++w) s += lds[(size_t)w * 2 * npad + npad + j];
    lds[npad + j] = s * rg;
  }
  if (tid == 0) sCount = 0;
  __syncthreads();
  float* wbar = lds + npad;
  const size_t row = ((size_t)gi * geo.nqb + i);
  if (weights) {
    for (int j = tid; j < geo.nkb; j += 64 * kRouteWaves) weights[row * geo.nkb + j] = j < n ? wbar[j] : 0.f;
  }
  // support size, then (if it exceeds topk - 1) the rank of each block by weight
  int cnt = 0;
  for (int j = tid; j < n; j += 64 * kRouteWaves) cnt += wbar[j] > 0.f ? 1 : 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) atomicAdd(&sCount, cnt);  // integer sum: order-independent
  __syncthreads();
  const int nsup = sCount;
  const int keep = geo.topk - 1;
  float* flag = lds;  // wave 0's score buffer, reused: 1 = block kept
  for (int j = tid; j < n; j += 64 * kRouteWaves) {
    const float wj = wbar[j];
    bool kept = wj > 0.f;
    if (kept && nsup > keep) {
      int rank = 0;
      for (int j2 = 0; j2 < n; ++j2) {
        const float w2 = wbar[j2];
        rank += (w2 > wj || (w2 == wj && j2 < j)) ? 1 : 0;
      }
      kept = rank < keep;
    }
    flag[j] = kept ? 1.f : 0.f;
  }
  __syncthreads();
  if (wave == 0) {
    // ascending compaction of the kept blocks, then the diagonal, then -1
    int outp = 0;
    int32_t* irow = idx + row * geo.topk;
    float* brow = bias + row * geo.topk;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      const bool kept = j < n && flag[j] != 0.f;
      const uint64_t m = __builtin_amdgcn_ballot_w64(kept);
      if (kept) {
        const int e = outp + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull));
        irow[e] = j;
        // the hardware log takes no subnormal input: those weights are scaled by 2^64 first
        const float wj = wbar[j];
        const bool tiny = wj < 1.17549435e-38f;
        const float lg2 = __builtin_amdgcn_logf(tiny ? wj * 18446744073709551616.f : wj) - (tiny ? 64.f : 0.f);
        brow[e] = sigma * (lg2 * kLn2);
      }
      outp += (int)__builtin_popcountll(m);
    }
    for (int e = outp + lane; e < geo.topk; e += 64) {
      irow[e] = e == outp ? jd : -1;
      brow[e] = 0.f;
    }
  }
}

}  // namespace

hipError_t launch_entmax_route(const float* scores, float alpha, float gamma, float sigma, int32_t* idx,
                               float* bias, float* weights, const Geometry& g, hipStream_t stream) {
  const size_t rows = (size_t)g.batch * g.hkv * g.nqb;
  if (rows == 0) return hipSuccess;
  const int npad = (g.nkb + 63) & ~63;
  const size_t lds = (size_t)kRouteWaves * 2 * npad * sizeof(float);
  hipLaunchKernelGGL(entmax_route_kernel, dim3((unsigned)rows), dim3(64 * kRouteWaves), lds, stream, scores, alpha,
                     gamma, sigma,
                     idx, bias, weights, g, npad);
  return hipGetLastError();
}

}  // namespace ssa
