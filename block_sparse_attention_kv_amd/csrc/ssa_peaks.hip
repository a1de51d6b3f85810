// Measured peaks of one MI355X (gfx950), beside which the attention kernels'
// rates are read: a loop of bf16 matrix instructions with no memory traffic,
// a compute-only replica of the attention tile, a streaming read and a
// streaming copy of device memory, and the shader
// clock (shader cycles over the 100 MHz real-time counter) seen by one
// wavefront while other work runs.  C ABI, caller-owned buffers, stream order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssa_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;  // independent accumulators per wave (keeps the matrix core fed back to back)

// Each wave runs iters x 16 v_mfma_f32_32x32x16_bf16 (4 chains of 4) on
// register operands.  out[4 * wave + 0..2] = checksum bits, shader cycles,
// real-time ticks of the loop.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  bf16x8 a[kChains], b;
  for (int r = 0; r < 8; ++r) b[r] = (__bf16)(0.001f * (lane + r));
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 8; ++r) a[c][r] = (__bf16)(0.002f * (c + r + lane));
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b, acc[c], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (lane == 0) {
    out[4 * wave + 0] = __float_as_uint(s);
    out[4 * wave + 1] = (uint32_t)(t1 - t0);
    out[4 * wave + 2] = (uint32_t)(r1 - r0);
    out[4 * wave + 3] = 0u;
  }
}

// Compute-only replica of one block-sparse attention tile (64 query rows x 64
// keys, d = 64, one wavefront): the score products (16 MFMAs), the softmax
// arithmetic of the tile's fast path (per score: one fma, one exp2, one add to
// the row sum; per pair: one bf16 pack) and the P.V products (16 MFMAs) that
// consume the packed probabilities, with the same register layout and the same
// dependencies as the attention kernels' tile, but with the K, V and Q operands
// in registers: no LDS, no memory traffic, no masking.  Each wave runs `tiles`
// such tiles; out[4 * wave + 0..2] = checksum bits, shader cycles, real-time
// ticks of the loop.
__global__ __launch_bounds__(256, 2) void peak_tile_kernel(int tiles, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  bf16x8 qop[2][4], kop[2][4], vop[2][2];
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 4; ++y)
      for (int r = 0; r < 8; ++r) {
        qop[x][y][r] = (__bf16)(0.01f * ((lane + r + x + y) & 7));
        kop[x][y][r] = (__bf16)(0.01f * ((lane + 2 * r + x + 3 * y) & 7));
        if (y < 2) vop[x][y][r] = (__bf16)(0.001f * ((lane + r + 5 * x + y) & 15));
      }
  f32x16 o[2][2];
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 2; ++y)
      for (int r = 0; r < 16; ++r) o[x][y][r] = 0.f;
  float rs[2] = {0.f, 0.f};
  const float c = 0.18033688f, nm = -1.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int t = 0; t < tiles; ++t) {
    f32x16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 acc;
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kb][ks], qop[qb][ks], acc, 0, 0, 0);
        s[kb][qb] = acc;
      }
    u32x4 pk[2][2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ap = 0; ap < 2; ++ap)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * ap + 2 * e], c, nm));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * ap + 2 * e + 1], c, nm));
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const f32x2 v = {p0, p1};
            pk[kb][ap][qb][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
            rs0 += p0;
            rs1 += p1;
          }
      rs[qb] += rs0 + rs1;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[ap][db], __builtin_bit_cast(bf16x8, pk[kb][ap][qb]),
                                                                o[db][qb], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float sum = rs[0] + rs[1];
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 2; ++y)
      for (int r = 0; r < 16; ++r) sum += o[x][y][r];
  if (lane == 0) {
    out[4 * wave + 0] = __float_as_uint(sum);
    out[4 * wave + 1] = (uint32_t)(t1 - t0);
    out[4 * wave + 2] = (uint32_t)(r1 - r0);
    out[4 * wave + 3] = 0u;
  }
}

// Streaming read of n16 16-byte words: each block reads one contiguous chunk,
// four 4 KB steps (256 threads x 16 bytes) in flight, with the non-temporal
// policy; each block writes the XOR of what it read to out[blockIdx.x].
// (Over 1 GiB this pattern read 7.0 TB/s where a grid-stride loop of the same
// loads read 6.5 and temporal loads 6.2.)
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                        uint32_t* __restrict__ out) {
  __shared__ uint32_t red[4];
  uint32_t x = 0u;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  size_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
    x ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
    x ^= v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3];
  }
  for (; i < b1; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Streaming copy of n16 16-byte words, one contiguous chunk per block, two
// 4 KB steps in flight, non-temporal loads and stores.
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        size_t n16) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  size_t i = b0 + threadIdx.x;
  for (; i + 256 < b1; i += 2 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + 256);
  }
  for (; i < b1; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// One wavefront spins for `ticks` ticks of the 100 MHz real-time counter and
// records the shader cycles that passed: out[0] = cycles, out[1] = ticks.
__global__ __launch_bounds__(64) void peak_clock_kernel(uint32_t ticks, uint32_t* __restrict__ out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0, t1 = t0;
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(2);
    r1 = __builtin_amdgcn_s_memrealtime();
    t1 = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x == 0) {
    out[0] = (uint32_t)(t1 - t0);
    out[1] = (uint32_t)(r1 - r0);
  }
}

}  // namespace

extern "C" {

int ssa_peak_mfma(int32_t iters, int32_t n_blocks, uint32_t* out, hipStream_t stream) {
  if (iters < 1 || n_blocks < 1 || !out) return 1;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, (int)iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int ssa_peak_tile(int32_t tiles, int32_t n_blocks, uint32_t* out, hipStream_t stream) {
  if (tiles < 1 || n_blocks < 1 || !out) return 1;
  hipLaunchKernelGGL(peak_tile_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, (int)tiles, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int ssa_peak_read(const void* src, size_t bytes, uint32_t* out, int32_t n_blocks, hipStream_t stream) {
  if (!src || !out || bytes % 16 != 0 || ((uintptr_t)src % 16) != 0 || n_blocks < 1) return 1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, (const u32x4*)src,
                     bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int ssa_peak_copy(const void* src, void* dst, size_t bytes, int32_t n_blocks, hipStream_t stream) {
  if (!src || !dst || bytes % 16 != 0 || ((uintptr_t)src % 16) != 0 || ((uintptr_t)dst % 16) != 0 || n_blocks < 1)
    return 1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(peak_copy_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, (const u32x4*)src,
                     (u32x4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int ssa_peak_clock(uint32_t ticks, uint32_t* out, hipStream_t stream) {
  if (!out || ticks == 0 || ticks > 100000000u) return 1;
  hipLaunchKernelGGL(peak_clock_kernel, dim3(1), dim3(64), 0, stream, ticks, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
