// Measured peaks of one MI355X (gfx950), beside which the attention kernels'
// rates are read: a loop of bf16 matrix instructions with no memory traffic,
// a streaming read and a streaming copy of device memory, and the shader
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

// Grid-stride streaming read of n16 16-byte words; each block writes the XOR
// of what it read to out[blockIdx.x].
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                        uint32_t* __restrict__ out) {
  __shared__ uint32_t red[4];
  uint32_t x = 0u;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
    x ^= v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Grid-stride streaming copy of n16 16-byte words.
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + stride < n16; i += 2 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
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
