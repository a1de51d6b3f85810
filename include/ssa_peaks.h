/* libssa_peaks: measured peaks of the GPU, for reading the attention kernels'
 * rates against the machine rather than against its nominal figures.  Not
 * part of the method: a measurement aid loaded by the benchmark.
 *
 * Every call enqueues one kernel on `stream` (no host synchronisation) and
 * returns 0, 1 for an invalid argument (nothing launched), or 3 when the
 * launch failed.  Buffers are caller-owned device memory. */
#ifndef SSA_PEAKS_H
#define SSA_PEAKS_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_blocks workgroups of 4 wavefronts; each wavefront issues iters * 16
 * v_mfma_f32_32x32x16_bf16 (32768 flop each) on register operands, in 4
 * independent accumulation chains, with no memory traffic.
 *   out  uint32 [4 * 4 * n_blocks]: per wavefront a checksum, the shader
 *        cycles and the 100 MHz real-time ticks of its loop. */
int ssa_peak_mfma(int32_t iters, int32_t n_blocks, uint32_t* out, hipStream_t stream);

/* n_blocks workgroups of 4 wavefronts (2 * compute units of them gives two
 * wavefronts per SIMD, as the attention kernels run); each wavefront runs
 * `tiles` compute-only replicas of one block-sparse attention tile: 16
 * v_mfma_f32_32x32x16_bf16 score products, the fast-path softmax arithmetic
 * of the 4096 scores (fma, exp2 and a row-sum add per score, a bf16 pack per
 * pair) and 16 P.V products on the packed probabilities, with the attention
 * tile's register layout and dependencies but with operands in registers (no
 * LDS or memory traffic).  1 048 576 matrix flop per tile.
 *   out  uint32 [4 * 4 * n_blocks]: per wavefront a checksum, the shader
 *        cycles and the 100 MHz real-time ticks of its loop. */
int ssa_peak_tile(int32_t tiles, int32_t n_blocks, uint32_t* out, hipStream_t stream);

/* Streaming read of `bytes` (a multiple of 16, 16-byte aligned) by n_blocks
 * workgroups of 256 threads, one contiguous chunk each, non-temporal loads.
 *   out  uint32 [n_blocks]: each workgroup's XOR of the words it read. */
int ssa_peak_read(const void* src, size_t bytes, uint32_t* out, int32_t n_blocks, hipStream_t stream);

/* Streaming copy of `bytes` (a multiple of 16; both pointers 16-byte aligned;
 * the ranges must not overlap) by n_blocks workgroups of 256 threads, one
 * contiguous chunk each, non-temporal loads and stores. */
int ssa_peak_copy(const void* src, void* dst, size_t bytes, int32_t n_blocks, hipStream_t stream);

/* One wavefront waits `ticks` (1 .. 1e8) ticks of the 100 MHz real-time
 * counter and records the shader cycles of its compute unit meanwhile:
 *   out  uint32 [2]: cycles, ticks.  cycles / ticks * 0.1 GHz is the clock.
 * Launched on a second stream while another kernel runs, it reads the clock
 * under that load. */
int ssa_peak_clock(uint32_t ticks, uint32_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSA_PEAKS_H */
