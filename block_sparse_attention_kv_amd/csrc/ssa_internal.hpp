// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssa {

constexpr int kHeadDim = 64;  // the head dimension d the kernels implement
constexpr int kBlock = 64;    // the block size B the kernels implement (one 64-key tile per block)
constexpr int kMaxTopk = 256;

struct Geometry {
  int batch, hq, hkv, group;
  int seq_q, seq_kv, q_offset;
  int topk;
  int nqb, nkb;
  float scale;       // softmax / score scale
  float scale_log2;  // scale * log2(e)
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  int idx_shared;    // 1: one index row per (b, KV head, query block), else per query head
  const float* bias; // optional logit bias per index entry (same layout as idx; natural-log units)
  uint16_t* out;
  float* lse;
  float* dropped;    // full mode only
  int qb_begin;      // first query block handled
  int qb_count;      // number of query blocks handled
  int rows_out;      // rows per (b, h) in the output tensors
  int32_t* queue;    // prefill: work queue of a persistent launch (kQueueBytes, zero between calls), or null
  int n_xcc;         // shares the queue is split into (1..kMaxXcc), one per XCD
  uint32_t* trace;   // optional per-workgroup timing records (kTraceWords each), or null
  int trace_cap;     // records the trace buffer holds
};

// Timing record of one workgroup of a persistent prefill launch: 100 MHz
// real-time counter at start and end (low 32 bits), shader cycles from start
// to end, shader cycles inside the tile loops, units and tiles processed, the
// hardware id and the XCC id of the wavefront that wrote it.
constexpr int kTraceWords = 8;

// Work queue of the persistent prefill launches, in the caller's workspace:
// one counter per share of the launch, each on its own 128-byte line (all
// zero before and after every call).
constexpr int kMaxXcc = 8;
constexpr int kQueueStride = 32;  // int32 words between counters
constexpr size_t kQueueBytes = (size_t)kMaxXcc * kQueueStride * sizeof(int32_t);

// Decode split: the union of the key blocks that the query heads of one
// (batch, KV head) group selected is cut into `decode_pieces` equal slices, one
// wavefront each; every slice writes one partial (m, l, o[64]) per query head,
// merged afterwards.
#ifndef SSA_DECODE_RING
#define SSA_DECODE_RING 2
#endif
#ifndef SSA_DECODE_WAVES
#define SSA_DECODE_WAVES 1024
#endif
constexpr int kDecodeRing = SSA_DECODE_RING;        // K/V block slots per wavefront
constexpr int kDecodeTargetWaves = SSA_DECODE_WAVES;  // wavefronts the split aims for
constexpr int kDecodeMaxPieces = 64;
constexpr int kDecodeMaxList = 2048;    // query heads per group x topk
constexpr int kDecodeMaxBlocks = 65536; // key blocks of the cache
constexpr int kPartialFloats = 2 + 64;

inline int decode_pieces(int batch, int hkv) {
  const int groups = batch * hkv;
  if (groups <= 0) return 1;
  int p = (kDecodeTargetWaves + groups - 1) / groups;
  return p < 1 ? 1 : (p > kDecodeMaxPieces ? kDecodeMaxPieces : p);
}
inline size_t decode_workspace_bytes(int batch, int hq, int hkv) {
  return (size_t)batch * hq * decode_pieces(batch, hkv) * kPartialFloats * sizeof(float);
}

// Backward work split of the key side: key blocks are taken kpb at a time (a
// key unit); the (query head, query block) pairs that attend to the unit's
// first block j -- query blocks i in [lo, hi) with diagonal block qoffb + i >=
// j, in (query block, head) order -- are numbered per (batch, KV head) group
// in key-unit order, and the group's pairs are cut into `slots` contiguous
// ranges of equal length (floor(s * n / slots) .. floor((s+1) * n / slots) for
// n pairs), one per workgroup.  A range is walked P pairs at a time and gives
// one partial sum per key unit it touches (piece s + u of the group).  The
// unit's later blocks see a subset of its pairs (the rest lie wholly in their
// future).
struct BwdPlan {
  int lo, hi;     // query blocks handled
  int qoffb;      // q_offset / B (floor): query block i's diagonal key block is qoffb + i
  int P;          // pairs per step of the pair list
  int kpb;        // key blocks per key unit (1: block-sparse, 2: full)
  int slots;      // dK/dV workgroups per group (fewer when the group has fewer pairs)
  long long max_pairs;  // pairs of one group when every listed pair is present (bound)

  __host__ __device__ int first_block(int j) const { return j - qoffb > lo ? j - qoffb : lo; }
  __host__ __device__ int n_blocks(int j) const {
    const int n = hi - first_block(j);
    return n > 0 ? n : 0;
  }
  __host__ __device__ int n_units(int nkb) const { return (nkb + kpb - 1) / kpb; }
  // partial sums per group: one per (workgroup, key unit) piece, s + u < slots + units
  __host__ __device__ int n_pieces(int nkb) const { return slots + n_units(nkb); }
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;     // forward output, rows_out rows per (b, h)
  const uint16_t* dout;  // its gradient, same layout
  const float* lse;      // forward LSE (natural log), rows_out per (b, h)
  const int32_t* idx;    // sparse only
  int idx_shared;
  int full;
  uint16_t* dq;  // rows_out rows per (b, h)
  uint16_t* dk;  // [b, Hkv, seq_kv, d]
  uint16_t* dv;
  float* lse2;        // workspace: per-row LSE in log2 units, qb_count*B rows per (b, h)
  float* delta;       // workspace: per-row dO . O, same layout
  uint32_t* mask;     // workspace (sparse): [b*Hkv, nkb, nqb] head bits
  int* pairs;         // workspace (sparse): [b*Hkv, nkb] pairs per key block
  int* pair_base;     // workspace: [b*Hkv, nkb + 1] first pair of each key unit; [nku] = the group's pairs
  float* part;        // workspace: [b*Hkv, n_pieces][kpb][2][B][d] fp32 partial dK, dV
  int qb_begin, qb_count, rows_out;
  BwdPlan plan;
};

// Work plan and workspace layout of a backward call (byte offsets of lse2,
// delta, mask, pairs, pair_base, part; total bytes).
void bwd_plan(const Geometry& g, bool full, int qb_begin, int qb_count, BwdPlan* plan, size_t off[6],
              size_t* total);

hipError_t launch_block_summaries(const uint16_t* k, float* k_summary, const Geometry& g,
                                  hipStream_t stream);
hipError_t launch_learned_summaries(const uint16_t* k, const float* qbar, float* k_summary, const Geometry& g,
                                   hipStream_t stream);
hipError_t launch_entmax_route(const float* scores, float alpha, float gamma, float sigma, int32_t* idx,
                               float* bias, float* weights, const Geometry& g, hipStream_t stream);
hipError_t launch_prefill_scores(const uint16_t* q, const float* k_summary, float* scores,
                                 const Geometry& g, hipStream_t stream);
hipError_t launch_decode_scores(const uint16_t* q, const float* k_summary, float* scores,
                                const Geometry& g, hipStream_t stream);
// Fused decode scoring + selection: whether a shape fits (scores of a KV
// group held in LDS) and the launch.
bool decode_select_fits(const Geometry& g, bool shared);
hipError_t launch_decode_select(const uint16_t* q, const float* ksum, float* scores, int32_t* idx, const Geometry& g,
                                bool shared, hipStream_t stream);
hipError_t launch_select_topk(const float* scores, int32_t* idx, const Geometry& g, bool shared,
                              hipStream_t stream);
hipError_t launch_attn_prefill(const AttnArgs& a, bool full, const Geometry& g, hipStream_t stream);
hipError_t launch_attn_early_stop(const AttnArgs& a, const float* scores, float tau, int32_t* blocks_used,
                                  const Geometry& g, hipStream_t stream);
hipError_t launch_attn_backward(const BwdArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_attn_decode(const AttnArgs& a, float* workspace, const Geometry& g,
                              hipStream_t stream);

}  // namespace ssa
