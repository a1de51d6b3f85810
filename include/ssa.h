/*
 * ssa.h -- C ABI of libssa: causal block-sparse attention as used by SSA
 * (Sparse Sparse Attention), hand-written HIP kernels for AMD gfx950 (MI355X).
 *
 * The operations follow these pages:
 *   [SSA-summary] "Resumen Tecnico: SSA (Sparse Sparse Attention)" (gist.science 2511.20102)
 *   [SSA-guide]   "SSA: Guida a Sparse Sparse Attention per LLM" (mauroscia.it)
 *   [DashAttn]    "Resumen Tecnico: DashAttention" (gist.science 2605.18753)
 *   [S2O]         "Resumen Tecnico: S2O - Parada Temprana para Atencion Escasa mediante
 *                  Permutacion en Linea" (gist.science 2602.22575)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes.  b = batch, Hq / Hkv = query / key-value heads (Hq % Hkv == 0; query
 *   head h reads KV head h / (Hq/Hkv)), d = head_dim, B = block size,
 *   nqb = ceil(seq_q / B) query blocks, nkb = ceil(seq_kv / B) key blocks.
 * Positions.  Query row r sits at absolute position q_offset + r and sees keys
 *   c <= q_offset + r (causal).  seq_kv must equal q_offset + seq_q.  A
 *   multi-row query chunk must start on a block boundary (q_offset % B == 0);
 *   decode is seq_q == 1, q_offset == L - 1 (any L).  Query block i holds rows
 *   [i*B, (i+1)*B); its diagonal key block is (q_offset + i*B) / B.
 * Layouts.  Every tensor is dense, row-major, in the order written, with the
 *   last dimension contiguous.  Q [b,Hq,seq_q,d], K and V [b,Hkv,seq_kv,d] and
 *   attention outputs [b,Hq,rows,d] are bf16; summaries, scores, LSE and
 *   dropped mass are fp32; block indices are int32.  bf16 pointers must be
 *   16-byte aligned, fp32/int32 pointers 4-byte aligned.
 * Memory.  All pointers are device pointers owned by the caller (including
 *   any workspace).  The library allocates no device memory and keeps no
 *   mutable global state; concurrent calls on different streams are safe.
 * Streams.  Work is enqueued on `stream` and never synchronised; outputs are
 *   valid once the stream reaches that point.
 * Errors.  Arguments are validated on the host before anything is launched:
 *   SSA_ERR_INVALID_ARG (bad pointer, alignment, or inconsistent shape) or
 *   SSA_ERR_UNSUPPORTED (a valid shape the library does not implement: d != 64,
 *   B != 64, causal == 0, topk > 256, a negative scale).  A failed launch
 *   returns SSA_ERR_HIP.
 *   On error nothing is written.  ssa_last_error() gives a message for the
 *   calling thread's last failure.  Empty problems (batch == 0 or
 *   seq_q == 0) return SSA_OK without launching.
 * Determinism.  Identical inputs give bitwise-identical outputs (no
 *   floating-point atomics; fixed reduction orders).
 */
#ifndef SSA_H_
#define SSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssa_status {
  SSA_OK = 0,
  SSA_ERR_INVALID_ARG = 1,
  SSA_ERR_UNSUPPORTED = 2,
  SSA_ERR_HIP = 3,
  SSA_ERR_WORKSPACE = 4
} ssa_status_t;

typedef struct ssa_shape {
  int32_t batch;      /* b >= 0 */
  int32_t n_q_heads;  /* Hq >= 1 */
  int32_t n_kv_heads; /* Hkv >= 1, divides Hq */
  int32_t seq_q;      /* query rows per (b, h): N for prefill, 1 for decode */
  int32_t seq_kv;     /* key/value rows per (b, kv head); == q_offset + seq_q */
  int32_t q_offset;   /* absolute position of query row 0 */
  int32_t head_dim;   /* d; the library implements 64 */
  int32_t block;      /* B; the library implements 64 */
  int32_t topk;       /* k: blocks kept per query block, counting the forced diagonal
                         (most recent) block; 1 <= k <= 256 */
  int32_t causal;     /* must be 1 */
  float scale;        /* softmax and score scale, >= 0 (negative: SSA_ERR_UNSUPPORTED);
                         0 selects 1/sqrt(d) */
} ssa_shape_t;

typedef enum ssa_op {
  SSA_OP_BLOCK_SCORES = 0,
  SSA_OP_SELECT_TOPK = 1,
  SSA_OP_SPARSE_FWD = 2,
  SSA_OP_FULL_FWD = 3,
  SSA_OP_SPARSE_BWD = 4, /* ssa_block_sparse_attn_bwd and its _shared variant */
  SSA_OP_FULL_BWD = 5    /* ssa_full_attn_bwd (any query block range) */
} ssa_op_t;

/* Key-block summaries: k_summary[b,g,j,:] = fp32 rounding of the mean of the
 * rows of key block j that exist (c < seq_kv), summed exactly.
 * [SSA-guide] "Block-sparse attention e Receptive Field" (each contiguous
 * block is represented by its mean); [DashAttn] "Etapa 0" (a zero-initialised
 * learned chunk query is the uniform average; a finished chunk's summary is
 * cached and never recomputed -- this call is how a decode cache fills it).
 *   k          bf16 [b,Hkv,seq_kv,d]
 *   k_summary  fp32 [b,Hkv,nkb,d]  (output) */
ssa_status_t ssa_block_summaries(const ssa_shape_t* shape, const void* k, float* k_summary,
                                 hipStream_t stream);

/* Coarse block scores of each query block against the key-block summaries:
 *   scores[b,h,i,j] = fp32( scale * dot(qbar[b,h,i], kbar[b,h/G,j]) )  for j <= diag(i)
 *                   = -inf                                             for j >  diag(i)
 * where qbar is the fp32-rounded exact mean of the query rows of block i (the
 * row itself in decode) and kbar the key summaries; the dot product is
 * accumulated in fp64 from the fp32 summaries and rounded once.
 * [SSA-guide] "Block-sparse attention e Receptive Field" (query against the
 * mean representation of the preceding blocks); [DashAttn] "Etapa 1" (routing
 * logits of each query against the chunk summaries).
 *   q                  bf16 [b,Hq,seq_q,d]
 *   k                  bf16 [b,Hkv,seq_kv,d]; ignored (may be NULL) if summary_is_input
 *   k_summary          fp32 [b,Hkv,nkb,d]; written from k if summary_is_input == 0,
 *                      read (cached summaries) if summary_is_input != 0
 *   scores             fp32 [b,Hq,nqb,nkb] (output) */
ssa_status_t ssa_block_scores(const ssa_shape_t* shape, const void* q, const void* k,
                              float* k_summary, int summary_is_input, float* scores,
                              hipStream_t stream);

/* Top-k block selection per (b, h, query block i) with diagonal block
 * jd = diag(i) always kept: if jd + 1 <= topk every block 0..jd is kept,
 * otherwise jd plus the topk-1 earlier blocks ranked by (higher score, then
 * lower block index; NaN ranks below -inf).  Indices are written ascending
 * and padded with -1 to topk entries.
 * [SSA-guide] "Block-sparse attention e Receptive Field" (keep only the top-k
 * most relevant blocks, a fixed budget: receptive field = B * k tokens);
 * [DashAttn] "Declaracion del Problema" (fixed top-k budget) and "Etapa 2"
 * (near-diagonal chunks kept by a separate branch).
 *   scores     fp32 [b,Hq,nqb,nkb]
 *   block_idx  int32 [b,Hq,nqb,topk] (output) */
ssa_status_t ssa_select_topk(const ssa_shape_t* shape, const float* scores, int32_t* block_idx,
                             hipStream_t stream);

/* Block-sparse attention forward: query row r of block i attends to the keys
 * c <= q_offset + r whose block is listed in block_idx[b,h,i,:].  A row is
 * read as the set of blocks it names: entries in any order, -1 anywhere
 * skipped, entries outside [0, diag(i)] skipped, a block listed twice
 * attended once (ssa_select_topk writes them ascending and -1 padded):
 *   out[b,h,r,:] = sum_c softmax_c(scale * q_r . k_c) v_c   (bf16, fp32 accumulation)
 *   lse[b,h,r]   = natural log of sum_c exp(scale * q_r . k_c)  (fp32)
 * [SSA-summary] 2 "Mecanismo Central" (the sparse attention stream);
 * [SSA-guide] "Block-sparse attention e Receptive Field" (attention over the
 * tokens of the selected blocks only); [S2O] "Permutacion en Linea" (tiles
 * gathered by index from an unchanged HBM layout).
 * Workspace: ssa_workspace_bytes(shape, SSA_OP_SPARSE_FWD) bytes, 16-byte
 * aligned.
 *   decode (seq_q == 1): required (else SSA_ERR_WORKSPACE); the work is split
 *     over the key blocks of each KV-head group and the slices' partial
 *     results are merged through it.
 *   prefill: optional work queue.  With at least that many bytes, zero-filled
 *     before the first call, the launch is persistent (workgroups take further
 *     query blocks from the queue); every call leaves the queue zero again, so
 *     one buffer serves every later call, but calls sharing it must not
 *     overlap in time.  NULL or fewer bytes: one workgroup per query block.
 *     Bytes past the queue, if any, receive one timing record of 8 uint32 per
 *     workgroup of the launch (as many as fit): 100 MHz real-time counter at
 *     start and end (low 32 bits), shader cycles start to end, shader cycles
 *     in the tile loops, query blocks and tiles processed, hardware id, XCC id.
 *   q, k, v    bf16 as above;  block_idx int32 [b,Hq,nqb,topk]
 *   out        bf16 [b,Hq,seq_q,d] (output);  lse fp32 [b,Hq,seq_q] (output) */
ssa_status_t ssa_block_sparse_attn_fwd(const ssa_shape_t* shape, const void* q, const void* k,
                                       const void* v, const int32_t* block_idx, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Full causal attention (the counterpart output of the opposite mode) plus the
 * per-row dropped attention mass, for query blocks
 * [q_block_begin, q_block_begin + q_block_count) (rows past seq_q omitted):
 *   out_full[b,h,r',:]  full causal softmax attention of row r = q_block_begin*B + r'
 *   lse_full[b,h,r']    its natural-log log-sum-exp
 *   dropped_mass[b,h,r'] = sum over causal keys whose block is NOT in block_idx[b,h,i,:]
 *                          of the full-softmax probability (summed directly)
 * [SSA-summary] "Alineacion Bidireccional" (auxiliary output computed in the
 * opposite mode, used only for alignment) and 1 "Planteamiento del Problema"
 * (approximation error linear in the attention weight on unselected tokens).
 * Outputs hold rows_out = min(seq_q, (begin+count)*B) - begin*B rows per (b,h).
 * block_idx rows are read as sets, as in ssa_block_sparse_attn_fwd.
 * Workspace: optional work queue of ssa_workspace_bytes(shape,
 * SSA_OP_FULL_FWD) bytes, as for a prefill ssa_block_sparse_attn_fwd
 * (zero-filled before the first call, left zero by every call; NULL: one
 * workgroup per group of query heads and query block); bytes past the queue
 * receive the same per-workgroup timing records. */
ssa_status_t ssa_full_attn_fwd_dropped_mass(const ssa_shape_t* shape, const void* q, const void* k,
                                            const void* v, const int32_t* block_idx,
                                            int32_t q_block_begin, int32_t q_block_count,
                                            void* out_full, float* lse_full, float* dropped_mass,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/* Group-shared selection: one list per (b, KV head g, query block i) for all
 * the query heads of the group.  Candidate j is ranked by the group mean
 *   sbar[j] = fp32( (sum over h in group g, in head order, in fp64, of
 *                    scores[b,h,i,j]) / G )
 * with the same rule as ssa_select_topk (diagonal kept; higher score, then
 * lower index; NaN below -inf; ascending, -1 padded).
 * [DashAttn] "Etapa 1" (with grouped-query attention the routing of the
 * query heads that share a KV head is averaged into one shared support).
 *   scores     fp32 [b,Hq,nqb,nkb]
 *   block_idx  int32 [b,Hkv,nqb,topk] (output) */
ssa_status_t ssa_select_topk_shared(const ssa_shape_t* shape, const float* scores, int32_t* block_idx,
                                    hipStream_t stream);

/* Decode (seq_q == 1) scoring and selection in one launch: the block scores
 * of every query head against the cached key summaries, exactly as
 * ssa_block_scores with summary_is_input = 1, and the top-k selection with the
 * most recent block kept, exactly as ssa_select_topk (shared == 0) or
 * ssa_select_topk_shared (shared != 0).  Results are identical to those two
 * calls; the scores stay on chip and the second launch is saved.
 * [SSA-guide] "Block-sparse attention e Receptive Field"; [DashAttn] "Etapa 0"
 * (cached chunk summaries), "Etapa 1" (routing logits, averaged over the
 * query heads of a KV head when shared) and "Etapa 2" (most recent chunk kept).
 *   q          bf16 [b,Hq,1,d];  k_summary fp32 [b,Hkv,nkb,d] (input)
 *   scores     fp32 [b,Hq,1,nkb] (output, may be NULL)
 *   block_idx  int32 [b,Hq,1,topk], or [b,Hkv,1,topk] when shared (output)
 * The scores of one KV group are held in 64 KB of LDS: (Hq/Hkv) * nkb (plus
 * nkb when shared) fp32 values, with at most 32 query heads per KV head;
 * larger shapes return SSA_ERR_UNSUPPORTED (the two calls cover them).
 * seq_q != 1 returns SSA_ERR_INVALID_ARG. */
ssa_status_t ssa_decode_scores_select(const ssa_shape_t* shape, const void* q, const float* k_summary,
                                      float* scores, int32_t* block_idx, int32_t shared, hipStream_t stream);

/* ssa_block_sparse_attn_fwd with a group-shared selection: query head h
 * attends over the list block_idx[b, h/G, i, :] (int32 [b,Hkv,nqb,topk], as
 * written by ssa_select_topk_shared); same outputs, workspace and errors. */
ssa_status_t ssa_block_sparse_attn_fwd_shared(const ssa_shape_t* shape, const void* q, const void* k,
                                              const void* v, const int32_t* block_idx, void* out,
                                              float* lse, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream);

/* ssa_full_attn_fwd_dropped_mass with a group-shared selection: the dropped
 * mass of query head h counts the keys whose block is not in
 * block_idx[b, h/G, i, :] (int32 [b,Hkv,nqb,topk]); same outputs and errors. */
ssa_status_t ssa_full_attn_fwd_dropped_mass_shared(const ssa_shape_t* shape, const void* q, const void* k,
                                                   const void* v, const int32_t* block_idx,
                                                   int32_t q_block_begin, int32_t q_block_count,
                                                   void* out_full, float* lse_full, float* dropped_mass,
                                                   void* workspace, size_t workspace_bytes,
                                                   hipStream_t stream);

/* Block-sparse attention forward with early stopping over the selected
 * blocks.  Query block i visits the blocks of block_idx[b,h,i,:] in
 * decreasing estimated importance: its diagonal block first, then the others
 * by scores[b,h,i,j] (higher first, lower index on ties, NaN last).  After
 * each block past the first, if every row r of the block (r < seq_q) has
 *   gain_r < tau * before_r,
 * where gain_r is the softmax mass (sum of exp(scale * q_r . k_c) over the
 * block's keys c <= q_offset + r) and before_r the same mass over the blocks
 * visited before it, the block is kept and the remaining ones are skipped.
 * Rows then attend over the keys of the visited blocks (out, lse as in
 * ssa_block_sparse_attn_fwd) and blocks_used[b,h,i] counts them.  tau = 0
 * never stops; larger tau stops sooner.  The decision is taken in fp32.
 * [S2O] "Regla de Parada Temprana" (stop once the marginal gain in attention
 * mass of a processed block falls below a threshold relative to the
 * accumulated mass; blocks processed in descending estimated importance) and
 * "Implementacion del Kernel" (the query's own segment first).
 *   scores       fp32 [b,Hq,nqb,nkb] (as written by ssa_block_scores)
 *   block_idx    int32 [b,Hq,nqb,topk] (as written by ssa_select_topk)
 *   tau          >= 0 (else SSA_ERR_INVALID_ARG)
 *   out, lse     as ssa_block_sparse_attn_fwd;  blocks_used int32 [b,Hq,nqb] (output)
 * No workspace is needed (workspace may be NULL). */
ssa_status_t ssa_block_sparse_attn_fwd_early_stop(const ssa_shape_t* shape, const void* q, const void* k,
                                                  const void* v, const float* scores, const int32_t* block_idx,
                                                  float tau, void* out, float* lse, int32_t* blocks_used,
                                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and results as ssa_block_sparse_attn_fwd, with the
 * workspace taken from a static array of the library instead of an argument.
 * The call allocates nothing.  The array holds 8 MiB + 1 KiB per GPU, from
 * the first call on that GPU until the process ends:
 *   decode (seq_q == 1): batch * n_q_heads * slices * 264 bytes of partials,
 *     at most 8 MiB (64 sequences x 32 query heads on 2 KV heads use 4.3 MB);
 *     a larger shape fails with SSA_ERR_WORKSPACE and launches nothing.
 *   prefill: the 1 KiB work queue of the persistent launch.
 * The first call on a GPU looks the array up and enqueues one clearing of
 * the queue on `stream` (repeated on later calls while it has only been
 * captured into a graph).  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU, from any stream or graph, race and
 * give wrong results; calls ordered one after another are safe. */
ssa_status_t ssa_block_sparse_attn_fwd_noalloc(const ssa_shape_t* shape, const void* q, const void* k,
                                               const void* v, const int32_t* block_idx, void* out, float* lse,
                                               hipStream_t stream);

/* Backward of the block-sparse forward: for the scalar L = sum(dout * out),
 * with P = exp(scale * q_r . k_c - lse_r) on the keys c that row r attends to
 * in ssa_block_sparse_attn_fwd (block_idx as there) and D_r = dout_r . out_r,
 *   dv[b,g,c,:] = sum over rows r of heads in group g of P_rc dout_r
 *   dk[b,g,c,:] = scale * sum_r dS_rc q_r,  dq[b,h,r,:] = scale * sum_c dS_rc k_c,
 *   dS_rc = P_rc (dout_r . v_c - D_r)
 * (keys outside a row's blocks get nothing from it); fp32 accumulation, bf16
 * outputs.  out and lse must be what the forward wrote for these inputs.
 * [SSA-summary] 1 "Planteamiento del Problema" (the sparse stream gives
 * unselected tokens zero gradient and normalises over the selected subset
 * only) and 2 "Mecanismo Central" (the sparse stream is trained directly).
 *   q, k, v, block_idx, out, lse  as ssa_block_sparse_attn_fwd (inputs)
 *   dout  bf16 [b,Hq,seq_q,d];  dq bf16 [b,Hq,seq_q,d] (output)
 *   dk, dv  bf16 [b,Hkv,seq_kv,d] (outputs; every row written, zero for keys
 *           no row attends to)
 *   workspace  >= ssa_workspace_bytes(shape, SSA_OP_SPARSE_BWD) bytes,
 *              256-byte aligned (else SSA_ERR_WORKSPACE / SSA_ERR_INVALID_ARG)
 * More than 32 query heads per KV head, or more than 2^31 - 1 listed
 * (query head, query block, key block) pairs in one KV group:
 * SSA_ERR_UNSUPPORTED.  Results are bitwise reproducible (no atomics on
 * gradients; the work split depends only on the listed pairs). */
ssa_status_t ssa_block_sparse_attn_bwd(const ssa_shape_t* shape, const void* q, const void* k, const void* v,
                                       const int32_t* block_idx, const void* out, const float* lse,
                                       const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* ssa_block_sparse_attn_bwd for a group-shared selection (block_idx int32
 * [b,Hkv,nqb,topk] as for ssa_block_sparse_attn_fwd_shared); same outputs,
 * workspace and errors. */
ssa_status_t ssa_block_sparse_attn_bwd_shared(const ssa_shape_t* shape, const void* q, const void* k,
                                              const void* v, const int32_t* block_idx, const void* out,
                                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward of the full causal counterpart on query blocks
 * [q_block_begin, q_block_begin + q_block_count): the gradients of
 * L = sum(dout_full * out_full) over those rows (P over every key c <= the
 * row's position; otherwise as ssa_block_sparse_attn_bwd).
 * [SSA-summary] 2 "Mecanismo Central" (the full stream passes gradient to
 * every token) and "Alineacion Bidireccional" (the counterpart output is
 * trained through the alignment objective).
 *   out_full, lse_full  as written by ssa_full_attn_fwd_dropped_mass for the same range
 *   dout_full, dq  bf16 [b,Hq,rows_out,d] (rows_out as for the forward)
 *   dk, dv  bf16 [b,Hkv,seq_kv,d] (outputs; every row written)
 *   workspace  >= ssa_workspace_bytes(shape, SSA_OP_FULL_BWD) bytes, 256-byte aligned
 * An empty range (q_block_count == 0) writes nothing. */
ssa_status_t ssa_full_attn_bwd(const ssa_shape_t* shape, const void* q, const void* k, const void* v,
                               int32_t q_block_begin, int32_t q_block_count, const void* out_full,
                               const float* lse_full, const void* dout_full, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Chunk summaries from a learned query: for KV head g and key block j,
 *   k_summary[b,g,j,:] = fp32 rounding of sum_c softmax_c(scale * qbar[g] . k_c) k_c
 * over the rows c < seq_kv of block j (computed in fp64).  qbar == 0 gives the
 * plain mean of ssa_block_summaries.  Feed the result to ssa_block_scores
 * with summary_is_input = 1.
 * [DashAttn] "Etapa 0" (a learned query attends to each chunk's keys by local
 * scaled dot-product attention; zero-initialised it is the uniform average;
 * a finished chunk's summary is cached).
 *   k          bf16 [b,Hkv,seq_kv,d]
 *   qbar       fp32 [Hkv,d] (one learned query per KV head)
 *   k_summary  fp32 [b,Hkv,nkb,d]  (output) */
ssa_status_t ssa_block_summaries_learned(const ssa_shape_t* shape, const void* k, const float* qbar,
                                         float* k_summary, hipStream_t stream);

/* alpha-entmax routing with a group-shared support.  For each (b, KV head g,
 * query block i) and each query head h of the group,
 *   w_h = alpha-entmax(gamma * scores[b,h,i,j]) over j < diag(i),
 *   alpha-entmax(z)_j = max(0, (alpha-1) z_j - tau)^(1/(alpha-1)), tau such that sum_j = 1,
 * and the group's weights are wbar = mean_h w_h (fp32; tau by Newton
 * iterations from below in fp32).  block_idx lists diag(i) plus every j with wbar_j > 0 -- past topk
 * blocks, the topk-1 largest wbar (lower index on ties) -- ascending, -1
 * padded; block_bias holds sigma * ln(wbar_j) for each listed j != diag(i)
 * and 0 for diag(i) and padding.  Non-finite scores take no weight.
 * [DashAttn] "Etapa 1" (entmax routing instead of a fixed top-k: the support
 * size follows from the scores; with GQA the probabilities of the heads
 * sharing a KV head are averaged into one support) and "Etapa 2" (the
 * routing weights become a prior on the token softmax, zero where they are
 * zero, of strength sigma; near-diagonal chunks have their own branch).
 *   scores      fp32 [b,Hq,nqb,nkb] (ssa_block_scores)
 *   alpha       in (1, 2] (NaN: SSA_ERR_INVALID_ARG; otherwise outside: SSA_ERR_UNSUPPORTED)
 *   gamma, sigma  finite, >= 0 (else SSA_ERR_INVALID_ARG)
 *   block_idx   int32 [b,Hkv,nqb,topk] (output);  block_bias fp32 [b,Hkv,nqb,topk] (output)
 *   weights     fp32 [b,Hkv,nqb,nkb] (optional output, NULL to skip: wbar, 0 from diag(i) on)
 * More than 1024 key blocks (65536 keys): SSA_ERR_UNSUPPORTED. */
ssa_status_t ssa_entmax_route(const ssa_shape_t* shape, const float* scores, float alpha, float gamma, float sigma,
                              int32_t* block_idx, float* block_bias, float* weights, hipStream_t stream);

/* Block-sparse attention forward with a per-block logit bias and a
 * group-shared selection: row r of query head h, query block i attends to the
 * keys c <= q_offset + r of the blocks listed in block_idx[b, h/G, i, :], with
 * logits scale * q_r . k_c + block_bias[b, h/G, i, e] for c in the e-th listed
 * block (out, lse as ssa_block_sparse_attn_fwd; lse includes the bias).  With
 * the output of ssa_entmax_route this is the softmax taken relative to the
 * prior g proportional to wbar^sigma.  A block whose bias is -inf (prior
 * weight 0) contributes nothing; a row whose every listed block has bias -inf
 * has an empty support and gets NaN in out and lse.  A block listed twice
 * takes the bias of its first listing.
 * [DashAttn] "Etapa 2" (prior-induced sparse softmax: a FlashAttention-style
 * loop over the active chunks adding the routing bias to the logits).
 *   block_idx   int32 [b,Hkv,nqb,topk];  block_bias fp32 [b,Hkv,nqb,topk]
 * Decode (seq_q == 1) needs ssa_workspace_bytes(shape, SSA_OP_SPARSE_FWD)
 * bytes of workspace, as ssa_block_sparse_attn_fwd; prefill needs none. */
ssa_status_t ssa_block_sparse_attn_fwd_biased(const ssa_shape_t* shape, const void* q, const void* k,
                                              const void* v, const int32_t* block_idx, const float* block_bias,
                                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream);

/* Workspace bytes an entry point needs for this shape (0 if none; SIZE_MAX if
 * the shape is invalid). */
size_t ssa_workspace_bytes(const ssa_shape_t* shape, ssa_op_t op);

/* Static description of a status code. */
const char* ssa_status_string(ssa_status_t status);

/* Message describing the calling thread's most recent failure ("" if none). */
const char* ssa_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t ssa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H_ */
