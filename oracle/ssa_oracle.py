"""Plain, slow fp64 CPU oracle for causal block-sparse attention as used by SSA.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing).

Sources (titles of the web pages the method is described on):
  [SSA-summary]  "Resumen Tecnico: SSA (Sparse Sparse Attention)", gist.science 2511.20102
  [SSA-guide]    "SSA: Guida a Sparse Sparse Attention per LLM", mauroscia.it
  [DashAttn]     "Resumen Tecnico: DashAttention", gist.science 2605.18753
  [S2O]          "Resumen Tecnico: S2O - Parada Temprana para Atencion Escasa ...", gist.science 2602.22575

What is computed (all arithmetic in float64 unless a step says it rounds):
  1. block means of K (and of the queries of each query block)      [SSA-guide] "Block-sparse attention e Receptive Field";
                                                                     [DashAttn] "Etapa 0" (zero-initialised learned
                                                                     query == uniform average over the chunk)
  2. coarse block scores  s = scale * qbar . kbar  for causal blocks [SSA-guide] same section; [DashAttn] "Etapa 1"
  3. top-k block selection per query block, diagonal always kept    [SSA-guide] same section; [DashAttn] "Etapa 2"
                                                                     (separate branch for near-diagonal chunks)
  3'. optional group-shared selection: one list per KV group from the
     mean of its query heads' block scores                          [DashAttn] "Etapa 1" (GQA: routing averaged
                                                                     over the heads sharing a KV head)
  4. softmax attention restricted to the selected blocks            [SSA-summary] 2 "Mecanismo Central" (SA stream)
  5. full causal softmax attention (the counterpart output)         [SSA-summary] "Alineacion Bidireccional"
  4'. optional early stopping: selected blocks visited in decreasing
     estimated importance, stopping once a block's marginal mass gain
     falls below a threshold relative to the accumulated mass       [S2O] "Regla de Parada Temprana"
  6. dropped attention mass: full-softmax probability on keys the
     sparse pattern leaves out                                      [SSA-summary] 1 "Planteamiento del Problema",
                                                                     "Alineacion Bidireccional" (delta(t))
  3''. optional DashAttention stages: chunk summaries from a learned
     query, alpha-entmax routing averaged over a KV group, and softmax
     with a prior bias sigma * ln(w) over the routed blocks           [DashAttn] "Etapa 0", "Etapa 1", "Etapa 2"
  7. gradients of steps 4 and 5 with respect to Q, K, V for a given
     output gradient (chain rule through the masked softmax)       [SSA-summary] 1 "Planteamiento del Problema"
                                                                     (dropped keys get no gradient in the sparse
                                                                     stream), 2 "Mecanismo Central" (the full
                                                                     stream reaches every token)

Readings where the pages leave a step open:
  * selection is per query block (block-mean query), per query head; the
    budget ``topk`` counts the forced diagonal block;
  * group-shared selection (one list per KV group) ranks blocks by the mean
    of the group's per-head block scores;
  * early stopping visits the diagonal block first, then the other selected
    blocks by coarse score; a query block stops after the first block whose
    gain is below tau times the accumulated mass for all of its rows (that
    block is kept);
  * DashAttention routing is per query block (block-mean query scores, as
    in step 2), over the blocks before the diagonal; the diagonal block is
    always kept with bias 0; the prior is g proportional to w ** sigma, i.e.
    a logit bias sigma * ln(w); the list is capped at ``topk`` blocks by
    weight (diagonal kept);
  * the backward takes the output gradient as given (the alignment losses
    that would produce it have no stated functional form); only O carries
    gradient (not LSE or the dropped mass);
  * summaries are held in fp32 and scores are rounded to fp32 before the
    top-k decision (the decision is taken in the precision the scores are
    stored in, on both sides);
  * ties order by lower block index first; a NaN score ranks below -inf;
  * with fewer than ``topk`` causal blocks, all of them are selected;
  * softmax scale 1/sqrt(d) unless given; logs are natural logs;
  * query row r (0-based within the query tensor) sits at absolute position
    ``q_offset + r`` and sees keys c <= q_offset + r; query block i holds rows
    [i*B, (i+1)*B) and its diagonal key block is (q_offset + i*B) // B.
    Decode is the case seq_q == 1, q_offset == L-1.

Arrays: Q [b, Hq, seq_q, d], K/V [b, Hkv, seq_kv, d] (any float dtype whose
values are exactly the bf16 inputs), query head h uses KV head h // (Hq/Hkv).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------- helpers

def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even) and return
    them as float64 again."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def n_blocks(n: int, block: int) -> int:
    return -(-n // block)


def diag_block(i: int, q_offset: int, block: int) -> int:
    """Key block holding the first row of query block i."""
    return (q_offset + i * block) // block


def _check_geometry(seq_q: int, seq_kv: int, q_offset: int, block: int):
    if seq_kv != q_offset + seq_q:
        raise ValueError("causal layout requires seq_kv == q_offset + seq_q")
    if seq_q > 1 and q_offset % block != 0:
        raise ValueError("a multi-row query chunk must start on a block boundary")


# --------------------------------------------------------------------------- step 1: summaries

def block_means(x, block: int) -> np.ndarray:
    """Mean of the rows of each contiguous block of ``block`` rows (the last,
    possibly partial, block averages the rows it has).

    x: [..., n, d]  ->  [..., ceil(n/block), d], float64 (exact sums, one division).
    [SSA-guide] "Block-sparse attention e Receptive Field": the sequence is cut
    into contiguous blocks and each is represented by its mean."""
    x = _f64(x)
    n = x.shape[-2]
    nb = n_blocks(n, block)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]), dtype=np.float64)
    for j in range(nb):
        rows = x[..., j * block: min((j + 1) * block, n), :]
        out[..., j, :] = rows.sum(axis=-2) / rows.shape[-2]
    return out


def key_summaries(k, block: int) -> np.ndarray:
    """Stored key-block summaries: block means rounded to fp32 (float64 array)."""
    return round_f32(block_means(k, block))


def query_summaries(q, block: int) -> np.ndarray:
    """Query-block summaries: block means of the query rows, rounded to fp32."""
    return round_f32(block_means(q, block))


# --------------------------------------------------------------------------- step 2: scores

def block_scores(q, k, block: int, scale: Optional[float] = None, q_offset: int = 0,
                 k_summary=None) -> np.ndarray:
    """Coarse block scores s[b,h,i,j] = fp32(scale * qbar[b,h,i] . kbar[b,g(h),j])
    for key blocks j up to the diagonal block of query block i, -inf beyond it.

    [SSA-guide] "Block-sparse attention e Receptive Field" (query vs block mean
    representations); [DashAttn] "Etapa 1" (logits of each query against the
    chunk summaries).  ``k_summary`` (fp32 values) replaces the pooled K when
    summaries were cached once their block completed ([DashAttn] "Etapa 0")."""
    q = _f64(q)
    b, hq, seq_q, d = q.shape
    if k_summary is None:
        kbar = key_summaries(k, block)
        seq_kv = _f64(k).shape[-2]
    else:
        kbar = round_f32(k_summary)
        seq_kv = q_offset + seq_q
    hkv = kbar.shape[1]
    group = hq // hkv
    _check_geometry(seq_q, seq_kv, q_offset, block)
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    qbar = query_summaries(q, block)
    nqb, nkb = qbar.shape[2], kbar.shape[2]
    s = np.full((b, hq, nqb, nkb), -np.inf, dtype=np.float64)
    for bi in range(b):
        for h in range(hq):
            g = h // group
            dots = qbar[bi, h] @ kbar[bi, g].T           # [nqb, nkb]
            for i in range(nqb):
                jd = diag_block(i, q_offset, block)
                s[bi, h, i, : jd + 1] = round_f32(scale * dots[i, : jd + 1])
    return s


# --------------------------------------------------------------------------- step 3: selection

def _rank_key(score: float, j: int):
    """Sort key: larger score first, then smaller block index; NaN below -inf."""
    if math.isnan(score):
        return (1, 0.0, j)
    return (0, -score, j)


def select_blocks(scores, topk: int, block: int, q_offset: int = 0) -> np.ndarray:
    """Selected key blocks per (b, h, query block): the diagonal block plus the
    ``topk - 1`` best-scoring earlier blocks (all causal blocks when there are
    at most ``topk``), listed in ascending order and padded with -1.

    [SSA-guide] "Block-sparse attention e Receptive Field" (keep only the top-k
    most relevant blocks); [DashAttn] "Etapa 2" (near-diagonal chunks handled
    by their own branch).  Returns int64 [b, Hq, nqb, topk]."""
    scores = _f64(scores)
    b, hq, nqb, _ = scores.shape
    out = np.full((b, hq, nqb, topk), -1, dtype=np.int64)
    for bi in range(b):
        for h in range(hq):
            for i in range(nqb):
                jd = diag_block(i, q_offset, block)
                if jd + 1 <= topk:
                    chosen = list(range(jd + 1))
                else:
                    ranked = sorted(range(jd), key=lambda j: _rank_key(scores[bi, h, i, j], j))
                    chosen = sorted(ranked[: topk - 1] + [jd])
                out[bi, h, i, : len(chosen)] = chosen
    return out


# --------------------------------------------------------------------------- group-shared selection

def shared_block_scores(scores, n_kv_heads: int) -> np.ndarray:
    """Block scores shared by the query heads of each KV group: the mean of the
    group's per-head block scores (summed in head order in float64, divided by
    the group size, rounded to fp32); -inf where the heads have -inf.

    [DashAttn] "Etapa 1" (with grouped-query attention, the routing of the
    query heads that share a KV head is averaged into one shared selection).
    Returns float64 [b, Hkv, nqb, nkb]."""
    s = _f64(scores)
    b, hq, nqb, nkb = s.shape
    group = hq // n_kv_heads
    out = np.empty((b, n_kv_heads, nqb, nkb))
    for g in range(n_kv_heads):
        acc = np.zeros((b, nqb, nkb))
        for hh in range(group):
            acc = acc + s[:, g * group + hh]
        out[:, g] = round_f32(acc / group)
    return out


def select_blocks_shared(scores, n_kv_heads: int, topk: int, block: int, q_offset: int = 0) -> np.ndarray:
    """Group-shared selection: the selection rule of select_blocks applied to
    shared_block_scores, one list per (b, KV head, query block).
    Returns int64 [b, Hkv, nqb, topk]."""
    return select_blocks(shared_block_scores(scores, n_kv_heads), topk, block, q_offset)


def expand_shared(sel_shared, n_q_heads: int) -> np.ndarray:
    """Per-query-head view of a group-shared selection (query head h uses the
    list of its KV head h // G), for sparse_attention and
    full_attention_dropped_mass."""
    sel_shared = np.asarray(sel_shared)
    return np.repeat(sel_shared, n_q_heads // sel_shared.shape[1], axis=1)


# --------------------------------------------------------------------------- steps 4-6: attention

def _row_attention(qrow, keys, vals, scale):
    """Softmax attention of one query row over the given keys (float64).
    Returns (output [d], lse, logits [n])."""
    logits = scale * (keys @ qrow)
    m = logits.max()
    w = np.exp(logits - m)
    z = w.sum()
    return (w @ vals) / z, m + math.log(z), logits


def _listed_blocks(sel_row):
    """(position, block) of each block an index row names: its non-negative
    entries, a block listed twice taken at its first listing.  The selection
    is a set of blocks ([SSA-guide] "Block-sparse attention e Receptive
    Field": the chosen blocks), so order and repetition carry no meaning."""
    seen, out = set(), []
    for e, j in enumerate(sel_row):
        j = int(j)
        if j >= 0 and j not in seen:
            seen.add(j)
            out.append((e, j))
    return out


def _allowed_keys(sel_row, pos: int, block: int, seq_kv: int) -> np.ndarray:
    """Key positions c <= pos whose block is in the selected set."""
    cols = []
    for _, j in _listed_blocks(sel_row):
        lo, hi = j * block, min((j + 1) * block, seq_kv, pos + 1)
        if lo < hi:
            cols.append(np.arange(lo, hi))
    return np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)


def sparse_attention(q, k, v, sel, block: int, scale: Optional[float] = None, q_offset: int = 0,
                     rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Block-sparse attention: row r of query block i attends to keys c <= its
    position whose block is selected for (b, h, i).
    [SSA-summary] 2 "Mecanismo Central" (SA stream); [SSA-guide]
    "Block-sparse attention e Receptive Field" (attention only over the tokens
    inside the chosen blocks).

    Returns (O [b,Hq,seq_q,d], LSE [b,Hq,seq_q]) or, when ``rows`` lists
    (b, h, r) triples, (O [n,d], LSE [n]) for just those rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    group = hq // hkv
    _check_geometry(seq_q, seq_kv, q_offset, block)
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))

    def one(bi, h, r):
        g = h // group
        cols = _allowed_keys(sel[bi, h, r // block], q_offset + r, block, seq_kv)
        o, lse, _ = _row_attention(q[bi, h, r], k[bi, g, cols], v[bi, g, cols], scale)
        return o, lse

    if rows is not None:
        res = [one(*t) for t in rows]
        return np.stack([o for o, _ in res]), np.array([l for _, l in res])
    out = np.empty((b, hq, seq_q, d))
    lse = np.empty((b, hq, seq_q))
    for bi in range(b):
        for h in range(hq):
            g = h // group
            for i in range(n_blocks(seq_q, block)):
                r0, r1 = i * block, min((i + 1) * block, seq_q)
                # key columns of the selected blocks, up to the last row's position
                cols = _allowed_keys(sel[bi, h, i], q_offset + r1 - 1, block, seq_kv)
                logits = scale * (q[bi, h, r0:r1] @ k[bi, g, cols].T)
                pos = q_offset + np.arange(r0, r1)
                logits[cols[None, :] > pos[:, None]] = -np.inf          # causal
                m = logits.max(axis=1, keepdims=True)
                w = np.exp(logits - m)
                z = w.sum(axis=1, keepdims=True)
                out[bi, h, r0:r1] = (w @ v[bi, g, cols]) / z
                lse[bi, h, r0:r1] = (m + np.log(z))[:, 0]
    return out, lse


def full_attention_dropped_mass(q, k, v, sel, block: int, scale: Optional[float] = None,
                                q_offset: int = 0, row_range: Optional[Tuple[int, int]] = None,
                                rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Full causal attention (the counterpart output) and the dropped mass
        delta_r = sum over keys c <= pos(r) whose block is NOT selected for r's
                  query block of  exp(logit_rc - LSE_full[r]),
    i.e. the full-softmax probability that the sparse pattern leaves out,
    summed directly.
    [SSA-summary] "Alineacion Bidireccional" (auxiliary output in the opposite
    mode; delta(t)) and 1 "Planteamiento del Problema" (approximation error
    linear in the attention weight on unselected tokens).

    ``row_range`` = (lo, hi) restricts to query rows [lo, hi) (lo, hi multiples
    of the block size or hi == seq_q).  Returns (O, LSE, delta) over those rows,
    or per listed (b, h, r) triple when ``rows`` is given."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    group = hq // hkv
    _check_geometry(seq_q, seq_kv, q_offset, block)
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))

    def one(bi, h, r):
        g = h // group
        pos = q_offset + r
        o, lse, logits = _row_attention(q[bi, h, r], k[bi, g, : pos + 1], v[bi, g, : pos + 1], scale)
        keep = np.zeros(pos + 1, dtype=bool)
        keep[_allowed_keys(sel[bi, h, r // block], pos, block, seq_kv)] = True
        delta = np.exp(logits[~keep] - lse).sum()
        return o, lse, delta

    if rows is not None:
        res = [one(*t) for t in rows]
        return (np.stack([t[0] for t in res]), np.array([t[1] for t in res]),
                np.array([t[2] for t in res]))
    lo, hi = (0, seq_q) if row_range is None else row_range
    out = np.empty((b, hq, hi - lo, d))
    lse = np.empty((b, hq, hi - lo))
    delta = np.empty((b, hq, hi - lo))
    for bi in range(b):
        for h in range(hq):
            g = h // group
            for i in range(lo // block, n_blocks(hi, block)):
                r0, r1 = max(i * block, lo), min((i + 1) * block, hi)
                last = q_offset + r1 - 1
                logits = scale * (q[bi, h, r0:r1] @ k[bi, g, : last + 1].T)
                pos = q_offset + np.arange(r0, r1)
                cols = np.arange(last + 1)
                future = cols[None, :] > pos[:, None]
                logits[future] = -np.inf
                m = logits.max(axis=1, keepdims=True)
                w = np.exp(logits - m)
                z = w.sum(axis=1, keepdims=True)
                out[bi, h, r0 - lo:r1 - lo] = (w @ v[bi, g, : last + 1]) / z
                row_lse = m + np.log(z)
                lse[bi, h, r0 - lo:r1 - lo] = row_lse[:, 0]
                selected = np.zeros(last + 1, dtype=bool)
                selected[_allowed_keys(sel[bi, h, i], last, block, seq_kv)] = True
                dropped = (~selected)[None, :] & ~future
                delta[bi, h, r0 - lo:r1 - lo] = np.where(dropped, np.exp(logits - row_lse), 0.0).sum(axis=1)
    return out, lse, delta


# --------------------------------------------------------------------------- DashAttention stages

def learned_key_summaries(k, qbar, block: int, scale: Optional[float] = None) -> np.ndarray:
    """Chunk summaries from a learned query: for KV head g and chunk j, the
    softmax-weighted average of the chunk's key rows,
        kbar[b,g,j] = sum_c softmax_c(scale * qbar[g] . k_c) k_c   (rows c < seq_kv of chunk j),
    rounded to fp32.  qbar == 0 gives the plain block mean (step 1).
    [DashAttn] "Etapa 0" (a learned query attends to the keys of each chunk by
    local scaled dot-product attention; zero-initialised it is the uniform
    average; a finished chunk's summary is cached).
    qbar: [Hkv, d].  Returns float64 [b, Hkv, nkb, d]."""
    k, qbar = _f64(k), _f64(qbar)
    b, hkv, n, d = k.shape
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    nb = n_blocks(n, block)
    out = np.empty((b, hkv, nb, d))
    for bi in range(b):
        for g in range(hkv):
            for j in range(nb):
                rows = k[bi, g, j * block: min((j + 1) * block, n)]
                logits = scale * (rows @ qbar[g])
                w = np.exp(logits - logits.max())
                out[bi, g, j] = (w / w.sum()) @ rows
    return round_f32(out)


def entmax(z, alpha: float) -> np.ndarray:
    """alpha-entmax of a score vector (1 < alpha <= 2):
        p_j = max(0, (alpha - 1) z_j - tau) ** (1 / (alpha - 1)),
    with the threshold tau fixed by sum_j p_j = 1 (-inf scores get 0).  The sum
    decreases in tau, and tau lies in [max - 1, max - n**(1 - alpha)] for the
    scaled scores, so it is found by bisection in float64; the result is then
    normalised.  alpha = 2 is sparsemax; alpha -> 1 tends to softmax.
    [DashAttn] "Etapa 1" (routing by alpha-entmax: a sparse probability vector
    whose support size follows from the scores)."""
    z = _f64(z)
    if not 1.0 < alpha <= 2.0:
        raise ValueError("alpha must be in (1, 2]")
    out = np.zeros_like(z)
    fin = np.isfinite(z)
    if not fin.any():
        return out
    zt = (alpha - 1.0) * z[fin]
    inv = 1.0 / (alpha - 1.0)
    lo, hi = zt.max() - 1.0, zt.max() - len(zt) ** (1.0 - alpha)

    def total(tau):
        return (np.maximum(zt - tau, 0.0) ** inv).sum()

    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if total(mid) >= 1.0:
            lo = mid
        else:
            hi = mid
    p = np.maximum(zt - lo, 0.0) ** inv
    out[fin] = p / p.sum()
    return out


def entmax_routing(scores, n_kv_heads: int, alpha: float, gamma: float, block: int,
                   q_offset: int = 0) -> np.ndarray:
    """Routing weights of each (b, KV head g, query block i): for every query
    head h of the group, w_h = alpha-entmax(gamma * scores[b,h,i,j]) over the
    earlier blocks j < diag(i); the group's weights are the mean of its heads'.
    The diagonal block is not routed (it has its own branch).
    [DashAttn] "Etapa 1" (entmax routing of the chunk logits; with GQA the
    probabilities of the heads sharing a KV head are averaged into one sparse
    support) and "Etapa 2" (near-diagonal chunks kept apart).
    Returns float64 [b, Hkv, nqb, nkb] (0 outside the support and from the
    diagonal on)."""
    s = _f64(scores)
    b, hq, nqb, nkb = s.shape
    group = hq // n_kv_heads
    out = np.zeros((b, n_kv_heads, nqb, nkb))
    for bi in range(b):
        for g in range(n_kv_heads):
            for i in range(nqb):
                jd = diag_block(i, q_offset, block)
                if jd == 0:
                    continue
                acc = np.zeros(jd)
                for hh in range(group):
                    acc = acc + entmax(gamma * s[bi, g * group + hh, i, :jd], alpha)
                out[bi, g, i, :jd] = acc / group
    return out


def routing_support(weights, topk: int, block: int, q_offset: int = 0) -> np.ndarray:
    """Block lists from routing weights: the diagonal block plus every earlier
    block of positive weight; past ``topk`` blocks, the diagonal plus the
    topk - 1 largest weights (lower index on ties).  Ascending, -1 padded.
    [DashAttn] "Etapa 2" (attention restricted to the chunks the routing
    selected plus the diagonal branch; the kernel walks the active chunks).
    Returns int64 [b, Hkv, nqb, topk]."""
    w = _f64(weights)
    b, hkv, nqb, nkb = w.shape
    out = np.full((b, hkv, nqb, topk), -1, dtype=np.int64)
    for bi in range(b):
        for g in range(hkv):
            for i in range(nqb):
                jd = diag_block(i, q_offset, block)
                live = [j for j in range(jd) if w[bi, g, i, j] > 0]
                live = sorted(live, key=lambda j: (-w[bi, g, i, j], j))[: topk - 1]
                chosen = sorted(live + [jd])
                out[bi, g, i, : len(chosen)] = chosen
    return out


def prior_bias(weights, sel, sigma: float, block: int, q_offset: int = 0) -> np.ndarray:
    """Logit bias of each listed block: sigma * ln(w) for a routed block, 0 for
    the diagonal block (and for padding).  Adding it to the logits is the
    softmax taken relative to the prior g proportional to w ** sigma (zero where
    w is zero): sigma = 0 is the plain softmax over the listed blocks.
    [DashAttn] "Etapa 2" (softmax with the reference distribution replaced by a
    prior built from the routing weights, zero where they are zero; sigma sets
    how strongly the prior counts; the routing bias is added to the logits).
    Returns float64, the shape of sel."""
    w = _f64(weights)
    sel = np.asarray(sel)
    out = np.zeros(sel.shape)
    b, hkv, nqb, topk = sel.shape
    for bi in range(b):
        for g in range(hkv):
            for i in range(nqb):
                jd = diag_block(i, q_offset, block)
                for e in range(topk):
                    j = int(sel[bi, g, i, e])
                    if j >= 0 and j != jd:
                        out[bi, g, i, e] = sigma * math.log(w[bi, g, i, j])
    return out


def prior_attention(q, k, v, sel, bias, block: int, scale: Optional[float] = None, q_offset: int = 0):
    """Softmax attention over the keys of the listed blocks (causal), each
    logit shifted by its block's bias:
        logit_rc = scale * q_r . k_c + bias[b, g, i, e]   for c in block sel[b,g,i,e].
    sel and bias are per KV group [b, Hkv, nqb, topk].  Returns (O, LSE), LSE
    the natural log-sum-exp of the shifted logits.
    [DashAttn] "Etapa 2" (prior-induced sparse softmax over the selected
    chunks)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    sel, bias = np.asarray(sel), _f64(bias)
    b, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    group = hq // hkv
    _check_geometry(seq_q, seq_kv, q_offset, block)
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    out = np.empty((b, hq, seq_q, d))
    lse = np.empty((b, hq, seq_q))
    for bi in range(b):
        for h in range(hq):
            g = h // group
            for i in range(n_blocks(seq_q, block)):
                r0, r1 = i * block, min((i + 1) * block, seq_q)
                last = q_offset + r1 - 1
                cols, shift = [], []
                for e, j in _listed_blocks(sel[bi, g, i]):
                    c = _allowed_keys([j], last, block, seq_kv)
                    cols.append(c)
                    shift.append(np.full(len(c), bias[bi, g, i, e]))
                cols = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
                shift = np.concatenate(shift) if shift else np.zeros(0)
                logits = scale * (q[bi, h, r0:r1] @ k[bi, g, cols].T) + shift[None, :]
                pos = q_offset + np.arange(r0, r1)
                logits[cols[None, :] > pos[:, None]] = -np.inf
                m = logits.max(axis=1, keepdims=True)
                w = np.exp(logits - m)
                z = w.sum(axis=1, keepdims=True)
                out[bi, h, r0:r1] = (w @ v[bi, g, cols]) / z
                lse[bi, h, r0:r1] = (m + np.log(z))[:, 0]
    return out, lse


# --------------------------------------------------------------------------- backward

def _block_backward(qb, kc, vc, dob, allowed, scale):
    """Gradients of L = sum(dob * o) for the query rows qb [n, d] of one query
    block, where row r's output o_r is softmax attention over the keys kc
    [m, d] / values vc [m, d] that ``allowed`` [n, m] marks for it.  With P the
    masked softmax probabilities:
        dV  = P^T dO
        dP  = dO V^T
        dS  = P * (dP - rowsum(P * dP))      (the softmax Jacobian applied to dP)
        dQ  = scale * dS K
        dK  = scale * dS^T Q
    A row with no allowed key has no output and gets zero gradients.
    Returns (dq [n, d], dk [m, d], dv [m, d])."""
    logits = np.where(allowed, scale * (qb @ kc.T), -np.inf)
    live = allowed.any(axis=1, keepdims=True)
    m = np.where(live, logits.max(axis=1, keepdims=True), 0.0)
    w = np.where(allowed, np.exp(logits - m), 0.0)
    p = w / np.where(live, w.sum(axis=1, keepdims=True), 1.0)
    dv = p.T @ dob
    dp = dob @ vc.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ kc), scale * (ds.T @ qb), dv


def attention_backward(q, k, v, dout, sel, block: int, scale: Optional[float] = None, q_offset: int = 0,
                       full: bool = False, row_range: Optional[Tuple[int, int]] = None):
    """Gradients of the scalar sum(dout * O) with respect to Q, K and V, where
    O is the block-sparse attention of sparse_attention (``full`` False: row r
    of query block i sees keys c <= its position whose block is in sel[b,h,i])
    or the full causal attention of full_attention_dropped_mass (``full`` True;
    sel unused).  Keys outside a row's set get no gradient from that row.
    [SSA-summary] 1 "Planteamiento del Problema" (the sparse stream gives
    unselected keys zero gradient and normalises over the selected subset
    only) and 2 "Mecanismo Central" (the full stream passes gradient to every
    token); the formulas are the chain rule through softmax attention.

    ``row_range`` = (lo, hi) (lo a multiple of the block size) restricts the
    outputs to query rows [lo, hi); dout then holds just those rows.
    Returns dq [b,Hq,hi-lo,d], dk and dv [b,Hkv,seq_kv,d] (float64); the
    gradient of a query head's rows lands on its KV head (GQA: summed over the
    group)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    b, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    group = hq // hkv
    _check_geometry(seq_q, seq_kv, q_offset, block)
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    lo, hi = (0, seq_q) if row_range is None else row_range
    if dout.shape != (b, hq, hi - lo, d):
        raise ValueError("dout must cover the rows of row_range")
    dq = np.zeros((b, hq, hi - lo, d))
    dk = np.zeros((b, hkv, seq_kv, d))
    dv = np.zeros((b, hkv, seq_kv, d))
    for bi in range(b):
        for h in range(hq):
            g = h // group
            for i in range(lo // block, n_blocks(hi, block)):
                r0, r1 = max(i * block, lo), min((i + 1) * block, hi)
                last = q_offset + r1 - 1
                if full:
                    cols = np.arange(last + 1)
                else:
                    cols = _allowed_keys(sel[bi, h, i], last, block, seq_kv)
                pos = q_offset + np.arange(r0, r1)
                allowed = cols[None, :] <= pos[:, None]
                gq, gk, gv = _block_backward(q[bi, h, r0:r1], k[bi, g, cols], v[bi, g, cols],
                                             dout[bi, h, r0 - lo:r1 - lo], allowed, scale)
                dq[bi, h, r0 - lo:r1 - lo] = gq
                np.add.at(dk[bi, g], cols, gk)
                np.add.at(dv[bi, g], cols, gv)
    return dq, dk, dv


# --------------------------------------------------------------------------- the whole path

# --------------------------------------------------------------------------- early stopping

def early_stop_order(sel_row, score_row, jd: int):
    """Visiting order of one query block's selected blocks under early
    stopping: the diagonal block first, then the other listed blocks by coarse
    score (higher first, then lower index, NaN last), i.e. in decreasing
    estimated importance.

    [S2O] "Regla de Parada Temprana" (candidate blocks processed in descending
    order of estimated importance) and "Implementacion del Kernel" (a dense
    pass over the query's own segment initialises the softmax state first)."""
    listed = [j for _, j in _listed_blocks(sel_row)]
    others = sorted((j for j in listed if j != jd), key=lambda j: _rank_key(float(score_row[j]), j))
    return ([jd] if jd in listed else []) + others


def _early_stop_count(gains, tau: float) -> int:
    """Number of blocks visited: stop after the first block t >= 1 whose gain
    is below tau times the mass of the blocks before it, for every row."""
    for t in range(1, len(gains)):
        if np.all(gains[t] < tau * sum(gains[:t])):
            return t + 1
    return len(gains)


def early_stop_attention(q, k, v, scores, sel, tau: float, block: int, scale: Optional[float] = None,
                         q_offset: int = 0, used=None):
    """Block-sparse attention with early stopping over the selected blocks.

    Query block i visits its blocks in early_stop_order.  For every block
    after the first, the marginal gain of row r is
        g_r = sum over the block's keys c <= pos_r of exp(scale * q_r . k_c)
    and the mass accumulated before it is L_r = the same sum over the blocks
    visited before it.  When g_r < tau * L_r for every row of the query block,
    that block is kept and the remaining ones are skipped.  Each row then
    attends over the keys c <= pos_r of the visited blocks.

    [S2O] "Regla de Parada Temprana" (stop once the marginal gain in attention
    mass of a processed block falls below a threshold relative to the
    accumulated mass) and "Implementacion del Kernel".

    ``used`` (int [b, Hq, nqb]) imposes the number of visited blocks instead of
    the rule.  Returns (O [b,Hq,seq_q,d], LSE [b,Hq,seq_q], used [b,Hq,nqb],
    ratio [b,Hq,nqb,topk]) where ratio[..., t] = max over the block's rows of
    g_r / L_r at block t of the order (t >= 1; NaN where there is none)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    scores = _f64(scores)
    b, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    group = hq // hkv
    _check_geometry(seq_q, seq_kv, q_offset, block)
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    nqb = n_blocks(seq_q, block)
    topk = sel.shape[-1]
    out = np.empty((b, hq, seq_q, d))
    lse = np.empty((b, hq, seq_q))
    used_out = np.zeros((b, hq, nqb), dtype=np.int64)
    ratio = np.full((b, hq, nqb, topk), np.nan)
    for bi in range(b):
        for h in range(hq):
            g = h // group
            for i in range(nqb):
                jd = diag_block(i, q_offset, block)
                order = early_stop_order(sel[bi, h, i], scores[bi, h, i], jd)
                r0, r1 = i * block, min((i + 1) * block, seq_q)
                pos = q_offset + np.arange(r0, r1)
                # per-block logits of the rows, causal keys only (-inf elsewhere)
                blk_logits = []
                for j in order:
                    c = np.arange(j * block, min((j + 1) * block, seq_kv))
                    lg = scale * (q[bi, h, r0:r1] @ k[bi, g, c].T)
                    lg[c[None, :] > pos[:, None]] = -np.inf
                    blk_logits.append((c, lg))
                mrow = np.max(np.concatenate([lg for _, lg in blk_logits], axis=1), axis=1)
                gains = [np.exp(lg - mrow[:, None]).sum(axis=1) for _, lg in blk_logits]
                acc = gains[0].copy() if gains else np.zeros(r1 - r0)
                for t in range(1, len(order)):
                    ratio[bi, h, i, t] = float(np.max(gains[t] / acc))
                    acc = acc + gains[t]
                n_used = _early_stop_count(gains, tau) if used is None else int(used[bi, h, i])
                used_out[bi, h, i] = n_used
                cols = np.concatenate([c for c, _ in blk_logits[:n_used]])
                lg = np.concatenate([lg for _, lg in blk_logits[:n_used]], axis=1)
                m = lg.max(axis=1, keepdims=True)
                w = np.exp(lg - m)
                z = w.sum(axis=1, keepdims=True)
                out[bi, h, r0:r1] = (w @ v[bi, g, cols]) / z
                lse[bi, h, r0:r1] = (m + np.log(z))[:, 0]
    return out, lse, used_out, ratio


def hot_path(q, k, v, block: int, topk: int, scale: Optional[float] = None, q_offset: int = 0,
             k_summary=None, full_row_range: Optional[Tuple[int, int]] = None, with_full: bool = True,
             shared: bool = False):
    """Summaries -> scores -> selection -> sparse attention -> full attention and
    dropped mass, as one dict of float64 / int64 arrays.  ``shared`` selects one
    list per KV group (select_blocks_shared; "idx_shared" holds it and "idx" its
    per-head view)."""
    res = {}
    if k_summary is None:
        res["k_summary"] = key_summaries(k, block)
    res["scores"] = block_scores(q, k, block, scale, q_offset, k_summary=k_summary)
    if shared:
        res["idx_shared"] = select_blocks_shared(res["scores"], _f64(v).shape[1], topk, block, q_offset)
        res["idx"] = expand_shared(res["idx_shared"], _f64(q).shape[1])
    else:
        res["idx"] = select_blocks(res["scores"], topk, block, q_offset)
    res["o_sparse"], res["lse_sparse"] = sparse_attention(q, k, v, res["idx"], block, scale, q_offset)
    if with_full:
        res["o_full"], res["lse_full"], res["dropped"] = full_attention_dropped_mass(
            q, k, v, res["idx"], block, scale, q_offset, row_range=full_row_range)
    return res

