"""Independent library-based checks used to pin the oracle (tests only).

Everything here is built from PyTorch library routines in float64 on the CPU
(scaled_dot_product_attention, logsumexp, avg_pool1d, matmul).  It shares no
code with ``oracle/`` and is never used as the parity reference for the HIP
path; it exists so the oracle is checked against something other than itself.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def t64(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def block_mask_from_idx(idx, seq_q: int, seq_kv: int, block: int, q_offset: int) -> torch.Tensor:
    """Boolean [b, Hq, seq_q, seq_kv]: key c allowed for query row r iff
    block(c) is in r's query-block list and c <= q_offset + r."""
    idx = torch.as_tensor(np.asarray(idx))
    b, hq, nqb, _ = idx.shape
    nkb = -(-seq_kv // block)
    bm = torch.zeros((b, hq, nqb, nkb + 1), dtype=torch.bool)
    safe = torch.where(idx < 0, torch.full_like(idx, nkb), idx)
    bm.scatter_(-1, safe, True)
    bm = bm[..., :nkb]
    rows = bm.repeat_interleave(block, dim=2)[:, :, :seq_q]
    full = rows.repeat_interleave(block, dim=3)[..., :seq_kv]
    causal = torch.ones((seq_q, seq_kv), dtype=torch.bool).tril(diagonal=q_offset)
    return full & causal


def causal_mask(seq_q: int, seq_kv: int, q_offset: int) -> torch.Tensor:
    return torch.ones((seq_q, seq_kv), dtype=torch.bool).tril(diagonal=q_offset)


def sdpa(q, k, v, mask, scale):
    """(O, LSE) via torch SDPA (GQA-aware) and logsumexp of the masked logits."""
    q, k, v = t64(q), t64(k), t64(v)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale, enable_gqa=True)
    group = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(group, dim=1)
    logits = torch.matmul(q, kk.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~mask, -math.inf)
    return o.numpy(), torch.logsumexp(logits, dim=-1).numpy()


def avg_pool_blocks(x, block: int) -> np.ndarray:
    """Block means along the row axis via avg_pool1d (ceil mode averages the
    rows a partial last window actually covers)."""
    x = t64(x)
    lead = x.shape[:-2]
    n, d = x.shape[-2:]
    y = x.reshape(-1, n, d).transpose(1, 2)  # [B*, d, n]
    p = F.avg_pool1d(y, kernel_size=block, stride=block, ceil_mode=True)
    return p.transpose(1, 2).reshape(*lead, -1, d).numpy()
