"""Seeded synthetic workloads shared by the HIP path's tests/bench and the oracle.

This module only *draws inputs*: it holds none of the method's arithmetic
(no pooling, scoring, selection or attention).  Both sides of every parity
check receive the same bf16 tensors produced here.

Recipe (identical for every workload):
  1. ``torch.Generator('cpu').manual_seed(seed)``
  2. fp32 ``randn`` for Q ``[b, Hq, seq_q, d]``, then K and V ``[b, Hkv, seq_kv, d]``
  3. workload-specific edits in fp32 (planted direction / tie construction)
  4. cast to bf16 (round-to-nearest-even)

The shapes are those of one attention layer of a Llama-3.2-1B-like model with
few KV heads (32 query heads sharing 2 KV heads, head_dim 64), trained at 8k
and extrapolated to 32k, with block size 64 and a 1024-token receptive field
(16 blocks).  SSA guide (mauroscia.it), sections "Approccio generale di SSA",
"Block-sparse attention e Receptive Field" and "Training recipe in pratica";
SSA summary (gist.science 2511.20102), section 4 "Resultados Experimentales".
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_q: int
    seq_kv: int
    head_dim: int
    block: int
    topk: int  # total blocks per query block, including the forced diagonal / most recent block
    seed: int
    variant: str = "iid"  # "iid" | "planted" | "tie"
    # rows [lo, hi) of the full-attention counterpart (None = every query row)
    full_rows: Optional[Tuple[int, int]] = None
    description: str = ""

    @property
    def q_offset(self) -> int:
        return self.seq_kv - self.seq_q

    @property
    def is_decode(self) -> bool:
        return self.seq_q == 1 and self.seq_kv > 1

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Seeds are fixed constants; any fixed values would do.
TINY_512 = Workload(
    "tiny_512", batch=1, n_q_heads=2, n_kv_heads=1, seq_q=512, seq_kv=512,
    head_dim=64, block=64, topk=4, seed=1001,
    description="tiny causal block-sparse fwd: 2 query heads on 1 KV head, N=512, k=4")
PREFILL_8K = Workload(
    "prefill_8k", batch=1, n_q_heads=32, n_kv_heads=2, seq_q=8192, seq_kv=8192,
    head_dim=64, block=64, topk=16, seed=1002,
    description="prefill of a Llama-3.2-1B-like layer: 32/2 heads, N=8192, k=16 (1024-token budget)")
STRUCTURED_8K = Workload(
    "structured_8k", batch=4, n_q_heads=32, n_kv_heads=2, seq_q=8192, seq_kv=8192,
    head_dim=64, block=64, topk=16, seed=1003, variant="planted",
    description="planted shared direction on ~1/8 of the key blocks, queries pulled towards it")
STRUCTURED_8K_TIE = Workload(
    "structured_8k_tie", batch=4, n_q_heads=32, n_kv_heads=2, seq_q=8192, seq_kv=8192,
    head_dim=64, block=64, topk=16, seed=1013, variant="tie",
    description="uniform-score tie case: one K row per (batch, KV head) repeated at every position")
EXTRAP_32K = Workload(
    "extrap_32k", batch=1, n_q_heads=32, n_kv_heads=2, seq_q=32768, seq_kv=32768,
    head_dim=64, block=64, topk=16, seed=1004, full_rows=(32768 - 4096, 32768),
    description="length extrapolation: N=32768, fixed 1024-token budget; counterpart on the last 4096 rows")
DECODE_32K = Workload(
    "decode_32k", batch=64, n_q_heads=32, n_kv_heads=2, seq_q=1, seq_kv=32768,
    head_dim=64, block=64, topk=17, seed=1005,
    description="decode: 64 sequences x 1 token against a 32768-entry KV cache, 16 scored blocks + the most recent")

ALL = (TINY_512, PREFILL_8K, STRUCTURED_8K, STRUCTURED_8K_TIE, EXTRAP_32K, DECODE_32K)
BY_NAME = {w.name: w for w in ALL}

PLANT_PROB = 1.0 / 8.0   # chance that a key block carries the planted direction
PLANT_K_SCALE = 3.0
PLANT_Q_SCALE = 2.0


def make_inputs(w: Workload, device: str | torch.device = "cpu"):
    """Return (q, k, v) as contiguous bf16 tensors on ``device``.

    Random numbers are always drawn on the CPU so the oracle and the GPU see
    bit-identical inputs."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    d = w.head_dim
    q = torch.randn((w.batch, w.n_q_heads, w.seq_q, d), generator=g, dtype=torch.float32)
    k = torch.randn((w.batch, w.n_kv_heads, w.seq_kv, d), generator=g, dtype=torch.float32)
    v = torch.randn((w.batch, w.n_kv_heads, w.seq_kv, d), generator=g, dtype=torch.float32)
    if w.variant == "planted":
        u = torch.randn((d,), generator=g, dtype=torch.float32)
        u = u / u.norm()
        nkb = -(-w.seq_kv // w.block)
        planted = torch.rand((w.batch, w.n_kv_heads, nkb), generator=g) < PLANT_PROB
        row_mask = planted.repeat_interleave(w.block, dim=-1)[..., : w.seq_kv]
        k = k + PLANT_K_SCALE * row_mask.unsqueeze(-1).to(torch.float32) * u
        q = q + PLANT_Q_SCALE * u
    elif w.variant == "tie":
        k = k[:, :, :1, :].expand(-1, -1, w.seq_kv, -1).contiguous()
    elif w.variant != "iid":
        raise ValueError(f"unknown variant {w.variant!r}")
    out = []
    for t in (q, k, v):
        out.append(t.to(torch.bfloat16).contiguous().to(device))
    return tuple(out)



def make_output_grad(w: Workload, rows: Optional[Tuple[int, int]] = None, device: str | torch.device = "cpu"):
    """Seeded synthetic gradient of the attention output, bf16
    [b, Hq, hi - lo, d] for query rows [lo, hi) (default: every row), drawn
    from its own generator (seed + 500000) so the forward inputs are unchanged.
    Row r of the full tensor holds the same values whatever the range."""
    lo, hi = (0, w.seq_q) if rows is None else rows
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 500000)
    full = torch.randn((w.batch, w.n_q_heads, w.seq_q, w.head_dim), generator=g, dtype=torch.float32)
    return full[:, :, lo:hi].to(torch.bfloat16).contiguous().to(device)


def make_learned_query(w: Workload, scale: float = 1.0, device: str | torch.device = "cpu"):
    """Seeded synthetic learned chunk query, fp32 [Hkv, d]: N(0, scale^2),
    drawn from its own generator (seed + 700000); it stands in for the trained
    vector of a chunk-summary stage (there are no trained weights here)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 700000)
    return (torch.randn((w.n_kv_heads, w.head_dim), generator=g, dtype=torch.float32) * scale).to(device)
