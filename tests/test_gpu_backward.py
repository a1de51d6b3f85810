"""GPU parity of the backward entry points (through the C ABI) against the fp64
oracle's gradients on the same seeded inputs and output gradients.

The GPU forward supplies O and LSE (as a training step would); the oracle
recomputes everything from the inputs and the GPU's own index lists."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_attention_kv_amd import ssa
from block_sparse_attention_kv_amd import workloads as W
from oracle import ssa_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu
B = 64


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssa.load_library()  # raises if the library is missing: there is no fallback
    return torch.device("cuda:0")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def sparse_bwd_gpu(w, dev, shared=False, repeat=1):
    """GPU scores -> top-k -> sparse forward -> sparse backward."""
    q, k, v = W.make_inputs(w)
    dout = W.make_output_grad(w)
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), dout.to(dev)
    scores, _ = ssa.ssa_block_scores(shape, qd, kd)
    idx = (ssa.ssa_select_topk_shared if shared else ssa.ssa_select_topk)(shape, scores)
    o, lse = ssa.ssa_block_sparse_attn_fwd(shape, qd, kd, vd, idx, shared=shared)
    outs = [ssa.ssa_block_sparse_attn_bwd(shape, qd, kd, vd, idx, o, lse, dod, shared=shared) for _ in range(repeat)]
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    if shared:
        gidx = O.expand_shared(gidx, w.n_q_heads)
    return (q, k, v, dout), gidx, [tuple(t.cpu() for t in r) for r in outs]


def full_bwd_gpu(w, dev, qb_range):
    q, k, v = W.make_inputs(w)
    b0, cnt = qb_range
    rows = (b0 * B, min(w.seq_q, (b0 + cnt) * B))
    dout = W.make_output_grad(w, rows)
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), dout.to(dev)
    scores, _ = ssa.ssa_block_scores(shape, qd, kd)
    idx = ssa.ssa_select_topk(shape, scores)
    of, lf, _ = ssa.ssa_full_attn_fwd_dropped_mass(shape, qd, kd, vd, idx, b0, cnt)
    dq, dk, dv = ssa.ssa_full_attn_bwd(shape, qd, kd, vd, of, lf, dod, b0, cnt)
    torch.cuda.synchronize()
    return (q, k, v, dout), rows, (dq.cpu(), dk.cpu(), dv.cpu())


def compare(got, ref, tag):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        mx, rel = P.check_grad(g, r, f"{tag} {name}")
        print(f"  {tag} {name}: max|diff|/max|ref| {mx:.2e}  rel-L2 {rel:.2e}", flush=True)


SMALL = [
    W.TINY_512,
    W.Workload("bwd_ragged_200", 2, 4, 2, 200, 200, 64, 64, 2, seed=21),
    W.Workload("bwd_ragged_g3_1000", 1, 6, 2, 1000, 1000, 64, 64, 5, seed=22),
    W.Workload("bwd_k1_blockdiag", 1, 4, 1, 384, 384, 64, 64, 1, seed=23),
    W.Workload("bwd_single_row_block", 1, 2, 1, 65, 65, 64, 64, 1, seed=24),
    W.Workload("bwd_chunked", 1, 4, 2, 192, 320, 64, 64, 3, seed=25),
    W.Workload("bwd_planted_1k", 1, 32, 2, 1024, 1024, 64, 64, 4, seed=26, variant="planted"),
    W.Workload("bwd_gqa16_2k", 1, 32, 2, 2048, 2048, 64, 64, 16, seed=27),
    W.Workload("bwd_mha_topk256", 1, 2, 2, 4096, 4096, 64, 64, 256, seed=32),   # every block selected
    W.Workload("bwd_g32", 1, 32, 1, 1024, 1024, 64, 64, 8, seed=33),            # 32 heads on one KV head
    # 1088 KV groups: more groups than dK/dV workgroups, so one pair range per group
    W.Workload("bwd_many_groups", 17, 64, 64, 192, 192, 64, 64, 2, seed=34),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_sparse_backward_small(dev, w):
    say(f"sparse backward {w}")
    (q, k, v, dout), gidx, outs = sparse_bwd_gpu(w, dev)
    ref = O.attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                               gidx, B, q_offset=w.q_offset)
    compare(outs[0], ref, w.name)


@pytest.mark.parametrize("w", [SMALL[1], SMALL[2], SMALL[5], SMALL[7], SMALL[9]], ids=lambda w: w.name)
def test_shared_backward_small(dev, w):
    say(f"shared-selection backward {w}")
    (q, k, v, dout), gidx, outs = sparse_bwd_gpu(w, dev, shared=True)
    ref = O.attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                               gidx, B, q_offset=w.q_offset)
    compare(outs[0], ref, w.name + " shared")


FULL_CASES = [
    (W.TINY_512, (0, 8)),
    (W.Workload("bwd_full_ragged_1000", 1, 6, 2, 1000, 1000, 64, 64, 5, seed=28), (0, 16)),
    (W.Workload("bwd_full_slice", 1, 4, 2, 1000, 1000, 64, 64, 5, seed=29), (9, 5)),   # last 5 blocks, ragged
    (W.Workload("bwd_full_slice_mid", 2, 4, 1, 640, 640, 64, 64, 2, seed=30), (3, 4)),
    (W.Workload("bwd_full_chunked", 1, 4, 2, 192, 320, 64, 64, 3, seed=31), (0, 3)),
    (W.Workload("bwd_full_many_groups", 17, 64, 64, 192, 192, 64, 64, 2, seed=35), (0, 3)),
]


@pytest.mark.parametrize("case", FULL_CASES, ids=lambda c: f"{c[0].name}-{c[1][0]}-{c[1][1]}")
def test_full_backward_small(dev, case):
    w, qb = case
    say(f"full backward {w} blocks {qb}")
    (q, k, v, dout), rows, got = full_bwd_gpu(w, dev, qb)
    ref = O.attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                               None, B, q_offset=w.q_offset, full=True, row_range=rows)
    compare(got, ref, w.name + " full")


def test_sparse_backward_with_every_block_equals_full(dev):
    """topk >= number of blocks: the block-sparse gradients are the full ones."""
    w = SMALL[8]
    say(f"sparse == full backward {w.name}")
    (q, k, v, dout), gidx, outs = sparse_bwd_gpu(w, dev)
    _, _, full = full_bwd_gpu(w, dev, (0, ssa.n_blocks(w.seq_q, B)))
    for name, a, b in zip(("dQ", "dK", "dV"), outs[0], full):
        P.check_grad(a, b.double().numpy(), f"sparse vs full {name}")


def test_backward_is_deterministic(dev):
    w = SMALL[7]
    say(f"determinism {w}")
    _, _, outs = sparse_bwd_gpu(w, dev, repeat=3)
    for r in outs[1:]:
        for a, b in zip(outs[0], r):
            assert torch.equal(a, b)


def test_sparse_backward_prefill_8k(dev):
    """Full-size workload: every gradient against the oracle (about 10 s of CPU)."""
    w = W.PREFILL_8K
    say(f"sparse backward {w.name}")
    (q, k, v, dout), gidx, outs = sparse_bwd_gpu(w, dev)
    ref = O.attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                               gidx, B)
    compare(outs[0], ref, w.name)


def test_full_backward_prefill_8k_slice(dev):
    """Full counterpart on the last 1024 rows of the 8k workload."""
    w = W.PREFILL_8K
    say(f"full backward {w.name} last 16 blocks")
    (q, k, v, dout), rows, got = full_bwd_gpu(w, dev, (112, 16))
    ref = O.attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                               None, B, full=True, row_range=rows)
    compare(got, ref, w.name + " full slice")
