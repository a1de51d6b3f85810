"""The fused decode scoring + selection (ssa_decode_scores_select) against the
two calls it fuses (ssa_block_scores with cached summaries, then
ssa_select_topk or ssa_select_topk_shared), through the C ABI: scores and
indices must be identical bit for bit.  One case is also checked against the
oracle's scores and selection."""
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

CASES = [
    W.DECODE_32K,                                                                # 16 heads per KV head, 512 blocks
    W.Workload("decode_ragged_1000", 3, 8, 2, 1, 1000, 64, 64, 5, seed=41),    # last block partial
    W.Workload("decode_g32_4096", 2, 64, 2, 1, 4096, 64, 64, 9, seed=42),      # 32 heads per KV head
    W.Workload("decode_one_key", 2, 4, 4, 1, 1, 64, 64, 3, seed=43),           # a single key
    W.Workload("decode_short", 2, 6, 2, 1, 300, 64, 64, 8, seed=44),           # every block kept
    W.Workload("decode_long_40000", 1, 4, 2, 1, 40000, 64, 64, 16, seed=45),   # 625 blocks: the long-row path
    W.Workload("decode_g5_2000", 2, 10, 2, 1, 2000, 64, 64, 6, seed=46),       # group of 5 heads
]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssa.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fused_equals_two_calls(dev, w, shared):
    say(f"{w.name} shared={shared}: b={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} seq_kv={w.seq_kv} topk={w.topk}")
    q, k, _ = W.make_inputs(w)
    q, k = q.to(dev), k.to(dev)
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    ks = ssa.ssa_block_summaries(k, block=w.block)
    s_ref, _ = ssa.ssa_block_scores(shape, q, None, ks)
    i_ref = (ssa.ssa_select_topk_shared if shared else ssa.ssa_select_topk)(shape, s_ref)
    scores, idx = ssa.ssa_decode_scores_select(shape, q, ks, shared=shared)
    _, idx2 = ssa.ssa_decode_scores_select(shape, q, ks, shared=shared, with_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(scores, s_ref), f"{w.name}: scores differ from ssa_block_scores"
    assert torch.equal(idx, i_ref), f"{w.name}: indices differ from the separate selection"
    assert torch.equal(idx2, i_ref), f"{w.name}: indices differ when the scores are not written"


def test_fused_matches_oracle(dev):
    w = CASES[2]
    say(f"{w.name}: fused scores and selection against the oracle")
    q, k, _ = W.make_inputs(w)
    shape = ssa.make_shape(q.to(dev), w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    ks = ssa.ssa_block_summaries(k.to(dev), block=w.block)
    scores, idx = ssa.ssa_decode_scores_select(shape, q.to(dev), ks)
    torch.cuda.synchronize()
    qn, kn = q.double().numpy(), k.double().numpy()
    ks_ref = O.key_summaries(kn, B)
    s_ref = O.block_scores(qn, None, B, q_offset=w.q_offset, k_summary=ks_ref)
    s_gpu = P.np64(scores)
    assert np.array_equal(np.isneginf(s_gpu), np.isneginf(s_ref))
    fin = np.isfinite(s_ref)
    assert np.all(np.abs(s_gpu[fin] - s_ref[fin]) <= 1e-6 * np.maximum(np.abs(s_ref[fin]), 1e-3))
    idx_ref = O.select_blocks(s_ref, w.topk, B, q_offset=w.q_offset)
    P.check_indices(idx, s_ref, idx_ref, w.topk, B, w.q_offset)


def test_fused_refuses_what_does_not_fit(dev):
    """64 query heads per KV head exceed the fused kernel: a clear refusal on
    the host, nothing launched; prefill shapes are refused as invalid."""
    q = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device=dev)
    ks = torch.zeros((1, 1, 16, 64), dtype=torch.float32, device=dev)
    shape = ssa.make_shape(q, 1, 16 * 64, block=64, topk=4)
    with pytest.raises(ssa.SSAError) as ei:
        ssa.ssa_decode_scores_select(shape, q, ks)
    assert ei.value.status == ssa.SSA_ERR_UNSUPPORTED
    q2 = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16, device=dev)
    ks2 = torch.zeros((1, 1, 2, 64), dtype=torch.float32, device=dev)
    shape2 = ssa.make_shape(q2, 1, 128, block=64, topk=2)
    with pytest.raises(ssa.SSAError) as ei:
        ssa.ssa_decode_scores_select(shape2, q2, ks2)
    assert ei.value.status == ssa.SSA_ERR_INVALID_ARG
