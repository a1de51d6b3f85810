"""The allocation-free block-sparse forward (ssa_block_sparse_attn_fwd_noalloc,
workspace in the library's static scratch array) against the entry point it
varies, ssa_block_sparse_attn_fwd with a caller workspace, through the C ABI.
Both run the same kernels on the same inputs, so the outputs must be
identical bit for bit.  Calls follow one another on one stream, each later
call smaller than the one before, decode and prefill interleaved (the two
use different parts of the array)."""
from __future__ import annotations

import pytest
import torch

from block_sparse_attention_kv_amd import ssa
from block_sparse_attention_kv_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssa.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(w: W.Workload, dev):
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    scores, _ = ssa.ssa_block_scores(shape, q, k)
    idx = ssa.ssa_select_topk(shape, scores)
    return shape, q, k, v, idx


def _reference(shape, q, k, v, idx):
    ws = torch.zeros((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD),), dtype=torch.uint8, device=q.device)
    return ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=ws)


# decode and prefill workloads, each later one smaller than the one before it of its kind
DECODE_BIG = W.DECODE_32K                                                    # 4.3 MB of partials
DECODE_SMALL = W.DECODE_32K.scaled(name="decode_8x4k", batch=8, seq_kv=4096, topk=9)
PREFILL_BIG = W.PREFILL_8K
PREFILL_SMALL = W.TINY_512.scaled(name="ragged_1000", seq_q=1000, seq_kv=1000, n_q_heads=8, n_kv_heads=2)


def test_noalloc_matches_workspace_entry(dev):
    torch.manual_seed(0)
    runs = []
    for w in (DECODE_BIG, PREFILL_BIG, DECODE_SMALL, PREFILL_SMALL):
        say(f"noalloc {w.name}: b={w.batch} Hq={w.n_q_heads} seq_q={w.seq_q} seq_kv={w.seq_kv} topk={w.topk}")
        shape, q, k, v, idx = _inputs(w, dev)
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
        ssa.ssa_block_sparse_attn_fwd_noalloc(shape, q, k, v, idx, out, lse)
        runs.append((w, shape, q, k, v, idx, out, lse))
    torch.cuda.synchronize()
    for w, shape, q, k, v, idx, out, lse in runs:
        o_ref, l_ref = _reference(shape, q, k, v, idx)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), f"{w.name}: out differs from ssa_block_sparse_attn_fwd"
        assert torch.equal(lse, l_ref), f"{w.name}: lse differs from ssa_block_sparse_attn_fwd"


def test_noalloc_repeated_prefill_keeps_queue_zero(dev):
    """Back-to-back prefill calls reuse the work queue in the array: each must
    find it zero (left so by the call before)."""
    say("noalloc prefill_8k three times in a row")
    shape, q, k, v, idx = _inputs(PREFILL_BIG, dev)
    o_ref, l_ref = _reference(shape, q, k, v, idx)
    outs = []
    for _ in range(3):
        out, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        ssa.ssa_block_sparse_attn_fwd_noalloc(shape, q, k, v, idx, out, lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    for out, lse in outs:
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)


def test_noalloc_rejects_decode_beyond_the_array(dev):
    """A decode shape whose partials exceed the 8 MiB array fails on the host
    with SSA_ERR_WORKSPACE and launches nothing."""
    say("noalloc oversize decode (host-side refusal)")
    b, hq, hkv, skv = 1024, 32, 2, 128
    q = torch.zeros((b, hq, 1, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((b, hkv, skv, 64), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    idx = torch.zeros((b, hq, 1, 2), dtype=torch.int32, device=dev)
    shape = ssa.make_shape(q, hkv, skv, block=64, topk=2)
    out = torch.full_like(q, 7.0)
    lse = torch.full((b, hq, 1), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(ssa.SSAError) as ei:
        ssa.ssa_block_sparse_attn_fwd_noalloc(shape, q, k, v, idx, out, lse)
    assert ei.value.status == ssa.SSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
