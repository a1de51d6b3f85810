"""The entry points launch kernels only (no allocation, no memset, no host
synchronisation), so a caller can capture a step in a HIP graph.  Each test
captures a step, replays it several times with the program's own eager work
and synchronisations in between, and checks every replay against the eager
result bit for bit."""
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


def replay_and_compare(step, outputs, dev, replays=3):
    """Eager reference, then capture and replays of `step`; every replay must
    reproduce the eager outputs exactly."""
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()  # warm the caching allocator outside the capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(replays):
        for t in outputs:
            t.zero_()                          # the program's own eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs, ref):
            assert torch.equal(a, b), f"replay {r} differs from the eager result"


def test_prefill_step_in_a_graph(dev):
    w = W.Workload("graph_prefill_1k", 1, 8, 2, 1000, 1000, 64, 64, 5, seed=41)
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nqb, nkb = ssa.n_blocks(w.seq_q, w.block), ssa.n_blocks(w.seq_kv, w.block)
    scores = torch.empty((w.batch, w.n_q_heads, nqb, nkb), dtype=torch.float32, device=dev)
    ksum = torch.empty((w.batch, w.n_kv_heads, nkb, w.head_dim), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.n_q_heads, nqb, w.topk), dtype=torch.int32, device=dev)
    out, out_f = torch.empty_like(q), torch.empty_like(q)
    lse, lse_f, drop = (torch.empty(q.shape[:3], dtype=torch.float32, device=dev) for _ in range(3))

    def step():
        ssa.ssa_block_scores(shape, q, k, summary_out=ksum, scores=scores)
        ssa.ssa_select_topk(shape, scores, idx)
        ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, out=out, lse=lse)
        ssa.ssa_full_attn_fwd_dropped_mass(shape, q, k, v, idx, 0, nqb, out=out_f, lse=lse_f, dropped=drop)

    replay_and_compare(step, [scores, idx, out, lse, out_f, lse_f, drop], dev)


@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
def test_decode_step_in_a_graph(dev, shared):
    w = W.Workload("graph_decode_2560", 2, 32, 2, 1, 2560, 64, 64, 17, seed=42)
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nkb = ssa.n_blocks(w.seq_kv, w.block)
    ks = ssa.ssa_block_summaries(k, block=w.block)
    scores = torch.empty((w.batch, w.n_q_heads, 1, nkb), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.n_kv_heads if shared else w.n_q_heads, 1, w.topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD),), dtype=torch.uint8, device=dev)
    select = ssa.ssa_select_topk_shared if shared else ssa.ssa_select_topk

    def step():
        ssa.ssa_block_scores(shape, q, None, ks, scores=scores)
        select(shape, scores, idx)
        ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=ws, out=out, lse=lse, shared=shared)

    replay_and_compare(step, [scores, idx, out, lse], dev)


def test_persistent_prefill_step_in_a_graph(dev):
    """The persistent launches take units from a work queue in the workspace
    and leave it zero: zeroed once before capture, every replay must find it
    zero again and reproduce the eager outputs."""
    w = W.Workload("graph_prefill_2k", 1, 8, 2, 2048, 2048, 64, 64, 6, seed=43)
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nqb, nkb = ssa.n_blocks(w.seq_q, w.block), ssa.n_blocks(w.seq_kv, w.block)
    scores = torch.empty((w.batch, w.n_q_heads, nqb, nkb), dtype=torch.float32, device=dev)
    ksum = torch.empty((w.batch, w.n_kv_heads, nkb, w.head_dim), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.n_q_heads, nqb, w.topk), dtype=torch.int32, device=dev)
    out, out_f = torch.empty_like(q), torch.empty_like(q)
    lse, lse_f, drop = (torch.empty(q.shape[:3], dtype=torch.float32, device=dev) for _ in range(3))
    ws_sp = torch.zeros((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD),), dtype=torch.uint8, device=dev)
    ws_full = torch.zeros((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_FULL_FWD),), dtype=torch.uint8, device=dev)

    def step():
        ssa.ssa_block_scores(shape, q, k, summary_out=ksum, scores=scores)
        ssa.ssa_select_topk(shape, scores, idx)
        ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=ws_sp, out=out, lse=lse)
        ssa.ssa_full_attn_fwd_dropped_mass(shape, q, k, v, idx, 0, nqb, out=out_f, lse=lse_f, dropped=drop,
                                           workspace=ws_full)

    replay_and_compare(step, [scores, idx, out, lse, out_f, lse_f, drop], dev)
    assert int(ws_sp.count_nonzero()) == 0 and int(ws_full.count_nonzero()) == 0


@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
def test_fused_decode_step_in_a_graph(dev, shared):
    w = W.Workload("graph_decode_fused_2560", 2, 32, 2, 1, 2560, 64, 64, 17, seed=44)
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    nkb = ssa.n_blocks(w.seq_kv, w.block)
    ks = ssa.ssa_block_summaries(k, block=w.block)
    scores = torch.empty((w.batch, w.n_q_heads, 1, nkb), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.n_kv_heads if shared else w.n_q_heads, 1, w.topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD),), dtype=torch.uint8, device=dev)

    def step():
        ssa.ssa_decode_scores_select(shape, q, ks, scores=scores, idx=idx, shared=shared)
        ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=ws, out=out, lse=lse, shared=shared)

    replay_and_compare(step, [scores, idx, out, lse], dev)
