"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Small problems are compared element by element; the
full-size workloads on every block index and element by element over every
row of: prefill_8k (all heads, both selections), batch row 0 of structured_8k
in both variants, eight heads spanning both KV groups of extrap_32k (every
sparse row and the full slice), and all 64 decode_32k sequences; plus
properties that hold at any size."""
from __future__ import annotations

import math

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


def gpu_path(w: W.Workload, q, k, v, dev, full_range=None, with_full=True, shared=False):
    """Run summaries -> scores -> top-k -> sparse -> full on the GPU (``shared``:
    group-shared selection)."""
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    res = {}
    if w.seq_q == 1:
        ks = ssa.ssa_block_summaries(kd, block=w.block)
        res["scores"], res["k_summary"] = ssa.ssa_block_scores(shape, qd, None, ks)
    else:
        res["scores"], res["k_summary"] = ssa.ssa_block_scores(shape, qd, kd)
    select = ssa.ssa_select_topk_shared if shared else ssa.ssa_select_topk
    res["idx"] = select(shape, res["scores"])
    res["o"], res["lse"] = ssa.ssa_block_sparse_attn_fwd(shape, qd, kd, vd, res["idx"], shared=shared)
    if with_full:
        nqb = ssa.n_blocks(w.seq_q, w.block)
        b0, cnt = (0, nqb) if full_range is None else full_range
        res["of"], res["lf"], res["dm"] = ssa.ssa_full_attn_fwd_dropped_mass(shape, qd, kd, vd, res["idx"], b0, cnt,
                                                                             shared=shared)
    torch.cuda.synchronize()
    return {k2: v2.cpu() for k2, v2 in res.items()}


def np_inputs(q, k, v):
    return q.double().numpy(), k.double().numpy(), v.double().numpy()


def reference_selection(s_ref, w: W.Workload, shared: bool):
    """(selection scores, oracle index lists) for per-head or group-shared selection."""
    if shared:
        sel_scores = O.shared_block_scores(s_ref, w.n_kv_heads)
    else:
        sel_scores = s_ref
    return sel_scores, O.select_blocks(sel_scores, w.topk, B, q_offset=w.q_offset)


def per_head(idx, w: W.Workload, shared: bool):
    idx = np.asarray(idx)
    return O.expand_shared(idx, w.n_q_heads) if shared else idx


def check_small(w: W.Workload, dev, full_range=None, shared=False):
    say(f"{w} shared={shared}")
    q, k, v = W.make_inputs(w)
    g = gpu_path(w, q, k, v, dev, full_range, shared=shared)
    qn, kn, vn = np_inputs(q, k, v)
    off = w.q_offset
    ks_ref = O.key_summaries(kn, B)
    assert np.array_equal(P.np64(g["k_summary"]), ks_ref), "key summaries differ"
    s_ref = O.block_scores(qn, kn, B, q_offset=off)
    s_gpu = P.np64(g["scores"])
    assert np.array_equal(np.isneginf(s_gpu), np.isneginf(s_ref))
    fin = np.isfinite(s_ref)
    assert np.all(np.abs(s_gpu[fin] - s_ref[fin]) <= 1e-6 * np.maximum(np.abs(s_ref[fin]), 1e-3))
    sel_scores, idx_ref = reference_selection(s_ref, w, shared)
    P.check_indices(g["idx"], sel_scores, idx_ref, w.topk, B, off)
    gidx = per_head(g["idx"].numpy(), w, shared)
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, gidx, B, q_offset=off)
    P.check_close_outputs(g["o"], o_ref, "O_sparse")
    P.check_abs(g["lse"], lse_ref, P.LSE_ABS, "LSE_sparse")
    nqb = ssa.n_blocks(w.seq_q, B)
    b0, cnt = (0, nqb) if full_range is None else full_range
    rr = (b0 * B, min(w.seq_q, (b0 + cnt) * B))
    of_ref, lf_ref, dm_ref = O.full_attention_dropped_mass(qn, kn, vn, gidx, B, q_offset=off, row_range=rr)
    P.check_close_outputs(g["of"], of_ref, "O_full")
    P.check_abs(g["lf"], lf_ref, P.LSE_ABS, "LSE_full")
    P.check_abs(g["dm"], dm_ref, P.DROP_ABS, "dropped_mass")
    return g


SMALL = [
    W.TINY_512,
    W.Workload("ragged_200", 2, 4, 2, 200, 200, 64, 64, 2, seed=11),
    W.Workload("ragged_g3_1000", 1, 6, 2, 1000, 1000, 64, 64, 5, seed=12),
    W.Workload("k1_blockdiag", 1, 4, 1, 384, 384, 64, 64, 1, seed=13),
    W.Workload("mha_g1", 2, 2, 2, 256, 256, 64, 64, 2, seed=14),
    W.Workload("single_row_block", 1, 2, 1, 65, 65, 64, 64, 1, seed=15),
    W.Workload("chunked_prefill", 1, 4, 2, 192, 320, 64, 64, 3, seed=16),
    W.Workload("planted_1k", 2, 32, 2, 1024, 1024, 64, 64, 4, seed=17, variant="planted"),
    W.Workload("gqa16_2k", 1, 32, 2, 2048, 2048, 64, 64, 16, seed=18),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_parity(dev, w):
    check_small(w, dev)


def test_all_blocks_selected_equals_full(dev):
    w = W.Workload("k_covers_all", 1, 4, 2, 320, 320, 64, 64, 8, seed=19)
    g = check_small(w, dev)
    assert torch.all(g["dm"] == 0)
    P.check_close_outputs(g["o"].double(), g["of"].double(), "sparse vs full")


def test_full_slice_with_ragged_tail(dev):
    w = W.Workload("slice_ragged", 1, 4, 2, 400, 400, 64, 64, 2, seed=20)
    check_small(w, dev, full_range=(2, 5))


def test_max_topk(dev):
    w = W.Workload("topk256", 1, 2, 1, 64 * 300, 64 * 300, 64, 64, 256, seed=21)
    say(w)
    q, k, v = W.make_inputs(w)
    g = gpu_path(w, q, k, v, dev, with_full=False)
    qn, kn, vn = np_inputs(q, k, v)
    s_ref = O.block_scores(qn, kn, B)
    idx_ref = O.select_blocks(s_ref, w.topk, B)
    P.check_indices(g["idx"], s_ref, idx_ref, w.topk, B)
    rows = P.sample_rows(np.random.default_rng(5), 1, 2, w.seq_q, 24)
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, g["idx"].numpy(), B, rows=rows)
    P.check_close_outputs(torch.stack([g["o"][t] for t in rows]), o_ref, "O_sparse sampled")
    P.check_abs(torch.stack([g["lse"][t] for t in rows]), lse_ref, P.LSE_ABS, "LSE sampled")


DECODE_SMALL = [
    W.Workload("decode_ragged_1000", 3, 8, 2, 1, 1000, 64, 64, 5, seed=31),
    W.Workload("decode_gqa16_2560", 2, 32, 2, 1, 2560, 64, 64, 17, seed=32),
    W.Workload("decode_one_key", 2, 4, 4, 1, 1, 64, 64, 3, seed=33),
    W.Workload("decode_65", 1, 6, 2, 1, 65, 64, 64, 1, seed=34),
    W.Workload("decode_long_scan", 1, 2, 1, 1, 64 * 700, 64, 64, 9, seed=35),   # > 512 candidate blocks
    W.Workload("decode_long_list", 2, 32, 2, 1, 64 * 300 - 17, 64, 64, 40, seed=36),  # 16 x 40 = 640 entries per group
    W.Workload("decode_g32_list", 1, 64, 2, 1, 64 * 90, 64, 64, 48, seed=37),  # 32 heads per group, 1536 entries
]


@pytest.mark.parametrize("w", DECODE_SMALL, ids=lambda w: w.name)
def test_decode_parity(dev, w):
    check_small(w, dev)


def test_deterministic(dev):
    w = W.Workload("det", 1, 8, 2, 640, 640, 64, 64, 3, seed=41)
    say(w)
    q, k, v = W.make_inputs(w)
    a = gpu_path(w, q, k, v, dev)
    b = gpu_path(w, q, k, v, dev)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_select_topk_nan_inf_ties(dev):
    say("select_topk with NaN / -inf / exact ties")
    rng = np.random.default_rng(3)
    nb = 40
    s = np.round(rng.standard_normal((2, 3, nb, nb)), 1).astype(np.float32)
    s[0, 0, 30, 5] = np.nan
    s[0, 1, 35, :10] = np.nan
    s[1, 2, 39, :] = -np.inf
    s[1, 0, 20, 3] = -0.0
    s[1, 0, 20, 4] = 0.0
    for i in range(nb):
        s[..., i, i + 1:] = -np.inf
    shape = ssa.Shape(batch=2, n_q_heads=3, n_kv_heads=1, seq_q=nb * B, seq_kv=nb * B, q_offset=0,
                      head_dim=64, block=64, topk=6, causal=1, scale=0.0)
    idx = ssa.ssa_select_topk(shape, torch.from_numpy(s).to(dev)).cpu().numpy()
    ref = O.select_blocks(s.astype(np.float64), 6, B)
    assert np.array_equal(idx, ref)


def _long_row_scores(nkb: int, nqb: int, rng) -> np.ndarray:
    """Scores for rows of many candidates, one pattern per head: continuous
    values; coarse exact ties; one constant; and rows where exactly 64 or 65
    candidates tie at the threshold (the narrowed search gathers at most 64
    keys and falls back to the full search beyond), with NaN, -inf and +-0."""
    s = rng.standard_normal((2, 4, nqb, nkb)).astype(np.float32)
    s[:, 1] = np.round(s[:, 1])
    s[:, 2] = 1.0
    h3 = s[:, 3]
    h3[...] = np.float32(-1.0) - np.abs(h3)
    for bi in range(2):
        for i in range(nqb):
            n_tied = 64 if (i + bi) % 2 == 0 else 65
            cols = rng.choice(nkb - nqb, size=n_tied + 3, replace=False)
            h3[bi, i, cols[:n_tied]] = 2.0
            h3[bi, i, cols[n_tied:n_tied + 3]] = (np.nan, -np.inf, -0.0)
    s[0, 0, 0, :5] = (np.nan, np.inf, -np.inf, 0.0, -0.0)
    return s


@pytest.mark.parametrize("nkb", [300, 600])
def test_select_topk_long_rows(dev, nkb):
    say(f"select_topk, per head and group-shared, {nkb} key blocks (ties, NaN, 64/65 tied at the threshold)")
    rng = np.random.default_rng(nkb)
    nqb, k = 12, 16
    q_offset = (nkb - nqb) * B
    s = _long_row_scores(nkb, nqb, rng)
    for i in range(nqb):
        s[..., i, nkb - nqb + i + 1:] = -np.inf
    shape = ssa.Shape(batch=2, n_q_heads=4, n_kv_heads=2, seq_q=nqb * B, seq_kv=nkb * B, q_offset=q_offset,
                      head_dim=64, block=64, topk=k, causal=1, scale=0.0)
    sd = torch.from_numpy(s).to(dev)
    idx = ssa.ssa_select_topk(shape, sd).cpu().numpy()
    assert np.array_equal(idx, O.select_blocks(s.astype(np.float64), k, B, q_offset))
    idx_s = ssa.ssa_select_topk_shared(shape, sd).cpu().numpy()
    assert np.array_equal(idx_s, O.select_blocks_shared(s.astype(np.float64), 2, k, B, q_offset))


def test_empty_problem_writes_nothing(dev):
    say("empty problems")
    import ctypes
    lib = ssa.load_library()
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device=dev)
    out = torch.full((1, 2, 64, 64), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((1, 2, 64), 7.0, device=dev)
    idx = torch.zeros((1, 2, 1, 2), dtype=torch.int32, device=dev)
    for kw in (dict(batch=0), dict(seq_q=0, seq_kv=0)):
        sh = dict(batch=1, n_q_heads=2, n_kv_heads=1, seq_q=64, seq_kv=64, q_offset=0, head_dim=64,
                  block=64, topk=2, causal=1, scale=0.0)
        sh.update(kw)
        shape = ssa.Shape(**sh)
        st = lib.ssa_block_sparse_attn_fwd(ctypes.byref(shape), ssa._ptr(q), ssa._ptr(q), ssa._ptr(q),
                                           ssa._ptr(idx), ssa._ptr(out), ssa._ptr(lse), None, 0, None)
        assert st == ssa.SSA_OK
        st = lib.ssa_full_attn_fwd_dropped_mass(ctypes.byref(shape), ssa._ptr(q), ssa._ptr(q), ssa._ptr(q),
                                                ssa._ptr(idx), 0, 0, ssa._ptr(out), ssa._ptr(lse),
                                                ssa._ptr(lse), None, 0, None)
        assert st == ssa.SSA_OK
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


# ----------------------------------------------------------------------------- full-size workloads

def check_full_size(w: W.Workload, dev, nrows=96, seq_subset=None, shared=False):
    say(f"{w} shared={shared}")
    q, k, v = W.make_inputs(w)
    nqb = ssa.n_blocks(w.seq_q, B)
    if w.full_rows is None:
        fr = (0, nqb)
    else:
        fr = (w.full_rows[0] // B, ssa.n_blocks(w.full_rows[1], B) - w.full_rows[0] // B)
    g = gpu_path(w, q, k, v, dev, full_range=fr, with_full=True, shared=shared)
    bsel = list(range(w.batch)) if seq_subset is None else seq_subset
    qn = q[bsel].double().numpy()
    kn = k[bsel].double().numpy()
    vn = v[bsel].double().numpy()
    off = w.q_offset
    assert np.array_equal(P.np64(g["k_summary"][bsel]), O.key_summaries(kn, B))
    s_ref = O.block_scores(qn, kn, B, q_offset=off)
    sel_scores, idx_ref = reference_selection(s_ref, w, shared)
    ndiff = P.check_indices(g["idx"][bsel], sel_scores, idx_ref, w.topk, B, off)
    print(f"[case] {w.name}: index rows differing inside the tie band: {ndiff}", flush=True)
    gidx = per_head(g["idx"][bsel].numpy(), w, shared)
    rng = np.random.default_rng(w.seed)
    rows = P.sample_rows(rng, len(bsel), w.n_q_heads, w.seq_q, nrows)
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, gidx, B, q_offset=off, rows=rows)
    got_o = torch.stack([g["o"][bsel[b], h, r] for b, h, r in rows])
    got_l = torch.stack([g["lse"][bsel[b], h, r] for b, h, r in rows])
    P.check_close_outputs(got_o, o_ref, "O_sparse sampled")
    P.check_abs(got_l, lse_ref, P.LSE_ABS, "LSE_sparse sampled")
    lo = fr[0] * B
    frows = [(b, h, lo + (r % (g["of"].shape[2]))) for b, h, r in rows]
    of_ref, lf_ref, dm_ref = O.full_attention_dropped_mass(qn, kn, vn, gidx, B, q_offset=off, rows=frows)
    P.check_close_outputs(torch.stack([g["of"][bsel[b], h, r - lo] for b, h, r in frows]), of_ref, "O_full sampled")
    P.check_abs(torch.stack([g["lf"][bsel[b], h, r - lo] for b, h, r in frows]), lf_ref, P.LSE_ABS, "LSE_full sampled")
    P.check_abs(torch.stack([g["dm"][bsel[b], h, r - lo] for b, h, r in frows]), dm_ref, P.DROP_ABS, "dropped sampled")
    # properties at every row: 0 <= delta < 1, delta = 1 - exp(LSE_sparse - LSE_full)
    dm = g["dm"].double()
    assert torch.all(dm >= 0) and torch.all(dm < 1)
    hi = lo + g["of"].shape[2]
    ident = 1 - torch.exp(g["lse"][:, :, lo:hi].double() - g["lf"].double())
    assert float((dm - ident).abs().max()) < 2e-3
    return g


def check_every_row(w: W.Workload, g, q, k, v, batches, heads, shared=False):
    """Element-wise parity over every row of the given batch rows and query
    heads: O, LSE of the block-sparse forward and O, LSE, dropped mass of the
    full counterpart (over its query-block range), against the oracle run
    with the GPU's own indices, one KV group at a time."""
    G = w.n_q_heads // w.n_kv_heads
    gidx = per_head(g["idx"].numpy(), w, shared)
    lo = (0 if w.full_rows is None else w.full_rows[0] // B * B)
    hi = lo + g["of"].shape[2]
    for bi in batches:
        for kvh in range(w.n_kv_heads):
            hs = [h for h in heads if h // G == kvh]
            if not hs:
                continue
            qn = q[bi:bi + 1, hs].double().numpy()
            kn = k[bi:bi + 1, kvh:kvh + 1].double().numpy()
            vn = v[bi:bi + 1, kvh:kvh + 1].double().numpy()
            sel = gidx[bi:bi + 1, hs]
            tag = f"{w.name} b{bi} heads {hs[0]}..{hs[-1]}"
            o_ref, l_ref = O.sparse_attention(qn, kn, vn, sel, B, q_offset=w.q_offset)
            P.check_close_outputs(g["o"][bi:bi + 1, hs], o_ref, f"O_sparse every row, {tag}")
            P.check_abs(g["lse"][bi:bi + 1, hs], l_ref, P.LSE_ABS, f"LSE_sparse every row, {tag}")
            of_ref, lf_ref, dm_ref = O.full_attention_dropped_mass(qn, kn, vn, sel, B, q_offset=w.q_offset,
                                                                   row_range=(lo, hi))
            P.check_close_outputs(g["of"][bi:bi + 1, hs], of_ref, f"O_full every row, {tag}")
            P.check_abs(g["lf"][bi:bi + 1, hs], lf_ref, P.LSE_ABS, f"LSE_full every row, {tag}")
            P.check_abs(g["dm"][bi:bi + 1, hs], dm_ref, P.DROP_ABS, f"dropped mass every row, {tag}")


def test_prefill_8k_full_size(dev):
    w = W.PREFILL_8K
    g = check_full_size(w, dev)
    # rows of the first k blocks keep every causal key
    assert torch.all(g["dm"][:, :, : w.topk * B] == 0)
    # every row of every head
    q, k, v = W.make_inputs(w)
    check_every_row(w, g, q, k, v, batches=[0], heads=list(range(w.n_q_heads)))


def test_structured_8k_planted_full_size(dev):
    w = W.STRUCTURED_8K
    g = check_full_size(w, dev, nrows=64)
    q, k, v = W.make_inputs(w)
    check_every_row(w, g, q, k, v, batches=[0], heads=list(range(w.n_q_heads)))


def test_structured_8k_tie_full_size(dev):
    w = W.STRUCTURED_8K_TIE
    say(w)
    q, k, v = W.make_inputs(w)
    g = gpu_path(w, q, k, v, dev)
    k_ = w.topk
    nqb = ssa.n_blocks(w.seq_q, B)
    idx = g["idx"].numpy()
    # all scores tie exactly -> blocks 0..k-2 plus the diagonal, for every row
    s = g["scores"].numpy()
    for i in range(k_, nqb):
        assert np.all(s[:, :, i, :i] == s[:, :, i, :1])
    want = np.array([list(range(i + 1)) + [-1] * (k_ - i - 1) if i + 1 <= k_ else list(range(k_ - 1)) + [i]
                     for i in range(nqb)])
    assert np.array_equal(idx, np.broadcast_to(want, idx.shape))
    # uniform softmax: closed forms at every row
    r = np.arange(w.seq_q)
    blk = r // B
    kept = np.where(blk < k_, r + 1, (k_ - 1) * B + (r - blk * B + 1))
    P.check_abs(g["dm"], np.broadcast_to(1 - kept / (r + 1), g["dm"].shape), P.DROP_ABS, "dropped closed form")
    vn = v.double()
    csum = torch.cumsum(vn, dim=2)
    mean_full = csum / torch.arange(1, w.seq_q + 1, dtype=torch.float64)[:, None]
    P.check_close_outputs(g["of"], mean_full.repeat_interleave(w.n_q_heads // w.n_kv_heads, dim=1), "O_full closed form")
    # sparse: keys of blocks 0..k-2 plus the causal part of the row's own block
    pre = csum[:, :, (k_ - 1) * B - 1]                                  # sum over the first k-1 blocks
    blk_start = torch.from_numpy((blk * B).astype(np.int64))
    before = torch.where(blk_start[None, None, :, None] > 0,
                         csum[:, :, (blk_start - 1).clamp(min=0)], torch.zeros_like(csum))
    num = torch.where(torch.from_numpy(blk < k_)[None, None, :, None], csum, pre[:, :, None, :] + csum - before)
    mean_sp = num / torch.from_numpy(kept.astype(np.float64))[:, None]
    P.check_close_outputs(g["o"], mean_sp.repeat_interleave(w.n_q_heads // w.n_kv_heads, dim=1), "O_sparse closed form")
    # and every row of batch row 0 against the oracle
    check_every_row(w, g, q, k, v, batches=[0], heads=list(range(w.n_q_heads)))


def test_extrap_32k_full_size(dev):
    w = W.EXTRAP_32K
    g = check_full_size(w, dev, nrows=64)
    # every sparse row and every row of the full slice, four heads of each KV group
    q, k, v = W.make_inputs(w)
    check_every_row(w, g, q, k, v, batches=[0], heads=[0, 5, 10, 15, 16, 21, 26, 31])


def test_decode_32k_full_size(dev):
    w = W.DECODE_32K
    say(w)
    q, k, v = W.make_inputs(w)
    g = gpu_path(w, q, k, v, dev, with_full=False)
    # every sequence, eight at a time (the fp64 copies of one chunk's cache are 0.5 GB)
    for s0 in range(0, w.batch, 8):
        sub = list(range(s0, min(s0 + 8, w.batch)))
        qn, kn, vn = q[sub].double().numpy(), k[sub].double().numpy(), v[sub].double().numpy()
        ks_ref = O.key_summaries(kn, B)
        assert np.array_equal(P.np64(g["k_summary"][sub]), ks_ref)
        s_ref = O.block_scores(qn, None, B, q_offset=w.q_offset, k_summary=ks_ref)
        idx_ref = O.select_blocks(s_ref, w.topk, B, q_offset=w.q_offset)
        P.check_indices(g["idx"][sub], s_ref, idx_ref, w.topk, B, w.q_offset)
        o_ref, lse_ref = O.sparse_attention(qn, kn, vn, g["idx"][sub].numpy(), B, q_offset=w.q_offset)
        P.check_close_outputs(g["o"][sub], o_ref, f"O_decode sequences {sub[0]}..{sub[-1]}")
        P.check_abs(g["lse"][sub], lse_ref, P.LSE_ABS, f"LSE_decode sequences {sub[0]}..{sub[-1]}")
        del qn, kn, vn
    # every sequence: the forced block is the most recent one
    assert torch.all(g["idx"][..., -1] == (w.seq_kv - 1) // B)


# ----------------------------------------------------------------------------- group-shared selection

SHARED_SMALL = [W.TINY_512, SMALL[2], SMALL[4], SMALL[6], SMALL[7], SMALL[8]]


@pytest.mark.parametrize("w", SHARED_SMALL, ids=lambda w: w.name)
def test_small_parity_shared(dev, w):
    g = check_small(w, dev, shared=True)
    assert g["idx"].shape[1] == w.n_kv_heads


@pytest.mark.parametrize("w", DECODE_SMALL[:3], ids=lambda w: w.name)
def test_decode_parity_shared(dev, w):
    check_small(w, dev, shared=True)


def test_shared_one_head_per_group_matches_per_head(dev):
    # with one query head per KV head the shared entry points are the per-head ones
    w = W.Workload("mha_shared", 2, 4, 4, 512, 512, 64, 64, 3, seed=41)
    say(w)
    q, k, v = W.make_inputs(w)
    a = gpu_path(w, q, k, v, dev)
    b = gpu_path(w, q, k, v, dev, shared=True)
    for key in ("idx", "o", "lse", "of", "lf", "dm"):
        assert torch.equal(a[key], b[key]), key


def test_prefill_8k_shared_full_size(dev):
    w = W.PREFILL_8K
    g = check_full_size(w, dev, nrows=64, shared=True)
    assert torch.all(g["dm"][:, :, : w.topk * B] == 0)
    q, k, v = W.make_inputs(w)
    check_every_row(w, g, q, k, v, batches=[0], heads=list(range(w.n_q_heads)), shared=True)


def test_decode_32k_shared_full_size(dev):
    w = W.DECODE_32K
    say(f"{w} shared=True")
    q, k, v = W.make_inputs(w)
    g = gpu_path(w, q, k, v, dev, with_full=False, shared=True)
    sub = [0, 17, 63]
    qn, kn, vn = q[sub].double().numpy(), k[sub].double().numpy(), v[sub].double().numpy()
    ks_ref = O.key_summaries(kn, B)
    s_ref = O.block_scores(qn, None, B, q_offset=w.q_offset, k_summary=ks_ref)
    sel_scores, idx_ref = reference_selection(s_ref, w, True)
    P.check_indices(g["idx"][sub], sel_scores, idx_ref, w.topk, B, w.q_offset)
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, per_head(g["idx"][sub].numpy(), w, True), B, q_offset=w.q_offset)
    P.check_close_outputs(g["o"][sub], o_ref, "O_decode shared")
    P.check_abs(g["lse"][sub], lse_ref, P.LSE_ABS, "LSE_decode shared")


# ----------------------------------------------------------------------------- early stopping

def check_early_stop(w: W.Workload, taus, dev, heads=None):
    """GPU early stopping vs the oracle.  The oracle orders the blocks with the
    GPU's own (checked) scores and index lists; the number of visited blocks
    must match except where the deciding ratio lies within 1e-3 of tau, and
    the outputs must match the oracle evaluated with the GPU's counts."""
    q, k, v = W.make_inputs(w)
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    scores, _ = ssa.ssa_block_scores(shape, qd, kd)
    idx = ssa.ssa_select_topk(shape, scores)
    o_all, l_all = ssa.ssa_block_sparse_attn_fwd(shape, qd, kd, vd, idx)
    hs = list(range(w.n_q_heads)) if heads is None else heads
    G = w.n_q_heads // w.n_kv_heads
    qn = q[:, hs].double().numpy()
    kn, vn = k.double().numpy(), v.double().numpy()
    # the oracle takes K/V per query head here (head h -> its KV head)
    kn = np.stack([kn[:, h // G] for h in hs], axis=1)
    vn = np.stack([vn[:, h // G] for h in hs], axis=1)
    s_g = P.np64(scores.cpu())[:, hs]
    i_g = idx.cpu().numpy()[:, hs]
    for tau in taus:
        say(f"{w.name} early stop tau={tau}")
        o, lse, used = ssa.ssa_block_sparse_attn_fwd_early_stop(shape, qd, kd, vd, scores, idx, tau)
        torch.cuda.synchronize()
        used_g = used.cpu().numpy()[:, hs]
        _, _, used_ref, ratio = O.early_stop_attention(qn, kn, vn, s_g, i_g, tau, B, q_offset=w.q_offset)
        for bi, hh, i in np.argwhere(used_g != used_ref):
            t = min(used_g[bi, hh, i], used_ref[bi, hh, i]) - 1      # the decision the two sides took differently
            r = ratio[bi, hh, i, t]
            assert abs(r - tau) <= 1e-3 * tau, (w.name, tau, (bi, hh, i), used_g[bi, hh, i], used_ref[bi, hh, i], r)
        o_ref, lse_ref, _, _ = O.early_stop_attention(qn, kn, vn, s_g, i_g, tau, B, q_offset=w.q_offset,
                                                       used=used_g)
        P.check_close_outputs(o[:, hs].cpu(), o_ref, f"O early stop tau={tau}")
        P.check_abs(lse[:, hs].cpu(), lse_ref, P.LSE_ABS, f"LSE early stop tau={tau}")
        if tau == 0.0:
            assert np.array_equal(used_g, (i_g >= 0).sum(-1))
            P.check_close_outputs(o.cpu(), o_all.cpu(), "tau=0 vs block-sparse forward")
        if tau >= 1.0:  # the rule must actually stop somewhere on these inputs
            assert used_g.sum() < (i_g >= 0).sum()
        print(f"[case] {w.name} tau={tau}: mean blocks visited {used_g.mean():.2f} of {(i_g >= 0).sum(-1).mean():.2f}",
              flush=True)


EARLY_STOP = [
    (W.Workload("es_gqa8_2k", 1, 8, 2, 2048, 2048, 64, 64, 8, seed=51), [0.0, 0.05, 0.2, 1.0]),
    (W.Workload("es_ragged_1000", 2, 4, 2, 1000, 1000, 64, 64, 5, seed=52), [0.0, 0.1, 2.0]),
    (W.Workload("es_planted_2k", 1, 8, 2, 2048, 2048, 64, 64, 6, seed=53, variant="planted"), [0.02, 0.3, 1.0]),
    (W.Workload("es_chunked", 1, 4, 2, 192, 320, 64, 64, 3, seed=54), [0.1, 1e30]),
]


@pytest.mark.parametrize("case", EARLY_STOP, ids=lambda c: c[0].name)
def test_early_stop_parity(dev, case):
    check_early_stop(case[0], case[1], dev)


def test_early_stop_prefill_8k(dev):
    check_early_stop(W.PREFILL_8K, [0.05, 1.0], dev, heads=[0, 17])


def test_work_queue_reuse_and_static_grid(dev):
    """The persistent prefill launches take units from a work queue in the
    caller's workspace and leave it zeroed: one workspace serves call after
    call, and the results equal those of the one-workgroup-per-unit grid
    (used when no workspace is given) bit for bit.  prefill_8k has more units
    than resident workgroups, so waves take several units each."""
    w = W.BY_NAME["prefill_8k"]
    say(f"work queue reuse on {w.name}")
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    scores, _ = ssa.ssa_block_scores(shape, q, k)
    idx = ssa.ssa_select_topk(shape, scores)
    none = torch.zeros((0,), dtype=torch.uint8, device=dev)  # too small: static grid
    o0, l0 = ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=none)
    of0, lf0, d0 = ssa.ssa_full_attn_fwd_dropped_mass(shape, q, k, v, idx, workspace=none)
    ws = torch.zeros((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD),), dtype=torch.uint8, device=dev)
    wsf = torch.zeros((ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_FULL_FWD),), dtype=torch.uint8, device=dev)
    for rep in range(3):
        o, l = ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=ws)
        of, lf, d = ssa.ssa_full_attn_fwd_dropped_mass(shape, q, k, v, idx, workspace=wsf)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0 and int(wsf.count_nonzero()) == 0, f"queue not zeroed after call {rep}"
        assert torch.equal(o, o0) and torch.equal(l, l0), f"sparse forward differs from the static grid (call {rep})"
        assert torch.equal(of, of0) and torch.equal(lf, lf0) and torch.equal(d, d0), \
            f"full counterpart differs from the static grid (call {rep})"


@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
def test_index_rows_read_as_sets(dev, shared):
    """An index row names a set of blocks: rows shuffled, with a -1 in the
    middle and a block listed twice, give the results of the ascending rows
    bit for bit in the block-sparse forward, the full counterpart's dropped
    mass and the backward (the kernels put every row in ascending order
    first); and both match the oracle."""
    w = W.TINY_512.scaled(n_q_heads=8, n_kv_heads=2, seq_q=1000, seq_kv=1000, topk=5)
    say(f"scrambled index rows, {w.seq_q} rows, topk {w.topk}, shared={shared}")
    q, k, v = W.make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    shape = ssa.make_shape(qd, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    scores, _ = ssa.ssa_block_scores(shape, qd, kd)
    idx = (ssa.ssa_select_topk_shared if shared else ssa.ssa_select_topk)(shape, scores)
    rng = np.random.default_rng(77)
    src = idx.cpu().numpy()
    scr = np.full(src.shape[:-1] + (w.topk + 2,), -1, dtype=np.int32)
    for pos in np.ndindex(*src.shape[:-1]):
        lst = list(rng.permutation([int(j) for j in src[pos] if j >= 0]))
        row = lst[: len(lst) // 2] + [-1] + lst[len(lst) // 2:] + lst[:1]
        scr[pos][: len(row)] = row
    shape2 = ssa.make_shape(qd, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk + 2)
    scr_d = torch.from_numpy(scr).to(dev)
    o0, l0 = ssa.ssa_block_sparse_attn_fwd(shape, qd, kd, vd, idx, shared=shared)
    o1, l1 = ssa.ssa_block_sparse_attn_fwd(shape2, qd, kd, vd, scr_d, shared=shared)
    _, _, d0 = ssa.ssa_full_attn_fwd_dropped_mass(shape, qd, kd, vd, idx, shared=shared)
    _, _, d1 = ssa.ssa_full_attn_fwd_dropped_mass(shape2, qd, kd, vd, scr_d, shared=shared)
    dout = W.make_output_grad(w, device=dev)
    g0 = ssa.ssa_block_sparse_attn_bwd(shape, qd, kd, vd, idx, o0, l0, dout, shared=shared)
    g1 = ssa.ssa_block_sparse_attn_bwd(shape2, qd, kd, vd, scr_d, o0, l0, dout, shared=shared)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0), "sparse forward depends on the order of the index row"
    assert torch.equal(d1, d0), "dropped mass depends on the order of the index row"
    for a0, a1, name in zip(g0, g1, ("dq", "dk", "dv")):
        assert torch.equal(a1, a0), f"{name} depends on the order of the index row"
    # and the scrambled rows against the oracle (which reads rows as sets too)
    per_head = scr if not shared else np.repeat(scr, w.n_q_heads // w.n_kv_heads, axis=1)
    qn, kn, vn = np_inputs(q, k, v)
    o_ref, l_ref = O.sparse_attention(qn, kn, vn, per_head, w.block)
    P.check_close_outputs(o1, o_ref, "O_sparse (scrambled rows)")
    P.check_abs(l1, l_ref, P.LSE_ABS, "LSE_sparse (scrambled rows)")
    _, _, d_ref = O.full_attention_dropped_mass(qn, kn, vn, per_head, w.block)
    P.check_abs(d1, d_ref, P.DROP_ABS, "dropped mass (scrambled rows)")


def test_workgroup_timing_records(dev):
    """The timing records a persistent launch writes past its work queue are
    consistent with the launch: one per workgroup, every unit and every tile
    of the selection counted once, end after start, and the outputs equal
    those of a launch without records."""
    from block_sparse_attention_kv_amd.profiling import TRACE_WORDS, trace_summary
    w = W.Workload("trace_2k", 2, 8, 2, 2048, 2048, 64, 64, 6, seed=61)
    say(f"{w.name}: timing records of the sparse and full forward")
    q, k, v = (t.to(dev) for t in W.make_inputs(w))
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    scores, _ = ssa.ssa_block_scores(shape, q, k)
    idx = ssa.ssa_select_topk(shape, scores)
    qbytes = ssa.ssa_workspace_bytes(shape, ssa.SSA_OP_SPARSE_FWD)
    ws = torch.zeros((qbytes + 4096 * TRACE_WORDS * 4,), dtype=torch.uint8, device=dev)
    o1, l1 = ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx, workspace=ws)
    o2, l2 = ssa.ssa_block_sparse_attn_fwd(shape, q, k, v, idx)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rec = ws[qbytes:].view(torch.int32).cpu().numpy().view(np.uint32).reshape(-1, TRACE_WORDS)
    used = rec[rec[:, 4] > 0]
    nqb = ssa.n_blocks(w.seq_q, B)
    assert int(used[:, 4].sum()) == w.batch * w.n_q_heads * nqb           # every unit once
    listed = int((idx >= 0).sum())                                       # the kernels visit every listed block
    assert int(used[:, 5].sum()) == listed
    s = trace_summary(rec)
    assert s["workgroups"] == len(used) and s["span_us"] > 0 and s["busy_fraction"] <= 1.0
    assert 0.5 < s["clock_ghz_p0_10_50_90_100"][2] < 3.0
    # full counterpart: tiles = every causal block of every query block, per group of 4 heads
    wsf = torch.zeros_like(ws)
    ssa.ssa_full_attn_fwd_dropped_mass(shape, q, k, v, idx, workspace=wsf)
    torch.cuda.synchronize()
    recf = wsf[qbytes:].view(torch.int32).cpu().numpy().view(np.uint32).reshape(-1, TRACE_WORDS)
    usedf = recf[recf[:, 4] > 0]
    assert int(usedf[:, 4].sum()) == w.batch * w.n_q_heads * nqb // 4
    assert int(usedf[:, 5].sum()) == w.batch * w.n_q_heads // 4 * sum(i + 1 for i in range(nqb))
