"""GPU parity of the DashAttention-style entry points (learned-query chunk
summaries, alpha-entmax routing, prior-biased block-sparse forward) against
the fp64 oracle on the same seeded inputs.

Routing is compared on the GPU's own fp32 scores (the scores themselves are
checked against the oracle first); the biased forward is compared against the
oracle evaluated with the GPU's own lists and biases, so a support decision
taken differently at the threshold cannot masquerade as an attention error."""
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
W_ABS = 1e-5          # routing weights: fp32 Newton iterations from below and fp32 sums
SUMMARY_ULPS = 2      # learned summaries: fp64 on both sides, one fp32 rounding


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


def check_support(idx_gpu, w_ref, topk, q_offset):
    """The GPU lists against routing_support(w_ref): identical except for blocks
    whose reference weight is within W_ABS of the support threshold (0) or of
    the cap boundary.  Returns the mean list length."""
    idx_ref = O.routing_support(w_ref, topk, B, q_offset=q_offset)
    g = np.asarray(idx_gpu)
    b, hkv, nqb, _ = g.shape
    lens = []
    for bi in range(b):
        for gg in range(hkv):
            for i in range(nqb):
                jd = (q_offset + i * B) // B
                row = [int(j) for j in g[bi, gg, i] if j >= 0]
                lens.append(len(row))
                assert row == sorted(set(row)) and jd in row and all(0 <= j <= jd for j in row), (bi, gg, i, row)
                assert all(j == -1 for j in g[bi, gg, i, len(row):])
                ref = [int(j) for j in idx_ref[bi, gg, i] if j >= 0]
                diff = set(row) ^ set(ref)
                if not diff:
                    continue
                wr = w_ref[bi, gg, i]
                live = sorted((wr[j] for j in range(jd) if wr[j] > 0), reverse=True)
                cap = live[topk - 2] if 1 < topk <= len(live) else None
                for j in diff:
                    near_zero = wr[j] <= W_ABS
                    near_cap = cap is not None and abs(wr[j] - cap) <= W_ABS
                    assert near_zero or near_cap, f"row {(bi, gg, i)}: block {j} (w={wr[j]:.3e}) differs"
    return float(np.mean(lens))


def dash_path(w, dev, alpha, gamma, sigma, qscale=1.0):
    q, k, v = W.make_inputs(w)
    qbar = W.make_learned_query(w, qscale)
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ks = ssa.ssa_block_summaries_learned(kd, qbar.to(dev))
    scores, _ = ssa.ssa_block_scores(shape, qd, None, ks)
    idx, bias, wts = ssa.ssa_entmax_route(shape, scores, alpha, gamma, sigma)
    o, lse = ssa.ssa_block_sparse_attn_fwd_biased(shape, qd, kd, vd, idx, bias)
    torch.cuda.synchronize()
    return (q, k, v, qbar), {n: t.cpu() for n, t in dict(ks=ks, scores=scores, idx=idx, bias=bias, w=wts, o=o,
                                                          lse=lse).items()}


def check_dash(w, dev, alpha, gamma, sigma):
    say(f"{w.name} alpha={alpha} gamma={gamma} sigma={sigma} topk={w.topk}")
    (q, k, v, qbar), g = dash_path(w, dev, alpha, gamma, sigma)
    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    off = w.q_offset
    # stage 0: learned summaries
    ks_ref = O.learned_key_summaries(kn, qbar.double().numpy(), B)
    ks = np64(g["ks"])
    assert np.all(np.abs(ks - ks_ref) <= SUMMARY_ULPS * np.spacing(np.abs(ks_ref).astype(np.float32)).astype(np.float64)
                  + 1e-30), "learned summaries"
    # scores from those summaries
    s_ref = O.block_scores(qn, kn, B, q_offset=off, k_summary=ks)
    s_gpu = np64(g["scores"])
    fin = np.isfinite(s_ref)
    assert np.array_equal(np.isfinite(s_gpu), fin)
    assert np.all(np.abs(s_gpu[fin] - s_ref[fin]) <= 1e-6 * np.maximum(np.abs(s_ref[fin]), 1e-3))
    # stage 1: routing on the GPU's scores
    w_ref = O.entmax_routing(s_gpu, w.n_kv_heads, alpha, gamma, B, q_offset=off)
    wg = np64(g["w"])
    err = float(np.abs(wg - w_ref).max())
    assert err <= W_ABS, f"routing weights: max |diff| {err:.3e}"
    mean_len = check_support(g["idx"].numpy(), w_ref, w.topk, off)
    idx = g["idx"].numpy()
    bias = np64(g["bias"])
    bias_ref = O.prior_bias(wg, idx, sigma, B, q_offset=off)   # the rule applied to the GPU's own weights
    live = bias_ref != 0
    assert np.all(np.abs(bias[live] - bias_ref[live]) <= 1e-5 * np.maximum(1.0, np.abs(bias_ref[live])))
    assert np.all(bias[~live] == 0)
    # stage 2: the biased forward against the oracle with the GPU's lists and biases
    o_ref, lse_ref = O.prior_attention(qn, kn, vn, idx, bias, B, q_offset=off)
    P.check_close_outputs(g["o"], o_ref, "O_prior")
    P.check_abs(g["lse"], lse_ref, P.LSE_ABS, "LSE_prior")
    print(f"  mean list length {mean_len:.2f}, routing max |dw| {err:.2e}", flush=True)
    return mean_len


CASES = [
    (W.Workload("dash_tiny_512", 1, 2, 1, 512, 512, 64, 64, 8, seed=41), 1.5, 200.0, 1.0),
    (W.Workload("dash_ragged_1000", 1, 6, 2, 1000, 1000, 64, 64, 16, seed=42), 2.0, 300.0, 0.5),
    (W.Workload("dash_gqa16_2k", 1, 32, 2, 2048, 2048, 64, 64, 32, seed=43), 1.5, 800.0, 1.0),
    (W.Workload("dash_gqa16_2k_cap", 1, 32, 2, 2048, 2048, 64, 64, 6, seed=44), 1.5, 800.0, 1.0),   # cap binds
    (W.Workload("dash_alpha125", 2, 8, 2, 1024, 1024, 64, 64, 16, seed=45), 1.25, 400.0, 2.0),
    (W.Workload("dash_sigma0", 1, 8, 1, 768, 768, 64, 64, 12, seed=46), 1.5, 200.0, 0.0),
    (W.Workload("dash_chunked", 1, 8, 2, 320, 640, 64, 64, 8, seed=47), 1.5, 300.0, 1.0),
    (W.Workload("dash_g3", 1, 6, 2, 640, 640, 64, 64, 10, seed=48), 2.0, 100.0, 1.0),
    # decode: one query token per sequence against a cache (ragged last block)
    (W.Workload("dash_decode_4133", 4, 32, 2, 1, 4133, 64, 64, 17, seed=52), 1.5, 800.0, 1.0),
    (W.Workload("dash_decode_g8_cap", 3, 16, 2, 1, 2048, 64, 64, 6, seed=53), 2.0, 400.0, 0.5),
    (W.Workload("dash_decode_32k", 8, 32, 2, 1, 32768, 64, 64, 64, seed=54), 1.5, 800.0, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_dash_parity(dev, case):
    w, alpha, gamma, sigma = case
    check_dash(w, dev, alpha, gamma, sigma)


def test_zero_learned_query_is_the_mean(dev):
    w = W.Workload("dash_zero_q", 2, 4, 2, 300, 300, 64, 64, 4, seed=49)
    say(w.name)
    _, k, _ = W.make_inputs(w)
    kd = k.to(dev)
    a = ssa.ssa_block_summaries_learned(kd, torch.zeros((2, 64), device=dev))
    b = ssa.ssa_block_summaries(kd)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), b.cpu())


def test_bias_shift_invariance(dev):
    """One constant added to every bias of a list leaves O and shifts LSE."""
    w = W.Workload("dash_shift", 1, 8, 2, 512, 512, 64, 64, 8, seed=50)
    say(w.name)
    (q, k, v, qbar), g = dash_path(w, dev, 1.5, 200.0, 1.0)
    shape = ssa.make_shape(q, 2, 512, topk=8)
    idx = g["idx"].to(dev)
    bias = g["bias"].to(dev)
    shifted = torch.where(idx >= 0, bias + 0.75, bias)
    o2, l2 = ssa.ssa_block_sparse_attn_fwd_biased(shape, q.to(dev), k.to(dev), v.to(dev), idx, shifted)
    torch.cuda.synchronize()
    P.check_close_outputs(o2.cpu(), np64(g["o"]), "O shifted")
    P.check_abs(l2.cpu(), np64(g["lse"]) + 0.75, P.LSE_ABS, "LSE shifted")


def test_dash_prefill_8k(dev):
    """Full-size workload: stages 0 and 1 everywhere, the forward on sampled rows."""
    w = W.PREFILL_8K.scaled(topk=64)
    alpha, gamma, sigma = 1.5, 800.0, 1.0
    say(f"{w.name} topk=64")
    (q, k, v, qbar), g = dash_path(w, dev, alpha, gamma, sigma)
    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ks_ref = O.learned_key_summaries(kn, qbar.double().numpy(), B)
    ks = np64(g["ks"])
    assert np.all(np.abs(ks - ks_ref) <= SUMMARY_ULPS * np.spacing(np.abs(ks_ref).astype(np.float32)).astype(np.float64)
                  + 1e-30)
    s_gpu = np64(g["scores"])
    w_ref = O.entmax_routing(s_gpu, 2, alpha, gamma, B)
    assert float(np.abs(np64(g["w"]) - w_ref).max()) <= W_ABS
    mean_len = check_support(g["idx"].numpy(), w_ref, w.topk, 0)
    print(f"  mean list length {mean_len:.2f}", flush=True)
    idx, bias = g["idx"].numpy(), np64(g["bias"])
    rng = np.random.default_rng(51)
    for h in (0, 17):
        for i in sorted(set(rng.integers(0, 128, 6).tolist()) | {127}):
            rows = slice(i * B, (i + 1) * B)
            sub_q = qn[:, h:h + 1, rows]
            # the query block's rows alone, against every key up to its diagonal
            o_ref, lse_ref = O.prior_attention(
                np.concatenate([np.zeros((1, 1, i * B, 64)), sub_q], axis=2), kn[:, h // 16:h // 16 + 1, :(i + 1) * B],
                vn[:, h // 16:h // 16 + 1, :(i + 1) * B], idx[:, h // 16:h // 16 + 1, :i + 1],
                bias[:, h // 16:h // 16 + 1, :i + 1], B)
            P.check_close_outputs(g["o"][:, h:h + 1, rows], o_ref[:, :, i * B:], f"O_prior h{h} i{i}")
            P.check_abs(g["lse"][:, h:h + 1, rows], lse_ref[:, :, i * B:], P.LSE_ABS, f"LSE_prior h{h} i{i}")


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[8]], ids=lambda c: c[0].name)
def test_minus_inf_bias(dev, case):
    """A listed block whose bias is -inf (a prior weight of 0) contributes
    nothing, also when it is the first block a row visits (the diagonal, or the
    first of a decode slice): the biased forward stays finite and matches the
    oracle.  Every other row's diagonal bias is set to -inf, and the first
    other listed block of every third row; each row keeps a finite block."""
    w, alpha, gamma, sigma = case
    say(f"{w.name}: -inf biases on listed blocks")
    q, k, v = W.make_inputs(w)
    qbar = W.make_learned_query(w)
    shape = ssa.make_shape(q, w.n_kv_heads, w.seq_kv, block=w.block, topk=w.topk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ks = ssa.ssa_block_summaries_learned(kd, qbar.to(dev))
    scores, _ = ssa.ssa_block_scores(shape, qd, None, ks)
    idx, bias, _ = ssa.ssa_entmax_route(shape, scores, alpha, gamma, sigma, with_weights=False)
    idx_n, bias_n = idx.cpu().numpy(), bias.cpu().numpy().astype(np.float32)
    nrow = 0
    for pos in np.ndindex(*idx_n.shape[:-1]):
        listed = [e for e in range(idx_n.shape[-1]) if idx_n[pos][e] >= 0]
        if len(listed) < 2:
            continue
        if nrow % 2 == 0:
            bias_n[pos][listed[-1]] = -np.inf          # the diagonal (listed last, visited first)
        if nrow % 3 == 0 and (len(listed) > 2 or nrow % 2 == 1):
            bias_n[pos][listed[0]] = -np.inf           # the first other block (one listed block stays finite)
        nrow += 1
    assert nrow > 0
    assert np.all(np.any(np.isfinite(bias_n) & (idx_n >= 0), axis=-1) | (idx_n < 0).all(-1))
    o, lse = ssa.ssa_block_sparse_attn_fwd_biased(shape, qd, kd, vd, idx, torch.from_numpy(bias_n).to(dev))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all(), "-inf bias produced non-finite outputs"
    o_ref, lse_ref = O.prior_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), idx_n,
                                       bias_n.astype(np.float64), B, q_offset=w.q_offset)
    P.check_close_outputs(o, o_ref, "O_prior with -inf biases")
    P.check_abs(lse, lse_ref, P.LSE_ABS, "LSE_prior with -inf biases")
