"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself: a hand-worked
example, closed forms, PyTorch library routines (SDPA, logsumexp, avg_pool1d,
matmul), brute-force enumeration on tiny inputs, and identities the
mathematics fixes.  Each ``check_*`` takes the oracle module so the mutation
tests at the bottom can show that a planted mistake in the oracle fails at
least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ssa_oracle
from tests import torch_reference as tr

RNG = np.random.default_rng(20261203)


def bf16_values(shape, rng=RNG, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16).to(torch.float64).numpy()


def rand_qkv(b, hq, hkv, n, d, rng=RNG):
    return bf16_values((b, hq, n, d), rng), bf16_values((b, hkv, n, d), rng), bf16_values((b, hkv, n, d), rng)


# ----------------------------------------------------------------------------- checks

def check_hand_example(O, golden_dir):
    with open(os.path.join(golden_dir, "hand_example.json")) as f:
        g = json.load(f)
    B, k, sc = g["block"], g["topk"], g["scale"]
    q = np.array(g["q"], float)[None, None]
    kk = np.array(g["k"], float)[None, None]
    v = np.array(g["v"], float)[None, None]
    ks = O.key_summaries(kk, B)
    assert np.array_equal(ks[0, 0], np.array(g["k_summary"], float))
    s = O.block_scores(q, kk, B, scale=sc)
    exp_s = np.array([[np.inf * -1 if x is None else x for x in row] for row in g["scores"]])
    assert np.array_equal(s[0, 0], exp_s)
    idx = O.select_blocks(s, k, B)
    assert np.array_equal(idx[0, 0], np.array(g["idx"]))
    o_sp, lse_sp = O.sparse_attention(q, kk, v, idx, B, scale=sc)
    o_f, lse_f, dm = O.full_attention_dropped_mass(q, kk, v, idx, B, scale=sc)
    r5 = g["row5"]
    w = np.exp(np.array(r5["sparse_logits"]))
    vs = v[0, 0, r5["sparse_keys"]]
    np.testing.assert_allclose(o_sp[0, 0, 5], (w[:, None] * vs).sum(0) / w.sum(), rtol=1e-14)
    np.testing.assert_allclose(lse_sp[0, 0, 5], math.log(w.sum()), rtol=1e-14)
    wf = np.exp(np.array(r5["full_logits"]))
    vf = v[0, 0, r5["full_keys"]]
    np.testing.assert_allclose(o_f[0, 0, 5], (wf[:, None] * vf).sum(0) / wf.sum(), rtol=1e-14)
    dropped = [r5["full_keys"].index(c) for c in r5["dropped_keys"]]
    np.testing.assert_allclose(dm[0, 0, 5], wf[dropped].sum() / wf.sum(), rtol=1e-14)


def check_block_means(O):
    # library: avg_pool1d (ceil mode averages the rows a partial window has)
    for n, B in [(256, 64), (200, 64), (37, 8), (5, 5), (1, 64)]:
        x = bf16_values((2, 3, n, 4))
        np.testing.assert_allclose(O.block_means(x, B), tr.avg_pool_blocks(x, B), rtol=1e-14, atol=0)
    # closed form: row c holds the value c  ->  block j mean = midpoint of its rows
    n, B = 13, 4
    x = np.repeat(np.arange(n, dtype=float)[:, None], 3, axis=1)[None, None]
    got = O.block_means(x, B)[0, 0, :, 0]
    want = [(j * B + min((j + 1) * B, n) - 1) / 2 for j in range(-(-n // B))]
    assert np.array_equal(got, np.array(want))
    # a constant block is its own mean, exactly
    row = bf16_values((1, 1, 1, 64))
    assert np.array_equal(O.block_means(np.repeat(row, 64, axis=2), 64), row)


def check_scores_token_level(O):
    # block size 1: block scores are the token logits fp32(scale * q_r . k_c) for c <= r
    b, hq, hkv, n, d = 1, 4, 2, 24, 16
    q, k, _ = rand_qkv(b, hq, hkv, n, d)
    sc = 0.3
    s = O.block_scores(q, k, 1, scale=sc)
    kk = torch.from_numpy(k).double().repeat_interleave(hq // hkv, dim=1)
    logits = (torch.matmul(torch.from_numpy(q).double(), kk.transpose(-1, -2)) * float(np.float32(sc)))
    want = logits.to(torch.float32).double().numpy()
    want = np.where(np.tril(np.ones((n, n), bool))[None, None], want, -np.inf)
    assert np.array_equal(s, want)


def check_scores_gqa_and_causal(O):
    # KV head g holds rows (g+1)*e0; every query row is e0  ->  s = scale*(g(h)+1) on causal blocks
    b, hq, hkv, n, d, B = 2, 6, 3, 48, 8, 16
    q = np.zeros((b, hq, n, d)); q[..., 0] = 1
    k = np.zeros((b, hkv, n, d))
    for g in range(hkv):
        k[:, g, :, 0] = g + 1
    s = O.block_scores(q, k, B, scale=0.5)
    for h in range(hq):
        g = h // (hq // hkv)
        for i in range(n // B):
            assert np.all(s[:, h, i, : i + 1] == 0.5 * (g + 1))
            assert np.all(np.isneginf(s[:, h, i, i + 1:]))


def _brute_top(scores_row, cands, m):
    """The unique m-subset T of cands such that every member outranks every
    non-member under (higher score, then lower index); NaN ranks lowest."""
    def beats(a, c):
        sa, sb = scores_row[a], scores_row[c]
        if math.isnan(sb) and not math.isnan(sa):
            return True
        if math.isnan(sa):
            return math.isnan(sb) and a < c
        return sa > sb or (sa == sb and a < c)
    found = [set(T) for T in itertools.combinations(cands, m)
             if all(beats(t, u) for t in T for u in cands if u not in T)]
    assert len(found) == 1
    return found[0]


def check_select_brute_force(O):
    rng = np.random.default_rng(7)
    nqb, k, B = 9, 4, 4
    for trial in range(40):
        s = np.round(rng.standard_normal((1, 2, nqb, nqb)), 1)  # coarse values force exact ties
        if trial % 5 == 0:
            s[0, 0, 6, 2] = np.nan
        idx = O.select_blocks(s, k, B)
        for h in range(2):
            for i in range(nqb):
                if i + 1 <= k:
                    want = set(range(i + 1))
                else:
                    want = _brute_top(s[0, h, i], list(range(i)), k - 1) | {i}
                got = [j for j in idx[0, h, i] if j >= 0]
                assert got == sorted(want)
                assert list(idx[0, h, i, len(got):]) == [-1] * (k - len(got))


def check_select_ties_and_decode(O):
    # all scores equal -> blocks 0..k-2 plus the diagonal
    s = np.zeros((1, 1, 10, 10))
    idx = O.select_blocks(s, 4, 64)
    assert list(idx[0, 0, 9]) == [0, 1, 2, 9]
    # decode: one query row at position L-1; the forced block is the one holding it
    L, B = 1000, 64
    row = np.linspace(-1, 1, 16)[None, None, None, :]
    idx = O.select_blocks(row, 5, B, q_offset=L - 1)
    assert (L - 1) // B == 15
    assert list(idx[0, 0, 0]) == [11, 12, 13, 14, 15]


def check_sparse_vs_sdpa(O):
    for (b, hq, hkv, n, d, B, k, q_off) in [(2, 4, 2, 160, 16, 16, 4, 0),   # ragged: 160 = 10 blocks
                                           (1, 3, 1, 100, 8, 16, 3, 0),      # ragged tail block
                                           (1, 2, 2, 64, 8, 8, 2, 0)]:
        q, kk, v = rand_qkv(b, hq, hkv, n, d)
        sc = float(np.float32(1.0 / math.sqrt(d)))   # the scale argument is an fp32 value
        s = O.block_scores(q, kk, B)
        idx = O.select_blocks(s, k, B)
        o, lse = O.sparse_attention(q, kk, v, idx, B)
        mask = tr.block_mask_from_idx(idx, n, n, B, 0)
        o_ref, lse_ref = tr.sdpa(q, kk, v, mask, sc)
        np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
        # per-row evaluation agrees with the blocked evaluation
        rows = [(0, hq - 1, n - 1), (b - 1, 0, 5), (0, 1 % hq, n // 2)]
        o_r, lse_r = O.sparse_attention(q, kk, v, idx, B, rows=rows)
        for t, (bi, h, r) in enumerate(rows):
            np.testing.assert_allclose(o_r[t], o[bi, h, r], rtol=1e-12, atol=1e-13)


def check_sparse_special_cases(O):
    b, hq, hkv, n, d, B = 1, 4, 2, 128, 16, 16
    q, kk, v = rand_qkv(b, hq, hkv, n, d)
    sc = 0.25
    causal = tr.causal_mask(n, n, 0)
    full_ref = tr.sdpa(q, kk, v, causal, sc)
    # k >= number of blocks: sparse == full causal attention, dropped mass == 0
    idx = O.select_blocks(O.block_scores(q, kk, B, scale=sc), n // B, B)
    o, lse = O.sparse_attention(q, kk, v, idx, B, scale=sc)
    np.testing.assert_allclose(o, full_ref[0], rtol=1e-11, atol=1e-12)
    _, _, dm = O.full_attention_dropped_mass(q, kk, v, idx, B, scale=sc)
    assert np.all(dm == 0)
    # B == N: one block, always the diagonal -> full causal attention
    idx1 = O.select_blocks(O.block_scores(q, kk, n, scale=sc), 1, n)
    o1, _ = O.sparse_attention(q, kk, v, idx1, n, scale=sc)
    np.testing.assert_allclose(o1, full_ref[0], rtol=1e-11, atol=1e-12)
    # k == 1: block-diagonal causal attention
    idxd = O.select_blocks(O.block_scores(q, kk, B, scale=sc), 1, B)
    od, _ = O.sparse_attention(q, kk, v, idxd, B, scale=sc)
    blockdiag = torch.block_diag(*[torch.ones(B, B, dtype=torch.bool)] * (n // B)) & causal
    np.testing.assert_allclose(od, tr.sdpa(q, kk, v, blockdiag, sc)[0], rtol=1e-11, atol=1e-12)


def check_sparse_brute_force_loops(O):
    # pure-Python loops over a tiny problem, straight from the definition
    n, d, B, k = 10, 3, 3, 2
    rng = np.random.default_rng(3)
    q, kk, v = rand_qkv(1, 2, 1, n, d, rng)
    sc = 0.7
    idx = O.select_blocks(O.block_scores(q, kk, B, scale=sc), k, B)
    o, lse = O.sparse_attention(q, kk, v, idx, B, scale=sc)
    of, lsef, dm = O.full_attention_dropped_mass(q, kk, v, idx, B, scale=sc)
    scf = float(np.float32(sc))
    for h in range(2):
        for r in range(n):
            sel = [j for j in idx[0, h, r // B] if j >= 0]
            num = [0.0] * d
            den = 0.0
            numf = [0.0] * d
            denf = 0.0
            drop = 0.0
            for c in range(r + 1):
                logit = scf * sum(float(q[0, h, r, t]) * float(kk[0, 0, c, t]) for t in range(d))
                e = math.exp(logit)
                denf += e
                for t in range(d):
                    numf[t] += e * float(v[0, 0, c, t])
                if c // B in sel:
                    den += e
                    for t in range(d):
                        num[t] += e * float(v[0, 0, c, t])
                else:
                    drop += e
            np.testing.assert_allclose(o[0, h, r], np.array(num) / den, rtol=1e-12)
            np.testing.assert_allclose(lse[0, h, r], math.log(den), rtol=1e-12)
            np.testing.assert_allclose(of[0, h, r], np.array(numf) / denf, rtol=1e-12)
            np.testing.assert_allclose(dm[0, h, r], drop / denf, rtol=1e-12, atol=1e-15)


def check_full_and_dropped_identities(O):
    b, hq, hkv, n, d, B, k = 2, 4, 2, 192, 16, 16, 3
    q, kk, v = rand_qkv(b, hq, hkv, n, d)
    sc = 1 / 4
    idx = O.select_blocks(O.block_scores(q, kk, B), k, B)
    o_sp, lse_sp = O.sparse_attention(q, kk, v, idx, B)
    o_f, lse_f, dm = O.full_attention_dropped_mass(q, kk, v, idx, B)
    ref_o, ref_lse = tr.sdpa(q, kk, v, tr.causal_mask(n, n, 0), sc)
    np.testing.assert_allclose(o_f, ref_o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse_f, ref_lse, rtol=1e-12, atol=1e-12)
    # (i) rows of the first k blocks keep every causal key
    assert np.all(dm[:, :, : k * B] == 0)
    # (iv) 0 <= delta < 1
    assert np.all(dm >= 0) and np.all(dm < 1)
    # (ii) delta = 1 - exp(LSE_sparse - LSE_full)
    np.testing.assert_allclose(dm, 1 - np.exp(lse_sp - lse_f), rtol=1e-9, atol=1e-12)
    # (iii) O_full - O_sparse = delta * (O_dropped - O_sparse), O_dropped from SDPA on the complement
    keep = tr.block_mask_from_idx(idx, n, n, B, 0)
    comp = tr.causal_mask(n, n, 0) & ~keep
    rows_with_drop = comp.any(-1)
    comp_safe = comp | ~rows_with_drop[..., None]     # rows without dropped keys: any valid mask
    o_drop = tr.sdpa(q, kk, v, comp_safe, sc)[0]
    lhs = o_f - o_sp
    rhs = dm[..., None] * (o_drop - o_sp)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-8, atol=1e-12)
    # the row-range slice equals the matching rows of the whole
    o_s, lse_s, dm_s = O.full_attention_dropped_mass(q, kk, v, idx, B, row_range=(64, 192))
    np.testing.assert_allclose(o_s, o_f[:, :, 64:], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dm_s, dm[:, :, 64:], rtol=1e-12, atol=1e-15)


def check_tie_closed_form(O):
    # every K row identical -> all logits of a row equal -> uniform softmax
    b, hq, hkv, n, d, B, k = 1, 2, 1, 160, 8, 16, 3
    q, kk, v = rand_qkv(b, hq, hkv, n, d)
    kk = np.repeat(kk[:, :, :1], n, axis=2)
    s = O.block_scores(q, kk, B)
    idx = O.select_blocks(s, k, B)
    o_sp, _ = O.sparse_attention(q, kk, v, idx, B)
    o_f, _, dm = O.full_attention_dropped_mass(q, kk, v, idx, B)
    for i in range(n // B):
        want = list(range(i + 1)) if i + 1 <= k else list(range(k - 1)) + [i]
        assert [j for j in idx[0, 0, i] if j >= 0] == want
    for r in range(n):
        i = r // B
        kept = (r + 1) if i < k else (k - 1) * B + (r - i * B + 1)
        np.testing.assert_allclose(dm[0, 0, r], 1 - kept / (r + 1), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o_f[0, 0, r], v[0, 0, : r + 1].mean(0), rtol=1e-11, atol=1e-13)
        cols = [c for c in range(r + 1) if (c // B) in [j for j in idx[0, 0, i] if j >= 0]]
        np.testing.assert_allclose(o_sp[0, 0, r], v[0, 0, cols].mean(0), rtol=1e-11, atol=1e-13)


def check_decode(O):
    # one query token per (seq, head) at position L-1 against a cache of L keys
    b, hq, hkv, L, d, B, k = 2, 4, 2, 300, 8, 32, 4
    rng = np.random.default_rng(11)
    q = bf16_values((b, hq, 1, d), rng)
    kk, v = bf16_values((b, hkv, L, d), rng), bf16_values((b, hkv, L, d), rng)
    ksum = O.key_summaries(kk, B)
    s = O.block_scores(q, kk, B, q_offset=L - 1)
    s2 = O.block_scores(q, None, B, q_offset=L - 1, k_summary=ksum)
    assert np.array_equal(s, s2)
    jd = (L - 1) // B
    idx = O.select_blocks(s, k, B, q_offset=L - 1)
    o, lse = O.sparse_attention(q, kk, v, idx, B, q_offset=L - 1)
    sc = float(np.float32(1 / math.sqrt(d)))
    for bi in range(b):
        for h in range(hq):
            g = h // 2
            # scores straight from avg_pool1d summaries and a dot product
            kb = tr.avg_pool_blocks(kk[bi, g][None, None], B)[0, 0].astype(np.float32).astype(np.float64)
            logits = (kb @ q[bi, h, 0].astype(np.float64)) * float(np.float32(sc))
            sf = logits.astype(np.float32).astype(np.float64)
            assert np.array_equal(s[bi, h, 0, : jd + 1], sf[: jd + 1])
            want = sorted(_brute_top(sf, list(range(jd)), k - 1) | {jd})
            assert list(idx[bi, h, 0]) == want
    mask = tr.block_mask_from_idx(idx, 1, L, B, L - 1)
    o_ref, lse_ref = tr.sdpa(q, kk, v, mask, sc)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)



def check_shared_hand_example(O):
    # Two query heads share one KV head; four earlier blocks plus the diagonal
    # (block 4), budget 3 = 2 earlier blocks + diagonal.  Worked by hand:
    #   head 0 scores 3.0 1.0 2.0 0.0   -> its own choice {0, 2}
    #   head 1 scores 0.0 2.5 1.0 3.0   -> its own choice {1, 3}
    #   mean          1.5 1.75 1.5 1.5  -> block 1, then the lowest of the
    #                                      three tied at 1.5 (block 0)
    s = np.full((1, 2, 5, 5), -np.inf)
    s[0, 0, 4, :5] = [3.0, 1.0, 2.0, 0.0, 0.5]
    s[0, 1, 4, :5] = [0.0, 2.5, 1.0, 3.0, 0.5]
    for i in range(4):                       # earlier query blocks: any finite values
        s[0, :, i, : i + 1] = 1.0
    own = O.select_blocks(s, 3, 1)
    assert list(own[0, 0, 4]) == [0, 2, 4] and list(own[0, 1, 4]) == [1, 3, 4]
    sh = O.shared_block_scores(s, 1)
    assert list(sh[0, 0, 4]) == [1.5, 1.75, 1.5, 1.5, 0.5]
    assert list(O.select_blocks_shared(s, 1, 3, 1)[0, 0, 4]) == [0, 1, 4]


def check_shared_scores_pool_queries(O):
    # The mean of the heads' scores is the score of the head-averaged block
    # query (the score is linear in the query); pooled independently here.
    q, k, _ = rand_qkv(2, 8, 2, 256, 16)
    s = O.block_scores(q, k, 64)
    sh = O.shared_block_scores(s, 2)
    qt = torch.from_numpy(q)
    qbar = torch.nn.functional.avg_pool1d(qt.reshape(-1, 256, 16).transpose(1, 2), 64).transpose(1, 2)
    qbar = qbar.to(torch.float32).to(torch.float64).reshape(2, 2, 4, 4, 16).mean(dim=2)   # [b, g, nqb, d]
    kbar = torch.nn.functional.avg_pool1d(torch.from_numpy(k).reshape(-1, 256, 16).transpose(1, 2), 64)
    kbar = kbar.transpose(1, 2).to(torch.float32).to(torch.float64).reshape(2, 2, 4, 16)
    ref = (qbar @ kbar.transpose(-1, -2) / 4.0).numpy()
    causal = np.tril(np.ones((4, 4), bool))
    assert np.all(np.isneginf(sh[..., ~causal]))
    np.testing.assert_allclose(sh[..., causal], ref[..., causal], rtol=2e-6, atol=1e-7)


def check_shared_reductions(O):
    # one query head per KV head: the shared selection is the per-head one
    q, k, _ = rand_qkv(1, 3, 3, 512, 8)
    s = O.block_scores(q, k, 64)
    assert np.array_equal(O.shared_block_scores(s, 3), s)
    assert np.array_equal(O.select_blocks_shared(s, 3, 3, 64), O.select_blocks(s, 3, 64))
    # identical query heads within each group: shared == every head's own choice
    q1 = np.repeat(q[:, :1], 4, axis=1)
    k1 = k[:, :1]
    s1 = O.block_scores(q1, k1, 64)
    own = O.select_blocks(s1, 3, 64)
    shared = O.select_blocks_shared(s1, 1, 3, 64)
    assert np.array_equal(O.expand_shared(shared, 4), own)


def check_shared_brute_force(O):
    # the shared choice is the best pair under (group-mean score desc, index
    # asc), found by enumerating every pair
    rng = np.random.default_rng(7)
    s = np.full((1, 3, 6, 6), -np.inf)
    for i in range(6):
        s[0, :, i, : i + 1] = np.round(rng.standard_normal((3, i + 1)), 1)   # many ties
    sel = O.select_blocks_shared(s, 1, 3, 1)
    for i in range(6):
        if i + 1 <= 3:
            assert list(sel[0, 0, i][: i + 1]) == list(range(i + 1))
            continue
        tot = s[0, 0, i, :i] + s[0, 1, i, :i] + s[0, 2, i, :i]
        # the chosen pair is the one whose (fp32 mean desc, index asc) sorted
        # list is smallest: it holds the two best blocks under that order
        best = min(itertools.combinations(range(i), 2),
                   key=lambda comb: sorted((-float(np.float32(tot[j] / 3)), j) for j in comb))
        assert list(sel[0, 0, i]) == sorted(list(best) + [i]), (i, sel[0, 0, i], best)


def check_early_stop_hand_example(O):
    # One head, d = 1, B = 1 (each block is one key), scale 1: logits equal
    # the keys 0, 1, 2, 3.  Query row 3 visits its own block 3 first, then
    # blocks 2, 0, 1 (coarse scores 5, 4, 1).  Worked by hand:
    #   block 2: gain e^2 against e^3            ratio e^-1            = 0.3679
    #   block 0: gain 1 against e^3 + e^2        ratio 1/(e^3 + e^2)   = 0.0367
    #   block 1: gain e against e^3 + e^2 + 1    ratio e/(e^3 + e^2 + 1) = 0.0992
    q = np.ones((1, 1, 4, 1))
    kk = np.array([0.0, 1.0, 2.0, 3.0]).reshape(1, 1, 4, 1)
    v = np.arange(4.0).reshape(1, 1, 4, 1) * 10.0
    sc = np.full((1, 1, 4, 4), -np.inf)
    sc[0, 0, 3, :4] = [4.0, 1.0, 5.0, 0.0]
    for i in range(3):
        sc[0, 0, i, : i + 1] = 0.0
    sel = O.select_blocks(sc, 4, 1)
    e = math.e
    _, _, used, ratio = O.early_stop_attention(q, kk, v, sc, sel, 0.3, 1, scale=1.0)
    np.testing.assert_allclose(ratio[0, 0, 3, 1:], [1 / e, 1 / (e ** 3 + e ** 2), e / (e ** 3 + e ** 2 + 1)], rtol=1e-14)
    assert used[0, 0, 3] == 3                       # stops after block 0, which is kept
    o, lse, used, _ = O.early_stop_attention(q, kk, v, sc, sel, 0.5, 1, scale=1.0)
    assert used[0, 0, 3] == 2                       # stops after block 2
    w = np.array([e ** 3, e ** 2])
    np.testing.assert_allclose(o[0, 0, 3, 0], (w * [30.0, 20.0]).sum() / w.sum(), rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 3], math.log(w.sum()), rtol=1e-14)
    _, _, used, _ = O.early_stop_attention(q, kk, v, sc, sel, 0.03, 1, scale=1.0)
    assert used[0, 0, 3] == 4                       # no ratio below 0.03: every block


def check_early_stop_limits(O):
    q, k, v = rand_qkv(1, 4, 2, 512, 16)
    s = O.block_scores(q, k, 64)
    sel = O.select_blocks(s, 4, 64)
    o_sp, l_sp = O.sparse_attention(q, k, v, sel, 64)
    # tau = 0 never stops: the plain block-sparse forward
    o0, l0, used0, _ = O.early_stop_attention(q, k, v, s, sel, 0.0, 64)
    assert np.array_equal(used0, (sel >= 0).sum(-1))
    np.testing.assert_allclose(o0, o_sp, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l0, l_sp, rtol=1e-12, atol=1e-12)
    # tau = inf stops after the first block past the diagonal: the best-scored one
    oi, li, usedi, _ = O.early_stop_attention(q, k, v, s, sel, np.inf, 64)
    assert np.array_equal(usedi, np.minimum((sel >= 0).sum(-1), 2))
    best = sel.copy()
    for h in range(4):
        for i in range(8):
            order = O.early_stop_order(sel[0, h, i], s[0, h, i], i)
            row = sorted(order[:2])
            best[0, h, i] = row + [-1] * (4 - len(row))
    o_b, l_b = O.sparse_attention(q, k, v, best, 64)
    np.testing.assert_allclose(oi, o_b, rtol=1e-12, atol=1e-12)
    # monotone: a larger threshold never visits more blocks
    prev = None
    for tau in (0.0, 0.01, 0.05, 0.2, 1.0, np.inf):
        u = O.early_stop_attention(q, k, v, s, sel, tau, 64)[2]
        if prev is not None:
            assert np.all(u <= prev)
        prev = u


def check_early_stop_loops(O):
    # the ratios and decisions recomputed key by key with math.exp
    q, k, v = rand_qkv(1, 2, 1, 192, 8)
    s = O.block_scores(q, k, 64)
    sel = O.select_blocks(s, 3, 64)
    tau = 0.05
    _, _, used, ratio = O.early_stop_attention(q, k, v, s, sel, tau, 64)
    sc = 1 / math.sqrt(8)
    sc = float(np.float32(sc))
    for h in range(2):
        for i in range(3):
            order = [i] + sorted((int(j) for j in sel[0, h, i] if 0 <= j < i), key=lambda j: (-s[0, h, i, j], j))
            rows = range(64 * i, 64 * i + 64)
            gains = []
            for j in order:
                gr = []
                for r in rows:
                    lg = [sc * sum(q[0, h, r, t] * k[0, 0, c, t] for t in range(8)) for c in range(64 * j, 64 * j + 64) if c <= r]
                    mx = max(sc * sum(q[0, h, r, t] * k[0, 0, c, t] for t in range(8)) for jj in order
                             for c in range(64 * jj, 64 * jj + 64) if c <= r)
                    gr.append(sum(math.exp(x - mx) for x in lg))
                gains.append(gr)
            want = len(order)
            for t in range(1, len(order)):
                rt = max(gains[t][n] / sum(gains[u][n] for u in range(t)) for n in range(64))
                assert abs(rt - ratio[0, h, i, t]) <= 1e-12 * max(1.0, rt)
                if want == len(order) and all(gains[t][n] < tau * sum(gains[u][n] for u in range(t)) for n in range(64)):
                    want = t + 1
            assert used[0, h, i] == want

# ----------------------------------------------------------------------------- backward

def _loss(O, q, kk, v, dout, idx, B, sc, q_off, full, row_range=None):
    """sum(dout * O) from the oracle's own forward (the scalar the gradients are of)."""
    if full:
        o, _, _ = O.full_attention_dropped_mass(q, kk, v, idx, B, scale=sc, q_offset=q_off, row_range=row_range)
    else:
        o, _ = O.sparse_attention(q, kk, v, idx, B, scale=sc, q_offset=q_off)
    return float((o * dout).sum())


def check_backward_finite_differences(O):
    # central differences of the forward loss, element by element, on tiny inputs
    rng = np.random.default_rng(11)
    for (n_q, q_off, B, k, full, rr) in [(10, 0, 4, 2, False, None),    # ragged last block
                                          (10, 0, 4, 2, True, None),
                                          (8, 8, 4, 2, False, None),      # a chunk at q_offset 8
                                          (12, 0, 4, 1, True, (4, 12))]:  # full on a row slice
        n_kv, d = n_q + q_off, 3
        q = rng.standard_normal((1, 2, n_q, d))
        kk = rng.standard_normal((1, 1, n_kv, d))
        v = rng.standard_normal((1, 1, n_kv, d))
        lo, hi = (0, n_q) if rr is None else rr
        dout = rng.standard_normal((1, 2, hi - lo, d))
        sc = 0.6
        idx = O.select_blocks(O.block_scores(q, kk, B, scale=sc, q_offset=q_off), k, B, q_offset=q_off)
        dq, dk, dv = O.attention_backward(q, kk, v, dout, idx, B, scale=sc, q_offset=q_off, full=full,
                                          row_range=rr)
        eps = 1e-5
        for name, x, g in (("q", q, dq), ("k", kk, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for ix in np.ndindex(x.shape):
                x0 = x[ix]
                x[ix] = x0 + eps
                lp = _loss(O, q, kk, v, dout, idx, B, sc, q_off, full, rr)
                x[ix] = x0 - eps
                lm = _loss(O, q, kk, v, dout, idx, B, sc, q_off, full, rr)
                x[ix] = x0
                fd[ix] = (lp - lm) / (2 * eps)
            if name == "q":
                fd = fd[:, :, lo:hi]
            np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=f"d{name} full={full} off={q_off}")


def check_backward_autograd(O):
    # torch autograd through float64 SDPA with the same boolean mask (GQA)
    b, hq, hkv, n, d, B, k = 2, 4, 2, 40, 8, 8, 3
    q, kk, v = rand_qkv(b, hq, hkv, n, d)
    dout = bf16_values((b, hq, n, d))
    sc = float(np.float32(1 / math.sqrt(d)))
    idx = O.select_blocks(O.block_scores(q, kk, B), k, B)
    for full in (False, True):
        mask = tr.causal_mask(n, n, 0) if full else tr.block_mask_from_idx(idx, n, n, B, 0)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, kk, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=sc, enable_gqa=True)
        (o * torch.tensor(dout)).sum().backward()
        dq, dk, dv = O.attention_backward(q, kk, v, dout, idx, B, full=full)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def check_backward_identities(O):
    b, hq, hkv, n, d, B, k = 1, 4, 2, 96, 8, 16, 2
    q, kk, v = rand_qkv(b, hq, hkv, n, d)
    dout = bf16_values((b, hq, n, d))
    idx = O.select_blocks(O.block_scores(q, kk, B), k, B)
    for full in (False, True):
        dq, dk, dv = O.attention_backward(q, kk, v, dout, idx, B, full=full)
        # each row's softmax Jacobian annihilates constants: the key gradients of a group sum to zero
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
        # each row's probabilities sum to one: the value gradients sum to the group's output gradients
        np.testing.assert_allclose(dv.sum(axis=2), dout.reshape(b, hkv, hq // hkv, n, d).sum(axis=(2, 3)),
                                   rtol=1e-11, atol=1e-11)
        # row 0 attends to its own key only: its output is v_0 whatever q_0 is
        np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-14)
        # GQA: the same as one KV head per query head, summed over each group
        g = hq // hkv
        dq1, dk1, dv1 = O.attention_backward(q, np.repeat(kk, g, axis=1), np.repeat(v, g, axis=1), dout, idx, B,
                                             full=full)
        np.testing.assert_allclose(dq1, dq, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dk1.reshape(b, hkv, g, n, d).sum(axis=2), dk, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv1.reshape(b, hkv, g, n, d).sum(axis=2), dv, rtol=1e-11, atol=1e-12)
    # every block selected: the sparse gradients are the full ones
    idx_all = O.select_blocks(O.block_scores(q, kk, B), n // B, B)
    for a_, b_ in zip(O.attention_backward(q, kk, v, dout, idx_all, B),
                      O.attention_backward(q, kk, v, dout, idx_all, B, full=True)):
        np.testing.assert_allclose(a_, b_, rtol=1e-12, atol=1e-13)
    # the sparse stream passes no gradient to keys outside a row's blocks
    idx_diag = O.select_blocks(O.block_scores(q, kk, B), 1, B)
    _, dkd, dvd = O.attention_backward(q, kk, v, dout, idx_diag, B)
    _, _, dvf = O.attention_backward(q, kk, v, dout, idx_diag, B, full=True)
    for j in range(n // B):   # k == 1: block j only sees itself, so its keys only get block j's gradient
        rows = slice(j * B, (j + 1) * B)
        np.testing.assert_allclose(dvd[:, :, rows].sum(axis=2),
                                   dout[:, :, rows].reshape(b, hkv, hq // hkv, B, d).sum(axis=(2, 3)),
                                   rtol=1e-11, atol=1e-11)
    assert not np.allclose(dvd, dvf)


# ----------------------------------------------------------------------------- DashAttention stages

def check_entmax_hand_example(O):
    # sparsemax of (0, 0.5, 1): support {0.5, 1}, tau = 0.25
    np.testing.assert_allclose(O.entmax(np.array([0.0, 0.5, 1.0]), 2.0), [0.0, 0.25, 0.75], atol=1e-14)
    # 1.5-entmax of (0, 1): halved scores (0, 0.5), both in the support, tau the smaller root of
    # (0.5 - tau)^2 + tau^2 = 1, i.e. tau = (1 - sqrt 7) / 4
    r7 = math.sqrt(7.0)
    np.testing.assert_allclose(O.entmax(np.array([0.0, 1.0]), 1.5), [(4 - r7) / 8, (4 + r7) / 8], atol=1e-14)
    # -inf scores take no mass; a single finite score takes all of it
    np.testing.assert_allclose(O.entmax(np.array([-np.inf, 3.0, -np.inf]), 1.5), [0.0, 1.0, 0.0], atol=0)


def _sparsemax_sorted(z):
    zs = np.sort(z)[::-1]
    css = np.cumsum(zs)
    k = np.arange(1, len(z) + 1)
    kmax = k[1 + k * zs > css].max()
    tau = (css[kmax - 1] - 1) / kmax
    return np.maximum(z - tau, 0)


def _entmax15_sorted(z):
    # exact 1.5-entmax: with the support of size k (largest scaled scores), tau solves
    # sum (zt - tau)^2 = 1, tau = mean - sqrt((1 - ss) / k); the support is the largest
    # k whose smallest member stays above its tau
    zt = np.sort(z / 2)[::-1]
    best = None
    for k in range(1, len(z) + 1):
        top = zt[:k]
        mean = top.mean()
        ss = ((top - mean) ** 2).sum()
        if ss > 1:
            break
        tau = mean - math.sqrt((1 - ss) / k)
        if top[-1] > tau:
            best = tau
    return np.maximum(z / 2 - best, 0) ** 2


def check_entmax_closed_forms(O):
    rng = np.random.default_rng(5)
    for n in (1, 2, 5, 17, 64):
        for scale in (0.1, 1.0, 4.0):
            z = rng.standard_normal(n) * scale
            np.testing.assert_allclose(O.entmax(z, 2.0), _sparsemax_sorted(z), atol=1e-12)
            np.testing.assert_allclose(O.entmax(z, 1.5), _entmax15_sorted(z), atol=1e-12)
            for alpha in (1.2, 1.5, 1.8, 2.0):
                p = O.entmax(z, alpha)
                assert abs(p.sum() - 1) < 1e-12 and np.all(p >= 0)
                np.testing.assert_allclose(O.entmax(z + 3.25, alpha), p, atol=1e-12)   # shift invariance
                # optimality: p^(alpha-1) = (alpha-1) z - tau on the support, (alpha-1) z <= tau off it
                sup = p > 0
                taus = (alpha - 1) * z[sup] - p[sup] ** (alpha - 1)
                assert np.ptp(taus) < 1e-9
                assert np.all((alpha - 1) * z[~sup] <= taus[0] + 1e-12)


def check_learned_summaries(O):
    b, hkv, n, d, B = 2, 2, 200, 8, 64          # ragged last chunk (8 rows)
    kk = bf16_values((b, hkv, n, d))
    qbar = bf16_values((hkv, d), scale=2.0)
    # zero query: the plain block mean
    np.testing.assert_array_equal(O.learned_key_summaries(kk, np.zeros((hkv, d)), B), O.key_summaries(kk, B))
    # library: one-row SDPA of qbar over each chunk's keys (keys as values)
    got = O.learned_key_summaries(kk, qbar, B, scale=0.5)
    for j in range(-(-n // B)):
        rows = tr.t64(kk[:, :, j * B: (j + 1) * B])
        qq = tr.t64(np.broadcast_to(qbar[None, :, None, :], (b, hkv, 1, d)).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(qq, rows, rows, scale=0.5)[:, :, 0].numpy()
        np.testing.assert_allclose(got[:, :, j], ref, rtol=1e-6, atol=1e-7)   # got is fp32-rounded


def check_entmax_routing(O):
    rng = np.random.default_rng(6)
    b, hq, hkv, nqb, B = 1, 4, 2, 6, 16
    s = rng.standard_normal((b, hq, nqb, nqb))
    for i in range(nqb):
        s[:, :, i, i + 1:] = -np.inf
    for alpha, gamma in ((1.5, 2.0), (2.0, 0.7)):
        w = O.entmax_routing(s, hkv, alpha, gamma, B)
        for g in range(hkv):
            for i in range(nqb):
                assert np.all(w[0, g, i, i:] == 0)                 # nothing routed from the diagonal on
                if i == 0:
                    continue
                ref = sum(O.entmax(gamma * s[0, g * 2 + hh, i, :i], alpha) for hh in range(2)) / 2
                np.testing.assert_allclose(w[0, g, i, :i], ref, atol=1e-15)
                assert abs(w[0, g, i].sum() - 1) < 1e-12
    # one head per KV head: the per-head entmax itself
    w1 = O.entmax_routing(s, hq, 1.5, 1.0, B)
    np.testing.assert_allclose(w1[0, 3, 5, :5], O.entmax(s[0, 3, 5, :5], 1.5), atol=1e-15)


def check_routing_support_and_bias(O):
    w = np.zeros((1, 1, 2, 5))
    w[0, 0, 1] = [0.5, 0.0, 0.3, 0.2, 0.0]                        # query block 1 of a 4-block offset
    sel = O.routing_support(w, 3, 16, q_offset=64)                  # diag(1) = 5 // ... = (64 + 16) // 16 = 5
    assert list(sel[0, 0, 1]) == [0, 2, 5]
    assert list(O.routing_support(w, 8, 16, q_offset=64)[0, 0, 1]) == [0, 2, 3, 5, -1, -1, -1, -1]
    assert list(sel[0, 0, 0]) == [4, -1, -1]                        # no weight: the diagonal only
    bias = O.prior_bias(w, sel, 0.5, 16, q_offset=64)
    np.testing.assert_allclose(bias[0, 0, 1], [0.5 * math.log(0.5), 0.5 * math.log(0.3), 0.0], atol=1e-15)
    assert np.all(bias[0, 0, 0] == 0)


def check_prior_attention(O):
    b, hq, hkv, n, d, B, k = 1, 4, 2, 192, 8, 32, 3
    q, kk, v = rand_qkv(b, hq, hkv, n, d)
    rng = np.random.default_rng(7)
    s = O.block_scores(q, kk, B)
    w = O.entmax_routing(s, hkv, 1.5, 4.0, B)
    sel = O.routing_support(w, k, B)
    sc = float(np.float32(1 / math.sqrt(d)))
    # sigma = 0: the plain block-sparse softmax over the listed blocks
    o0, l0 = O.prior_attention(q, kk, v, sel, O.prior_bias(w, sel, 0.0, B), B)
    o_ref, l_ref = O.sparse_attention(q, kk, v, O.expand_shared(sel, hq), B)
    np.testing.assert_allclose(o0, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l0, l_ref, rtol=1e-12, atol=1e-13)
    # library: SDPA with an additive float mask (bias on listed causal keys, -inf elsewhere)
    bias = O.prior_bias(w, sel, 0.7, B)
    o1, l1 = O.prior_attention(q, kk, v, sel, bias, B)
    mask = np.full((b, hq, n, n), -np.inf)
    for h in range(hq):
        for i in range(n // B):
            for e, j in enumerate(sel[0, h // 2, i]):
                if j >= 0:
                    mask[0, h, i * B:(i + 1) * B, j * B:(j + 1) * B] = bias[0, h // 2, i, e]
    mask = np.where(np.tril(np.ones((n, n), dtype=bool))[None, None], mask, -np.inf)
    tm = torch.tensor(mask)
    ref = torch.nn.functional.scaled_dot_product_attention(tr.t64(q), tr.t64(kk), tr.t64(v), attn_mask=tm, scale=sc,
                                                           enable_gqa=True).numpy()
    np.testing.assert_allclose(o1, ref, rtol=1e-11, atol=1e-12)
    logits = torch.matmul(tr.t64(q), tr.t64(np.repeat(kk, 2, axis=1)).transpose(-1, -2)) * sc + tm
    np.testing.assert_allclose(l1, torch.logsumexp(logits, dim=-1).numpy(), rtol=1e-12, atol=1e-12)
    # one constant added to every bias of a query block (diagonal included) leaves O and shifts LSE
    o2, l2 = O.prior_attention(q, kk, v, sel, bias + 1.5 * (sel >= 0), B)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + 1.5, rtol=1e-12, atol=1e-12)
    del rng


# ----------------------------------------------------------------------------- per-row branches, list reading

def _masked_lse(q, kk, mask, sc):
    """Natural log-sum-exp over the allowed keys of each row (torch, float64;
    -inf where a row allows none)."""
    qt, kt = tr.t64(q), tr.t64(kk)
    group = qt.shape[1] // kt.shape[1]
    logits = torch.matmul(qt, kt.repeat_interleave(group, dim=1).transpose(-1, -2)) * sc
    return torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1).numpy()


def check_full_rows_branch(O):
    """The per-row evaluation of the full counterpart (rows=...) against torch:
    SDPA for O, logsumexp for LSE, and the log-sum-exp over the dropped keys for
    delta; a prefill with a ragged tail and a decode-shaped call."""
    rng = np.random.default_rng(31)
    for (b, hq, hkv, n, d, B, k, qo) in [(1, 4, 2, 200, 16, 32, 3, 0),   # 200 rows = 6 blocks + 8
                                         (2, 4, 1, 1, 8, 32, 4, 299)]:  # one row at position 299
        seq_kv = qo + n
        q = bf16_values((b, hq, n, d), rng)
        kk, v = bf16_values((b, hkv, seq_kv, d), rng), bf16_values((b, hkv, seq_kv, d), rng)
        sc = float(np.float32(1.0 / math.sqrt(d)))
        idx = O.select_blocks(O.block_scores(q, kk, B, q_offset=qo), k, B, q_offset=qo)
        rows = sorted({(bi, h, r) for bi in range(b) for h in (0, hq - 1) for r in (0, n // 2, n - 1)})
        o_r, l_r, d_r = O.full_attention_dropped_mass(q, kk, v, idx, B, q_offset=qo, rows=rows)
        causal = tr.causal_mask(n, seq_kv, qo)
        o_ref, l_ref = tr.sdpa(q, kk, v, causal, sc)
        drop = causal & ~tr.block_mask_from_idx(idx, n, seq_kv, B, qo)
        l_drop = _masked_lse(q, kk, drop, sc)
        for t, (bi, h, r) in enumerate(rows):
            np.testing.assert_allclose(o_r[t], o_ref[bi, h, r], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(l_r[t], l_ref[bi, h, r], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(d_r[t], math.exp(l_drop[bi, h, r] - l_ref[bi, h, r]), rtol=1e-10, atol=1e-15)
        if n > B:   # some row of the prefill case must drop keys, or delta is not exercised
            assert max(d_r) > 0.05


def check_early_stop_used_branch(O):
    """An imposed block count (used=...) attends over the first `used` blocks
    of the visiting order -- the diagonal, then by coarse score -- which is
    block-sparse attention over those blocks (SDPA with their mask)."""
    rng = np.random.default_rng(37)
    q, k, v = rand_qkv(1, 2, 1, 256, 16, rng)
    B = 32
    s = O.block_scores(q, k, B)
    sel = O.select_blocks(s, 4, B)
    nqb = 256 // B
    listed = (sel >= 0).sum(-1)
    used = np.array([[[rng.integers(1, listed[0, h, i] + 1) for i in range(nqb)] for h in range(2)]])
    o, lse, u, _ = O.early_stop_attention(q, k, v, s, sel, 0.1, B, used=used)
    assert np.array_equal(u, used)
    first = np.full_like(sel, -1)
    for h in range(2):
        for i in range(nqb):
            others = sorted((int(j) for j in sel[0, h, i] if 0 <= j < i), key=lambda j: (-s[0, h, i, j], j))
            keep = ([i] + others)[: used[0, h, i]]
            first[0, h, i, : len(keep)] = keep
    sc = float(np.float32(1.0 / 4.0))
    o_ref, l_ref = tr.sdpa(q, k, v, tr.block_mask_from_idx(first, 256, 256, B, 0), sc)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, rtol=1e-12, atol=1e-12)


def _scramble_rows(idx, rng):
    """Each index row shuffled, a -1 put in its middle and its first entry
    listed once more at the end (width topk + 2): the same set of blocks."""
    b, h, nqb, k = idx.shape
    out = np.full((b, h, nqb, k + 2), -1, dtype=idx.dtype)
    for bi in range(b):
        for hh in range(h):
            for i in range(nqb):
                lst = list(rng.permutation([int(j) for j in idx[bi, hh, i] if j >= 0]))
                mid = len(lst) // 2
                row = lst[:mid] + [-1] + lst[mid:] + lst[:1]
                out[bi, hh, i, : len(row)] = row
    return out


def check_index_row_as_set(O):
    """An index row names a set of blocks: shuffling it, putting a -1 in its
    middle and listing a block twice change nothing.  Pinned against SDPA with
    the mask of the set, and the scrambled rows against the ascending ones in
    the full counterpart, the prior-biased softmax (a repeated listing's bias
    is ignored), the early-stopping order and the backward."""
    rng = np.random.default_rng(41)
    b, hq, hkv, n, d, B, k = 1, 4, 2, 256, 16, 32, 4
    q, kk, v = rand_qkv(b, hq, hkv, n, d, rng)
    sc = float(np.float32(0.25))
    s = O.block_scores(q, kk, B)
    idx = O.select_blocks(s, k, B)
    scr = _scramble_rows(idx, rng)
    o, lse = O.sparse_attention(q, kk, v, scr, B)
    o_ref, l_ref = tr.sdpa(q, kk, v, tr.block_mask_from_idx(idx, n, n, B, 0), sc)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, rtol=1e-12, atol=1e-12)
    _, _, dm0 = O.full_attention_dropped_mass(q, kk, v, idx, B)
    _, _, dm1 = O.full_attention_dropped_mass(q, kk, v, scr, B)
    np.testing.assert_allclose(dm1, dm0, rtol=1e-13, atol=1e-15)
    for h in range(hq):
        for i in range(n // B):
            assert O.early_stop_order(scr[0, h, i], s[0, h, i], i) == O.early_stop_order(idx[0, h, i], s[0, h, i], i)
    dout = bf16_values((b, hq, n, d), rng)
    g0 = O.attention_backward(q, kk, v, dout, idx, B)
    g1 = O.attention_backward(q, kk, v, dout, scr, B)
    for a0, a1 in zip(g0, g1):
        np.testing.assert_allclose(a1, a0, rtol=1e-12, atol=1e-13)
    # prior-biased softmax on group-shared rows: the first listing's bias counts
    sel_g = idx[:, ::2]
    bias = rng.standard_normal(sel_g.shape) * (sel_g >= 0)
    scr_g = np.full(sel_g.shape[:-1] + (k + 2,), -1, dtype=sel_g.dtype)
    bias_g = np.zeros(scr_g.shape)
    for g in range(hkv):
        for i in range(n // B):
            ent = [(int(j), float(bb)) for j, bb in zip(sel_g[0, g, i], bias[0, g, i]) if j >= 0]
            order = rng.permutation(len(ent))
            row = [ent[t] for t in order] + [(ent[order[0]][0], 7.0)]   # repeat with another bias
            for e, (j, bb) in enumerate(row):
                scr_g[0, g, i, e], bias_g[0, g, i, e] = j, bb
    p0 = O.prior_attention(q, kk, v, sel_g, bias, B)
    p1 = O.prior_attention(q, kk, v, scr_g, bias_g, B)
    np.testing.assert_allclose(p1[0], p0[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p1[1], p0[1], rtol=1e-12, atol=1e-13)


ALL_CHECKS = [check_block_means, check_scores_token_level, check_scores_gqa_and_causal,
              check_select_brute_force, check_select_ties_and_decode, check_sparse_vs_sdpa,
              check_sparse_special_cases, check_sparse_brute_force_loops,
              check_full_and_dropped_identities, check_tie_closed_form, check_decode,
              check_shared_hand_example, check_shared_scores_pool_queries, check_shared_reductions,
              check_shared_brute_force, check_early_stop_hand_example, check_early_stop_limits,
              check_early_stop_loops, check_backward_finite_differences, check_backward_autograd,
              check_backward_identities, check_entmax_hand_example, check_entmax_closed_forms,
              check_learned_summaries, check_entmax_routing, check_routing_support_and_bias,
              check_prior_attention, check_full_rows_branch, check_early_stop_used_branch,
              check_index_row_as_set]


# ----------------------------------------------------------------------------- the pins

def test_hand_example(golden_dir):
    check_hand_example(ssa_oracle, golden_dir)


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(ssa_oracle)


def test_geometry_rejected():
    q = np.zeros((1, 1, 3, 4))
    k = np.zeros((1, 1, 5, 4))
    with pytest.raises(ValueError):
        ssa_oracle.block_scores(q, k, 2, q_offset=0)        # seq_kv != q_offset + seq_q
    with pytest.raises(ValueError):
        ssa_oracle.block_scores(q, k, 4, q_offset=2)        # chunk not on a block boundary


# ----------------------------------------------------------------------------- planted mistakes
# Each mutant plants one plausible mistake in the oracle (on the CPU); at least
# one pin must fail for it.

def _fails(check, *args):
    try:
        check(ssa_oracle, *args)
    except AssertionError:
        return True
    return False


def _any_pin_fails(golden_dir):
    if _fails(check_hand_example, golden_dir):
        return True
    return any(_fails(c) for c in ALL_CHECKS)


MUTANTS = {
    "tie_break_higher_index_first": ("_rank_key", lambda s, j: (1, 0.0, -j) if math.isnan(s) else (0, -s, -j)),
    "nan_ranks_highest": ("_rank_key", lambda s, j: (-1, 0.0, j) if math.isnan(s) else (0, -s, j)),
    "diagonal_off_by_one": ("diag_block", lambda i, q_offset, block: max(0, (q_offset + i * block) // block - 1)),
    "partial_block_divides_by_block": ("block_means", None),
    "scale_one_over_d": ("default_scale", lambda d: 1.0 / d),
    "no_fp32_rounding": ("round_f32", lambda x: np.asarray(x, dtype=np.float64)),
    "drops_last_selected_block": ("_allowed_keys", None),
    "shared_uses_first_head": ("shared_block_scores", None),
    "shared_sum_not_mean": ("shared_block_scores", None),
    "early_stop_drops_trigger_block": ("_early_stop_count", None),
    "early_stop_counts_own_gain": ("_early_stop_count", None),
    "early_stop_index_order": ("early_stop_order", None),
    "bwd_no_softmax_correction": ("_block_backward", None),
    "bwd_dk_unscaled": ("_block_backward", None),
    "bwd_dv_unnormalised": ("_block_backward", None),
    "entmax_linear_for_any_alpha": ("entmax", None),
    "routing_includes_diagonal": ("entmax_routing", None),
    "prior_bias_ignores_sigma": ("prior_bias", None),
    "summaries_ignore_learned_query": ("learned_key_summaries", None),
    "repeated_block_counted_twice": ("_listed_blocks", None),
    "full_rows_delta_off_by_one_key": ("full_attention_dropped_mass", None),
    "early_stop_used_ignored": ("early_stop_attention", None),
}


def _mutant_block_means(x, block):
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-2]
    nb = -(-n // block)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]))
    for j in range(nb):
        out[..., j, :] = x[..., j * block: (j + 1) * block, :].sum(axis=-2) / block
    return out


_orig_allowed = ssa_oracle._allowed_keys


def _mutant_allowed(sel_row, pos, block, seq_kv):
    kept = [j for j in sel_row if j >= 0]
    return _orig_allowed(kept[:-1] if len(kept) > 1 else kept, pos, block, seq_kv)


_orig_shared = ssa_oracle.shared_block_scores


def _mutant_shared_first_head(scores, n_kv_heads):
    s = np.asarray(scores, dtype=np.float64)
    g = s.shape[1] // n_kv_heads
    return s[:, ::g].copy()


def _mutant_shared_sum(scores, n_kv_heads):
    g = np.asarray(scores).shape[1] // n_kv_heads
    return _orig_shared(scores, n_kv_heads) * g


def _mutant_drop_trigger(gains, tau):
    for t in range(1, len(gains)):
        if np.all(gains[t] < tau * sum(gains[:t])):
            return t
    return len(gains)


def _mutant_own_gain(gains, tau):
    for t in range(1, len(gains)):
        if np.all(gains[t] < tau * sum(gains[: t + 1])):
            return t + 1
    return len(gains)


def _mutant_index_order(sel_row, score_row, jd):
    listed = sorted(int(j) for j in sel_row if j >= 0)
    return ([jd] if jd in listed else []) + [j for j in listed if j != jd]


def _mutant_bwd(kind):
    def f(qb, kc, vc, dob, allowed, scale):
        logits = np.where(allowed, scale * (qb @ kc.T), -np.inf)
        m = logits.max(axis=1, keepdims=True)
        w = np.where(allowed, np.exp(logits - m), 0.0)
        p = w / w.sum(axis=1, keepdims=True)
        dv = (w if kind == "unnormalised" else p).T @ dob
        dp = dob @ vc.T
        ds = p * dp if kind == "no_correction" else p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dk = (ds.T @ qb) if kind == "unscaled" else scale * (ds.T @ qb)
        return scale * (ds @ kc), dk, dv
    return f


_orig_entmax = ssa_oracle.entmax
_orig_routing = ssa_oracle.entmax_routing
_orig_prior_bias = ssa_oracle.prior_bias


def _mutant_entmax_linear(z, alpha):
    return _orig_entmax(z, 2.0)


def _mutant_routing_diag(scores, n_kv_heads, alpha, gamma, block, q_offset=0):
    s = np.asarray(scores, dtype=np.float64)
    b, hq, nqb, nkb = s.shape
    group = hq // n_kv_heads
    out = np.zeros((b, n_kv_heads, nqb, nkb))
    for bi in range(b):
        for g in range(n_kv_heads):
            for i in range(nqb):
                jd = ssa_oracle.diag_block(i, q_offset, block)
                acc = sum(_orig_entmax(gamma * s[bi, g * group + hh, i, :jd + 1], alpha) for hh in range(group))
                out[bi, g, i, :jd + 1] = acc / group
    return out


def _mutant_bias_no_sigma(weights, sel, sigma, block, q_offset=0):
    return _orig_prior_bias(weights, sel, 1.0, block, q_offset)


def _mutant_summaries_mean(k, qbar, block, scale=None):
    return ssa_oracle.key_summaries(k, block)


def _mutant_listed_with_repeats(sel_row):
    return [(e, int(j)) for e, j in enumerate(sel_row) if j >= 0]


_orig_full = ssa_oracle.full_attention_dropped_mass


def _mutant_full_rows(q, k, v, sel, block, scale=None, q_offset=0, row_range=None, rows=None):
    """Per-row branch that leaves the row's own key out of delta's complement."""
    if rows is None:
        return _orig_full(q, k, v, sel, block, scale=scale, q_offset=q_offset, row_range=row_range)
    o, lse, delta = _orig_full(q, k, v, sel, block, scale=scale, q_offset=q_offset, rows=rows)
    q64, k64 = np.asarray(q, np.float64), np.asarray(k, np.float64)
    sc = float(np.float32(scale if scale is not None else 1.0 / math.sqrt(q64.shape[-1])))
    g = q64.shape[1] // k64.shape[1]
    extra = np.array([math.exp(sc * float(q64[bi, h, r] @ k64[bi, h // g, q_offset + r]) - lse[t])
                      for t, (bi, h, r) in enumerate(rows)])
    return o, lse, delta + extra


_orig_es = ssa_oracle.early_stop_attention


def _mutant_es_used(q, k, v, scores, sel, tau, block, scale=None, q_offset=0, used=None):
    return _orig_es(q, k, v, scores, sel, tau, block, scale=scale, q_offset=q_offset, used=None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch, golden_dir):
    attr, fn = MUTANTS[name]
    fn = {"early_stop_drops_trigger_block": _mutant_drop_trigger, "early_stop_counts_own_gain": _mutant_own_gain,
          "early_stop_index_order": _mutant_index_order}.get(name, fn)
    if name == "shared_uses_first_head":
        fn = _mutant_shared_first_head
    if name == "shared_sum_not_mean":
        fn = _mutant_shared_sum
    if name == "partial_block_divides_by_block":
        fn = _mutant_block_means
    if name == "drops_last_selected_block":
        fn = _mutant_allowed
    fn = {"entmax_linear_for_any_alpha": _mutant_entmax_linear, "routing_includes_diagonal": _mutant_routing_diag,
          "prior_bias_ignores_sigma": _mutant_bias_no_sigma,
          "summaries_ignore_learned_query": _mutant_summaries_mean,
          "repeated_block_counted_twice": _mutant_listed_with_repeats,
          "full_rows_delta_off_by_one_key": _mutant_full_rows,
          "early_stop_used_ignored": _mutant_es_used}.get(name, fn)
    if name.startswith("bwd_"):
        fn = _mutant_bwd({"bwd_no_softmax_correction": "no_correction", "bwd_dk_unscaled": "unscaled",
                          "bwd_dv_unnormalised": "unnormalised"}[name])
    monkeypatch.setattr(ssa_oracle, attr, fn)
    assert _any_pin_fails(golden_dir), f"no pin catches mutant {name}"
