"""Comparison helpers for GPU-vs-oracle parity (tests only).

Tolerances (bf16 inputs, fp32 accumulation):
  outputs O      max |diff| <= 2e-2 and ||diff||_2 / ||ref||_2 <= 5e-3
  LSE            max |diff| <= 1e-3
  dropped mass   max |diff| <= 1e-3
  gradients      max |diff| <= 2e-2 * max |ref| and ||diff||_2 / ||ref||_2 <= 1e-2
                 (dQ, dK, dV are sums of products with one bf16-rounded factor, P
                 or dS (relative error <= 2^-9 each), rounded once more to bf16,
                 and D is taken from the bf16 forward output: about three bf16
                 roundings against the output's one, hence twice O's rel-L2 bound;
                 their scale varies with how many rows reach a key, so the
                 element bound is relative to the tensor's largest entry)
  block indices  identical, except rows whose (k-1)-th and k-th best candidate
                 scores tie within 1e-5 relative; there every swapped block
                 must itself lie inside that tie band.
Outputs are compared against the oracle evaluated with the GPU's own indices,
so a legitimate tie-break difference cannot masquerade as an output error.
"""
from __future__ import annotations

import numpy as np
import torch

O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
LSE_ABS = 1e-3
DROP_ABS = 1e-3
TIE_REL = 1e-5


def np64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def check_close_outputs(got, ref, what="O"):
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30)) if diff.size else 0.0
    assert max_abs <= O_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {O_MAX_ABS}"
    assert rel <= O_REL_L2, f"{what}: rel-L2 {rel:.3e} > {O_REL_L2}"
    return max_abs, rel


GRAD_MAX_REL = 2e-2
GRAD_REL_L2 = 1e-2


def check_grad(got, ref, what="grad"):
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if ref.size == 0:
        return 0.0, 0.0
    scale = max(float(np.abs(ref).max()), 1e-30)
    diff = got - ref
    max_rel = float(np.abs(diff).max()) / scale
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))
    assert max_rel <= GRAD_MAX_REL, f"{what}: max |diff| / max |ref| = {max_rel:.3e} > {GRAD_MAX_REL}"
    assert rel <= GRAD_REL_L2, f"{what}: rel-L2 {rel:.3e} > {GRAD_REL_L2}"
    return max_rel, rel


def check_abs(got, ref, tol, what):
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    assert err <= tol, f"{what}: max abs {err:.3e} > {tol}"
    return err


def _ranked(scores_row, jd):
    def key(j):
        s = scores_row[j]
        return (1, 0.0, j) if np.isnan(s) else (0, -s, j)
    return sorted(range(jd), key=key)


def check_indices(idx_gpu, scores_ref, idx_ref, topk, block, q_offset=0):
    """Returns the number of rows whose index set differs (all inside the tie band)."""
    g = np.asarray(idx_gpu.cpu() if isinstance(idx_gpu, torch.Tensor) else idx_gpu).astype(np.int64)
    r = np.asarray(idx_ref).astype(np.int64)
    assert g.shape == r.shape, (g.shape, r.shape)
    rows = np.argwhere(np.any(g != r, axis=-1))
    for (b, h, i) in rows:
        jd = (q_offset + i * block) // block
        row = g[b, h, i]
        kept = [int(j) for j in row if j >= 0]
        assert kept == sorted(set(kept)), f"row {(b, h, i)} not ascending/distinct: {row}"
        assert jd in kept and all(0 <= j <= jd for j in kept), f"row {(b, h, i)} invalid: {row}"
        assert len(kept) == min(topk, jd + 1) and all(j == -1 for j in row[len(kept):])
        s = np.asarray(scores_ref[b, h, i], dtype=np.float64)
        order = _ranked(s, jd)
        s_k, s_k1 = s[order[topk - 2]], s[order[topk - 1]]
        tol = TIE_REL * max(abs(s_k), abs(s_k1))
        assert abs(s_k - s_k1) <= tol, (
            f"row {(b, h, i)}: index sets differ outside a tie (s_k={s_k!r}, s_k+1={s_k1!r})")
        swapped = set(kept) ^ set(int(j) for j in r[b, h, i] if j >= 0)
        for j in swapped:
            assert s_k1 - tol <= s[j] <= s_k + tol, f"row {(b, h, i)}: block {j} outside the tie band"
    return len(rows)


def sample_rows(rng, b, hq, seq_q, n, block=64):
    """Seeded (b, h, r) triples: the first/last row of several blocks and random rows."""
    out = {(0, 0, 0), (b - 1, hq - 1, seq_q - 1), (0, hq - 1, min(seq_q - 1, block - 1))}
    while len(out) < n:
        bi, h = int(rng.integers(b)), int(rng.integers(hq))
        if rng.random() < 0.3:
            blk = int(rng.integers(-(-seq_q // block)))
            r = min(seq_q - 1, blk * block + (block - 1 if rng.random() < 0.5 else 0))
        else:
            r = int(rng.integers(seq_q))
        out.add((bi, h, r))
    return sorted(out)
