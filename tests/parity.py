"""Comparison rules between the HIP library and the fp64 oracle.

bf16 outputs: max-abs <= 2e-2 and relative L2 <= 1e-2 over the checked rows
(all heads, all d). fp32 outputs: relative L2 <= 1e-5. Top-K index sets: exact
on every (head, query block) whose oracle gap between the K-th and (K+1)-th
score exceeds 1e-3; elsewhere every GPU pick must score at least the oracle's
K-th score minus 1e-3.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
F32_REL_L2 = 1e-5
TOPK_GAP = 1e-3


def host(x: torch.Tensor) -> np.ndarray:
    """Exact host copy (bf16 widened to fp32, fp32 kept)."""
    return x.detach().to("cpu").float().numpy()


def oracle_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def stats(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / (den if den > 0 else 1.0)
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str):
    max_abs, rel = stats(got, ref)
    print(f"[parity] {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    if dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, rel)
    else:
        assert rel <= F32_REL_L2, (what, max_abs, rel)


def check_topk(idx_gpu, idx_ref, ranked_ref, q_blk_ref, k_cmp_ref, what: str, score_of=None):
    """idx_gpu / idx_ref [H, n, K] (same rows); ranked_ref [H, n, K+1] oracle
    scores in rank order; q_blk_ref [n, H, d], k_cmp_ref [nk, H, d] fp64.
    score_of(h, b, picks) gives the oracle scores of picked keys in ranked_ref's
    units (default: the pooled query's logit)."""
    idx_gpu = np.asarray(idx_gpu)
    H, n, K = idx_ref.shape
    kth = ranked_ref[:, :, K - 1]
    nxt = ranked_ref[:, :, K] if ranked_ref.shape[2] > K else np.full_like(kth, -np.inf)
    decided = (kth - nxt) > TOPK_GAP
    exact = np.all(idx_gpu == idx_ref, axis=2)
    bad = decided & ~exact
    print(f"[parity] {what}: {decided.mean() * 100:.1f}% of (head, block) rows decided "
          f"(gap > {TOPK_GAP}), {int(bad.sum())} mismatches", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} decided rows differ"
    # each row is a set of distinct ascending indices
    assert np.all(np.diff(idx_gpu, axis=2) > 0), f"{what}: rows not strictly ascending"
    d = q_blk_ref.shape[-1] if score_of is None else None
    for h in range(H):
        und = np.nonzero(~decided[h])[0]
        for b in und:
            if score_of is not None:
                s = score_of(h, b, idx_gpu[h, b])
            else:
                s = k_cmp_ref[idx_gpu[h, b], h, :] @ q_blk_ref[b, h, :] / math.sqrt(d)
            assert np.all(s >= kth[h, b] - TOPK_GAP), (what, h, b)
    return decided


def decided_blocks(ranked_ref, K):
    kth = ranked_ref[:, :, K - 1]
    nxt = ranked_ref[:, :, K] if ranked_ref.shape[2] > K else np.full_like(kth, -np.inf)
    return (kth - nxt) > TOPK_GAP
