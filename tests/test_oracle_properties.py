"""Randomised small geometries: the fp64 oracle against definitions written
out token by token, independently of the oracle's own tables (CPU only).

For every drawn geometry (1-4 frames, a 1..9 x 1..9 patch grid, 0-5 special
tokens, 1-2 heads), pooling stride 1..4 and top_k 1..all, each step of the
layer is rebuilt here from the token layout alone and compared with what the
oracle returns:

* dense and frame attention: torch's scaled_dot_product_attention (fp64, CPU)
  with an explicit key mask;
* pooling: the mean of every 4x4 window's in-grid tokens, gathered by
  enumerating (row, column) pairs;
* top-K: a full sort of the block scores by (score desc, index asc);
* the fine branch: SDPA with a per-query mask built from the selected windows
  and the always-kept tokens;
* the whole GSA layer with every block selected and the gate forced to the
  fine branch: dense attention;
* subsampled attention (modes 0 and 2, with and without the log-count bias):
  SDPA over K extended by one mean row per frame, with an additive mask that
  encodes which keys each query sees.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle.layer as L
from synth import Geometry

D = 8  # head dim of these checks (the definitions do not depend on it)

PROPS = settings(max_examples=40, deadline=None, derandomize=True,
                 suppress_health_check=[HealthCheck.too_slow])


@st.composite
def geometries(draw):
    return Geometry(draw(st.integers(1, 4)), draw(st.integers(0, 5)), draw(st.integers(1, 9)),
                    draw(st.integers(1, 9)), draw(st.integers(1, 2)), D, "f32")


def _qkv(g, seed):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((g.n_tokens, g.n_heads, D)) for _ in range(3))


def _close(a, b, tol=1e-11):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape
    if a.size:
        assert np.max(np.abs(a - b)) <= tol * max(1.0, float(np.max(np.abs(b)))), np.max(np.abs(a - b))


def _sdpa(q, k, v, mask=None):
    """torch SDPA, fp64 on the CPU; ``mask`` boolean (True = attend) or an
    additive float bias."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).double()[None] for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0].numpy()


def _token(g, t):
    """(frame, special index or -1, grid row, grid column) of token t."""
    f, p = divmod(t, g.tokens_per_frame)
    if p < g.n_special:
        return f, p, -1, -1
    r, c = divmod(p - g.n_special, g.grid_w)
    return f, -1, r, c


def _nbw(g):
    return -(-g.grid_w // 4)


def _nb(g):
    return _nbw(g) * -(-g.grid_h // 4)


def _window_of(g, t):
    """Global pooled-window index of a patch token (None for a special token)."""
    f, s, r, c = _token(g, t)
    return None if s >= 0 else f * _nb(g) + (r // 4) * _nbw(g) + c // 4


def _query_block_of(g, t):
    f, s, r, c = _token(g, t)
    nqb = _nb(g) + (1 if g.n_special else 0)
    return f * nqb + _nb(g) if s >= 0 else f * nqb + (r // 4) * _nbw(g) + c // 4


@PROPS
@given(geometries(), st.integers(0, 2 ** 31))
def test_dense_and_frame_vs_masked_sdpa(g, seed):
    q, k, v = _qkv(g, seed)
    o = L.dense_attention(q, k, v)
    of = L.frame_attention(q, k, v, g)
    frame = np.array([_token(g, t)[0] for t in range(g.n_tokens)])
    same = frame[:, None] == frame[None, :]
    for h in range(g.n_heads):
        _close(o[:, h], _sdpa(q[:, h], k[:, h], v[:, h]), 1e-12)
        _close(of[:, h], _sdpa(q[:, h], k[:, h], v[:, h], same), 1e-12)


@PROPS
@given(geometries(), st.integers(0, 2 ** 31))
def test_pooling_vs_enumerated_windows(g, seed):
    q, k, v = _qkv(g, seed)
    kc, vc = L.compress(k, v, g, 4)
    kp, _ = L.compress(k, v, g, 4, include_pad=True)
    members = {}
    for t in range(g.n_tokens):
        j = _window_of(g, t)
        if j is not None:
            members.setdefault(j, []).append(t)
    assert kc.shape[0] == g.n_frames * _nb(g) == len(members)
    for j, rows in members.items():
        _close(kc[j], k[rows].mean(axis=0), 1e-14)
        _close(vc[j], v[rows].mean(axis=0), 1e-14)
        _close(kp[j], k[rows].sum(axis=0) / 16.0, 1e-14)
    blocks = {}
    for t in range(g.n_tokens):
        blocks.setdefault(_query_block_of(g, t), []).append(t)
    qb = L.pooled_queries(q, g, 4)
    assert qb.shape[0] == len(blocks)
    for b, rows in blocks.items():
        _close(qb[b], q[rows].mean(axis=0), 1e-14)


@PROPS
@given(geometries(), st.integers(0, 2 ** 31), st.data())
def test_topk_vs_full_sort(g, seed, data):
    q, k, v = _qkv(g, seed)
    kc, _ = L.compress(k, v, g, 4)
    # round the pooled keys coarsely so that exact score ties occur
    kc = np.round(kc * 2.0) / 2.0
    qb = np.round(L.pooled_queries(q, g, 4) * 2.0) / 2.0
    nk = kc.shape[0]
    first = data.draw(st.sampled_from([0, _nb(g)] if g.n_frames > 1 else [0]))
    K = data.draw(st.integers(1, nk - first))
    idx, ranked = L.select_topk(qb, kc, K, first=first)
    for h in range(g.n_heads):
        for b in range(qb.shape[0]):
            s = [float(qb[b, h] @ kc[j, h]) / math.sqrt(D) for j in range(nk)]
            order = sorted(range(first, nk), key=lambda j: (-s[j], j))
            assert idx[h, b].tolist() == sorted(order[:K]), (K, h, b)
            _close(ranked[h, b, :min(K + 1, nk - first)], [s[j] for j in order[:K + 1]], 1e-12)


def _fine_mask(g, idx_h, keep_special, keep_ref):
    T = g.n_tokens
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        chosen = set(int(j) for j in idx_h[_query_block_of(g, t)])
        for u in range(T):
            fu, su, _, _ = _token(g, u)
            if keep_ref and fu == 0:
                mask[t, u] = True
            elif su >= 0:
                mask[t, u] = keep_special
            else:
                mask[t, u] = _window_of(g, u) in chosen
    return mask


@PROPS
@given(geometries(), st.integers(0, 2 ** 31), st.data())
def test_fine_branch_vs_masked_sdpa(g, seed, data):
    q, k, v = _qkv(g, seed)
    keep_ref = data.draw(st.booleans()) and g.n_frames > 1
    keep_special = data.draw(st.booleans()) or g.n_special == 0 or keep_ref
    first = _nb(g) if keep_ref else 0
    nk = g.n_frames * _nb(g)
    K = data.draw(st.integers(1, nk - first))
    r = np.random.default_rng(seed + 1)
    nqb = g.n_frames * (_nb(g) + (1 if g.n_special else 0))
    idx = np.stack([np.stack([np.sort(r.choice(np.arange(first, nk), K, replace=False))
                              for _ in range(nqb)]) for _ in range(g.n_heads)]).astype(np.int32)
    o = L.fine_attention(q, k, v, g, 4, idx, keep_special=keep_special, keep_ref=keep_ref)
    for h in range(g.n_heads):
        mask = _fine_mask(g, idx[h], keep_special, keep_ref)
        _close(o[:, h], _sdpa(q[:, h], k[:, h], v[:, h], mask), 1e-12)


@PROPS
@given(geometries(), st.integers(0, 2 ** 31), st.booleans())
def test_gsa_all_blocks_forced_fine_is_dense(g, seed, keep_ref):
    keep_ref = keep_ref and g.n_frames > 1
    q, k, v = _qkv(g, seed)
    nk = g.n_frames * _nb(g) - (_nb(g) if keep_ref else 0)
    w = np.zeros((g.n_heads, 2, D))
    b = np.array([[-np.inf, np.inf]] * g.n_heads)
    out = L.gsa_layer(q, k, v, g, w, b, nk, keep_ref=keep_ref)
    _close(out["o"], L.dense_attention(q, k, v), 1e-12)


@PROPS
@given(geometries(), st.integers(0, 2 ** 31), st.integers(1, 4), st.integers(1, 4),
       st.sampled_from([0, 2]), st.booleans())
def test_subsampled_vs_masked_sdpa(g, seed, s_h, s_w, mode, log_count):
    q, k, v = _qkv(g, seed)
    T, N, Lf = g.n_tokens, g.n_frames, g.tokens_per_frame
    kept = np.zeros(T, dtype=bool)       # a special token or a patch on the stride grid
    for t in range(T):
        _, s, r, c = _token(g, t)
        kept[t] = s >= 0 or (r % s_h == 0 and c % s_w == 0)
    frame = np.arange(T) // Lf
    n_drop = int((~kept[:Lf]).sum())
    o = L.subsampled_attention(q, k, v, g, s_h, s_w, mode=mode, mean_log_count=log_count)
    for h in range(g.n_heads):
        means_k, means_v = [], []
        for f in range(N):
            drop = np.nonzero((frame == f) & ~kept)[0]
            if len(drop):
                means_k.append(k[drop, h].mean(axis=0))
                means_v.append(v[drop, h].mean(axis=0))
        ke = np.concatenate([k[:, h], np.array(means_k).reshape(-1, D)])
        ve = np.concatenate([v[:, h], np.array(means_v).reshape(-1, D)])
        bias = np.full((T, ke.shape[0]), -np.inf)
        for t in range(T):
            f = frame[t]
            for u in range(T):
                if mode == 0:
                    see = frame[u] == f or kept[u]
                else:               # token-level diagonal: every frame compacted, plus itself
                    see = kept[u] or u == t
                if see:
                    bias[t, u] = 0.0
            if n_drop:
                for fu in range(N):
                    if mode == 2 or fu != f:
                        bias[t, T + fu] = math.log(n_drop) if log_count else 0.0
        _close(o[:, h], _sdpa(q[:, h], ke, ve, bias), 1e-12)


@pytest.mark.parametrize("workers", [2, 4])
def test_head_map_threads_bit_identical(workers):
    """The oracle's thread pool only splits independent heads: every form
    returns bit-identical arrays with 1 and with several workers."""
    g = Geometry(3, 2, 7, 9, 4, D, "f32")
    q, k, v = _qkv(g, 5)
    r = np.random.default_rng(6)
    w, b = r.uniform(-0.125, 0.125, (4, 2, D)), r.uniform(-0.125, 0.125, (4, 2))
    rows = np.arange(0, g.n_tokens, 3)
    runs = []
    for n in (1, workers):
        gl = L.gsa_layer(q, k, v, g, w, b, 3, rows=rows, workers=n)
        runs.append([L.dense_attention(q, k, v, rows=rows, workers=n)] + [gl[key] for key in sorted(gl)] +
                    [L.subsampled_attention(q, k, v, g, 2, 3, rows=rows, workers=n),
                     L.subsampled_attention(q, k, v, g, 2, 3, mode=2, rows=rows, workers=n),
                     L.probability_block_scores(q, gl["k_cmp"], g, 4, [0, 3, 5], workers=n)])
    for a, c in zip(*runs):
        assert np.array_equal(a, c)
