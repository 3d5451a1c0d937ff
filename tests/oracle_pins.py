"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle (reached through
``oracle.layer`` at call time, so a test can plant a mistake in it) disagrees
with a closed form, an invariant, an independent library routine, a brute
force over a tiny input, or a count fixed by the pages and the workload
statement. ``test_oracle_pins.py`` runs them on the oracle as written;
``test_oracle_mutations.py`` plants plausible mistakes and checks that some pin
catches each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle.layer as L
from synth import Geometry

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(geom, seed, scale=1.0):
    r = _rng(seed)
    shape = (geom.n_tokens, geom.n_heads, geom.head_dim)
    return tuple(r.standard_normal(shape) * scale for _ in range(3))


def _close(a, b, tol=1e-11):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * max(1.0, np.max(np.abs(b)) if b.size else 1.0), err


def _sdpa(q, k, v, mask=None):
    """torch's scaled_dot_product_attention in fp64 on the CPU."""
    qt = torch.from_numpy(np.ascontiguousarray(q)).double()[None]
    kt = torch.from_numpy(np.ascontiguousarray(k)).double()[None]
    vt = torch.from_numpy(np.ascontiguousarray(v)).double()[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0].numpy()


G_SMALL = Geometry(3, 2, 5, 6, 2, 16, "f32")     # ragged 5x6 grid, 2 specials
G_FULL = Geometry(2, 0, 8, 8, 2, 16, "f32")      # full 4x4 windows, no specials


# --------------------------------------------------------------------- dense

def pin_hand_example():
    """A two-key softmax worked by hand (tests/golden/attend_hand.json)."""
    g = json.load(open(os.path.join(GOLDEN, "attend_hand.json")))
    o, lse = L.attend(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]))
    _close(o, g["o"], 1e-15)
    _close(lse, g["lse"], 1e-15)


def pin_dense_vs_sdpa():
    """Dense attention equals torch SDPA (fp64, CPU) head by head."""
    q, k, v = _qkv(G_SMALL, 1, 0.7)
    o = L.dense_attention(q, k, v)
    for h in range(G_SMALL.n_heads):
        _close(o[:, h], _sdpa(q[:, h], k[:, h], v[:, h]), 1e-12)


def pin_dense_lse():
    """The returned log-sum-exp equals log(sum(exp(q.k/sqrt(d)))) summed directly."""
    q, k, v = _qkv(G_SMALL, 2)
    _, lse = L.dense_attention(q, k, v, with_lse=True)
    d = G_SMALL.head_dim
    for h in range(G_SMALL.n_heads):
        s = q[:, h] @ k[:, h].T / math.sqrt(d)
        _close(lse[:, h], np.log(np.exp(s).sum(axis=1)), 1e-12)


def pin_dense_closed_forms():
    """Equal keys give the mean value; constant values give that constant; a
    single key gives its value; permuting keys changes nothing; a query that is
    a large multiple of one key (orthogonal keys) returns that key's value."""
    r = _rng(3)
    d = 8
    q = r.standard_normal((5, d))
    k1 = np.tile(r.standard_normal((1, d)), (7, 1))
    v = r.standard_normal((7, d))
    _close(L.attend(q, k1, v)[0], np.tile(v.mean(axis=0), (5, 1)), 1e-13)
    c = r.standard_normal(d)
    _close(L.attend(q, r.standard_normal((7, d)), np.tile(c, (7, 1)))[0], np.tile(c, (5, 1)), 1e-13)
    _close(L.attend(q, k1[:1], v[:1])[0], np.tile(v[0], (5, 1)), 1e-14)
    k = r.standard_normal((7, d))
    perm = r.permutation(7)
    _close(L.attend(q, k, v)[0], L.attend(q, k[perm], v[perm])[0], 1e-13)
    eye = np.eye(d)[:6] * 3.0
    qq = 40.0 * eye[4:5]
    o = L.attend(qq, eye, v[:6])[0]
    assert np.max(np.abs(o - v[4])) < 1e-9


def pin_frame_vs_masked_sdpa():
    """Frame attention equals SDPA with a block-diagonal frame mask."""
    q, k, v = _qkv(G_SMALL, 4)
    Lf = G_SMALL.tokens_per_frame
    f = np.arange(G_SMALL.n_tokens) // Lf
    mask = f[:, None] == f[None, :]
    o = L.frame_attention(q, k, v, G_SMALL)
    for h in range(G_SMALL.n_heads):
        _close(o[:, h], _sdpa(q[:, h], k[:, h], v[:, h], mask), 1e-12)


def pin_one_frame_global_is_frame():
    """With a single frame, global attention is frame attention."""
    g = G_SMALL.replace(n_frames=1)
    q, k, v = _qkv(g, 5)
    _close(L.dense_attention(q, k, v), L.frame_attention(q, k, v, g), 1e-13)


# -------------------------------------------------------------- compression

def pin_window_counts_37():
    """37x37 grid, 4x4 windows: 100 windows/frame with 81x16 + 18x4 + 1x1 valid
    tokens and 101 query blocks per frame (tests/golden/grid_37x37.json)."""
    gold = json.load(open(os.path.join(GOLDEN, "grid_37x37.json")))
    g = Geometry(1, 5, 37, 37, 1, 64, "bf16")
    win = L.window_table(g, 4)
    assert len(win) == gold["pooled_per_frame"]
    hist = {}
    for w in win:
        hist[str(len(w))] = hist.get(str(len(w)), 0) + 1
    assert hist == gold["window_valid_histogram"], hist
    assert sum(len(w) for w in win) == 37 * 37
    assert len(np.unique(np.concatenate(win))) == 37 * 37
    assert len(L.query_block_table(g, 4)) == gold["query_blocks_per_frame"]


def pin_pool_arithmetic():
    """On inputs K[t] = (row, col, 1) of the patch, every window mean is the
    mean row/col of its clipped extent -- known in closed form."""
    g = Geometry(2, 3, 7, 10, 1, 3, "f32")
    T = g.n_tokens
    k = np.zeros((T, 1, 3))
    Lf = g.tokens_per_frame
    for t in range(T):
        p = t % Lf - g.n_special
        if p >= 0:
            k[t, 0] = (p // g.grid_w, p % g.grid_w, 1.0)
        else:
            k[t, 0] = (-1.0, -1.0, 1.0)
    kc, vc = L.compress(k, k * 2.0, g, 4)
    nbw = 3
    for j in range(kc.shape[0]):
        by, bx = divmod(j % 6, nbw)
        r0, r1 = 4 * by, min(4 * by + 4, 7)
        c0, c1 = 4 * bx, min(4 * bx + 4, 10)
        _close(kc[j, 0], [(r0 + r1 - 1) / 2, (c0 + c1 - 1) / 2, 1.0], 1e-15)
        _close(vc[j, 0], 2.0 * kc[j, 0], 1e-15)


def pin_pooled_queries():
    """A window block's pooled query is the mean of its tokens; the special
    block's pooled query is the mean of the frame's special tokens."""
    q, _, _ = _qkv(G_SMALL, 6)
    qb = L.pooled_queries(q, G_SMALL, 4)
    Lf = G_SMALL.tokens_per_frame
    nqb = 2 * 2 + 1
    assert qb.shape[0] == G_SMALL.n_frames * nqb
    for f in range(G_SMALL.n_frames):
        _close(qb[f * nqb + 4], q[f * Lf:f * Lf + 2].mean(axis=0), 1e-14)
        # window (by=1, bx=0) covers grid row 4 and cols 0..3
        rows = [f * Lf + 2 + 4 * 6 + c for c in range(4)]
        _close(qb[f * nqb + 2], q[rows].mean(axis=0), 1e-14)


def pin_compressed_duplicate_keys():
    """Full 4x4 windows with keys/values constant inside each window: the
    compressed branch equals dense attention exactly (each pooled logit stands
    for 16 equal logits, which scale numerator and denominator alike)."""
    g = G_FULL
    q, k, v = _qkv(g, 7)
    for rows in L.window_table(g, 4):
        k[rows] = k[rows[0]]
        v[rows] = v[rows[0]]
    kc, vc = L.compress(k, v, g, 4)
    _close(L.compressed_attention(q, kc, vc), L.dense_attention(q, k, v), 1e-12)


def pin_block1_compression_is_dense():
    """With 1x1 windows and no special tokens, pooling is the identity and the
    compressed branch is dense attention."""
    g = G_FULL
    q, k, v = _qkv(g, 8)
    kc, vc = L.compress(k, v, g, 1)
    _close(kc, k, 0)
    _close(L.compressed_attention(q, kc, vc), L.dense_attention(q, k, v), 1e-13)


# ------------------------------------------------------------------ top-K

def pin_block_score_is_mean_token_logit():
    """The block score equals the mean over the block's tokens of the per-token
    compressed logits (the definition the pooled query rewrites)."""
    q, k, v = _qkv(G_SMALL, 9)
    kc, _ = L.compress(k, v, G_SMALL, 4)
    s = L.block_scores(L.pooled_queries(q, G_SMALL, 4), kc)
    d = G_SMALL.head_dim
    for b, rows in enumerate(L.query_block_table(G_SMALL, 4)):
        for h in range(G_SMALL.n_heads):
            per_token = q[rows, h] @ kc[:, h].T / math.sqrt(d)
            _close(s[h, b], per_token.mean(axis=0), 1e-13)


def _brute_topk(scores, K):
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    return sorted(order[:K]), [scores[j] for j in order[:K + 1]]


def pin_topk_brute_force():
    """Top-K equals a full sort by (score desc, index asc) on tiny inputs, for
    every K from 1 to all."""
    r = _rng(10)
    qb = r.standard_normal((6, 2, 8))
    kc = r.standard_normal((11, 2, 8))
    s = L.block_scores(qb, kc)
    for K in range(1, 12):
        idx, ranked = L.select_topk(qb, kc, K)
        for h in range(2):
            for b in range(6):
                want, wr = _brute_topk(list(s[h, b]), K)
                assert idx[h, b].tolist() == want, (K, h, b)
                _close(ranked[h, b, :len(wr)], wr, 1e-13)


def pin_topk_ties_lower_index():
    """Exactly tied scores resolve toward the lower pooled-block index."""
    r = _rng(11)
    base = r.standard_normal((5, 1, 8))
    kc = np.concatenate([base, base, base])  # every key three times: 0..4, 5..9, 10..14
    qb = r.standard_normal((4, 1, 8))
    s = L.block_scores(qb, kc)[0]
    for K in (1, 2, 3, 6, 7):
        idx, _ = L.select_topk(qb, kc, K)
        for b in range(4):
            best = np.argsort(-s[b, :5], kind="stable")
            want = []
            for j in best:          # copies of one key: lowest copy index first
                want += [j, j + 5, j + 10]
            assert idx[0, b].tolist() == sorted(want[:K]), (K, b)


def pin_topk_all():
    """K = number of pooled keys returns every block."""
    q, k, v = _qkv(G_SMALL, 12)
    kc, _ = L.compress(k, v, G_SMALL, 4)
    qb = L.pooled_queries(q, G_SMALL, 4)
    idx, _ = L.select_topk(qb, kc, kc.shape[0])
    assert (idx == np.arange(kc.shape[0])[None, None, :]).all()


def pin_topk_planted():
    """Designed pooled keys with known, well separated winners per block."""
    r = _rng(13)
    d, nk, nb = 16, 40, 7
    kc = r.standard_normal((nk, 1, d)) * 0.01
    qb = np.zeros((nb, 1, d))
    want = []
    for b in range(nb):
        win = sorted(r.choice(nk, 5, replace=False).tolist())
        qb[b, 0, b] = 1.0
        kc[win, 0, b] += 2.0 + np.arange(5)
        want.append(win)
    idx, _ = L.select_topk(qb, kc, 5)
    # block b's score against key j reads only coordinate b of k~_j
    for b in range(nb):
        assert idx[0, b].tolist() == want[b], (b, idx[0, b], want[b])


def pin_topk_first_brute_force():
    """With the first F pooled keys left out of the competition (the reference
    frame's blocks), top-K equals a full sort of the remaining keys' scores, in
    global indices, for every K."""
    r = _rng(26)
    qb = r.standard_normal((6, 2, 8))
    kc = r.standard_normal((11, 2, 8))
    s = L.block_scores(qb, kc)
    F = 4
    for K in range(1, 8):
        idx, ranked = L.select_topk(qb, kc, K, first=F)
        for h in range(2):
            for b in range(6):
                want, wr = _brute_topk(list(s[h, b, F:]), K)
                assert idx[h, b].tolist() == [F + j for j in want], (K, h, b)
                _close(ranked[h, b, :len(wr)], wr, 1e-13)


# ------------------------------------------------------------------- fine

def pin_fine_all_blocks_is_dense():
    """Selecting every pooled block (specials always kept) is dense attention."""
    q, k, v = _qkv(G_SMALL, 14)
    nb, nqb = G_SMALL.n_frames * 4, G_SMALL.n_frames * 5
    idx = np.tile(np.arange(nb, dtype=np.int32), (G_SMALL.n_heads, nqb, 1))
    _close(L.fine_attention(q, k, v, G_SMALL, 4, idx), L.dense_attention(q, k, v), 1e-12)


def pin_fine_single_corner_token():
    """No special tokens, K = 1 and the selected block the 1x1 corner window of
    a 37x37 grid: every query of the block returns that token's value."""
    g = Geometry(1, 0, 37, 37, 1, 8, "f32")
    q, k, v = _qkv(g, 15)
    nqb = 100
    idx = np.full((1, nqb, 1), 99, dtype=np.int32)   # window (by=9, bx=9)
    rows = np.arange(0, g.n_tokens, 97)
    o = L.fine_attention(q, k, v, g, 4, idx, rows=rows)
    corner = 36 * 37 + 36
    _close(o, np.tile(v[corner], (len(rows), 1, 1)), 1e-15)


def _fine_mask(g, idx_h, keep_special=True, keep_ref=False):
    """Key mask of the fine branch built token by token: query t sees key u
    when u is a special token (and specials are kept), when u lies in frame 0
    and the reference frame is kept, or when u's 4x4 window is selected for
    t's query block. Needs a grid of at most 8 columns (2 windows per row)."""
    Lf, S = g.tokens_per_frame, g.n_special
    nbw = -(-g.grid_w // 4)
    nb = nbw * -(-g.grid_h // 4)
    nqb = nb + (1 if S else 0)
    mask = np.zeros((g.n_tokens, g.n_tokens), dtype=bool)
    for t in range(g.n_tokens):
        f, p = divmod(t, Lf)
        if p < S:
            b = f * nqb + nb
        else:
            rr, cc = divmod(p - S, g.grid_w)
            b = f * nqb + (rr // 4) * nbw + cc // 4
        for u in range(g.n_tokens):
            fu, pu = divmod(u, Lf)
            if keep_ref and fu == 0:
                mask[t, u] = True
            elif pu < S:
                mask[t, u] = keep_special
            else:
                ru, cu = divmod(pu - S, g.grid_w)
                mask[t, u] = fu * nb + (ru // 4) * nbw + cu // 4 in idx_h[b]
    return mask


def pin_fine_vs_masked_sdpa():
    """Fine attention equals SDPA with an explicit per-query key mask built
    token by token from the selected windows and the special tokens."""
    g = G_SMALL
    q, k, v = _qkv(g, 16)
    r = _rng(17)
    nb, nqb = g.n_frames * 4, g.n_frames * 5
    idx = np.stack([np.stack([np.sort(r.choice(nb, 3, replace=False)) for _ in range(nqb)])
                    for _ in range(g.n_heads)]).astype(np.int32)
    o = L.fine_attention(q, k, v, g, 4, idx)
    for h in range(g.n_heads):
        _close(o[:, h], _sdpa(q[:, h], k[:, h], v[:, h], _fine_mask(g, idx[h])), 1e-12)


def pin_ref_frame_vs_masked_sdpa():
    """The VGGT adaptation: with the reference frame kept, fine attention equals
    SDPA under the token-by-token mask that adds all of frame 0 to the selected
    windows (drawn from frames 1..N-1), with and without the special tokens."""
    g = G_SMALL
    q, k, v = _qkv(g, 24)
    r = _rng(25)
    nqb = g.n_frames * 5
    idx = np.stack([np.stack([np.sort(r.choice(np.arange(4, g.n_frames * 4), 3, replace=False))
                              for _ in range(nqb)]) for _ in range(g.n_heads)]).astype(np.int32)
    for keep_special in (True, False):
        o = L.fine_attention(q, k, v, g, 4, idx, keep_special=keep_special, keep_ref=True)
        for h in range(g.n_heads):
            mask = _fine_mask(g, idx[h], keep_special=keep_special, keep_ref=True)
            _close(o[:, h], _sdpa(q[:, h], k[:, h], v[:, h], mask), 1e-12)
    rows = L.fine_key_rows(g, 4, idx[0, 0], keep_special=True, keep_ref=True)
    want = np.nonzero(_fine_mask(g, idx[0], keep_ref=True)[g.n_special])[0]  # a query of block 0
    assert sorted(rows.tolist()) == want.tolist()


# ------------------------------------------------------------------- gate

def pin_gate_special_cases():
    """W=0, b=0 gives the half sum; b = (-inf, +inf) gives the fine branch;
    b = (+inf, -inf) the compressed branch; the gate equals scipy's expit."""
    from scipy.special import expit
    r = _rng(18)
    q, a, c = (r.standard_normal((9, 2, 8)) for _ in range(3))
    w0 = np.zeros((2, 2, 8))
    _close(L.gate(q, a, c, w0, np.zeros((2, 2))), 0.5 * (a + c), 1e-15)
    _close(L.gate(q, a, c, w0, np.tile([-np.inf, np.inf], (2, 1))), c, 0)
    _close(L.gate(q, a, c, w0, np.tile([np.inf, -np.inf], (2, 1))), a, 0)
    w = r.standard_normal((2, 2, 8))
    b = r.standard_normal((2, 2))
    z = np.einsum("thd,hgd->thg", q, w) + b
    want = expit(z[..., :1]) * a + expit(z[..., 1:]) * c
    _close(L.gate(q, a, c, w, b), want, 1e-14)


def pin_gsa_forced_fine_all_is_dense():
    """The whole GSA layer with K = all blocks and the gate forced to the fine
    branch is dense attention."""
    g = G_SMALL
    q, k, v = _qkv(g, 19)
    nb = g.n_frames * 4
    w = np.zeros((g.n_heads, 2, g.head_dim))
    b = np.tile([-np.inf, np.inf], (g.n_heads, 1))
    out = L.gsa_layer(q, k, v, g, w, b, top_k=nb)
    _close(out["o"], L.dense_attention(q, k, v), 1e-12)


def pin_gsa_ref_frame_all_is_dense():
    """The VGGT adaptation with K = every block outside the reference frame and
    the gate forced to the fine branch is dense attention: every token is
    attended exactly once, frame 0 through the kept reference frame."""
    g = G_SMALL
    q, k, v = _qkv(g, 27)
    w = np.zeros((g.n_heads, 2, g.head_dim))
    b = np.tile([-np.inf, np.inf], (g.n_heads, 1))
    out = L.gsa_layer(q, k, v, g, w, b, top_k=(g.n_frames - 1) * 4, keep_ref=True)
    assert out["idx"].min() >= 4
    _close(out["o"], L.dense_attention(q, k, v), 1e-12)


# ------------------------------------------------------------- subsampled

def pin_sga_counts_37():
    """37x37 at stride 4x4 keeps 100 patches, drops 1269, and a query sees its
    1374 own-frame tokens plus 106 per other frame (tests/golden/grid_37x37.json)."""
    gold = json.load(open(os.path.join(GOLDEN, "grid_37x37.json")))
    g = Geometry(3, 5, 37, 37, 1, 4, "f32")
    kept, dropped = L.subsample_plan(g, 4, 4)
    assert len(kept) == gold["kept_patches_per_frame"]
    assert len(dropped) == gold["dropped_patches_per_frame"]
    ck, _ = L.sga_compact(np.zeros((g.n_tokens, 1, 4)), np.zeros((g.n_tokens, 1, 4)), g, 4, 4)
    assert ck.shape[0] == 3 * gold["compacted_per_frame"]
    m = gold["compacted_per_frame"]
    assert 1374 + 255 * m == gold["keys_per_query_N256"]
    assert 1374 + 999 * m == gold["keys_per_query_N1000"]


def pin_sga_kept_rows_exact():
    """Kept rows of the compacted set are bit-exact copies of K/V rows: the
    specials, then the (r % s_h == 0, c % s_w == 0) patches, then the mean of
    the dropped patches."""
    g = G_SMALL
    q, k, v = _qkv(g, 20)
    ck, cv = L.sga_compact(k, v, g, 2, 3)
    Lf = g.tokens_per_frame
    keep = [0, 1] + [2 + r * 6 + c for r in range(0, 5, 2) for c in range(0, 6, 3)]
    drop = [2 + r * 6 + c for r in range(5) for c in range(6) if r % 2 or c % 3]
    m = len(keep) + 1
    for f in range(g.n_frames):
        assert np.array_equal(ck[f * m:f * m + len(keep)], k[[f * Lf + p for p in keep]])
        assert np.array_equal(cv[f * m:f * m + len(keep)], v[[f * Lf + p for p in keep]])
        _close(ck[f * m + m - 1], k[[f * Lf + p for p in drop]].mean(axis=0), 1e-14)
        _close(cv[f * m + m - 1], v[[f * Lf + p for p in drop]].mean(axis=0), 1e-14)


def pin_sga_stride1_is_dense():
    """Stride 1x1 drops nothing (no mean token): subsampled attention is dense."""
    q, k, v = _qkv(G_SMALL, 21)
    _close(L.subsampled_attention(q, k, v, G_SMALL, 1, 1), L.dense_attention(q, k, v), 1e-12)


def pin_sga_one_frame_and_frame_mode():
    """One frame: subsampled = frame attention; frame mode = frame attention."""
    g1 = G_SMALL.replace(n_frames=1)
    q, k, v = _qkv(g1, 22)
    _close(L.subsampled_attention(q, k, v, g1, 2, 2), L.frame_attention(q, k, v, g1), 1e-12)
    q, k, v = _qkv(G_SMALL, 23)
    _close(L.subsampled_attention(q, k, v, G_SMALL, 2, 2, mode=1),
           L.frame_attention(q, k, v, G_SMALL), 1e-13)


def pin_sga_log_count_identity():
    """When every dropped patch of a frame carries the same key and value, the
    mean token with log(#dropped) added to its logit stands exactly for the
    dropped columns: subsampled attention equals dense attention."""
    g = G_SMALL
    q, k, v = _qkv(g, 24)
    Lf = g.tokens_per_frame
    _, dropped = L.subsample_plan(g, 2, 2)
    for f in range(g.n_frames):
        rows = [f * Lf + p for p in dropped]
        k[rows] = k[rows[0]]
        v[rows] = v[rows[0]]
    _close(L.subsampled_attention(q, k, v, g, 2, 2, mean_log_count=True),
           L.dense_attention(q, k, v), 1e-12)


def pin_sga_vs_explicit_keys():
    """Subsampled attention equals attention over an explicitly enumerated key
    list (own frame + per other frame: specials, kept patches, dropped mean)."""
    g = G_SMALL
    q, k, v = _qkv(g, 25)
    Lf = g.tokens_per_frame
    o = L.subsampled_attention(q, k, v, g, 2, 3)
    d = g.head_dim
    for t in range(0, g.n_tokens, 3):
        f = t // Lf
        for h in range(g.n_heads):
            keys, vals = [], []
            for u in range(g.n_tokens):
                fu, pu = divmod(u, Lf)
                if fu == f:
                    keys.append(k[u, h]); vals.append(v[u, h])
                elif pu < g.n_special:
                    keys.append(k[u, h]); vals.append(v[u, h])
                else:
                    rr, cc = divmod(pu - g.n_special, g.grid_w)
                    if rr % 2 == 0 and cc % 3 == 0:
                        keys.append(k[u, h]); vals.append(v[u, h])
            for fu in range(g.n_frames):
                if fu == f:
                    continue
                drop = [fu * Lf + g.n_special + rr * g.grid_w + cc for rr in range(g.grid_h)
                        for cc in range(g.grid_w) if rr % 2 or cc % 3]
                keys.append(k[drop, h].mean(axis=0)); vals.append(v[drop, h].mean(axis=0))
            s = np.array(keys) @ q[t, h] / math.sqrt(d)
            p = np.exp(s - s.max())
            _close(o[t, h], p @ np.array(vals) / p.sum(), 1e-12)



def pin_sga_token_diagonal_vs_explicit_keys():
    """The token-level diagonal reading (mode 2) equals attention over an
    explicitly enumerated key list: per frame, own frame included, its
    specials, its kept patches and the mean of its dropped patches (with
    log(#dropped) on the mean's logit when asked), plus the query's own key
    when its patch was dropped."""
    g = G_SMALL
    q, k, v = _qkv(g, 26)
    Lf = g.tokens_per_frame
    d = g.head_dim
    for log_count in (False, True):
        o = L.subsampled_attention(q, k, v, g, 2, 3, mode=2, mean_log_count=log_count)
        for t in range(0, g.n_tokens, 2):
            for h in range(g.n_heads):
                keys, vals, bias = [], [], []
                for u in range(g.n_tokens):
                    pu = u % Lf
                    rr, cc = divmod(pu - g.n_special, g.grid_w)
                    if pu < g.n_special or (rr % 2 == 0 and cc % 3 == 0) or u == t:
                        keys.append(k[u, h]); vals.append(v[u, h]); bias.append(0.0)
                for fu in range(g.n_frames):
                    drop = [fu * Lf + g.n_special + rr * g.grid_w + cc for rr in range(g.grid_h)
                            for cc in range(g.grid_w) if rr % 2 or cc % 3]
                    keys.append(k[drop, h].mean(axis=0)); vals.append(v[drop, h].mean(axis=0))
                    bias.append(math.log(len(drop)) if log_count else 0.0)
                s_ = np.array(keys) @ q[t, h] / math.sqrt(d) + np.array(bias)
                p_ = np.exp(s_ - s_.max())
                _close(o[t, h], p_ @ np.array(vals) / p_.sum(), 1e-12)


def pin_sga_token_diagonal_stride1_is_dense():
    """Stride 1x1 drops nothing: the token-level diagonal reading is dense."""
    q, k, v = _qkv(G_SMALL, 27)
    _close(L.subsampled_attention(q, k, v, G_SMALL, 1, 1, mode=2), L.dense_attention(q, k, v), 1e-12)


def pin_pooled_compressed_equal_queries():
    """Block-level compressed branch (R18): when every token of a query block
    carries the same query, it equals the token-level branch."""
    g = G_SMALL
    q, k, v = _qkv(g, 28)
    for members in L.query_block_table(g, 4):
        q[members] = q[members[0]]
    kc, vc = L.compress(k, v, g, 4)
    _close(L.compressed_attention_pooled(q, kc, vc, g, 4), L.compressed_attention(q, kc, vc), 1e-13)


def pin_pooled_compressed_vs_sdpa():
    """Block-level compressed branch (R18) against torch SDPA over the pooled
    keys for each block's mean query, formed token by token from the grid
    (4x4 windows clipped to the grid, a frame's specials as one block), then
    copied to every token of the block; also on a row subset."""
    g = G_SMALL
    q, k, v = _qkv(g, 29)
    kc, vc = L.compress(k, v, g, 4)
    o = L.compressed_attention_pooled(q, kc, vc, g, 4)
    Lf, S = g.tokens_per_frame, g.n_special
    for h in range(g.n_heads):
        for t in range(g.n_tokens):
            f, p = divmod(t, Lf)
            if p < S:
                members = [f * Lf + s for s in range(S)]
            else:
                r, c = divmod(p - S, g.grid_w)
                members = [f * Lf + S + rr * g.grid_w + cc for rr in range(g.grid_h)
                           for cc in range(g.grid_w) if rr // 4 == r // 4 and cc // 4 == c // 4]
            qb = q[members, h].mean(axis=0)
            want = _sdpa(qb[None], kc[:, h], vc[:, h])[0]
            _close(o[t, h], want, 1e-12)
    rows = np.array([0, 3, 17, 40, g.n_tokens - 1])
    _close(L.compressed_attention_pooled(q, kc, vc, g, 4, rows=rows), o[rows], 0)


def pin_pool_zero_padded():
    """Zero-padded pooling (R19) equals numpy: the grid padded with zeros to
    whole 4x4 windows, reshaped into windows and averaged over all 16 slots;
    on a grid of whole windows it equals the valid-token mean (R4)."""
    g = G_SMALL
    q, k, v = _qkv(g, 30)
    kc, vc = L.compress(k, v, g, 4, include_pad=True)
    Lf, S = g.tokens_per_frame, g.n_special
    nbh, nbw = -(-g.grid_h // 4), -(-g.grid_w // 4)
    for f in range(g.n_frames):
        for x, xc in ((k, kc), (v, vc)):
            grid = x[f * Lf + S:(f + 1) * Lf].reshape(g.grid_h, g.grid_w, g.n_heads, g.head_dim)
            pad = np.zeros((4 * nbh, 4 * nbw, g.n_heads, g.head_dim))
            pad[:g.grid_h, :g.grid_w] = grid
            want = pad.reshape(nbh, 4, nbw, 4, g.n_heads, g.head_dim).mean(axis=(1, 3))
            _close(xc[f * nbh * nbw:(f + 1) * nbh * nbw], want.reshape(-1, g.n_heads, g.head_dim),
                   1e-14)
    q, k, v = _qkv(G_FULL, 31)
    for a, b in zip(L.compress(k, v, G_FULL, 4, include_pad=True), L.compress(k, v, G_FULL, 4)):
        _close(a, b, 1e-15)

# ------------------------------------------------- probability block score (R20)

def _prob_inputs(seed):
    q, k, v = _qkv(G_SMALL, seed)
    kc, _ = L.compress(k, v, G_SMALL, 4)
    return q, kc


def pin_probability_scores_sum_to_one():
    """Each token's compressed probabilities sum to one, so a block's mean of
    them does too: summed over every pooled key, each block's scores are 1."""
    q, kc = _prob_inputs(30)
    blocks = list(range(G_SMALL.n_frames * 5))
    sc = L.probability_block_scores(q, kc, G_SMALL, 4, blocks)
    _close(sc.sum(axis=2), np.ones(sc.shape[:2]), 1e-13)
    assert (sc > 0).all()


def pin_probability_scores_brute_force():
    """R20 against a plain loop over tokens and keys (tiny input): softmax of
    each token's scaled logits over all pooled keys, averaged over the
    block's valid tokens; with the first F keys out of the competition the
    returned scores are the same numbers for the other keys."""
    q, kc = _prob_inputs(31)
    H, d = q.shape[1], q.shape[2]
    qbt = L.query_block_table(G_SMALL, 4)
    blocks = [0, 3, 4, 9, 14]          # full, edge and corner windows, a specials block
    F = 4
    sc = L.probability_block_scores(q, kc, G_SMALL, 4, blocks)
    scf = L.probability_block_scores(q, kc, G_SMALL, 4, blocks, first=F)
    for h in range(H):
        for i, bb in enumerate(blocks):
            rows = list(qbt[bb])
            want = [0.0] * kc.shape[0]
            for t in rows:
                logits = [sum(q[t, h, e] * kc[j, h, e] for e in range(d)) / math.sqrt(d)
                          for j in range(kc.shape[0])]
                z = sum(math.exp(x) for x in logits)
                for j in range(kc.shape[0]):
                    want[j] += math.exp(logits[j]) / z / len(rows)
            _close(sc[h, i], want, 1e-12)
            _close(scf[h, i], want[F:], 1e-12)


def pin_probability_equal_queries_is_logit_order():
    """When every token of a block has the same query, its probability-mean
    scores are that query's softmax over the pooled keys -- a monotone map of
    the R2 logits -- so both readings select the same blocks, in the same rank
    order, and the log scores differ from the logits by one constant."""
    q, kc = _prob_inputs(32)
    qbt = L.query_block_table(G_SMALL, 4)
    for members in qbt:               # each block's tokens take its first token's query
        q[members] = q[members[0]]
    blocks = list(range(len(qbt)))
    q_blk = L.pooled_queries(q, G_SMALL, 4, blocks=blocks)
    for K in (1, 3, 6, kc.shape[0]):
        i_p, r_p = L.select_topk_probability(q, kc, G_SMALL, K, 4, blocks)
        i_l, r_l = L.select_topk(q_blk, kc, K)
        assert np.array_equal(i_p, i_l), K
        assert np.array_equal(np.isinf(r_p), np.isinf(r_l)), K   # K = all: no (K+1)-th, -inf
        fin = np.isfinite(r_l)
        diff = r_p[fin] - r_l[fin]                                 # one constant per (head, block)
        first = np.broadcast_to((r_p[..., :1] - r_l[..., :1]), r_l.shape)[fin]
        _close(diff, first, 1e-12)


def pin_probability_key_shift_invariance():
    """Adding one vector c to every pooled key shifts each token's logits by the
    constant q.c/sqrt(d): its softmax, and so the scores, stay the same."""
    q, kc = _prob_inputs(33)
    blocks = [0, 2, 5, 9]
    c = _rng(34).standard_normal((1,) + kc.shape[1:]) * 2.0
    a = L.probability_block_scores(q, kc, G_SMALL, 4, blocks)
    b = L.probability_block_scores(q, kc + c, G_SMALL, 4, blocks)
    _close(a, b, 1e-10)


ALL_PINS = [obj for name, obj in sorted(globals().items()) if name.startswith("pin_")]
