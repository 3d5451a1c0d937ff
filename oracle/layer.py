"""Plain fp64 definitions of the global cross-frame attention layer.

TEST INFRASTRUCTURE ONLY -- imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library.

Sources (web pages, cited by page title and section):

* [Speed3R-ja] "Speed3R: Sparse Feed-forward 3D Reconstruction Models",
  Japanese technical summary, section 2.1 (dual-branch attention:
  compression branch, selection branch, gated aggregation) and section 2.2
  (streaming top-K inside a FlashAttention-style loop).
* [Speed3R-it] the same paper, Italian technical summary ("Sommario tecnico"),
  section 2 "Metodologia" (S_guide score matrix, selection guided by it,
  gated fusion; camera tokens kept in the VGGT adaptation).
* [AVGGT] "AVGGT: Rethinking Global Attention for Accelerating VGGT",
  technical summary section 2.2 (global-to-frame conversion; subsampled global
  attention with all queries and special tokens kept, the diagonal kept and
  the dropped columns replaced by one mean key/value pair).
* [VGG-T3] "VGG-T3" technical summary section 1 (softmax attention of every
  query over the keys/values of all input image tokens, O(N^2)).

Readings taken where the pages leave a step open (each is restated where it is
used):

R1  the compressed branch attends full-resolution queries over pooled K/V, so
    the "upsampling back to full resolution" is the identity;
R2  the block score used for selection is the mean over the query block's
    tokens of q.k~/sqrt(d), i.e. the pooled query's logit against k~;
R3  query blocks are the same 4x4 windows as the K/V pooling, plus one block
    holding a frame's special tokens;
R4  pooling windows that overhang the grid average their valid tokens only;
R5  special tokens are never pooled and are always attended by the fine branch;
R6  top-K per head and query block, ties to the lower block index, the index
    set returned in ascending order;
R7  gate g = sigmoid(q . W[h]^T + b[h]) in (0,1)^2, o = g0*o_cmp + g1*o_slc;
R8  softmax scale 1/sqrt(d) everywhere;
R9  the subsampled form keeps the query's own frame whole;
R10 a patch (r, c) is kept iff r % s_h == 0 and c % s_w == 0;
R11 one mean key/value per *other* frame, the plain mean of that frame's
    dropped patches, entering the softmax as one ordinary key (optionally with
    log(#dropped) added to its logit); omitted when nothing is dropped;
R12 token order inside a frame: special tokens first, then patches row-major;
R15 the VGGT adaptation of the selection branch ([Speed3R-ja] section 2.2,
    architecture adaptation; [Speed3R-it] section 2) keeps the reference frame
    -- frame 0, whose camera fixes VGGT's world coordinates -- whole: every
    query's fine branch attends to all tokens of frame 0, and the top-K is
    taken over the pooled blocks of the other frames only, so that no token is
    counted twice;
R17 AVGGT's "diagonal" read at token level (the alternative to R9, mode 2):
    the query's own frame is subsampled like every other frame (its compacted
    set and mean token included), and the query's own key/value is added when
    its patch was dropped; the means stay per frame, over all dropped patches;
R18 the compressed branch read at block level (the alternative to R1): each
    query block's mean query attends over the pooled keys/values and every
    token of the block takes that output (nearest upsampling);
R19 the grid zero-padded to whole windows before the 4x4 average (the
    alternative to R4): a window that overhangs the grid sums its in-grid
    tokens and divides by 16. The mean queries of the query blocks (R2, R3)
    stay over their tokens.
R20 the block score read as probabilities (the alternative to R2): the mean
    over the query block's tokens of their compressed-branch softmax
    probabilities, p_tj = exp(s_tj - lse_t) with lse_t over all N*nb pooled
    keys (with R15 frame 0's blocks still normalise, they only do not
    compete); ties and order as R6.

Arrays are ``[rows, H, d]`` of any float dtype; every computation widens them
to fp64 first.
"""
from __future__ import annotations

import math
import os
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "attend", "attend_union", "dense_attention", "frame_attention", "window_table",
    "query_block_table", "compress", "pooled_queries", "compressed_attention",
    "compressed_attention_pooled",
    "block_scores", "select_topk", "probability_block_scores", "select_topk_probability",
    "fine_key_rows", "fine_attention", "gate",
    "gsa_layer", "subsample_plan", "sga_compact", "subsampled_attention",
    "head_map",
]


# ---------------------------------------------------------------------------
# the primitive
# ---------------------------------------------------------------------------

def attend(q, k, v, bias=None):
    """Softmax attention of query rows ``q`` [m, d] over keys ``k``/``v`` [n, d].

    s = q k^T / sqrt(d) (+ bias), p = exp(s - max s), o = p v / sum p: a plain
    two-pass softmax in fp64 (R8; [VGG-T3] section 1 states the operation).
    ``bias`` [n] or [m, n] adds to the logits (-inf removes a key).
    Returns (o [m, d], lse [m]) with lse = log sum exp(s).
    """
    return attend_union(q, [(k, v, bias)])


def attend_union(q, parts):
    """``attend`` over the union of several key sets, each given separately as
    (k [n_i, d], v [n_i, d], bias or None); one softmax spans all of them."""
    q = np.asarray(q, dtype=np.float64)
    scale = 1.0 / math.sqrt(q.shape[-1])
    scores = []
    for k, v, bias in parts:
        s = (q @ np.asarray(k, dtype=np.float64).T) * scale
        if bias is not None:
            s = s + bias
        scores.append(s)
    m = np.max([s.max(axis=1) for s in scores], axis=0)[:, None]
    num = np.zeros((q.shape[0], np.asarray(parts[0][1]).shape[-1]))
    den = np.zeros((q.shape[0], 1))
    for s, (k, v, bias) in zip(scores, parts):
        p = np.exp(s - m)
        num += p @ np.asarray(v, dtype=np.float64)
        den += p.sum(axis=1, keepdims=True)
    return num / den, (m + np.log(den))[:, 0]


def head_map(fn, n_heads: int, workers: Optional[int] = None):
    """Run ``fn(h)`` for every head, on a pool of threads when asked.

    Parallelism only splits independent heads (NumPy releases the interpreter
    lock inside its array kernels); the arithmetic of ``fn`` is unchanged.
    ``workers`` defaults to $ORACLE_WORKERS or 1. BLAS runs single-threaded
    inside the pool.
    """
    if workers is None:
        workers = int(os.environ.get("ORACLE_WORKERS", "1"))
    if workers <= 1 or n_heads == 1:
        return [fn(h) for h in range(n_heads)]
    from concurrent.futures import ThreadPoolExecutor
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limit = None
    try:
        with ThreadPoolExecutor(max_workers=min(workers, n_heads)) as ex:
            return list(ex.map(fn, range(n_heads)))
    finally:
        if limit is not None:
            limit.restore_original_limits()


def _rows(rows, T):
    return np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)


def _frame_len(geom) -> int:
    return geom.n_special + geom.grid_h * geom.grid_w


# ---------------------------------------------------------------------------
# dense and frame attention
# ---------------------------------------------------------------------------

def dense_attention(q, k, v, rows=None, chunk: int = 64, workers=None, with_lse=False):
    """Every query attends to every key of all frames ([VGG-T3] section 1;
    [Speed3R-ja] section 1; [AVGGT] section 1)."""
    T, H, d = k.shape
    rows = _rows(rows, q.shape[0])

    def one_head(h):
        kh = np.asarray(k[:, h, :], dtype=np.float64)
        vh = np.asarray(v[:, h, :], dtype=np.float64)
        o = np.empty((len(rows), d))
        lse = np.empty(len(rows))
        for a in range(0, len(rows), chunk):
            sl = slice(a, a + chunk)
            o[sl], lse[sl] = attend(q[rows[sl], h, :], kh, vh)
        return o, lse

    res = head_map(one_head, H, workers)
    o = np.stack([r[0] for r in res], axis=1)
    if with_lse:
        return o, np.stack([r[1] for r in res], axis=1)
    return o


def frame_attention(q, k, v, geom, rows=None, with_lse=False):
    """Attention restricted to the query's own frame: the global-to-frame
    conversion of the early layers ([AVGGT] section 2.2)."""
    T, H, d = k.shape
    L = _frame_len(geom)
    rows = _rows(rows, T)
    o = np.empty((len(rows), H, d))
    lse = np.empty((len(rows), H))
    frames = rows // L
    for f in np.unique(frames):
        sel = np.nonzero(frames == f)[0]
        keys = slice(f * L, (f + 1) * L)
        for h in range(H):
            o[sel, h], lse[sel, h] = attend(q[rows[sel], h, :], k[keys, h, :], v[keys, h, :])
    return (o, lse) if with_lse else o


# ---------------------------------------------------------------------------
# Global Sparse Attention: compression branch
# ---------------------------------------------------------------------------

def window_table(geom, block: int) -> List[np.ndarray]:
    """Token rows of every pooling window, in global compressed-key order.

    Window (f, by, bx) covers patch rows block*by .. block*by+block-1 and
    columns block*bx .. block*bx+block-1 of frame f, clipped to the grid (R4),
    and gets global index f*nb + by*nbw + bx with nbw = ceil(grid_w/block).
    Special tokens belong to no window (R5).
    """
    gh, gw, S = geom.grid_h, geom.grid_w, geom.n_special
    L = _frame_len(geom)
    nbh, nbw = -(-gh // block), -(-gw // block)
    out = []
    for f in range(geom.n_frames):
        for by in range(nbh):
            for bx in range(nbw):
                rows = []
                for r in range(block * by, min(block * by + block, gh)):
                    for c in range(block * bx, min(block * bx + block, gw)):
                        rows.append(f * L + S + r * gw + c)
                out.append(np.array(rows, dtype=np.int64))
    return out


def query_block_table(geom, block: int) -> List[np.ndarray]:
    """Token rows of every query block (R3): the pooling windows of a frame in
    the same order, then (when the frame has special tokens) one block holding
    them. Global index f*nqb + j, nqb = nb + (1 if n_special else 0)."""
    gh, gw, S = geom.grid_h, geom.grid_w, geom.n_special
    L = _frame_len(geom)
    nb = (-(-gh // block)) * (-(-gw // block))
    per_frame = window_table(_one_frame(geom), block)
    out = []
    for f in range(geom.n_frames):
        for j in range(nb):
            out.append(per_frame[j] + f * L)
        if S:
            out.append(np.arange(f * L, f * L + S, dtype=np.int64))
    return out


class _one_frame:
    def __init__(self, geom):
        self.n_frames, self.n_special = 1, geom.n_special
        self.grid_h, self.grid_w = geom.grid_h, geom.grid_w


def compress(k, v, geom, block: int = 4, include_pad: bool = False):
    """4x4 average pooling of keys and values into the coarse context
    ([Speed3R-ja] section 2.1, compression branch, first bullet;
    [Speed3R-it] section 2, "Ramo di Compressione"). Mean over the valid
    tokens of each window (R4); with ``include_pad`` the grid is zero-padded to
    whole windows and every window is divided by block^2 (R19).
    Returns fp64 (k_cmp, v_cmp) [N*nb, H, d]."""
    win = window_table(geom, block)
    H, d = k.shape[1], k.shape[2]
    kc = np.empty((len(win), H, d))
    vc = np.empty((len(win), H, d))
    for j, rows in enumerate(win):
        den = block * block if include_pad else len(rows)
        kc[j] = np.asarray(k[rows], dtype=np.float64).sum(axis=0) / den
        vc[j] = np.asarray(v[rows], dtype=np.float64).sum(axis=0) / den
    return kc, vc


def pooled_queries(q, geom, block: int = 4, blocks: Optional[Sequence[int]] = None):
    """Mean query of every query block (R2, R3): fp64 [n_blocks, H, d]."""
    qb = query_block_table(geom, block)
    if blocks is None:
        blocks = range(len(qb))
    return np.stack([np.asarray(q[qb[b]], dtype=np.float64).mean(axis=0) for b in blocks])


def compressed_attention(q, k_cmp, v_cmp, rows=None, chunk: int = 256, workers=None):
    """Full-resolution queries attend over all pooled keys/values of all frames
    ([Speed3R-ja] section 2.1, compression branch, second and third bullets;
    R1: per-token outputs, so the upsampling step is the identity)."""
    return dense_attention(q, k_cmp, v_cmp, rows=rows, chunk=chunk, workers=workers)


def compressed_attention_pooled(q, k_cmp, v_cmp, geom, block: int = 4, rows=None, workers=None):
    """The compressed branch at block level (R18): the mean query of every
    query block (R3) attends over all pooled keys/values; each token takes its
    block's output, i.e. the coarse result upsampled to full resolution by
    nearest neighbour ([Speed3R-ja] section 2.1, compression branch)."""
    T = q.shape[0]
    rows = _rows(rows, T)
    qbt = query_block_table(geom, block)
    owner = np.empty(T, dtype=np.int64)
    for b, members in enumerate(qbt):
        owner[members] = b
    need = np.unique(owner[rows])
    o_blk = dense_attention(pooled_queries(q, geom, block, blocks=need), k_cmp, v_cmp,
                            workers=workers)
    pos = np.searchsorted(need, owner[rows])
    return o_blk[pos]


# ---------------------------------------------------------------------------
# Global Sparse Attention: selection branch
# ---------------------------------------------------------------------------

def block_scores(q_blk, k_cmp):
    """Compressed-space score of every (query block, pooled key) pair, per head:
    S[h, b, j] = q_blk[b, h] . k_cmp[j, h] / sqrt(d) (R2; the S_guide matrix of
    [Speed3R-it] section 2). Returns fp64 [H, n_blocks, n_keys]."""
    qb = np.asarray(q_blk, dtype=np.float64)
    kc = np.asarray(k_cmp, dtype=np.float64)
    d = qb.shape[-1]
    return np.einsum("bhd,jhd->hbj", qb, kc) / math.sqrt(d)


def _topk_rows(s, top_k: int, first: int):
    """Top-K of each row of s [n, nk] (larger first, ties to the lower column,
    R6): (idx [n, K] int32 ascending, offset by ``first``; ranked [n, K+1]
    fp64, the K+1 best in rank order, -inf padded)."""
    n, nk = s.shape
    m = min(top_k + 1, nk)
    idx = np.empty((n, top_k), dtype=np.int32)
    ranked = np.full((n, top_k + 1), -np.inf)
    # every key ranked within the first m scores at least the m-th largest
    thr = np.partition(s, nk - m, axis=1)[:, nk - m]
    for i in range(n):
        row = s[i]
        cand = np.nonzero(row >= thr[i])[0]
        order = sorted(cand.tolist(), key=lambda j: (-row[j], j))
        idx[i] = first + np.sort(np.array(order[:top_k], dtype=np.int32))
        ranked[i, :m] = row[order[:m]]
    return idx, ranked


def probability_block_scores(q, k_cmp, geom, block: int, blocks, first: int = 0, workers=None):
    """R20 block scores of the query blocks ``blocks``: for every pooled key j
    >= ``first``, the mean over the block's tokens t of their compressed
    softmax probability exp(s_tj - lse_t), s_tj = q_t . k~_j / sqrt(d), lse_t
    over all pooled keys ([Speed3R-ja] section 2.1: the compressed branch's
    attention in the compressed space guides the selection). Returns fp64
    [H, len(blocks), N*nb - first]."""
    qq = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cmp, dtype=np.float64)
    H, d = qq.shape[1], qq.shape[2]
    qbt = query_block_table(geom, block)
    out = np.empty((H, len(blocks), kc.shape[0] - first))

    def one_head(h):
        kh = kc[:, h, :]
        for i, bb in enumerate(blocks):
            s = (qq[qbt[bb], h, :] @ kh.T) / math.sqrt(d)      # [tokens, all pooled keys]
            mx = s.max(axis=1, keepdims=True)
            lse = mx + np.log(np.exp(s - mx).sum(axis=1, keepdims=True))
            out[h, i] = np.exp(s - lse).mean(axis=0)[first:]

    head_map(one_head, H, workers)
    return out


def select_topk_probability(q, k_cmp, geom, top_k: int, block: int, blocks, first: int = 0,
                            workers=None):
    """Top-K pooled blocks per (head, query block in ``blocks``) under R20
    scores, the selection rule of R6. Returns (idx [H, n, K] int32 ascending,
    global; ranked [H, n, K+1] fp64 = the natural log of the K+1 best scores in
    rank order, so that gaps between them read as relative)."""
    sc = probability_block_scores(q, k_cmp, geom, block, blocks, first=first, workers=workers)
    H, n, nk = sc.shape
    if not 1 <= top_k <= nk:
        raise ValueError("top_k must lie in [1, number of competing pooled keys]")
    idx = np.empty((H, n, top_k), dtype=np.int32)
    ranked = np.empty((H, n, top_k + 1))
    for h in range(H):
        idx[h], r = _topk_rows(sc[h], top_k, first)
        # a missing (K+1)-th entry stays -inf, as in select_topk
        with np.errstate(divide="ignore", invalid="ignore"):
            ranked[h] = np.where(r > 0, np.log(np.maximum(r, 0.0)), -np.inf)
    return idx, ranked


def select_topk(q_blk, k_cmp, top_k: int, chunk: int = 64, workers=None, first: int = 0):
    """Top-K pooled blocks per (head, query block) from the compressed scores
    ([Speed3R-ja] section 2.1, selection branch, first bullet; [Speed3R-it]
    section 2, "Ramo di Selezione"). Order: larger score first, ties to the
    lower block index (R6). Returns (idx [H, n, K] int32 ascending,
    ranked [H, n, K+1] fp64 = the K+1 best scores in rank order, +-inf padded).
    Only pooled keys j >= ``first`` compete (R15: ``first`` = the reference
    frame's block count); the returned indices are global.
    """
    qb = np.asarray(q_blk, dtype=np.float64)
    kc = np.asarray(k_cmp, dtype=np.float64)[first:]
    n, H, d = qb.shape
    nk = kc.shape[0]
    if not 1 <= top_k <= nk:
        raise ValueError("top_k must lie in [1, number of competing pooled keys]")
    idx = np.empty((H, n, top_k), dtype=np.int32)
    ranked = np.full((H, n, top_k + 1), -np.inf)

    def one_head(h):
        kh = kc[:, h, :]
        for a in range(0, n, chunk):
            s = (qb[a:a + chunk, h, :] @ kh.T) / math.sqrt(d)
            idx[h, a:a + chunk], ranked[h, a:a + chunk] = _topk_rows(s, top_k, first)

    head_map(one_head, H, workers)
    return idx, ranked


def fine_key_rows(geom, block: int, selected: Sequence[int], keep_special: bool = True,
                  keep_ref: bool = False):
    """Token rows attended by the fine branch of one query block: the valid
    tokens of the selected pooled blocks plus, when ``keep_special``, every
    special token of every frame (R5; [Speed3R-it] section 2 keeps the camera
    tokens, [AVGGT] section 2.2 keeps the special tokens), plus, when
    ``keep_ref``, every token of the reference frame 0 (R15)."""
    win = window_table(geom, block)
    parts = [win[j] for j in selected]
    L = _frame_len(geom)
    f0 = 1 if keep_ref else 0   # frame 0's special tokens belong to the kept reference frame
    if keep_ref:
        parts.append(np.arange(L))
    if keep_special and geom.n_special:
        parts.append(np.array([f * L + s for f in range(f0, geom.n_frames)
                               for s in range(geom.n_special)], dtype=np.int64))
    return np.concatenate(parts).astype(np.int64)


def fine_attention(q, k, v, geom, block: int, idx, rows=None, keep_special=True,
                   workers=None, keep_ref=False):
    """Fine-grained attention of each query over only its block's selected
    token blocks ([Speed3R-ja] section 2.1, selection branch, second bullet),
    plus every special token (R5) and, with ``keep_ref``, the whole reference
    frame (R15). ``idx`` [H, N*nqb, K] holds the selected pooled-block indices
    of every query block (with ``keep_ref`` none of them in frame 0)."""
    T, H, d = k.shape
    rows = _rows(rows, T)
    qbt = query_block_table(geom, block)
    win = window_table(geom, block)
    owner = np.empty(T, dtype=np.int64)
    for b, members in enumerate(qbt):
        owner[members] = b
    blocks = owner[rows]
    L = _frame_len(geom)
    f0 = 1 if keep_ref else 0   # frame 0's special tokens belong to the kept reference frame
    spec = np.array([f * L + s for f in range(f0, geom.n_frames) for s in range(geom.n_special)],
                    dtype=np.int64)
    use_spec = keep_special and len(spec) > 0
    ref = np.arange(L if keep_ref else 0)

    def one_head(h):
        o = np.empty((len(rows), d))
        ks = np.asarray(k[spec, h, :], np.float64)
        vs = np.asarray(v[spec, h, :], np.float64)
        for b in np.unique(blocks):
            sel = np.nonzero(blocks == b)[0]
            chosen = np.concatenate([win[j] for j in idx[h, b]])
            parts = [(k[chosen, h, :], v[chosen, h, :], None)]
            if use_spec:
                parts.append((ks, vs, None))
            if keep_ref:
                parts.append((k[ref, h, :], v[ref, h, :], None))
            o[sel], _ = attend_union(q[rows[sel], h, :], parts)
        return o

    return np.stack(head_map(one_head, H, workers), axis=1)


def gate(q, o_cmp, o_slc, w, b):
    """Gated aggregation ([Speed3R-ja] section 2.1; [Speed3R-it] section 2,
    "Aggregazione Guidata"): g = sigmoid(q . W[h]^T + b[h]) per token and head,
    o = g0 * o_cmp + g1 * o_slc (R7). ``q``, ``o_cmp``, ``o_slc`` [m, H, d];
    ``w`` [H, 2, d]; ``b`` [H, 2]."""
    q = np.asarray(q, dtype=np.float64)
    z = np.einsum("thd,hgd->thg", q, np.asarray(w, dtype=np.float64)) + np.asarray(b, np.float64)
    g = 1.0 / (1.0 + np.exp(-z))
    return (g[..., 0:1] * np.asarray(o_cmp, np.float64)
            + g[..., 1:2] * np.asarray(o_slc, np.float64))


def gsa_layer(q, k, v, geom, w, b, top_k: int, block: int = 4, rows=None,
              keep_special=True, workers=None, keep_ref=False, pooled_q=False,
              include_pad=False, probability_scores=False):
    """The whole Global Sparse Attention layer for the query rows ``rows``:
    pool, compressed branch, block scores + top-K, fine branch, gate.
    ``keep_ref`` is the VGGT adaptation (R15); ``pooled_q`` the block-level
    compressed branch (R18); ``include_pad`` the zero-padded pooling (R19);
    ``probability_scores`` the probability-mean block score (R20; ``ranked``
    then holds log scores). Returns a dict with every intermediate."""
    T = q.shape[0]
    rows = _rows(rows, T)
    k_cmp, v_cmp = compress(k, v, geom, block, include_pad=include_pad)
    if pooled_q:
        o_cmp = compressed_attention_pooled(q, k_cmp, v_cmp, geom, block, rows=rows, workers=workers)
    else:
        o_cmp = compressed_attention(q, k_cmp, v_cmp, rows=rows, workers=workers)
    qbt = query_block_table(geom, block)
    owner = np.empty(T, dtype=np.int64)
    for bi, members in enumerate(qbt):
        owner[members] = bi
    need = np.unique(owner[rows])
    q_blk = pooled_queries(q, geom, block, blocks=need)
    first = len(window_table(_one_frame(geom), block)) if keep_ref else 0
    if probability_scores:
        idx_need, ranked = select_topk_probability(q, k_cmp, geom, top_k, block, need, first=first,
                                                   workers=workers)
    else:
        idx_need, ranked = select_topk(q_blk, k_cmp, top_k, workers=workers, first=first)
    H = q.shape[1]
    idx_full = np.zeros((H, len(qbt), top_k), dtype=np.int32)
    idx_full[:, need] = idx_need
    o_slc = fine_attention(q, k, v, geom, block, idx_full, rows=rows,
                           keep_special=keep_special, workers=workers, keep_ref=keep_ref)
    o = gate(np.asarray(q[rows]), o_cmp, o_slc, w, b)
    return {"k_cmp": k_cmp, "v_cmp": v_cmp, "o_cmp": o_cmp, "blocks": need,
            "q_blk": q_blk, "idx": idx_need, "ranked": ranked, "o_slc": o_slc, "o": o}


# ---------------------------------------------------------------------------
# Subsampled global attention (AVGGT)
# ---------------------------------------------------------------------------

def subsample_plan(geom, s_h: int, s_w: int):
    """Per-frame patch positions kept and dropped on the 2D grid ([AVGGT]
    section 2.2: one kept patch per s_h x s_w window; R10 fixes the phase).
    Returns (kept, dropped) lists of in-frame token offsets (specials excluded)."""
    S, gh, gw = geom.n_special, geom.grid_h, geom.grid_w
    kept, dropped = [], []
    for r in range(gh):
        for c in range(gw):
            (kept if (r % s_h == 0 and c % s_w == 0) else dropped).append(S + r * gw + c)
    return kept, dropped


def sga_compact(k, v, geom, s_h: int, s_w: int):
    """The compacted key/value set of every frame ([AVGGT] section 2.2): its
    special tokens, its kept grid patches (exact copies), and -- when anything
    is dropped -- one mean key/value over its dropped patches (R11).
    Returns (c_k, c_v) fp64 [N*m, H, d], m = S + #kept + (1 if #dropped else 0)."""
    L = _frame_len(geom)
    kept, dropped = subsample_plan(geom, s_h, s_w)
    ck, cv = [], []
    for f in range(geom.n_frames):
        base = f * L
        keep_rows = list(range(base, base + geom.n_special)) + [base + p for p in kept]
        ck.append(np.asarray(k[keep_rows], dtype=np.float64))
        cv.append(np.asarray(v[keep_rows], dtype=np.float64))
        if dropped:
            drop_rows = [base + p for p in dropped]
            ck.append(np.asarray(k[drop_rows], dtype=np.float64).mean(axis=0, keepdims=True))
            cv.append(np.asarray(v[drop_rows], dtype=np.float64).mean(axis=0, keepdims=True))
    return np.concatenate(ck), np.concatenate(cv)


def subsampled_attention(q, k, v, geom, s_h: int, s_w: int, mode: int = 0,
                         mean_log_count: bool = False, rows=None, chunk: int = 64,
                         workers=None):
    """Subsampled global attention ([AVGGT] section 2.2): every query is kept;
    a query of frame f attends to all of frame f (R9) and to the compacted set
    of every other frame. ``mode`` 1 is the frame-attention conversion of the
    early layers; ``mode`` 2 the token-level diagonal (R17). With
    ``mean_log_count`` the mean key's logit gets log(#dropped) added (it then
    stands for the sum of the dropped columns)."""
    if mode == 1:
        return frame_attention(q, k, v, geom, rows=rows)
    if mode == 2:
        return _subsampled_token_diagonal(q, k, v, geom, s_h, s_w, mean_log_count, rows, chunk,
                                          workers)
    T, H, d = k.shape
    L = _frame_len(geom)
    N = geom.n_frames
    rows = _rows(rows, T)
    kept, dropped = subsample_plan(geom, s_h, s_w)
    m = geom.n_special + len(kept) + (1 if dropped else 0)
    ck, cv = sga_compact(k, v, geom, s_h, s_w)
    bias_c = np.zeros(N * m)
    if dropped and mean_log_count:
        bias_c[m - 1::m] = math.log(len(dropped))
    frames = rows // L

    scale = 1.0 / math.sqrt(d)

    def one_head(h):
        o = np.empty((len(rows), d))
        ckh = np.ascontiguousarray(ck[:, h, :], np.float64)
        cvh = np.ascontiguousarray(cv[:, h, :], np.float64)
        for a in range(0, len(rows), chunk):
            idx = np.arange(a, min(a + chunk, len(rows)))
            qc = np.asarray(q[rows[idx], h, :], np.float64)
            # scores against the compacted sets of all frames ...
            s_c = (qc @ ckh.T) * scale + bias_c
            for i, f in enumerate(frames[idx]):
                s_c[i, f * m:(f + 1) * m] = -np.inf  # ... minus the query's own frame
            # ... plus its own frame whole; one softmax over the union per row
            s_own = np.empty((len(idx), L))
            v_own = np.empty((len(idx), L, d))
            for i, f in enumerate(frames[idx]):
                own = slice(f * L, (f + 1) * L)
                s_own[i] = (np.asarray(k[own, h, :], np.float64) @ qc[i]) * scale
                v_own[i] = v[own, h, :]
            mx = np.maximum(s_own.max(axis=1), s_c.max(axis=1))[:, None]
            p_own = np.exp(s_own - mx)
            p_c = np.exp(s_c - mx)
            num = np.einsum("il,ild->id", p_own, v_own) + p_c @ cvh
            o[idx] = num / (p_own.sum(axis=1) + p_c.sum(axis=1))[:, None]
        return o

    return np.stack(head_map(one_head, H, workers), axis=1)


def _subsampled_token_diagonal(q, k, v, geom, s_h, s_w, mean_log_count, rows, chunk, workers):
    """R17: the compacted set of every frame, the query's own frame included,
    plus the query's own key/value when its patch was dropped; one softmax
    over the union per query."""
    T, H, d = k.shape
    L = _frame_len(geom)
    N = geom.n_frames
    rows = _rows(rows, T)
    kept, dropped = subsample_plan(geom, s_h, s_w)
    m = geom.n_special + len(kept) + (1 if dropped else 0)
    ck, cv = sga_compact(k, v, geom, s_h, s_w)
    bias_c = np.zeros(N * m)
    if dropped and mean_log_count:
        bias_c[m - 1::m] = math.log(len(dropped))
    was_dropped = np.zeros(L, dtype=bool)
    was_dropped[dropped] = True
    diag = was_dropped[rows % L]          # the query's own column is not in its frame's compacted set
    scale = 1.0 / math.sqrt(d)

    def one_head(h):
        o = np.empty((len(rows), d))
        ckh = np.ascontiguousarray(ck[:, h, :], np.float64)
        cvh = np.ascontiguousarray(cv[:, h, :], np.float64)
        for a in range(0, len(rows), chunk):
            idx = np.arange(a, min(a + chunk, len(rows)))
            qc = np.asarray(q[rows[idx], h, :], np.float64)
            kd = np.asarray(k[rows[idx], h, :], np.float64)
            vd = np.asarray(v[rows[idx], h, :], np.float64)
            s_c = (qc @ ckh.T) * scale + bias_c
            s_d = np.where(diag[idx], np.einsum("id,id->i", qc, kd) * scale, -np.inf)
            mx = np.maximum(s_c.max(axis=1), s_d)
            p_c = np.exp(s_c - mx[:, None])
            p_d = np.exp(s_d - mx)
            num = p_c @ cvh + p_d[:, None] * vd
            o[idx] = num / (p_c.sum(axis=1) + p_d)[:, None]
        return o

    return np.stack(head_map(one_head, H, workers), axis=1)
