"""HIP library vs the fp64 oracle on the same seeded inputs (needs a gfx950 GPU).

Small cases check every output row; the workload-sized cases check a seeded
sample of query rows (all heads, all d) plus every intermediate the sampled
rows depend on.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_global_amd as sga
from parity import (assert_close, check_topk, decided_blocks, host, oracle_workers)
from synth import WORKLOADS, Geometry, make_gate, make_qkv, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _sync():
    torch.cuda.synchronize()


def _announce(what):
    print(f"[case] {what}", flush=True)


def _nb(geom):
    return -(-geom.grid_h // 4) * -(-geom.grid_w // 4)


def _nqb(geom):
    return _nb(geom) + (1 if geom.n_special else 0)


def _owner_blocks(geom, rows):
    """Query block of each token row (windows, then a frame's specials block)."""
    L = geom.tokens_per_frame
    out = np.empty(len(rows), dtype=np.int64)
    nbw = -(-geom.grid_w // 4)
    for i, t in enumerate(np.asarray(rows)):
        f, p = divmod(int(t), L)
        if p < geom.n_special:
            out[i] = f * _nqb(geom) + _nb(geom)
        else:
            r, c = divmod(p - geom.n_special, geom.grid_w)
            out[i] = f * _nqb(geom) + (r // 4) * nbw + c // 4
    return out


# ---------------------------------------------------------------------------
# every op, every row, on small geometries
# ---------------------------------------------------------------------------

SMALL = [
    pytest.param(WORKLOADS["tiny"].geom, 4, (2, 2), id="tiny-f32"),
    pytest.param(Geometry(3, 5, 13, 11, 2, 64, "bf16"), 5, (4, 4), id="ragged-bf16"),
    pytest.param(Geometry(2, 2, 9, 9, 3, 64, "f32"), 3, (3, 2), id="ragged-f32"),
    pytest.param(Geometry(1, 1, 5, 7, 1, 64, "bf16"), 2, (2, 3), id="one-frame-bf16"),
    # degenerate shapes: one-token frames, the most special tokens, one whole window
    pytest.param(Geometry(5, 0, 1, 1, 1, 64, "bf16"), 3, (2, 2), id="1x1-grid-bf16"),
    pytest.param(Geometry(2, 16, 3, 5, 2, 64, "bf16"), 2, (2, 2), id="16-specials-bf16"),
    pytest.param(Geometry(4, 1, 4, 4, 1, 64, "f32"), 4, (4, 4), id="one-window-f32"),
]


@pytest.mark.parametrize("geom,top_k,stride", SMALL)
def test_small_every_op(geom, top_k, stride):
    _announce(f"small {geom} top_k={top_k} stride={stride}")
    dist = "normal" if geom.dtype == "f32" else "scene"
    q, k, v = make_qkv(geom, seed=11, device=DEV, distribution=dist)
    w, b = make_gate(geom.n_heads, 64, seed=11, device=DEV)
    qh, kh, vh = host(q), host(k), host(v)
    dt = geom.dtype
    N = geom.n_frames

    # dense + lse, frame
    o, lse = sga.dense_global_attn(q, k, v, geom, want_lse=True)
    of = sga.dense_global_attn(q, k, v, geom, frame_local=True)
    _sync()
    ro, rlse = oracle.dense_attention(qh, kh, vh, with_lse=True)
    assert_close(host(o), ro, dt, "dense")
    assert_close(host(lse), rlse, "f32" if dt == "f32" else "bf16", "dense lse")
    assert_close(host(of), oracle.frame_attention(qh, kh, vh, geom), dt, "frame")

    # GSA step by step
    k_cmp, v_cmp, k32, q32 = sga.gsa_compress(q, k, v, geom)
    _sync()
    rkc, rvc = oracle.compress(kh, vh, geom, 4)
    rqb = oracle.pooled_queries(qh, geom, 4)
    assert_close(host(k_cmp), rkc, dt, "k_cmp")
    assert_close(host(v_cmp), rvc, dt, "v_cmp")
    assert_close(host(k32), rkc, "f32", "k_cmp_f32")
    assert_close(host(q32), rqb, "f32", "q_blk_f32")

    o_cmp = sga.dense_global_attn(q, k_cmp, v_cmp, geom, n_keys=N * _nb(geom))
    _sync()
    r_cmp = oracle.compressed_attention(qh, rkc, rvc)
    assert_close(host(o_cmp), r_cmp, dt, "o_cmp")

    idx, score = sga.gsa_select_topk(q32, k32, geom, top_k, want_score=True)
    _sync()
    ridx, ranked = oracle.select_topk(rqb, rkc, top_k)
    check_topk(host(idx).astype(np.int64), ridx, ranked, rqb, rkc, "top-K")
    idx_h, score_h = host(idx).astype(np.int64), host(score)
    for h in range(geom.n_heads):
        for bb in range(idx_h.shape[1]):
            s = rkc[idx_h[h, bb], h, :] @ rqb[bb, h, :] / 8.0
            assert np.max(np.abs(score_h[h, bb] - s)) < 1e-4

    # fine branch on the oracle's index sets (same input both sides)
    idx_in = torch.from_numpy(ridx).to(DEV)
    o_slc, lse_slc = sga.gsa_sparse_attn(q, k, v, idx_in, geom, top_k, want_lse=True)
    o_slc0 = sga.gsa_sparse_attn(q, k, v, idx_in, geom, top_k, keep_special=False)
    _sync()
    r_slc = oracle.fine_attention(qh, kh, vh, geom, 4, ridx)
    assert_close(host(o_slc), r_slc, dt, "o_slc")
    assert_close(host(o_slc0), oracle.fine_attention(qh, kh, vh, geom, 4, ridx, keep_special=False),
                 dt, "o_slc (no specials)")

    # gate on shared inputs
    o_g = sga.gsa_gate(q, o_cmp, o_slc, w, b, geom)
    _sync()
    assert_close(host(o_g), oracle.gate(qh, host(o_cmp), host(o_slc), host(w), host(b)), dt, "gate")
    # the gate folded into the fine branch: oracle fine result (same index
    # sets), GPU compressed output (shared input)
    o_gf = sga.gsa_sparse_attn_gated(q, k, v, idx_in, o_cmp, w, b, geom, top_k)
    _sync()
    assert_close(host(o_gf), oracle.gate(qh, host(o_cmp), r_slc, host(w), host(b)), dt, "gate fused into fine")

    # the whole layer, on rows whose blocks are decided in every head
    out = sga.gsa_layer(q, k, v, w, b, geom, top_k)
    _sync()
    ref = oracle.gsa_layer(qh, kh, vh, geom, host(w), host(b), top_k)
    dec = decided_blocks(ref["ranked"], top_k).all(axis=0)
    owner = _owner_blocks(geom, np.arange(geom.n_tokens))
    pos = {bb: i for i, bb in enumerate(ref["blocks"])}
    rows = np.array([t for t in range(geom.n_tokens) if dec[pos[owner[t]]]])
    assert len(rows) > 0.5 * geom.n_tokens
    assert_close(host(out)[rows], ref["o"][rows], dt, "gsa layer")

    # subsampled: compaction, attention, log-count variant, frame mode
    sh, sw = stride
    c_k, c_v = sga.sga_compact(k, v, geom, sh, sw)
    _sync()
    rck, rcv = oracle.sga_compact(kh, vh, geom, sh, sw)
    mk, has_mean = sga.compact_rows(geom, sh, sw)
    m = mk + has_mean
    for f in range(N):
        assert np.array_equal(host(c_k)[f * mk:(f + 1) * mk], rck[f * m:f * m + mk])
        assert np.array_equal(host(c_v)[f * mk:(f + 1) * mk], rcv[f * m:f * m + mk])
    if has_mean:
        assert_close(host(c_k)[N * mk:], rck[m - 1::m], dt, "mean keys")
        assert_close(host(c_v)[N * mk:], rcv[m - 1::m], dt, "mean values")
    o_s = sga.subsampled_global_attn(q, k, v, geom, sh, sw)
    o_sl = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mean_log_count=True)
    o_sf = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=1)
    _sync()
    assert_close(host(o_s), oracle.subsampled_attention(qh, kh, vh, geom, sh, sw), dt, "subsampled")
    assert_close(host(o_sl), oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, mean_log_count=True),
                 dt, "subsampled log-count")
    assert_close(host(o_sf), oracle.frame_attention(qh, kh, vh, geom), dt, "subsampled frame mode")


def test_loose_bound_redo():
    """Rows whose logits sit far below |q| max|k|: the bf16 kernels start each
    query at that bound, so here every probability of the first pass underflows
    and the workgroups holding these rows must redo them exactly."""
    geom = Geometry(3, 5, 13, 11, 2, 64, "bf16")
    _announce(f"loose logit bound {geom}")
    q, k, v = make_qkv(geom, seed=21, device=DEV, distribution="scene")
    far = [0, 1, 2, 15, 130, 300, 301, 443]
    k[7] = 0
    k[7, :, 0] = 40.0   # one key of norm 40 along d = 0 ...
    q[far] = 0
    q[far, :, 1] = 40.0  # ... queries of norm 40 orthogonal to it: bound 288 log2 units
    qh, kh, vh = host(q), host(k), host(v)
    o, lse = sga.dense_global_attn(q, k, v, geom, want_lse=True)
    of = sga.dense_global_attn(q, k, v, geom, frame_local=True)
    os_ = sga.subsampled_global_attn(q, k, v, geom, 2, 2)
    _sync()
    ro, rlse = oracle.dense_attention(qh, kh, vh, with_lse=True)
    assert_close(host(o), ro, "bf16", "dense (loose bound)")
    assert_close(host(lse), rlse, "bf16", "dense lse (loose bound)")
    assert_close(host(of), oracle.frame_attention(qh, kh, vh, geom), "bf16", "frame (loose bound)")
    assert_close(host(os_), oracle.subsampled_attention(qh, kh, vh, geom, 2, 2), "bf16",
                 "subsampled (loose bound)")


def test_invariants_on_gpu():
    """The pages' reductions hold on the GPU path too: K = all blocks with the
    gate forced to the fine branch is dense; stride 1x1 is dense."""
    geom = Geometry(2, 5, 8, 12, 2, 64, "bf16")
    _announce(f"invariants {geom}")
    q, k, v = make_qkv(geom, seed=3, device=DEV, distribution="scene")
    nb = geom.n_frames * _nb(geom)
    w = torch.zeros((2, 2, 64), device=DEV)
    b = torch.tensor([[-float("inf"), float("inf")]] * 2, device=DEV)
    o_gsa = sga.gsa_layer(q, k, v, w, b, geom, nb)
    o_s1 = sga.subsampled_global_attn(q, k, v, geom, 1, 1)
    o_d = sga.dense_global_attn(q, k, v, geom)
    _sync()
    ref = oracle.dense_attention(host(q), host(k), host(v))
    assert_close(host(o_gsa), ref, "bf16", "gsa(K=all, fine gate) vs dense oracle")
    assert_close(host(o_s1), ref, "bf16", "stride 1 vs dense oracle")
    assert_close(host(o_d), ref, "bf16", "dense")


@pytest.mark.parametrize("top_k", [16, 100, 128])
def test_topk_planted_winners(top_k):
    """Designed pooled scores with known, separated winners: block b's pooled
    query is the unit vector of coordinate c_b, so only keys of class c_b score,
    by their planted magnitudes (spaced 0.01 apart, i.e. 1.25e-3 in score)."""
    geom = Geometry(128, 5, 37, 37, 2, 64, "bf16")
    _announce(f"planted top-{top_k} {geom}")
    N, H = geom.n_frames, geom.n_heads
    nk, nq = N * _nb(geom), N * _nqb(geom)
    rng = np.random.default_rng(5)
    cls = np.arange(nk) % 64
    k32 = rng.standard_normal((nk, H, 64)) * 1e-6
    mag = np.empty(nk)
    for c in range(64):
        members = np.nonzero(cls == c)[0]
        mag[members] = 1.0 + 0.01 * rng.permutation(len(members))
    for h in range(H):
        k32[np.arange(nk), h, cls] += mag
    qc = rng.integers(0, 64, size=(nq, H))
    q32 = np.zeros((nq, H, 64))
    for h in range(H):
        q32[np.arange(nq), h, qc[:, h]] = 1.0
    idx = sga.gsa_select_topk(torch.tensor(q32, dtype=torch.float32, device=DEV),
                              torch.tensor(k32, dtype=torch.float32, device=DEV), geom, top_k)
    _sync()
    got = host(idx).astype(np.int64)
    for h in range(H):
        for bb in range(0, nq, 97):
            members = np.nonzero(cls == qc[bb, h])[0]
            want = np.sort(members[np.argsort(-mag[members], kind="stable")[:top_k]])
            assert np.array_equal(got[h, bb], want), (h, bb)


@pytest.mark.parametrize("top_k", [7, 16, 17, 32, 64, 100, 128])
def test_topk_widths(top_k):
    """Every selection path: register lists up to 16; beyond, the bound /
    filter / sort kernel (its sorts of 128 to 1024 keys per block)."""
    geom = Geometry(16, 5, 37, 37, 2, 64, "bf16")
    _announce(f"top-K width {top_k} {geom}")
    q, k, v = make_qkv(geom, seed=31, device=DEV, distribution="scene")
    _, _, k32, q32 = sga.gsa_compress(q, k, v, geom)
    idx, score = sga.gsa_select_topk(q32, k32, geom, top_k, want_score=True)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    rkc, _ = oracle.compress(kh, vh, geom, 4)
    rqb = oracle.pooled_queries(qh, geom, 4)
    ridx, ranked = oracle.select_topk(rqb, rkc, top_k)
    check_topk(host(idx).astype(np.int64), ridx, ranked, rqb, rkc, f"top-{top_k}")
    idx_h = host(idx).astype(np.int64)
    s_h = host(score)
    for h in range(geom.n_heads):
        ref = np.einsum("bkd,bd->bk", rkc[idx_h[h], h, :], rqb[:, h, :]) / 8.0
        assert np.max(np.abs(s_h[h] - ref)) < 1e-4


# ---------------------------------------------------------------------------
# Speed3R architecture variants: VGGT (reference frame 0 kept whole, the top-K
# over the other frames) and pi^3 (no register tokens)
# ---------------------------------------------------------------------------

def _layer_on_decided_rows(geom, q, k, v, w, b, top_k, keep_ref, what):
    out = sga.gsa_layer(q, k, v, w, b, geom, top_k, keep_ref=keep_ref)
    _sync()
    ref = oracle.gsa_layer(host(q), host(k), host(v), geom, host(w), host(b), top_k,
                           keep_ref=keep_ref)
    dec = decided_blocks(ref["ranked"], top_k).all(axis=0)
    owner = _owner_blocks(geom, np.arange(geom.n_tokens))
    pos = {bb: i for i, bb in enumerate(ref["blocks"])}
    rows = np.array([t for t in range(geom.n_tokens) if dec[pos[owner[t]]]])
    # many close block scores (top-32 of 175) leave few blocks decided in every
    # head; the index sets and the fine branch are checked in full separately
    print(f"[parity] {what}: {len(rows)} of {geom.n_tokens} rows decided in every head", flush=True)
    assert len(rows) >= 64
    assert_close(host(out)[rows], ref["o"][rows], geom.dtype, what)


VGGT = [
    pytest.param(Geometry(3, 5, 13, 11, 2, 64, "bf16"), 5, id="ragged-bf16"),
    pytest.param(Geometry(2, 2, 9, 9, 3, 64, "f32"), 3, id="ragged-f32"),
    pytest.param(Geometry(8, 5, 20, 20, 2, 64, "bf16"), 16, id="3-tiles-top16"),
    pytest.param(Geometry(8, 5, 20, 20, 2, 64, "bf16"), 32, id="3-tiles-top32"),
    pytest.param(Geometry(4, 0, 13, 11, 2, 64, "bf16"), 6, id="no-specials"),
]


@pytest.mark.parametrize("geom,top_k", VGGT)
def test_reference_frame_kept(geom, top_k):
    """The VGGT adaptation: selection among frames 1..N-1 only, frame 0 attended
    whole by every query (with and without the special tokens), and a frame-0
    window slipped into an index list contributes nothing."""
    _announce(f"reference frame kept {geom} top_k={top_k}")
    dist = "normal" if geom.dtype == "f32" else "scene"
    q, k, v = make_qkv(geom, seed=41, device=DEV, distribution=dist)
    w, b = make_gate(geom.n_heads, 64, seed=41, device=DEV)
    qh, kh, vh = host(q), host(k), host(v)
    nb = _nb(geom)
    _, _, k32, q32 = sga.gsa_compress(q, k, v, geom)
    idx, score = sga.gsa_select_topk(q32, k32, geom, top_k, want_score=True, keep_ref=True)
    _sync()
    rkc, _ = oracle.compress(kh, vh, geom, 4)
    rqb = oracle.pooled_queries(qh, geom, 4)
    ridx, ranked = oracle.select_topk(rqb, rkc, top_k, first=nb)
    idx_h = host(idx).astype(np.int64)
    assert idx_h.min() >= nb
    check_topk(idx_h, ridx, ranked, rqb, rkc, "top-K (reference frame kept)")
    for h in range(geom.n_heads):
        s = np.einsum("bkd,bd->bk", rkc[idx_h[h], h, :], rqb[:, h, :]) / 8.0
        assert np.max(np.abs(host(score)[h] - s)) < 1e-4

    idx_in = torch.from_numpy(ridx).to(DEV)
    for keep_special in (True, False):
        o_slc = sga.gsa_sparse_attn(q, k, v, idx_in, geom, top_k, keep_special=keep_special,
                                    keep_ref=True)
        _sync()
        want = oracle.fine_attention(qh, kh, vh, geom, 4, ridx, keep_special=keep_special,
                                     keep_ref=True)
        assert_close(host(o_slc), want, geom.dtype, f"o_slc (reference frame, specials={keep_special})")
        # the gate folded in, over the same index sets (o_cmp: any shared input)
        o_cmp = torch.flip(q, dims=[0]).contiguous()
        o_g = sga.gsa_sparse_attn_gated(q, k, v, idx_in, o_cmp, w, b, geom, top_k, keep_special=keep_special,
                                        keep_ref=True)
        _sync()
        assert_close(host(o_g), oracle.gate(qh, host(o_cmp), want, host(w), host(b)), geom.dtype,
                     f"gated fine (reference frame, specials={keep_special})")
    if top_k > 1:
        slipped = idx_in.clone()
        slipped[..., 0] = 0       # a window of frame 0: must add nothing
        o_slc = sga.gsa_sparse_attn(q, k, v, slipped, geom, top_k, keep_ref=True)
        _sync()
        want = oracle.fine_attention(qh, kh, vh, geom, 4, ridx[..., 1:], keep_ref=True)
        assert_close(host(o_slc), want, geom.dtype, "o_slc (frame-0 window ignored)")
    _layer_on_decided_rows(geom, q, k, v, w, b, top_k, True, "gsa layer (reference frame)")


@pytest.mark.parametrize("n_special", [0, 1])
def test_pi3_no_registers(n_special):
    """The pi^3 adaptation: GSA applied directly, without register tokens (no
    special token at all, or a single one)."""
    geom = Geometry(6, n_special, 13, 11, 2, 64, "bf16")
    _announce(f"pi3 {geom}")
    q, k, v = make_qkv(geom, seed=43, device=DEV, distribution="scene")
    w, b = make_gate(geom.n_heads, 64, seed=43, device=DEV)
    _layer_on_decided_rows(geom, q, k, v, w, b, 8, False, f"gsa layer (S={n_special})")


def test_topk_wide_ties_fall_back():
    """Every pooled key equal: every score ties, so the wide selection's
    filter keeps all 1600 candidates, overflows its buffers and leaves every
    block to the exact LDS-list kernel; ties go to the lowest indices."""
    geom = Geometry(16, 5, 37, 37, 2, 64, "bf16")
    _announce(f"wide top-K, all scores tied {geom}")
    N, H = geom.n_frames, geom.n_heads
    rng = np.random.default_rng(7)
    k32 = np.tile(rng.standard_normal((1, H, 64)), (N * _nb(geom), 1, 1))
    q32 = rng.standard_normal((N * _nqb(geom), H, 64))
    for top_k in (17, 100, 128):
        idx, score = sga.gsa_select_topk(torch.tensor(q32, dtype=torch.float32, device=DEV),
                                         torch.tensor(k32, dtype=torch.float32, device=DEV), geom,
                                         top_k, want_score=True)
        _sync()
        got = host(idx).astype(np.int64)
        assert (got == np.arange(top_k)[None, None, :]).all(), top_k
        ridx, ranked = oracle.select_topk(q32[::37], k32, top_k)
        assert (ridx == np.arange(top_k)[None, None, :]).all()
        assert np.max(np.abs(host(score)[:, ::37] - ranked[:, :, :top_k])) < 1e-4


@pytest.mark.parametrize("keep_ref", [False, True])
def test_topk_register_ties(keep_ref):
    """Exact ties on the register-list selection (top_k <= 16): (a) every
    competing pooled key equal, so every score ties and the lowest competing
    indices win; (b) every competing key present in three identical copies
    500 apart (500 = 4 mod 8: consecutive copies sit in the two different
    lane halves of a block), with the distinct keys' scores planted 1.25e-3
    apart, so each copy group ties exactly and the lower copies win. With the
    reference frame kept, frame 0's blocks score far above the rest and must
    still not be picked."""
    geom = Geometry(16, 5, 37, 37, 2, 64, "bf16")
    _announce(f"register top-K ties, keep_ref={keep_ref} {geom}")
    N, H = geom.n_frames, geom.n_heads
    nk, nq = N * _nb(geom), N * _nqb(geom)
    first = _nb(geom) if keep_ref else 0
    rng = np.random.default_rng(17)
    q32 = rng.standard_normal((nq, H, 64))
    n0 = 500
    assert 3 * n0 <= nk - first and n0 % 8 == 4
    # (b) planted classes: block b's query is the unit vector of coordinate cls_q
    base_cls = np.arange(n0) % 64
    base_mag = np.empty(n0)
    for c in range(64):
        members = np.nonzero(base_cls == c)[0]
        base_mag[members] = 1.0 + 0.01 * rng.permutation(len(members))
    k_b = np.zeros((nk, H, 64))
    k_b[:first, :, :] = 50.0          # frame 0 (kept whole, must not compete)
    rest = first + 3 * n0
    k_b[rest:, :, :] = -50.0          # the leftover keys score far below
    for copy in range(3):
        for h in range(H):
            k_b[first + copy * n0 + np.arange(n0), h, base_cls] = base_mag
    cls_q = rng.integers(0, 64, size=(nq, H))
    q_b = np.zeros((nq, H, 64))
    for h in range(H):
        q_b[np.arange(nq), h, cls_q[:, h]] = 1.0
    # (a) all competing keys equal
    k_a = np.tile(rng.standard_normal((1, H, 64)), (nk, 1, 1))
    if keep_ref:
        k_a[:first] += 3.0
    for top_k in (1, 4, 16):
        idx_a = sga.gsa_select_topk(torch.tensor(q32, dtype=torch.float32, device=DEV),
                                    torch.tensor(k_a, dtype=torch.float32, device=DEV), geom, top_k,
                                    keep_ref=keep_ref)
        idx_b, sc_b = sga.gsa_select_topk(torch.tensor(q_b, dtype=torch.float32, device=DEV),
                                          torch.tensor(k_b, dtype=torch.float32, device=DEV), geom, top_k,
                                          want_score=True, keep_ref=keep_ref)
        _sync()
        got_a = host(idx_a).astype(np.int64)
        assert (got_a == first + np.arange(top_k)[None, None, :]).all(), ("all equal", top_k)
        got_b = host(idx_b).astype(np.int64)
        for h in range(H):
            for bb in range(nq):
                members = np.nonzero(base_cls == cls_q[bb, h])[0]
                order = members[np.argsort(-base_mag[members], kind="stable")]
                seq = [first + copy * n0 + i for i in order for copy in range(3)]
                want = np.sort(seq[:top_k])
                assert np.array_equal(got_b[h, bb], want), ("copies", top_k, h, bb, got_b[h, bb], want)
        want_sc = np.take_along_axis(np.einsum("bhd,jhd->hbj", q_b, k_b), got_b, axis=2) / 8.0
        assert np.max(np.abs(host(sc_b) - want_sc)) < 1e-5
        print(f"[parity] register top-{top_k} ties (keep_ref={keep_ref}): all rows exact", flush=True)


@pytest.mark.parametrize("top_k", [5, 16])
def test_topk_two_stage_fallback(top_k):
    """The two-stage selection's exact fallback at both of its sizes: with every
    pooled key equal, no block can be certified, so all 4,848 blocks per head
    go to the exact kernel -- the first 4,096 with their keys split over
    segments and merged, the rest streamed whole -- and ties go to the lowest
    indices; on the scene inputs of the same geometry the certified and the
    fallback blocks together must match the oracle."""
    geom = Geometry(48, 5, 37, 37, 2, 64, "bf16")
    _announce(f"two-stage fallback top-{top_k} {geom}")
    N, H = geom.n_frames, geom.n_heads
    rng = np.random.default_rng(19)
    k32 = np.tile(rng.standard_normal((1, H, 64)), (N * _nb(geom), 1, 1))
    q32 = rng.standard_normal((N * _nqb(geom), H, 64))
    idx, sc = sga.gsa_select_topk(torch.tensor(q32, dtype=torch.float32, device=DEV),
                                  torch.tensor(k32, dtype=torch.float32, device=DEV), geom, top_k,
                                  want_score=True)
    _sync()
    assert (host(idx).astype(np.int64) == np.arange(top_k)[None, None, :]).all()
    s_ref = np.einsum("bhd,hd->hb", q32, k32[0]) / 8.0
    assert np.max(np.abs(host(sc) - s_ref[:, :, None])) < 1e-4
    q, k, v = make_qkv(geom, seed=23, device=DEV, distribution="scene")
    _, _, k32g, q32g = sga.gsa_compress(q, k, v, geom)
    idx_g = sga.gsa_select_topk(q32g, k32g, geom, top_k)
    _sync()
    rkc, _ = oracle.compress(host(k), host(v), geom, 4)
    rqb = oracle.pooled_queries(host(q), geom, 4)
    ridx, ranked = oracle.select_topk(rqb, rkc, top_k, workers=oracle_workers())
    check_topk(host(idx_g).astype(np.int64), ridx, ranked, rqb, rkc, f"two-stage top-{top_k}, 48 frames")


def test_topk_wide_few_candidates():
    """Fewer competing blocks than the bound's 128 buckets: the bound is -inf,
    every candidate is kept and sorted (3 frames x 12 blocks, top-20; 2 frames
    with frame 0 kept whole, top-12 of 12)."""
    geom = Geometry(3, 5, 13, 11, 2, 64, "bf16")
    _announce(f"wide top-K, few candidates {geom}")
    q, k, v = make_qkv(geom, seed=51, device=DEV, distribution="scene")
    _, _, k32, q32 = sga.gsa_compress(q, k, v, geom)
    rkc, _ = oracle.compress(host(k), host(v), geom, 4)
    rqb = oracle.pooled_queries(host(q), geom, 4)
    for top_k, keep_ref in ((20, False), (24, True)):
        idx = sga.gsa_select_topk(q32, k32, geom, top_k, keep_ref=keep_ref)
        _sync()
        ridx, ranked = oracle.select_topk(rqb, rkc, top_k, first=_nb(geom) if keep_ref else 0)
        check_topk(host(idx).astype(np.int64), ridx, ranked, rqb, rkc, f"top-{top_k} of few")


@pytest.mark.parametrize("sigma", range(2, 10))
def test_subsampled_sigma(sigma):
    """AVGGT's subsampling factor over its tested range (sigma x sigma windows,
    2..9), every row of a 6-frame scene, with and without the log-count bias."""
    geom = Geometry(6, 5, 37, 37, 2, 64, "bf16")
    _announce(f"subsampled sigma={sigma} {geom}")
    q, k, v = make_qkv(geom, seed=60 + sigma, device=DEV, distribution="scene")
    o = sga.subsampled_global_attn(q, k, v, geom, sigma, sigma)
    ol = sga.subsampled_global_attn(q, k, v, geom, sigma, sigma, mean_log_count=True)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    W = oracle_workers()
    assert_close(host(o), oracle.subsampled_attention(qh, kh, vh, geom, sigma, sigma, workers=W),
                 "bf16", f"subsampled sigma={sigma}")
    assert_close(host(ol), oracle.subsampled_attention(qh, kh, vh, geom, sigma, sigma,
                                                       mean_log_count=True, workers=W),
                 "bf16", f"subsampled sigma={sigma} log-count")


@pytest.mark.parametrize("geom,stride", [
    pytest.param(Geometry(3, 5, 13, 11, 2, 64, "bf16"), (4, 4), id="ragged-bf16"),
    pytest.param(Geometry(2, 2, 9, 9, 3, 64, "f32"), (3, 2), id="ragged-f32"),
    pytest.param(Geometry(1, 1, 5, 7, 1, 64, "bf16"), (2, 3), id="one-frame-bf16"),
    pytest.param(Geometry(6, 5, 37, 37, 2, 64, "bf16"), (4, 4), id="scene-bf16"),
    pytest.param(Geometry(2, 0, 8, 8, 2, 64, "bf16"), (1, 1), id="stride1-bf16"),
])
def test_subsampled_token_diagonal(geom, stride):
    """AVGGT's diagonal read at token level (mode 2): every frame subsampled,
    the query's own key added when its patch was dropped; every row, with and
    without the log-count bias; stride 1 is dense attention."""
    _announce(f"subsampled token diagonal {geom} stride={stride}")
    dist = "normal" if geom.dtype == "f32" else "scene"
    q, k, v = make_qkv(geom, seed=71, device=DEV, distribution=dist)
    sh, sw = stride
    o = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=2)
    ol = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=2, mean_log_count=True)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    assert_close(host(o), oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, mode=2), geom.dtype,
                 "token diagonal")
    assert_close(host(ol), oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, mode=2,
                                                       mean_log_count=True), geom.dtype,
                 "token diagonal log-count")
    if stride == (1, 1):
        assert_close(host(o), oracle.dense_attention(qh, kh, vh), geom.dtype, "token diagonal stride 1")


@pytest.mark.parametrize("geom", [
    pytest.param(Geometry(2, 0, 16, 16, 2, 64, "bf16"), id="L256-whole-tiles"),
    pytest.param(Geometry(2, 4, 16, 18, 2, 64, "bf16"), id="L292-split-96"),
    pytest.param(Geometry(2, 4, 16, 22, 2, 64, "bf16"), id="L356-split-128"),
    pytest.param(Geometry(2, 0, 20, 20, 2, 64, "bf16"), id="L400-partial-256-tile"),
    pytest.param(Geometry(3, 0, 8, 16, 2, 64, "bf16"), id="L128-rest-only"),
])
def test_subsampled_query_tiling(geom):
    """The subsampled form runs a frame's whole 256-query tiles and the rest
    (one tile of 96 or 128 rows) in two launches, or one launch when the rest
    is empty, longer than 128 rows or the whole frame: every row of each case,
    modes 0 and 2, against the oracle."""
    _announce(f"subsampled query tiling {geom}")
    q, k, v = make_qkv(geom, seed=73, device=DEV, distribution="scene")
    o0 = sga.subsampled_global_attn(q, k, v, geom, 2, 2, mode=0, mean_log_count=True)
    o2 = sga.subsampled_global_attn(q, k, v, geom, 2, 2, mode=2)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    assert_close(host(o0), oracle.subsampled_attention(qh, kh, vh, geom, 2, 2, mean_log_count=True),
                 "bf16", "subsampled tiling mode 0")
    assert_close(host(o2), oracle.subsampled_attention(qh, kh, vh, geom, 2, 2, mode=2), "bf16",
                 "subsampled tiling mode 2")


@pytest.mark.parametrize("geom,top_k", [
    pytest.param(Geometry(3, 5, 13, 11, 2, 64, "bf16"), 5, id="ragged-bf16"),
    pytest.param(Geometry(2, 2, 9, 9, 3, 64, "f32"), 3, id="ragged-f32"),
    pytest.param(Geometry(6, 5, 37, 37, 2, 64, "bf16"), 16, id="scene-bf16"),
    pytest.param(Geometry(2, 0, 8, 8, 2, 64, "bf16"), 4, id="no-specials-bf16"),
])
def test_compressed_pooled(geom, top_k):
    """The block-level compressed branch: every row against the oracle (the
    oracle's own pooling and block means), and the whole layer on decided rows."""
    _announce(f"compressed branch at block level {geom}")
    dist = "normal" if geom.dtype == "f32" else "scene"
    q, k, v = make_qkv(geom, seed=81, device=DEV, distribution=dist)
    w, b = make_gate(geom.n_heads, 64, seed=81, device=DEV)
    k_cmp, v_cmp, _, q32 = sga.gsa_compress(q, k, v, geom)
    o = sga.gsa_compressed_pooled(q32, k_cmp, v_cmp, geom)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    rkc, rvc = oracle.compress(kh, vh, geom, 4)
    assert_close(host(o), oracle.compressed_attention_pooled(qh, rkc, rvc, geom, 4), geom.dtype,
                 "o_cmp (block level)")
    out = sga.gsa_layer(q, k, v, w, b, geom, top_k, pooled_q=True)
    _sync()
    ref = oracle.gsa_layer(qh, kh, vh, geom, host(w), host(b), top_k, pooled_q=True)
    dec = decided_blocks(ref["ranked"], top_k).all(axis=0)
    owner = _owner_blocks(geom, np.arange(geom.n_tokens))
    pos = {bb: i for i, bb in enumerate(ref["blocks"])}
    rows = np.array([t for t in range(geom.n_tokens) if dec[pos[owner[t]]]])
    assert len(rows) >= 64
    assert_close(host(out)[rows], ref["o"][rows], geom.dtype, "gsa layer (block-level compressed)")


@pytest.mark.parametrize("geom,top_k", [
    pytest.param(Geometry(3, 5, 13, 11, 2, 64, "bf16"), 5, id="ragged-bf16"),
    pytest.param(Geometry(2, 2, 9, 9, 3, 64, "f32"), 3, id="ragged-f32"),
    pytest.param(Geometry(6, 5, 37, 37, 2, 64, "bf16"), 16, id="scene-bf16"),
])
def test_zero_padded_pooling(geom, top_k):
    """Pooling of the zero-padded grid (edge windows divided by 16): every
    pooled key/value and mean query against the oracle, then the whole layer
    on decided rows."""
    _announce(f"zero-padded pooling {geom}")
    dist = "normal" if geom.dtype == "f32" else "scene"
    q, k, v = make_qkv(geom, seed=91, device=DEV, distribution=dist)
    w, b = make_gate(geom.n_heads, 64, seed=91, device=DEV)
    k_cmp, v_cmp, k32, q32 = sga.gsa_compress(q, k, v, geom, include_pad=True)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    rkc, rvc = oracle.compress(kh, vh, geom, 4, include_pad=True)
    assert_close(host(k_cmp), rkc, geom.dtype, "k_cmp (zero-padded)")
    assert_close(host(v_cmp), rvc, geom.dtype, "v_cmp (zero-padded)")
    assert_close(host(k32), rkc, "f32", "k_cmp_f32 (zero-padded)")
    assert_close(host(q32), oracle.pooled_queries(qh, geom, 4), "f32", "q_blk_f32 (zero-padded run)")
    out = sga.gsa_layer(q, k, v, w, b, geom, top_k, include_pad=True)
    _sync()
    ref = oracle.gsa_layer(qh, kh, vh, geom, host(w), host(b), top_k, include_pad=True)
    dec = decided_blocks(ref["ranked"], top_k).all(axis=0)
    owner = _owner_blocks(geom, np.arange(geom.n_tokens))
    pos = {bb: i for i, bb in enumerate(ref["blocks"])}
    rows = np.array([t for t in range(geom.n_tokens) if dec[pos[owner[t]]]])
    assert len(rows) >= 64
    assert_close(host(out)[rows], ref["o"][rows], geom.dtype, "gsa layer (zero-padded pooling)")


def test_deterministic():
    geom = Geometry(8, 5, 37, 37, 4, 64, "bf16")
    _announce(f"determinism {geom}")
    q, k, v = make_qkv(geom, seed=9, device=DEV, distribution="scene")
    w, b = make_gate(geom.n_heads, 64, seed=9, device=DEV)
    a = sga.gsa_layer(q, k, v, w, b, geom, 16, keep_intermediates=True)
    c = sga.gsa_layer(q, k, v, w, b, geom, 16, keep_intermediates=True)
    d1 = sga.dense_global_attn(q, k, v, geom)
    d2 = sga.dense_global_attn(q, k, v, geom)
    s1 = sga.subsampled_global_attn(q, k, v, geom, 4, 4)
    s2 = sga.subsampled_global_attn(q, k, v, geom, 4, 4)
    _sync()
    for key in a:
        assert torch.equal(a[key], c[key]), key
    assert torch.equal(d1, d2)
    assert torch.equal(s1, s2)
    # the variants: bit-identical repeats too (the wide selection's persistent
    # workgroups and per-lane buffers involve no atomics or races)
    for kw in (dict(top_k=128), dict(top_k=16, keep_ref=True), dict(top_k=16, pooled_q=True),
               dict(top_k=16, include_pad=True)):
        top_k = kw.pop("top_k")
        e = sga.gsa_layer(q, k, v, w, b, geom, top_k, keep_intermediates=True, **kw)
        f = sga.gsa_layer(q, k, v, w, b, geom, top_k, keep_intermediates=True, **kw)
        _sync()
        for key in e:
            assert torch.equal(e[key], f[key]), (kw, key)
    t1 = sga.subsampled_global_attn(q, k, v, geom, 4, 4, mode=2)
    t2 = sga.subsampled_global_attn(q, k, v, geom, 4, 4, mode=2)
    f1 = sga.subsampled_global_attn(q, k, v, geom, 4, 4, mode=1)
    f2 = sga.dense_global_attn(q, k, v, geom, frame_local=True)
    f3 = sga.dense_global_attn(q, k, v, geom, frame_local=True)
    _sync()
    assert torch.equal(t1, t2)
    assert torch.equal(f1, f2) and torch.equal(f2, f3)


# ---------------------------------------------------------------------------
# workload-sized cases: seeded row samples
# ---------------------------------------------------------------------------

def _workload_inputs(name, seed=1):
    wl = WORKLOADS[name]
    geom = wl.geom
    q, k, v = make_qkv(geom, seed=seed, device=DEV, distribution=wl.distribution)
    return wl, geom, q, k, v


def _plant_probes(q, k, geom, n_probe, seed):
    """Give n_probe query rows one sharply matching key each, far away in the
    token order, so that an indexing slip changes their output completely."""
    rng = np.random.default_rng(seed)
    T, H = geom.n_tokens, geom.n_heads
    probes = rng.choice(T, n_probe, replace=False)
    targets = rng.choice(T, n_probe, replace=False)
    u = torch.randn((n_probe, H, 64), generator=torch.Generator().manual_seed(seed))
    u = u / u.norm(dim=-1, keepdim=True) * 15.5
    u = u.to(q.dtype).to(q.device)
    k[torch.from_numpy(targets).to(q.device)] = u
    q[torch.from_numpy(probes).to(q.device)] = u
    return np.sort(probes)


@pytest.mark.timeout(900)
def test_dense32():
    wl, geom, q, k, v = _workload_inputs("dense32")
    probes = _plant_probes(q, k, geom, 64, seed=2)
    rows = np.union1d(sample_rows(geom.n_tokens, wl.check_rows, seed=1).numpy(), probes)
    _announce(f"dense32 dense+frame, {len(rows)} rows")
    o = sga.dense_global_attn(q, k, v, geom)
    of = sga.dense_global_attn(q, k, v, geom, frame_local=True)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    W = oracle_workers()
    assert_close(host(o)[rows], oracle.dense_attention(qh, kh, vh, rows=rows, workers=W), "bf16",
                 "dense32 dense")
    assert_close(host(of)[rows], oracle.frame_attention(qh, kh, vh, geom, rows=rows), "bf16",
                 "dense32 frame")


def _fine_on_oracle_sets(q, k, v, geom, w, b, out, ref, rows, top_k, name, keep_ref=False):
    """The fine branch and the gate on every sampled row: the fine kernel gets
    the oracle's index sets for the sampled rows' query blocks (the same input
    on both sides), so rows whose selection is undecided are checked too."""
    idx_mix = out["idx"].clone()
    idx_mix[:, torch.from_numpy(ref["blocks"]).to(DEV)] = torch.from_numpy(ref["idx"]).to(DEV)
    o_slc = sga.gsa_sparse_attn(q, k, v, idx_mix, geom, top_k, keep_ref=keep_ref)
    o = sga.gsa_gate(q, out["o_cmp"], o_slc, w, b, geom)
    o_fused = sga.gsa_sparse_attn_gated(q, k, v, idx_mix, out["o_cmp"], w, b, geom, top_k, keep_ref=keep_ref)
    _sync()
    assert_close(host(o_slc)[rows], ref["o_slc"], "bf16", f"{name} o_slc (oracle sets, all rows)")
    assert_close(host(o)[rows], ref["o"], "bf16", f"{name} gsa layer (oracle sets, all rows)")
    assert_close(host(o_fused)[rows], ref["o"], "bf16", f"{name} gate fused into fine (oracle sets, all rows)")


def _layer_on_own_selection(qh, kh, vh, geom, w, b, out, o_layer, ref, rows, name, keep_ref, W):
    """The GSA layer with the GPU's own top-K on every sampled row: the oracle's
    fine branch and gate run on the index sets the GPU selected (each of them
    already checked valid: exact on decided blocks, within the score gap
    elsewhere), with the oracle's compressed branch; the GPU's fine branch,
    its separate gate and the layer with the gate folded in must all match."""
    idx_gpu = host(out["idx"]).astype(np.int32)
    o_slc = oracle.fine_attention(qh, kh, vh, geom, 4, idx_gpu, rows=rows, keep_ref=keep_ref, workers=W)
    o = oracle.gate(qh[rows], ref["o_cmp"], o_slc, host(w), host(b))
    assert_close(host(out["o_slc"])[rows], o_slc, "bf16", f"{name} o_slc (own selection, all rows)")
    assert_close(host(out["o"])[rows], o, "bf16", f"{name} gsa layer (own selection, all rows)")
    assert_close(host(o_layer)[rows], o, "bf16", f"{name} gsa layer, fused gate (own selection, all rows)")


def _gsa_check(name, rows_cap=None, keep_ref=False, pooled_q=False, include_pad=False,
               probability_scores=False):
    wl, geom, q, k, v = _workload_inputs(name)
    w, b = make_gate(geom.n_heads, 64, seed=1, device=DEV)
    rows = sample_rows(geom.n_tokens, rows_cap or wl.check_rows, seed=1).numpy()
    _announce(f"{name} GSA layer (reference frame kept: {keep_ref}, block-level compressed: "
              f"{pooled_q}), {len(rows)} rows")
    out = sga.gsa_layer(q, k, v, w, b, geom, wl.top_k, keep_intermediates=True, keep_ref=keep_ref,
                        pooled_q=pooled_q, include_pad=include_pad, probability_scores=probability_scores)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    W = oracle_workers()
    ref = oracle.gsa_layer(qh, kh, vh, geom, host(w), host(b), wl.top_k, rows=rows, workers=W,
                           keep_ref=keep_ref, pooled_q=pooled_q, include_pad=include_pad,
                           probability_scores=probability_scores)
    assert_close(host(out["k_cmp"]), ref["k_cmp"], "bf16", f"{name} k_cmp")
    assert_close(host(out["v_cmp"]), ref["v_cmp"], "bf16", f"{name} v_cmp")
    assert_close(host(out["k_cmp_f32"]), ref["k_cmp"], "f32", f"{name} k_cmp_f32")
    assert_close(host(out["q_blk_f32"])[ref["blocks"]], ref["q_blk"], "f32", f"{name} q_blk_f32")
    assert_close(host(out["o_cmp"])[rows], ref["o_cmp"], "bf16", f"{name} o_cmp")
    idx = host(out["idx"]).astype(np.int64)[:, ref["blocks"]]
    score_of = None
    if probability_scores:
        first = _nb(geom) if keep_ref else 0
        psc = oracle.probability_block_scores(qh, ref["k_cmp"], geom, 4, ref["blocks"], first=first, workers=W)
        score_of = lambda h, bi, picks: np.log(psc[h, bi, picks - first])  # noqa: E731
    check_topk(idx, ref["idx"], ref["ranked"], ref["q_blk"], ref["k_cmp"], f"{name} top-K", score_of=score_of)
    if probability_scores:
        again = sga.gsa_select_topk_probability(q, out["k_cmp_f32"], geom, wl.top_k, keep_ref=keep_ref)
    else:
        again = sga.gsa_select_topk(out["q_blk_f32"], out["k_cmp_f32"], geom, wl.top_k, keep_ref=keep_ref)
    _sync()
    assert torch.equal(again, out["idx"]), f"{name} top-K repeat differs"
    # rows whose query block is decided in every head see identical index sets
    dec = decided_blocks(ref["ranked"], wl.top_k).all(axis=0)
    owner = _owner_blocks(geom, rows)
    pos = {bb: i for i, bb in enumerate(ref["blocks"])}
    keep = np.array([dec[pos[o]] for o in owner])
    print(f"[parity] {name}: {keep.mean() * 100:.1f}% of sampled rows fully decided", flush=True)
    if keep.any():  # (with close block scores no sampled row may be decided in all 16 heads)
        assert_close(host(out["o_slc"])[rows][keep], ref["o_slc"][keep], "bf16", f"{name} o_slc")
        assert_close(host(out["o"])[rows][keep], ref["o"][keep], "bf16", f"{name} gsa layer")
    # the layer as one calls it (the gate folded into the fine branch), on every
    # sampled row
    o_fused = sga.gsa_layer(q, k, v, w, b, geom, wl.top_k, keep_ref=keep_ref, pooled_q=pooled_q,
                            include_pad=include_pad, probability_scores=probability_scores)
    _sync()
    _layer_on_own_selection(qh, kh, vh, geom, w, b, out, o_fused, ref, rows, name, keep_ref, W)
    _fine_on_oracle_sets(q, k, v, geom, w, b, out, ref, rows, wl.top_k, name, keep_ref)


@pytest.mark.timeout(900)
def test_gsa128():
    _gsa_check("gsa128")


@pytest.mark.timeout(900)
def test_gsa128_reference_frame():
    _gsa_check("gsa128", rows_cap=1024, keep_ref=True)


@pytest.mark.timeout(900)
def test_gsa128_block_level_compressed():
    _gsa_check("gsa128", rows_cap=1024, pooled_q=True)


@pytest.mark.timeout(900)
def test_gsa128_zero_padded_pooling():
    _gsa_check("gsa128", rows_cap=1024, include_pad=True)


def _sga_check(name, rows_cap=None):
    wl, geom, q, k, v = _workload_inputs(name)
    rows = sample_rows(geom.n_tokens, rows_cap or wl.check_rows, seed=1).numpy()
    _announce(f"{name} subsampled + frame, {len(rows)} rows")
    sh, sw = wl.stride
    o = sga.subsampled_global_attn(q, k, v, geom, sh, sw)
    of = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=1)
    od = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=2)
    # repeats are bit-identical: a stage refilled while another wave still
    # reads it would show here first (hundreds of workgroups per CU in turn)
    o2 = sga.subsampled_global_attn(q, k, v, geom, sh, sw)
    of2 = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=1)
    _sync()
    assert torch.equal(o, o2), f"{name} subsampled repeat differs"
    assert torch.equal(of, of2), f"{name} frame repeat differs"
    del o2, of2
    qh, kh, vh = host(q), host(k), host(v)
    W = oracle_workers()
    assert_close(host(o)[rows], oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, rows=rows,
                                                            workers=W), "bf16", f"{name} subsampled")
    assert_close(host(od)[rows], oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, mode=2,
                                                             rows=rows, workers=W), "bf16",
                 f"{name} subsampled token diagonal")
    assert_close(host(of)[rows], oracle.frame_attention(qh, kh, vh, geom, rows=rows), "bf16",
                 f"{name} frame")


PROB_GEOMS = [
    pytest.param(Geometry(3, 5, 13, 11, 2, 64, "bf16"), id="ragged"),
    pytest.param(Geometry(1, 1, 5, 7, 1, 64, "bf16"), id="one-frame"),
    pytest.param(Geometry(5, 0, 1, 1, 1, 64, "bf16"), id="1x1-grid"),
    pytest.param(Geometry(2, 16, 3, 5, 2, 64, "bf16"), id="16-specials"),
    pytest.param(Geometry(6, 5, 37, 37, 2, 64, "bf16"), id="scene"),
]


@pytest.mark.parametrize("geom", PROB_GEOMS)
def test_probability_block_scores(geom):
    """Selection by probability-mean block scores against the oracle on every
    query block, for several widths and with the reference frame kept."""
    _announce(f"probability-mean selection {geom}")
    q, k, v = make_qkv(geom, seed=41, device=DEV, distribution="scene")
    _, _, k32, _ = sga.gsa_compress(q, k, v, geom)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    rkc, _ = oracle.compress(kh, vh, geom, 4)
    N, nb = geom.n_frames, _nb(geom)
    blocks = list(range(N * _nqb(geom)))
    for keep_ref in ((False, True) if N >= 2 else (False,)):
        first = nb if keep_ref else 0
        n_cand = N * nb - first
        psc = oracle.probability_block_scores(qh, rkc, geom, 4, blocks, first=first)
        for top_k in sorted({1, min(5, n_cand), min(16, n_cand)}):
            idx, sc = sga.gsa_select_topk_probability(q, k32, geom, top_k, want_score=True, keep_ref=keep_ref)
            again = sga.gsa_select_topk_probability(q, k32, geom, top_k, keep_ref=keep_ref)
            _sync()
            assert torch.equal(idx, again)
            ridx, ranked = oracle.select_topk_probability(qh, rkc, geom, top_k, 4, blocks, first=first)
            idx_h = host(idx).astype(np.int64)
            check_topk(idx_h, ridx, ranked, None, None, f"probability top-{top_k} keep_ref={keep_ref}",
                       score_of=lambda h, bi, picks: np.log(psc[h, bi, picks - first]))
            # the scores the kernel reports are the oracle's for its picks
            want = np.take_along_axis(psc, idx_h - first, axis=2)
            rel = np.max(np.abs(host(sc) - want) / want)
            print(f"[parity] probability scores top-{top_k}: max rel err {rel:.2e}", flush=True)
            assert rel < 1e-4


def test_probability_rising_logits():
    """Logits that rise by hundreds of log2 units from frame to frame (the
    first frame's far below zero): each token's log-sum-exp must move its
    reference several times along the key stream and still match the oracle."""
    geom = Geometry(6, 5, 37, 37, 2, 64, "bf16")
    _announce(f"probability-mean selection, rising logits {geom}")
    q, k, v = make_qkv(geom, seed=43, device=DEV, distribution="scene")
    gen = torch.Generator().manual_seed(44)
    u = torch.randn(geom.n_heads, 64, generator=gen, dtype=torch.float64)
    u = (u / u.norm(dim=1, keepdim=True)).to(torch.float32)
    L = geom.n_special + geom.grid_h * geom.grid_w
    s_f = torch.tensor([-60.0, -20.0, 0.0, 10.0, 20.0, 40.0]).repeat_interleave(L)
    q = (q.float() + 30.0 * u.to(DEV)).to(torch.bfloat16).contiguous()
    k = (k.float() + s_f.to(DEV)[:, None, None] * u.to(DEV)).to(torch.bfloat16).contiguous()
    _, _, k32, _ = sga.gsa_compress(q, k, v, geom)
    _sync()
    qh, kh, vh = host(q), host(k), host(v)
    rkc, _ = oracle.compress(kh, vh, geom, 4)
    blocks = list(range(geom.n_frames * _nqb(geom)))
    psc = oracle.probability_block_scores(qh, rkc, geom, 4, blocks)
    idx, sc = sga.gsa_select_topk_probability(q, k32, geom, 16, want_score=True)
    _sync()
    ridx, ranked = oracle.select_topk_probability(qh, rkc, geom, 16, 4, blocks)
    idx_h = host(idx).astype(np.int64)
    check_topk(idx_h, ridx, ranked, None, None, "probability top-16, rising logits",
               score_of=lambda h, bi, picks: np.log(psc[h, bi, picks]))
    want = np.take_along_axis(psc, idx_h, axis=2)
    rel = np.max(np.abs(host(sc) - want) / want)
    # The kernels hold each key times log2(e) as two bf16 planes (hi + lo,
    # 2^-18 relative), so a logit s carries an error up to 2^-18 A with
    # A = sum_i |q_i k_i| log2(e) / 8, and s - lse up to twice that: the
    # probability's relative error is bounded by ln(2) 2^-17 max A.
    a_max = max(float((np.abs(qh[:, h]) @ np.abs(rkc[:, h]).T).max()) for h in range(geom.n_heads))
    a_max *= math.log2(math.e) / 8
    tol = 1e-4 + math.log(2) * 2.0 ** -17 * a_max
    print(f"[parity] probability scores, rising logits: max rel err {rel:.2e} (bound {tol:.2e}, "
          f"max A {a_max:.0f} log2 units)", flush=True)
    assert rel < tol


def test_gsa128_probability_scores():
    _gsa_check("gsa128", rows_cap=1024, probability_scores=True)


@pytest.mark.timeout(900)
def test_sga256():
    _sga_check("sga256")


# ---------------------------------------------------------------------------
# the 1000-frame workload (1,374,000 tokens) in the launch configuration the
# benchmark times; seeded row samples, one shared input set
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def scene1000():
    wl, geom, q, k, v = _workload_inputs("scene1000")
    probes = _plant_probes(q, k, geom, 64, seed=3)
    torch.cuda.synchronize()
    _announce("scene1000 inputs ready; copying to host")
    host_qkv = (host(q), host(k), host(v))
    return wl, geom, q, k, v, probes, host_qkv


@pytest.mark.timeout(1200)
def test_scene1000_dense(scene1000):
    wl, geom, q, k, v, probes, (qh, kh, vh) = scene1000
    # 4096 sampled rows + the 64 planted probes: every head, all d (the dense
    # oracle over 1.374M keys costs ~2e9 fp64 flop per row; eight passes, each
    # reported)
    rows = np.union1d(sample_rows(geom.n_tokens, wl.check_rows, seed=5).numpy(), probes)
    _announce(f"scene1000 dense, {len(rows)} rows")
    o = sga.dense_global_attn(q, k, v, geom)
    _sync()
    ref = []
    for part in np.array_split(rows, 8):
        ref.append(oracle.dense_attention(qh, kh, vh, rows=part, workers=oracle_workers()))
        print(f"[oracle] scene1000 dense: {sum(len(r) for r in ref)} rows", flush=True)
    assert_close(host(o)[rows], np.concatenate(ref), "bf16", "scene1000 dense")
    assert_close(host(o)[probes], oracle.dense_attention(qh, kh, vh, rows=probes,
                                                         workers=oracle_workers()),
                 "bf16", "scene1000 dense planted probes")


@pytest.mark.timeout(1200)
def test_scene1000_gsa(scene1000):
    wl, geom, q, k, v, probes, (qh, kh, vh) = scene1000
    w, b = make_gate(geom.n_heads, 64, seed=1, device=DEV)
    rows = sample_rows(geom.n_tokens, wl.check_rows, seed=1).numpy()
    _announce(f"scene1000 GSA layer, {len(rows)} rows")
    out = sga.gsa_layer(q, k, v, w, b, geom, wl.top_k, keep_intermediates=True)
    _sync()
    W = oracle_workers()
    ref = oracle.gsa_layer(qh, kh, vh, geom, host(w), host(b), wl.top_k, rows=rows, workers=W)
    assert_close(host(out["k_cmp"]), ref["k_cmp"], "bf16", "scene1000 k_cmp")
    assert_close(host(out["v_cmp"]), ref["v_cmp"], "bf16", "scene1000 v_cmp")
    assert_close(host(out["o_cmp"])[rows], ref["o_cmp"], "bf16", "scene1000 o_cmp")
    idx = host(out["idx"]).astype(np.int64)[:, ref["blocks"]]
    check_topk(idx, ref["idx"], ref["ranked"], ref["q_blk"], ref["k_cmp"], "scene1000 top-K")
    # the selection repeats bit for bit at full size, the register path and the
    # wide one (a tile read before its direct-to-LDS loads landed changed a few
    # rows per head from call to call)
    for top_k in (wl.top_k, 128):
        first = sga.gsa_select_topk(out["q_blk_f32"], out["k_cmp_f32"], geom, top_k)
        again = sga.gsa_select_topk(out["q_blk_f32"], out["k_cmp_f32"], geom, top_k)
        _sync()
        assert torch.equal(first, again), f"scene1000 top-{top_k} repeat differs"
        if top_k == wl.top_k:
            assert torch.equal(first, out["idx"]), "scene1000 top-K differs from the layer's"
        del first, again
    dec = decided_blocks(ref["ranked"], wl.top_k).all(axis=0)
    owner = _owner_blocks(geom, rows)
    pos = {bb: i for i, bb in enumerate(ref["blocks"])}
    keep = np.array([dec[pos[o]] for o in owner])
    print(f"[parity] scene1000: {keep.mean() * 100:.1f}% of sampled rows fully decided", flush=True)
    assert keep.sum() > 0
    assert_close(host(out["o_slc"])[rows][keep], ref["o_slc"][keep], "bf16", "scene1000 o_slc")
    assert_close(host(out["o"])[rows][keep], ref["o"][keep], "bf16", "scene1000 gsa layer")
    o_fused = sga.gsa_layer(q, k, v, w, b, geom, wl.top_k)
    _sync()
    _layer_on_own_selection(qh, kh, vh, geom, w, b, out, o_fused, ref, rows, "scene1000", False, W)
    del o_fused
    _fine_on_oracle_sets(q, k, v, geom, w, b, out, ref, rows, wl.top_k, "scene1000")


@pytest.mark.timeout(600)
def test_scene1000_repeat(scene1000):
    """Every form and variant twice on the 1000-frame batch: bit-identical.
    Races between a tile's loads and its readers show only at this size."""
    wl, geom, q, k, v, probes, _ = scene1000
    w, b = make_gate(geom.n_heads, 64, seed=1, device=DEV)
    calls = {
        "frame": lambda: sga.dense_global_attn(q, k, v, geom, frame_local=True),
        "subsampled": lambda: sga.subsampled_global_attn(q, k, v, geom, 4, 4),
        "subsampled log-count": lambda: sga.subsampled_global_attn(q, k, v, geom, 4, 4, mean_log_count=True),
        "token diagonal": lambda: sga.subsampled_global_attn(q, k, v, geom, 4, 4, mode=2),
        "gsa top-16": lambda: sga.gsa_layer(q, k, v, w, b, geom, 16, keep_intermediates=True),
        "gsa top-128": lambda: sga.gsa_layer(q, k, v, w, b, geom, 128, keep_intermediates=True),
        "gsa reference frame": lambda: sga.gsa_layer(q, k, v, w, b, geom, 16, keep_intermediates=True,
                                                     keep_ref=True),
        "gsa block-level": lambda: sga.gsa_layer(q, k, v, w, b, geom, 16, keep_intermediates=True,
                                                 pooled_q=True),
        "gsa zero-padded": lambda: sga.gsa_layer(q, k, v, w, b, geom, 16, keep_intermediates=True,
                                                 include_pad=True),
        "gsa probability scores": lambda: sga.gsa_layer(q, k, v, w, b, geom, 16, keep_intermediates=True,
                                                        probability_scores=True),
        "gsa fused gate": lambda: sga.gsa_layer(q, k, v, w, b, geom, 16),
    }
    for name, fn in calls.items():
        _announce(f"scene1000 repeat: {name}")
        a = fn()
        c = fn()
        _sync()
        if isinstance(a, dict):
            for key in a:
                assert torch.equal(a[key], c[key]), f"scene1000 {name}: {key} differs between calls"
        else:
            assert torch.equal(a, c), f"scene1000 {name} differs between calls"
        del a, c


@pytest.mark.timeout(1200)
def test_scene1000_subsampled(scene1000):
    wl, geom, q, k, v, probes, (qh, kh, vh) = scene1000
    rows = sample_rows(geom.n_tokens, wl.check_rows, seed=1).numpy()
    _announce(f"scene1000 subsampled + frame, {len(rows)} rows")
    sh, sw = wl.stride
    o = sga.subsampled_global_attn(q, k, v, geom, sh, sw)
    of = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=1)
    _sync()
    W = oracle_workers()
    ref = []
    for part in np.array_split(rows, 4):  # four oracle passes, each reported
        ref.append(oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, rows=part, workers=W))
        print(f"[oracle] scene1000 subsampled: {sum(len(r) for r in ref)} rows", flush=True)
    assert_close(host(o)[rows], np.concatenate(ref), "bf16", "scene1000 subsampled")
    assert_close(host(of)[rows], oracle.frame_attention(qh, kh, vh, geom, rows=rows), "bf16",
                 "scene1000 frame")


@pytest.mark.timeout(1200)
def test_scene1000_variants(scene1000):
    """The variants the benchmark times at 1000 frames, on 4096 sampled rows:
    top-128 selection, the VGGT reference frame (selection and fine branch, on
    the oracle's index sets and on the GPU's own), the block-level compressed
    branch and the token-level AVGGT diagonal."""
    wl, geom, q, k, v, probes, (qh, kh, vh) = scene1000
    rows = sample_rows(geom.n_tokens, wl.check_rows, seed=9).numpy()
    nb = _nb(geom)
    W = oracle_workers()
    _announce(f"scene1000 variants, {len(rows)} rows")
    k_cmp, v_cmp, k32, q32 = sga.gsa_compress(q, k, v, geom)
    idx128 = sga.gsa_select_topk(q32, k32, geom, 128)
    idx_ref = sga.gsa_select_topk(q32, k32, geom, wl.top_k, keep_ref=True)
    o_blk = sga.gsa_compressed_pooled(q32, k_cmp, v_cmp, geom)
    o_diag = sga.subsampled_global_attn(q, k, v, geom, *wl.stride, mode=2)
    _sync()
    rkc, rvc = oracle.compress(kh, vh, geom, 4)
    print("[oracle] scene1000 pooled keys ready", flush=True)
    need = np.unique(_owner_blocks(geom, rows))
    rqb = oracle.pooled_queries(qh, geom, 4, blocks=need)
    ridx, ranked = oracle.select_topk(rqb, rkc, 128, workers=W)
    check_topk(host(idx128).astype(np.int64)[:, need], ridx, ranked, rqb, rkc, "scene1000 top-128")
    ridx_r, ranked_r = oracle.select_topk(rqb, rkc, wl.top_k, workers=W, first=nb)
    check_topk(host(idx_ref).astype(np.int64)[:, need], ridx_r, ranked_r, rqb, rkc,
               "scene1000 top-K (reference frame kept)")
    # the fine branch with frame 0 kept whole, fed the oracle's index sets
    idx_mix = idx_ref.clone()
    idx_mix[:, torch.from_numpy(need).to(DEV)] = torch.from_numpy(ridx_r).to(DEV)
    o_slc = sga.gsa_sparse_attn(q, k, v, idx_mix, geom, wl.top_k, keep_ref=True)
    _sync()
    idx_full = np.zeros((geom.n_heads, geom.n_frames * _nqb(geom), wl.top_k), dtype=np.int32)
    idx_full[:, need] = ridx_r
    assert_close(host(o_slc)[rows], oracle.fine_attention(qh, kh, vh, geom, 4, idx_full, rows=rows,
                                                          keep_ref=True, workers=W),
                 "bf16", "scene1000 o_slc (reference frame kept)")
    # ... and on the GPU's own selection (checked valid above)
    o_slc_own = sga.gsa_sparse_attn(q, k, v, idx_ref, geom, wl.top_k, keep_ref=True)
    _sync()
    assert_close(host(o_slc_own)[rows],
                 oracle.fine_attention(qh, kh, vh, geom, 4, host(idx_ref).astype(np.int32), rows=rows,
                                       keep_ref=True, workers=W),
                 "bf16", "scene1000 o_slc (reference frame kept, own selection)")
    del o_slc_own
    assert_close(host(o_blk)[rows], oracle.compressed_attention_pooled(qh, rkc, rvc, geom, 4,
                                                                      rows=rows, workers=W),
                 "bf16", "scene1000 o_cmp (block level)")
    sh, sw = wl.stride
    assert_close(host(o_diag)[rows], oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, mode=2,
                                                                 rows=rows, workers=W),
                 "bf16", "scene1000 subsampled token diagonal")
