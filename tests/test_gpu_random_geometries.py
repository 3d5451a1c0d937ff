"""Seeded random small geometries through the C ABI, every row against the
oracle: dense attention (with its log-sum-exp), frame attention, the subsampled
form (modes 0 and 2, with and without the log-count bias, at a random stride)
and the GSA layer on the GPU's own selection (its picks checked valid against
the oracle's ranking, then the oracle's fine branch and gate run on those same
index sets and compared with the fused-gate layer). The draws cover frame
lengths on both sides of the query-tile sizes (128 and 256 rows), grids whose
sides are not multiples of the 4x4 pooling window, 0-5 special tokens, 1-3
heads, bf16 and fp32, and every top_k from 1 to all pooled keys.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_global_amd as sga
from parity import assert_close, check_topk, host
from synth import Geometry, make_gate, make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _draws(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        n_frames = int(rng.integers(1, 6))
        gh, gw = (int(x) for x in rng.integers(1, 21, size=2))
        n_special = int(rng.integers(0, 6))
        heads = int(rng.integers(1, 4))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        nb = -(-gh // 4) * -(-gw // 4)
        top_k = int(rng.integers(1, n_frames * nb + 1))
        sh, sw = int(rng.integers(1, min(gh, 5) + 1)), int(rng.integers(1, min(gw, 5) + 1))
        out.append(pytest.param(Geometry(n_frames, n_special, gh, gw, heads, 64, dtype), top_k, (sh, sw),
                                id=f"d{i}-N{n_frames}-S{n_special}-{gh}x{gw}-H{heads}-{dtype}-k{top_k}-s{sh}x{sw}"))
    return out


@pytest.mark.parametrize("geom,top_k,stride", _draws(40))
def test_random_geometry(geom, top_k, stride):
    print(f"[case] random geometry {geom} top_k={top_k} stride={stride}", flush=True)
    dt = geom.dtype
    dist = "normal" if dt == "f32" else "scene"
    q, k, v = make_qkv(geom, seed=97, device=DEV, distribution=dist)
    w, b = make_gate(geom.n_heads, 64, seed=97, device=DEV)
    qh, kh, vh = host(q), host(k), host(v)

    o, lse = sga.dense_global_attn(q, k, v, geom, want_lse=True)
    of = sga.dense_global_attn(q, k, v, geom, frame_local=True)
    torch.cuda.synchronize()
    ro, rlse = oracle.dense_attention(qh, kh, vh, with_lse=True)
    assert_close(host(o), ro, dt, "dense")
    assert_close(host(lse), rlse, "f32" if dt == "f32" else "bf16", "dense lse")
    assert_close(host(of), oracle.frame_attention(qh, kh, vh, geom), dt, "frame")

    sh, sw = stride
    for mode in (0, 2):
        for bias in (False, True):
            o_s = sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=mode, mean_log_count=bias)
            torch.cuda.synchronize()
            ref = oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, mode=mode, mean_log_count=bias)
            assert_close(host(o_s), ref, dt, f"subsampled mode {mode} log-count {bias}")

    # the GSA layer as one calls it, on the GPU's own selection
    out = sga.gsa_layer(q, k, v, w, b, geom, top_k, keep_intermediates=True)
    o_layer = sga.gsa_layer(q, k, v, w, b, geom, top_k)
    torch.cuda.synchronize()
    ref = oracle.gsa_layer(qh, kh, vh, geom, host(w), host(b), top_k)
    assert_close(host(out["o_cmp"]), ref["o_cmp"], dt, "o_cmp")
    idx_gpu = host(out["idx"]).astype(np.int64)
    check_topk(idx_gpu[:, ref["blocks"]], ref["idx"], ref["ranked"], ref["q_blk"], ref["k_cmp"], "top-K")
    o_slc = oracle.fine_attention(qh, kh, vh, geom, 4, idx_gpu.astype(np.int32))
    o_ref = oracle.gate(qh, ref["o_cmp"], o_slc, host(w), host(b))
    assert_close(host(out["o_slc"]), o_slc, dt, "o_slc (own selection)")
    assert_close(host(out["o"]), o_ref, dt, "gsa layer (own selection)")
    assert_close(host(o_layer), o_ref, dt, "gsa layer, fused gate (own selection)")
