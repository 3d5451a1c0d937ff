"""The allocation-free selection entry point (gsa_select_topk_noalloc) against
gsa_select_topk, through the C ABI: the same kernels on the library's per-GPU
scratch array instead of a caller workspace, so the results must be identical
bit for bit -- on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), over the two-stage path (top_k <=
16, with its exact fallback) and the wide path; a problem whose selection
scratch does not fit is refused before anything runs."""
from __future__ import annotations

import pytest
import torch

import sparse_attention_global_amd as sga
from synth import Geometry, make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(geom, seed):
    q, k, v = make_qkv(geom, seed=seed, device=DEV, distribution="scene")
    _, _, k32, q32 = sga.gsa_compress(q, k, v, geom)
    return q32, k32


@pytest.mark.parametrize("top_k", [16, 5, 32])
def test_noalloc_matches_workspace_entry(top_k):
    if top_k <= 16:
        cases = [
            (Geometry(96, 5, 37, 37, 16, 64, "bf16"), False),  # the scratch reduces the fallback split
            (Geometry(12, 5, 37, 37, 2, 64, "bf16"), True),    # then a smaller call, reference frame kept
        ]
    else:  # the wide path's candidate buffers take 1 MiB per 128-block tile and head
        cases = [
            (Geometry(24, 5, 37, 37, 4, 64, "bf16"), False),
            (Geometry(6, 5, 37, 37, 2, 64, "bf16"), True),
        ]
    for i, (geom, keep_ref) in enumerate(cases):
        print(f"[case] noalloc top-{top_k} call {i}: {geom} keep_ref={keep_ref}", flush=True)
        q32, k32 = _inputs(geom, seed=50 + i)
        want_i, want_s = sga.gsa_select_topk(q32, k32, geom, top_k, want_score=True, keep_ref=keep_ref)
        got_i, got_s = sga.gsa_select_topk_noalloc(q32, k32, geom, top_k, want_score=True, keep_ref=keep_ref)
        again = sga.gsa_select_topk_noalloc(q32, k32, geom, top_k, keep_ref=keep_ref)
        torch.cuda.synchronize()
        assert torch.equal(got_i, want_i), (top_k, i)
        assert torch.equal(got_s, want_s), (top_k, i)
        assert torch.equal(again, want_i), (top_k, i)
        del q32, k32


def test_noalloc_no_split_capacity():
    """At 209 frames and 16 heads the selection scratch leaves the fallback no
    split capacity (the next 128 listed rows would not fit): every block that
    misses the certificate streams all keys in one workgroup, and the result
    still equals the workspace entry point's (split fallback, merged)."""
    geom = Geometry(209, 5, 37, 37, 16, 64, "bf16")
    print(f"[case] noalloc, no split capacity: {geom}", flush=True)
    q32, k32 = _inputs(geom, seed=61)
    want_i, want_s = sga.gsa_select_topk(q32, k32, geom, 16, want_score=True)
    got_i, got_s = sga.gsa_select_topk_noalloc(q32, k32, geom, 16, want_score=True)
    torch.cuda.synchronize()
    assert torch.equal(got_i, want_i)
    assert torch.equal(got_s, want_s)


def test_noalloc_all_ties_fallback():
    """Every block misses the certificate (all pooled keys equal), so the exact
    fallback runs with the capacity the scratch leaves it; ties go to the
    lowest indices, as with the workspace entry point."""
    geom = Geometry(96, 5, 37, 37, 16, 64, "bf16")
    N, H = geom.n_frames, geom.n_heads
    g = torch.Generator(device="cpu").manual_seed(3)
    k32 = torch.randn((1, H, 64), generator=g).repeat(N * 100, 1, 1).to(DEV)
    q32 = torch.randn((N * 101, H, 64), generator=g).to(DEV)
    got = sga.gsa_select_topk_noalloc(q32, k32, geom, 16)
    want = sga.gsa_select_topk(q32, k32, geom, 16)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert (got.cpu() == torch.arange(16, dtype=torch.int32)[None, None, :]).all()


def test_noalloc_refuses_oversized():
    geom = Geometry(1000, 5, 37, 37, 16, 64, "bf16")
    q32 = torch.zeros((1000 * 101, 16, 64), dtype=torch.float32, device=DEV)
    k32 = torch.zeros((1000 * 100, 16, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError, match="scratch"):
        sga.gsa_select_topk_noalloc(q32, k32, geom, 16)
