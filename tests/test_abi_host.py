"""The C-ABI library on the host (no GPU): it loads, exports every function
include/sga.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import sparse_attention_global_amd as sga
from sparse_attention_global_amd._lib import SgaGeom, library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sga.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert set(names) >= {"dense_global_attn", "gsa_compress", "gsa_select_topk", "gsa_sparse_attn",
                          "gsa_gate", "subsampled_global_attn"}
    lib = library()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sga.EXPORTS)


def test_version():
    assert library().sga_version() == 60200


def geom(**kw):
    base = dict(n_frames=2, n_special=5, grid_h=37, grid_w=37, n_heads=16, head_dim=64, dtype=0)
    base.update(kw)
    return SgaGeom(**base)


FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: calls fail validation first
MISALIGNED = ctypes.c_void_p(0x10004)


def last_error():
    return library().sga_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(head_dim=128), UNSUPPORTED, "head_dim"),
    (dict(n_frames=0), INVALID, ">= 1"),
    (dict(n_special=17), INVALID, "n_special"),
    (dict(dtype=5), INVALID, "dtype"),
    (dict(grid_h=70000, grid_w=70000), INVALID, "2^31"),
])
def test_dense_rejects_bad_geometry(kw, code, msg):
    g = geom(**kw)
    st = library().dense_global_attn(ctypes.byref(g), FAKE, FAKE, FAKE, 0, 0, FAKE, None, FAKE, 1 << 40, None)
    assert st == code
    assert msg in last_error()


def test_dense_rejects_null_and_misaligned():
    L = library()
    g = geom()
    big = 1 << 40
    assert L.dense_global_attn(ctypes.byref(g), None, FAKE, FAKE, 0, 0, FAKE, None, FAKE, big, None) == INVALID
    assert "q must not be null" in last_error()
    assert L.dense_global_attn(ctypes.byref(g), FAKE, FAKE, FAKE, 0, 0, MISALIGNED, None, FAKE, big, None) == INVALID
    assert "aligned" in last_error()
    assert L.dense_global_attn(ctypes.byref(g), FAKE, FAKE, FAKE, 5, 1, FAKE, None, FAKE, big, None) == INVALID
    assert "frame_local" in last_error()
    assert L.dense_global_attn(ctypes.byref(g), FAKE, FAKE, FAKE, -1, 0, FAKE, None, FAKE, big, None) == INVALID
    # bf16 needs the V^T staging workspace
    assert L.dense_global_attn(ctypes.byref(g), FAKE, FAKE, FAKE, 0, 0, FAKE, None, None, 0, None) == WORKSPACE
    assert L.dense_global_attn(ctypes.byref(g), FAKE, FAKE, FAKE, 0, 0, FAKE, None, FAKE, 64, None) == WORKSPACE
    assert "workspace" in last_error()


def test_gsa_calls_reject_bad_arguments():
    L = library()
    g = geom()
    assert L.gsa_compress(ctypes.byref(g), 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == UNSUPPORTED
    assert "block" in last_error()
    # pooled queries requested without q
    assert L.gsa_compress(ctypes.byref(g), 4, 0, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == INVALID
    assert L.gsa_compress(ctypes.byref(g), 4, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == INVALID
    assert "include_pad" in last_error()
    nb = 2 * 100
    for bad_k in (0, nb + 1, 129):
        assert L.gsa_select_topk(ctypes.byref(g), 4, FAKE, FAKE, bad_k, 0, FAKE, None, None, 0, None) == INVALID
        assert "top_k" in last_error()
    # with the reference frame kept whole only the other frame's 100 blocks compete
    assert L.gsa_select_topk(ctypes.byref(g), 4, FAKE, FAKE, 101, 2, FAKE, None, None, 0, None) == INVALID
    assert "competing blocks = 100" in last_error()
    assert L.gsa_select_topk(ctypes.byref(geom(n_frames=1)), 4, FAKE, FAKE, 4, 2, FAKE, None,
                             None, 0, None) == INVALID
    assert "2 frames" in last_error()
    for bad_keep in (-1, 4):
        assert L.gsa_select_topk(ctypes.byref(g), 4, FAKE, FAKE, 16, bad_keep, FAKE, None,
                                 None, 0, None) == INVALID
        assert L.gsa_sparse_attn(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, bad_keep, FAKE, None,
                                 None, 0, None) == INVALID
        assert "keep" in last_error()
    assert L.gsa_sparse_attn(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 101, 3, FAKE, None, None, 0,
                             None) == INVALID
    assert L.gsa_gate(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == INVALID
    # the gated fine entry point: the gate's inputs, and an output that would
    # overwrite o_cmp while it is read
    OTHER = ctypes.c_void_p(0x20000)
    gated = L.gsa_sparse_attn_gated
    assert gated(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, 1, None, FAKE, FAKE, OTHER, None, 0,
                 None) == INVALID
    assert "o_cmp" in last_error()
    assert gated(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, 1, FAKE, FAKE, None, OTHER, None, 0,
                 None) == INVALID
    assert "b_gate" in last_error()
    assert gated(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, 1, FAKE, FAKE, FAKE, FAKE, None, 0,
                 None) == INVALID
    assert "alias" in last_error()
    assert gated(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, 1, FAKE, FAKE, FAKE, None, None, 0,
                 None) == INVALID
    assert "o must not be null" in last_error()
    assert gated(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, 4, FAKE, FAKE, FAKE, OTHER, None, 0,
                 None) == INVALID
    assert "keep" in last_error()
    assert gated(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, 1, FAKE, FAKE, FAKE, OTHER, None, 0,
                 None) == WORKSPACE


def test_subsampled_rejects_bad_arguments():
    L = library()
    g = geom()
    args = (FAKE, FAKE, FAKE, FAKE)
    assert L.subsampled_global_attn(ctypes.byref(g), 0, 4, 0, 0, *args, FAKE, 1 << 30, None) == INVALID
    assert L.subsampled_global_attn(ctypes.byref(g), 4, 4, 3, 0, *args, FAKE, 1 << 30, None) == INVALID
    assert "token diagonal" in last_error()
    assert L.subsampled_global_attn(ctypes.byref(g), 4, 4, 0, 3, *args, FAKE, 1 << 30, None) == INVALID
    assert L.subsampled_global_attn(ctypes.byref(g), 4, 4, 0, 0, *args, None, 0, None) == WORKSPACE
    assert L.subsampled_global_attn(ctypes.byref(g), 4, 4, 0, 0, *args, FAKE, 16, None) == WORKSPACE
    assert "workspace" in last_error()
    assert L.sga_compact(ctypes.byref(g), 4, 0, FAKE, FAKE, FAKE, FAKE, None) == INVALID


def _ws(g, op, a, b):
    n = ctypes.c_size_t(0)
    st = library().sga_workspace_size(ctypes.byref(g), op, a, b, ctypes.byref(n))
    return st, n.value


def r256(x):
    return (x + 255) // 256 * 256


def test_workspace_sizes():
    g = geom(n_frames=256)
    T = 256 * 1374
    # dense bf16: V^T staging, keys rounded up to 64 columns, 16 heads x 64 rows
    # of d, then 256 key-norm partial maxima per head (fp32), then one redo flag
    # byte per workgroup of 256 queries
    norms = 16 * 256 * 4
    flags = r256(-(-T // 256) * 16)
    assert _ws(g, 2, 0, 0) == (OK, 16 * 64 * ((T + 63) // 64 * 64) * 2 + norms + flags)
    assert _ws(g, 2, 25600, 0) == (OK, 16 * 64 * 25600 * 2 + norms + flags)
    # frame mode: every frame padded to 1408 columns, 11 workgroups per frame
    frame_flags = r256(11 * 256 * 16)
    assert _ws(g, 2, 0, 1) == (OK, 16 * 64 * 1408 * 256 * 2 + norms + frame_flags)
    assert _ws(g, 2, 5, 1)[0] == INVALID
    # subsampled: per frame 5 specials + 100 kept + 1 mean = 106 rows of K and V,
    # then the frame-padded V^T and the V^T of the 27,136 compacted rows; a
    # frame's queries run as 5 workgroups of 256 and one of 128 (94 rows), each
    # launch with its own redo flags
    half = r256(256 * 106 * 16 * 64 * 2)
    sub_flags = r256(5 * 256 * 16) + r256(1 * 256 * 16)
    flash = r256(16 * 64 * 1408 * 256 * 2 + 16 * 64 * ((256 * 106 + 63) // 64 * 64) * 2 + norms
                 + sub_flags)
    assert _ws(g, 1, 4, 4) == (OK, 2 * half + flash)
    assert sga.compact_rows(g, 4, 4) == (105, 1)
    # fp32 keeps only the compacted set, dense needs nothing
    g1 = geom(n_frames=3, dtype=1)
    assert _ws(g1, 1, 1, 1) == (OK, 2 * r256(3 * (5 + 37 * 37) * 16 * 64 * 4))
    assert _ws(g1, 2, 0, 0) == (OK, 0)
    assert _ws(g1, 7, 1, 1)[0] == INVALID


def test_fine_workspace():
    g = geom(n_frames=256)
    T = 256 * 1374
    lse = r256(T * 16 * 4)

    def expect(rows):
        # the kept tokens' gathered K and V, the queries' log-sum-exp over them,
        # and the dense staging for those keys (V^T, key-norm partials, one redo
        # flag per 256-query workgroup)
        kv = r256(rows * 16 * 64 * 2)
        flash = r256(16 * 64 * ((rows + 63) // 64 * 64) * 2 + 16 * 256 * 4 + r256(-(-T // 256) * 16))
        return 2 * kv + lse + flash

    # special tokens only: 256 frames x 5
    assert _ws(g, 3, 1, 0) == (OK, expect(1280))
    # reference frame only: frame 0's 1374 tokens
    assert _ws(g, 3, 2, 0) == (OK, expect(1374))
    # both: frame 0 whole, then the 255 other frames' 5 specials
    assert _ws(g, 3, 3, 0) == (OK, expect(1374 + 255 * 5))
    assert _ws(g, 3, 0, 0) == (OK, 0)
    assert _ws(geom(n_frames=4, n_special=0), 3, 1, 0) == (OK, 0)
    assert _ws(geom(n_frames=4, dtype=1), 3, 3, 0) == (OK, 0)
    assert _ws(g, 3, 4, 0)[0] == INVALID
    assert _ws(geom(n_frames=1), 3, 2, 0)[0] == INVALID
    assert _ws(g, 3, 1, 7)[0] == INVALID
    # a missing workspace is reported before anything is launched
    L = library()
    for keep in (1, 2, 3):
        assert L.gsa_sparse_attn(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, 16, keep, FAKE, None,
                                 None, 0, None) == WORKSPACE
        assert "workspace" in last_error()


def test_topk_workspace():
    g = geom(n_frames=256)
    n_rows = 256 * 101
    # every width: the pooled keys split into bf16 hi/lo planes (256 bytes per
    # key and head)
    planes = r256(256 * 100 * 16 * 256)
    # top_k <= 16 (two stages while the competing keys fill at most 2048 tiles of
    # 64): 32 candidate words per (head, query block), 256 key-norm partial
    # maxima per head, a count per head and a row list per head of the blocks
    # the certificate missed, then (values and indices) the per-segment lists of
    # the exact fallback: up to 4096 listed rows per head x 8 key segments x 32
    two = (r256(n_rows * 16 * 32 * 4) + r256(16 * 256 * 4) + r256(16 * 4) + r256(n_rows * 16 * 4)
           + 2 * r256(16 * 4096 * 8 * 32 * 4))
    assert _ws(g, 4, 16, 0) == (OK, planes + two)
    assert _ws(g, 4, 1, 2) == (OK, planes + two)
    # past 2048 tiles (131,072 pooled keys) the exact single-stage kernel: planes only
    big = geom(n_frames=1311)
    assert _ws(big, 4, 16, 0) == (OK, r256(1311 * 100 * 16 * 256))
    # wider: then one 1 MiB key buffer per persistent workgroup (128 blocks x 2
    # lanes x 512 keys x 8 bytes), at most 1024 of them, then a score bound
    # (fp32) and a flag byte per (head, query block)
    tiles = -(-n_rows // 128) * 16
    assert _ws(g, 4, 17, 0) == (OK, planes + min(tiles, 1024) * (1 << 20) + r256(n_rows * 16 * 4)
                                + r256(n_rows * 16))
    small = geom(n_frames=3, n_heads=2)
    assert _ws(small, 4, 20, 0) == (OK, r256(3 * 100 * 2 * 256) + 3 * 2 * (1 << 20)
                                    + r256(3 * 101 * 2 * 4) + r256(3 * 101 * 2))  # 3 row tiles x 2 heads
    assert _ws(g, 4, 129, 0)[0] == INVALID
    assert _ws(geom(n_frames=1), 4, 20, 2)[0] == INVALID
    # a missing workspace is reported before anything is launched
    assert library().gsa_select_topk(ctypes.byref(g), 4, FAKE, FAKE, 17, 0, FAKE, None, None, 0,
                                     None) == WORKSPACE
    assert "workspace" in last_error()


def test_topk_probability_workspace_and_checks():
    g = geom(n_frames=256)
    T = 256 * (5 + 37 * 37)
    planes = r256(256 * 100 * 16 * 256)
    # the key planes, then an fp32 log-sum-exp per (token, head)
    assert _ws(g, 6, 16, 0) == (OK, planes + r256(T * 16 * 4))
    assert _ws(g, 6, 16, 2) == (OK, planes + r256(T * 16 * 4))
    assert _ws(g, 6, 17, 0)[0] == UNSUPPORTED
    assert _ws(g, 6, 0, 0)[0] == INVALID
    assert _ws(geom(n_frames=4, dtype=1), 6, 4, 0)[0] == UNSUPPORTED
    L = library()
    sel = L.gsa_select_topk_probability
    assert sel(ctypes.byref(g), 4, FAKE, FAKE, 17, 0, FAKE, None, FAKE, 1 << 40, None) == UNSUPPORTED
    assert "16" in last_error()
    assert sel(ctypes.byref(geom(n_frames=4, dtype=1)), 4, FAKE, FAKE, 4, 0, FAKE, None, FAKE, 1 << 40,
               None) == UNSUPPORTED
    assert "bf16" in last_error()
    assert sel(ctypes.byref(g), 4, None, FAKE, 16, 0, FAKE, None, FAKE, 1 << 40, None) == INVALID
    assert sel(ctypes.byref(g), 4, FAKE, FAKE, 16, 0, FAKE, None, None, 0, None) == WORKSPACE
    assert "workspace" in last_error()


def test_pooled_workspace():
    g = geom(n_frames=256)
    nq = 256 * 101
    # bf16: the pooled queries in bf16, the per-block outputs, and the dense
    # staging over the 25,600 pooled keys (V^T, key-norm partials, one redo flag
    # per 256-query workgroup)
    blk = r256(nq * 16 * 64 * 2)
    flash = r256(16 * 64 * 25600 * 2 + 16 * 256 * 4 + r256(-(-nq // 256) * 16))
    assert _ws(g, 5, 0, 0) == (OK, 2 * blk + flash)
    # fp32: the per-block outputs only
    assert _ws(geom(n_frames=3, dtype=1), 5, 0, 0) == (OK, r256(3 * 101 * 16 * 64 * 4))
    assert _ws(g, 5, 1, 0)[0] == INVALID
    L = library()
    assert L.gsa_compressed_pooled(ctypes.byref(g), 4, FAKE, FAKE, FAKE, FAKE, None, 0, None) == WORKSPACE
    assert "workspace" in last_error()
    assert L.gsa_compressed_pooled(ctypes.byref(g), 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                   None) == UNSUPPORTED
    assert L.gsa_compressed_pooled(ctypes.byref(g), 4, None, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                   None) == INVALID


def test_python_layer_requires_gpu_tensors():
    import torch
    from synth import Geometry
    gm = Geometry(1, 0, 4, 4, 1, 64, "f32")
    x = torch.zeros((16, 1, 64))
    with pytest.raises(ValueError, match="GPU tensor"):
        sga.dense_global_attn(x, x, x, gm)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every call raises; nothing falls back to a
    CPU path."""
    import sparse_attention_global_amd._lib as lib_mod
    monkeypatch.setattr(lib_mod, "_lib", None)
    monkeypatch.setattr(lib_mod, "_LIB_PATH", str(tmp_path / "libsga.so"))
    with pytest.raises(RuntimeError, match="is not built"):
        lib_mod.library()


def test_workspace_size_sweep():
    """Every workspace query over a sweep of geometries, from one token to
    about 2^31 tokens: each returns OK or a validation status, never a size
    that shrinks when the frame count grows (the host layout arithmetic is
    checked for overflow by the sanitizer build of this file's tests)."""
    cases = []
    for n_frames in (1, 2, 7, 1000, 100_000, 1_000_000):
        for (gh, gw, S) in ((1, 1, 0), (37, 37, 5), (9, 13, 16)):
            for H in (1, 16):
                for dt in (0, 1):
                    cases.append(geom(n_frames=n_frames, grid_h=gh, grid_w=gw, n_special=S, n_heads=H,
                                      dtype=dt))
    ops = [(2, 0, 0), (2, 0, 1), (2, 100, 0), (1, 4, 4), (1, 1, 1), (1, 9, 9), (3, 1, 0), (3, 3, 0),
           (4, 1, 0), (4, 16, 0), (4, 17, 0), (4, 128, 2), (5, 0, 0), (6, 16, 0), (6, 4, 2)]
    last = {}
    for g in cases:
        for op in ops:
            st, n = _ws(g, *op)
            assert st in (OK, INVALID, UNSUPPORTED), (op, st)
            if st == OK:
                key = (g.grid_h, g.grid_w, g.n_special, g.n_heads, g.dtype, op)
                assert n >= last.get(key, 0), (key, n)
                last[key] = n
