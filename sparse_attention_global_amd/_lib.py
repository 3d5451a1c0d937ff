"""ctypes binding of libsga.so (include/sga.h): argument marshalling only.

Every step of the layer runs in the HIP library; these wrappers check torch
tensors against the geometry, allocate outputs with torch on the tensors'
device, pass raw device pointers and the current HIP stream, and raise
RuntimeError with the library's message on any non-OK status. There is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# The in-tree build; SGA_LIBRARY names another build of the same sources (the
# host-sanitizer build the ABI tests load).
_LIB_PATH = os.environ.get("SGA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libsga.so")
_lib = None

SGA_BF16, SGA_F32 = 0, 1
SGA_OP_SUBSAMPLED = 1
SGA_OP_DENSE = 2
SGA_OP_FINE = 3
SGA_OP_TOPK = 4
SGA_OP_POOLED = 5
SGA_OP_TOPK_PROB = 6
SGA_KEEP_SPECIAL = 1
SGA_KEEP_REF_FRAME = 2

EXPORTS = ("dense_global_attn", "gsa_compress", "gsa_compressed_pooled", "gsa_select_topk",
           "gsa_select_topk_noalloc",
           "gsa_select_topk_probability",
           "gsa_sparse_attn", "gsa_sparse_attn_gated", "gsa_gate",
           "sga_compact", "subsampled_global_attn", "sga_workspace_size", "sga_last_error",
           "sga_version")


class SgaGeom(ctypes.Structure):
    _fields_ = [("n_frames", ctypes.c_int32), ("n_special", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


def library() -> ctypes.CDLL:
    """Load libsga.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run python -m sparse_attention_global_amd.build")
    L = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    G = ctypes.POINTER(SgaGeom)
    sig = {
        "dense_global_attn": [G, P, P, P, I64, I32, P, P, P, SZ, P],
        "gsa_compress": [G, I32, I32, P, P, P, P, P, P, P, P],
        "gsa_compressed_pooled": [G, I32, P, P, P, P, P, SZ, P],
        "gsa_select_topk": [G, I32, P, P, I32, I32, P, P, P, SZ, P],
        "gsa_select_topk_noalloc": [G, I32, P, P, I32, I32, P, P, P],
        "gsa_select_topk_probability": [G, I32, P, P, I32, I32, P, P, P, SZ, P],
        "gsa_sparse_attn": [G, I32, P, P, P, P, I32, I32, P, P, P, SZ, P],
        "gsa_sparse_attn_gated": [G, I32, P, P, P, P, I32, I32, P, P, P, P, P, SZ, P],
        "gsa_gate": [G, P, P, P, P, P, P, P],
        "sga_compact": [G, I32, I32, P, P, P, P, P],
        "subsampled_global_attn": [G, I32, I32, I32, I32, P, P, P, P, P, SZ, P],
        "sga_workspace_size": [G, I32, I32, I32, ctypes.POINTER(SZ)],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.sga_last_error.argtypes = []
    L.sga_last_error.restype = ctypes.c_char_p
    L.sga_version.argtypes = []
    L.sga_version.restype = ctypes.c_int32
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = library().sga_last_error().decode(errors="replace")
        raise RuntimeError(f"{what} failed (status {status}): {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SGA_BF16
    if t.dtype == torch.float32:
        return SGA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32 expected")


def make_geom(geom, dtype_code: int) -> SgaGeom:
    return SgaGeom(geom.n_frames, geom.n_special, geom.grid_h, geom.grid_w, geom.n_heads,
                   getattr(geom, "head_dim", 64), dtype_code)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, rows: int, H: int, d: int, dtype=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != (rows, H, d):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(rows, H, d)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def tokens(geom) -> int:
    return geom.n_frames * (geom.n_special + geom.grid_h * geom.grid_w)


def pooled_shape(geom, block: int = 4):
    nb = (-(-geom.grid_h // block)) * (-(-geom.grid_w // block))
    return nb, nb + (1 if geom.n_special else 0)


# ---------------------------------------------------------------------------

def dense_workspace_bytes(geom, dtype_code: int, n_keys: int = 0, frame_local: bool = False) -> int:
    n = ctypes.c_size_t(0)
    g = make_geom(geom, dtype_code)
    _check(library().sga_workspace_size(ctypes.byref(g), SGA_OP_DENSE, n_keys, int(frame_local),
                                        ctypes.byref(n)), "sga_workspace_size")
    return n.value


def _workspace(nbytes: int, device, ws=None):
    if nbytes == 0:
        return ws
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace of {nbytes} bytes needed")
    return ws


def dense_global_attn(q, k, v, geom, n_keys: int = 0, frame_local: bool = False,
                      want_lse: bool = False, ws=None):
    """Dense (or frame-local, or pooled-key) attention; see include/sga.h."""
    T, H, d = tokens(geom), geom.n_heads, 64
    _need(q, "q", T, H, d)
    nk = T if n_keys == 0 else n_keys
    _need(k, "k", nk, H, d, q.dtype)
    _need(v, "v", nk, H, d, q.dtype)
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if want_lse else None
    code = _dtype_code(q)
    ws = _workspace(dense_workspace_bytes(geom, code, n_keys, frame_local), q.device, ws)
    g = make_geom(geom, code)
    _check(library().dense_global_attn(ctypes.byref(g), _ptr(q), _ptr(k), _ptr(v), n_keys,
                                       int(frame_local), _ptr(o), _ptr(lse), _ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(),
                                       _stream(q)), "dense_global_attn")
    return (o, lse) if want_lse else o


def gsa_compress(q, k, v, geom, block: int = 4, want_f32: bool = True, include_pad: bool = False):
    """Pooled K/V (+ fp32 pooled K and pooled queries); ``include_pad`` pools
    the zero-padded grid; see include/sga.h."""
    T, H, d = tokens(geom), geom.n_heads, 64
    nb, nqb = pooled_shape(geom, block)
    _need(k, "k", T, H, d)
    _need(v, "v", T, H, d, k.dtype)
    if q is not None:
        _need(q, "q", T, H, d, k.dtype)
    N = geom.n_frames
    k_cmp = torch.empty((N * nb, H, d), dtype=k.dtype, device=k.device)
    v_cmp = torch.empty_like(k_cmp)
    k32 = torch.empty((N * nb, H, d), dtype=torch.float32, device=k.device) if want_f32 else None
    q32 = (torch.empty((N * nqb, H, d), dtype=torch.float32, device=k.device)
           if (want_f32 and q is not None) else None)
    g = make_geom(geom, _dtype_code(k))
    _check(library().gsa_compress(ctypes.byref(g), block, int(include_pad), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(k_cmp),
                                  _ptr(v_cmp), _ptr(k32), _ptr(q32), _stream(k)), "gsa_compress")
    return k_cmp, v_cmp, k32, q32


def pooled_workspace_bytes(geom, dtype_code: int) -> int:
    n = ctypes.c_size_t(0)
    g = make_geom(geom, dtype_code)
    _check(library().sga_workspace_size(ctypes.byref(g), SGA_OP_POOLED, 0, 0, ctypes.byref(n)),
           "sga_workspace_size")
    return n.value


def gsa_compressed_pooled(q_blk_f32, k_cmp, v_cmp, geom, block: int = 4, ws=None):
    """Block-level compressed branch: each block's mean query over the pooled
    keys, upsampled to its tokens; see include/sga.h."""
    T, H, d, N = tokens(geom), geom.n_heads, 64, geom.n_frames
    nb, nqb = pooled_shape(geom, block)
    _need(q_blk_f32, "q_blk_f32", N * nqb, H, d, torch.float32)
    _need(k_cmp, "k_cmp", N * nb, H, d)
    _need(v_cmp, "v_cmp", N * nb, H, d, k_cmp.dtype)
    o = torch.empty((T, H, d), dtype=k_cmp.dtype, device=k_cmp.device)
    code = _dtype_code(k_cmp)
    g = make_geom(geom, code)
    ws = _workspace(pooled_workspace_bytes(geom, code), k_cmp.device, ws)
    _check(library().gsa_compressed_pooled(ctypes.byref(g), block, _ptr(q_blk_f32), _ptr(k_cmp),
                                           _ptr(v_cmp), _ptr(o), _ptr(ws),
                                           0 if ws is None else ws.numel() * ws.element_size(),
                                           _stream(k_cmp)), "gsa_compressed_pooled")
    return o


def keep_flags(keep_special: bool = True, keep_ref: bool = False) -> int:
    """The SGA_KEEP_* flags: the special tokens and/or the reference frame 0."""
    return (SGA_KEEP_SPECIAL if keep_special else 0) | (SGA_KEEP_REF_FRAME if keep_ref else 0)


def topk_workspace_bytes(geom, top_k: int, dtype_code: int = SGA_BF16, keep_ref: bool = False) -> int:
    n = ctypes.c_size_t(0)
    g = make_geom(geom, dtype_code)
    _check(library().sga_workspace_size(ctypes.byref(g), SGA_OP_TOPK, top_k,
                                        keep_flags(False, keep_ref), ctypes.byref(n)),
           "sga_workspace_size")
    return n.value


def gsa_select_topk(q_blk_f32, k_cmp_f32, geom, top_k: int, block: int = 4,
                    want_score: bool = False, dtype_code: int = SGA_BF16, keep_ref: bool = False,
                    ws=None):
    """Top-K pooled blocks per (head, query block), ascending; with ``keep_ref``
    frame 0's blocks do not compete (it is kept whole); see include/sga.h."""
    H, d, N = geom.n_heads, 64, geom.n_frames
    nb, nqb = pooled_shape(geom, block)
    _need(q_blk_f32, "q_blk_f32", N * nqb, H, d, torch.float32)
    _need(k_cmp_f32, "k_cmp_f32", N * nb, H, d, torch.float32)
    idx = torch.empty((H, N * nqb, top_k), dtype=torch.int32, device=q_blk_f32.device)
    score = torch.empty((H, N * nqb, top_k), dtype=torch.float32,
                        device=q_blk_f32.device) if want_score else None
    g = make_geom(geom, dtype_code)
    ws = _workspace(topk_workspace_bytes(geom, top_k, dtype_code, keep_ref), q_blk_f32.device, ws)
    _check(library().gsa_select_topk(ctypes.byref(g), block, _ptr(q_blk_f32), _ptr(k_cmp_f32),
                                     top_k, keep_flags(False, keep_ref), _ptr(idx), _ptr(score),
                                     _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(q_blk_f32)),
           "gsa_select_topk")
    return (idx, score) if want_score else idx


def gsa_select_topk_noalloc(q_blk_f32, k_cmp_f32, geom, top_k: int, block: int = 4,
                            want_score: bool = False, dtype_code: int = SGA_BF16, keep_ref: bool = False):
    """gsa_select_topk on the library's own per-GPU scratch (no workspace; the
    outputs are still allocated here); see include/sga.h."""
    H, d, N = geom.n_heads, 64, geom.n_frames
    nb, nqb = pooled_shape(geom, block)
    _need(q_blk_f32, "q_blk_f32", N * nqb, H, d, torch.float32)
    _need(k_cmp_f32, "k_cmp_f32", N * nb, H, d, torch.float32)
    idx = torch.empty((H, N * nqb, top_k), dtype=torch.int32, device=q_blk_f32.device)
    score = torch.empty((H, N * nqb, top_k), dtype=torch.float32,
                        device=q_blk_f32.device) if want_score else None
    g = make_geom(geom, dtype_code)
    _check(library().gsa_select_topk_noalloc(ctypes.byref(g), block, _ptr(q_blk_f32), _ptr(k_cmp_f32), top_k,
                                             keep_flags(False, keep_ref), _ptr(idx), _ptr(score),
                                             _stream(q_blk_f32)),
           "gsa_select_topk_noalloc")
    return (idx, score) if want_score else idx


def fine_workspace_bytes(geom, dtype_code: int, keep_special: bool = True,
                         keep_ref: bool = False) -> int:
    n = ctypes.c_size_t(0)
    g = make_geom(geom, dtype_code)
    _check(library().sga_workspace_size(ctypes.byref(g), SGA_OP_FINE,
                                        keep_flags(keep_special, keep_ref), 0,
                                        ctypes.byref(n)), "sga_workspace_size")
    return n.value


def topk_prob_workspace_bytes(geom, top_k: int, keep_ref: bool = False) -> int:
    n = ctypes.c_size_t(0)
    g = make_geom(geom, SGA_BF16)
    _check(library().sga_workspace_size(ctypes.byref(g), SGA_OP_TOPK_PROB, top_k,
                                        keep_flags(False, keep_ref), ctypes.byref(n)),
           "sga_workspace_size")
    return n.value


def gsa_select_topk_probability(q, k_cmp_f32, geom, top_k: int, block: int = 4, want_score: bool = False,
                                keep_ref: bool = False, ws=None):
    """Top-K pooled blocks per (head, query block) by the mean over the block's
    tokens of their compressed softmax probabilities (bf16 q, top_k <= 16);
    see include/sga.h."""
    T, H, d, N = tokens(geom), geom.n_heads, 64, geom.n_frames
    nb, nqb = pooled_shape(geom, block)
    _need(q, "q", T, H, d, torch.bfloat16)
    _need(k_cmp_f32, "k_cmp_f32", N * nb, H, d, torch.float32)
    idx = torch.empty((H, N * nqb, top_k), dtype=torch.int32, device=q.device)
    score = torch.empty((H, N * nqb, top_k), dtype=torch.float32, device=q.device) if want_score else None
    g = make_geom(geom, SGA_BF16)
    ws = _workspace(topk_prob_workspace_bytes(geom, top_k, keep_ref), q.device, ws)
    _check(library().gsa_select_topk_probability(ctypes.byref(g), block, _ptr(q), _ptr(k_cmp_f32), top_k,
                                                 keep_flags(False, keep_ref), _ptr(idx), _ptr(score),
                                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(q)),
           "gsa_select_topk_probability")
    return (idx, score) if want_score else idx


def gsa_sparse_attn(q, k, v, idx, geom, top_k: int, keep_special: bool = True, block: int = 4,
                    want_lse: bool = False, ws=None, keep_ref: bool = False):
    """Fine attention over the selected blocks (+ all special tokens, + frame 0
    whole with ``keep_ref``); see include/sga.h."""
    T, H, d, N = tokens(geom), geom.n_heads, 64, geom.n_frames
    nb, nqb = pooled_shape(geom, block)
    _need(q, "q", T, H, d)
    _need(k, "k", T, H, d, q.dtype)
    _need(v, "v", T, H, d, q.dtype)
    if tuple(idx.shape) != (H, N * nqb, top_k) or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError(f"idx must be a contiguous int32 tensor of shape {(H, N * nqb, top_k)}")
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if want_lse else None
    code = _dtype_code(q)
    g = make_geom(geom, code)
    ws = _workspace(fine_workspace_bytes(geom, code, keep_special, keep_ref), q.device, ws)
    _check(library().gsa_sparse_attn(ctypes.byref(g), block, _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                     top_k, keep_flags(keep_special, keep_ref), _ptr(o), _ptr(lse),
                                     _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(q)),
           "gsa_sparse_attn")
    return (o, lse) if want_lse else o


def gsa_sparse_attn_gated(q, k, v, idx, o_cmp, w_gate, b_gate, geom, top_k: int,
                          keep_special: bool = True, block: int = 4, ws=None, keep_ref: bool = False):
    """Fine attention with the gated aggregation folded into its epilogue: the
    layer output from the compressed branch's o_cmp; see include/sga.h."""
    T, H, d, N = tokens(geom), geom.n_heads, 64, geom.n_frames
    nb, nqb = pooled_shape(geom, block)
    for name, t in (("q", q), ("k", k), ("v", v), ("o_cmp", o_cmp)):
        _need(t, name, T, H, d, q.dtype)
    if tuple(idx.shape) != (H, N * nqb, top_k) or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError(f"idx must be a contiguous int32 tensor of shape {(H, N * nqb, top_k)}")
    if tuple(w_gate.shape) != (H, 2, d) or w_gate.dtype != torch.float32 or not w_gate.is_contiguous():
        raise ValueError(f"w_gate must be a contiguous float32 tensor of shape {(H, 2, d)}")
    if tuple(b_gate.shape) != (H, 2) or b_gate.dtype != torch.float32 or not b_gate.is_contiguous():
        raise ValueError(f"b_gate must be a contiguous float32 tensor of shape {(H, 2)}")
    o = torch.empty_like(q)
    code = _dtype_code(q)
    g = make_geom(geom, code)
    ws = _workspace(fine_workspace_bytes(geom, code, keep_special, keep_ref), q.device, ws)
    _check(library().gsa_sparse_attn_gated(ctypes.byref(g), block, _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                           top_k, keep_flags(keep_special, keep_ref), _ptr(o_cmp),
                                           _ptr(w_gate), _ptr(b_gate), _ptr(o), _ptr(ws),
                                           0 if ws is None else ws.numel() * ws.element_size(),
                                           _stream(q)),
           "gsa_sparse_attn_gated")
    return o


def gsa_gate(q, o_cmp, o_slc, w_gate, b_gate, geom, out=None):
    """Sigmoid-gated mix of the two GSA branches; see include/sga.h."""
    T, H, d = tokens(geom), geom.n_heads, 64
    for name, t in (("q", q), ("o_cmp", o_cmp), ("o_slc", o_slc)):
        _need(t, name, T, H, d, q.dtype)
    if tuple(w_gate.shape) != (H, 2, d) or w_gate.dtype != torch.float32:
        raise ValueError(f"w_gate must be fp32 of shape {(H, 2, d)}")
    if tuple(b_gate.shape) != (H, 2) or b_gate.dtype != torch.float32:
        raise ValueError(f"b_gate must be fp32 of shape {(H, 2)}")
    w_gate, b_gate = w_gate.contiguous(), b_gate.contiguous()
    o = torch.empty_like(q) if out is None else out
    g = make_geom(geom, _dtype_code(q))
    _check(library().gsa_gate(ctypes.byref(g), _ptr(q), _ptr(o_cmp), _ptr(o_slc), _ptr(w_gate),
                              _ptr(b_gate), _ptr(o), _stream(q)), "gsa_gate")
    return o


def compact_rows(geom, s_h: int, s_w: int):
    """(kept rows per frame, has_mean) of the subsampled compacted set."""
    kh, kw = -(-geom.grid_h // s_h), -(-geom.grid_w // s_w)
    mk = geom.n_special + kh * kw
    return mk, (1 if geom.grid_h * geom.grid_w > kh * kw else 0)


def sga_compact(k, v, geom, s_h: int, s_w: int):
    """The AVGGT compacted K/V set (kept part, then mean rows); see include/sga.h."""
    T, H, d, N = tokens(geom), geom.n_heads, 64, geom.n_frames
    _need(k, "k", T, H, d)
    _need(v, "v", T, H, d, k.dtype)
    mk, has_mean = compact_rows(geom, s_h, s_w)
    rows = N * (mk + has_mean)
    c_k = torch.empty((rows, H, d), dtype=k.dtype, device=k.device)
    c_v = torch.empty_like(c_k)
    g = make_geom(geom, _dtype_code(k))
    _check(library().sga_compact(ctypes.byref(g), s_h, s_w, _ptr(k), _ptr(v), _ptr(c_k), _ptr(c_v),
                                 _stream(k)), "sga_compact")
    return c_k, c_v


def workspace_bytes(geom, s_h: int, s_w: int, dtype_code: int) -> int:
    n = ctypes.c_size_t(0)
    g = make_geom(geom, dtype_code)
    _check(library().sga_workspace_size(ctypes.byref(g), SGA_OP_SUBSAMPLED, s_h, s_w,
                                        ctypes.byref(n)), "sga_workspace_size")
    return n.value


def subsampled_global_attn(q, k, v, geom, s_h: int, s_w: int, mode: int = 0,
                           mean_log_count: bool = False, ws=None):
    """AVGGT subsampled attention (mode 0), frame attention (mode 1) or the
    token-level diagonal (mode 2); see include/sga.h."""
    T, H, d = tokens(geom), geom.n_heads, 64
    _need(q, "q", T, H, d)
    _need(k, "k", T, H, d, q.dtype)
    _need(v, "v", T, H, d, q.dtype)
    code = _dtype_code(q)
    nbytes = workspace_bytes(geom, max(s_h, 1), max(s_w, 1), code)
    ws = _workspace(nbytes, q.device, ws)
    o = torch.empty_like(q)
    g = make_geom(geom, code)
    _check(library().subsampled_global_attn(ctypes.byref(g), s_h, s_w, mode, int(mean_log_count),
                                            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(ws),
                                            0 if ws is None else ws.numel() * ws.element_size(),
                                            _stream(q)), "subsampled_global_attn")
    return o


def gsa_layer(q, k, v, w_gate, b_gate, geom, top_k: int, block: int = 4,
              keep_special: bool = True, keep_intermediates: bool = False, keep_ref: bool = False,
              pooled_q: bool = False, include_pad: bool = False, probability_scores: bool = False):
    """The Global Sparse Attention layer: compress, compressed attention,
    select, then fine attention with the gate folded into its epilogue (with
    ``keep_intermediates``, fine attention and the gate as separate calls, so
    that the fine branch's output is kept too). ``keep_ref`` is the VGGT
    adaptation: frame 0 kept whole by the fine branch; ``pooled_q`` the
    block-level compressed branch (pooled queries, upsampled); ``include_pad``
    the zero-padded pooling; ``probability_scores`` selects by the mean of the
    block's tokens' compressed probabilities instead of their mean logit."""
    N = geom.n_frames
    nb, _ = pooled_shape(geom, block)
    k_cmp, v_cmp, k32, q32 = gsa_compress(q, k, v, geom, block, include_pad=include_pad)
    if pooled_q:
        o_cmp = gsa_compressed_pooled(q32, k_cmp, v_cmp, geom, block)
    else:
        o_cmp = dense_global_attn(q, k_cmp, v_cmp, geom, n_keys=N * nb)
    if probability_scores:
        idx = gsa_select_topk_probability(q, k32, geom, top_k, block, keep_ref=keep_ref)
    else:
        idx = gsa_select_topk(q32, k32, geom, top_k, block, dtype_code=_dtype_code(q), keep_ref=keep_ref)
    if not keep_intermediates:
        return gsa_sparse_attn_gated(q, k, v, idx, o_cmp, w_gate, b_gate, geom, top_k, keep_special, block,
                                     keep_ref=keep_ref)
    o_slc = gsa_sparse_attn(q, k, v, idx, geom, top_k, keep_special, block, keep_ref=keep_ref)
    o = gsa_gate(q, o_cmp, o_slc, w_gate, b_gate, geom)
    return {"k_cmp": k_cmp, "v_cmp": v_cmp, "k_cmp_f32": k32, "q_blk_f32": q32,
            "o_cmp": o_cmp, "idx": idx, "o_slc": o_slc, "o": o}
