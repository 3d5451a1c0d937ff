"""Seeded synthetic inputs for the global cross-frame attention layer.

This module is shared by the tests, the benchmark and the CPU checker. It
holds the workload table and the random-number recipes only: no attention,
pooling, selection, gating or subsampling arithmetic lives here.

Token layout of every ``[T, H, d]`` tensor (T = N * L): frame-major; inside a
frame the ``n_special`` special tokens come first (0 = camera, then the
register tokens), followed by the patch tokens of the ``grid_h x grid_w``
patch grid in row-major order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["Geometry", "Workload", "WORKLOADS", "make_qkv", "make_gate",
           "sample_rows", "to_host_f64"]


@dataclasses.dataclass(frozen=True)
class Geometry:
    n_frames: int
    n_special: int
    grid_h: int
    grid_w: int
    n_heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"

    @property
    def tokens_per_frame(self) -> int:
        return self.n_special + self.grid_h * self.grid_w

    @property
    def n_tokens(self) -> int:
        return self.n_frames * self.tokens_per_frame

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Geometry":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    geom: Geometry
    distribution: str          # "normal" (i.i.d. N(0,1)) or "scene" (low-rank shared)
    top_k: int                 # fine blocks selected per query block
    block: int                 # pooling window side
    stride: tuple              # (s_h, s_w) of the subsampled form
    check_rows: Optional[int]  # None: every row is checked; else a seeded sample


WORKLOADS: Dict[str, Workload] = {
    # 4 frames x 16x16 patches, 1 head, d=64, fp32, Q/K/V ~ N(0,1).
    "tiny": Workload("tiny", Geometry(4, 0, 16, 16, 1, 64, "f32"), "normal",
                     top_k=4, block=4, stride=(2, 2), check_rows=None),
    # 32 frames x (37x37 patches + camera + 4 registers), 16 heads, bf16.
    "dense32": Workload("dense32", Geometry(32, 5, 37, 37, 16, 64, "bf16"), "scene",
                        top_k=16, block=4, stride=(4, 4), check_rows=4096),
    "gsa128": Workload("gsa128", Geometry(128, 5, 37, 37, 16, 64, "bf16"), "scene",
                       top_k=16, block=4, stride=(4, 4), check_rows=4096),
    "sga256": Workload("sga256", Geometry(256, 5, 37, 37, 16, 64, "bf16"), "scene",
                       top_k=16, block=4, stride=(4, 4), check_rows=4096),
    # 1000 frames: 1,374,000 tokens.
    "scene1000": Workload("scene1000", Geometry(1000, 5, 37, 37, 16, 64, "bf16"), "scene",
                          top_k=16, block=4, stride=(4, 4), check_rows=4096),
}

_TENSOR_ID = {"q": 1, "k": 2, "v": 3, "scene": 4, "offsets": 5, "special": 6,
              "basis_qk": 7, "basis_v": 8, "gate_w": 9, "gate_b": 10, "rows": 11}


def _gen(seed: int, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + _TENSOR_ID[tensor] * 7919) & 0x7FFF_FFFF_FFFF)
    return g


def make_qkv(geom: Geometry, seed: int, device="cpu", distribution: str = "normal",
             rank: int = 8):
    """Return seeded Q, K, V of shape [T, H, d] in ``geom.dtype`` on ``device``.

    ``normal``: i.i.d. N(0, 1) entries.
    ``scene``:  X = E / sqrt(d) + U @ B_X with E ~ N(0, 1). U is a rank-``rank``
    code per token: patch (r, c) of frame f reads a scene code F[r + dy_f, c + dx_f]
    shared by all frames (a seeded per-frame offset into a 2gh x 2gw code map),
    special tokens draw an independent N(0, I) code. B_Q = B_K ~ N(0,1)/sqrt(d)
    (so co-visible patches get positive logits), B_V is drawn independently.
    Values are produced in fp32 and rounded once (round-to-nearest-even) to bf16.
    """
    T, H, d = geom.n_tokens, geom.n_heads, geom.head_dim
    N, S, gh, gw = geom.n_frames, geom.n_special, geom.grid_h, geom.grid_w
    out = []
    if distribution == "normal":
        for name in ("q", "k", "v"):
            x = torch.randn((T, H, d), generator=_gen(seed, name, device), device=device,
                            dtype=torch.float32)
            out.append(x.to(geom.torch_dtype))
        return tuple(out)
    if distribution != "scene":
        raise ValueError(f"unknown distribution {distribution!r}")
    code = torch.randn((2 * gh, 2 * gw, rank), generator=_gen(seed, "scene", device),
                       device=device)
    offs = torch.randint(0, max(gh, gw), (N, 2), generator=_gen(seed, "offsets", device),
                         device=device)
    dy = offs[:, 0] % gh
    dx = offs[:, 1] % gw
    rr = torch.arange(gh, device=device)
    cc = torch.arange(gw, device=device)
    # patch codes: [N, gh, gw, rank]
    pr = (rr[None, :] + dy[:, None])  # [N, gh]
    pc = (cc[None, :] + dx[:, None])  # [N, gw]
    u_patch = code[pr[:, :, None], pc[:, None, :]]
    u_spec = torch.randn((N, S, rank), generator=_gen(seed, "special", device), device=device)
    u = torch.cat([u_spec, u_patch.reshape(N, gh * gw, rank)], dim=1).reshape(T, rank)
    b_qk = torch.randn((H, rank, d), generator=_gen(seed, "basis_qk", device),
                       device=device) / math.sqrt(d)
    b_v = torch.randn((H, rank, d), generator=_gen(seed, "basis_v", device),
                      device=device) / math.sqrt(d)
    for name, basis in (("q", b_qk), ("k", b_qk), ("v", b_v)):
        x = torch.randn((T, H, d), generator=_gen(seed, name, device), device=device,
                        dtype=torch.float32)
        x.mul_(1.0 / math.sqrt(d))
        # [T, rank] x [H, rank, d] -> [T, H, d], one head at a time to bound memory
        for h in range(H):
            x[:, h, :].add_(u @ basis[h])
        out.append(x.to(geom.torch_dtype))
        del x
    return tuple(out)


def make_gate(n_heads: int, head_dim: int, seed: int, device="cpu"):
    """Gate weights W [H, 2, d] and bias b [H, 2], fp32, ~ U(-1/8, 1/8)."""
    w = (torch.rand((n_heads, 2, head_dim), generator=_gen(seed, "gate_w", device),
                    device=device) - 0.5) / 4.0
    b = (torch.rand((n_heads, 2), generator=_gen(seed, "gate_b", device),
                    device=device) - 0.5) / 4.0
    return w.float(), b.float()


def sample_rows(n_tokens: int, count: Optional[int], seed: int):
    """Sorted seeded sample of query rows (all rows if ``count`` is None or >= T)."""
    if count is None or count >= n_tokens:
        return torch.arange(n_tokens)
    g = _gen(seed, "rows", "cpu")
    return torch.randperm(n_tokens, generator=g)[:count].sort().values


def to_host_f64(x: torch.Tensor):
    """Exact widening of a tensor's values to a host fp64 NumPy array."""
    return x.detach().to("cpu").to(torch.float64).numpy()
