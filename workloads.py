"""Seeded synthetic inputs for head-major vision attention.

This module only draws random tensors; it holds none of the attention
arithmetic, and both the CPU oracle's tests and the GPU path's tests and
benchmark take their inputs from it.

Generator: ``numpy.random.default_rng(seed)`` (PCG64), float32 draws, drawn
in the fixed order Q, K, V, each of shape ``[n_heads][n_patches][head_dim]``,
C-contiguous.  Any caller-side pre-scaling of Q (the attention itself applies
no scale; the caller folds 1/sqrt(d) or any other factor into Q) is done here
in float32, before either side sees the data.

Workloads (vision patches: i.i.d. features, one head per image-head pair):

====  ======  ======  ========  ===================================================
id    H       N       d         distribution
====  ======  ======  ========  ===================================================
1     4       64      64        Q ~ N(0,1)/8, K, V ~ N(0,1)      (single tile)
2     16      256     64        same                              (small N)
3     16      1024    64        same
4     12      4097    32        Q ~ N(0,1)/sqrt(32), K, V ~ N(0,1) (ragged tails)
5     128     4096    64        Q, K ~ N(0, 3^2) unscaled, V ~ U(-1,1)
                                (16 heads x 8 images; sharp softmax)
6     128     4096    64        as 5, stored patch-major [N][H][d]
7     16      1024    40        Q ~ N(0,1)/sqrt(40), K, V ~ N(0,1) (head_dim 40)
8     16      1024    64        as 3, stored as f16
9     128     4096    64        as 5, stored as f16
10    16      1024    64        as 3, Q and K rotated (NeoX, rope_dims 64, base 1e4)
11    128     4096    64        as 5, Q and K rotated (NeoX, rope_dims 64, base 1e4)
====  ======  ======  ========  ===================================================

Workloads 1-5 are the head-major f32 [H][N][d] cases; 6 and 7 exercise the
strided (patch-major) access and a head_dim that is neither 32 nor 64; 8
and 9 the f16 tensors (the f32 draws rounded to f16, round-to-nearest-even;
both sides then see the same f16 values); 10 and 11 the rotary transform of
Q and K, patch n at position n (the drawn arrays are the unrotated inputs).
``make_inputs`` always returns head-major arrays; ``to_layout`` gives the
storage order a workload is run in.

The default seed of workload ``i`` is ``1000 + i``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    n_heads: int
    n_patches: int
    head_dim: int
    kind: str  # "normal" or "sharp"
    layout: str = "head"  # "head": [H][N][d]; "patch": [N][H][d]
    dtype: str = "f32"    # element type in HBM: "f32" or "f16"
    rope_dims: int = 0    # rotary dimensions of Q and K (0: none)
    rope_base: float = 10000.0

    @property
    def shape(self):
        return (self.n_heads, self.n_patches, self.head_dim)

    @property
    def flops(self) -> int:
        """Attention flop count 4*H*N^2*d (two N x N x d contractions)."""
        return 4 * self.n_heads * self.n_patches ** 2 * self.head_dim

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once and out written once: 4 * H*N*d elements (16 bytes
        per element quad for f32, 8 for f16)."""
        elem = 2 if self.dtype == "f16" else 4
        return 4 * elem * self.n_heads * self.n_patches * self.head_dim

    def describe(self) -> str:
        return "%s (H=%d, N=%d, d=%d)" % (self.name, self.n_heads,
                                          self.n_patches, self.head_dim)


WORKLOADS = {
    1: Workload(1, "vit_h4_n64_d64", 4, 64, 64, "normal"),
    2: Workload(2, "vit_h16_n256_d64", 16, 256, 64, "normal"),
    3: Workload(3, "vit_h16_n1024_d64", 16, 1024, 64, "normal"),
    4: Workload(4, "vit_ragged_h12_n4097_d32", 12, 4097, 32, "normal"),
    5: Workload(5, "vit_sharp_h128_n4096_d64", 128, 4096, 64, "sharp"),
    6: Workload(6, "vit_sharp_patchmajor_h128_n4096_d64", 128, 4096, 64, "sharp", "patch"),
    7: Workload(7, "vit_h16_n1024_d40", 16, 1024, 40, "normal"),
    8: Workload(8, "vit_f16_h16_n1024_d64", 16, 1024, 64, "normal", dtype="f16"),
    9: Workload(9, "vit_f16_sharp_h128_n4096_d64", 128, 4096, 64, "sharp", dtype="f16"),
    10: Workload(10, "vit_rope_h16_n1024_d64", 16, 1024, 64, "normal", rope_dims=64),
    11: Workload(11, "vit_rope_sharp_h128_n4096_d64", 128, 4096, 64, "sharp", rope_dims=64),
}


def to_layout(x, layout: str):
    """A head-major [H][N][d] array in the storage order ``layout`` names
    ("head": itself; "patch": a contiguous [N][H][d] copy)."""
    if layout == "head":
        return np.ascontiguousarray(x)
    if layout == "patch":
        return np.ascontiguousarray(np.transpose(x, (1, 0, 2)))
    raise ValueError("unknown layout %r" % layout)


def default_seed(wid: int) -> int:
    return 1000 + int(wid)


def make_inputs(wid: int, seed: int | None = None, n_heads: int | None = None):
    """Q, K, V arrays of workload ``wid`` (float32, or float16 for the f16
    workloads).

    ``n_heads`` (optional) draws only the first heads of the workload's
    stream shape-wise, i.e. a workload with fewer heads but the same
    per-head distribution (used for bounded CPU samples); it is not a prefix
    of the full draw.
    """
    w = WORKLOADS[wid]
    h = w.n_heads if n_heads is None else int(n_heads)
    q, k, v = make_custom(h, w.n_patches, w.head_dim, w.kind,
                          default_seed(wid) if seed is None else seed)
    if w.dtype == "f16":
        q, k, v = (x.astype(np.float16) for x in (q, k, v))
    return q, k, v


def make_custom(n_heads: int, n_patches: int, head_dim: int,
                kind: str = "normal", seed: int = 0):
    """Q, K, V of any shape with a workload's distribution.

    kind "normal": Q ~ N(0,1) * float32(1/sqrt(d)), K, V ~ N(0,1).
    kind "sharp":  Q, K ~ N(0,1) * 3, V ~ U(-1, 1).
    kind "unit":   Q, K, V ~ N(0,1), no pre-scaling.
    """
    rng = np.random.default_rng(seed)
    shape = (int(n_heads), int(n_patches), int(head_dim))
    if kind == "normal":
        qs = np.float32(1.0 / np.sqrt(head_dim))  # 1/8 exactly at d = 64
        q = rng.standard_normal(shape, dtype=np.float32) * qs
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
    elif kind == "sharp":
        three = np.float32(3.0)
        q = rng.standard_normal(shape, dtype=np.float32) * three
        k = rng.standard_normal(shape, dtype=np.float32) * three
        v = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    elif kind == "unit":
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
    else:
        raise ValueError("unknown kind %r" % kind)
    return (np.ascontiguousarray(q, dtype=np.float32),
            np.ascontiguousarray(k, dtype=np.float32),
            np.ascontiguousarray(v, dtype=np.float32))


def sample_rows(n_heads: int, n_patches: int, per_head: int, seed: int = 7):
    """Flat row ids h*N+i: the first, last and ``per_head`` random rows of
    every head (sorted, unique).  Used to check full-size outputs row by row."""
    rng = np.random.default_rng(seed)
    rows = []
    for h in range(n_heads):
        picks = {0, n_patches - 1}
        if n_patches > 2:
            picks.update(int(x) for x in rng.integers(0, n_patches, size=per_head))
        rows.extend(h * n_patches + i for i in sorted(picks))
    return np.array(rows, dtype=np.int64)
