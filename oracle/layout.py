"""Oracle token orders: frame-major raster and 3-D cuboid tiling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The SPADE explainer's blueprint part ("Der Bauplan (vDiT-SSR)") describes the
video's blocks as cells of a 3-D (time, height, width) grid that may be cut
into flat, tall or mixed shapes, rather than the one cut earlier methods use.
It gives no storage rule.  The reading implemented here, for a cuboid shape
(ct, ch, cw) with ct * ch * cw equal to the block size:

  The grid (T, H, W) is covered by the cuboid grid (ceil(T/ct), ceil(H/ch),
  ceil(W/cw)); cuboid (a, b, c) holds the tokens with a*ct <= t < (a+1)*ct,
  b*ch <= y < (b+1)*ch, c*cw <= x < (c+1)*cw that lie inside the grid.  A
  cuboid is full when it holds ct*ch*cw tokens, partial otherwise (it touches
  the far edge of an axis the cuboid does not divide).  Tokens are stored
  cuboid after cuboid: first every full cuboid in lexicographic (a, b, c)
  order, then every partial cuboid in lexicographic order; inside a cuboid in
  frame-major order (t, then y, then x).  Block j holds storage slots
  [j*block, (j+1)*block): every full cuboid is exactly one block, and the
  partial cuboids are packed, in order, into the last blocks.

``order[p]`` is the frame-major index t*H*W + y*W + x of the token stored at
slot p.  No cuboid (None or (0, 0, 0)) means the frame-major order itself.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def is_raster(cuboid: Optional[Sequence[int]]) -> bool:
    return cuboid is None or tuple(int(v) for v in cuboid) == (0, 0, 0)


def cuboid_order(T: int, H: int, W: int, cuboid: Optional[Sequence[int]]) -> np.ndarray:
    """Storage order, int64 [T*H*W]: frame-major index of the token at each slot."""
    N = T * H * W
    if is_raster(cuboid):
        return np.arange(N, dtype=np.int64)
    ct, ch, cw = (int(v) for v in cuboid)
    if min(ct, ch, cw) < 1:
        raise ValueError("cuboid extents must all be >= 1 (or all 0 for frame-major order)")
    full, partial = [], []
    for a in range(-(-T // ct)):
        ts = np.arange(a * ct, min(T, (a + 1) * ct))
        for b in range(-(-H // ch)):
            ys = np.arange(b * ch, min(H, (b + 1) * ch))
            for c in range(-(-W // cw)):
                xs = np.arange(c * cw, min(W, (c + 1) * cw))
                toks = (ts[:, None, None] * (H * W) + ys[None, :, None] * W
                        + xs[None, None, :]).reshape(-1)
                (full if toks.size == ct * ch * cw else partial).append(toks)
    order = np.concatenate(full + partial).astype(np.int64)
    assert order.size == N
    return order


def slot_coords(T: int, H: int, W: int, order: Optional[np.ndarray] = None):
    """(t, y, x) of the token stored at each slot, int64 [N] each."""
    n = np.arange(T * H * W, dtype=np.int64) if order is None else np.asarray(order, dtype=np.int64)
    return n // (H * W), (n // W) % H, n % W


def permute_tokens(x: np.ndarray, order: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Move the token axis (axis -2, length n_pad >= N) between frame-major and storage order.

    Forward: out[..., p, :] = x[..., order[p], :]; inverse: out[..., order[p], :] = x[..., p, :].
    Slots from N on (padding) are carried over unchanged.
    """
    N = order.size
    out = np.array(x, copy=True)
    if inverse:
        out[..., order, :] = x[..., :N, :]
    else:
        out[..., :N, :] = x[..., order, :]
    return out
