"""Oracle block masks: static spatio-temporal window, pooled-score top-k and SICS.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say the method works with static sliding-window sparse attention and
with dynamic Top-K sparse attention ("SALAD" explainer, technical summary
section 5), name a spatio-temporal sliding window (ST-SWA) as the base sparse
model (sciencestack "SALAD", Figure 1), and describe sparse attention as "only
talk to your neighbours" (explainer, part 2 of the lay explanation).  They give
no rule for either mask.  The readings implemented here:

Window (per head: t_window Tw, r_max, density rho)
  Token n of the (T, H, W) grid, frame-major, sits at t = n // (H*W),
  y = (n // W) % H, x = n % W.  Block b holds tokens [b*block, (b+1)*block)
  that are < N.  For a query block q and key block k, r*(q, k) is the least
  Chebyshev spatial distance max(|y_i - y_j|, |x_i - x_j|) over token pairs
  i in q, j in k with |t_i - t_j| <= Tw; r* is infinite if no pair is that
  close in time.  Candidates are the pairs with finite r* (and r* <= r_max when
  r_max >= 0).  With rho <= 0 every candidate is kept.  Otherwise the candidates
  are ranked by the key (q != k, r*, |q - k|, q, k), ascending, and the first
  K = floor(rho * nbq * nbk + 0.5) are kept (rho taken as the float32 the
  C interface carries); K above the candidate count is infeasible.

Top-k (per head: density rho)
  pq[q, c] = (sum over the valid tokens of block q, in token order, of Q[n, c])
  / nvalid(q), every addition and the division rounded to float32 (a
  sequential float32 sum starting from +0); pk likewise from K.  The score of
  (q, k) is the float32 sum over c = 0..d-1, in order, of fl32(pq[q,c]*pk[k,c]),
  each product and each addition rounded separately (no fused multiply-add).
  Each query block keeps the k = max(1, floor(rho * nbk + 0.5)) key blocks with
  the highest scores, ties going to the lower key block.  The diagonal is not
  forced.  Fixing the float32 order of operations makes the ranking, and hence
  the CSR, exactly reproducible.

SICS (per head: density rho; the SPADE explainer's scheme generation, "Der
sofortige Entscheidungsträger": blocks whose tokens agree, measured by the sum
of intra-block cosine similarities, are the ones attention goes to)
  For key block b, SICS(b) = sum over token pairs i, j of b (valid tokens
  only) of cos(k_i, k_j) = || sum_i k_i / |k_i| ||^2, in a fixed float32
  order: |k_i|^2 = sequential float32 sum over c of fl32(k[i,c]^2); a zero
  vector contributes nothing, else khat[i,c] = fl32(k[i,c] / fl32(sqrt(|k_i|^2)))
  (correctly rounded square root and division); s[c] = sequential float32 sum
  over the block's tokens, in order, of khat[i,c]; SICS = sequential float32
  sum over c of fl32(s[c]^2).  No fused multiply-add anywhere.  Per (b, h) the
  m = max(1, floor(rho * nb + 0.5)) key blocks with the highest SICS are kept
  (ties to the lower key block) for every query block, and each query block
  also keeps its own (diagonal) block, so a row holds m or m + 1 blocks.  The
  pages give the score's name and purpose only; this plain reading scores key
  blocks and shares the selection across the query blocks of a head.

Gate from Q (the stand-in for the input-aware scale s of explainer section 2.2)
  g = sigmoid(mean over valid tokens of Q[b, h, n, :] . w_g), in fp64.

Output: CSR over rows r = (b*H + h)*nb + q, ``row_ptr`` int32 [B*H*nb + 1] and
``col_idx`` int32, ascending key blocks within each row.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

RSTAR_INF = 1 << 30

WINDOW = 0
TOPK = 1
SICS = 2


class InfeasibleMask(ValueError):
    """A window head asked for more block pairs than it has candidates."""


# ---------------------------------------------------------------- geometry

def _token_coords(T: int, H: int, W: int):
    n = np.arange(T * H * W, dtype=np.int64)
    return n // (H * W), (n // W) % H, n % W


def window_rstar_bruteforce(T: int, H: int, W: int, block: int, t_window: int,
                            qblocks: Optional[Sequence[int]] = None,
                            order: Optional[np.ndarray] = None) -> np.ndarray:
    """r*(q, k) by direct minimisation over every token pair (small grids, or a few rows).

    ``order`` (from ``layout.cuboid_order``) gives the token stored at each slot;
    None is the frame-major order.  Returns int64 [len(qblocks) or nb, nb];
    RSTAR_INF marks "no pair within Tw frames".
    """
    N = T * H * W
    nb = -(-N // block)
    n_pad = nb * block
    t, y, x = _token_coords(T, H, W)
    if order is not None:
        order = np.asarray(order, dtype=np.int64)
        t, y, x = t[order], y[order], x[order]
    # int32 coordinates, padded to n_pad with a frame far outside every window
    far = np.int32(-(4 * (T + H + W + t_window + 1)))
    tp = np.full(n_pad, far, dtype=np.int32)
    tp[:N] = t
    yp = np.zeros(n_pad, dtype=np.int32)
    yp[:N] = y
    xp = np.zeros(n_pad, dtype=np.int32)
    xp[:N] = x
    rows = range(nb) if qblocks is None else list(qblocks)
    out = np.full((len(rows), nb), RSTAR_INF, dtype=np.int64)
    for r, qb in enumerate(rows):
        i = np.arange(qb * block, min((qb + 1) * block, N))
        if i.size == 0:
            continue
        dt = np.abs(tp[i, None] - tp[None, :])
        dist = np.maximum(np.abs(yp[i, None] - yp[None, :]), np.abs(xp[i, None] - xp[None, :]))
        dist[dt > t_window] = RSTAR_INF
        out[r] = dist.reshape(i.size, nb, block).min(axis=(0, 2))
    return out


def _block_segments(T: int, H: int, W: int, block: int):
    """Each block as at most S horizontal runs (t, y, x0, x1), x1 inclusive."""
    N = T * H * W
    nb = -(-N // block)
    segs = []
    for b in range(nb):
        first = b * block
        last = min((b + 1) * block, N) - 1
        runs = []
        for row in range(first // W, last // W + 1):
            x0 = max(first, row * W) - row * W
            x1 = min(last, row * W + W - 1) - row * W
            runs.append((row // H, row % H, x0, x1))
        segs.append(runs)
    S = max(len(r) for r in segs)
    arr = np.zeros((4, nb, S), dtype=np.int64)
    valid = np.zeros((nb, S), dtype=bool)
    for b, runs in enumerate(segs):
        for s, run in enumerate(runs):
            arr[:, b, s] = run
            valid[b, s] = True
    return arr, valid


def window_rstar_segments(T: int, H: int, W: int, block: int, t_window: int) -> np.ndarray:
    """r*(q, k) for every block pair via the runs of each block.

    Between two runs the least Chebyshev distance is max(|y1 - y2|, gap), where gap
    is the distance between the x-intervals (0 if they overlap); r* is the least of
    that over run pairs at most Tw frames apart.  Tied to the token-level brute force
    by the CPU tests.
    """
    (st, sy, sx0, sx1), valid = _block_segments(T, H, W, block)
    nb, S = valid.shape
    best = np.full((nb, nb), RSTAR_INF, dtype=np.int64)
    for a in range(S):
        for c in range(S):
            ok = valid[:, a][:, None] & valid[:, c][None, :]
            ok &= np.abs(st[:, a][:, None] - st[:, c][None, :]) <= t_window
            gap = np.maximum(0, np.maximum(sx0[:, c][None, :] - sx1[:, a][:, None],
                                           sx0[:, a][:, None] - sx1[:, c][None, :]))
            d = np.maximum(np.abs(sy[:, a][:, None] - sy[:, c][None, :]), gap)
            best = np.where(ok, np.minimum(best, d), best)
    return best


# ---------------------------------------------------------------- window selection

def window_count(density: float, nbq: int, nbk: int) -> int:
    """K = floor(rho * nbq * nbk + 0.5), rho as float32 widened to double."""
    return int(math.floor(float(np.float32(density)) * nbq * nbk + 0.5))


def window_select(rstar: np.ndarray, r_max: int, density: float) -> np.ndarray:
    """Boolean keep[q, k] for one window head (see the module docstring)."""
    nbq, nbk = rstar.shape
    cand = rstar < RSTAR_INF
    if r_max >= 0:
        cand &= rstar <= r_max
    if density <= 0:
        return cand
    K = window_count(density, nbq, nbk)
    qb, kb = np.nonzero(cand)
    if K > qb.size:
        raise InfeasibleMask(f"window asks for {K} block pairs, only {qb.size} candidates")
    r = rstar[qb, kb]
    order = np.lexsort((kb, qb, np.abs(qb - kb), r, (qb != kb).astype(np.int64)))
    keep = np.zeros_like(cand)
    sel = order[:K]
    keep[qb[sel], kb[sel]] = True
    return keep


# ---------------------------------------------------------------- top-k selection

def pooled_means_f32(x: np.ndarray, N: int, block: int) -> np.ndarray:
    """Block means in the canonical float32 order: sequential sum from +0, then one division.

    x: float32 [B, H, n_pad, d] -> float32 [B, H, nb, d].
    """
    x = np.asarray(x, dtype=np.float32)
    B, Hh, n_pad, d = x.shape
    nb = n_pad // block
    xb = x.reshape(B, Hh, nb, block, d)
    nvalid = np.array([min(block, N - b * block) for b in range(nb)], dtype=np.float32)
    acc = np.zeros((B, Hh, nb, d), dtype=np.float32)
    last_valid = int(nvalid[-1])
    for o in range(block):
        if o < last_valid:
            acc = acc + xb[:, :, :, o, :]
        else:
            acc[:, :, :-1] = acc[:, :, :-1] + xb[:, :, :-1, o, :]
    return acc / nvalid[None, None, :, None]


def pooled_scores_f32(pq: np.ndarray, pk: np.ndarray) -> np.ndarray:
    """score[q, k] = sequential float32 sum over c of fl32(pq[q,c] * pk[k,c]); no FMA."""
    pq = np.asarray(pq, dtype=np.float32)
    pk = np.asarray(pk, dtype=np.float32)
    d = pq.shape[-1]
    acc = np.zeros(pq.shape[:-1] + (pk.shape[-2],), dtype=np.float32)
    for c in range(d):
        prod = pq[..., :, None, c] * pk[..., None, :, c]
        acc = acc + prod
    return acc


def topk_count(density: float, nbk: int) -> int:
    k = int(math.floor(float(np.float32(density)) * nbk + 0.5))
    return min(max(1, k), nbk)


def topk_select(scores: np.ndarray, density: float) -> np.ndarray:
    """keep[..., q, k]: the top-k scores of each row, ties to the lower key block."""
    nbk = scores.shape[-1]
    k = topk_count(density, nbk)
    order = np.argsort(-scores, axis=-1, kind="stable")[..., :k]
    keep = np.zeros(scores.shape, dtype=bool)
    np.put_along_axis(keep, order, True, axis=-1)
    return keep


# ---------------------------------------------------------------- SICS selection

def sics_block_scores_f32(k: np.ndarray, N: int, block: int) -> np.ndarray:
    """SICS of every key block in the canonical float32 order (module docstring).

    k: float32 [B, H, n_pad, d] -> float32 [B, H, nb].
    """
    k = np.asarray(k, dtype=np.float32)
    B, Hh, n_pad, d = k.shape
    nb = n_pad // block
    n2 = np.zeros((B, Hh, n_pad), dtype=np.float32)
    for c in range(d):
        n2 = n2 + k[..., c] * k[..., c]
    r = np.sqrt(n2)
    zero = n2 == 0
    safe_r = np.where(zero, np.float32(1), r)
    khat = np.where(zero[..., None], np.float32(0), k / safe_r[..., None]).astype(np.float32)
    kb = khat.reshape(B, Hh, nb, block, d)
    last_valid = N - (nb - 1) * block
    acc = np.zeros((B, Hh, nb, d), dtype=np.float32)
    for o in range(block):
        if o < last_valid:
            acc = acc + kb[:, :, :, o, :]
        else:
            acc[:, :, :-1] = acc[:, :, :-1] + kb[:, :, :-1, o, :]
    sics = np.zeros((B, Hh, nb), dtype=np.float32)
    for c in range(d):
        sics = sics + acc[..., c] * acc[..., c]
    return sics


def sics_select(scores: np.ndarray, density: float) -> np.ndarray:
    """keep[q, k] for one head: the top-m key blocks by SICS (ties to the lower block) plus the diagonal.

    scores: float32 [nb] -> bool [nb, nb].
    """
    nb = scores.shape[-1]
    m = topk_count(density, nb)
    top = np.zeros(nb, dtype=bool)
    top[np.argsort(-scores, kind="stable")[:m]] = True
    keep = np.repeat(top[None, :], nb, axis=0)
    keep[np.arange(nb), np.arange(nb)] = True
    return keep


# ---------------------------------------------------------------- gate

def gate_from_q(q: np.ndarray, w_g: np.ndarray, N: int) -> np.ndarray:
    """g[b*H + h] = sigmoid(mean_{n<N} Q[b,h,n,:] . w_g), fp64."""
    mean = np.asarray(q[:, :, :N], dtype=np.float64).mean(axis=2)
    logit = mean @ np.asarray(w_g, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-logit))).reshape(-1)


# ---------------------------------------------------------------- CSR

def csr_from_keep(keep: np.ndarray):
    """keep bool [B, H, nbq, nbk] -> (row_ptr int32 [B*H*nbq + 1], col_idx int32)."""
    rows = keep.reshape(-1, keep.shape[-1])
    counts = rows.sum(axis=1)
    row_ptr = np.zeros(rows.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(rows)[1]
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def keep_from_csr(row_ptr: np.ndarray, col_idx: np.ndarray, B: int, Hh: int, nbq: int, nbk: int) -> np.ndarray:
    keep = np.zeros((B * Hh * nbq, nbk), dtype=bool)
    for r in range(B * Hh * nbq):
        keep[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return keep.reshape(B, Hh, nbq, nbk)


def build_masks(T: int, H: int, W: int, block: int, specs: Iterable, batch: int,
                q: Optional[np.ndarray] = None, k: Optional[np.ndarray] = None,
                rstar_method: str = "segments", order: Optional[np.ndarray] = None) -> np.ndarray:
    """keep bool [B, H, nb, nb] for per-head specs (objects with kind, t_window, r_max, density).

    q and k are in storage order.  With ``order`` (a cuboid storage order, see
    ``layout.py``) window r* is taken by token-pair brute force on the stored
    coordinates; top-k and SICS depend only on the stored tokens.
    """
    specs = list(specs)
    N = T * H * W
    nb = -(-N // block)
    keep = np.zeros((batch, len(specs), nb, nb), dtype=bool)
    rstar_cache = {}
    pooled = None
    sics = None
    for h, sp in enumerate(specs):
        if sp.kind == WINDOW:
            if sp.t_window not in rstar_cache:
                if order is not None:
                    rstar_cache[sp.t_window] = window_rstar_bruteforce(T, H, W, block, sp.t_window,
                                                                       order=order)
                else:
                    fn = window_rstar_segments if rstar_method == "segments" else window_rstar_bruteforce
                    rstar_cache[sp.t_window] = fn(T, H, W, block, sp.t_window)
            keep[:, h] = window_select(rstar_cache[sp.t_window], sp.r_max, sp.density)[None]
        elif sp.kind == TOPK:
            if pooled is None:
                pooled = (pooled_means_f32(q, N, block), pooled_means_f32(k, N, block))
            scores = pooled_scores_f32(pooled[0][:, h], pooled[1][:, h])
            keep[:, h] = topk_select(scores, sp.density)
        elif sp.kind == SICS:
            if sics is None:
                sics = sics_block_scores_f32(k, N, block)
            for b in range(batch):
                keep[b, h] = sics_select(sics[b, h], sp.density)
        else:
            raise ValueError(f"unknown mask kind {sp.kind}")
    return keep
