"""Oracle forward of the hybrid layer: masked softmax, ReLU linear attention, gated mix.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Everything is fp64 on the exact input values.  Shapes: q, k, v are [B, H, n_pad, d]
with tokens N..n_pad-1 padding; padded keys take part in neither branch and
padded query rows output 0.

Sparse branch ("SALAD" explainer, technical summary section 2.1; sciencestack
"SALAD" abstract): for a valid query row i of query block q,

    o_s[i] = sum_j softmax_j(l_i)[j] v_j,   l_ij = scale * <q_i, k_j>

where l_ij = -inf unless key j < N lies in a key block that row q of the CSR
keeps.  A row that keeps no valid key outputs 0 (the pages never produce one;
this is the convention).  scale defaults to 1/sqrt(d).

Linear branch (explainer section 2.1: ReLU-based linear attention, O(N),
global token interaction), quadratic form over the valid tokens:

    A = ReLU(Q) ReLU(K)^T,   o_l[i] = (A V)[i] / (sum_j A[i, j] + eps).

Its linear form ReLU(q_i)^T S / (ReLU(q_i)^T z + eps) with S = ReLU(K)^T V and
z = sum_j ReLU(k_j) is the same number; ``linear_state`` and
``linear_attention_from_state`` exist so the tests can check that identity and
compare a device-side S and z directly.

Mix (explainer section 2.2: zero-initialised projection on the linear output,
sigmoid-bounded scale s; sciencestack TL;DR: input-dependent scalar gate):

    out[i] = o_s[i] + g[b, h] * (o_l[i] . W_lin)

with one W_lin [d, d] shared by the heads, applied on the right.  Branch
dropping (explainer section 2.3: at inference, drop linear branches whose scale
is very small): when ``drop_tau`` is given, heads with g < drop_tau output o_s.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


def _relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0)


def _rows_of(qb: int, block: int, N: int) -> np.ndarray:
    return np.arange(qb * block, min((qb + 1) * block, N))


def _sparse_block(qf, kf, vf, kept: np.ndarray, qb: int, N: int, block: int, scale: float) -> np.ndarray:
    """Output rows of query block qb (valid rows only) as a dense masked softmax."""
    rows = _rows_of(qb, block, N)
    out = np.zeros((rows.size, vf.shape[-1]), dtype=np.float64)
    if rows.size == 0:
        return out
    allowed = np.zeros(N, dtype=bool)
    for kb in kept:
        allowed[kb * block:min((kb + 1) * block, N)] = True
    if not allowed.any():
        return out
    logits = scale * (qf[rows] @ kf[:N].T)
    logits[:, ~allowed] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vf[:N]


def _blocks_to_visit(B: int, Hh: int, nb: int, qblocks) -> list:
    if qblocks is None:
        return [(b, h, qb) for b in range(B) for h in range(Hh) for qb in range(nb)]
    return [tuple(int(t) for t in x) for x in qblocks]


def sparse_attention(q, k, v, row_ptr, col_idx, N: int, block: int, scale: Optional[float] = None,
                     qblocks: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Sparse branch o_s.

    With qblocks None: returns fp64 [B, H, n_pad, d].  Otherwise returns fp64
    [len(qblocks), block, d] holding the rows of each listed (b, h, qb).
    """
    B, Hh, n_pad, d = q.shape
    nb = n_pad // block
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dv = v.shape[-1]
    visit = _blocks_to_visit(B, Hh, nb, qblocks)
    full = qblocks is None
    out = np.zeros((B, Hh, n_pad, dv) if full else (len(visit), block, dv), dtype=np.float64)
    cache = {}
    for idx, (b, h, qb) in enumerate(visit):
        if (b, h) not in cache:
            cache = {(b, h): (np.asarray(q[b, h], np.float64), np.asarray(k[b, h], np.float64),
                              np.asarray(v[b, h], np.float64))}
        qf, kf, vf = cache[(b, h)]
        r = (b * Hh + h) * nb + qb
        kept = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]])
        o = _sparse_block(qf, kf, vf, kept, qb, N, block, scale)
        if full:
            out[b, h, qb * block:qb * block + o.shape[0]] = o
        else:
            out[idx, :o.shape[0]] = o
    return out


def sparse_lse2(q, k, row_ptr, col_idx, N: int, block: int, scale: Optional[float] = None) -> np.ndarray:
    """Row statistic the forward keeps for training: log2 of sum_j exp(l_ij) over the kept keys.

    l_ij = scale * <q_i, k_j> as in ``sparse_attention``; log2 because the
    kernels work in base 2 (x = l * log2(e)).  +inf for padding rows and rows
    that keep no valid key.  Returns fp64 [B, H, n_pad].
    """
    B, Hh, n_pad, d = q.shape
    nb = n_pad // block
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.full((B, Hh, n_pad), np.inf)
    for b in range(B):
        for h in range(Hh):
            kf = np.asarray(k[b, h], np.float64)
            for qb in range(nb):
                rows = _rows_of(qb, block, N)
                if rows.size == 0:
                    continue
                r = (b * Hh + h) * nb + qb
                keys = np.concatenate([np.arange(kb * block, min((kb + 1) * block, N))
                                       for kb in col_idx[row_ptr[r]:row_ptr[r + 1]]] or [np.zeros(0, np.int64)])
                if keys.size == 0:
                    continue
                lg = scale * (np.asarray(q[b, h, rows], np.float64) @ kf[keys].T)
                m = lg.max(axis=1, keepdims=True)
                out[b, h, rows] = (m[:, 0] + np.log(np.exp(lg - m).sum(axis=1))) / np.log(2.0)
    return out


def linear_attention(q, k, v, N: int, eps: float, block: Optional[int] = None,
                     qblocks: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Linear branch o_l in quadratic form; same return convention as ``sparse_attention``."""
    B, Hh, n_pad, _ = q.shape
    dv = v.shape[-1]
    if qblocks is None:
        out = np.zeros((B, Hh, n_pad, dv), dtype=np.float64)
        for b in range(B):
            for h in range(Hh):
                kr = _relu(np.asarray(k[b, h, :N], np.float64))
                vf = np.asarray(v[b, h, :N], np.float64)
                for r0 in range(0, N, 4096):
                    r1 = min(N, r0 + 4096)
                    A = _relu(np.asarray(q[b, h, r0:r1], np.float64)) @ kr.T
                    out[b, h, r0:r1] = (A @ vf) / (A.sum(axis=1, keepdims=True) + eps)
        return out
    assert block is not None
    visit = _blocks_to_visit(B, Hh, n_pad // block, qblocks)
    out = np.zeros((len(visit), block, dv), dtype=np.float64)
    for idx, (b, h, qb) in enumerate(visit):
        rows = _rows_of(qb, block, N)
        if rows.size == 0:
            continue
        kr = _relu(np.asarray(k[b, h, :N], np.float64))
        A = _relu(np.asarray(q[b, h, rows], np.float64)) @ kr.T
        out[idx, :rows.size] = (A @ np.asarray(v[b, h, :N], np.float64)) / (A.sum(axis=1, keepdims=True) + eps)
    return out


def linear_state(k, v, N: int):
    """S[b,h] = ReLU(K)^T V (d x d) and z[b,h] = sum_j ReLU(k_j) over valid tokens, fp64."""
    kr = _relu(np.asarray(k[:, :, :N], np.float64))
    vf = np.asarray(v[:, :, :N], np.float64)
    S = np.einsum("bhnc,bhne->bhce", kr, vf)
    z = kr.sum(axis=2)
    return S, z


def linear_attention_from_state(q, S, z, N: int, eps: float):
    """Linear form ReLU(q)^T S / (ReLU(q)^T z + eps); rows >= N are 0."""
    qr = _relu(np.asarray(q, np.float64))
    num = np.einsum("bhnc,bhce->bhne", qr, S)
    den = np.einsum("bhnc,bhc->bhn", qr, z)[..., None] + eps
    out = num / den
    out[:, :, N:] = 0.0
    return out


def mix(o_s, o_l, gate, w_lin, N: Optional[int] = None, drop_tau: Optional[float] = None,
        gate_index: Optional[Sequence[int]] = None):
    """out = o_s + g * (o_l . W_lin).

    Full tensors: o_s, o_l [B, H, n_pad, d] with N given (rows >= N become 0).
    Sampled blocks: o_s, o_l [M, block, d] and ``gate_index`` the b*H + h of each of
    the M blocks (``gate`` is indexed by b*H + h).
    """
    w = np.asarray(w_lin, np.float64)
    g = np.asarray(gate, np.float64)
    if gate_index is None:
        B, Hh = o_s.shape[:2]
        gg = g.reshape(B, Hh)[:, :, None, None]
        if drop_tau is not None:
            gg = np.where(gg < drop_tau, 0.0, gg)
        out = o_s + gg * (o_l @ w)
        out[:, :, N:] = 0.0
        return out
    out = np.empty_like(o_s)
    for idx, gi in enumerate(gate_index):
        gv = g[gi]
        if drop_tau is not None and gv < drop_tau:
            gv = 0.0
        out[idx] = o_s[idx] + gv * (o_l[idx] @ w)
    return out


def layer_forward(q, k, v, row_ptr, col_idx, gate, w_lin, N: int, block: int, eps: float,
                  scale: Optional[float] = None, drop_tau: Optional[float] = None,
                  qblocks: Optional[Iterable[Tuple[int, int, int]]] = None):
    """(out, o_s, o_l) of the whole layer, full or for the listed (b, h, qb) blocks.

    For sampled blocks the rows of a block beyond N are 0 in all three outputs.
    """
    if qblocks is None:
        o_s = sparse_attention(q, k, v, row_ptr, col_idx, N, block, scale)
        o_l = linear_attention(q, k, v, N, eps)
        return mix(o_s, o_l, gate, w_lin, N=N, drop_tau=drop_tau), o_s, o_l
    qblocks = [tuple(int(t) for t in x) for x in qblocks]
    Hh = q.shape[1]
    o_s = sparse_attention(q, k, v, row_ptr, col_idx, N, block, scale, qblocks=qblocks)
    o_l = linear_attention(q, k, v, N, eps, block=block, qblocks=qblocks)
    gidx = [b * Hh + h for (b, h, _) in qblocks]
    out = mix(o_s, o_l, gate, w_lin, drop_tau=drop_tau, gate_index=gidx)
    for idx, (_, _, qb) in enumerate(qblocks):
        nvalid = max(0, min(block, N - qb * block))
        out[idx, nvalid:] = 0.0
    return out, o_s, o_l
