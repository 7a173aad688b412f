"""Oracle gradients of the hybrid layer (reverse mode through the plain forward), fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer is fine-tuned, not used frozen: the "SALAD" explainer's technical
summary, section 2.2, makes the projection on the linear branch a learnable
layer that starts at zero and the scale s the output of a small learned module,
and section 3 reports the fine-tuning budget.  Training needs the gradient of a
loss through the layer with respect to Q, K, V (which come from the shared
projections), to W_lin and to the gate g.  Given dout = dL/dout, this module
returns dq, dk, dv, dW_lin and dgate of

    out = o_s + g[b, h] * (o_l . W_lin)          (``attention.layer_forward``)

by writing that forward once more in torch (fp64, CPU: dense masked softmax over
the kept key blocks, the quadratic form of ReLU linear attention, the gated mix)
and differentiating it with ``torch.autograd``.  Padded query rows (>= N) output
0 and receive no gradient; padded keys take part in neither branch.  ReLU's
derivative is taken as 0 at 0 (torch's convention; the inputs never hit 0
exactly).
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def _keep_matrix(row_ptr, col_idx, B: int, Hh: int, nb: int) -> np.ndarray:
    keep = np.zeros((B * Hh * nb, nb), dtype=bool)
    for r in range(B * Hh * nb):
        keep[r, np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]])] = True
    return keep.reshape(B, Hh, nb, nb)


def _forward_torch(q, k, v, w, g, allowed, N: int, eps: float, scale: float):
    import torch
    qv, kv, vv = q[:, :, :N], k[:, :, :N], v[:, :, :N]
    logits = scale * torch.einsum("bhic,bhjc->bhij", qv, kv)
    # a row that keeps no valid key outputs 0 (its logits stay finite so that
    # no NaN enters the softmax; the where() passes it no gradient)
    empty = ~allowed.any(dim=-1, keepdim=True)
    logits = logits.masked_fill(~allowed & ~empty, float("-inf"))
    p = torch.softmax(logits, dim=-1)
    p = torch.where(empty, torch.zeros_like(p), p)
    o_s = p @ vv
    a = torch.relu(qv) @ torch.relu(kv).transpose(-1, -2)
    o_l = (a @ vv) / (a.sum(dim=-1, keepdim=True) + eps)
    out = o_s + g[:, :, None, None] * (o_l @ w)
    return out, o_s, o_l


def layer_backward(q, k, v, row_ptr, col_idx, gate, w_lin, N: int, block: int, eps: float, dout,
                   scale: Optional[float] = None):
    """Gradients of <dout, out> for the layer; returns a dict of fp64 numpy arrays.

    q, k, v, dout: [B, H, n_pad, d]; gate: [B*H]; w_lin: [d, d].
    Keys: out, o_s, o_l ([B, H, n_pad, d], rows >= N zero), dq, dk, dv ([B, H, n_pad, d],
    rows >= N zero), dw_lin [d, d], dgate [B*H].
    """
    import torch
    B, Hh, n_pad, d = q.shape
    nb = n_pad // block
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    keep = _keep_matrix(row_ptr, col_idx, B, Hh, nb)
    tok_blk = np.arange(N) // block
    allowed = torch.from_numpy(keep[:, :, tok_blk][:, :, :, tok_blk])
    t = {name: torch.tensor(np.asarray(x, np.float64), requires_grad=True)
         for name, x in (("q", q), ("k", k), ("v", v), ("w", w_lin))}
    t["g"] = torch.tensor(np.asarray(gate, np.float64).reshape(B, Hh), requires_grad=True)
    out, o_s, o_l = _forward_torch(t["q"], t["k"], t["v"], t["w"], t["g"], allowed, N, eps, scale)
    dout_t = torch.from_numpy(np.asarray(dout, np.float64)[:, :, :N])
    loss = (out * dout_t).sum()
    loss.backward()

    def full(x):
        y = np.zeros((B, Hh, n_pad, d), dtype=np.float64)
        y[:, :, :N] = x.detach().numpy()
        return y

    return {
        "out": full(out), "o_s": full(o_s), "o_l": full(o_l),
        "dq": t["q"].grad.numpy(), "dk": t["k"].grad.numpy(), "dv": t["v"].grad.numpy(),
        "dw_lin": t["w"].grad.numpy(), "dgate": t["g"].grad.numpy().reshape(-1),
    }


def _row_softmax(qf, kf, rows, keys, scale):
    lg = scale * (qf[rows] @ kf[keys].T)
    lg = lg - lg.max(axis=1, keepdims=True)
    p = np.exp(lg)
    return p / p.sum(axis=1, keepdims=True)


def _kept_keys(row_ptr, col_idx, r, block, N):
    parts = [np.arange(kb * block, min((kb + 1) * block, N)) for kb in col_idx[row_ptr[r]:row_ptr[r + 1]]]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def layer_backward_sampled(q, k, v, row_ptr, col_idx, gate, w_lin, N: int, block: int, eps: float, dout,
                           qblocks, kblocks, scale: Optional[float] = None):
    """The same gradients as ``layer_backward`` at sampled blocks of a layer too large for it (fp64).

    Written from the closed forms instead of autograd (pinned against it by the
    CPU tests).  With phi = ReLU, u = phi(q) S, den = phi(q).z + eps, o_l = u/den,
    t = dout W^T, r = <t, o_l>, dU = g t / den, dden = -g r / den over every
    valid token of a head:
      dS_lin = sum phi(q) dU^T, dz_lin = sum phi(q) dden,
      dW = sum over heads of g o_l^T dout, dgate = sum r;
    for a query block: P = softmax over its kept keys, o_s = P V,
      D = <dout, o_s>, dS = P (dout V^T - D), dq = scale dS K + (S dU + z dden) [q > 0];
    for a key block: the same P and dS of every query block that keeps it,
      dv = P^T dout + dS_lin^T phi(k), dk = scale dS^T q + (dS_lin v + dz_lin) [k > 0].
    qblocks, kblocks: lists of (b, h, block).  Returns dict with dq [len(qblocks), block, d],
    dk, dv [len(kblocks), block, d] (rows past N zero), dw_lin [d, d], dgate [B*H].
    """
    B, Hh, n_pad, d = q.shape
    nb = n_pad // block
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    w = np.asarray(w_lin, np.float64)
    g = np.asarray(gate, np.float64)
    lin = {}
    dW = np.zeros((d, d))
    dg = np.zeros(B * Hh)
    for b in range(B):
        for h in range(Hh):
            gv = g[b * Hh + h]
            qf = np.asarray(q[b, h, :N], np.float64)
            kf = np.asarray(k[b, h, :N], np.float64)
            vf = np.asarray(v[b, h, :N], np.float64)
            do = np.asarray(dout[b, h, :N], np.float64)
            pq, pk = np.maximum(qf, 0), np.maximum(kf, 0)
            S, z = pk.T @ vf, pk.sum(axis=0)
            den = pq @ z + eps
            ol = (pq @ S) / den[:, None]
            t = do @ w.T
            r = np.sum(t * ol, axis=1)
            dU = gv * t / den[:, None]
            dden = -gv * r / den
            dW += gv * ol.T @ do
            dg[b * Hh + h] = r.sum()
            lin[(b, h)] = dict(qf=qf, kf=kf, vf=vf, do=do, S=S, z=z, dU=dU, dden=dden,
                               dS=pq.T @ dU, dz=pq.T @ dden)

    def sparse_rows(b, h, qb):
        L = lin[(b, h)]
        rows = np.arange(qb * block, min((qb + 1) * block, N))
        keys = _kept_keys(row_ptr, col_idx, (b * Hh + h) * nb + qb, block, N)
        if keys.size == 0:
            return rows, keys, np.zeros((rows.size, 0)), np.zeros((rows.size, 0))
        P = _row_softmax(L["qf"], L["kf"], rows, keys, scale)
        D = np.sum(L["do"][rows] * (P @ L["vf"][keys]), axis=1)
        dS = P * (L["do"][rows] @ L["vf"][keys].T - D[:, None])
        return rows, keys, P, dS

    dq = np.zeros((len(qblocks), block, d))
    for idx, (b, h, qb) in enumerate(qblocks):
        L = lin[(b, h)]
        rows, keys, _, dS = sparse_rows(b, h, qb)
        dq_s = scale * dS @ L["kf"][keys] if keys.size else np.zeros((rows.size, d))
        dq_l = (L["dU"][rows] @ L["S"].T + L["dden"][rows, None] * L["z"][None, :]) * (L["qf"][rows] > 0)
        dq[idx, :rows.size] = dq_s + dq_l
    dk = np.zeros((len(kblocks), block, d))
    dv = np.zeros((len(kblocks), block, d))
    for idx, (b, h, kb) in enumerate(kblocks):
        L = lin[(b, h)]
        cols = np.arange(kb * block, min((kb + 1) * block, N))
        acc_k = np.zeros((cols.size, d))
        acc_v = np.zeros((cols.size, d))
        for qb in range(nb):
            r = (b * Hh + h) * nb + qb
            if kb not in set(col_idx[row_ptr[r]:row_ptr[r + 1]].tolist()):
                continue
            rows, keys, P, dS = sparse_rows(b, h, qb)
            sel = np.searchsorted(keys, cols)
            acc_v += P[:, sel].T @ L["do"][rows]
            acc_k += scale * dS[:, sel].T @ L["qf"][rows]
        pk = np.maximum(L["kf"][cols], 0)
        dv[idx, :cols.size] = acc_v + pk @ L["dS"]
        dk[idx, :cols.size] = acc_k + (L["vf"][cols] @ L["dS"].T + L["dz"][None, :]) * (L["kf"][cols] > 0)
    return {"dq": dq, "dk": dk, "dv": dv, "dw_lin": dW, "dgate": dg}
