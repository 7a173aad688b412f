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
