"""Convenience wrapper that owns the device buffers of one hybrid-attention layer.

Buffer ownership and argument marshalling only; every computation is a call
into libsalad through ``block_sparse_linear_st_amd.salad``.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import salad as S

_TORCH_DTYPE = {S.SALAD_F32: torch.float32, S.SALAD_BF16: torch.bfloat16}


class SaladLayer:
    """One layer shape plus per-head mask specs, with workspace and CSR buffers."""

    def __init__(self, batch: int, heads: int, head_dim: int, T: int, H: int, W: int, block: int,
                 dtype: int, specs: Sequence, device: str = "cuda", cuboid=(0, 0, 0)):
        self.shape = S.make_shape(batch, heads, head_dim, T, H, W, block, dtype, cuboid=cuboid)
        self.specs = S.make_specs(specs)
        self.device = torch.device(device)
        self.torch_dtype = _TORCH_DTYPE[dtype]
        self.N = T * H * W
        self.nb = self.shape.n_pad // block
        ws_bytes = S.salad_workspace_bytes(self.shape)
        if ws_bytes == 0:
            raise S.SaladError(S.SALAD_EINVAL, "invalid or unsupported layer shape")
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        self.row_ptr = torch.empty(batch * heads * self.nb + 1, dtype=torch.int32, device=self.device)
        self.col_idx = torch.empty(max(1, S.salad_mask_nnz(self.shape, self.specs)), dtype=torch.int32,
                                   device=self.device)

    def tensor_shape(self):
        s = self.shape
        return (s.batch, s.heads, s.n_pad, s.head_dim)

    def to_storage(self, src: torch.Tensor, dst: torch.Tensor, stream=None):
        """Frame-major src -> dst in the layer's storage order (a copy for frame-major layers)."""
        S.salad_permute_tokens(self.shape, 0, src, dst, stream)
        return dst

    def from_storage(self, src: torch.Tensor, dst: torch.Tensor, stream=None):
        """Storage-order src -> frame-major dst."""
        S.salad_permute_tokens(self.shape, 1, src, dst, stream)
        return dst

    def build_mask(self, q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
                   w_g: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None, stream=None):
        S.salad_build_mask(self.shape, self.specs, q, k, self.row_ptr, self.col_idx, w_g, gate, self.ws, stream)

    def gate_from_q(self, q, w_g, gate, stream=None):
        S.salad_gate_from_q(self.shape, q, w_g, gate, self.ws, stream)

    def linear_state(self, k, v, S_out, z_out, stream=None):
        S.salad_linear_state(self.shape, k, v, S_out, z_out, self.ws, stream)

    def forward(self, q, k, v, gate, w_lin, out, eps: float = 1e-6, scale: float = 0.0,
                drop_tau: float = 0.0, stream=None, lse=None):
        S.salad_attn_fwd(self.shape, q, k, v, self.row_ptr, self.col_idx, gate, w_lin, eps, scale, drop_tau,
                         out, self.ws, stream, lse=lse)
        return out

    def branches(self, q, k, v, out_sparse, out_lin, eps: float = 1e-6, scale: float = 0.0, stream=None):
        S.salad_attn_fwd_branches(self.shape, q, k, v, self.row_ptr, self.col_idx, eps, scale, out_sparse,
                                  out_lin, self.ws, stream)

    def backward(self, q, k, v, gate, w_lin, out, dout, dq, dk, dv, dw_lin, dgate, eps: float = 1e-6,
                 scale: float = 0.0, lse=None, stream=None, row_ptr=None, col_idx=None):
        """Gradients of the layer (salad_attn_bwd) into caller buffers; the backward workspace is owned here.
        The mask is the layer's current one unless the forward's (row_ptr, col_idx) are given."""
        ws = self.backward_workspace()
        rp = self.row_ptr if row_ptr is None else row_ptr
        ci = self.col_idx if col_idx is None else col_idx
        S.salad_attn_bwd(self.shape, q, k, v, rp, ci, gate, w_lin, eps, scale, out, dout,
                         dq, dk, dv, dw_lin, dgate, ws, stream, lse=lse)

    def backward_workspace(self) -> torch.Tensor:
        if getattr(self, "_bwd_ws", None) is None:
            n = S.salad_bwd_workspace_bytes(self.shape)
            if n == 0:
                raise S.SaladError(S.SALAD_EINVAL, "invalid or unsupported layer shape")
            self._bwd_ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._bwd_ws

    def attention(self, q, k, v, gate, w_lin, eps: float = 1e-6, scale: float = 0.0):
        """out = layer(q, k, v, gate, w_lin) as a differentiable torch op (bf16 layers) over the mask the last
        build_mask call made; the backward gives dq, dk, dv, dgate and dW_lin (cast to W_lin's dtype) over that
        same mask, even if build_mask runs again before the backward (the op keeps a copy of the CSR)."""
        return _SaladAttention.apply(self, q, k, v, gate, w_lin, eps, scale)


class _SaladAttention(torch.autograd.Function):
    """Forward through salad_attn_fwd keeping each row's log2-sum-exp, backward through salad_attn_bwd.
    Marshalling only: outputs and gradient buffers are allocated here, every step runs in libsalad."""

    @staticmethod
    def forward(ctx, layer, q, k, v, gate, w_lin, eps, scale):
        if layer.torch_dtype != torch.bfloat16:
            raise S.SaladError(S.SALAD_EUNSUPPORTED, "the differentiable layer needs a bf16 shape")
        q, k, v, w_lin = (t.contiguous() for t in (q, k, v, w_lin))
        gate = gate.contiguous()
        out = torch.empty_like(q)
        s = layer.shape
        lse = torch.empty(s.batch * s.heads * s.n_pad, dtype=torch.float32, device=q.device)
        layer.forward(q, k, v, gate, w_lin, out, eps=eps, scale=scale, lse=lse,
                      stream=torch.cuda.current_stream().cuda_stream)
        # the mask this forward used: a later build_mask on the layer must not change the backward's
        nnz = layer.col_idx.numel()
        row_ptr, col_idx = layer.row_ptr.clone(), layer.col_idx[:nnz].clone()
        ctx.save_for_backward(q, k, v, gate, w_lin, out, lse, row_ptr, col_idx)
        ctx.layer, ctx.eps, ctx.scale = layer, eps, scale
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, gate, w_lin, out, lse, row_ptr, col_idx = ctx.saved_tensors
        layer = ctx.layer
        dout = dout.to(torch.bfloat16).contiguous()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        d = layer.shape.head_dim
        dw = torch.empty((d, d), dtype=torch.float32, device=q.device)
        dg = torch.empty(gate.numel(), dtype=torch.float32, device=q.device)
        layer.backward(q, k, v, gate, w_lin, out, dout, dq, dk, dv, dw, dg, eps=ctx.eps, scale=ctx.scale,
                       lse=lse, stream=torch.cuda.current_stream().cuda_stream, row_ptr=row_ptr, col_idx=col_idx)
        return None, dq, dk, dv, dg.view_as(gate).to(gate.dtype), dw.to(w_lin.dtype), None, None
