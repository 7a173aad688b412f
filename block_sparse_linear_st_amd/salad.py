"""ctypes binding of libsalad (include/salad.h).

Argument marshalling only: every step of the operator runs in the HIP library.
PyTorch provides device memory and the current HIP stream.  The functions keep
the C names; tensors are passed by data pointer and must be contiguous device
tensors of the shape's dtype.  A missing library raises ``SaladError`` at the
first call: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsalad.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG), "include", "salad.h")

SALAD_OK = 0
SALAD_EINVAL = -1
SALAD_EUNSUPPORTED = -2
SALAD_ENOSPACE = -3
SALAD_EINFEASIBLE = -4
SALAD_EHIP = -5
SALAD_F32 = 0
SALAD_BF16 = 1
SALAD_MASK_WINDOW = 0
SALAD_MASK_TOPK = 1
SALAD_MASK_SICS = 2


class SaladError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class salad_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "head_dim", "T", "H", "W", "n_pad", "block", "dtype",
                 "cuboid_t", "cuboid_h", "cuboid_w")]


class salad_mask_spec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("t_window", ctypes.c_int32),
                ("r_max", ctypes.c_int32), ("density", ctypes.c_float)]


_lib = None

_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i64 = ctypes.c_int64
_f = ctypes.c_float
_SIGS = {
    "salad_version": (ctypes.c_int, []),
    "salad_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "salad_mask_nnz_max": (_i64, [ctypes.POINTER(salad_shape), ctypes.POINTER(salad_mask_spec)]),
    "salad_workspace_bytes": (_sz, [ctypes.POINTER(salad_shape)]),
    "salad_build_mask": (ctypes.c_int, [ctypes.POINTER(salad_shape), ctypes.POINTER(salad_mask_spec),
                                        _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "salad_bwd_workspace_bytes": (_sz, [ctypes.POINTER(salad_shape)]),
    "salad_attn_bwd": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _f,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "salad_token_order": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp]),
    "salad_permute_tokens": (ctypes.c_int, [ctypes.POINTER(salad_shape), ctypes.c_int, _vp, _vp, _vp]),
    "salad_gate_from_q": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _sz, _vp]),
    "salad_linear_state": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "salad_attn_fwd": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _f, _f, _f, _vp, _vp, _vp, _sz, _vp]),
    "salad_linear_prepare": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, ctypes.c_float,
                                            _vp, _sz, _vp]),
    "salad_attn_apply": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _vp,
                                        _f, _f, _f, _vp, _vp, _vp, _sz, _vp]),
    "salad_attn_fwd_branches": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp,
                                               _f, _f, _vp, _vp, _vp, _sz, _vp]),
}


def header_functions() -> list:
    """Names of the functions include/salad.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*SALAD_API\s+(?:const\s+)?[a-z_0-9]+\**\s+\**(salad_[a-z_0-9]+)\s*\(", text, re.M)))


def lib():
    """The loaded libsalad; raises SaladError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SaladError(SALAD_EHIP, f"{LIB_PATH} is missing: build it with "
                                         "`python -m block_sparse_linear_st_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != SALAD_OK:
        raise SaladError(status, f"{what}: {lib().salad_status_str(status).decode()} ({status})")


def make_shape(batch, heads, head_dim, T, H, W, block, dtype, n_pad=None, cuboid=(0, 0, 0)) -> salad_shape:
    N = T * H * W
    if n_pad is None:
        n_pad = -(-N // block) * block
    ct, ch, cw = (int(v) for v in cuboid)
    return salad_shape(batch, heads, head_dim, T, H, W, n_pad, block, dtype, ct, ch, cw)


def make_specs(specs: Sequence) -> ctypes.Array:
    """Host spec array from objects with kind, t_window, r_max, density."""
    arr = (salad_mask_spec * len(specs))()
    for i, s in enumerate(specs):
        arr[i] = salad_mask_spec(int(s.kind), int(s.t_window), int(s.r_max), float(s.density))
    return arr


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise SaladError(SALAD_EINVAL, "tensors must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---- the C entry points, by their C names ----------------------------------------------

def salad_version() -> int:
    return lib().salad_version()


def salad_status_str(status: int) -> str:
    return lib().salad_status_str(status).decode()


def salad_mask_nnz_max(shape: salad_shape, specs) -> int:
    n = lib().salad_mask_nnz_max(ctypes.byref(shape), specs)
    if n < 0:
        _check(int(n), "salad_mask_nnz_max")
    return int(n)


def salad_workspace_bytes(shape: salad_shape) -> int:
    return int(lib().salad_workspace_bytes(ctypes.byref(shape)))


def salad_build_mask(shape, specs, q, k, row_ptr, col_idx, info=None, w_g=None, gate=None,
                     ws=None, stream=None):
    st = lib().salad_build_mask(ctypes.byref(shape), specs, _p(q), _p(k), _p(row_ptr), _p(col_idx),
                                col_idx.numel(), _p(info), _p(w_g), _p(gate), _p(ws),
                                ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "salad_build_mask")


def salad_token_order(shape: salad_shape):
    """Host int32 numpy array [n_pad]: frame-major index of the token at each slot."""
    import numpy as np
    order = np.empty(shape.n_pad, dtype=np.int32)
    _check(lib().salad_token_order(ctypes.byref(shape), order.ctypes.data), "salad_token_order")
    return order


def salad_permute_tokens(shape, inverse, src, dst, stream=None):
    _check(lib().salad_permute_tokens(ctypes.byref(shape), int(inverse), _p(src), _p(dst), _stream(stream)),
           "salad_permute_tokens")


def salad_gate_from_q(shape, q, w_g, gate, ws, stream=None):
    _check(lib().salad_gate_from_q(ctypes.byref(shape), _p(q), _p(w_g), _p(gate), _p(ws), ws.numel(),
                                   _stream(stream)), "salad_gate_from_q")


def salad_linear_state(shape, k, v, S, z, ws, stream=None):
    _check(lib().salad_linear_state(ctypes.byref(shape), _p(k), _p(v), _p(S), _p(z), _p(ws), ws.numel(),
                                    _stream(stream)), "salad_linear_state")


def salad_attn_fwd(shape, q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, drop_tau, out, ws,
                   stream=None, lse=None):
    _check(lib().salad_attn_fwd(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(row_ptr), _p(col_idx),
                                _p(gate), _p(w_lin), eps, scale, drop_tau, _p(out), _p(lse), _p(ws), ws.numel(),
                                _stream(stream)), "salad_attn_fwd")


def salad_attn_fwd_branches(shape, q, k, v, row_ptr, col_idx, eps, scale, out_sparse, out_lin, ws,
                            stream=None):
    _check(lib().salad_attn_fwd_branches(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(row_ptr),
                                         _p(col_idx), eps, scale, _p(out_sparse), _p(out_lin), _p(ws),
                                         ws.numel(), _stream(stream)), "salad_attn_fwd_branches")


def salad_linear_prepare(shape, k, v, gate, w_lin, ws, stream=None, drop_tau=0.0):
    _check(lib().salad_linear_prepare(ctypes.byref(shape), _p(k), _p(v), _p(gate), _p(w_lin), drop_tau,
                                      _p(ws), ws.numel(), _stream(stream)), "salad_linear_prepare")


def salad_attn_apply(shape, q, k, v, row_ptr, col_idx, gate, eps, scale, drop_tau, out, ws, stream=None,
                     lse=None):
    _check(lib().salad_attn_apply(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(row_ptr), _p(col_idx),
                                  _p(gate), eps, scale, drop_tau, _p(out), _p(lse), _p(ws), ws.numel(),
                                  _stream(stream)), "salad_attn_apply")


def salad_bwd_workspace_bytes(shape: salad_shape) -> int:
    return int(lib().salad_bwd_workspace_bytes(ctypes.byref(shape)))


def salad_attn_bwd(shape, q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, out, dout, dq, dk, dv, dw_lin,
                   dgate, ws, stream=None, lse=None):
    _check(lib().salad_attn_bwd(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(row_ptr), _p(col_idx), _p(gate),
                                _p(w_lin), eps, scale, _p(out), _p(lse), _p(dout), _p(dq), _p(dk), _p(dv),
                                _p(dw_lin), _p(dgate), _p(ws), ws.numel(), _stream(stream)), "salad_attn_bwd")
