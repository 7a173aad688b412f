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
SALAD_MASK_BAD_START = 1
SALAD_MASK_BAD_ROW_PTR = 2
SALAD_MASK_BAD_COL = 4
SALAD_MASK_BAD_ORDER = 8


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
    "salad_mask_nnz": (_i64, [ctypes.POINTER(salad_shape), ctypes.POINTER(salad_mask_spec)]),
    "salad_workspace_bytes": (_sz, [ctypes.POINTER(salad_shape)]),
    "salad_build_mask": (ctypes.c_int, [ctypes.POINTER(salad_shape), ctypes.POINTER(salad_mask_spec),
                                        _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "salad_bwd_workspace_bytes": (_sz, [ctypes.POINTER(salad_shape)]),
    "salad_attn_bwd": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _f,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "salad_token_order": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp]),
    "salad_check_mask": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _i64, _vp, _vp]),
    "salad_permute_tokens": (ctypes.c_int, [ctypes.POINTER(salad_shape), ctypes.c_int, _vp, _vp, _vp]),
    "salad_gate_from_q": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _sz, _vp]),
    "salad_linear_state": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "salad_attn_fwd": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _f, _f, _f, _vp, _vp, _vp, _sz, _vp]),
    "salad_attn_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(salad_shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _f, _f, _f, _vp, _vp, _vp]),
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


def _torch_dtype(code):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32, "u8": torch.uint8}[code]


def _t(t, dtype, numel, what: str, optional: bool = False) -> Optional[int]:
    """Data pointer of a contiguous device tensor after checking its dtype and element count.

    dtype: "f32", "bf16", "i32", "u8", or a salad_dtype code (the layer's dtype); numel: the exact count
    the C function reads or writes, or (lo,) for a lower bound."""
    if t is None:
        if optional:
            return None
        raise SaladError(SALAD_EINVAL, f"{what}: a tensor is required")
    want = _torch_dtype(("f32", "bf16")[dtype] if isinstance(dtype, int) else dtype)
    if t.dtype != want:
        raise SaladError(SALAD_EINVAL, f"{what}: dtype {t.dtype}, expected {want}")
    n = t.numel()
    if isinstance(numel, tuple):
        if n < numel[0]:
            raise SaladError(SALAD_EINVAL, f"{what}: {n} elements, at least {numel[0]} needed")
    elif n != numel:
        raise SaladError(SALAD_EINVAL, f"{what}: {n} elements, expected {numel}")
    return _p(t)


def _sizes(shape: salad_shape):
    """(elements of a [B, H, n_pad, d] tensor, B*H, rows of the CSR + 1, d*d)."""
    bh = shape.batch * shape.heads
    return bh * shape.n_pad * shape.head_dim, bh, bh * (shape.n_pad // shape.block) + 1, shape.head_dim ** 2


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


def salad_mask_nnz(shape: salad_shape, specs) -> int:
    n = lib().salad_mask_nnz(ctypes.byref(shape), specs)
    if n < 0:
        _check(int(n), "salad_mask_nnz")
    return int(n)


def salad_workspace_bytes(shape: salad_shape) -> int:
    return int(lib().salad_workspace_bytes(ctypes.byref(shape)))


def salad_build_mask(shape, specs, q, k, row_ptr, col_idx, w_g=None, gate=None, ws=None, stream=None):
    nt, bh, nrp, _ = _sizes(shape)
    dt = shape.dtype
    st = lib().salad_build_mask(ctypes.byref(shape), specs, _t(q, dt, nt, "q", True), _t(k, dt, nt, "k", True),
                                _t(row_ptr, "i32", nrp, "row_ptr"), _t(col_idx, "i32", (1,), "col_idx"),
                                col_idx.numel(), _t(w_g, "f32", shape.head_dim, "w_g", True),
                                _t(gate, "f32", bh, "gate", True), _t(ws, "u8", (1,), "ws"),
                                ws.numel(), _stream(stream))
    _check(st, "salad_build_mask")


def salad_check_mask(shape, row_ptr, col_idx, result, stream=None):
    """Enqueue the CSR check; result (device int32 [1]) receives 0 or the SALAD_MASK_BAD_* bits."""
    nrp = _sizes(shape)[2]
    _check(lib().salad_check_mask(ctypes.byref(shape), _t(row_ptr, "i32", nrp, "row_ptr"),
                                  _t(col_idx, "i32", (0,), "col_idx"), col_idx.numel(),
                                  _t(result, "i32", 1, "result"), _stream(stream)), "salad_check_mask")


def salad_token_order(shape: salad_shape):
    """Host int32 numpy array [n_pad]: frame-major index of the token at each slot."""
    import numpy as np
    order = np.empty(shape.n_pad, dtype=np.int32)
    _check(lib().salad_token_order(ctypes.byref(shape), order.ctypes.data), "salad_token_order")
    return order


def salad_permute_tokens(shape, inverse, src, dst, stream=None):
    nt = _sizes(shape)[0]
    _check(lib().salad_permute_tokens(ctypes.byref(shape), int(inverse), _t(src, shape.dtype, nt, "src"),
                                      _t(dst, shape.dtype, nt, "dst"), _stream(stream)), "salad_permute_tokens")


def salad_gate_from_q(shape, q, w_g, gate, ws, stream=None):
    nt, bh, _, _ = _sizes(shape)
    _check(lib().salad_gate_from_q(ctypes.byref(shape), _t(q, shape.dtype, nt, "q"),
                                   _t(w_g, "f32", shape.head_dim, "w_g"), _t(gate, "f32", bh, "gate"),
                                   _t(ws, "u8", (1,), "ws"), ws.numel(), _stream(stream)), "salad_gate_from_q")


def salad_linear_state(shape, k, v, S, z, ws, stream=None):
    nt, bh, _, dd = _sizes(shape)
    _check(lib().salad_linear_state(ctypes.byref(shape), _t(k, shape.dtype, nt, "k"), _t(v, shape.dtype, nt, "v"),
                                    _t(S, "f32", bh * dd, "S"), _t(z, "f32", bh * shape.head_dim, "z"),
                                    _t(ws, "u8", (1,), "ws"), ws.numel(), _stream(stream)), "salad_linear_state")


def _qkv_csr(shape, q, k, v, row_ptr, col_idx):
    nt, _, nrp, _ = _sizes(shape)
    dt = shape.dtype
    return (_t(q, dt, nt, "q"), _t(k, dt, nt, "k"), _t(v, dt, nt, "v"), _t(row_ptr, "i32", nrp, "row_ptr"),
            _t(col_idx, "i32", (1,), "col_idx"))


def salad_attn_fwd(shape, q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, drop_tau, out, ws,
                   stream=None, lse=None):
    nt, bh, _, dd = _sizes(shape)
    _check(lib().salad_attn_fwd(ctypes.byref(shape), *_qkv_csr(shape, q, k, v, row_ptr, col_idx),
                                _t(gate, "f32", bh, "gate"), _t(w_lin, shape.dtype, dd, "w_lin"), eps, scale,
                                drop_tau, _t(out, shape.dtype, nt, "out"),
                                _t(lse, "f32", bh * shape.n_pad, "lse", True), _t(ws, "u8", (1,), "ws"),
                                ws.numel(), _stream(stream)), "salad_attn_fwd")


def salad_attn_fwd_noalloc(shape, q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, drop_tau, out, stream=None,
                           lse=None):
    """salad_attn_fwd on the library's static scratch: no workspace argument, nothing allocated."""
    nt, bh, _, dd = _sizes(shape)
    _check(lib().salad_attn_fwd_noalloc(ctypes.byref(shape), *_qkv_csr(shape, q, k, v, row_ptr, col_idx),
                                        _t(gate, "f32", bh, "gate"), _t(w_lin, shape.dtype, dd, "w_lin"), eps,
                                        scale, drop_tau, _t(out, shape.dtype, nt, "out"),
                                        _t(lse, "f32", bh * shape.n_pad, "lse", True), _stream(stream)),
           "salad_attn_fwd_noalloc")


def salad_attn_fwd_branches(shape, q, k, v, row_ptr, col_idx, eps, scale, out_sparse, out_lin, ws,
                            stream=None):
    nt = _sizes(shape)[0]
    _check(lib().salad_attn_fwd_branches(ctypes.byref(shape), *_qkv_csr(shape, q, k, v, row_ptr, col_idx), eps,
                                         scale, _t(out_sparse, shape.dtype, nt, "out_sparse", True),
                                         _t(out_lin, shape.dtype, nt, "out_lin", True), _t(ws, "u8", (1,), "ws"),
                                         ws.numel(), _stream(stream)), "salad_attn_fwd_branches")


def salad_linear_prepare(shape, k, v, gate, w_lin, ws, stream=None, drop_tau=0.0):
    nt, bh, _, dd = _sizes(shape)
    _check(lib().salad_linear_prepare(ctypes.byref(shape), _t(k, shape.dtype, nt, "k"), _t(v, shape.dtype, nt, "v"),
                                      _t(gate, "f32", bh, "gate"), _t(w_lin, shape.dtype, dd, "w_lin"), drop_tau,
                                      _t(ws, "u8", (1,), "ws"), ws.numel(), _stream(stream)), "salad_linear_prepare")


def salad_attn_apply(shape, q, k, v, row_ptr, col_idx, gate, eps, scale, drop_tau, out, ws, stream=None,
                     lse=None):
    nt, bh, _, _ = _sizes(shape)
    _check(lib().salad_attn_apply(ctypes.byref(shape), *_qkv_csr(shape, q, k, v, row_ptr, col_idx),
                                  _t(gate, "f32", bh, "gate"), eps, scale, drop_tau, _t(out, shape.dtype, nt, "out"),
                                  _t(lse, "f32", bh * shape.n_pad, "lse", True), _t(ws, "u8", (1,), "ws"),
                                  ws.numel(), _stream(stream)), "salad_attn_apply")


def salad_bwd_workspace_bytes(shape: salad_shape) -> int:
    return int(lib().salad_bwd_workspace_bytes(ctypes.byref(shape)))


def salad_attn_bwd(shape, q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, out, dout, dq, dk, dv, dw_lin,
                   dgate, ws, stream=None, lse=None):
    nt, bh, _, dd = _sizes(shape)
    dt = shape.dtype
    _check(lib().salad_attn_bwd(ctypes.byref(shape), *_qkv_csr(shape, q, k, v, row_ptr, col_idx),
                                _t(gate, "f32", bh, "gate"), _t(w_lin, dt, dd, "w_lin"), eps, scale,
                                _t(out, dt, nt, "out"), _t(lse, "f32", bh * shape.n_pad, "lse", True),
                                _t(dout, dt, nt, "dout"), _t(dq, dt, nt, "dq"), _t(dk, dt, nt, "dk"),
                                _t(dv, dt, nt, "dv"), _t(dw_lin, "f32", dd, "dw_lin"), _t(dgate, "f32", bh, "dgate"),
                                _t(ws, "u8", (1,), "ws"), ws.numel(), _stream(stream)), "salad_attn_bwd")
