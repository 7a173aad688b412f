"""Seeded generator for Q, K, V, W_lin and the gate inputs of one layer.

Recipe (the SALAD pages give none; this one gives video-like, locality-biased
attention):

    X[b,h,n,c] = eps + 0.5 * sin(w_t[c]*t + w_y[c]*y + w_x[c]*x + phi[h,c])

with eps ~ N(0,1) i.i.d., w_t, w_y, w_x ~ U(0, pi/4) per channel, phi ~ U(0, 2pi)
per (head, channel), and (t, y, x) the frame-major coordinates of token n.  Q and
K share (w, phi) so that nearby tokens attend to each other; V draws its own.
W_lin ~ N(0, 1/d); the gate is a constant, U(0, 0.3) per head, or (for the
"from_q" configs) a vector w_g ~ N(0, 1/d) that the operator turns into a gate.

Every draw comes from its own stream ``default_rng([seed, stream])`` so that the
values do not depend on which other arrays were requested.  bf16 configs round
every tensor to bf16 (round to nearest even) here, once; both the GPU path and
the oracle then consume exactly the same numbers.

The padded tail (tokens N..n_pad-1) holds 0, or the finite canary 1e4 when
``canary=True``: the operator must ignore it either way.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import LayerConfig

# stream ids of default_rng([seed, stream])
_S_QK_FREQ, _S_V_FREQ, _S_QN, _S_KN, _S_VN, _S_WLIN, _S_GATE, _S_WG = 0, 1, 2, 3, 4, 5, 6, 7
_S_DOUT = 9  # stream 8 is the c5 densities (configs.py)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    q: np.ndarray  # float32 [B, H, n_pad, d]: exact values (bf16-representable for bf16 configs)
    k: np.ndarray
    v: np.ndarray
    w_lin: np.ndarray  # float32 [d, d]
    gate: Optional[np.ndarray]  # float32 [B*H], or None when the gate comes from Q
    w_g: Optional[np.ndarray]  # float32 [d] for "from_q" configs
    q_bits: Optional[np.ndarray] = None  # uint16 bf16 bits, same shape as q (bf16 configs)
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    w_lin_bits: Optional[np.ndarray] = None


def _coords(cfg: LayerConfig) -> np.ndarray:
    n = np.arange(cfg.N, dtype=np.int64)
    t = n // (cfg.H * cfg.W)
    y = (n // cfg.W) % cfg.H
    x = n % cfg.W
    return np.stack([t, y, x], axis=1).astype(np.float64)


def _smooth_tensor(cfg: LayerConfig, freq_stream: int, noise_stream: int, canary: bool) -> np.ndarray:
    B, Hh, d, N, n_pad = cfg.batch, cfg.heads, cfg.head_dim, cfg.N, cfg.n_pad
    frng = np.random.default_rng([cfg.seed, freq_stream])
    omega = frng.uniform(0.0, np.pi / 4.0, size=(3, d))  # rows: w_t, w_y, w_x
    phi = frng.uniform(0.0, 2.0 * np.pi, size=(Hh, d))
    base = _coords(cfg) @ omega  # [N, d] float64
    nrng = np.random.default_rng([cfg.seed, noise_stream])
    out = np.empty((B, Hh, n_pad, d), dtype=np.float32)
    for b in range(B):
        for h in range(Hh):
            noise = nrng.standard_normal(size=(N, d), dtype=np.float32)
            smooth = (0.5 * np.sin(base + phi[h][None, :])).astype(np.float32)
            out[b, h, :N] = noise + smooth
    out[:, :, N:] = 1.0e4 if canary else 0.0
    return out


def make_inputs(cfg: LayerConfig, canary: bool = False) -> LayerInputs:
    d = cfg.head_dim
    q = _smooth_tensor(cfg, _S_QK_FREQ, _S_QN, canary)
    k = _smooth_tensor(cfg, _S_QK_FREQ, _S_KN, canary)
    v = _smooth_tensor(cfg, _S_V_FREQ, _S_VN, canary)
    w_lin = (np.random.default_rng([cfg.seed, _S_WLIN]).standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)

    gate = None
    w_g = None
    if cfg.gate_kind == "const":
        gate = np.full(cfg.batch * cfg.heads, cfg.gate_const, dtype=np.float32)
    elif cfg.gate_kind == "uniform":
        gate = np.random.default_rng([cfg.seed, _S_GATE]).uniform(0.0, 0.3, size=cfg.batch * cfg.heads).astype(np.float32)
    elif cfg.gate_kind == "from_q":
        w_g = (np.random.default_rng([cfg.seed, _S_WG]).standard_normal(d) / np.sqrt(d)).astype(np.float32)
    else:
        raise ValueError(cfg.gate_kind)

    inp = LayerInputs(cfg=cfg, q=q, k=k, v=v, w_lin=w_lin, gate=gate, w_g=w_g)
    if cfg.dtype == "bf16":
        for name in ("q", "k", "v", "w_lin"):
            bits = bf16_round(getattr(inp, name))
            setattr(inp, name + "_bits", bits)
            setattr(inp, name, bf16_bits_to_f32(bits))
    elif cfg.dtype != "f32":
        raise ValueError(cfg.dtype)
    return inp


def make_grad_output(cfg: LayerConfig, scale: float = 1.0):
    """Upstream gradient dL/dout for a backward pass: scale * N(0, 1), [B, H, n_pad, d].

    Returns (values float32, bf16 bits uint16 or None): bf16 configs round once so
    that both sides see the same values; padding rows hold the canary 1e4, which
    no result may read.
    """
    rng = np.random.default_rng([cfg.seed, _S_DOUT])
    x = (scale * rng.standard_normal((cfg.batch, cfg.heads, cfg.n_pad, cfg.head_dim))).astype(np.float32)
    x[:, :, cfg.N:] = 1e4
    if cfg.dtype == "bf16":
        bits = bf16_round(x)
        return bf16_bits_to_f32(bits), bits
    return x, None
