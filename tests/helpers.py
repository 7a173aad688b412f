"""Shared helpers for the GPU parity tests: device copies of seeded inputs and comparisons."""

from __future__ import annotations

import functools

import numpy as np

import oracle
from synth import CONFIGS, make_inputs

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
F32_MAX_ABS = 1e-4


def assert_close(got, ref, max_abs, rel_l2, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rl2 = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got - ref))
    print(f"{what}: max-abs {err:.3e} (bar {max_abs:g}), rel-L2 {rl2:.3e} (bar {rel_l2:g})", flush=True)
    assert err <= max_abs, f"{what}: max-abs {err:.3e} > {max_abs:g}"
    assert rl2 <= rel_l2, f"{what}: rel-L2 {rl2:.3e} > {rel_l2:g}"


@functools.lru_cache(maxsize=4)
def inputs(name: str, canary: bool = False):
    return make_inputs(CONFIGS[name], canary=canary)


@functools.lru_cache(maxsize=4)
def storage_order(name: str):
    """The oracle's storage order of the config (identity for frame-major configs)."""
    c = CONFIGS[name]
    return oracle.cuboid_order(c.T, c.H, c.W, c.cuboid)


@functools.lru_cache(maxsize=4)
def stored_inputs(name: str):
    """(q, k, v) of the config moved into its storage order by the oracle."""
    inp = inputs(name)
    o = storage_order(name)
    return tuple(oracle.permute_tokens(x, o) for x in (inp.q, inp.k, inp.v))


@functools.lru_cache(maxsize=4)
def oracle_csr(name: str):
    c = CONFIGS[name]
    if tuple(c.cuboid) != (0, 0, 0):
        q, k, _ = stored_inputs(name)
        keep = oracle.build_masks(c.T, c.H, c.W, c.block, c.specs, c.batch, q, k, order=storage_order(name))
    else:
        inp = inputs(name)
        keep = oracle.build_masks(c.T, c.H, c.W, c.block, c.specs, c.batch, inp.q, inp.k)
    return oracle.csr_from_keep(keep)


def oracle_gate(cfg, inp, device_gate=None):
    """The gate the oracle references use: the config's drawn gate, or (gate from Q) the oracle's own
    gate_from_q, never the device's.  When the device gate is given, it is checked against it (rtol 1e-5)."""
    if cfg.gate_kind == "from_q":
        g = oracle.gate_from_q(inp.q, inp.w_g, cfg.N)
    else:
        g = np.asarray(inp.gate, dtype=np.float64)
    if device_gate is not None:
        np.testing.assert_allclose(device_gate.cpu().numpy(), g, rtol=1e-5, atol=1e-6)
    return g


def device_tensors(inp, dtype=None):
    """q, k, v, w_lin as torch device tensors in the config's dtype (or the given one)."""
    import torch
    cfg = inp.cfg
    dtype = dtype or cfg.dtype
    if dtype == "bf16":
        if inp.q_bits is None:
            raise ValueError("bf16 requested for an fp32 config")

        def conv(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        return conv(inp.q_bits), conv(inp.k_bits), conv(inp.v_bits), conv(inp.w_lin_bits)

    def f(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return f(inp.q), f(inp.k), f(inp.v), f(inp.w_lin)


def to_numpy(t):
    return t.float().cpu().numpy().astype(np.float64)


def make_layer(cfg, dtype=None, specs=None):
    from block_sparse_linear_st_amd import salad as S
    from block_sparse_linear_st_amd.layer import SaladLayer
    dt = S.SALAD_BF16 if (dtype or cfg.dtype) == "bf16" else S.SALAD_F32
    return SaladLayer(cfg.batch, cfg.heads, cfg.head_dim, cfg.T, cfg.H, cfg.W, cfg.block, dt,
                      specs if specs is not None else cfg.specs, cuboid=cfg.cuboid)


def sample_blocks(cfg, n_random=12, seed=0):
    """(b, h, qb) triples: first, second, middle and last (tail) blocks of a few heads plus random ones."""
    rng = np.random.default_rng(seed)
    picks = set()
    for h in sorted({0, cfg.heads // 2, cfg.heads - 1}):
        for qb in (0, 1, cfg.nb // 2, cfg.nb - 2, cfg.nb - 1):
            picks.add((0, h, qb))
    while len(picks) < 15 + n_random:
        picks.add((int(rng.integers(cfg.batch)), int(rng.integers(cfg.heads)), int(rng.integers(cfg.nb))))
    return sorted(picks)
