"""Pins for the oracle's attention arithmetic (CPU only).

The oracle is checked against: hand-worked fixtures, a library routine in a
special case (torch's scaled_dot_product_attention on the CPU in fp64 when every
block is kept, or per block for a block-diagonal mask), closed-form identities
(linear vs quadratic form of the ReLU branch, constant V), invariants, and a
pure-Python brute force on a tiny layer.  The last tests plant mistakes in a
copy of the oracle and check that these pins catch each of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
from oracle import masks as om
from synth import CONFIGS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLDEN, "attention_hand_cases.json")) as f:
        return json.load(f)["cases"]


def _t(a):
    return np.asarray(a, np.float64)[None, None]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    if "expect_sparse" in case:
        o = oracle.sparse_attention(_t(case["q"]), _t(case["k"]), _t(case["v"]),
                                    np.array(case["row_ptr"]), np.array(case["col_idx"]),
                                    case["N"], case["block"], case["scale"])
        np.testing.assert_allclose(o[0, 0], np.array(case["expect_sparse"], float), rtol=0, atol=case["tol"])
    if "expect_linear" in case:
        o = oracle.linear_attention(_t(case["q"]), _t(case["k"]), _t(case["v"]), case["N"], case["eps"])
        np.testing.assert_allclose(o[0, 0, case["query_row"]], case["expect_linear"], rtol=0, atol=case["tol"])
    if "expect_out" in case:
        o = oracle.mix(_t([case["o_s"]]), _t([case["o_l"]]), np.array([case["gate"]]),
                       np.array(case["w_lin"], float), N=1)
        np.testing.assert_allclose(o[0, 0, 0], case["expect_out"], rtol=0, atol=case["tol"])


# ------------------------------------------------------------ helpers

def _rand_layer(seed, B=1, Hh=2, T=2, H=3, W=5, block=8, d=16):
    rng = np.random.default_rng(seed)
    N = T * H * W
    nb = -(-N // block)
    shape = (B, Hh, nb * block, d)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    return q, k, v, N, nb


def _all_kept(B, Hh, nb):
    return om.csr_from_keep(np.ones((B, Hh, nb, nb), bool))


def _sdpa(q, k, v, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()


# ------------------------------------------------------------ sparse branch pins

def test_all_kept_equals_full_attention_sdpa():
    q, k, v, N, nb = _rand_layer(0)
    rp, ci = _all_kept(1, 2, nb)
    scale = 1 / math.sqrt(q.shape[-1])
    o = oracle.sparse_attention(q, k, v, rp, ci, N, 8)
    ref = _sdpa(q[:, :, :N], k[:, :, :N], v[:, :, :N], scale)
    np.testing.assert_allclose(o[:, :, :N], ref, rtol=0, atol=1e-12)
    assert np.all(o[:, :, N:] == 0)


def test_all_kept_equals_direct_softmax_formula_c1():
    inp = make_inputs(CONFIGS["c1"])
    c = inp.cfg
    rp, ci = _all_kept(1, c.heads, c.nb)
    o = oracle.sparse_attention(inp.q, inp.k, inp.v, rp, ci, c.N, c.block)
    for h in range(c.heads):
        qf, kf, vf = (x[0, h, :c.N].astype(np.float64) for x in (inp.q, inp.k, inp.v))
        s = qf @ kf.T / math.sqrt(c.head_dim)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (e / e.sum(axis=1, keepdims=True)) @ vf
        np.testing.assert_allclose(o[0, h, :c.N], ref, rtol=0, atol=1e-12)


def test_block_diagonal_mask_is_independent_block_attention():
    q, k, v, N, nb = _rand_layer(1, T=3, H=4, W=6, block=13)  # N=72, nb=6, tail block has 7 valid
    keep = np.zeros((1, 2, nb, nb), bool)
    for i in range(nb):
        keep[:, :, i, i] = True
    rp, ci = om.csr_from_keep(keep)
    o = oracle.sparse_attention(q, k, v, rp, ci, N, 13)
    scale = 1 / math.sqrt(q.shape[-1])
    for i in range(nb):
        a, b = i * 13, min(N, i * 13 + 13)
        ref = _sdpa(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], scale)
        np.testing.assert_allclose(o[:, :, a:b], ref, rtol=0, atol=1e-12)


def test_probability_rows_sum_to_one_and_vanish_outside_kept_blocks():
    # V = identity over the N valid keys turns o_s into the probability rows themselves.
    T, H, W, block = 2, 3, 5, 8
    N = T * H * W
    nb = -(-N // block)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, nb * block, 8))
    k = rng.standard_normal((1, 1, nb * block, 8))
    v = np.zeros((1, 1, nb * block, N))
    v[0, 0, :N] = np.eye(N)
    keep = rng.random((1, 1, nb, nb)) < 0.5
    keep[0, 0, np.arange(nb), np.arange(nb)] = True
    rp, ci = om.csr_from_keep(keep)
    p = oracle.sparse_attention(q, k, v, rp, ci, N, block)[0, 0, :N]
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    for i in range(N):
        allowed = np.zeros(N, bool)
        for kb in np.nonzero(keep[0, 0, i // block])[0]:
            allowed[kb * block:min(N, kb * block + block)] = True
        assert np.all(p[i, ~allowed] == 0) and np.all(p[i, allowed] > 0)


def test_constant_v_and_permuted_kept_lists():
    q, k, v, N, nb = _rand_layer(3)
    rng = np.random.default_rng(4)
    keep = rng.random((1, 2, nb, nb)) < 0.6
    keep[0, :, np.arange(nb), np.arange(nb)] = True
    rp, ci = om.csr_from_keep(keep)
    vc = np.full_like(v, 2.5)
    o = oracle.sparse_attention(q, k, vc, rp, ci, N, 8)
    np.testing.assert_allclose(o[:, :, :N], 2.5, rtol=0, atol=1e-13)
    ci_perm = ci.copy()
    for r in range(len(rp) - 1):
        seg = ci_perm[rp[r]:rp[r + 1]]
        ci_perm[rp[r]:rp[r + 1]] = seg[rng.permutation(seg.size)]
    np.testing.assert_allclose(oracle.sparse_attention(q, k, v, rp, ci_perm, N, 8),
                               oracle.sparse_attention(q, k, v, rp, ci, N, 8), rtol=0, atol=1e-14)


def test_single_block_with_equal_keys_gives_block_mean_of_v():
    q, k, v, N, nb = _rand_layer(5)
    k = k.copy()
    k[:, :, 8:16] = k[:, :, 8:9]  # every key of block 1 equal
    keep = np.zeros((1, 2, nb, nb), bool)
    keep[..., 1] = True
    rp, ci = om.csr_from_keep(keep)
    o = oracle.sparse_attention(q, k, v, rp, ci, N, 8)
    np.testing.assert_allclose(o[:, :, :N], np.broadcast_to(v[:, :, 8:16].mean(axis=2, keepdims=True), o[:, :, :N].shape),
                               rtol=0, atol=1e-13)


def test_padding_is_ignored_canary():
    c = CONFIGS["c1"]
    # a ragged variant of c1's grid: 4x8x7 tokens in 64-token blocks leaves 32 padded slots
    T, H, W, block = 4, 8, 7, 64
    N = T * H * W
    nb = -(-N // block)
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, nb * block, 16)) for _ in range(3))
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, :, N:] = 1e4
    rp, ci = _all_kept(1, 2, nb)
    w = rng.standard_normal((16, 16))
    g = np.array([0.2, 0.3])
    a = oracle.layer_forward(q, k, v, rp, ci, g, w, N, block, 1e-6)
    b = oracle.layer_forward(q2, k2, v2, rp, ci, g, w, N, block, 1e-6)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
        assert np.all(x[:, :, N:] == 0)


def _python_bruteforce(q, k, v, keep, N, block, scale, eps, gate, w):
    """Triple loops in plain Python floats, for a tiny layer."""
    Hh, d = q.shape[1], q.shape[-1]
    out = np.zeros((Hh, N, d))
    for h in range(Hh):
        for i in range(N):
            logits = []
            for j in range(N):
                if keep[0, h, i // block, j // block]:
                    logits.append((j, scale * sum(q[0, h, i, c] * k[0, h, j, c] for c in range(d))))
            m = max(s for _, s in logits)
            ws = [(j, math.exp(s - m)) for j, s in logits]
            tot = sum(e for _, e in ws)
            os_ = [sum(e * v[0, h, j, c] for j, e in ws) / tot for c in range(d)]
            a = [sum(max(q[0, h, i, c], 0.0) * max(k[0, h, j, c], 0.0) for c in range(d)) for j in range(N)]
            den = sum(a) + eps
            ol = [sum(a[j] * v[0, h, j, c] for j in range(N)) / den for c in range(d)]
            for e in range(d):
                out[h, i, e] = os_[e] + gate[h] * sum(ol[c] * w[c, e] for c in range(d))
    return out


def test_pure_python_bruteforce_tiny_layer():
    T, H, W, block, d = 2, 2, 5, 4, 3  # N=20, 5 blocks
    N = T * H * W
    nb = N // block
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    keep = rng.random((1, 2, nb, nb)) < 0.5
    keep[0, :, np.arange(nb), np.arange(nb)] = True
    rp, ci = om.csr_from_keep(keep)
    w = rng.standard_normal((d, d))
    g = np.array([0.7, 0.15])
    out, _, _ = oracle.layer_forward(q, k, v, rp, ci, g, w, N, block, 1e-3, scale=0.4)
    np.testing.assert_allclose(out[0], _python_bruteforce(q, k, v, keep, N, block, 0.4, 1e-3, g, w), rtol=0, atol=1e-12)


# ------------------------------------------------------------ linear branch pins

def test_linear_quadratic_equals_linear_form():
    inp = make_inputs(CONFIGS["c1"])
    c = inp.cfg
    ol = oracle.linear_attention(inp.q, inp.k, inp.v, c.N, c.eps)
    S, z = oracle.linear_state(inp.k, inp.v, c.N)
    ol2 = oracle.linear_attention_from_state(inp.q, S, z, c.N, c.eps)
    assert np.max(np.abs(ol - ol2)) <= 1e-10 * np.max(np.abs(ol))


def test_linear_closed_forms():
    q, k, v, N, nb = _rand_layer(9)
    eps = 0.25
    vc = np.full_like(v, -1.5)
    ol = oracle.linear_attention(q, k, vc, N, eps)
    Z = np.einsum("bhnc,bhc->bhn", np.maximum(q[:, :, :N], 0), np.maximum(k[:, :, :N], 0).sum(axis=2))
    np.testing.assert_allclose(ol[:, :, :N], (-1.5 * Z / (Z + eps))[..., None] * np.ones(q.shape[-1]), rtol=1e-13, atol=0)
    # queries with no positive entry see nothing through ReLU
    qn = -np.abs(q)
    assert np.all(oracle.linear_attention(qn, k, v, N, eps) == 0)
    # one valid key with positive features: o_l = v_j * Z / (Z + eps)
    ol1 = oracle.linear_attention(np.abs(q), np.abs(k), v, 1, 0.0)
    np.testing.assert_allclose(ol1[:, :, 0], v[:, :, 0], rtol=1e-14, atol=0)


def test_linear_state_matches_explicit_sums():
    q, k, v, N, nb = _rand_layer(10)
    S, z = oracle.linear_state(k, v, N)
    for h in range(2):
        Sh = sum(np.outer(np.maximum(k[0, h, j], 0), v[0, h, j]) for j in range(N))
        np.testing.assert_allclose(S[0, h], Sh, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(z[0, h], np.maximum(k[0, h, :N], 0).sum(axis=0), rtol=1e-14)


# ------------------------------------------------------------ mix pins

def test_mix_reductions():
    q, k, v, N, nb = _rand_layer(11)
    rp, ci = _all_kept(1, 2, nb)
    d = q.shape[-1]
    w = np.random.default_rng(0).standard_normal((d, d))
    out0, os_, ol = oracle.layer_forward(q, k, v, rp, ci, np.zeros(2), w, N, 8, 1e-6)
    np.testing.assert_array_equal(out0[:, :, :N], os_[:, :, :N])
    outw, _, _ = oracle.layer_forward(q, k, v, rp, ci, np.array([0.3, 0.9]), np.zeros((d, d)), N, 8, 1e-6)
    np.testing.assert_array_equal(outw[:, :, :N], os_[:, :, :N])
    outi, _, _ = oracle.layer_forward(q, k, v, rp, ci, np.ones(2), np.eye(d), N, 8, 1e-6)
    np.testing.assert_allclose(outi[:, :, :N], os_[:, :, :N] + ol[:, :, :N], rtol=0, atol=1e-14)
    outd, _, _ = oracle.layer_forward(q, k, v, rp, ci, np.array([0.05, 0.5]), w, N, 8, 1e-6, drop_tau=0.1)
    np.testing.assert_array_equal(outd[:, 0, :N], os_[:, 0, :N])
    np.testing.assert_allclose(outd[:, 1, :N], os_[:, 1, :N] + 0.5 * ol[:, 1, :N] @ w, rtol=0, atol=1e-14)


def test_sampled_blocks_equal_full_forward():
    inp = make_inputs(CONFIGS["c2"])
    c = inp.cfg
    keep = oracle.build_masks(c.T, c.H, c.W, c.block, c.specs, c.batch)
    rp, ci = om.csr_from_keep(keep)
    full = oracle.layer_forward(inp.q[:, :2], inp.k[:, :2], inp.v[:, :2], *_sub_csr(keep[:, :2]),
                                inp.gate[:2], inp.w_lin, c.N, c.block, c.eps)
    picks = [(0, 0, 0), (0, 1, 17), (0, 1, c.nb - 1)]
    samp = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, c.N, c.block, c.eps, qblocks=picks)
    for x, y in zip(full, samp):
        for idx, (b, h, qb) in enumerate(picks):
            np.testing.assert_allclose(y[idx], x[b, h, qb * c.block:(qb + 1) * c.block], rtol=0, atol=1e-13)


def _sub_csr(keep):
    return om.csr_from_keep(keep)


# ------------------------------------------------------------ planted mistakes are caught

def _planted(monkeypatch, kind):
    if kind == "mask_ignored":
        orig = oa._sparse_block

        def bad(qf, kf, vf, kept, qb, N, block, scale):
            return orig(qf, kf, vf, np.arange(-(-N // block)), qb, N, block, scale)
        monkeypatch.setattr(oa, "_sparse_block", bad)
    elif kind == "scale_dropped":
        orig = oa._sparse_block
        monkeypatch.setattr(oa, "_sparse_block", lambda qf, kf, vf, kept, qb, N, block, scale:
                            orig(qf, kf, vf, kept, qb, N, block, 1.0))
    elif kind == "relu_on_values":
        orig = oa.linear_attention

        def bad(q, k, v, N, eps, block=None, qblocks=None):
            return orig(q, k, np.maximum(v, 0), N, eps, block, qblocks)
        monkeypatch.setattr(oa, "linear_attention", bad)
        monkeypatch.setattr(oracle, "linear_attention", bad)
    elif kind == "w_transposed":
        orig = oa.mix

        def bad(o_s, o_l, gate, w_lin, **kw):
            return orig(o_s, o_l, gate, np.asarray(w_lin).T, **kw)
        monkeypatch.setattr(oa, "mix", bad)
        monkeypatch.setattr(oracle, "mix", bad)
    elif kind == "eps_dropped":
        orig = oa.linear_attention

        def bad(q, k, v, N, eps, block=None, qblocks=None):
            return orig(q, k, v, N, 0.0, block, qblocks)
        monkeypatch.setattr(oa, "linear_attention", bad)
        monkeypatch.setattr(oracle, "linear_attention", bad)


@pytest.mark.parametrize("kind", ["mask_ignored", "scale_dropped", "relu_on_values", "w_transposed", "eps_dropped"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    _planted(monkeypatch, kind)
    failures = 0
    for fn in (test_block_diagonal_mask_is_independent_block_attention, test_all_kept_equals_full_attention_sdpa,
               test_linear_closed_forms, test_pure_python_bruteforce_tiny_layer):
        try:
            fn()
        except AssertionError:
            failures += 1
    for case in _cases():
        try:
            test_hand_cases(case)
        except AssertionError:
            failures += 1
    assert failures > 0, f"planted mistake '{kind}' went unnoticed"
