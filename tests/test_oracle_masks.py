"""Pins for the oracle's block masks (CPU only).

Each test checks the oracle against something other than itself: hand-worked
fixtures, token-level brute force, a pure-Python sort, closed-form counts, or
structural invariants.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import masks as om
from synth import CONFIGS, HeadSpec, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rows(keep2d):
    return [np.nonzero(r)[0].tolist() for r in keep2d]


# ------------------------------------------------------------ window: hand-worked fixtures

@pytest.mark.parametrize("case", _load("window_mask_hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_window_hand_cases(case):
    for method in (om.window_rstar_bruteforce, om.window_rstar_segments):
        rs = method(case["T"], case["H"], case["W"], case["block"], case["t_window"])
        keep = om.window_select(rs, case["r_max"], case["density"])
        assert _rows(keep) == case["rows"], method.__name__


# ------------------------------------------------------------ window: r* segment form vs brute force

TINY_GRIDS = [
    (3, 5, 7, 16, 0), (3, 5, 7, 16, 1), (2, 3, 11, 8, 1), (5, 4, 6, 32, 2), (4, 6, 9, 13, 1),
    (1, 7, 7, 5, 0), (6, 2, 3, 4, 3), (3, 9, 10, 64, 1), (2, 16, 5, 24, 1),
]


@pytest.mark.parametrize("grid", TINY_GRIDS)
def test_rstar_segments_equal_bruteforce_tiny(grid):
    T, H, W, block, tw = grid
    a = om.window_rstar_bruteforce(T, H, W, block, tw)
    b = om.window_rstar_segments(T, H, W, block, tw)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_rstar_segments_equal_bruteforce_small_configs(name):
    c = CONFIGS[name]
    for tw in (0, 1, 2):
        np.testing.assert_array_equal(om.window_rstar_bruteforce(c.T, c.H, c.W, c.block, tw),
                                      om.window_rstar_segments(c.T, c.H, c.W, c.block, tw))


@pytest.mark.parametrize("name,tw", [("c3", 1), ("c5", 2)])
def test_rstar_segments_equal_bruteforce_sampled_rows_large(name, tw):
    c = CONFIGS[name]
    seg = om.window_rstar_segments(c.T, c.H, c.W, c.block, tw)
    rows = [0, 1, 37, c.nb // 2, c.nb - 2, c.nb - 1]
    brute = om.window_rstar_bruteforce(c.T, c.H, c.W, c.block, tw, qblocks=rows)
    np.testing.assert_array_equal(seg[rows], brute)


# ------------------------------------------------------------ window: selection vs brute-force sort

def _python_window_select(rs, r_max, density):
    nb = rs.shape[0]
    cands = [(int(q != k), int(rs[q, k]), abs(q - k), q, k)
             for q in range(nb) for k in range(nb)
             if rs[q, k] < om.RSTAR_INF and (r_max < 0 or rs[q, k] <= r_max)]
    if density <= 0:
        chosen = cands
    else:
        K = math.floor(float(np.float32(density)) * nb * nb + 0.5)
        chosen = sorted(cands)[:K]
    keep = np.zeros(rs.shape, dtype=bool)
    for c in chosen:
        keep[c[3], c[4]] = True
    return keep


@pytest.mark.parametrize("density,r_max", [(0.10, -1), (0.05, -1), (0.20, 5), (0.0, 3), (0.02, -1)])
def test_window_select_equals_python_sort_c2(density, r_max):
    c = CONFIGS["c2"]
    rs = om.window_rstar_bruteforce(c.T, c.H, c.W, c.block, 1)
    if density > 0 and om.window_count(density, c.nb, c.nb) > np.sum((rs < om.RSTAR_INF) & ((rs <= r_max) | (r_max < 0))):
        with pytest.raises(om.InfeasibleMask):
            om.window_select(rs, r_max, density)
        return
    np.testing.assert_array_equal(om.window_select(rs, r_max, density), _python_window_select(rs, r_max, density))


def test_window_c2_closed_form_counts():
    # 64-token blocks are 4 rows of a 16x16 frame.  r*=0 needs overlapping (y, x):
    # the diagonal (32 pairs) plus the same rows one frame earlier or later
    # (2 * 7 frame pairs * 4 row-blocks = 56), 88 in all.  K = floor(0.1*1024+0.5) = 102,
    # so 14 pairs at r* = 1 are added by the (|q-k|, q, k) tie-break.
    c = CONFIGS["c2"]
    rs = om.window_rstar_segments(c.T, c.H, c.W, c.block, 1)
    assert int(np.sum(rs == 0)) == 88
    keep = om.window_select(rs, -1, 0.10)
    assert int(keep.sum()) == 102
    assert int(np.sum(keep & (rs == 0))) == 88
    assert int(np.sum(keep & (rs == 1))) == 14


def test_window_full_time_window_keeps_everything():
    T, H, W, block = 3, 5, 7, 16
    rs = om.window_rstar_segments(T, H, W, block, T)
    keep = om.window_select(rs, -1, 0.0)
    assert keep.all()


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_window_structure(name):
    c = CONFIGS[name]
    for h, sp in enumerate(c.specs):
        if sp.kind != om.WINDOW:
            continue
        rs = om.window_rstar_segments(c.T, c.H, c.W, c.block, sp.t_window)
        keep = om.window_select(rs, sp.r_max, sp.density)
        assert keep.sum() == om.window_count(sp.density, c.nb, c.nb)
        assert np.all(np.diag(keep))  # the diagonal ranks first
        rp, ci = om.csr_from_keep(keep[None, None])
        for r in range(c.nb):
            row = ci[rp[r]:rp[r + 1]]
            assert np.all(np.diff(row) > 0)
        if name == "c3":
            # exactly 90% block sparsity: K = round(0.1 * 512^2) = 26214
            assert keep.sum() == 26214
            # threshold r* <= 12 holds 26152 pairs; 62 more come from r* = 13
            assert int(np.sum(keep & (rs <= 12))) == int(np.sum(rs <= 12)) == 26152
            assert int(np.sum(keep & (rs == 13))) == 62
        break


def test_window_infeasible_raises():
    rs = om.window_rstar_segments(4, 8, 8, 64, 1)
    with pytest.raises(om.InfeasibleMask):
        om.window_select(rs, -1, 0.9)


def test_window_rmax_caps_candidates():
    c = CONFIGS["c2"]
    rs = om.window_rstar_segments(c.T, c.H, c.W, c.block, 1)
    keep = om.window_select(rs, 1, 0.0)
    np.testing.assert_array_equal(keep, rs <= 1)


# ------------------------------------------------------------ top-k

@pytest.mark.parametrize("case", _load("topk_hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_topk_hand_cases(case):
    if "q" in case:
        q = np.array(case["q"], np.float32)[None, None]
        k = np.array(case["k"], np.float32)[None, None]
        pq = om.pooled_means_f32(q, case["N"], case["block"])
        pk = om.pooled_means_f32(k, case["N"], case["block"])
        np.testing.assert_array_equal(pq[0, 0], np.array(case["pq"], np.float32))
        np.testing.assert_array_equal(pk[0, 0], np.array(case["pk"], np.float32))
        sc = om.pooled_scores_f32(pq, pk)
        np.testing.assert_array_equal(sc[0, 0], np.array(case["scores"], np.float32))
        keep = om.topk_select(sc, case["density"])
        assert _rows(keep[0, 0]) == case["rows"]
    else:
        x = np.array(case["x"], np.float32)[None, None]
        np.testing.assert_array_equal(om.pooled_means_f32(x, case["N"], case["block"])[0, 0],
                                      np.array(case["pooled"], np.float32))


def _python_pooled(x, N, block):
    n_pad, d = x.shape
    out = []
    for b in range(n_pad // block):
        row = []
        nvalid = min(block, N - b * block)
        for c in range(d):
            acc = np.float32(0.0)
            for o in range(nvalid):
                acc = np.float32(acc + np.float32(x[b * block + o, c]))
            row.append(np.float32(acc / np.float32(nvalid)))
        out.append(row)
    return np.array(out, np.float32)


def _python_scores(pq, pk):
    nbq, d = pq.shape
    out = np.zeros((nbq, pk.shape[0]), np.float32)
    for i in range(nbq):
        for j in range(pk.shape[0]):
            acc = np.float32(0.0)
            for c in range(d):
                acc = np.float32(acc + np.float32(pq[i, c] * pk[j, c]))
            out[i, j] = acc
    return out


def test_pooled_and_scores_equal_scalar_float32_loops():
    rng = np.random.default_rng(123)
    N, block, d = 45, 8, 5  # ragged tail: last block has 5 valid tokens
    x = rng.standard_normal((48, d)).astype(np.float32)
    y = rng.standard_normal((48, d)).astype(np.float32)
    pq = om.pooled_means_f32(x[None, None], N, block)[0, 0]
    pk = om.pooled_means_f32(y[None, None], N, block)[0, 0]
    np.testing.assert_array_equal(pq, _python_pooled(x, N, block))
    np.testing.assert_array_equal(pk, _python_pooled(y, N, block))
    np.testing.assert_array_equal(om.pooled_scores_f32(pq, pk), _python_scores(pq, pk))


def test_pooled_small_integers_are_exact_means():
    rng = np.random.default_rng(7)
    x = rng.integers(-8, 9, size=(1, 2, 64, 3)).astype(np.float32)
    pooled = om.pooled_means_f32(x, 60, 16)
    exact = np.stack([x[:, :, b * 16:min(60, b * 16 + 16)].astype(np.float64).mean(axis=2) for b in range(4)], axis=2)
    np.testing.assert_allclose(pooled, exact, rtol=2 ** -23, atol=0)


def test_topk_equals_python_sort_and_ties_go_low():
    rng = np.random.default_rng(5)
    sc = rng.integers(0, 6, size=(3, 17, 17)).astype(np.float32)  # many ties
    for density in (0.1, 0.3, 0.5, 1.0, 0.001):
        keep = om.topk_select(sc, density)
        k = om.topk_count(density, 17)
        for a in range(3):
            for i in range(17):
                order = sorted(range(17), key=lambda j: (-float(sc[a, i, j]), j))[:k]
                assert sorted(order) == np.nonzero(keep[a, i])[0].tolist()


def test_topk_negative_zero_ties_positive_zero():
    sc = np.array([[[-0.0, 0.0, -1.0]]], np.float32)
    keep = om.topk_select(sc, 0.34)  # k = 1
    assert np.nonzero(keep[0, 0])[0].tolist() == [0]


def test_topk_all_blocks_and_dominant_block():
    c = CONFIGS["c2"]
    inp = make_inputs(c)
    pq = om.pooled_means_f32(inp.q, c.N, c.block)
    pk = om.pooled_means_f32(inp.k, c.N, c.block).copy()
    assert om.topk_select(om.pooled_scores_f32(pq, pk), 1.0).all()
    # with every pooled query positive, a key block of large positive means wins every row
    pq_pos = om.pooled_means_f32(np.abs(inp.q) + np.float32(0.1), c.N, c.block)
    pk[:, :, 7, :] = 1e3
    keep = om.topk_select(om.pooled_scores_f32(pq_pos, pk), 1.0 / c.nb)
    assert keep[..., 7].all() and keep.sum() == c.batch * c.heads * c.nb


def test_topk_count_rounding_uses_float32_density():
    # 0.1 as float32 is 0.100000001490116..., 0.1f * 512 = 51.2000008 -> 51
    assert om.topk_count(0.10, 512) == 51
    assert om.window_count(0.10, 512, 512) == 26214
    assert om.topk_count(0.0, 100) == 1
    assert om.topk_count(2.0, 100) == 100


# ------------------------------------------------------------ gate

def test_gate_special_cases():
    q = np.ones((1, 3, 10, 4), np.float32)
    q[:, :, 8:] = 99.0  # padding is ignored
    assert np.allclose(om.gate_from_q(q, np.zeros(4, np.float32), 8), 0.5)
    w = np.array([0.25, 0, 0, 0], np.float32)
    assert np.allclose(om.gate_from_q(q, w, 8), 1.0 / (1.0 + math.exp(-0.25)))
    q2 = q.copy()
    q2[0, 1, :8, 0] = np.arange(8)  # mean 3.5
    g = om.gate_from_q(q2, w, 8)
    assert abs(g[1] - 1.0 / (1.0 + math.exp(-0.875))) < 1e-15


# ------------------------------------------------------------ CSR plumbing and multi-head build

def test_csr_round_trip():
    rng = np.random.default_rng(3)
    keep = rng.random((2, 3, 5, 6)) < 0.4
    rp, ci = om.csr_from_keep(keep)
    assert rp.dtype == np.int32 and ci.dtype == np.int32 and rp[0] == 0 and rp[-1] == keep.sum()
    np.testing.assert_array_equal(om.keep_from_csr(rp, ci, 2, 3, 5, 6), keep)


def test_build_masks_mixed_heads_c5_like_small():
    specs = [HeadSpec(om.WINDOW, 1, -1, 0.2), HeadSpec(om.TOPK, 0, -1, 0.25)]
    T, H, W, block = 3, 6, 7, 16
    N = T * H * W
    nb = -(-N // block)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 2, nb * block, 8)).astype(np.float32)
    k = rng.standard_normal((2, 2, nb * block, 8)).astype(np.float32)
    keep = om.build_masks(T, H, W, block, specs, 2, q, k)
    rs = om.window_rstar_bruteforce(T, H, W, block, 1)
    np.testing.assert_array_equal(keep[0, 0], om.window_select(rs, -1, 0.2))
    np.testing.assert_array_equal(keep[1, 0], keep[0, 0])
    assert np.all(keep[:, 1].sum(axis=-1) == om.topk_count(0.25, nb))
    pq = om.pooled_means_f32(q, N, block)
    pk = om.pooled_means_f32(k, N, block)
    for b in range(2):
        np.testing.assert_array_equal(keep[b, 1], om.topk_select(_python_scores(pq[b, 1], pk[b, 1]), 0.25))


# ------------------------------------------------------------ SICS

def _sics_case_k(case):
    k = np.asarray(case["k"], dtype=np.float32)
    return k[None, None]  # [B=1, H=1, n_pad, d]


@pytest.mark.parametrize("case", _load("sics_hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_sics_hand_cases(case):
    s = om.sics_block_scores_f32(_sics_case_k(case), case["N"], case["block"])[0, 0]
    assert s.tolist() == [float(x) for x in case["sics"]]
    keep = om.sics_select(s, case["density"])
    assert _rows(keep) == case["rows"]


def _pairwise_cosine_sum(kblock):
    """Sum over all token pairs of cos(k_i, k_j), fp64, pair by pair (zero vectors contribute 0)."""
    kb = np.asarray(kblock, dtype=np.float64)
    tot = 0.0
    for a in kb:
        na = math.sqrt(float(a @ a))
        for b in kb:
            nb_ = math.sqrt(float(b @ b))
            if na > 0 and nb_ > 0:
                tot += float(a @ b) / (na * nb_)
    return tot


@pytest.mark.parametrize("N,block,d", [(12, 4, 8), (10, 4, 8), (7, 3, 5)])
def test_sics_equals_pairwise_cosine_sum(N, block, d):
    rng = np.random.default_rng(1234 + N)
    nb = -(-N // block)
    k = rng.standard_normal((1, 2, nb * block, d)).astype(np.float32)
    k[:, :, N:] = 1e4  # padding must not count
    s = om.sics_block_scores_f32(k, N, block)
    for h in range(2):
        for b in range(nb):
            toks = k[0, h, b * block:min((b + 1) * block, N)]
            ref = _pairwise_cosine_sum(toks)
            n = toks.shape[0]
            assert abs(float(s[0, h, b]) - ref) <= 1e-5 * n * n, (h, b, float(s[0, h, b]), ref)


def test_sics_closed_forms():
    d, n = 16, 8
    rng = np.random.default_rng(7)
    v = rng.standard_normal(d).astype(np.float32)
    scales = rng.uniform(0.5, 4.0, size=n).astype(np.float32)
    parallel = (scales[:, None] * v[None, :]).astype(np.float32)
    ortho = np.eye(d, dtype=np.float32)[:n] * np.float32(3.0)
    opposite = np.stack([v, -2 * v] * (n // 2)).astype(np.float32)
    k = np.concatenate([parallel, ortho, opposite])[None, None]
    s = om.sics_block_scores_f32(k, 3 * n, n)[0, 0]
    assert abs(s[0] - n * n) <= 1e-4 * n * n  # all agree: n^2
    assert s[1] == n  # orthonormal directions: only the n self-pairs
    assert abs(s[2]) <= 1e-5  # pairs cancel: 0


def test_sics_select_structure_and_ties():
    rng = np.random.default_rng(3)
    scores = rng.integers(0, 5, size=40).astype(np.float32)  # many ties
    for density in (0.05, 0.1, 0.3, 1.0):
        keep = om.sics_select(scores, density)
        m = om.topk_count(density, 40)
        top = sorted(range(40), key=lambda j: (-scores[j], j))[:m]
        for q in range(40):
            expect = sorted(set(top) | {q})
            assert np.nonzero(keep[q])[0].tolist() == expect
    # -0 ranks like +0
    z = np.array([0.0, -0.0, 1.0, -0.0], dtype=np.float32)
    assert om.sics_select(z, 0.5)[3].tolist() == [True, False, True, True]


def test_sics_planted_mistakes_are_caught():
    case = _load("sics_hand_cases.json")["cases"][0]
    k = _sics_case_k(case)
    # forgetting the normalisation (sum of raw dot products) breaks the hand values
    raw = np.asarray(k[0, 0], dtype=np.float64).reshape(3, 2, 2).sum(axis=1)
    assert ((raw ** 2).sum(axis=1)).tolist() != case["sics"]
    # summing cosines over distinct pairs only (no self pairs) breaks them too
    s = om.sics_block_scores_f32(k, case["N"], case["block"])[0, 0]
    assert (s - 2).tolist() != case["sics"]


def test_build_masks_sics_heads():
    specs = [HeadSpec(2, 0, -1, 0.1), HeadSpec(0, 1, -1, 0.1), HeadSpec(2, 0, -1, 0.25)]
    rng = np.random.default_rng(11)
    T, H, W, block = 4, 8, 8, 32
    N = T * H * W
    k = rng.standard_normal((2, 3, N, 16)).astype(np.float32)
    q = rng.standard_normal((2, 3, N, 16)).astype(np.float32)
    keep = om.build_masks(T, H, W, block, specs, 2, q, k)
    s = om.sics_block_scores_f32(k, N, block)
    for b in range(2):
        for h in (0, 2):
            assert np.array_equal(keep[b, h], om.sics_select(s[b, h], specs[h].density))
        # diagonal always kept, every row m or m + 1 blocks
        m = om.topk_count(0.1, N // block)
        counts = keep[b, 0].sum(axis=1)
        assert set(counts.tolist()) <= {m, m + 1} and keep[b, 0].diagonal().all()
