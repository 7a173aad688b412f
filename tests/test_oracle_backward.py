"""Pins for the oracle's layer gradients (CPU only).

The gradients come from torch autograd on a second, torch-written copy of the
forward.  They are pinned to things that do not go through that copy:
central finite differences of the NumPy forward (``oracle.layer_forward``),
torch's own scaled-dot-product-attention backward for an all-kept mask, the
closed forms of dW_lin and dgate from the NumPy forward's o_l, and a
hand-derived chain rule for the linear branch written on its linear form
(S = ReLU(K)^T V, z = sum ReLU(k)).
"""

import numpy as np
import pytest

import oracle
from oracle import backward as ob

torch = pytest.importorskip("torch")


def _tiny(seed=0, B=1, Hh=2, T=1, H=5, W=5, block=8, d=4, density=0.6, empty_row=True):
    rng = np.random.default_rng(seed)
    N = T * H * W
    nb = -(-N // block)
    n_pad = nb * block
    q = rng.standard_normal((B, Hh, n_pad, d))
    k = rng.standard_normal((B, Hh, n_pad, d))
    v = rng.standard_normal((B, Hh, n_pad, d))
    q[:, :, N:] = 7.0  # padding must not matter
    k[:, :, N:] = -3.0
    v[:, :, N:] = 5.0
    keep = rng.random((B, Hh, nb, nb)) < density
    keep[..., np.arange(nb), np.arange(nb)] = True
    if empty_row:
        keep[0, 0, 1] = False
    rp, ci = oracle.csr_from_keep(keep)
    gate = rng.uniform(0.1, 0.9, size=B * Hh)
    w = rng.standard_normal((d, d)) / np.sqrt(d)
    dout = rng.standard_normal((B, Hh, n_pad, d))
    return dict(q=q, k=k, v=v, rp=rp, ci=ci, gate=gate, w=w, N=N, block=block, eps=1e-3, dout=dout)


def _loss(c, **over):
    a = dict(c)
    a.update(over)
    out, _, _ = oracle.layer_forward(a["q"], a["k"], a["v"], a["rp"], a["ci"], a["gate"], a["w"], a["N"],
                                     a["block"], a["eps"])
    return float(np.sum(out[:, :, :a["N"]] * a["dout"][:, :, :a["N"]]))


def _grads(c):
    return ob.layer_backward(c["q"], c["k"], c["v"], c["rp"], c["ci"], c["gate"], c["w"], c["N"], c["block"],
                             c["eps"], c["dout"])


@pytest.mark.parametrize("seed", [0, 1])
def test_forward_copy_matches_numpy_forward(seed):
    c = _tiny(seed)
    g = _grads(c)
    out, o_s, o_l = oracle.layer_forward(c["q"], c["k"], c["v"], c["rp"], c["ci"], c["gate"], c["w"], c["N"],
                                         c["block"], c["eps"])
    np.testing.assert_allclose(g["out"], out, atol=1e-12)
    np.testing.assert_allclose(g["o_s"], o_s, atol=1e-12)
    np.testing.assert_allclose(g["o_l"][:, :, :c["N"]], o_l[:, :, :c["N"]], atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["q", "k", "v", "w", "gate"])
def test_directional_finite_differences(seed, name):
    """<grad, E> against (L(x + hE) - L(x - hE)) / 2h along random directions, the NumPy forward as L."""
    c = _tiny(seed)
    g = _grads(c)
    grad = {"q": g["dq"], "k": g["dk"], "v": g["dv"], "w": g["dw_lin"], "gate": g["dgate"]}[name]
    rng = np.random.default_rng(100 + seed)
    x = c[name]
    for _ in range(3):
        E = rng.standard_normal(x.shape)
        h = 1e-6
        fd = (_loss(c, **{name: x + h * E}) - _loss(c, **{name: x - h * E})) / (2 * h)
        an = float(np.sum(grad * E))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_padding_rows_get_no_gradient():
    c = _tiny(3)
    g = _grads(c)
    for n in ("dq", "dk", "dv"):
        assert np.all(g[n][:, :, c["N"]:] == 0.0)


def test_sparse_part_matches_torch_sdpa_all_kept():
    """Gate 0 leaves the sparse branch: for an all-kept mask its gradients are SDPA's."""
    c = _tiny(4, empty_row=False, density=1.1)
    c["gate"] = np.zeros_like(c["gate"])
    g = _grads(c)
    N = c["N"]
    qt, kt, vt = (torch.tensor(c[n][:, :, :N], requires_grad=True) for n in ("q", "k", "v"))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    (o * torch.from_numpy(c["dout"][:, :, :N])).sum().backward()
    np.testing.assert_allclose(g["dq"][:, :, :N], qt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"][:, :, :N], kt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"][:, :, :N], vt.grad.numpy(), atol=1e-12)
    assert np.all(g["dw_lin"] == 0.0)


def test_dw_and_dgate_closed_forms():
    """dW = sum over heads of g * o_l^T dout; dgate = <dout, o_l W> per head (o_l from the NumPy forward)."""
    c = _tiny(5)
    g = _grads(c)
    N = c["N"]
    _, _, o_l = oracle.layer_forward(c["q"], c["k"], c["v"], c["rp"], c["ci"], c["gate"], c["w"], N, c["block"],
                                     c["eps"])
    B, Hh = c["q"].shape[:2]
    dW = np.zeros_like(c["w"])
    dg = np.zeros(B * Hh)
    for b in range(B):
        for h in range(Hh):
            ol = o_l[b, h, :N]
            do = c["dout"][b, h, :N]
            dW += c["gate"][b * Hh + h] * ol.T @ do
            dg[b * Hh + h] = np.sum(do * (ol @ c["w"]))
    np.testing.assert_allclose(g["dw_lin"], dW, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dgate"], dg, rtol=1e-12, atol=1e-12)


def test_linear_branch_chain_rule_on_the_linear_form():
    """Full gradients minus the gate-0 (sparse-only) gradients equal the hand-derived linear-branch gradients.

    With phi = ReLU, u = phi(q) S, den = phi(q) z + eps, o_l = u / den and dO_l = g dout W^T:
      du = dO_l / den, dden = -<dO_l, o_l> / den, dphi(q) = S du + z dden,
      dS = sum_n phi(q_n) du_n^T, dz = sum_n phi(q_n) dden_n, dphi(k_j) = dS v_j + dz, dv_j = dS^T phi(k_j).
    """
    c = _tiny(6)
    full = _grads(c)
    c0 = dict(c)
    c0["gate"] = np.zeros_like(c["gate"])
    sparse = _grads(c0)
    N = c["N"]
    S, z = oracle.linear_state(c["k"], c["v"], N)
    B, Hh = c["q"].shape[:2]
    for b in range(B):
        for h in range(Hh):
            gv = c["gate"][b * Hh + h]
            q, k, v = (c[n][b, h, :N] for n in ("q", "k", "v"))
            pq, pk = np.maximum(q, 0), np.maximum(k, 0)
            Sb, zb = S[b, h], z[b, h]
            u = pq @ Sb
            den = pq @ zb + c["eps"]
            ol = u / den[:, None]
            dOl = gv * c["dout"][b, h, :N] @ c["w"].T
            du = dOl / den[:, None]
            dden = -np.sum(dOl * ol, axis=1) / den
            dpq = du @ Sb.T + dden[:, None] * zb[None, :]
            dq = dpq * (q > 0)
            dS = pq.T @ du
            dz = pq.T @ dden
            dpk = v @ dS.T + dz[None, :]
            dk = dpk * (k > 0)
            dv = pk @ dS
            np.testing.assert_allclose(full["dq"][b, h, :N] - sparse["dq"][b, h, :N], dq, atol=1e-11)
            np.testing.assert_allclose(full["dk"][b, h, :N] - sparse["dk"][b, h, :N], dk, atol=1e-11)
            np.testing.assert_allclose(full["dv"][b, h, :N] - sparse["dv"][b, h, :N], dv, atol=1e-11)


def test_lse2_closed_forms():
    """Equal keys: log2 of n e^l = l log2(e) + log2(n); a two-key hand case; +inf for empty rows and padding."""
    B, Hh, block, d = 1, 1, 4, 2
    N = 7
    n_pad = 8
    q = np.zeros((B, Hh, n_pad, d))
    k = np.zeros((B, Hh, n_pad, d))
    q[0, 0, :, 0] = 2.0
    k[0, 0, :, 0] = 0.5           # every logit = scale * 1.0
    keep = np.array([[[[True, True], [False, False]]]])
    rp, ci = oracle.csr_from_keep(keep)
    scale = 0.7
    got = oracle.sparse_lse2(q, k, rp, ci, N, block, scale)
    np.testing.assert_allclose(got[0, 0, :4], scale * np.log2(np.e) + np.log2(7.0), rtol=1e-13)
    assert np.all(np.isinf(got[0, 0, 4:]))  # rows of a block that keeps nothing, and the padding row
    # two keys with logits 0 and ln 3: log2(1 + 3) = 2
    q2 = np.zeros((1, 1, 2, 1)); q2[0, 0, :, 0] = 1.0
    k2 = np.zeros((1, 1, 2, 1)); k2[0, 0, 1, 0] = np.log(3.0)
    rp2, ci2 = oracle.csr_from_keep(np.ones((1, 1, 1, 1), dtype=bool))
    np.testing.assert_allclose(oracle.sparse_lse2(q2, k2, rp2, ci2, 2, 2, 1.0)[0, 0], [2.0, 2.0], rtol=1e-14)


def test_lse2_normalises_the_sparse_branch():
    """2^(x - lse2) summed over a row's kept keys is 1 (x = scale q.k log2 e)."""
    c = _tiny(7, empty_row=False)
    N, block = c["N"], c["block"]
    lse = oracle.sparse_lse2(c["q"], c["k"], c["rp"], c["ci"], N, block)
    d = c["q"].shape[-1]
    keep = ob._keep_matrix(c["rp"], c["ci"], 1, 2, -(-N // block))
    for h in range(2):
        for i in range(N):
            keys = [j for j in range(N) if keep[0, h, i // block, j // block]]
            x = (c["q"][0, h, i] @ c["k"][0, h, keys].T) / np.sqrt(d) * np.log2(np.e)
            assert abs(np.sum(2.0 ** (x - lse[0, h, i])) - 1.0) < 1e-12


@pytest.mark.parametrize("seed", [0, 3])
def test_sampled_gradients_equal_autograd(seed):
    """The closed-form sampled gradients equal the autograd ones at every block of a small layer."""
    c = _tiny(seed)
    full = _grads(c)
    B, Hh, n_pad, d = c["q"].shape
    nb = n_pad // c["block"]
    blocks = [(b, h, x) for b in range(B) for h in range(Hh) for x in range(nb)]
    s = ob.layer_backward_sampled(c["q"], c["k"], c["v"], c["rp"], c["ci"], c["gate"], c["w"], c["N"], c["block"],
                                  c["eps"], c["dout"], blocks, blocks)
    blk = c["block"]
    for idx, (b, h, x) in enumerate(blocks):
        sl = slice(x * blk, (x + 1) * blk)
        np.testing.assert_allclose(s["dq"][idx], full["dq"][b, h, sl], atol=1e-11)
        np.testing.assert_allclose(s["dk"][idx], full["dk"][b, h, sl], atol=1e-11)
        np.testing.assert_allclose(s["dv"][idx], full["dv"][b, h, sl], atol=1e-11)
    np.testing.assert_allclose(s["dw_lin"], full["dw_lin"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s["dgate"], full["dgate"], rtol=1e-11, atol=1e-12)
