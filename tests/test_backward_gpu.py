"""GPU parity of the backward pass (salad_attn_bwd) against the oracle's gradients.

The oracle differentiates the fp64 forward on the exact bf16 input values
(``oracle.layer_backward``).  The kernels round P and dS to bf16 before their
products (as the forward rounds P) and store dq, dk, dv in bf16; each rounding
is a relative 2^-9, three of them stack on a typical element (four on dK, whose
dS is formed from the bf16-rounded P), so the bars are rel-L2 <= 1.5e-2 and
max-abs <= 3e-2 * max|ref| per tensor (about 2.5x the expected error).  dW_lin and dgate are fp32 sums of bf16-rounded o_l and dU:
rel-L2 <= 1e-2.  Padding rows of dq, dk, dv must be exactly 0, and two runs
must agree bit for bit.  Both paths are checked: the softmax statistic kept by
the forward (its log2-sum-exp output, itself checked against the oracle's
definition) and the one the backward recomputes.
"""

import numpy as np
import pytest

import oracle
from helpers import (device_tensors, inputs, make_layer, oracle_csr, oracle_gate, storage_order, stored_inputs,
                     to_numpy)
from synth import CONFIGS, HeadSpec, LayerConfig, make_grad_output, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_linear_st_amd import salad as S  # noqa: E402

REL_L2 = 1.5e-2
MAX_REL = 3e-2
FP32_REL_L2 = 1e-2

B128 = LayerConfig(
    name="b128", seed=21, batch=2, heads=2, head_dim=128, T=3, H=10, W=20, block=128, dtype="bf16",
    specs=(HeadSpec(0, 1, -1, 0.5), HeadSpec(1, 0, -1, 0.4)), gate_kind="uniform",
    description="ragged 128-token blocks, d=128, batch 2: window and top-k heads")


def _check(got, ref, what, rel_l2=REL_L2, max_rel=MAX_REL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    rl2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"{what}: max-abs {err:.3e} (bar {max_rel * scale:.3e}), rel-L2 {rl2:.3e} (bar {rel_l2:g})", flush=True)
    assert rl2 <= rel_l2, f"{what}: rel-L2 {rl2:.3e}"
    assert err <= max_rel * scale, f"{what}: max-abs {err:.3e}"


def _run(cfg, inp, cuboid=False):
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    if cuboid:
        qs, ks, vs = (torch.empty_like(t) for t in (q, k, v))
        layer.to_storage(q, qs)
        layer.to_storage(k, ks)
        layer.to_storage(v, vs)
        q, k, v = qs, ks, vs
    if cfg.gate_kind == "from_q":
        gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
        layer.build_mask(q, k, torch.from_numpy(inp.w_g).cuda(), gate)
    else:
        gate = torch.from_numpy(inp.gate).cuda()
        layer.build_mask(q, k)
    out = torch.empty_like(q)
    lse = torch.full((cfg.batch * cfg.heads * cfg.n_pad,), float("nan"), dtype=torch.float32, device="cuda")
    layer.forward(q, k, v, gate, w, out, eps=cfg.eps, lse=lse)
    dvals, dbits = make_grad_output(cfg)
    dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    ws = torch.empty(S.salad_bwd_workspace_bytes(layer.shape), dtype=torch.uint8, device="cuda")
    res = []
    for lse_arg in (lse, lse, None):  # forward's statistic twice (determinism), then recomputed
        g = {n: torch.full_like(q, float("nan")) for n in ("dq", "dk", "dv")}
        dw = torch.full((cfg.head_dim, cfg.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        dg = torch.full((cfg.batch * cfg.heads,), float("nan"), dtype=torch.float32, device="cuda")
        S.salad_attn_bwd(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, w, cfg.eps, 0.0, out, dout,
                         g["dq"], g["dk"], g["dv"], dw, dg, ws, lse=lse_arg)
        torch.cuda.synchronize()
        g["dw"], g["dg"] = dw, dg
        res.append(g)
    for n in res[0]:
        assert torch.equal(res[0][n], res[1][n]), f"{n} differs between two runs"
    return layer, gate, res, dvals, lse.view(cfg.batch, cfg.heads, cfg.n_pad).cpu().numpy(), (q, k)


def _oracle(cfg, name_or_inp, gate, dvals, stored=None):
    inp = name_or_inp
    q, k, v = stored if stored is not None else (inp.q, inp.k, inp.v)
    if isinstance(cfg, LayerConfig) and cfg.name in CONFIGS and CONFIGS[cfg.name] is cfg:
        rp, ci = oracle_csr(cfg.name)
    else:
        keep = oracle.build_masks(cfg.T, cfg.H, cfg.W, cfg.block, cfg.specs, cfg.batch, q, k)
        rp, ci = oracle.csr_from_keep(keep)
    return oracle.layer_backward(q, k, v, rp, ci, oracle_gate(cfg, inp, gate), inp.w_lin, cfg.N,
                                 cfg.block, cfg.eps, dvals), rp, ci


def _compare_all(cfg, res, ref, lse, stored, rp, ci, tag):
    """Both backward paths against the oracle; the forward's log2-sum-exp against its definition."""
    _compare(cfg, res[0], ref, f"{tag} (forward lse)")
    _compare(cfg, res[2], ref, f"{tag} (recomputed lse)")
    want = oracle.sparse_lse2(stored[0], stored[1], rp, ci, cfg.N, cfg.block)
    N = cfg.N
    assert np.all(np.isinf(lse[:, :, N:])) and np.all(np.isfinite(lse[:, :, :N]))
    err = float(np.max(np.abs(lse[:, :, :N] - want[:, :, :N])))
    print(f"{tag} lse: max-abs {err:.3e} (bar 2e-2)", flush=True)
    assert err <= 2e-2  # probabilities summed after bf16 rounding (relative 2^-9): |log2(1 +- 2^-9)| = 2.8e-3


def _compare(cfg, got, ref, tag):
    N = cfg.N
    for n in ("dq", "dk", "dv"):
        t = to_numpy(got[n])
        _check(t[:, :, :N], ref[n][:, :, :N], f"{tag} {n}")
        assert np.all(t[:, :, N:] == 0.0), f"{tag} {n}: padding rows not zero"
    _check(got["dw"].cpu().numpy(), ref["dw_lin"], f"{tag} dW_lin", rel_l2=FP32_REL_L2)
    _check(got["dg"].cpu().numpy(), ref["dgate"], f"{tag} dgate", rel_l2=FP32_REL_L2)


def test_backward_c2():
    print("backward c2", flush=True)
    cfg = CONFIGS["c2"]
    inp = inputs("c2")
    layer, gate, res, dvals, lse, _ = _run(cfg, inp)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), oracle_csr("c2")[0])
    ref, rp, ci = _oracle(cfg, inp, gate, dvals)
    _compare_all(cfg, res, ref, lse, (inp.q, inp.k), rp, ci, "c2")


def test_backward_b128_ragged():
    print("backward b128", flush=True)
    cfg = B128
    inp = make_inputs(cfg)
    layer, gate, res, dvals, lse, _ = _run(cfg, inp)
    ref, rp, ci = _oracle(cfg, inp, gate, dvals)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    _compare_all(cfg, res, ref, lse, (inp.q, inp.k), rp, ci, "b128")


D64B128 = LayerConfig(
    name="d64b128", seed=22, batch=1, heads=3, head_dim=64, T=3, H=9, W=15, block=128, dtype="bf16",
    specs=(HeadSpec(0, 1, -1, 0.4), HeadSpec(1, 0, -1, 0.5), HeadSpec(0, 2, -1, 0.0)), gate_kind="uniform",
    description="ragged 128-token blocks at d=64 (3 blocks per head, the last one partial): window and top-k heads")


def test_backward_d64_b128_ragged():
    print("backward d64b128", flush=True)
    cfg = D64B128
    inp = make_inputs(cfg)
    layer, gate, res, dvals, lse, _ = _run(cfg, inp)
    ref, rp, ci = _oracle(cfg, inp, gate, dvals)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    _compare_all(cfg, res, ref, lse, (inp.q, inp.k), rp, ci, "d64b128")


def test_backward_c9_cuboid_mixed_masks():
    """Ragged 5x10x14 layer in cuboid order with window, top-k and SICS heads and a gate from Q."""
    print("backward c9", flush=True)
    cfg = CONFIGS["c9"]
    inp = inputs("c9")
    layer, gate, res, dvals, lse, _ = _run(cfg, inp, cuboid=True)
    stored = stored_inputs("c9")
    ref, rp, ci = _oracle(cfg, inp, gate, dvals, stored=stored)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    _compare_all(cfg, res, ref, lse, stored, rp, ci, "c9")


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_backward_sampled_large(name):
    """Full-size layers in the bench's launch configuration: sampled query blocks (dq) and key blocks (dk, dv)
    against the oracle's closed-form gradients at those blocks; dW_lin and dgate in full."""
    print(f"backward sampled {name}", flush=True)
    from helpers import sample_blocks
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer, gate, res, dvals, _, _ = _run(cfg, inp)
    rp, ci = oracle_csr(name)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    qbl = sample_blocks(cfg, n_random=8, seed=1)
    kbl = sample_blocks(cfg, n_random=4, seed=2)[::2]
    g = oracle_gate(cfg, inp, gate)
    ref = oracle.layer_backward_sampled(inp.q, inp.k, inp.v, rp, ci, g, inp.w_lin, cfg.N, cfg.block, cfg.eps,
                                        dvals, qbl, kbl)
    blk = cfg.block
    for which in (0, 2):  # forward's log2-sum-exp, recomputed
        got = res[which]
        tag = f"{name} ({'forward' if which == 0 else 'recomputed'} lse)"
        dq = np.stack([to_numpy(got["dq"][b, h, x * blk:(x + 1) * blk]) for b, h, x in qbl])
        dk = np.stack([to_numpy(got["dk"][b, h, x * blk:(x + 1) * blk]) for b, h, x in kbl])
        dv = np.stack([to_numpy(got["dv"][b, h, x * blk:(x + 1) * blk]) for b, h, x in kbl])
        _check(dq, ref["dq"], f"{tag} dq (sampled)")
        _check(dk, ref["dk"], f"{tag} dk (sampled)")
        _check(dv, ref["dv"], f"{tag} dv (sampled)")
        _check(got["dw"].cpu().numpy(), ref["dw_lin"], f"{tag} dW_lin", rel_l2=FP32_REL_L2)
        _check(got["dg"].cpu().numpy(), ref["dgate"], f"{tag} dgate", rel_l2=FP32_REL_L2)


def test_differentiable_layer_op_c2():
    """layer.attention(...) under torch autograd gives the entry points' output and gradients bit for bit, and
    its gradients meet the oracle's bars."""
    print("autograd op c2", flush=True)
    cfg = CONFIGS["c2"]
    inp = inputs("c2")
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    layer.build_mask(q, k)
    gate = torch.from_numpy(inp.gate).cuda()
    dvals, dbits = make_grad_output(cfg)
    dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()

    leaves = [t.clone().requires_grad_(True) for t in (q, k, v, gate, w)]
    out = layer.attention(*leaves, eps=cfg.eps)
    out.backward(dout)
    torch.cuda.synchronize()

    ref_out = torch.empty_like(q)
    lse = torch.empty(cfg.batch * cfg.heads * cfg.n_pad, dtype=torch.float32, device="cuda")
    layer.forward(q, k, v, gate, w, ref_out, eps=cfg.eps, lse=lse)
    g = {n: torch.empty_like(q) for n in ("dq", "dk", "dv")}
    dw = torch.empty((cfg.head_dim, cfg.head_dim), dtype=torch.float32, device="cuda")
    dg = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
    layer.backward(q, k, v, gate, w, ref_out, dout, g["dq"], g["dk"], g["dv"], dw, dg, eps=cfg.eps, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    for leaf, want in zip(leaves[:3], (g["dq"], g["dk"], g["dv"])):
        assert torch.equal(leaf.grad, want)
    assert torch.equal(leaves[3].grad, dg)
    assert torch.equal(leaves[4].grad, dw.to(torch.bfloat16))

    ref, _, _ = _oracle(cfg, inp, gate, dvals)
    N = cfg.N
    for n, leaf in zip(("dq", "dk", "dv"), leaves[:3]):
        _check(to_numpy(leaf.grad)[:, :, :N], ref[n][:, :, :N], f"autograd c2 {n}")
    _check(leaves[3].grad.cpu().numpy(), ref["dgate"], "autograd c2 dgate", rel_l2=FP32_REL_L2)


def test_autograd_op_keeps_its_forward_mask():
    """build_mask runs again (a different, sparser mask) between the autograd op's forward and its backward:
    the gradients are still those over the forward's mask, against the oracle on the oracle's CSR."""
    print("autograd op, mask rebuilt before backward", flush=True)
    from block_sparse_linear_st_amd import salad as S
    cfg = CONFIGS["c2"]
    inp = inputs("c2")
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    layer.build_mask(q, k)
    gate = torch.from_numpy(inp.gate).cuda()
    dvals, dbits = make_grad_output(cfg)
    dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v, gate, w)]
    out = layer.attention(*leaves, eps=cfg.eps)
    rp0 = layer.row_ptr.clone()
    layer.specs = S.make_specs([HeadSpec(0, 1, -1, 0.05)] * cfg.heads)
    layer.build_mask(q, k)
    torch.cuda.synchronize()
    assert not torch.equal(layer.row_ptr, rp0)
    out.backward(dout)
    torch.cuda.synchronize()
    ref, _, _ = _oracle(cfg, inp, gate, dvals)
    N = cfg.N
    for n, leaf in zip(("dq", "dk", "dv"), leaves[:3]):
        _check(to_numpy(leaf.grad)[:, :, :N], ref[n][:, :, :N], f"autograd c2 (mask rebuilt) {n}")
    _check(leaves[3].grad.cpu().numpy(), ref["dgate"], "autograd c2 (mask rebuilt) dgate", rel_l2=FP32_REL_L2)


def test_skewed_heads_hand_built_mask():
    """One dense head beside eleven diagonal-only heads, so that the run of work items each XCD takes is cut far
    from equal counts and clamped at its longest: forward, its log2-sum-exp and both backward paths against the
    oracle."""
    print("skewed heads", flush=True)
    from helpers import BF16_MAX_ABS, BF16_REL_L2, assert_close
    cfg = LayerConfig(name="skew", seed=31, batch=1, heads=12, head_dim=64, T=8, H=16, W=16, block=64,
                      dtype="bf16", specs=(HeadSpec(0, 1, -1, 0.0),) * 12, gate_kind="uniform")
    nb = cfg.nb
    keep = np.zeros((1, cfg.heads, nb, nb), bool)
    keep[0, 0] = True
    keep[0, 1:, np.arange(nb), np.arange(nb)] = True
    rp, ci = oracle.csr_from_keep(keep)
    inp = make_inputs(cfg)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    row_ptr = torch.from_numpy(rp).cuda()
    col_idx = torch.from_numpy(ci).cuda()
    gate = torch.from_numpy(inp.gate).cuda()
    out = torch.empty_like(q)
    lse = torch.full((cfg.heads * cfg.n_pad,), float("nan"), dtype=torch.float32, device="cuda")
    S.salad_attn_fwd(layer.shape, q, k, v, row_ptr, col_idx, gate, w, cfg.eps, 0.0, 0.0, out, layer.ws, lse=lse)
    torch.cuda.synchronize()
    ref_out, _, _ = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block,
                                         cfg.eps)
    assert_close(to_numpy(out), ref_out, BF16_MAX_ABS, BF16_REL_L2, "skewed forward")
    want = oracle.sparse_lse2(inp.q, inp.k, rp, ci, cfg.N, cfg.block)
    got_lse = lse.view(1, cfg.heads, cfg.n_pad).cpu().numpy()
    assert float(np.max(np.abs(got_lse[:, :, :cfg.N] - want[:, :, :cfg.N]))) <= 2e-2
    dvals, dbits = make_grad_output(cfg)
    dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    ws = torch.empty(S.salad_bwd_workspace_bytes(layer.shape), dtype=torch.uint8, device="cuda")
    ref = oracle.layer_backward(inp.q, inp.k, inp.v, rp, ci, inp.gate.astype(np.float64), inp.w_lin, cfg.N,
                                cfg.block, cfg.eps, dvals)
    for lse_arg, tag in ((lse, "forward lse"), (None, "recomputed lse")):
        g = {n: torch.full_like(q, float("nan")) for n in ("dq", "dk", "dv")}
        g["dw"] = torch.full((cfg.head_dim, cfg.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        g["dg"] = torch.full((cfg.heads,), float("nan"), dtype=torch.float32, device="cuda")
        S.salad_attn_bwd(layer.shape, q, k, v, row_ptr, col_idx, gate, w, cfg.eps, 0.0, out, dout, g["dq"],
                         g["dk"], g["dv"], g["dw"], g["dg"], ws, lse=lse_arg)
        torch.cuda.synchronize()
        _compare(cfg, g, ref, f"skewed ({tag})")


def test_union_and_own_list_layouts_backward():
    """The mixed-overlap mask of the forward layout test (scattered, banded, disjoint-neighbour and half-empty
    heads; two batches; a 54-token tail block): the dQ kernel walks the union of paired lists for some heads and
    each block's own list for others; forward, its log2-sum-exp and both backward paths against the oracle."""
    print("list layouts backward", flush=True)
    from helpers import BF16_MAX_ABS, BF16_REL_L2, assert_close
    cfg = LayerConfig(name="layouts", seed=21, batch=2, heads=4, head_dim=128, T=3, H=10, W=21, block=64,
                      dtype="bf16", specs=(HeadSpec(0, 1, -1, 0.0),) * 4, gate_kind="uniform")
    nb = cfg.nb
    rng = np.random.default_rng(5)
    keep = np.zeros((2, 4, nb, nb), dtype=bool)
    for b in range(2):
        keep[b, 0] = rng.random((nb, nb)) < 0.35
        for qb in range(nb):
            keep[b, 1, qb, max(0, qb - 2):qb + 3] = True
            keep[b, 2, qb, (qb % 2)::2] = True
        keep[b, 3, 0::2, :] = True
    rp, ci = oracle.csr_from_keep(keep)
    inp = make_inputs(cfg)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    row_ptr = torch.from_numpy(rp).cuda()
    col_idx = torch.from_numpy(ci).cuda()
    gate = torch.from_numpy(inp.gate).cuda()
    out = torch.empty_like(q)
    lse = torch.full((cfg.batch * cfg.heads * cfg.n_pad,), float("nan"), dtype=torch.float32, device="cuda")
    S.salad_attn_fwd(layer.shape, q, k, v, row_ptr, col_idx, gate, w, cfg.eps, 0.0, 0.0, out, layer.ws, lse=lse)
    torch.cuda.synchronize()
    ref_out, _, _ = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block,
                                         cfg.eps)
    assert_close(to_numpy(out), ref_out, BF16_MAX_ABS, BF16_REL_L2, "layouts forward")
    want = oracle.sparse_lse2(inp.q, inp.k, rp, ci, cfg.N, cfg.block)[:, :, :cfg.N]
    got_lse = lse.view(cfg.batch, cfg.heads, cfg.n_pad).cpu().numpy()[:, :, :cfg.N]
    kept = np.isfinite(want)  # rows of head 3's empty query blocks keep no key: +inf on both sides
    assert np.array_equal(np.isfinite(got_lse), kept) and np.all(got_lse[~kept] == np.inf)
    assert float(np.max(np.abs(got_lse[kept] - want[kept]))) <= 2e-2
    dvals, dbits = make_grad_output(cfg)
    dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    ws = torch.empty(S.salad_bwd_workspace_bytes(layer.shape), dtype=torch.uint8, device="cuda")
    ref = oracle.layer_backward(inp.q, inp.k, inp.v, rp, ci, inp.gate.astype(np.float64), inp.w_lin, cfg.N,
                                cfg.block, cfg.eps, dvals)
    for lse_arg, tag in ((lse, "forward lse"), (None, "recomputed lse")):
        g = {n: torch.full_like(q, float("nan")) for n in ("dq", "dk", "dv")}
        g["dw"] = torch.full((cfg.head_dim, cfg.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        g["dg"] = torch.full((cfg.batch * cfg.heads,), float("nan"), dtype=torch.float32, device="cuda")
        S.salad_attn_bwd(layer.shape, q, k, v, row_ptr, col_idx, gate, w, cfg.eps, 0.0, out, dout, g["dq"],
                         g["dk"], g["dv"], g["dw"], g["dg"], ws, lse=lse_arg)
        torch.cuda.synchronize()
        _compare(cfg, g, ref, f"layouts ({tag})")
