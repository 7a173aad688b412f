"""GPU parity of the cuboid storage order, through the C-ABI.

The permutation is data movement: bit-exact against the oracle's order.  Masks
on cuboid blocks: CSR bit-exact against the oracle (window r* by token-pair
brute force on the stored coordinates; top-k and SICS on the stored blocks).
The whole path (into storage order, mask, forward, back to frame-major) on the
small ragged layer: element by element against the oracle forward on the
oracle-permuted inputs, at the bf16 bars of the other parity tests; on the
32k-token layer at sampled query blocks.
"""

import numpy as np
import pytest

import oracle
from helpers import (BF16_MAX_ABS, BF16_REL_L2, assert_close, device_tensors, inputs, make_layer, oracle_csr, oracle_gate,
                     sample_blocks, storage_order, stored_inputs, to_numpy)
from synth import CONFIGS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _to_storage(layer, *ts):
    out = []
    for t in ts:
        d = torch.empty_like(t)
        layer.to_storage(t, d)
        out.append(d)
    return out


@pytest.mark.parametrize("name,dtype", [("c9", "bf16"), ("c9", "f32"), ("c8", "bf16"), ("c8", "f32")])
def test_permute_bit_exact(name, dtype):
    """All four row widths of the copy kernel (8, 16, 16 and 32 chunks of 16 bytes)."""
    print(f"permute {name} {dtype}", flush=True)
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer = make_layer(cfg, dtype)
    q, k, _, _ = device_tensors(inp, dtype)
    qs, ks = _to_storage(layer, q, k)
    torch.cuda.synchronize()
    o = storage_order(name)
    np.testing.assert_array_equal(to_numpy(qs), oracle.permute_tokens(to_numpy(q), o))
    np.testing.assert_array_equal(to_numpy(ks), oracle.permute_tokens(to_numpy(k), o))
    back = torch.empty_like(qs)
    layer.from_storage(qs, back)
    torch.cuda.synchronize()
    assert torch.equal(back, q)


@pytest.mark.parametrize("name", ["c9", "c8"])
def test_cuboid_mask_csr_bit_exact(name):
    print(f"cuboid mask {name}", flush=True)
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer = make_layer(cfg)
    q, k, _, _ = device_tensors(inp)
    qs, ks = _to_storage(layer, q, k)
    gate = w_g = None
    if cfg.gate_kind == "from_q":
        w_g = torch.from_numpy(inp.w_g).cuda()
        gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
    layer.build_mask(qs, ks, w_g, gate)
    torch.cuda.synchronize()
    rp, ci = oracle_csr(name)
    got_rp = layer.row_ptr.cpu().numpy()
    np.testing.assert_array_equal(got_rp, rp)
    np.testing.assert_array_equal(layer.col_idx[:rp[-1]].cpu().numpy(), ci)
    if gate is not None:
        sq, _, _ = stored_inputs(name)
        np.testing.assert_allclose(gate.cpu().numpy(), oracle.gate_from_q(sq, inp.w_g, cfg.N), rtol=1e-5, atol=1e-6)


def _cuboid_forward(name):
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    qs, ks, vs = _to_storage(layer, q, k, v)
    if cfg.gate_kind == "from_q":
        gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
        layer.build_mask(qs, ks, torch.from_numpy(inp.w_g).cuda(), gate)
    else:
        gate = torch.from_numpy(inp.gate).cuda()
        layer.build_mask(qs, ks)
    out_s = torch.empty_like(qs)
    layer.forward(qs, ks, vs, gate, w, out_s, eps=cfg.eps)
    out = torch.empty_like(q)
    layer.from_storage(out_s, out)
    torch.cuda.synchronize()
    return layer, gate, out_s, out


def test_cuboid_forward_c9():
    """Whole path on the ragged layer, compared in frame-major order against the oracle."""
    print("cuboid forward c9", flush=True)
    cfg = CONFIGS["c9"]
    inp = inputs("c9")
    _, gate, _, out = _cuboid_forward("c9")
    rp, ci = oracle_csr("c9")
    sq, sk, sv = stored_inputs("c9")
    g = oracle_gate(cfg, inp, gate)
    ref_s, _, _ = oracle.layer_forward(sq, sk, sv, rp, ci, g, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    ref = oracle.permute_tokens(ref_s, storage_order("c9"), inverse=True)
    assert_close(to_numpy(out), ref, BF16_MAX_ABS, BF16_REL_L2, "c9 out bf16 (cuboid order)")
    assert torch.count_nonzero(out[:, :, cfg.N:]).item() == 0


def test_cuboid_forward_sampled_c8():
    print("cuboid forward c8 (sampled)", flush=True)
    cfg = CONFIGS["c8"]
    inp = inputs("c8")
    layer, gate, out_s, _ = _cuboid_forward("c8")
    rp, ci = oracle_csr("c8")
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    sq, sk, sv = stored_inputs("c8")
    picks = sample_blocks(cfg)
    ref, _, _ = oracle.layer_forward(sq, sk, sv, rp, ci, inp.gate.astype(np.float64), inp.w_lin, cfg.N,
                                     cfg.block, cfg.eps, qblocks=picks)
    blk = cfg.block
    got = np.stack([to_numpy(out_s[b, h, qb * blk:(qb + 1) * blk]) for b, h, qb in picks])
    assert_close(got, ref, BF16_MAX_ABS, BF16_REL_L2, "c8 out (sampled, storage order)")
