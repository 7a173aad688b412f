"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Bars: CSR row_ptr / col_idx bit-exact; bf16 outputs max-abs <= 2e-2 and
rel-L2 <= 1e-2 against the fp64 oracle on the same bf16-rounded inputs; fp32
outputs max-abs <= 1e-4.  Small layers are compared element by element in
full; the 32k- and 148k-token layers on sampled query blocks (first, second,
middle, last-with-tail blocks of several heads plus random ones), which the
oracle computes one by one from the dense definition.
"""

import numpy as np
import pytest

import oracle
from helpers import (BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, assert_close, device_tensors, inputs, oracle_gate,
                     make_layer, oracle_csr, sample_blocks, to_numpy)
from synth import CONFIGS, HeadSpec, LayerConfig, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_linear_st_amd import salad as S  # noqa: E402


def _gate_tensor(inp, cfg):
    if inp.gate is not None:
        return torch.from_numpy(inp.gate).cuda()
    return torch.zeros(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")


def _run_mask(name, layer=None, q=None, k=None, want_gate=False):
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer = layer or make_layer(cfg)
    if q is None:
        q, k, _, _ = device_tensors(inp)
    gate = w_g = None
    if want_gate:
        w_g = torch.from_numpy(inp.w_g).cuda()
        gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
    layer.build_mask(q, k, w_g, gate)
    torch.cuda.synchronize()
    return layer, gate


# ------------------------------------------------------------------ masks

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c6", "c7"])
def test_mask_csr_bit_exact(name):
    print(f"mask parity {name}", flush=True)
    layer, _ = _run_mask(name)
    rp, ci = oracle_csr(name)
    got_rp = layer.row_ptr.cpu().numpy()
    np.testing.assert_array_equal(got_rp, rp)
    got_ci = layer.col_idx[:rp[-1]].cpu().numpy()
    np.testing.assert_array_equal(got_ci, ci)


def test_sics_mask_forward_c6():
    """A layer whose heads use the SICS mask: full forward against the oracle on the oracle's CSR."""
    cfg = CONFIGS["c6"]
    inp = inputs("c6")
    _, out, o_s, _ = _forward("c6")
    rp, ci = oracle_csr("c6")
    ref, ref_s, _ = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    assert_close(to_numpy(out), ref, BF16_MAX_ABS, BF16_REL_L2, "c6 out bf16 (SICS mask)")
    assert_close(to_numpy(o_s), ref_s, BF16_MAX_ABS, BF16_REL_L2, "c6 sparse bf16 (SICS mask)")


def test_sics_rows_hold_m_or_m_plus_one_with_diagonal():
    cfg = CONFIGS["c7"]
    layer, _ = _run_mask("c7")
    rp = layer.row_ptr.cpu().numpy().astype(np.int64)
    ci = layer.col_idx[:rp[-1]].cpu().numpy()
    m = oracle.topk_count(cfg.specs[0].density, cfg.nb)
    counts = np.diff(rp)
    assert set(counts.tolist()) <= {m, m + 1}
    for h in range(cfg.heads):
        first = None
        for qb in range(cfg.nb):
            r = h * cfg.nb + qb
            row = ci[rp[r]:rp[r + 1]]
            assert np.all(np.diff(row) > 0) and qb in row
            kept = set(row.tolist()) - {qb} if counts[r] == m + 1 else set(row.tolist())
            if counts[r] == m:
                first = kept if first is None else first
                assert kept == first  # every row of a head shares the kept set


def test_gate_from_q_c4():
    print("gate parity c4", flush=True)
    cfg = CONFIGS["c4"]
    inp = inputs("c4")
    layer, gate_fused = _run_mask("c4", want_gate=True)
    q, _, _, _ = device_tensors(inp)
    gate2 = torch.empty_like(gate_fused)
    layer.gate_from_q(q, torch.from_numpy(inp.w_g).cuda(), gate2)
    torch.cuda.synchronize()
    ref = oracle.gate_from_q(inp.q, inp.w_g, cfg.N)
    np.testing.assert_allclose(gate_fused.cpu().numpy(), ref, rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(gate_fused.cpu().numpy(), gate2.cpu().numpy())


def test_window_at_and_past_the_candidate_count():
    """c1's +-1-frame window has 10 candidate pairs per head.  Asking for exactly 10 (K = every candidate) gives
    the oracle's CSR bit for bit; asking for 11 is refused on the host (SALAD_EINFEASIBLE, as the oracle raises
    InfeasibleMask) before anything is allocated or launched."""
    cfg = CONFIGS["c1"]
    at = [HeadSpec(0, 1, -1, 9.75 / 16), HeadSpec(0, 1, -1, 0.5)]  # K = 10 (all candidates) and 8
    assert oracle.window_count(at[0].density, cfg.nb, cfg.nb) == 10
    layer = make_layer(cfg, specs=at)
    layer.build_mask()
    torch.cuda.synchronize()
    keep = oracle.build_masks(cfg.T, cfg.H, cfg.W, cfg.block, at, cfg.batch)
    rp, ci = oracle.csr_from_keep(keep)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(layer.col_idx[:rp[-1]].cpu().numpy(), ci)
    past = [HeadSpec(0, 1, -1, 10.75 / 16), HeadSpec(0, 1, -1, 0.5)]  # K = 11 > 10 candidates
    with pytest.raises(oracle.InfeasibleMask):
        oracle.build_masks(cfg.T, cfg.H, cfg.W, cfg.block, past, cfg.batch)
    with pytest.raises(S.SaladError) as err:
        make_layer(cfg, specs=past)
    assert err.value.status == S.SALAD_EINFEASIBLE


# ------------------------------------------------------------------ linear state

@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_linear_state(name):
    print(f"linear state {name}", flush=True)
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer = make_layer(cfg)
    _, k, v, _ = device_tensors(inp)
    BH, d = cfg.batch * cfg.heads, cfg.head_dim
    S_out = torch.empty(BH * d * d, dtype=torch.float32, device="cuda")
    z_out = torch.empty(BH * d, dtype=torch.float32, device="cuda")
    layer.linear_state(k, v, S_out, z_out)
    torch.cuda.synchronize()
    S_ref, z_ref = oracle.linear_state(inp.k, inp.v, cfg.N)
    S_got = S_out.cpu().numpy().reshape(S_ref.shape)
    z_got = z_out.cpu().numpy().reshape(z_ref.shape)
    # fp32 accumulation of exact products over N terms
    assert_close(S_got, S_ref, 1e-5 * np.abs(S_ref).max() * np.sqrt(cfg.N), 1e-5, f"S {name}")
    assert_close(z_got, z_ref, 1e-6 * np.abs(z_ref).max() * np.sqrt(cfg.N), 1e-6, f"z {name}")
    # bitwise reproducible
    S2 = torch.empty_like(S_out)
    z2 = torch.empty_like(z_out)
    layer.linear_state(k, v, S2, z2)
    torch.cuda.synchronize()
    assert torch.equal(S2, S_out) and torch.equal(z2, z_out)


# ------------------------------------------------------------------ full forward, small layers

def _forward(name, dtype=None, v_shift=0.0, canary=False, drop_tau=0.0, gate_override=None, w_override=None):
    cfg = CONFIGS[name]
    inp = inputs(name, canary)
    layer = make_layer(cfg, dtype)
    q, k, v, w = device_tensors(inp, dtype)
    if v_shift:
        v = v + v_shift
    layer.build_mask(q, k)
    gate = _gate_tensor(inp, cfg) if gate_override is None else gate_override
    if w_override is not None:
        w = w_override
    out = torch.empty_like(q)
    layer.forward(q, k, v, gate, w, out, eps=cfg.eps, drop_tau=drop_tau)
    o_s = torch.empty_like(q)
    o_l = torch.empty_like(q)
    layer.branches(q, k, v, o_s, o_l, eps=cfg.eps)
    torch.cuda.synchronize()
    return layer, out, o_s, o_l


def test_forward_c1_fp32():
    cfg = CONFIGS["c1"]
    inp = inputs("c1")
    _, out, o_s, o_l = _forward("c1")
    rp, ci = oracle_csr("c1")
    ref, ref_s, ref_l = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    assert_close(to_numpy(out), ref, F32_MAX_ABS, 1e-5, "c1 out fp32")
    assert_close(to_numpy(o_s), ref_s, F32_MAX_ABS, 1e-5, "c1 sparse fp32")
    assert_close(to_numpy(o_l), ref_l, F32_MAX_ABS, 1e-4, "c1 linear fp32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_c2(dtype):
    cfg = CONFIGS["c2"]
    inp = inputs("c2")
    _, out, o_s, o_l = _forward("c2", dtype)
    rp, ci = oracle_csr("c2")
    ref, ref_s, ref_l = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    if dtype == "bf16":
        assert_close(to_numpy(out), ref, BF16_MAX_ABS, BF16_REL_L2, "c2 out bf16")
        assert_close(to_numpy(o_s), ref_s, BF16_MAX_ABS, BF16_REL_L2, "c2 sparse bf16")
        assert_close(to_numpy(o_l), ref_l, BF16_MAX_ABS, BF16_REL_L2, "c2 linear bf16 (own norm)")
    else:
        assert_close(to_numpy(out), ref, F32_MAX_ABS, 1e-5, "c2 out fp32")
        assert_close(to_numpy(o_s), ref_s, F32_MAX_ABS, 1e-5, "c2 sparse fp32")
        assert_close(to_numpy(o_l), ref_l, F32_MAX_ABS, 1e-4, "c2 linear fp32")


def test_mask_and_linear_state_on_two_streams_c3():
    """The mask pass and the linear-state pass with separate workspaces on two streams (as the bench runs them)
    give the serial path's CSR and output bit for bit, on the 32k-token layer, and the CSR matches the oracle."""
    print("two streams c3", flush=True)
    cfg = CONFIGS["c3"]
    inp = inputs("c3")
    q, k, v, w = device_tensors(inp)
    gate = torch.from_numpy(inp.gate).cuda()
    outs = []
    for concurrent in (False, True):
        layer = make_layer(cfg)
        ws_lin = torch.full_like(layer.ws, 0xFF) if concurrent else layer.ws
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream() if concurrent else main
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        S.salad_linear_prepare(layer.shape, k, v, gate, w, ws_lin, side.cuda_stream, drop_tau=0.0)
        join.record(side)
        layer.build_mask(q, k, stream=main.cuda_stream)
        main.wait_event(join)
        out = torch.empty_like(q)
        S.salad_attn_apply(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, cfg.eps, 0.0, 0.0, out,
                           ws_lin, main.cuda_stream)
        torch.cuda.synchronize()
        outs.append((layer.row_ptr.clone(), layer.col_idx.clone(), out))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2], outs[1][2]), "two-stream output differs from the serial one"
    np.testing.assert_array_equal(outs[1][0].cpu().numpy(), oracle_csr("c3")[0])


def test_linear_branch_shifted_v_c2():
    """V + 1 makes o_l of order 1, so the linear branch is visible at the bf16 bar."""
    cfg = CONFIGS["c2"]
    inp = inputs("c2")
    _, out, o_s, o_l = _forward("c2", v_shift=1.0)
    v1 = inp.v + np.float32(1.0)
    ref_l = oracle.linear_attention(inp.q, inp.k, v1, cfg.N, cfg.eps)
    assert_close(to_numpy(o_l), ref_l, BF16_MAX_ABS, BF16_REL_L2, "c2 linear, V+1")
    rp, ci = oracle_csr("c2")
    ref, _, _ = oracle.layer_forward(inp.q, inp.k, v1, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    assert_close(to_numpy(out), ref, BF16_MAX_ABS, BF16_REL_L2, "c2 out, V+1")


@pytest.mark.parametrize("head_dim", [64, 128])
def test_fused_linear_term_with_shifted_v(head_dim):
    """V + 1 (rounded to bf16 on the host) and unit gates make the linear term of order 1 (rms ~1), so the fused
    forward's gated, projected linear term out - o_s is compared on its own: head_dim 64 (two waves of the linear-state kernel
    hold the two V-channel halves of a row tile and add them through LDS) and 128, a ragged last token chunk,
    several splits per head."""
    from synth import bf16_bits_to_f32, bf16_round
    print(f"fused linear term head_dim {head_dim}", flush=True)
    cfg = LayerConfig(name=f"lin{head_dim}", seed=41, batch=1, heads=3, head_dim=head_dim, T=3, H=8, W=20, block=64,
                      dtype="bf16", specs=(HeadSpec(0, 1, -1, 0.0),) * 3, gate_kind="uniform")
    inp = make_inputs(cfg)
    v1_bits = bf16_round(inp.v + np.float32(1.0))
    v1 = bf16_bits_to_f32(v1_bits)
    layer = make_layer(cfg)
    q, k, _, w = device_tensors(inp)
    v = torch.from_numpy(np.ascontiguousarray(v1_bits).view(np.int16)).view(torch.bfloat16).cuda()
    layer.build_mask(q, k)
    g1 = np.ones(cfg.batch * cfg.heads, dtype=np.float32)
    gate = torch.from_numpy(g1).cuda()
    out = torch.empty_like(q)
    layer.forward(q, k, v, gate, w, out, eps=cfg.eps)
    o_s = torch.empty_like(q)
    layer.branches(q, k, v, o_s, None, eps=cfg.eps)
    torch.cuda.synchronize()
    keep = oracle.build_masks(cfg.T, cfg.H, cfg.W, cfg.block, cfg.specs, cfg.batch, inp.q, inp.k)
    rp, ci = oracle.csr_from_keep(keep)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    ref, ref_s, _ = oracle.layer_forward(inp.q, inp.k, v1, rp, ci, g1, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    N = cfg.N
    assert_close(to_numpy(out)[:, :, :N], ref[:, :, :N], BF16_MAX_ABS, BF16_REL_L2, f"d{head_dim} out, V+1")
    term = (to_numpy(out) - to_numpy(o_s))[:, :, :N]
    want = (ref - ref_s)[:, :, :N]
    rel = float(np.linalg.norm(term - want) / np.linalg.norm(want))
    print(f"d{head_dim} linear term: rel-L2 {rel:.3e}, rms {float(np.sqrt(np.mean(want ** 2))):.3e}", flush=True)
    # out and o_s each rounded to bf16 (relative 2^-9 of values of order 1): 3e-3 from that alone
    assert rel <= 2e-2


def test_gate_zero_and_projection_zero_give_sparse_bitwise():
    cfg = CONFIGS["c2"]
    zero_g = torch.zeros(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
    _, out, o_s, _ = _forward("c2", gate_override=zero_g)
    assert torch.equal(out, o_s)
    zero_w = torch.zeros(cfg.head_dim, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    _, out2, o_s2, _ = _forward("c2", w_override=zero_w)
    assert torch.equal(out2, o_s2)


def test_branch_dropping():
    cfg = CONFIGS["c2"]
    inp = inputs("c2")
    tau = float(np.median(inp.gate))
    _, out, o_s, _ = _forward("c2", drop_tau=tau)
    _, full, _, _ = _forward("c2")
    for h in range(cfg.heads):
        if inp.gate[h] < tau:
            assert torch.equal(out[0, h], o_s[0, h]), h
        else:
            assert torch.equal(out[0, h], full[0, h]), h


def test_branch_dropping_split_calls_skip_the_state():
    """prepare + apply with drop_tau: no linear state is computed for dropped heads, so their workspace slots may
    hold anything (here NaN bytes) without reaching the output; kept heads match the fused call bit for bit."""
    cfg = CONFIGS["c2"]
    inp = inputs("c2")
    tau = float(np.median(inp.gate))
    layer = make_layer(cfg, None)
    q, k, v, w = device_tensors(inp, None)
    layer.build_mask(q, k)
    gate = _gate_tensor(inp, cfg)
    layer.ws.fill_(0xFF)  # NaN in every fp32 / bf16 slot
    S.salad_linear_prepare(layer.shape, k, v, gate, w, layer.ws, drop_tau=tau)
    out = torch.empty_like(q)
    S.salad_attn_apply(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, cfg.eps, 0.0, tau, out, layer.ws)
    _, fused, o_s, _ = _forward("c2", drop_tau=tau)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    for h in range(cfg.heads):
        if inp.gate[h] < tau:
            assert torch.equal(out[0, h], o_s[0, h]), h
        else:
            assert torch.equal(out[0, h], fused[0, h]), h


# ------------------------------------------------------------------ large layers, sampled rows

@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_forward_sampled_large(name):
    print(f"sampled forward {name}", flush=True)
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    if cfg.gate_kind == "from_q":
        gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
        layer.build_mask(q, k, torch.from_numpy(inp.w_g).cuda(), gate)
    else:
        gate = _gate_tensor(inp, cfg)
        layer.build_mask(q, k)
    out = torch.empty_like(q)
    layer.forward(q, k, v, gate, w, out, eps=cfg.eps)
    o_s = torch.empty_like(q)
    o_l = torch.empty_like(q)
    layer.branches(q, k, v, o_s, o_l, eps=cfg.eps)
    torch.cuda.synchronize()
    rp = layer.row_ptr.cpu().numpy()
    ci = layer.col_idx[:rp[-1]].cpu().numpy()
    orp, oci = oracle_csr(name)
    np.testing.assert_array_equal(rp, orp)
    np.testing.assert_array_equal(ci, oci)
    g = oracle_gate(cfg, inp, gate)  # the device gate is checked, the reference uses the oracle's
    picks = sample_blocks(cfg)
    ref, ref_s, ref_l = oracle.layer_forward(inp.q, inp.k, inp.v, orp, oci, g, inp.w_lin, cfg.N, cfg.block,
                                             cfg.eps, qblocks=picks)
    blk = cfg.block
    got = np.stack([to_numpy(out[b, h, qb * blk:(qb + 1) * blk]) for b, h, qb in picks])
    got_s = np.stack([to_numpy(o_s[b, h, qb * blk:(qb + 1) * blk]) for b, h, qb in picks])
    got_l = np.stack([to_numpy(o_l[b, h, qb * blk:(qb + 1) * blk]) for b, h, qb in picks])
    assert_close(got, ref, BF16_MAX_ABS, BF16_REL_L2, f"{name} out (sampled)")
    assert_close(got_s, ref_s, BF16_MAX_ABS, BF16_REL_L2, f"{name} sparse (sampled)")
    assert_close(got_l, ref_l, BF16_MAX_ABS, BF16_REL_L2, f"{name} linear (sampled, own norm)")
    # padded rows are zero
    if cfg.n_pad > cfg.N:
        assert torch.count_nonzero(out[:, :, cfg.N:]).item() == 0
    # run-to-run bitwise determinism of the fused forward
    out2 = torch.empty_like(q)
    layer.forward(q, k, v, gate, w, out2, eps=cfg.eps)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_tail_canary_c3():
    """Padding filled with 1e4 must not change a single output bit."""
    cfg = CONFIGS["c3"]
    _, out0, _, _ = _forward("c3")
    _, out1, _, _ = _forward("c3", canary=True)
    assert torch.equal(out0, out1)
    assert torch.count_nonzero(out1[:, :, cfg.N:]).item() == 0


# ------------------------------------------------------------------ ragged and degenerate layers

RAGGED = [
    # (batch, heads, d, T, H, W, block, dtype, specs)
    (1, 2, 64, 3, 5, 7, 64, "bf16", [HeadSpec(0, 1, -1, 0.0), HeadSpec(1, 0, -1, 0.5)]),
    (2, 3, 128, 3, 5, 7, 64, "bf16", [HeadSpec(0, 0, 2, 0.0), HeadSpec(1, 0, -1, 0.34), HeadSpec(0, 1, -1, 0.6)]),
    (1, 2, 64, 2, 7, 9, 128, "bf16", [HeadSpec(1, 0, -1, 1.0), HeadSpec(0, 1, -1, 0.0)]),
    (1, 2, 128, 5, 9, 11, 128, "bf16", [HeadSpec(0, 2, -1, 0.3), HeadSpec(1, 0, -1, 0.2)]),
    (1, 3, 128, 3, 6, 37, 64, "f32", [HeadSpec(0, 1, 3, 0.0), HeadSpec(1, 0, -1, 0.1), HeadSpec(0, 1, -1, 0.15)]),
    (2, 2, 64, 4, 8, 9, 128, "f32", [HeadSpec(1, 0, -1, 0.5), HeadSpec(0, 1, -1, 0.5)]),
    (1, 128, 64, 1, 4, 40, 64, "bf16", [HeadSpec(h % 2, 1, -1, 0.5) for h in range(128)]),
    # one key block (no neighbouring pair to sample), and 192 sequences (per-head layout words past 128)
    (1, 2, 128, 1, 5, 9, 64, "bf16", [HeadSpec(0, 1, -1, 0.0), HeadSpec(1, 0, -1, 1.0)]),
    (2, 96, 64, 1, 4, 40, 64, "bf16", [HeadSpec(h % 2, 1, -1, 0.5) for h in range(96)]),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"r{i}" for i in range(len(RAGGED))])
def test_ragged_layers(case):
    B, Hh, d, T, H, W, blk, dt, specs = case
    print(f"ragged {case[:8]}", flush=True)
    cfg = LayerConfig(name="ragged", seed=11, batch=B, heads=Hh, head_dim=d, T=T, H=H, W=W, block=blk,
                      dtype=dt, specs=tuple(specs), gate_kind="uniform")
    inp = make_inputs(cfg, canary=True)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    layer.build_mask(q, k)
    gate = torch.from_numpy(inp.gate).cuda()
    out = torch.empty_like(q)
    layer.forward(q, k, v, gate, w, out, eps=cfg.eps)
    torch.cuda.synchronize()
    keep = oracle.build_masks(T, H, W, blk, specs, B, inp.q, inp.k)
    rp, ci = oracle.csr_from_keep(keep)
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(layer.col_idx[:rp[-1]].cpu().numpy(), ci)
    ref, _, _ = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, blk, cfg.eps)
    if dt == "bf16":
        assert_close(to_numpy(out), ref, BF16_MAX_ABS, BF16_REL_L2, f"ragged {case[:8]}")
    else:
        assert_close(to_numpy(out), ref, F32_MAX_ABS, 1e-5, f"ragged {case[:8]}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_empty_and_hand_built_rows(dt):
    """A hand-built CSR with empty rows: those rows carry only the linear branch."""
    from block_sparse_linear_st_amd import salad as S
    cfg = LayerConfig(name="holes", seed=12, batch=1, heads=2, head_dim=64, T=2, H=8, W=16, block=64,
                      dtype=dt, specs=(HeadSpec(0, 1, -1, 0.0),) * 2, gate_kind="uniform")
    inp = make_inputs(cfg)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    rng = np.random.default_rng(3)
    keep = rng.random((1, 2, cfg.nb, cfg.nb)) < 0.4
    keep[0, 0, 1] = False
    keep[0, 1, :] = False
    keep[0, 1, 2, 3] = True
    rp, ci = oracle.csr_from_keep(keep)
    layer.row_ptr.copy_(torch.from_numpy(rp))
    layer.col_idx[:len(ci)].copy_(torch.from_numpy(ci))
    gate = torch.from_numpy(inp.gate).cuda()
    out = torch.empty_like(q)
    layer.forward(q, k, v, gate, w, out, eps=cfg.eps)
    o_s = torch.empty_like(q)
    layer.branches(q, k, v, o_s, None, eps=cfg.eps)
    torch.cuda.synchronize()
    ref, ref_s, _ = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    tol = (BF16_MAX_ABS, BF16_REL_L2) if dt == "bf16" else (F32_MAX_ABS, 1e-5)
    assert_close(to_numpy(out), ref, *tol, f"holes {dt}")
    assert_close(to_numpy(o_s), ref_s, *tol, f"holes sparse {dt}")
    assert torch.count_nonzero(o_s[0, 0, 64:128]).item() == 0
    assert torch.count_nonzero(o_s[0, 1, :128]).item() == 0


def test_union_and_own_list_layouts_in_one_launch():
    """Heads whose neighbouring query blocks keep nearly the same key blocks (walked as the union of the two
    lists) beside heads whose neighbours share few or none (each wave pair walks its own block's list), two
    batches, 630 tokens (a 54-token tail block), against the oracle on every output row."""
    cfg = LayerConfig(name="layouts", seed=21, batch=2, heads=4, head_dim=128, T=3, H=10, W=21, block=64,
                      dtype="bf16", specs=(HeadSpec(0, 1, -1, 0.0),) * 4, gate_kind="uniform")
    inp = make_inputs(cfg)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    nb = cfg.nb
    rng = np.random.default_rng(5)
    keep = np.zeros((2, 4, nb, nb), dtype=bool)
    for b in range(2):
        keep[b, 0] = rng.random((nb, nb)) < 0.35                        # scattered: little overlap
        for qb in range(nb):                                            # a band: neighbours nearly equal
            keep[b, 1, qb, max(0, qb - 2):qb + 3] = True
        for qb in range(nb):                                            # neighbours disjoint
            keep[b, 2, qb, (qb % 2)::2] = True
        keep[b, 3, 0::2, :] = True                                      # every other row full, the rest empty
    rp, ci = oracle.csr_from_keep(keep)
    layer.row_ptr.copy_(torch.from_numpy(rp))
    layer.col_idx[:len(ci)].copy_(torch.from_numpy(ci))
    gate = torch.from_numpy(inp.gate).cuda()
    out = torch.empty_like(q)
    layer.forward(q, k, v, gate, w, out, eps=cfg.eps)
    torch.cuda.synchronize()
    ref, _, _ = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block, cfg.eps)
    assert_close(to_numpy(out), ref, BF16_MAX_ABS, BF16_REL_L2, "layouts")
    # branch dropping across both layouts: heads whose gate is below the median keep o_s only
    tau = float(np.median(inp.gate))
    out2 = torch.full_like(q, float("nan"))
    layer.forward(q, k, v, gate, w, out2, eps=cfg.eps, drop_tau=tau)
    torch.cuda.synchronize()
    ref2, _, _ = oracle.layer_forward(inp.q, inp.k, inp.v, rp, ci, inp.gate, inp.w_lin, cfg.N, cfg.block, cfg.eps,
                                      drop_tau=tau)
    assert_close(to_numpy(out2), ref2, BF16_MAX_ABS, BF16_REL_L2, "layouts, branch dropping")


@pytest.mark.parametrize("cuboid", [(0, 0, 0), (1, 2, 32)], ids=["runs", "cuboids"])
def test_window_mask_grid_wider_than_rank_range(cuboid):
    """max(H, W) above 4096, beyond the symmetric r* kernel's rank range: the table and its histogram come from
    the one-workgroup-per-query-block kernels instead (a cleared histogram and global atomics). Window heads only,
    so the CSR depends on the geometry alone; bit-exact against the oracle in frame-major and cuboid order."""
    print(f"wide grid {cuboid}", flush=True)
    T, H, W, blk = 2, 2, 4200, 64
    specs = (HeadSpec(0, 1, -1, 0.2), HeadSpec(0, 0, 40, 0.0))
    cfg = LayerConfig(name="wide", seed=13, batch=1, heads=2, head_dim=64, T=T, H=H, W=W, block=blk, dtype="bf16",
                      specs=specs, gate_kind="uniform", cuboid=cuboid)
    layer = make_layer(cfg)
    x = torch.zeros((1, 2, cfg.n_pad, 64), dtype=torch.bfloat16, device="cuda")
    layer.build_mask(x, x)
    torch.cuda.synchronize()
    z = np.zeros((1, 2, cfg.N, 64))
    order = None if cuboid == (0, 0, 0) else oracle.cuboid_order(T, H, W, cuboid)
    rp, ci = oracle.csr_from_keep(oracle.build_masks(T, H, W, blk, specs, 1, z, z, order=order))
    np.testing.assert_array_equal(layer.row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(layer.col_idx[:rp[-1]].cpu().numpy(), ci)
