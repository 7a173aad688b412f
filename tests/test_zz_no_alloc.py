"""salad_attn_fwd_noalloc: the forward on the library's static scratch gives the workspace forward's output bit
for bit, on two calls in a row, the second on a smaller layer (the scratch keeps the first call's contents), and
captured in a HIP graph it replays to the eager output."""

import numpy as np
import pytest

from helpers import device_tensors, inputs, make_layer
from synth import CONFIGS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from block_sparse_linear_st_amd import salad as S  # noqa: E402


def _layer_inputs(name):
    cfg = CONFIGS[name]
    inp = inputs(name)
    layer = make_layer(cfg)
    q, k, v, w = device_tensors(inp)
    if cfg.gate_kind == "from_q":
        gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
        layer.build_mask(q, k, torch.from_numpy(inp.w_g).cuda(), gate)
    else:
        gate = torch.from_numpy(inp.gate).cuda()
        layer.build_mask(q, k)
    return cfg, layer, q, k, v, w, gate


@pytest.mark.parametrize("names", [("c3", "c2"), ("c4", "c1")], ids=["c3-then-c2", "c4-then-c1"])
def test_noalloc_forward_equals_workspace_forward(names):
    for name in names:
        print(f"no-alloc forward {name}", flush=True)
        cfg, layer, q, k, v, w, gate = _layer_inputs(name)
        bf = cfg.dtype == "bf16"
        ref = torch.empty_like(q)
        got = torch.full_like(q, float("nan"))
        lse_ref = lse_got = None
        if bf:
            n = cfg.batch * cfg.heads * layer.shape.n_pad
            lse_ref = torch.empty(n, dtype=torch.float32, device="cuda")
            lse_got = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        layer.forward(q, k, v, gate, w, ref, eps=cfg.eps, lse=lse_ref)
        torch.cuda.synchronize()
        S.salad_attn_fwd_noalloc(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, w, cfg.eps, 0.0, 0.0,
                                 got, lse=lse_got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{name}: output differs from salad_attn_fwd"
        if bf:
            assert torch.equal(lse_got, lse_ref), f"{name}: lse differs from salad_attn_fwd"
        assert np.isfinite(got.float().cpu().numpy()).all()


def test_noalloc_forward_replays_in_a_graph():
    """The caller it exists for: captured once in a HIP graph, the allocation-free forward replays to the eager
    output bit for bit, three times, with other eager work on the same scratch and on the device between replays."""
    print("no-alloc forward in a graph c2", flush=True)
    cfg, layer, q, k, v, w, gate = _layer_inputs("c2")
    ref = torch.empty_like(q)
    S.salad_attn_fwd_noalloc(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, w, cfg.eps, 0.0, 0.0, ref)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on the capture stream before capturing
        S.salad_attn_fwd_noalloc(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, w, cfg.eps, 0.0, 0.0,
                                 out, stream=side.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        S.salad_attn_fwd_noalloc(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, w, cfg.eps, 0.0, 0.0,
                                 out, stream=side.cuda_stream)
    torch.cuda.synchronize()
    other = torch.empty_like(q)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager call"
        # eager work between replays: the same entry point on the shared scratch, with another gate
        S.salad_attn_fwd_noalloc(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate * 0.5, w, cfg.eps, 0.0,
                                 0.0, other)
        torch.cuda.synchronize()
