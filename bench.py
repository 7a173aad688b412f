"""Benchmark of the hybrid block-sparse + linear attention layer on one MI355X.

python bench.py [--steps K] [--warmup W] [--config c3] [--no-cpu]

A step is one pass of the whole hot path over the layer's synthetic inputs,
which are resident in HBM before timing starts:
  1. salad_build_mask      block mask -> CSR (window ranking; for top-k
                           layers also pooling, scoring, top-k and the gate)
  2. salad_linear_prepare  linear state S, z (split-N reduction) folded with
                           gate and W_lin
  3. salad_attn_apply      block-sparse flash attention + linear epilogue
Layers with cuboid blocks add salad_permute_tokens before (Q, K, V into the
cuboid storage order) and after (the output back to frame-major order) inside
the step: the conservative reading, since a model could keep its tokens in
cuboid order through every layer.
Prints one JSON line.  `value` is dense-equivalent TFLOP/s, 4*B*H*N^2*d over
the step time; ms_per_step is the step time.  The roofline object covers the
dominant kernel (the fused attention kernel), timed with HIP events on the
stream it runs on: achieved = kept-tile FLOP (4*block^2*d per kept block pair)
per launch over its mean duration, against the 2.5 PFLOP/s dense bf16 MFMA
peak.  cpu_baseline times the fp64 CPU oracle on a bounded sample of query
blocks of the same layer.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dense-equiv TFLOP/s and ms/layer, hybrid sparse+linear attn at 90% sparsity"
PEAK_BF16_TFLOPS = 2500.0
ATTN_SRC = os.path.join(ROOT, "block_sparse_linear_st_amd", "csrc", "attn_bf16.hip")
# HBM bytes per dispatch of the attention kernel from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs (KiB per dispatch), valid only for the kernel source they were
# taken on (sha256 prefix); scaled by a plain 512 MiB copy, which reads
# FETCH_SIZE = 262156.7 KiB and WRITE_SIZE = 524288 KiB.
ATTN_COUNTERS = {
    "source_sha256": "cc260356f526118f",
    "fetch_scale": 524288.0 / 262156.7,
    "write_scale": 1.0,
    "c3": {"fetch_kib": 171218.9, "write_kib": 98304.0},
}


def attn_traffic_bytes(config: str):
    """Measured HBM bytes per attention launch, or None if not measured for this source."""
    import hashlib
    with open(ATTN_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    rec = ATTN_COUNTERS.get(config)
    if rec is None or sha != ATTN_COUNTERS["source_sha256"]:
        return None
    return round(1024.0 * (rec["fetch_kib"] * ATTN_COUNTERS["fetch_scale"] +
                           rec["write_kib"] * ATTN_COUNTERS["write_scale"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--backward", action="store_true",
                    help="time a training step instead: forward (keeping its log2-sum-exp) + salad_attn_bwd")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device copy (torch copy_) 5 times, to scale HBM byte counters")
    return ap.parse_args()


def copy_calibration():
    """A copy of known size: 512 MiB read + 512 MiB written per launch."""
    import torch
    n = 512 * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def cpu_baseline(cfg, inp, row_ptr, col_idx, gate, budget_s):
    """Time the oracle forward on query blocks spread over heads until the budget is spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = 1
    order = []
    rng = np.random.default_rng(1234)
    for i in range(cfg.batch * cfg.heads * cfg.nb):
        order.append((int(rng.integers(cfg.batch)), int(rng.integers(cfg.heads)), int(rng.integers(cfg.nb))))
    done = []
    t0 = time.perf_counter()
    for blkid in order:
        oracle.layer_forward(inp.q, inp.k, inp.v, row_ptr, col_idx, gate, inp.w_lin, cfg.N, cfg.block,
                             cfg.eps, qblocks=[blkid])
        done.append(blkid)
        if time.perf_counter() - t0 >= budget_s and len(done) >= 2:
            break
    t = time.perf_counter() - t0
    rows = sum(max(0, min(cfg.block, cfg.N - qb * cfg.block)) for _, _, qb in done)
    dense_flop = 4.0 * rows * cfg.N * cfg.head_dim
    total_blocks = cfg.batch * cfg.heads * cfg.nb
    return {
        "value": dense_flop / t / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{len(done)} of {total_blocks} query blocks ({rows} query rows) of the same layer, "
                  f"fp64 dense masked softmax + quadratic ReLU linear branch + mix, in {t:.1f} s; "
                  f"projected full layer {t * total_blocks / len(done):.1f} s",
        "ms_per_layer_projected": t * total_blocks / len(done) * 1e3,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer would shard by head, with no communication between GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.backward:
        main_backward(args)
        return
    import torch

    from block_sparse_linear_st_amd import salad as S
    from block_sparse_linear_st_amd.layer import SaladLayer
    from synth import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    torch.cuda.set_device(0)
    inp = make_inputs(cfg)
    bf = cfg.dtype == "bf16"
    cub = tuple(cfg.cuboid) != (0, 0, 0)
    layer = SaladLayer(cfg.batch, cfg.heads, cfg.head_dim, cfg.T, cfg.H, cfg.W, cfg.block,
                       S.SALAD_BF16 if bf else S.SALAD_F32, cfg.specs, cuboid=cfg.cuboid)

    def dev(x, bits):
        if bf:
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()
    q, k, v = dev(inp.q, inp.q_bits), dev(inp.k, inp.k_bits), dev(inp.v, inp.v_bits)
    w = dev(inp.w_lin, inp.w_lin_bits)
    from_q = cfg.gate_kind == "from_q"
    gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda") if from_q \
        else torch.from_numpy(inp.gate).cuda()
    w_g = torch.from_numpy(inp.w_g).cuda() if from_q else None
    out = torch.empty_like(q)
    # tensors in the layer's storage order (the frame-major ones themselves without cuboids)
    qs, ks, vs, outs = (torch.empty_like(q) for _ in range(4)) if cub else (q, k, v, out)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if cub:
            layer.to_storage(q, qs, stream=sp)
            layer.to_storage(k, ks, stream=sp)
            layer.to_storage(v, vs, stream=sp)
        if ev is not None:
            ev[1].record(stream)
        layer.build_mask(qs, ks, w_g, gate if from_q else None, stream=sp)
        if ev is not None:
            ev[2].record(stream)
        S.salad_linear_prepare(layer.shape, ks, vs, gate, w, layer.ws, sp, drop_tau=0.0)
        if ev is not None:
            ev[3].record(stream)
        S.salad_attn_apply(layer.shape, qs, ks, vs, layer.row_ptr, layer.col_idx, gate, cfg.eps, 0.0, 0.0,
                           outs, layer.ws, sp)
        if ev is not None:
            ev[4].record(stream)
        if cub:
            layer.from_storage(outs, out, stream=sp)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    ms_perm = float(np.mean([e[0].elapsed_time(e[1]) + e[4].elapsed_time(e[5]) for e in evs]))
    ms_mask = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_lin = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    ms_attn = float(np.mean([e[3].elapsed_time(e[4]) for e in evs]))

    row_ptr = layer.row_ptr.cpu().numpy()
    nnz = int(row_ptr[-1])
    col_idx = layer.col_idx[:nnz].cpu().numpy()
    dense_flop = cfg.dense_equiv_flop()
    value = dense_flop / (ms_step * 1e-3) / 1e12
    kept_flop = 4.0 * cfg.block * cfg.block * cfg.head_dim * nnz
    achieved = kept_flop / (ms_attn * 1e-3) / 1e12
    density = nnz / float(cfg.batch * cfg.heads * cfg.nb * cfg.nb)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded N(0,1) + smooth spatio-temporal sinusoid, random-init W_lin)",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "batch": cfg.batch, "heads": cfg.heads, "head_dim": cfg.head_dim,
            "grid": f"{cfg.T}x{cfg.H}x{cfg.W}", "tokens": cfg.N, "n_pad": cfg.n_pad, "block": cfg.block,
            "kept_block_pairs": nnz, "block_density": round(density, 6),
            "block_shape": "x".join(str(c) for c in cfg.cuboid) if cub else "frame-major runs",
        },
        "ms_breakdown": {"mask": round(ms_mask, 5), "linear_prepare": round(ms_lin, 5),
                         "attn_kernel": round(ms_attn, 5)},
        "roofline": {
            "kernel": "k_attn_bf16 (block-sparse flash attention + linear epilogue)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": attn_traffic_bytes(cfg.name),
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_flop_per_launch": kept_flop,
        },
        "cpu_baseline": None,
    }
    if cub:
        result["ms_breakdown"]["permute_in_out"] = round(ms_perm, 5)
    if not args.no_cpu:
        g = gate.cpu().numpy().astype(np.float64)
        if cub:  # the oracle runs on the same stored token order as the kernels
            import dataclasses

            import oracle
            order = oracle.cuboid_order(cfg.T, cfg.H, cfg.W, cfg.cuboid)
            inp = dataclasses.replace(inp, **{n: oracle.permute_tokens(getattr(inp, n), order)
                                              for n in ("q", "k", "v")})
        result["cpu_baseline"] = cpu_baseline(cfg, inp, row_ptr, col_idx, g, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main_backward(args):
    """Training step on one layer: mask, forward with its log2-sum-exp, backward (bf16 layers).

    The roofline object prices the whole salad_attn_bwd call (its kernels run
    inside one library call) at the minimal algorithmic work: five block
    products per kept pair (S, dP, dV, dK, dQ: 10*block^2*d FLOP) plus 14*d^2
    per valid token and head for the linear branch (u, t, dphi(q), dS, dW,
    dphi(k), dv).  The kernels do two more products per pair, since dQ and
    dK/dV are formed in separate passes without atomics.
    """
    import torch

    from block_sparse_linear_st_amd import salad as S
    from block_sparse_linear_st_amd.layer import SaladLayer
    from synth import CONFIGS, make_grad_output, make_inputs

    cfg = CONFIGS[args.config]
    if cfg.dtype != "bf16" or tuple(cfg.cuboid) != (0, 0, 0):
        print("--backward covers bf16 layers in frame-major order", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    inp = make_inputs(cfg)
    layer = SaladLayer(cfg.batch, cfg.heads, cfg.head_dim, cfg.T, cfg.H, cfg.W, cfg.block, S.SALAD_BF16,
                       cfg.specs)

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, w = dev(inp.q_bits), dev(inp.k_bits), dev(inp.v_bits), dev(inp.w_lin_bits)
    from_q = cfg.gate_kind == "from_q"
    gate = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda") if from_q \
        else torch.from_numpy(inp.gate).cuda()
    w_g = torch.from_numpy(inp.w_g).cuda() if from_q else None
    _, dbits = make_grad_output(cfg)
    dout = dev(dbits)
    out = torch.empty_like(q)
    lse = torch.empty(cfg.batch * cfg.heads * cfg.n_pad, dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dw = torch.empty(cfg.head_dim, cfg.head_dim, dtype=torch.float32, device="cuda")
    dg = torch.empty(cfg.batch * cfg.heads, dtype=torch.float32, device="cuda")
    bws = torch.empty(S.salad_bwd_workspace_bytes(layer.shape), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        layer.build_mask(q, k, w_g, gate if from_q else None, stream=sp)
        S.salad_linear_prepare(layer.shape, k, v, gate, w, layer.ws, sp, drop_tau=0.0)
        S.salad_attn_apply(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, cfg.eps, 0.0, 0.0, out,
                           layer.ws, sp, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        S.salad_attn_bwd(layer.shape, q, k, v, layer.row_ptr, layer.col_idx, gate, w, cfg.eps, 0.0, out, dout,
                         dq, dk, dv, dw, dg, bws, sp, lse=lse)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ms_fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    nnz = int(layer.row_ptr[-1].item())
    d = cfg.head_dim
    bwd_flop = 10.0 * cfg.block * cfg.block * d * nnz + 14.0 * d * d * cfg.N * cfg.batch * cfg.heads
    achieved = bwd_flop / (ms_bwd * 1e-3) / 1e12
    dense_train = 3.5 * cfg.dense_equiv_flop()  # dense attention: forward 2 products, backward 5
    result = {
        "metric": "dense-equiv TFLOP/s and ms per training step (forward + backward), hybrid sparse+linear attn",
        "value": round(dense_train / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s (dense-equivalent, 3.5x the forward count)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + smooth spatio-temporal sinusoid; dL/dout ~ N(0,1))",
        "config": {"workload": f"{cfg.name}: {cfg.description}, forward + backward", "batch": cfg.batch,
                   "heads": cfg.heads, "head_dim": d, "grid": f"{cfg.T}x{cfg.H}x{cfg.W}", "tokens": cfg.N,
                   "block": cfg.block, "kept_block_pairs": nnz},
        "ms_breakdown": {"forward": round(ms_fwd, 5), "backward": round(ms_bwd, 5)},
        "roofline": {
            "kernel": "salad_attn_bwd (dQ and dK/dV kernels plus the linear-branch kernels, one call)",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
            "algorithmic_flop_per_launch": bwd_flop,
        },
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
