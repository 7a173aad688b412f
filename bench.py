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
# the dominant kernel's sources (its counters below are valid only for them)
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_linear_st_amd", "csrc", f) for f in ("attn_bf16.hip", "attn_common.h")]
ATTN_KERNEL = "k_attn_bf16 (block-sparse flash attention + linear epilogue)"
# HBM bytes per dispatch of the attention kernel from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs (KiB per dispatch), valid only for the kernel source they were
# taken on (sha256 prefix); scaled by a plain 512 MiB copy, which reads
# FETCH_SIZE = 262157.9 KiB and WRITE_SIZE = 524288 KiB.
ATTN_COUNTERS = {
    "source_sha256": "a60b71697c2430d2",
    "fetch_scale": 524288.0 / 262157.9,
    "write_scale": 1.0,
    "c3": {"fetch_kib": 202408.0, "write_kib": 98304.0},
}


def attn_source_sha() -> str:
    """sha256 prefix of the attention kernel's sources, concatenated in ATTN_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attn_traffic_bytes(config: str):
    """Measured HBM bytes per attention launch, or None if not measured for this source."""
    sha = attn_source_sha()
    rec = ATTN_COUNTERS.get(config)
    if rec is None or sha != ATTN_COUNTERS["source_sha256"]:
        return None
    return round(1024.0 * (rec["fetch_kib"] * ATTN_COUNTERS["fetch_scale"] +
                           rec["write_kib"] * ATTN_COUNTERS["write_scale"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU needs about 50 steps (~40 ms of this load after idling) to reach its
    # steady clock: with 3 warm-up steps the timed c3 step is ~8% slower
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
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


# The CPU oracle runs in worker processes forked before the GPU is touched, so
# they inherit the layer's inputs and mask without copying and share no GPU
# state; each uses one BLAS thread.
_POOL_STATE = {}


def _cpu_worker_init():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _cpu_worker_run(blocks):
    import oracle
    st = _POOL_STATE
    t0 = time.perf_counter()
    oracle.layer_forward(st["q"], st["k"], st["v"], st["row_ptr"], st["col_idx"], st["gate"], st["w_lin"],
                         st["N"], st["block"], st["eps"], qblocks=blocks)
    return len(blocks), time.perf_counter() - t0


def host_cpus():
    """(CPUs this process may run on, BLAS threads of this process)."""
    n_aff = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    return n_aff, int(blas)


def start_cpu_pool(cfg, inp, row_ptr, col_idx, gate):
    """Fork the oracle's worker processes (before any GPU call): one per host CPU, at most OMP_NUM_THREADS."""
    import multiprocessing as mp
    n_aff, _ = host_cpus()
    workers = max(1, min(n_aff, int(os.environ.get("OMP_NUM_THREADS", n_aff))))
    _POOL_STATE.update(q=inp.q, k=inp.k, v=inp.v, w_lin=inp.w_lin, row_ptr=row_ptr, col_idx=col_idx,
                       gate=np.asarray(gate, np.float64), N=cfg.N, block=cfg.block, eps=cfg.eps)
    return mp.get_context("fork").Pool(workers, initializer=_cpu_worker_init), workers


def cpu_baseline(cfg, pool, workers, budget_s):
    """The oracle forward over the layer's query blocks on `workers` processes, in a fixed random order,
    until every block is done or the budget is spent (the blocks already submitted still finish)."""
    n_aff, blas = host_cpus()
    rng = np.random.default_rng(1234)
    allb = [(b, h, qb) for b in range(cfg.batch) for h in range(cfg.heads) for qb in range(cfg.nb)]
    order = [allb[i] for i in rng.permutation(len(allb))]
    chunk = 8
    chunks = [order[i:i + chunk] for i in range(0, len(order), chunk)]
    t0 = time.perf_counter()
    pending, done_blocks, busy = [], 0, 0.0
    it = iter(chunks)
    exhausted = False
    while True:
        while not exhausted and len(pending) < 2 * workers and time.perf_counter() - t0 < budget_s:
            c = next(it, None)
            if c is None:
                exhausted = True
                break
            pending.append((c, pool.apply_async(_cpu_worker_run, (c,))))
        if not pending:
            break
        c, r = pending.pop(0)
        n, dt = r.get()
        done_blocks += n
        busy += dt
        if exhausted and not pending:
            break
        if time.perf_counter() - t0 >= budget_s and not exhausted:
            for c2, r2 in pending:
                n2, dt2 = r2.get()
                done_blocks += n2
                busy += dt2
            pending = []
            break
    t = time.perf_counter() - t0
    pool.close()
    pool.join()
    rows = 0
    # the blocks finished are the first done_blocks of the submission order
    for b, h, qb in order[:done_blocks]:
        rows += max(0, min(cfg.block, cfg.N - qb * cfg.block))
    dense_flop = 4.0 * rows * cfg.N * cfg.head_dim
    full = done_blocks == len(order)
    frac = done_blocks / len(order)
    return {
        "value": dense_flop / t / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"the full layer ({len(order)} query blocks) in {t:.1f} s" if full else
                   f"{done_blocks} of {len(order)} query blocks ({100 * frac:.1f}% of the layer, {rows} query rows, "
                   f"random order) in {t:.1f} s; the full layer projects to {t / frac:.1f} s") +
                  f"; fp64 dense masked softmax + quadratic ReLU linear branch + mix; {workers} worker processes "
                  f"with one BLAS thread each",
        "host_cpus": n_aff,
        "blas_threads_main": blas,
        "full_layer": full,
        "ms_per_layer": t * 1e3 if full else None,
        "ms_per_layer_projected": t / frac * 1e3,
    }


HBM_PEAK_GBS = 8000.0


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, np.float64), q))


def oracle_inputs_for_cpu(cfg, inp):
    """The oracle's own CSR and gate for the layer, and its inputs in storage order (CPU only)."""
    import dataclasses

    import oracle
    order = None
    if tuple(cfg.cuboid) != (0, 0, 0):
        order = oracle.cuboid_order(cfg.T, cfg.H, cfg.W, cfg.cuboid)
        inp = dataclasses.replace(inp, **{n: oracle.permute_tokens(getattr(inp, n), order) for n in ("q", "k", "v")})
    keep = oracle.build_masks(cfg.T, cfg.H, cfg.W, cfg.block, cfg.specs, cfg.batch, inp.q, inp.k, order=order)
    rp, ci = oracle.csr_from_keep(keep)
    gate = oracle.gate_from_q(inp.q, inp.w_g, cfg.N) if cfg.gate_kind == "from_q" else inp.gate
    return inp, rp, ci, gate


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
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS[args.config]
    inp = make_inputs(cfg)
    pool = None
    if not args.no_cpu:
        # forked before the first GPU call; the workers wait until the GPU part is done
        cinp, crp, cci, cgate = oracle_inputs_for_cpu(cfg, inp)
        pool, workers = start_cpu_pool(cfg, cinp, crp, cci, cgate)

    import torch

    from block_sparse_linear_st_amd import salad as S
    from block_sparse_linear_st_amd.layer import SaladLayer

    torch.cuda.set_device(0)
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

    def step(ev=None, ev_attn=None):
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
        if ev_attn is not None:
            ev_attn[0].record(stream)
        S.salad_attn_apply(layer.shape, qs, ks, vs, layer.row_ptr, layer.col_idx, gate, cfg.eps, 0.0, 0.0,
                           outs, layer.ws, sp)
        if ev_attn is not None:
            ev_attn[1].record(stream)
        if ev is not None:
            ev[4].record(stream)
        if cub:
            layer.from_storage(outs, out, stream=sp)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps; the only other records on the stream are the
    # HIP events around the attention call, whose mean is the roofline's kernel time
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    evs_attn = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(ev_attn=evs_attn[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    attn_timed = [e[0].elapsed_time(e[1]) for e in evs_attn]
    # the other phases and the per-step spread: K more steps after the timed
    # region, with HIP events between all the phases (six records per step cost
    # about 1% of a step, so they stay out of the timed region)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per_step = [e[0].elapsed_time(e[5]) for e in evs]
    perm = [e[0].elapsed_time(e[1]) + e[4].elapsed_time(e[5]) for e in evs]
    mask = [e[1].elapsed_time(e[2]) for e in evs]
    lin = [e[2].elapsed_time(e[3]) for e in evs]
    ms_mask, ms_lin = float(np.median(mask)), float(np.median(lin))
    ms_attn = float(np.mean(attn_timed))  # average launch duration over the timed region

    row_ptr = layer.row_ptr.cpu().numpy()
    nnz = int(row_ptr[-1])
    dense_flop = cfg.dense_equiv_flop()
    value = dense_flop / (ms_step * 1e-3) / 1e12
    kept_flop = 4.0 * cfg.block * cfg.block * cfg.head_dim * nnz
    achieved = kept_flop / (ms_attn * 1e-3) / 1e12
    density = nnz / float(cfg.batch * cfg.heads * cfg.nb * cfg.nb)
    esz = 2 if bf else 4
    tensor_b = cfg.batch * cfg.heads * cfg.n_pad * cfg.head_dim * esz
    BH, d = cfg.batch * cfg.heads, cfg.head_dim
    # phases and their algorithmic work: bytes each phase must move at least (mask: the pooled inputs;
    # linear: K and V once plus the state; attention: Q, K, V and out once), FLOP on the kept tiles
    topk_heads = sum(1 for sp_ in cfg.specs if sp_.kind == 1)
    sics_heads = sum(1 for sp_ in cfg.specs if sp_.kind == 2)
    per_head_b = cfg.batch * cfg.n_pad * cfg.head_dim * esz
    # Q and K of top-k heads, K of SICS heads, and (gate from Q) Q of the heads not pooled already
    mask_bytes = per_head_b * (2 * topk_heads + sics_heads + ((cfg.heads - topk_heads) if from_q else 0))
    lin_bytes = 2 * tensor_b + BH * (d * d + d) * 4
    attn_bytes = 4 * tensor_b
    phases = {
        "mask": {"ms": round(ms_mask, 5), "bound": "hbm" if mask_bytes else "latency",
                 "algorithmic_bytes": mask_bytes,
                 "gbs": round(mask_bytes / (ms_mask * 1e-3) / 1e9, 1) if mask_bytes else None,
                 "frac": round(mask_bytes / (ms_mask * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if mask_bytes else None,
                 "bound_ms": round(mask_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 5),
                 "share_of_attention": round(ms_mask / ms_attn, 4)},
        "linear_prepare": {"ms": round(ms_lin, 5), "bound": "hbm", "algorithmic_bytes": lin_bytes,
                           "gbs": round(lin_bytes / (ms_lin * 1e-3) / 1e9, 1),
                           "frac": round(lin_bytes / (ms_lin * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "bound_ms": round(lin_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 5)},
        "attention": {"ms": round(ms_attn, 5), "bound": "mfma", "algorithmic_flop": kept_flop,
                      "tflops": round(achieved, 2), "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                      "bound_ms": round(kept_flop / (PEAK_BF16_TFLOPS * 1e12) * 1e3, 5),
                      "hbm_bytes": attn_bytes},
    }
    if cub:
        phases["permute"] = {"ms": round(float(np.median(perm)), 5), "bound": "hbm",
                             "algorithmic_bytes": 8 * tensor_b,
                             "frac": round(8 * tensor_b / (float(np.median(perm)) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "bound_ms": round(8 * tensor_b / (HBM_PEAK_GBS * 1e9) * 1e3, 5)}
    layer_bound = sum(ph["bound_ms"] for ph in phases.values())

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
        "step_ms": {"mean": round(ms_step, 5), "median": round(pct(per_step, 50), 5),
                    "p10": round(pct(per_step, 10), 5), "p90": round(pct(per_step, 90), 5),
                    "note": "mean over the timed region; median and percentiles of the event-timed steps that follow it"},
        "ms_breakdown": {"mask": round(ms_mask, 5), "linear_prepare": round(ms_lin, 5),
                         "attn_kernel": round(ms_attn, 5)},
        "phases": phases,
        "layer_roofline": {"bound_ms": round(layer_bound, 5), "frac": round(layer_bound / ms_step, 4),
                           "note": "sum of the phases' bounds (they run one after another) over ms_per_step"},
        "roofline": {
            "kernel": ATTN_KERNEL,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": attn_traffic_bytes(cfg.name),
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_flop_per_launch": kept_flop,
            "timing": "mean of HIP events around salad_attn_apply (item split + attention kernel) on its stream, "
                      "over the timed region",
            "kernel_ms": {"mean": round(ms_attn, 5), "median": round(float(np.median(attn_timed)), 5)},
        },
        "cpu_baseline": None,
    }
    if pool is not None:
        result["cpu_baseline"] = cpu_baseline(cfg, pool, workers, args.cpu_seconds)
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
    # three HIP events per step in the timed region (the forward / backward split
    # and the backward call's time for the roofline; ~0.1% of a training step)
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
