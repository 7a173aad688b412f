"""Host-side checks of bench.py (no GPU): the one-GPU guard, the HBM traffic
constants against the committed counter summary, and the algorithmic FLOP count
of the attention roofline against the oracle's mask."""

import os
import re
import subprocess
import sys

import numpy as np

from helpers import oracle_csr
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_constants_match_the_committed_profile():
    """The fetch/write KiB and the copy calibration bench.py uses are the ones the profile summary reports,
    for the attention source it was taken on."""
    prof = open(os.path.join(ROOT, "profiles", "c3_32760tok_window_kernels.md")).read()
    hbm = prof[prof.index("## HBM bytes"):]
    row = re.search(r"\| k_attn_bf16<128, 64> \| ([0-9.]+) \| ([0-9.]+) \|", hbm)
    assert row, "attention row missing from the HBM table"
    assert float(row.group(1)) == bench.ATTN_COUNTERS["c3"]["fetch_kib"]
    assert float(row.group(2)) == bench.ATTN_COUNTERS["c3"]["write_kib"]
    cal = re.search(r"reads FETCH_SIZE =\s+([0-9.]+) KiB and WRITE_SIZE = ([0-9.]+) KiB", prof)
    assert cal, "copy calibration missing"
    assert bench.ATTN_COUNTERS["fetch_scale"] == 524288.0 / float(cal.group(1))
    assert bench.ATTN_COUNTERS["write_scale"] == 524288.0 / float(cal.group(2))
    assert re.search(r"sha256\s+prefix " + bench.ATTN_COUNTERS["source_sha256"], prof)
    got = bench.attn_traffic_bytes("c3")
    assert got is not None, "attention source changed since the counters were taken"
    want = 1024.0 * (float(row.group(1)) * 524288.0 / float(cal.group(1)) + float(row.group(2)))
    assert got == round(want)
    assert bench.attn_traffic_bytes("c4") is None  # not measured for that layer


def test_kept_tile_flop_count_from_the_oracle_mask():
    """4 * block^2 * head_dim per kept block pair (two products, 2 flops per MAC), from the oracle's CSR."""
    cfg = CONFIGS["c3"]
    rp, ci = oracle_csr("c3")
    nnz = int(rp[-1])
    assert nnz == 314568
    assert 4.0 * cfg.block * cfg.block * cfg.head_dim * nnz == 659696910336.0
    # the dense-equivalent count the metric divides by: all N x N query-key pairs, two products
    assert cfg.dense_equiv_flop() == 4.0 * cfg.batch * cfg.heads * float(cfg.N) ** 2 * cfg.head_dim
    assert np.isclose(nnz / (cfg.batch * cfg.heads * cfg.nb * cfg.nb), 0.1, atol=1e-4)


def test_phase_work_constants():
    """The algorithmic work bench.py prices each phase at, for the headline layer: the linear pass reads K and
    V once and writes S and z; the attention kernel reads Q, K, V and writes out; a window mask reads nothing."""
    cfg = CONFIGS["c3"]
    tensor = cfg.batch * cfg.heads * cfg.n_pad * cfg.head_dim * 2
    assert tensor == 100663296
    BH, d = cfg.batch * cfg.heads, cfg.head_dim
    assert 2 * tensor + BH * (d * d + d) * 4 == 202119168  # the "linear_prepare" algorithmic_bytes
    assert 202119168 / 8e12 * 1e3 == 0.025264896            # its bound at 8 TB/s, in ms
    assert abs(659696910336.0 / 2.5e15 * 1e3 - 0.2638787641344) < 1e-12  # the attention bound at 2.5 PFLOP/s, in ms
    # a top-k layer pools Q and K of every head (and the gate rides on the same pass over Q)
    c4 = CONFIGS["c4"]
    per_head = c4.batch * c4.n_pad * c4.head_dim * 2
    assert per_head * 2 * c4.heads == 671088640


def test_cpu_pool_is_forked_before_the_gpu_and_reports_its_cores():
    """The oracle's worker count is the host's CPUs capped by OMP_NUM_THREADS, and cpu_baseline labels a full
    layer as such (a tiny layer finishes within any budget)."""
    from synth import make_inputs
    cfg = CONFIGS["c1"]
    inp = make_inputs(cfg)
    cinp, rp, ci, gate = bench.oracle_inputs_for_cpu(cfg, inp)
    pool, workers = bench.start_cpu_pool(cfg, cinp, rp, ci, gate)
    n_aff, _ = bench.host_cpus()
    assert 1 <= workers <= n_aff
    r = bench.cpu_baseline(cfg, pool, workers, 30.0)
    assert r["full_layer"] and r["cores"] == workers and r["host_cpus"] == n_aff
    assert r["kind"] == "oracle" and "full layer" in r["sample"]
