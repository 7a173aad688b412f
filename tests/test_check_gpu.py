"""salad_check_mask on the GPU: masks from salad_build_mask pass, and each kind of malformed CSR is reported
with its bit.  Only the checker ever sees the malformed masks; no attention kernel runs on them."""

import numpy as np
import pytest

from helpers import inputs, make_layer, device_tensors
from synth import CONFIGS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from block_sparse_linear_st_amd import salad as S  # noqa: E402


def _ref_bits(rp, ci, nb, col_cap):
    """The checker's definition, written out on the host."""
    bits = 0
    if rp[0] != 0:
        bits |= S.SALAD_MASK_BAD_START
    if rp[-1] < 0 or rp[-1] > col_cap:
        bits |= S.SALAD_MASK_BAD_ROW_PTR
    for r in range(len(rp) - 1):
        b, e = int(rp[r]), int(rp[r + 1])
        if b < 0 or e < b or e > col_cap:
            bits |= S.SALAD_MASK_BAD_ROW_PTR
            continue
        row = ci[b:e].astype(np.int64)
        if np.any((row < 0) | (row >= nb)):
            bits |= S.SALAD_MASK_BAD_COL
        if np.any(np.diff(row) <= 0):
            bits |= S.SALAD_MASK_BAD_ORDER
    return bits


def _check(layer, rp, ci):
    res = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    S.salad_check_mask(layer.shape, rp, ci, res)
    torch.cuda.synchronize()
    return int(res.item())


@pytest.mark.parametrize("name", ["c2", "c4", "c5"])
def test_built_masks_pass(name):
    print(f"check mask {name}", flush=True)
    cfg = CONFIGS[name]
    layer = make_layer(cfg)
    q, k, _, _ = device_tensors(inputs(name))
    layer.build_mask(q, k)
    assert _check(layer, layer.row_ptr, layer.col_idx) == 0


def test_malformed_masks_are_reported():
    print("check mask: malformed CSRs", flush=True)
    cfg = CONFIGS["c2"]
    layer = make_layer(cfg)
    layer.build_mask()
    rp0 = layer.row_ptr.cpu().numpy()
    ci0 = layer.col_idx.cpu().numpy()
    cap = ci0.size
    nb = cfg.nb
    rng = np.random.default_rng(5)
    cases = []
    rp = rp0.copy(); rp[0] = 1; cases.append(("start", rp, ci0))
    rp = rp0.copy(); rp[7] = rp[8] + 1; cases.append(("decreasing", rp, ci0))
    rp = rp0.copy(); rp[-1] = cap + 64; cases.append(("past col_cap", rp, ci0))
    rp = rp0.copy(); rp[3] = -5; cases.append(("negative", rp, ci0))
    ci = ci0.copy(); ci[rp0[5]] = nb; cases.append(("col = nb", rp0, ci))
    ci = ci0.copy(); ci[rp0[9] + 1] = -1; cases.append(("col < 0", rp0, ci))
    ci = ci0.copy(); r = 11; ci[rp0[r]], ci[rp0[r] + 1] = ci0[rp0[r] + 1], ci0[rp0[r]]; cases.append(("unsorted", rp0, ci))
    ci = ci0.copy(); r = 13; ci[rp0[r] + 1] = ci0[rp0[r]]; cases.append(("duplicate", rp0, ci))
    # a long row (more than one 64-entry chunk) unsorted across the chunk boundary
    long_rp = np.zeros_like(rp0)
    long_rp[1:] = min(cap, 100)
    long_ci = np.zeros(cap, dtype=np.int32)
    long_ci[:min(cap, 100)] = np.arange(min(cap, 100)) % nb
    cases.append(("wrap at a chunk boundary", long_rp, long_ci))
    for _ in range(6):
        ci = ci0.copy()
        ci[rng.integers(0, rp0[-1], 3)] = rng.integers(-3, nb + 3, 3)
        cases.append(("random", rp0, ci))
    for what, rp, ci in cases:
        want = _ref_bits(rp, ci, nb, cap)
        got = _check(layer, torch.from_numpy(np.ascontiguousarray(rp)).cuda(),
                     torch.from_numpy(np.ascontiguousarray(ci)).cuda())
        print(f"  {what}: bits {got} (expected {want})", flush=True)
        assert got == want, what
        if what != "random":
            assert got != 0, what
