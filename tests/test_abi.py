"""The C-ABI library: it loads, exports what include/salad.h declares, and its
host-only paths (sizing, validation before any launch) behave.  No kernel runs
here, so these tests need no GPU."""

import ctypes
import os

import pytest

from block_sparse_linear_st_amd import salad as S
from synth import CONFIGS, HeadSpec

LIB = S.LIB_PATH


def _lib():
    if not os.path.exists(LIB):
        pytest.skip("libsalad.so not built (python -m block_sparse_linear_st_amd.build)")
    return S.lib()


def test_exports_every_declared_function():
    L = _lib()
    names = S.header_functions()
    assert "salad_attn_fwd" in names and "salad_build_mask" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(S._SIGS), "binding signatures and header disagree"
    assert S.salad_version() == 100


def _shape(name, **over):
    c = CONFIGS[name]
    sh = S.make_shape(c.batch, c.heads, c.head_dim, c.T, c.H, c.W, c.block,
                      S.SALAD_BF16 if c.dtype == "bf16" else S.SALAD_F32, cuboid=c.cuboid)
    for k, v in over.items():
        setattr(sh, k, v)
    return sh


def test_status_strings():
    _lib()
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(S.salad_status_str(st), str) and S.salad_status_str(st)


def _oracle_nnz(T, H, W, block, specs, batch, order=None):
    """Expected salad_mask_nnz from the oracle: window r* by token brute force, K or every candidate; k*nb for
    top-k; (m+1)*nb for SICS (a bound); InfeasibleMask propagates."""
    from oracle import masks as om
    nb = -(-T * H * W // block)
    total = 0
    for sp in specs:
        if sp.kind == om.WINDOW:
            if T * H * W <= 4096:
                rs = om.window_rstar_bruteforce(T, H, W, block, sp.t_window, order=order)
            else:
                assert order is None
                rs = om.window_rstar_segments(T, H, W, block, sp.t_window)
            total += int(om.window_select(rs, sp.r_max, sp.density).sum()) * batch
        elif sp.kind == om.TOPK:
            total += om.topk_count(sp.density, nb) * nb * batch
        else:
            total += min(om.topk_count(sp.density, nb) + 1, nb) * nb * batch
    return total


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c9"])
def test_nnz_matches_oracle_counts(name):
    """salad_mask_nnz equals the number of entries the oracle's mask holds (window and top-k heads), and the
    (m + 1) * nb bound for SICS heads."""
    _lib()
    c = CONFIGS[name]
    order = None
    if tuple(c.cuboid) != (0, 0, 0):
        from oracle import layout as ol
        order = ol.cuboid_order(c.T, c.H, c.W, c.cuboid)
    n = S.salad_mask_nnz(_shape(name), S.make_specs(c.specs))
    assert n == _oracle_nnz(c.T, c.H, c.W, c.block, c.specs, c.batch, order)


def _tiny_grids():
    import numpy as np
    rng = np.random.default_rng(11)
    cubs = [(0, 0, 0), (0, 0, 0), (1, 8, 8), (2, 4, 8), (4, 4, 4), (1, 4, 16), (64, 1, 1), (1, 1, 64), (2, 2, 16)]
    out = []
    for i in range(36):
        T, H, W = int(rng.integers(1, 7)), int(rng.integers(1, 10)), int(rng.integers(1, 21))
        cub = cubs[i % len(cubs)]
        tw, rmax = int(rng.integers(0, 3)), int(rng.integers(-1, 4))
        out.append((T, H, W, cub, tw, rmax))
    return out


@pytest.mark.parametrize("case", _tiny_grids(), ids=str)
def test_window_candidate_count_tiny_grids(case):
    """Keep-all windows on random tiny grids, frame-major and cuboid order, with and without a spatial cap:
    the host candidate count equals the oracle's token-level brute force."""
    _lib()
    from oracle import layout as ol
    T, H, W, cub, tw, rmax = case
    sh = S.make_shape(2, 1, 64, T, H, W, 64, S.SALAD_BF16, cuboid=cub)
    spec = [HeadSpec(0, tw, rmax, 0.0)]
    order = None if cub == (0, 0, 0) else ol.cuboid_order(T, H, W, cub)
    assert S.salad_mask_nnz(sh, S.make_specs(spec)) == _oracle_nnz(T, H, W, 64, spec, 2, order)


def test_infeasible_window_is_rejected_before_launch():
    """A window asking for more pairs than it has candidates: the oracle raises InfeasibleMask, and the library
    returns SALAD_EINFEASIBLE from salad_mask_nnz and from salad_build_mask, before any launch."""
    L = _lib()
    from oracle import masks as om
    c = CONFIGS["c2"]
    # +-0 frames with a spatial cap of 1 on the 8x16x16 grid has few candidates; ask for half of all pairs
    specs = [HeadSpec(0, 0, 1, 0.5)] + list(c.specs[1:])
    with pytest.raises(om.InfeasibleMask):
        om.build_masks(c.T, c.H, c.W, c.block, specs, c.batch)
    sh = _shape("c2")
    arr = S.make_specs(specs)
    assert L.salad_mask_nnz(ctypes.byref(sh), arr) == S.SALAD_EINFEASIBLE
    fake = ctypes.c_void_p(0x100000)
    assert L.salad_build_mask(ctypes.byref(sh), arr, None, None, fake, fake, 10 ** 9, None, None, fake,
                              S.salad_workspace_bytes(sh), None) == S.SALAD_EINFEASIBLE
    # exactly the candidate count is feasible: K = every candidate (keep-all gives the same count)
    n_cand = S.salad_mask_nnz(sh, S.make_specs([HeadSpec(0, 0, 1, 0.0)] * 12)) // 12
    rho = (n_cand - 0.25) / (c.nb * c.nb)  # floor(rho*nb^2 + 0.5) == n_cand
    assert om.window_count(rho, c.nb, c.nb) == n_cand
    feas = S.make_specs([HeadSpec(0, 0, 1, rho)] * 12)
    assert S.salad_mask_nnz(sh, feas) == 12 * n_cand
    more = S.make_specs([HeadSpec(0, 0, 1, (n_cand + 1.0) / (c.nb * c.nb))] * 12)
    assert L.salad_mask_nnz(ctypes.byref(sh), more) == S.SALAD_EINFEASIBLE


def test_mask_over_int32_entries_is_unsupported():
    """A keep-all window whose CSR would hold more than INT32_MAX entries: salad_mask_nnz gives the exact
    int64 count, salad_build_mask refuses it (row_ptr is int32) before any launch."""
    L = _lib()
    nb = 46340
    sh = S.make_shape(2, 1, 64, 1, nb, 64, 64, S.SALAD_BF16)  # one frame: every pair is a candidate
    specs = S.make_specs([HeadSpec(0, 0, -1, 0.0)])
    assert S.salad_mask_nnz(sh, specs) == 2 * nb * nb
    fake = ctypes.c_void_p(0x100000)
    assert L.salad_build_mask(ctypes.byref(sh), specs, None, None, fake, fake, 2 ** 40, None, None, fake,
                              S.salad_workspace_bytes(sh), None) == S.SALAD_EUNSUPPORTED
    huge = S.make_specs([HeadSpec(0, 0, -1, 3.0e38)])  # K far beyond nb^2: infeasible, no overflow
    assert L.salad_mask_nnz(ctypes.byref(sh), huge) == S.SALAD_EINFEASIBLE


def test_workspace_and_shape_validation():
    _lib()
    assert S.salad_workspace_bytes(_shape("c3")) > 0
    assert S.salad_workspace_bytes(_shape("c3", head_dim=96)) == 0
    assert S.salad_workspace_bytes(_shape("c3", block=32)) == 0
    assert S.salad_workspace_bytes(_shape("c3", n_pad=32760)) == 0  # not a multiple of the block
    assert S.salad_workspace_bytes(_shape("c3", n_pad=32768 + 64)) == 0  # a whole padded block
    assert S.salad_workspace_bytes(_shape("c3", heads=129)) == 0
    assert S.salad_workspace_bytes(_shape("c3", dtype=5)) == 0
    specs = S.make_specs(CONFIGS["c3"].specs)
    assert S.lib().salad_mask_nnz(ctypes.byref(_shape("c3", head_dim=96)), specs) == S.SALAD_EUNSUPPORTED
    assert S.lib().salad_mask_nnz(ctypes.byref(_shape("c3", n_pad=5)), specs) == S.SALAD_EINVAL
    bad = S.make_specs([HeadSpec(7, 1, -1, 0.1)] * 12)
    assert S.lib().salad_mask_nnz(ctypes.byref(_shape("c3")), bad) == S.SALAD_EINVAL


def test_entry_points_reject_bad_arguments_before_launch():
    L = _lib()
    sh = _shape("c3")
    specs = S.make_specs(CONFIGS["c3"].specs)
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    ws_bytes = S.salad_workspace_bytes(sh)
    # null shape / null buffers
    assert L.salad_build_mask(None, specs, None, None, fake, fake, 10 ** 7, None, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_build_mask(ctypes.byref(sh), specs, None, None, None, fake, 10 ** 7, None, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    # col_idx too small, workspace too small
    assert L.salad_build_mask(ctypes.byref(sh), specs, None, None, fake, fake, 10, None, None, fake, ws_bytes, None) == S.SALAD_ENOSPACE
    assert L.salad_build_mask(ctypes.byref(sh), specs, None, None, fake, fake, 10 ** 7, None, None, fake, 16, None) == S.SALAD_ENOSPACE
    # gate without w_g
    assert L.salad_build_mask(ctypes.byref(sh), specs, fake, None, fake, fake, 10 ** 7, None, fake, fake, ws_bytes, None) == S.SALAD_EINVAL
    # top-k heads need q and k
    topk = S.make_specs(CONFIGS["c4"].specs[:12])
    assert L.salad_build_mask(ctypes.byref(sh), topk, None, None, fake, fake, 10 ** 7, None, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    # misaligned pointers
    odd = ctypes.c_void_p(0x100004)
    assert L.salad_attn_fwd(ctypes.byref(sh), odd, fake, fake, fake, fake, fake, fake, 1e-6, 0.0, 0.0, fake, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    # w_lin is staged in 16-byte chunks
    assert L.salad_attn_fwd(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, odd, 1e-6, 0.0, 0.0, fake, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_linear_prepare(ctypes.byref(sh), fake, fake, fake, odd, 0.0, fake, ws_bytes, None) == S.SALAD_EINVAL
    # missing gate / w_lin / out; bad eps
    assert L.salad_attn_fwd(ctypes.byref(sh), fake, fake, fake, fake, fake, None, fake, 1e-6, 0.0, 0.0, fake, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_attn_fwd(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, None, 1e-6, 0.0, 0.0, fake, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_attn_fwd(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, fake, -1.0, 0.0, 0.0, fake, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_attn_fwd(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, fake, 1e-6, 0.0, 0.0, fake, None, fake, 1, None) == S.SALAD_ENOSPACE
    assert L.salad_attn_apply(ctypes.byref(sh), fake, fake, fake, fake, fake, None, 1e-6, 0.0, 0.0, fake, None, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_linear_prepare(ctypes.byref(sh), fake, fake, None, fake, 0.0, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_linear_prepare(ctypes.byref(sh), fake, fake, fake, fake, float("nan"), fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_linear_state(ctypes.byref(sh), fake, None, fake, fake, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_gate_from_q(ctypes.byref(sh), fake, None, fake, fake, ws_bytes, None) == S.SALAD_EINVAL
    assert L.salad_attn_fwd_branches(ctypes.byref(_shape("c3", block=32)), fake, fake, fake, fake, fake, 1e-6, 0.0, fake, None, fake, ws_bytes, None) == S.SALAD_EUNSUPPORTED


def test_binding_refuses_host_tensors():
    _lib()
    import torch
    c = CONFIGS["c1"]
    sh = _shape("c1")
    t = torch.zeros(4)
    with pytest.raises(S.SaladError):
        S.salad_linear_state(sh, t, t, t, t, t)


def test_sics_specs():
    """SICS heads: the bound is (m + 1) * nb per (b, h); K is required; nb above 4096 is not built."""
    c = CONFIGS["c7"]
    sh = _shape("c7")
    specs = S.make_specs(c.specs)
    from oracle import masks as om
    m = om.topk_count(c.specs[0].density, c.nb)
    assert S.salad_mask_nnz(sh, specs) == c.batch * c.heads * (m + 1) * c.nb
    L = S.lib()
    fake = ctypes.c_void_p(0x1000)
    ws_bytes = S.salad_workspace_bytes(sh)
    # k missing for a SICS head
    assert L.salad_build_mask(ctypes.byref(sh), specs, fake, None, fake, fake, 10 ** 7, None, None, fake,
                              ws_bytes, None) == S.SALAD_EINVAL
    big = S.make_shape(1, 1, 128, 1, 1, 64 * 4097, 64, S.SALAD_BF16)
    one = S.make_specs([c.specs[0]])
    assert S.lib().salad_mask_nnz(ctypes.byref(big), one) == S.SALAD_EUNSUPPORTED


# ------------------------------------------------------------------ cuboid storage order (host paths)

ORDER_GRIDS = [
    (21, 30, 52, 64, (4, 4, 4)), (21, 30, 52, 64, (1, 8, 8)), (21, 30, 52, 64, (2, 4, 8)),
    (41, 45, 80, 128, (2, 8, 8)), (41, 45, 80, 128, (1, 8, 16)), (5, 10, 14, 64, (2, 4, 8)),
    (3, 7, 5, 64, (4, 4, 4)), (7, 9, 11, 64, (64, 1, 1)), (13, 1, 1, 64, (4, 4, 4)), (6, 6, 6, 64, (4, 4, 4)),
    (21, 30, 52, 64, (0, 0, 0)),
]


@pytest.mark.parametrize("grid", ORDER_GRIDS, ids=str)
def test_token_order_matches_oracle(grid):
    """salad_token_order (a pure host function) lists the oracle's storage order, padding slots mapped to themselves."""
    _lib()
    import numpy as np
    from oracle import layout as ol
    T, H, W, blk, cub = grid
    sh = S.make_shape(1, 1, 64, T, H, W, blk, S.SALAD_BF16, cuboid=cub)
    got = S.salad_token_order(sh)
    N = T * H * W
    np.testing.assert_array_equal(got[:N], ol.cuboid_order(T, H, W, cub))
    np.testing.assert_array_equal(got[N:], np.arange(N, sh.n_pad))


def test_cuboid_shape_validation():
    _lib()
    assert S.salad_workspace_bytes(_shape("c8")) >= S.salad_workspace_bytes(_shape("c3"))  # + box lists
    assert S.salad_workspace_bytes(_shape("c8", cuboid_w=16)) == 0       # 1*8*16 != 64
    assert S.salad_workspace_bytes(_shape("c8", cuboid_w=0)) == 0        # partly zero
    assert S.salad_workspace_bytes(_shape("c8", cuboid_t=-1, cuboid_h=-8)) == 0
    assert S.salad_workspace_bytes(_shape("c8", cuboid_t=1, cuboid_h=1, cuboid_w=64)) > 0
    assert S.salad_workspace_bytes(_shape("c3", cuboid_t=64, cuboid_h=1, cuboid_w=1)) > 0  # taller than T
    bad = _shape("c8", cuboid_h=2)  # 1*2*8 != 64
    order = (ctypes.c_int32 * bad.n_pad)()
    assert S.lib().salad_token_order(ctypes.byref(bad), order) == S.SALAD_EINVAL
    assert S.lib().salad_token_order(ctypes.byref(_shape("c8")), None) == S.SALAD_EINVAL


def test_permute_rejects_bad_arguments_before_launch():
    L = _lib()
    sh = _shape("c8")
    nbytes = sh.batch * sh.heads * sh.n_pad * sh.head_dim * 2
    a = ctypes.c_void_p(0x10000000)
    b = ctypes.c_void_p(0x10000000 + nbytes)       # adjacent, not overlapping: would launch, not used here
    over = ctypes.c_void_p(0x10000000 + nbytes - 16)
    odd = ctypes.c_void_p(0x10000008)
    assert L.salad_permute_tokens(ctypes.byref(sh), 0, a, over, None) == S.SALAD_EINVAL
    assert L.salad_permute_tokens(ctypes.byref(sh), 0, over, a, None) == S.SALAD_EINVAL
    assert L.salad_permute_tokens(ctypes.byref(sh), 0, a, a, None) == S.SALAD_EINVAL
    assert L.salad_permute_tokens(ctypes.byref(sh), 2, a, b, None) == S.SALAD_EINVAL
    assert L.salad_permute_tokens(ctypes.byref(sh), 0, None, b, None) == S.SALAD_EINVAL
    assert L.salad_permute_tokens(ctypes.byref(sh), 1, odd, b, None) == S.SALAD_EINVAL
    assert L.salad_permute_tokens(ctypes.byref(_shape("c8", cuboid_w=2)), 0, a, b, None) == S.SALAD_EINVAL  # 1*8*2


def test_backward_rejects_bad_arguments_before_launch():
    L = _lib()
    sh = _shape("c3")
    ws_bytes = S.salad_bwd_workspace_bytes(sh)
    assert ws_bytes > S.salad_workspace_bytes(sh)
    assert S.salad_bwd_workspace_bytes(_shape("c3", head_dim=96)) == 0
    fake = ctypes.c_void_p(0x100000)
    args = [fake] * 5 + [fake, fake, 1e-6, 0.0, fake, None, fake, fake, fake, fake, fake, fake, fake, ws_bytes, None]
    # q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, out, lse, dout, dq, dk, dv, dw, dgate, ws, ws_bytes, stream

    def call(shape=sh, **over):
        a = list(args)
        names = ["q", "k", "v", "row_ptr", "col_idx", "gate", "w_lin", "eps", "scale", "out", "lse", "dout", "dq",
                 "dk", "dv", "dw", "dgate", "ws", "ws_bytes", "stream"]
        for key, val in over.items():
            a[names.index(key)] = val
        return L.salad_attn_bwd(ctypes.byref(shape), *a)

    assert call(shape=_shape("c1")) == S.SALAD_EUNSUPPORTED   # fp32 layer
    assert call(dout=None) == S.SALAD_EINVAL
    assert call(dgate=None) == S.SALAD_EINVAL
    assert call(dq=ctypes.c_void_p(0x100004)) == S.SALAD_EINVAL
    assert call(lse=ctypes.c_void_p(0x100004)) == S.SALAD_EINVAL  # forward statistic not 16-byte aligned
    assert call(eps=-1.0) == S.SALAD_EINVAL
    assert call(scale=float("inf")) == S.SALAD_EINVAL
    assert call(ws_bytes=ws_bytes - 1) == S.SALAD_ENOSPACE


def test_check_mask_rejects_bad_arguments_before_launch():
    L = _lib()
    sh = _shape("c2")
    fake = ctypes.c_void_p(0x100000)
    assert L.salad_check_mask(None, fake, fake, 10, fake, None) == S.SALAD_EINVAL
    assert L.salad_check_mask(ctypes.byref(sh), None, fake, 10, fake, None) == S.SALAD_EINVAL
    assert L.salad_check_mask(ctypes.byref(sh), fake, None, 10, fake, None) == S.SALAD_EINVAL
    assert L.salad_check_mask(ctypes.byref(sh), fake, fake, 10, None, None) == S.SALAD_EINVAL
    assert L.salad_check_mask(ctypes.byref(sh), fake, fake, -1, fake, None) == S.SALAD_EINVAL
    assert L.salad_check_mask(ctypes.byref(_shape("c2", head_dim=96)), fake, fake, 10, fake, None) == \
        S.SALAD_EUNSUPPORTED


def test_noalloc_forward_refuses_layers_beyond_its_scratch():
    """salad_attn_fwd_noalloc checks its arguments and the 32 MiB scratch limit before any HIP call."""
    L = _lib()
    fake = ctypes.c_void_p(0x100000)
    big = S.make_shape(4, 128, 128, 21, 30, 52, 64, S.SALAD_BF16)  # 512 (b, h): linear state over 32 MiB
    args = [fake] * 7 + [1e-6, 0.0, 0.0, fake, None, None]
    assert L.salad_attn_fwd_noalloc(ctypes.byref(big), *args) == S.SALAD_ENOSPACE
    sh = _shape("c3")
    assert L.salad_attn_fwd_noalloc(None, *args) == S.SALAD_EINVAL
    bad = list(args)
    bad[5] = None  # gate
    assert L.salad_attn_fwd_noalloc(ctypes.byref(sh), *bad) == S.SALAD_EINVAL
    bad = list(args)
    bad[0] = ctypes.c_void_p(0x100004)  # misaligned q
    assert L.salad_attn_fwd_noalloc(ctypes.byref(sh), *bad) == S.SALAD_EINVAL
    assert L.salad_attn_fwd_noalloc(ctypes.byref(_shape("c1")), *(args[:11] + [fake, None])) == \
        S.SALAD_EUNSUPPORTED  # lse on an fp32 layer
