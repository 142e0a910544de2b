"""The sampler backward that forms the MI gradient itself
(ngv_warp_bwd_adam_mi, the second sweep of a fused step) against the calls it
replaces: the MI gradient sweep into gW (ngv_mi_grad, adding to another
term's gradient or into a zeroed buffer) followed by ngv_warp_bwd_adam. The
fused call recomputes W from its own gathers and reads F, so u, m1, m2 and
the affine sums must come out bit for bit the same. Shapes are ragged
(partial tiles and work items), bin counts and ranges vary, and the step
number comes from the host or the device. The oracle parity of the path
itself is in test_gpu_step.py (the default step) and test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

from non_gemm_voxel_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ngv():
    from non_gemm_voxel_amd import ngv as lib
    lib.lib()
    return lib


def _say(*a):
    print("[case]", *a, flush=True)


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x)).to(DEV)


def _affine(seed):
    r = synth.scalars(seed, 1, 12)
    R = synth.euler_rotation(*(0.15 * (2 * r[:3] - 1)))
    A = R @ np.diag(1.0 + 0.05 * (2 * r[3:6] - 1))
    t = 0.04 * (2 * r[6:9] - 1)
    return A.astype(np.float32), t.astype(np.float32)


CASES = [
    # output shape, moving shape, bins, W range, with another term's gW, device step number
    ((29, 40, 66), (31, 38, 70), 32, (0.0, 1.0), True, False),
    ((29, 40, 66), (31, 38, 70), 32, (0.0, 1.0), False, True),
    ((17, 9, 130), (17, 9, 130), 16, (0.1, 0.9), True, True),
    ((5, 33, 65), (6, 30, 60), 64, (-0.2, 1.2), False, False),
    ((1, 3, 7), (2, 3, 7), 8, (0.0, 1.0), True, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_mi_grad_then_fused_backward(ngv, case):
    oshape, mshape, bins, wr, other, on_dev = CASES[case]
    _say("warp_bwd_adam_mi", oshape, mshape, bins, wr, "gW" if other else "no gW", "step_dev" if on_dev else "")
    seed = 70 + case
    M = _dev(synth.random_volume(mshape, seed, 0).numpy())
    F = _dev(synth.random_volume(oshape, seed, 1, -0.05, 1.05).numpy())
    A, t = _affine(seed)
    vol = (3,) + oshape
    u = (0.05 * synth.random_field(oshape, seed, 2, 1.0)).numpy()
    g_other = synth.random_volume(oshape, seed, 3, -1e-6, 1e-6).numpy()
    m1 = synth.random_volume(vol, seed, 4, -0.1, 0.1).numpy()
    m2 = synth.random_volume(vol, seed, 5, 0.0, 0.1).numpy()
    xf = ngv.make_xform(A, t)
    step, lr = 4, 0.02
    # the step's forward and MI forward (histogram, loss, table in ws)
    W = torch.empty(oshape, device=DEV)
    ngv.ngv_warp_fwd(M, _dev(u), xf, W)
    ws = torch.empty(ngv.ngv_workspace_bytes(bins, 9), dtype=torch.uint8, device=DEV)
    loss = torch.zeros(1, dtype=torch.float64, device=DEV)
    kw = dict(bins=bins, frange=(0.0, 1.0), wrange=wr, weight=1.5)
    ngv.ngv_mi_loss_fwd_bwd(F, W, loss, None, ws=ws, **kw)
    sd = torch.full((1,), step, dtype=torch.int32, device=DEV) if on_dev else None
    out = []
    for fused in (False, True):
        ud, m1d, m2d = _dev(u), _dev(m1), _dev(m2)
        gA = torch.full((9,), 0.25, dtype=torch.float64, device=DEV)
        gt = torch.full((3,), 0.25, dtype=torch.float64, device=DEV)
        if fused:
            ngv.ngv_warp_bwd_adam_mi(M, ud, xf, F, _dev(g_other) if other else None, m1d, m2d, step, lr, gA, gt,
                                     accumulate_affine=True, ws=ws, step_dev=sd, **kw)
        else:
            gW = _dev(g_other) if other else torch.zeros(oshape, device=DEV)
            ngv.ngv_mi_grad(F, W, gW, accumulate=other, ws=ws, **kw)
            ngv.ngv_warp_bwd_adam(M, ud, xf, gW, m1d, m2d, step, lr, gA, gt, accumulate_affine=True, ws=ws,
                                  step_dev=sd)
        out.append((ud, m1d, m2d, gA, gt))
    torch.cuda.synchronize()
    for a, b, what in zip(out[0], out[1], ("u", "m1", "m2", "dA", "dt")):
        assert torch.equal(a, b), what
    # the update moved u: the MI gradient is not zero here
    assert not torch.equal(out[1][0], _dev(u))


SLAB_CASES = [
    # output shape, moving shape, slabs, bins, with another term's gW
    ((29, 40, 66), (31, 38, 70), 3, 32, True),
    ((40, 33, 65), (36, 30, 60), 8, 16, False),
    ((21, 19, 37), (21, 19, 37), 2, 64, True),
    ((23, 30, 40), (25, 28, 44), 4, 128, True),  # a 64 KB table in LDS
]


@pytest.mark.parametrize("case", range(len(SLAB_CASES)))
def test_slab_sequence_matches_mi_grad_then_slab_backward(ngv, case):
    """The backward slab sequence forming the MI gradient from the stored W
    (ngv_warp_bwd_adam_slab_mi) against the MI gradient sweep into gW followed
    by ngv_warp_bwd_adam_slab: u, m1, m2 and the affine sums bit for bit."""
    oshape, mshape, slabs, bins, other = SLAB_CASES[case]
    _say("warp_bwd_adam_slab_mi", oshape, mshape, slabs, bins, "gW" if other else "no gW")
    seed = 80 + case
    M = _dev(synth.random_volume(mshape, seed, 0).numpy())
    F = _dev(synth.random_volume(oshape, seed, 1, -0.05, 1.05).numpy())
    A, t = _affine(seed)
    vol = (3,) + oshape
    u = (0.05 * synth.random_field(oshape, seed, 2, 1.0)).numpy()
    g_other = synth.random_volume(oshape, seed, 3, -1e-6, 1e-6).numpy()
    m1 = synth.random_volume(vol, seed, 4, -0.1, 0.1).numpy()
    m2 = synth.random_volume(vol, seed, 5, 0.0, 0.1).numpy()
    xf = ngv.make_xform(A, t)
    step, lr = 3, 0.02
    nz = mshape[0]
    bounds = [round(h * nz / slabs) for h in range(slabs + 1)]
    zr = torch.zeros(2, dtype=torch.float64, device=DEV)
    ws = torch.empty(ngv.ngv_workspace_bytes(bins, 9), dtype=torch.uint8, device=DEV)
    ud0 = _dev(u)
    ngv.ngv_warp_zrange(ud0, xf, zr, mshape, ws=ws)
    sl = [(bounds[h], bounds[h + 1] - bounds[h], zr) for h in range(slabs)]
    views = [M[z0:z0 + n] for z0, n, _ in sl]
    W = torch.empty(oshape, device=DEV)
    for h in range(slabs):
        ngv.ngv_warp_fwd_slab(views[h], ud0, xf, W, sl[h], mdims=mshape)
    loss = torch.zeros(1, dtype=torch.float64, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd(F, W, loss, None, bins=bins, ws=ws)
    out = []
    for fused in (False, True):
        ud, m1d, m2d = _dev(u), _dev(m1), _dev(m2)
        gA = torch.zeros(9, dtype=torch.float64, device=DEV)
        gt = torch.zeros(3, dtype=torch.float64, device=DEV)
        gu = torch.empty(vol, device=DEV)
        if not fused:
            gW = _dev(g_other) if other else torch.zeros(oshape, device=DEV)
            ngv.ngv_mi_grad(F, W, gW, bins=bins, accumulate=True, ws=ws)
        for h in range(slabs):
            kw = dict(mdims=mshape, accumulate_affine=h > 0, ws=ws)
            if fused:
                ngv.ngv_warp_bwd_adam_slab_mi(views[h], ud, xf, _dev(g_other) if other else None, F, W, gu, m1d, m2d,
                                              step, lr, gA, gt, sl[h], bins=bins, **kw)
            else:
                ngv.ngv_warp_bwd_adam_slab(views[h], ud, xf, gW, gu, m1d, m2d, step, lr, gA, gt, sl[h], **kw)
        out.append((ud, m1d, m2d, gA, gt))
    torch.cuda.synchronize()
    for a, b, what in zip(out[0], out[1], ("u", "m1", "m2", "dA", "dt")):
        assert torch.equal(a, b), what
    assert not torch.equal(out[1][0], _dev(u))


@pytest.mark.parametrize("wl_name,shape,slabs", [("c1", None, 1), ("c3", (48, 48, 48), 1), ("c4", (40, 48, 56), 1),
                                                 ("c5", (48, 56, 40), 8)])
def test_step_matches_separate_mi_gradient(wl_name, shape, slabs):
    """Three default steps (MI gradient formed in the backward) against three
    steps with the MI call writing its gradient: the same state bit for bit
    (with 8 slabs, from the stored W)."""
    from non_gemm_voxel_amd.step import RegistrationStep
    wl = synth.WORKLOADS[wl_name]
    _say("step mi in backward", wl_name, shape, "slabs", slabs)
    c = synth.make_case(wl, shape=shape)
    sts = [RegistrationStep(c.F.to(DEV), c.M.to(DEV), c.A, c.t, bins=wl.bins, win=wl.win, lr=c.lr, slabs=slabs,
                            mi_in_backward=flag) for flag in (False, True)]
    assert not sts[0].mi_bwd and sts[1].mi_bwd
    for st in sts:
        for _ in range(3):
            st.step()
    torch.cuda.synchronize()
    for name in ("u", "m1", "m2", "gA", "gt", "W", "loss"):
        assert torch.equal(getattr(sts[0], name), getattr(sts[1], name)), name


@pytest.mark.timeout(600)
def test_full_size_step_matches_separate_mi_gradient():
    """The 640 x 768 x 640 workload, one step each way."""
    from non_gemm_voxel_amd.step import RegistrationStep
    wl = synth.WORKLOADS["c4"]
    _say("step mi in backward, full size", wl.shape)
    c = synth.make_case(wl, device=DEV)
    res = []
    for flag in (False, True):
        st = RegistrationStep(c.F, c.M, c.A, c.t, bins=wl.bins, win=wl.win, lr=c.lr, mi_in_backward=flag)
        st.step()
        torch.cuda.synchronize()
        res.append({k: getattr(st, k) for k in ("u", "m1", "m2", "gA", "gt", "loss")})
        del st
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k
