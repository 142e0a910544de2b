"""Parity of each HIP entry point against the oracle, on seeded inputs at
sizes that span several tiles and end in ragged tails.

Every call goes through the C ABI (the ctypes binding); every expected value
comes from the oracle on the same inputs, never from the HIP path.
"""
import numpy as np
import pytest
import torch

from non_gemm_voxel_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ngv():
    from non_gemm_voxel_amd import ngv as lib
    lib.lib()
    return lib


def _say(*a):
    print("[case]", *a, flush=True)


def _rand_affine(seed, rot=0.15, scl=0.1, tr=0.1):
    r = synth.scalars(seed, 1, 12)
    R = synth.euler_rotation(*(rot * (2 * r[:3] - 1)))
    A = R @ np.diag(1.0 + scl * (2 * r[3:6] - 1))
    t = tr * (2 * r[6:9] - 1)
    return A.astype(np.float32), t.astype(np.float32)


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x)).to(DEV)


# ----------------------------------------------------------------- sampler

WARP_CASES = [
    # (output shape, moving shape, seed, S, bounds)
    ((37, 45, 71), (37, 45, 71), 1, None, None),
    ((19, 70, 130), (23, 64, 129), 2, np.diag([0.5, 1.0, 2.0]), None),
    ((33, 31, 29), (40, 33, 27), 3, np.array([[0.5, 0.1, 0.0], [0.0, 1.0, -0.2], [0.3, 0.0, 2.0]]),
     ((-0.9, -1.0, -0.8), (1.0, 0.85, 0.9))),
]


@pytest.mark.parametrize("case", range(len(WARP_CASES)))
def test_warp_fwd_parity(orc, ngv, case):
    oshape, mshape, seed, S, bounds = WARP_CASES[case]
    _say("warp_fwd", oshape, mshape, seed)
    M = synth.random_volume(mshape, seed, 0).numpy()
    A, t = _rand_affine(seed)
    u = (0.05 * synth.random_field(oshape, seed, 6, 1.0)).numpy()
    xmin, xmax = bounds if bounds else ((-1, -1, -1), (1, 1, 1))
    S = np.eye(3) if S is None else S
    xf = ngv.make_xform(A, t, S, xmin, xmax)
    W = torch.empty(oshape, dtype=torch.float32, device=DEV)
    ngv.ngv_warp_fwd(_dev(M), _dev(u), xf, W)
    torch.cuda.synchronize()
    ref = orc.warp_fwd(M, u, orc.pack_prm(A, t, S, xmin, xmax))
    P.elementwise(P.to_np(W), ref, P.RTOL_W, what="W")


def test_warp_identity_is_bit_exact(ngv):
    _say("warp_fwd identity")
    shape = (21, 34, 67)
    M = synth.random_volume(shape, 7, 0).to(DEV)
    u = torch.zeros((3,) + shape, device=DEV)
    W = torch.empty(shape, device=DEV)
    ngv.ngv_warp_fwd(M, u, ngv.make_xform(), W)
    torch.cuda.synchronize()
    assert torch.equal(W, M)


def test_warp_slabs_sum_to_whole(orc, ngv):
    """Key design 4: the moving image in z-slabs (ragged), partial results
    accumulated, equals the unsplit sampler (forward and backward)."""
    _say("warp slabs")
    oshape, mshape = (29, 40, 66), (31, 38, 70)
    M = synth.random_volume(mshape, 8, 0).numpy()
    A, t = _rand_affine(8)
    u = (0.05 * synth.random_field(oshape, 8, 6, 1.0)).numpy()
    gW = synth.random_volume(oshape, 8, 9, -1.0, 1.0).numpy()
    xf = ngv.make_xform(A, t)
    Md, ud, gWd = _dev(M), _dev(u), _dev(gW)
    W1 = torch.empty(oshape, device=DEV)
    ngv.ngv_warp_fwd(Md, ud, xf, W1)
    gu1 = torch.empty((3,) + oshape, device=DEV)
    gA1 = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt1 = torch.zeros(3, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_bwd(Md, ud, xf, gWd, gu1, gA1, gt1)
    W2 = torch.empty(oshape, device=DEV)
    gu2 = torch.empty((3,) + oshape, device=DEV)
    gA2 = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt2 = torch.zeros(3, dtype=torch.float64, device=DEV)
    for h, (z0, z1) in enumerate([(0, 7), (7, 8), (8, 20), (20, 31)]):
        Mh = Md[z0:z1].contiguous()
        ngv.ngv_warp_fwd(Mh, ud, xf, W2, mdims=mshape, slab=(z0, z1 - z0), accumulate=h > 0)
        ngv.ngv_warp_bwd(Mh, ud, xf, gWd, gu2, gA2, gt2, mdims=mshape, slab=(z0, z1 - z0), accumulate=h > 0)
    torch.cuda.synchronize()
    # each voxel's slab sum adds at most 2 nonzero partials: a few ulp
    assert torch.allclose(W2, W1, rtol=1e-6, atol=1e-7)
    assert torch.allclose(gu2, gu1, rtol=1e-5, atol=1e-6 * float(gu1.abs().max()))
    ref = orc.warp_fwd(M, u, orc.pack_prm(A, t))
    P.elementwise(P.to_np(W2), ref, P.RTOL_W, what="W slabs")
    _, dA, dt, mag = orc.warp_bwd(M, u, orc.pack_prm(A, t), gW.astype(np.float64))
    P.affine_sums(P.to_np(gA2), dA, mag, "dA slabs")
    P.affine_sums(P.to_np(gt2), dt, mag, "dt slabs")


@pytest.mark.parametrize("case", range(len(WARP_CASES)))
def test_warp_bwd_parity(orc, ngv, case):
    oshape, mshape, seed, S, bounds = WARP_CASES[case]
    _say("warp_bwd", oshape, mshape, seed)
    M = synth.random_volume(mshape, seed, 0).numpy()
    A, t = _rand_affine(seed)
    u = (0.05 * synth.random_field(oshape, seed, 6, 1.0)).numpy()
    gW = synth.random_volume(oshape, seed, 9, -1.0, 1.0).numpy()
    xmin, xmax = bounds if bounds else ((-1, -1, -1), (1, 1, 1))
    S = np.eye(3) if S is None else S
    xf = ngv.make_xform(A, t, S, xmin, xmax)
    gu = torch.empty((3,) + oshape, device=DEV)
    gA = torch.empty(9, dtype=torch.float64, device=DEV)
    gt = torch.empty(3, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_bwd(_dev(M), _dev(u), xf, _dev(gW), gu, gA, gt)
    torch.cuda.synchronize()
    prm = orc.pack_prm(A, t, S, xmin, xmax)
    gu_ref, dA, dt, mag = orc.warp_bwd(M, u, prm, gW.astype(np.float64))
    _, kink = orc.warp_fwd(M, u, prm, want_kink=True)
    mask = P.off_kink(kink)
    for k in range(3):
        P.elementwise(P.to_np(gu)[k], gu_ref[k], P.RTOL_GRAD, mask=mask, what=f"gu[{k}]")
    P.affine_sums(P.to_np(gA), dA.ravel(), mag, "dA")
    P.affine_sums(P.to_np(gt), dt, mag, "dt")


def test_warp_accumulate(ngv):
    _say("warp accumulate")
    shape = (9, 20, 70)
    M = synth.random_volume(shape, 9, 0).to(DEV)
    u = (0.05 * synth.random_field(shape, 9, 6, 1.0)).to(DEV)
    xf = ngv.make_xform(*_rand_affine(9))
    W = torch.empty(shape, device=DEV)
    ngv.ngv_warp_fwd(M, u, xf, W)
    W2 = torch.full(shape, 0.5, device=DEV)
    ngv.ngv_warp_fwd(M, u, xf, W2, accumulate=True)
    gW = synth.random_volume(shape, 9, 9, -1.0, 1.0).to(DEV)
    gu = torch.empty((3,) + shape, device=DEV)
    gA = torch.empty(9, dtype=torch.float64, device=DEV)
    gt = torch.empty(3, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_bwd(M, u, xf, gW, gu, gA, gt)
    gu2 = torch.full((3,) + shape, -1.0, device=DEV)
    gA2 = torch.full((9,), 2.0, dtype=torch.float64, device=DEV)
    gt2 = torch.full((3,), 3.0, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_bwd(M, u, xf, gW, gu2, gA2, gt2, accumulate=True)
    torch.cuda.synchronize()
    assert torch.allclose(W2, W + 0.5, atol=1e-6)
    assert torch.allclose(gu2, gu - 1.0, atol=1e-5)
    assert torch.allclose(gA2, gA + 2.0, rtol=1e-12, atol=1e-9)
    assert torch.allclose(gt2, gt + 3.0, rtol=1e-12, atol=1e-9)


# ---------------------------------------------------------------------- MI

MI_CASES = [
    ("random", (23, 41, 67), 16),
    ("random", (17, 33, 129), 32),
    ("random", (9, 64, 64), 64),
    ("brain", (40, 48, 56), 32),
    # the largest bin count whose histogram fits in LDS, and beyond it the
    # global histogram and table
    ("random", (19, 37, 53), 128),
    ("random", (21, 40, 61), 129),
    ("random", (33, 48, 64), 256),
    ("brain", (40, 48, 56), 256),
]


def _mi_inputs(kind, shape, seed=5):
    if kind == "random":
        F = synth.random_volume(shape, seed, 0, -0.05, 1.05).numpy()
        W = (0.6 * F + 0.4 * synth.random_volume(shape, seed, 1).numpy()).astype(np.float32)
        W.reshape(-1)[:4] = [0.0, 1.0, -0.2, 1.3]  # clamp edges and beyond
    else:
        c = synth.make_case("c3", shape=shape)
        F, W = c.F.numpy(), c.M.numpy()
    return F, W


@pytest.mark.parametrize("case", range(len(MI_CASES)))
def test_mi_parity(orc, ngv, case):
    kind, shape, bins = MI_CASES[case]
    _say("mi", kind, shape, bins)
    F, W = _mi_inputs(kind, shape)
    loss = torch.empty(1, dtype=torch.float64, device=DEV)
    gW = torch.empty(shape, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd(_dev(F), _dev(W), loss, gW, bins=bins, weight=1.25)
    torch.cuda.synchronize()
    lo, go, H = orc.mi_loss_grad(F, W.astype(np.float64), bins=bins, weight=1.25)
    P.scalar(float(loss[0]), lo, what="MI loss")
    _, L = orc.mi_finalize(H, F.size)
    mags = [orc.mi_grad_values(F, W.astype(np.float64), L, bins=bins, weight=1.25, N=F.size,
                               mode=m).reshape(F.shape) for m in (1, 2)]
    P.within(P.to_np(gW), go, P.mi_grad_bar(go, *mags, bins), what="MI gW")


def test_mi_deterministic_and_accumulate(ngv):
    _say("mi determinism")
    F, W = _mi_inputs("brain", (33, 40, 50))
    F, W = _dev(F), _dev(W)
    l1 = torch.empty(1, dtype=torch.float64, device=DEV)
    l2 = torch.empty(1, dtype=torch.float64, device=DEV)
    g1 = torch.empty_like(F)
    g2 = torch.empty_like(F)
    ngv.ngv_mi_loss_fwd_bwd(F, W, l1, g1)
    ngv.ngv_mi_loss_fwd_bwd(F, W, l2, g2)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(g1, g2)
    l3 = torch.full((1,), 0.25, dtype=torch.float64, device=DEV)
    g3 = torch.full_like(F, 0.5)
    ngv.ngv_mi_loss_fwd_bwd(F, W, l3, g3, accumulate=True)
    l4 = torch.empty(1, dtype=torch.float64, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd(F, W, l4, None)  # loss only
    torch.cuda.synchronize()
    assert abs(float(l3[0]) - (float(l1[0]) + 0.25)) < 1e-12
    assert torch.allclose(g3, g1 + 0.5, atol=1e-6)
    assert torch.equal(l4, l1)


# -------------------------------------------------------------------- LNCC

LNCC_CASES = [
    (3, (13, 21, 37)),
    (5, (20, 35, 40)),
    (7, (19, 33, 70)),
    (9, (26, 40, 45)),
    (9, (20, 149, 70)),  # 10 tile rows: a full strip of 8 and a partial one of 2; 3 tile columns
    (11, (24, 30, 35)),
    # the large-window kernel: ragged 16 x 16 tiles, several z-chunks, and
    # volumes smaller than the window in one axis or all
    (13, (23, 37, 41)),
    (17, (30, 20, 50)),
    (21, (5, 9, 70)),
    (25, (20, 33, 29)),  # the largest window whose per-plane buffers all fit in LDS
    (27, (18, 22, 35)),  # the smallest with its x-boxed sums in the workspace
    (31, (40, 45, 33)),
    (31, (12, 10, 14)),
]


@pytest.mark.parametrize("case", range(len(LNCC_CASES)))
def test_lncc_parity_random(orc, ngv, case):
    win, shape = LNCC_CASES[case]
    _say("lncc random", win, shape)
    F = synth.random_volume(shape, 6, 0).numpy()
    W = (0.5 * F + 0.5 * synth.random_volume(shape, 6, 1).numpy()).astype(np.float32)
    loss = torch.empty(1, dtype=torch.float64, device=DEV)
    gW = torch.empty(shape, device=DEV)
    ngv.ngv_lncc_loss_fwd_bwd(_dev(F), _dev(W), loss, gW, win=win, weight=0.8)
    torch.cuda.synchronize()
    lo, go = orc.lncc_loss_grad(F, W.astype(np.float64), win, weight=0.8)
    P.scalar(float(loss[0]), lo, what="LNCC loss")
    P.elementwise(P.to_np(gW), go, P.RTOL_GRAD, what="LNCC gW")


@pytest.mark.parametrize("wl,shape,win", [("c1", (64, 64, 64), 5), ("c2", (40, 48, 56), 7),
                                          ("c4", (48, 56, 48), 9), ("c2", (40, 48, 56), 15)])
def test_lncc_parity_phantoms(orc, ngv, wl, shape, win):
    _say("lncc phantom", wl, shape, win)
    c = synth.make_case(wl, shape=shape)
    F, W = c.F.numpy(), c.M.numpy()
    loss = torch.empty(1, dtype=torch.float64, device=DEV)
    gW = torch.zeros(shape, device=DEV)
    ngv.ngv_lncc_loss_fwd_bwd(_dev(F), _dev(W), loss, gW, win=win)
    torch.cuda.synchronize()
    lo, go = orc.lncc_loss_grad(F, W.astype(np.float64), win)
    P.scalar(float(loss[0]), lo, what="LNCC loss")
    P.elementwise(P.to_np(gW), go, P.RTOL_GRAD, what="LNCC gW")


@pytest.mark.parametrize("win,shape", [(5, (18, 25, 40)), (9, (21, 150, 75)), (15, (19, 30, 41))])
def test_lncc_accumulate_and_determinism(ngv, win, shape):
    """accumulate adds to the loss and gW; repeated calls are bitwise equal
    (w = 9 also runs the lane-mapped stages and a full and a partial strip of
    tile rows; w = 15 the large-window kernel); a loss-only call gives the
    same loss."""
    _say("lncc accumulate", win, shape)
    F = synth.random_volume(shape, 7, 0).to(DEV)
    W = synth.random_volume(shape, 7, 1).to(DEV)
    l1 = torch.empty(1, dtype=torch.float64, device=DEV)
    g1 = torch.empty(shape, device=DEV)
    ngv.ngv_lncc_loss_fwd_bwd(F, W, l1, g1, win=win)
    l2 = torch.full((1,), 1.0, dtype=torch.float64, device=DEV)
    g2 = torch.full(shape, 2.0, device=DEV)
    ngv.ngv_lncc_loss_fwd_bwd(F, W, l2, g2, win=win, accumulate=True)
    l3 = torch.empty(1, dtype=torch.float64, device=DEV)
    g3 = torch.empty(shape, device=DEV)
    ngv.ngv_lncc_loss_fwd_bwd(F, W, l3, g3, win=win)
    l4 = torch.empty(1, dtype=torch.float64, device=DEV)
    ngv.ngv_lncc_loss_fwd_bwd(F, W, l4, None, win=win)
    torch.cuda.synchronize()
    assert torch.equal(l1, l3) and torch.equal(g1, g3) and torch.equal(l1, l4)
    assert abs(float(l2[0]) - float(l1[0]) - 1.0) < 1e-12
    assert torch.allclose(g2, g1 + 2.0, atol=1e-6)


# -------------------------------------------------------------------- Adam

@pytest.mark.parametrize("sigma,shape", [(0.0, (13, 17, 33)), (1.0, (19, 37, 45)), (0.6, (9, 20, 70))])
def test_adam_parity(orc, ngv, sigma, shape):
    _say("adam", sigma, shape)
    vol = (3,) + shape
    u = synth.random_volume(vol, 11, 0, -0.1, 0.1).numpy()
    g = synth.random_volume(vol, 11, 1, -1.0, 1.0).numpy()
    m1 = synth.random_volume(vol, 11, 2, -0.1, 0.1).numpy()
    m2 = synth.random_volume(vol, 11, 3, 0.0, 0.1).numpy()
    step, lr = 3, 0.01
    ud, m1d, m2d = _dev(u), _dev(m1), _dev(m2)
    ngv.ngv_adam_step(ud, _dev(g), m1d, m2d, step, lr, smooth_sigma=sigma)
    torch.cuda.synchronize()
    gs = g.astype(np.float64)
    if sigma > 0:
        gs = np.stack([orc.gauss_smooth(gs[k], sigma) for k in range(3)])
    ur, m1r, m2r = orc.adam(u, gs, m1, m2, step, lr)
    P.elementwise(P.to_np(m1d).ravel(), m1r, P.RTOL_GRAD, what="m1")
    P.elementwise(P.to_np(m2d).ravel(), m2r, P.RTOL_GRAD, what="m2")
    # the update itself, relative to its own size
    P.elementwise(P.to_np(ud).ravel() - u.ravel(), ur - u.ravel().astype(np.float64), P.RTOL_GRAD, what="du")


@pytest.mark.parametrize("sigma,step", [(0.0, 1), (0.0, 7), (1.0, 40)])
def test_adam_device_step_number(orc, ngv, sigma, step):
    """The step number read on the device (step_dev) gives the host step's
    update: against the oracle at that step, and against the host-step call."""
    _say("adam step_dev", sigma, step)
    shape = (11, 19, 37)
    vol = (3,) + shape
    u = synth.random_volume(vol, 12, 0, -0.1, 0.1).numpy()
    g = synth.random_volume(vol, 12, 1, -1.0, 1.0).numpy()
    m1 = synth.random_volume(vol, 12, 2, -0.1, 0.1).numpy()
    m2 = synth.random_volume(vol, 12, 3, 0.0, 0.1).numpy()
    lr = 0.01
    sd = torch.tensor([step], dtype=torch.int32, device=DEV)
    ua, m1a, m2a = _dev(u), _dev(m1), _dev(m2)
    ngv.ngv_adam_step(ua, _dev(g), m1a, m2a, 0, lr, smooth_sigma=sigma, step_dev=sd)
    ub, m1b, m2b = _dev(u), _dev(m1), _dev(m2)
    ngv.ngv_adam_step(ub, _dev(g), m1b, m2b, step, lr, smooth_sigma=sigma)
    torch.cuda.synchronize()
    # the bias corrections agree to the fp32 rounding of an fp64 value
    assert torch.allclose(ua, ub, rtol=1e-6, atol=1e-9) and torch.equal(m1a, m1b) and torch.equal(m2a, m2b)
    gs = g.astype(np.float64)
    if sigma > 0:
        gs = np.stack([orc.gauss_smooth(gs[k], sigma) for k in range(3)])
    ur, _, _ = orc.adam(u, gs, m1, m2, step, lr)
    P.elementwise(P.to_np(ua).ravel() - u.ravel(), ur - u.ravel().astype(np.float64), P.RTOL_GRAD, what="du")


@pytest.mark.parametrize("split", [None, [(0, 7), (7, 8), (8, 20), (20, 31)]])
def test_warp_bwd_adam(orc, ngv, split):
    """The fused sampler backward + Adam step (no smoothing) equals the two
    separate calls, and its update matches the oracle's Adam step on the
    oracle's gradient; with a z-split moving image the earlier slabs' partial
    gradient comes in through gu_partial."""
    _say("warp_bwd_adam", split)
    oshape, mshape = (29, 40, 66), (31, 38, 70)
    M = synth.random_volume(mshape, 12, 0).numpy()
    A, t = _rand_affine(12)
    vol = (3,) + oshape
    u = (0.05 * synth.random_field(oshape, 12, 6, 1.0)).numpy()
    gW = synth.random_volume(oshape, 12, 9, -1.0, 1.0).numpy()
    m1 = synth.random_volume(vol, 12, 2, -0.1, 0.1).numpy()
    m2 = synth.random_volume(vol, 12, 3, 0.0, 0.1).numpy()
    step, lr = 3, 0.01
    xf = ngv.make_xform(A, t)
    Md, gWd = _dev(M), _dev(gW)
    slabs = split or [(0, mshape[0])]
    views = [Md[z0:z1].contiguous() for z0, z1 in slabs]

    def state():
        return (_dev(u), _dev(m1), _dev(m2), torch.full((9,), 0.5, dtype=torch.float64, device=DEV),
                torch.full((3,), 0.5, dtype=torch.float64, device=DEV))

    # separate calls
    u1, m11, m21, gA1, gt1 = state()
    gu = torch.empty(vol, device=DEV)
    for h, (z0, z1) in enumerate(slabs):
        ngv.ngv_warp_bwd(views[h], u1, xf, gWd, gu, gA1, gt1, mdims=mshape, slab=(z0, z1 - z0),
                         accumulate=h > 0)
    ngv.ngv_adam_step(u1, gu, m11, m21, step, lr)
    # fused
    u2, m12, m22, gA2, gt2 = state()
    gp = torch.empty(vol, device=DEV)
    for h, (z0, z1) in enumerate(slabs[:-1]):
        ngv.ngv_warp_bwd(views[h], u2, xf, gWd, gp, gA2, gt2, mdims=mshape, slab=(z0, z1 - z0), accumulate=h > 0)
    z0, z1 = slabs[-1]
    ngv.ngv_warp_bwd_adam(views[-1], u2, xf, gWd, m12, m22, step, lr, gA2, gt2,
                          gu_partial=gp if len(slabs) > 1 else None, mdims=mshape, slab=(z0, z1 - z0),
                          accumulate_affine=len(slabs) > 1)
    torch.cuda.synchronize()
    # the same arithmetic on the same values in the same order
    assert torch.equal(m12, m11) and torch.equal(m22, m21) and torch.equal(u2, u1)
    assert torch.equal(gA2, gA1) and torch.equal(gt2, gt1)
    # against the oracle
    prm = orc.pack_prm(A, t)
    gu_ref, dA, dt, mag = orc.warp_bwd(M, u, prm, gW.astype(np.float64))
    _, kink = orc.warp_fwd(M, u, prm, want_kink=True)
    mask = P.off_kink(kink)
    ur, m1r, m2r = orc.adam(u, gu_ref, m1, m2, step, lr)
    mk = np.broadcast_to(mask, vol).ravel()
    P.elementwise(P.to_np(m12).ravel(), m1r, P.RTOL_GRAD, mask=mk, what="m1")
    P.elementwise(P.to_np(m22).ravel(), m2r, P.RTOL_GRAD, mask=mk, what="m2")
    P.elementwise(P.to_np(u2).ravel() - u.ravel(), ur - u.ravel().astype(np.float64), P.RTOL_GRAD, mask=mk,
                  what="du")
    P.affine_sums(P.to_np(gA2) - 0.5, dA.ravel(), mag, "dA")
    P.affine_sums(P.to_np(gt2) - 0.5, dt, mag, "dt")


def test_zblock_walk_with_a_short_last_block(orc, ngv):
    """A volume tall enough that the sampler kernels walk z-blocks of more
    than one group, with a last block shorter than the others (355 planes: 71
    groups of 5 for the forward in blocks of 2, 178 groups of 2 for the fused
    backward in blocks of 5): W and the fused backward + Adam update against
    the oracle, the update bit for bit as the separate calls, and the slab
    sequence bit for bit as zeroing and adding over four slabs."""
    oshape = mshape = (355, 20, 70)
    _say("z-block walk", oshape)
    M = synth.random_volume(mshape, 41, 0).numpy()
    A, t = _rand_affine(41, rot=0.05)
    vol = (3,) + oshape
    u = (0.05 * synth.random_field(oshape, 41, 6, 1.0)).numpy()
    gW = synth.random_volume(oshape, 41, 9, -1.0, 1.0).numpy()
    m1 = synth.random_volume(vol, 41, 2, -0.1, 0.1).numpy()
    m2 = synth.random_volume(vol, 41, 3, 0.0, 0.1).numpy()
    step, lr = 2, 0.01
    xf = ngv.make_xform(A, t)
    prm = orc.pack_prm(A, t)
    Md, ud, gWd = _dev(M), _dev(u), _dev(gW)
    W = torch.empty(oshape, device=DEV)
    ngv.ngv_warp_fwd(Md, ud, xf, W)
    torch.cuda.synchronize()
    W_ref, kink = orc.warp_fwd(M, u, prm, want_kink=True)
    P.elementwise(P.to_np(W), W_ref, P.RTOL_W, what="W")
    # the slab sequence over four slabs against zeroing and adding
    bounds = [(0, 90), (90, 180), (180, 270), (270, 355)]
    views = [Md[z0:z1].contiguous() for z0, z1 in bounds]
    zr = torch.empty(2, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_zrange(ud, xf, zr, mshape)
    sl = [(z0, z1 - z0, zr) for z0, z1 in bounds]
    W1 = torch.zeros(oshape, device=DEV)
    W2 = torch.full(oshape, 7.0, device=DEV)
    for h in range(len(bounds)):
        ngv.ngv_warp_fwd(views[h], ud, xf, W1, mdims=mshape, slab=sl[h], accumulate=True)
        ngv.ngv_warp_fwd_slab(views[h], ud, xf, W2, sl[h], mdims=mshape)
    # the fused backward + Adam against the separate calls and the oracle
    u1, m11, m21 = _dev(u), _dev(m1), _dev(m2)
    gA1 = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt1 = torch.zeros(3, dtype=torch.float64, device=DEV)
    gu = torch.empty(vol, device=DEV)
    ngv.ngv_warp_bwd(Md, u1, xf, gWd, gu, gA1, gt1)
    ngv.ngv_adam_step(u1, gu, m11, m21, step, lr)
    u2, m12, m22 = _dev(u), _dev(m1), _dev(m2)
    gA2 = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt2 = torch.zeros(3, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_bwd_adam(Md, u2, xf, gWd, m12, m22, step, lr, gA2, gt2)
    torch.cuda.synchronize()
    assert torch.equal(W1.view(torch.int32), W2.view(torch.int32))
    assert torch.allclose(W2, W, rtol=1e-6, atol=1e-7)
    assert torch.equal(m12, m11) and torch.equal(m22, m21) and torch.equal(u2, u1)
    gu_ref, dA, dt, mag = orc.warp_bwd(M, u, prm, gW.astype(np.float64))
    ur, m1r, m2r = orc.adam(u, gu_ref, m1, m2, step, lr)
    mk = np.broadcast_to(P.off_kink(kink), vol).ravel()
    P.elementwise(P.to_np(m12).ravel(), m1r, P.RTOL_GRAD, mask=mk, what="m1")
    P.elementwise(P.to_np(u2).ravel() - u.ravel(), ur - u.ravel().astype(np.float64), P.RTOL_GRAD, mask=mk,
                  what="du")
    P.affine_sums(P.to_np(gA2), dA.ravel(), mag, "dA")
    P.affine_sums(P.to_np(gt2), dt, mag, "dt")


# ---------------------------------------------------------- slab z-range

def _tilted_case(seed, oshape, mshape):
    """A strong tilt about x and y plus a displacement with a spike, so that
    slabs see ragged, plane-crossing footprints."""
    r = synth.scalars(seed, 2, 6)
    R = synth.euler_rotation(0.3 * (2 * r[0] - 1) + 0.2, 0.3 * (2 * r[1] - 1) - 0.2, 0.1)
    A = (R @ np.diag([1.05, 0.97, 1.02])).astype(np.float32)
    t = np.array([0.03, -0.05, 0.02], np.float32)
    u = (0.08 * synth.random_field(oshape, seed, 6, 1.0)).numpy()
    u[2, oshape[0] // 2, oshape[1] // 3, oshape[2] // 4] = 0.9  # one far-reaching sample
    return A, t, u


@pytest.mark.parametrize("S", [[[0.9, 0.1, 0.0], [0.0, 1.1, -0.2], [0.3, -0.1, 1.3]],
                               [[0.9, 0.1, 0.0], [0.0, 1.1, -0.2], [0.0, 0.0, 1.3]]])
@pytest.mark.parametrize("oshape", [(23, 37, 51), (23, 37, 50)])
def test_warp_zrange(ngv, S, oshape):
    """The z-range of S u in M's voxels: a general S, and one whose z row
    holds only u_z (the call then reads one field: with an even voxel count
    u_z is 16-byte aligned and read in 16-byte loads, here with a tail of 2)."""
    _say("warp_zrange", S[2], oshape)
    mshape = (29, 33, 45)
    A, t, u = _tilted_case(21, oshape, mshape)
    S = np.array(S, np.float32)
    xf = ngv.make_xform(A, t, S)
    zr = torch.empty(2, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_zrange(_dev(u), xf, zr, mshape)
    torch.cuda.synchronize()
    # the z row of S in M's voxel units, applied to every output voxel
    dz = (mshape[0] - 1) / 2.0
    sz = dz * (S[2, 0].astype(np.float64) * u[0] + S[2, 1].astype(np.float64) * u[1] +
               S[2, 2].astype(np.float64) * u[2])
    got = zr.cpu().numpy()
    assert abs(got[0] - sz.min()) <= 1e-12 * (1 + abs(sz.min())), (got, sz.min())
    assert abs(got[1] - sz.max()) <= 1e-12 * (1 + abs(sz.max())), (got, sz.max())


@pytest.mark.parametrize("bounds", [[(0, 5), (5, 6), (6, 17), (17, 29)], [(0, 10), (10, 20), (20, 29)]])
def test_warp_slabs_with_zrange_match(ngv, bounds):
    """Slab calls that skip the output voxels outside a slab's reach (given the
    z-range bound) give the same W, gu, dA, dt and Adam update as slab calls
    that visit every voxel."""
    _say("slab zrange", bounds)
    oshape, mshape = (27, 41, 70), (29, 38, 66)
    A, t, u = _tilted_case(22, oshape, mshape)
    M = synth.random_volume(mshape, 22, 0).numpy()
    gW = synth.random_volume(oshape, 22, 9, -1.0, 1.0).numpy()
    m1 = synth.random_volume((3,) + oshape, 22, 2, -0.1, 0.1).numpy()
    m2 = synth.random_volume((3,) + oshape, 22, 3, 0.0, 0.1).numpy()
    xf = ngv.make_xform(A, t)
    Md, gWd = _dev(M), _dev(gW)
    views = [Md[z0:z1].contiguous() for z0, z1 in bounds]
    zr = torch.empty(2, dtype=torch.float64, device=DEV)
    ud = _dev(u)
    ngv.ngv_warp_zrange(ud, xf, zr, mshape)
    out = {}
    for tag, use in (("all", False), ("range", True)):
        sl = [(z0, z1 - z0, zr) if use else (z0, z1 - z0) for z0, z1 in bounds]
        W = torch.full(oshape, 7.0, device=DEV)  # the first slab must overwrite everything
        for h in range(len(bounds)):
            ngv.ngv_warp_fwd(views[h], ud, xf, W, mdims=mshape, slab=sl[h], accumulate=h > 0)
        gu = torch.full((3,) + oshape, 7.0, device=DEV)
        gA = torch.zeros(9, dtype=torch.float64, device=DEV)
        gt = torch.zeros(3, dtype=torch.float64, device=DEV)
        for h in range(len(bounds)):
            ngv.ngv_warp_bwd(views[h], ud, xf, gWd, gu, gA, gt, mdims=mshape, slab=sl[h], accumulate=h > 0)
        # fused: earlier slabs accumulate gu, the last applies Adam
        u2, a1, a2 = _dev(u), _dev(m1), _dev(m2)
        gp = torch.full((3,) + oshape, 7.0, device=DEV)
        gA2 = torch.zeros(9, dtype=torch.float64, device=DEV)
        gt2 = torch.zeros(3, dtype=torch.float64, device=DEV)
        for h in range(len(bounds) - 1):
            ngv.ngv_warp_bwd(views[h], u2, xf, gWd, gp, gA2, gt2, mdims=mshape, slab=sl[h], accumulate=h > 0)
        ngv.ngv_warp_bwd_adam(views[-1], u2, xf, gWd, a1, a2, 2, 0.01, gA2, gt2, gu_partial=gp, mdims=mshape,
                              slab=sl[-1], accumulate_affine=True)
        torch.cuda.synchronize()
        out[tag] = [W, gu, gA, gt, u2, a1, a2, gA2, gt2]
    names = ["W", "gu", "dA", "dt", "u", "m1", "m2", "dA fused", "dt fused"]
    for n, a, b in zip(names, out["all"], out["range"]):
        if n.startswith("dA") or n.startswith("dt"):
            # the same per-voxel terms, summed by other blocks in another order
            assert torch.allclose(a, b, rtol=1e-12, atol=1e-12 * float(a.abs().max())), n
        else:
            assert torch.equal(a, b), n  # skipped voxels contribute exact zeros
    # and the sum over slabs is the whole sampler
    W1 = torch.empty(oshape, device=DEV)
    ngv.ngv_warp_fwd(Md, ud, xf, W1)
    torch.cuda.synchronize()
    assert torch.allclose(out["range"][0], W1, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("bounds,shift", [([(0, 5), (5, 6), (6, 17), (17, 29)], 0.0),
                                          ([(0, 10), (10, 20), (20, 29)], 0.35),
                                          ([(0, 7), (7, 29)], -0.35)])
def test_warp_fwd_slab_sequence(ngv, bounds, shift):
    """The forward slab sequence gives W bit for bit as zeroing W and adding
    every slab's part with ngv_warp_fwd, from a W that starts with garbage;
    with a z-shift part of the output samples beyond the moving grid (above
    or below), and the top slab's call writes their zeros. The sum over the
    slabs is the whole sampler."""
    _say("fwd slab sequence", bounds, shift)
    oshape, mshape = (27, 41, 70), (29, 38, 66)
    A, t, u = _tilted_case(29, oshape, mshape)
    t = (t + np.array([0.0, 0.0, shift], np.float32)).astype(np.float32)
    M = synth.random_volume(mshape, 29, 0).numpy()
    xf = ngv.make_xform(A, t)
    Md, ud = _dev(M), _dev(u)
    views = [Md[z0:z1].contiguous() for z0, z1 in bounds]
    zr = torch.empty(2, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_zrange(ud, xf, zr, mshape)
    sl = [(z0, z1 - z0, zr) for z0, z1 in bounds]
    W1 = torch.zeros(oshape, device=DEV)
    for h in range(len(bounds)):
        ngv.ngv_warp_fwd(views[h], ud, xf, W1, mdims=mshape, slab=sl[h], accumulate=True)
    W2 = torch.full(oshape, 7.0, device=DEV)
    for h in range(len(bounds)):
        ngv.ngv_warp_fwd_slab(views[h], ud, xf, W2, sl[h], mdims=mshape)
    W3 = torch.empty(oshape, device=DEV)
    ngv.ngv_warp_fwd(Md, ud, xf, W3)
    torch.cuda.synchronize()
    assert torch.equal(W1.view(torch.int32), W2.view(torch.int32))
    if shift != 0.0:
        assert int((W2 == 0).sum()) > oshape[1] * oshape[2]  # whole planes sample outside the grid
    assert torch.allclose(W2, W3, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("bounds,shift,onz", [([(0, 5), (5, 6), (6, 17), (17, 29)], 0.0, 27),
                                              ([(0, 10), (10, 20), (20, 29)], 0.35, 27),
                                              ([(0, 10), (10, 20), (20, 29)], 0.2, 28),
                                              ([(0, 5), (5, 6), (6, 17), (17, 29)], -0.3, 29)])
def test_warp_bwd_adam_slab_sequence(ngv, bounds, shift, onz):
    """The slab sequence of the fused backward steps every voxel once, bit for
    bit as ngv_warp_bwd on every earlier slab followed by ngv_warp_bwd_adam on
    the last. With a z-shift part of the output samples beyond the moving
    grid; the top slab's call steps those voxels with a zero gradient. The
    scratch gu starts with garbage (it needs no initialisation). The affine
    sums are fp32 within a work item and fp64 across items; the sequence's
    items hold three planes and the banded calls' two, so the two round
    differently: they agree to fp32 partial-sum rounding, 1e-5 of the
    largest component (a missing or repeated item would be far beyond it)."""
    _say("bwd adam slab sequence", bounds, shift, onz)
    # output planes 27, 28, 29: the sequence's three-plane work items end
    # whole, with one plane, with two
    oshape, mshape = (onz, 41, 70), (29, 38, 66)
    A, t, u = _tilted_case(23, oshape, mshape)
    t = (t + np.array([0.0, 0.0, shift], np.float32)).astype(np.float32)
    M = synth.random_volume(mshape, 23, 0).numpy()
    gW = synth.random_volume(oshape, 23, 9, -1.0, 1.0).numpy()
    m1 = synth.random_volume((3,) + oshape, 23, 2, -0.1, 0.1).numpy()
    m2 = synth.random_volume((3,) + oshape, 23, 3, 0.0, 0.1).numpy()
    xf = ngv.make_xform(A, t)
    Md, gWd = _dev(M), _dev(gW)
    views = [Md[z0:z1].contiguous() for z0, z1 in bounds]
    zr = torch.empty(2, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_zrange(_dev(u), xf, zr, mshape)
    sl = [(z0, z1 - z0, zr) for z0, z1 in bounds]
    # reference: partial gradients in gu, the last slab fused with the update
    u1, a1, b1 = _dev(u), _dev(m1), _dev(m2)
    gp = torch.full((3,) + oshape, 7.0, device=DEV)
    gA1 = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt1 = torch.zeros(3, dtype=torch.float64, device=DEV)
    for h in range(len(bounds) - 1):
        ngv.ngv_warp_bwd(views[h], u1, xf, gWd, gp, gA1, gt1, mdims=mshape, slab=sl[h], accumulate=h > 0)
    ngv.ngv_warp_bwd_adam(views[-1], u1, xf, gWd, a1, b1, 3, 0.01, gA1, gt1, gu_partial=gp, mdims=mshape,
                          slab=sl[-1], accumulate_affine=True)
    # the sequence
    u2, a2, b2 = _dev(u), _dev(m1), _dev(m2)
    scratch = torch.full((3,) + oshape, 7.0, device=DEV)
    gA2 = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt2 = torch.zeros(3, dtype=torch.float64, device=DEV)
    for h in range(len(bounds)):
        ngv.ngv_warp_bwd_adam_slab(views[h], u2, xf, gWd, scratch, a2, b2, 3, 0.01, gA2, gt2, sl[h], mdims=mshape,
                                   accumulate_affine=h > 0)
    torch.cuda.synchronize()
    assert torch.equal(u1, u2) and torch.equal(a1, a2) and torch.equal(b1, b2)
    assert not torch.equal(u1, _dev(u))  # the step moved u
    for a, b, n in ((gA1, gA2, "dA"), (gt1, gt2, "dt")):
        assert torch.allclose(a, b, rtol=0.0, atol=1e-5 * float(a.abs().max())), n


# ---------------------------------------------- sampler sweep with MI forward

@pytest.mark.parametrize("split", [None, [(0, 9), (9, 20), (20, 29)]])
def test_warp_fwd_mi(orc, ngv, split):
    """The sampler sweep that also builds the MI histogram (ngv_warp_fwd_mi,
    then ngv_mi_grad from the table it leaves) gives the same W as
    ngv_warp_fwd, and the MI loss and gradient of the oracle on that W; with
    z-slabs and a z-range bound the last slab's call does the MI forward."""
    _say("warp_fwd_mi", split)
    oshape, mshape = (27, 41, 70), (29, 38, 66)
    A, t, u = _tilted_case(23, oshape, mshape)
    M = synth.random_volume(mshape, 23, 0).numpy()
    F = synth.random_volume(oshape, 23, 1, -0.05, 1.05).numpy()
    xf = ngv.make_xform(A, t)
    Md, ud, Fd = _dev(M), _dev(u), _dev(F)
    slabs = split or [(0, mshape[0])]
    views = [Md[z0:z1].contiguous() for z0, z1 in slabs]
    zr = torch.empty(2, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_zrange(ud, xf, zr, mshape)
    sl = [(z0, z1 - z0, zr) if split else (z0, z1 - z0) for z0, z1 in slabs]
    W1 = torch.full(oshape, 7.0, device=DEV)
    for h in range(len(slabs)):
        ngv.ngv_warp_fwd(views[h], ud, xf, W1, mdims=mshape, slab=sl[h], accumulate=h > 0)
    W2 = torch.full(oshape, 7.0, device=DEV)
    loss = torch.zeros(1, dtype=torch.float64, device=DEV)
    for h in range(len(slabs) - 1):
        ngv.ngv_warp_fwd(views[h], ud, xf, W2, mdims=mshape, slab=sl[h], accumulate=h > 0)
    ngv.ngv_warp_fwd_mi(views[-1], ud, xf, W2, Fd, loss, bins=32, mdims=mshape, slab=sl[-1],
                        accumulate=len(slabs) > 1)
    gW = torch.empty(oshape, device=DEV)
    ngv.ngv_mi_grad(Fd, W2, gW, bins=32)
    torch.cuda.synchronize()
    assert torch.equal(W1, W2)
    Wn = P.to_np(W2).astype(np.float32)
    l_ref, g_ref, _ = orc.mi_loss_grad(F, Wn, bins=32)
    P.scalar(float(loss[0]), l_ref, what="MI loss (sweep)")
    P.elementwise(P.to_np(gW), g_ref, P.RTOL_GRAD, what="MI gW (sweep)")
    # the separate call on the same W agrees to the grouping of fp32 window sums
    loss2 = torch.zeros(1, dtype=torch.float64, device=DEV)
    gW2 = torch.empty(oshape, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd(Fd, W2, loss2, gW2, bins=32)
    torch.cuda.synchronize()
    assert abs(float(loss[0]) - float(loss2[0])) <= 1e-6 * abs(float(loss2[0]))
