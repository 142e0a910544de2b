"""One whole registration step through the C ABI against the same step in the
oracle, on every workload's recipe at a size the oracle finishes in seconds
(C1 at its own size). Each stage is compared with the oracle's own previous
stage as input, never with a GPU result.
"""
import numpy as np
import pytest
import torch

from non_gemm_voxel_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

STEP_CASES = [
    ("c1", None),
    ("c2", (40, 48, 56)),
    ("c3", (48, 48, 48)),
    ("c4", (48, 56, 48)),
    ("c5", (64, 77, 64)),
]


def oracle_step(orc, c, wl, u0, lr):
    F, M = c.F.numpy(), c.M.numpy()
    prm = orc.pack_prm(c.A, c.t)
    W, kink = orc.warp_fwd(M, u0, prm, want_kink=True)
    gW = np.zeros_like(W)
    out = {"W": W, "kink": kink}
    if wl.bins:
        l, g, _ = orc.mi_loss_grad(F, W, bins=wl.bins)
        out["loss_mi"] = l
        gW += g
    if wl.win:
        l, g = orc.lncc_loss_grad(F, W, wl.win)
        out["loss_lncc"] = l
        gW += g
    gu, dA, dt, mag = orc.warp_bwd(M, u0, prm, gW)
    g = gu
    if wl.smooth_sigma > 0:
        g = np.stack([orc.gauss_smooth(gu[k], wl.smooth_sigma) for k in range(3)])
    z = np.zeros(u0.size)
    u1, _, _ = orc.adam(u0, g, z, z, 1, lr)
    out.update(gW=gW, gu=gu, dA=dA, dt=dt, mag=mag, g=g, u1=u1.reshape(u0.shape))
    return out


def _gu_at(st, gW):
    """gu of the sampler backward at u = 0 (the step's start) for gW: the fused
    backward feeds it straight into the update without storing it."""
    from non_gemm_voxel_amd import ngv
    if not st.fused:
        return st.gu
    u0 = torch.zeros_like(st.u)
    gA = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt = torch.zeros(3, dtype=torch.float64, device=DEV)
    for h, (z0, n) in enumerate(st.slabs):
        ngv.ngv_warp_bwd(st.M_views[h], u0, st.xf, gW, st.gu, gA, gt, mdims=st.shape, slab=(z0, n),
                         accumulate=h > 0)
    return st.gu


@pytest.mark.parametrize("mode", ["separate", "fused", "fused_mi", "fused_step"])
@pytest.mark.parametrize("wl_name,shape", STEP_CASES)
def test_step_parity(orc, wl_name, shape, mode):
    """separate: every stage stored; fused: the calls the step makes by default
    (the backward fused with the update and, with MI and one slab, forming the
    MI gradient itself); fused_mi: as fused, with the sampler sweep building
    the MI histogram too (both sweeps of the fused step for MI); fused_step:
    the two-sweep step (the MI forward on samples that are not stored, then
    LNCC and MI gradients into the sampler backward on samples taken again;
    neither W nor gW is stored, so gu and the update carry the check)."""
    from non_gemm_voxel_amd.step import RegistrationStep
    wl = synth.WORKLOADS[wl_name]
    if mode == "fused_mi" and not wl.bins:
        pytest.skip("no MI term")
    if mode == "fused_step" and (not wl.win or wl.slabs > 1):
        pytest.skip("the two-sweep step takes an LNCC term and the moving image in one piece")
    print("[case] step", wl_name, shape, mode, flush=True)
    c = synth.make_case(wl, shape=shape)
    slabs = wl.slabs
    st = RegistrationStep(c.F.to(DEV), c.M.to(DEV), c.A, c.t, bins=wl.bins, win=wl.win,
                          smooth_sigma=wl.smooth_sigma, lr=c.lr, slabs=slabs, fused=mode != "separate",
                          fused_mi=mode == "fused_mi", fused_step=mode == "fused_step")
    assert st.fused_step == (mode == "fused_step")
    st.step()
    torch.cuda.synchronize()
    u0 = np.zeros((3,) + c.shape, np.float32)
    ref = oracle_step(orc, c, wl, u0, c.lr)
    identity = not wl.affine_start
    if not st.fused_step:
        gW_step = P.step_gW(st)
        P.elementwise(P.to_np(st.W), ref["W"], P.RTOL_W, what="W")
    if wl.bins:
        P.scalar(float(st.loss[0]), ref["loss_mi"], what="MI loss")
    if wl.win:
        P.scalar(float(st.loss[1]), ref["loss_lncc"], what="LNCC loss")
    if not st.fused_step:
        P.elementwise(P.to_np(gW_step), ref["gW"], P.RTOL_GRAD, what="gW")
    # near a cell face either one-sided derivative is valid: their spread is
    # allowed on gu, and carried through the smoothing to the update
    kink = P.kink_allowance(orc, c.M.numpy(), u0, orc.pack_prm(c.A, c.t), ref["gW"], ref["kink"],
                            exact_lattice_ok=identity)
    print(f"[info] voxels with a kink allowance {np.mean(kink.max(axis=0) > 0):.2e}", flush=True)
    gu = P.to_np(st.gu if st.fused_step else _gu_at(st, gW_step))
    P.within(gu, ref["gu"], P.grad_bar(ref["gu"]) + kink, what="gu")
    P.affine_sums(P.to_np(st.gA), ref["dA"].ravel(), ref["mag"], "dA")
    P.affine_sums(P.to_np(st.gt), ref["dt"], ref["mag"], "dt")
    # the update: m1, m2 and u after Adam's first step against the oracle's
    # step from the same zero state, within the bars carried from the
    # gradient bar (so m1 = (1 - b1) g pins the gradient the fused backward
    # formed without storing it)
    g_extra = kink
    if wl.smooth_sigma > 0:
        g_extra = np.stack([orc.gauss_smooth(kink[k], wl.smooth_sigma) for k in range(3)])
    z = np.zeros_like(ref["g"])
    P.check_adam_step(orc, P.to_np(st.u), P.to_np(st.m1), P.to_np(st.m2), u0, z, z, ref["g"], 1, P.f32(c.lr),
                      what="Adam step", g_extra=g_extra)


@pytest.mark.parametrize("fused", [False, True])
def test_losses_are_per_step(fused):
    """After several steps each loss slot holds the loss of the last step's W
    alone (the LNCC call accumulates its gradient onto MI's, and must not
    carry its loss over from earlier steps): standalone calls on that W give
    the same values."""
    from non_gemm_voxel_amd import ngv
    from non_gemm_voxel_amd.step import RegistrationStep
    wl = synth.WORKLOADS["c4"]
    print("[case] losses per step", fused, flush=True)
    c = synth.make_case(wl, shape=(40, 48, 56))
    st = RegistrationStep(c.F.to(DEV), c.M.to(DEV), c.A, c.t, bins=wl.bins, win=wl.win, lr=c.lr, fused=fused)
    for _ in range(3):
        st.step()
    mi = torch.zeros(1, dtype=torch.float64, device=DEV)
    lc = torch.zeros(1, dtype=torch.float64, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd(st.F, st.W, mi, None, bins=wl.bins)
    ngv.ngv_lncc_loss_fwd_bwd(st.F, st.W, lc, None, win=wl.win)
    torch.cuda.synchronize()
    P.scalar(float(st.loss[0]), float(mi[0]), rtol=1e-12, what="MI loss of the last step")
    P.scalar(float(st.loss[1]), float(lc[0]), rtol=1e-12, what="LNCC loss of the last step")
