"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (one RegistrationStep: warp, MI, LNCC, then the sampler backward fused with
Adam when there is no smoothing, forming the MI gradient itself when the
moving image is in one piece; the step's whole gW is then completed by the MI
gradient sweep for the comparison).

C2 and C3 are compared element by element with the oracle's whole step. C4
(315 M voxels) is compared element by element for W and gW, exactly for the
losses and the affine gradient sums, and at sampled voxels for gu and the
update. C5 (2.5 G voxels, moving image in 8 z-slabs) is compared for the
losses (oracle over z-chunks), at sampled voxels for W, gW and gu (the
oracle's LNCC gradient at a voxel by direct sums over a local neighbourhood
of its own warped image), and by the slab-sum property against the unsplit
sampler over every voxel. Every expected value comes from the oracle.
"""
import gc
import time

import numpy as np
import pytest
import torch

from non_gemm_voxel_amd import synth
from tests import parity as P
from tests.test_gpu_step import oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(*a):
    print("[fullsize]", *a, flush=True)


def _run_step(wl, device=DEV):
    from non_gemm_voxel_amd.step import RegistrationStep
    t0 = time.time()
    c = synth.make_case(wl, device=device)
    st = RegistrationStep(c.F, c.M, c.A, c.t, bins=wl.bins, win=wl.win, smooth_sigma=wl.smooth_sigma, lr=c.lr,
                          slabs=wl.slabs)
    st.step()
    torch.cuda.synchronize()
    _log(wl.name, f"generated and stepped in {time.time() - t0:.1f} s (fused backward+update: {st.fused})")
    return c, st


def _gu_at_start(st, gW):
    """gu at the step's starting field u = 0 for the step's whole gradient gW.
    The fused backward feeds it straight into the update, so it is recomputed
    by the sampler backward."""
    if not st.fused:
        return st.gu
    from non_gemm_voxel_amd import ngv
    u0 = torch.zeros_like(st.u)
    gA = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt = torch.zeros(3, dtype=torch.float64, device=DEV)
    for h, (z0, n) in enumerate(st.slabs):
        ngv.ngv_warp_bwd(st.M_views[h], u0, st.xf, gW, st.gu, gA, gt, mdims=st.shape, slab=(z0, n),
                         accumulate=h > 0)
    torch.cuda.synchronize()
    del u0
    return st.gu


def _check_update(orc, u, m1, m2, g_ref, lr, mask, what):
    """The first Adam step from u = m1 = m2 = 0 (u, m1, m2 after it, (3, ...))
    against the oracle's from the same state, off the sampler's kinks, within
    the bars carried from the gradient bar: m1 = (1 - b1) g pins the gradient
    that the fused backward formed without storing it."""
    z = np.zeros(np.shape(g_ref))
    P.check_adam_step(orc, u, m1, m2, z.astype(np.float32), z, z, g_ref, 1, P.f32(lr), mask=mask, what=what)


def _sampled(t, ii):
    """Entries ii of each component of a (3, ...) device field, as (3, n)."""
    return torch.stack([t[k].reshape(-1)[ii] for k in range(3)], 0).cpu().numpy()


def _release():
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c2", "c3"])
def test_full_size_step_elementwise(orc, name):
    wl = synth.WORKLOADS[name]
    _log("case", name, wl.shape)
    c, st = _run_step(wl)
    host = synth.Case(wl, c.shape, c.F.cpu(), c.M.cpu(), c.A, c.t, lr=c.lr)
    u0 = np.zeros((3,) + c.shape, np.float32)
    ref = oracle_step(orc, host, wl, u0, c.lr)
    _log(name, "oracle done")
    P.elementwise(P.to_np(st.W), ref["W"], P.RTOL_W, what="W")
    if wl.bins:
        P.scalar(float(st.loss[0]), ref["loss_mi"], what="MI loss")
    if wl.win:
        P.scalar(float(st.loss[1]), ref["loss_lncc"], what="LNCC loss")
    gW_step = P.step_gW(st)
    P.elementwise(P.to_np(gW_step), ref["gW"], P.RTOL_GRAD, what="gW")
    P.affine_sums(P.to_np(st.gA), ref["dA"].ravel(), ref["mag"], "dA")
    P.affine_sums(P.to_np(st.gt), ref["dt"], ref["mag"], "dt")
    # near a cell face either one-sided derivative is valid: their spread is
    # allowed on gu, and carried through the smoothing to the update
    kink = P.kink_allowance(orc, host.M.numpy(), u0, orc.pack_prm(c.A, c.t), ref["gW"], ref["kink"],
                            exact_lattice_ok=not wl.affine_start)
    _log(name, f"voxels with a kink allowance {np.mean(kink.max(axis=0) > 0):.2e}")
    g_extra = kink
    if wl.smooth_sigma > 0:
        g_extra = np.stack([orc.gauss_smooth(kink[k], wl.smooth_sigma) for k in range(3)])
    z = np.zeros_like(ref["g"])
    P.check_adam_step(orc, P.to_np(st.u), P.to_np(st.m1), P.to_np(st.m2), u0, z, z, ref["g"], 1, P.f32(c.lr),
                      what="Adam step", g_extra=g_extra)
    gu = P.to_np(_gu_at_start(st, gW_step))
    P.within(gu, ref["gu"], P.grad_bar(ref["gu"]) + kink, what="gu")
    del c, st, gW_step
    _release()


def _samples(shape, n, seed):
    rng = np.random.default_rng(seed)
    N = int(np.prod(shape))
    return np.unique(rng.integers(0, N, n)).astype(np.int64)


@pytest.mark.timeout(900)
def test_c4_full_size(orc):
    wl = synth.WORKLOADS["c4"]
    _log("case c4", wl.shape)
    c, st = _run_step(wl)
    shape = c.shape
    nz = shape[0]
    F = c.F.cpu().numpy()
    M = c.M.cpu().numpy()
    u0 = np.zeros((3,) + shape, np.float32)
    prm = orc.pack_prm(c.A, c.t)
    W = orc.warp_fwd(M, u0, prm)
    _log("oracle W")
    P.elementwise(P.to_np(st.W), W, P.RTOL_W, what="W")
    N = F.size
    H = orc.mi_hist(F, W, bins=wl.bins)
    mi, L = orc.mi_finalize(H, N)
    P.scalar(float(st.loss[0]), -mi, what="MI loss")
    cc_sum = sum(orc.lncc_sum(F, W, wl.win, z_range=(z, min(nz, z + 64))) for z in range(0, nz, 64))
    P.scalar(float(st.loss[1]), -cc_sum / N, what="LNCC loss")
    _log("oracle losses")
    gW = orc.mi_grad_values(F, W, L, bins=wl.bins, N=N).reshape(shape)
    g_l = np.zeros(shape, np.float64)
    for z in range(0, nz, 32):
        orc.lncc_grad_range(F, W, wl.win, 1e-5, 1.0, N, (z, min(nz, z + 32)), g_l)
    gW += g_l
    del g_l
    _log("oracle gW")
    gW_step = P.step_gW(st)
    P.elementwise(P.to_np(gW_step), gW, P.RTOL_GRAD, what="gW")
    _, dA, dt, mag = orc.warp_bwd(M, u0, prm, gW, want_gu=False)
    P.affine_sums(P.to_np(st.gA), dA.ravel(), mag, "dA")
    P.affine_sums(P.to_np(st.gt), dt, mag, "dt")
    _log("oracle dA dt")
    idx = _samples(shape, 200000, 4)
    _, _, kink = orc.warp_points(M, u0, prm, idx)
    gu_ref = orc.warp_bwd_points(M, u0, prm, idx, gW.reshape(-1)[idx])
    ii = torch.as_tensor(idx, device=DEV)
    ok = kink >= P.KINK_BAND
    _check_update(orc, _sampled(st.u, ii), _sampled(st.m1, ii), _sampled(st.m2, ii), gu_ref.T, c.lr, ok,
                  "Adam step sampled")
    gu_all = _gu_at_start(st, gW_step)
    gu = torch.stack([gu_all[k].reshape(-1)[ii] for k in range(3)], 1).cpu().numpy()
    for k in range(3):
        P.elementwise(gu[:, k], gu_ref[:, k], P.RTOL_GRAD, mask=ok, what=f"gu[{k}] sampled")
    del c, st, gW_step
    _release()


def _lncc_grad_points_c5(orc, F_dev, M, u0_zero, prm, shape, win, pts):
    """Oracle LNCC gradient at points from local neighbourhoods: the oracle
    warps each 2r-neighbourhood itself (points function) and sums directly."""
    r = win // 2
    out = np.zeros(len(pts))
    nz, ny, nx = shape
    for i, (z, y, x) in enumerate(pts):
        lo = [max(0, z - 2 * r), max(0, y - 2 * r), max(0, x - 2 * r)]
        hi = [min(nz, z + 2 * r + 1), min(ny, y + 2 * r + 1), min(nx, x + 2 * r + 1)]
        zz, yy, xx = np.meshgrid(np.arange(lo[0], hi[0]), np.arange(lo[1], hi[1]), np.arange(lo[2], hi[2]),
                                 indexing="ij")
        lin = ((zz * ny + yy) * nx + xx).reshape(-1).astype(np.int64)
        Wl, _, _ = orc.warp_points(M, u0_zero, prm, lin)
        Fl = F_dev.reshape(-1)[torch.as_tensor(lin, device=F_dev.device)].cpu().numpy()
        sub = tuple(h - l for h, l in zip(hi, lo))
        out[i] = orc.lncc_grad_at(Fl.reshape(sub), Wl.reshape(sub), lo, shape, np.array([[z, y, x]]), win)[0]
    return out


@pytest.mark.timeout(1200)
def test_c5_gigavoxel_sampled(orc):
    wl = synth.WORKLOADS["c5"]
    _log("case c5", wl.shape)
    c, st = _run_step(wl)
    shape = c.shape
    nz, ny, nx = shape
    N = int(np.prod(shape))
    # property at every voxel: the 8-slab sampler equals the unsplit sampler
    from non_gemm_voxel_amd import ngv
    W1 = torch.empty_like(st.W)
    ngv.ngv_warp_fwd(c.M, st.u, st.xf, W1)
    # st.u has been updated by Adam: recompute the slab sum at the same u
    W8 = torch.empty_like(st.W)
    for h, (z0, n) in enumerate(st.slabs):
        ngv.ngv_warp_fwd(st.M_views[h], st.u, st.xf, W8, mdims=shape, slab=(z0, n), accumulate=h > 0)
    torch.cuda.synchronize()
    diff = float((W8 - W1).abs().max())
    _log("slab vs unsplit max diff", diff)
    assert diff <= 1e-6
    # the step's own banded path at this nonzero displacement: the z-range
    # bound of the updated u, the forward slab sequence into a W that starts
    # with garbage, against a zero-filled W and accumulating banded calls
    # (bit for bit) and against the unsplit sampler (every voxel)
    ngv.ngv_warp_zrange(st.u, st.xf, st.zrange, shape, ws=st.ws)
    zr = st.zrange.cpu().tolist()
    _log("z-range of the updated u", zr)
    assert zr[1] > zr[0]
    Wseq = W8
    Wseq.fill_(float("nan"))
    for h, sl in enumerate(st.slab_args):
        ngv.ngv_warp_fwd_slab(st.M_views[h], st.u, st.xf, Wseq, sl, mdims=shape)
    Wacc = torch.zeros_like(st.W)
    for h, sl in enumerate(st.slab_args):
        ngv.ngv_warp_fwd(st.M_views[h], st.u, st.xf, Wacc, mdims=shape, slab=sl, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(Wseq, Wacc), "slab sequence differs from zero-fill + banded accumulation"
    diff = float((Wseq - W1).abs().max())
    _log("banded slab sequence vs unsplit max diff", diff)
    assert diff <= 1e-6
    del W1, W8, Wseq, Wacc
    # oracle at u = 0 (the state the step started from)
    M = c.M.cpu().numpy()
    F_dev = c.F
    u0 = np.zeros((3,) + shape, np.float32)  # zero pages: not touched by the oracle's reads of 0.0
    prm = orc.pack_prm(c.A, c.t)
    idx = _samples(shape, 50000, 5)
    Wp, _, kink = orc.warp_points(M, u0, prm, idx)
    ii = torch.as_tensor(idx, device=DEV)
    P.elementwise(st.W.reshape(-1)[ii].cpu().numpy(), Wp, P.RTOL_W, what="W sampled")
    _log("W sampled ok")
    # losses over z-chunks of the oracle's own warped image
    F = c.F.cpu().numpy()
    H = np.zeros((wl.bins, wl.bins))
    r = wl.win // 2
    cc_sum = 0.0
    step = 64
    for z0 in range(0, nz, step):
        z1 = min(nz, z0 + step)
        a, b = max(0, z0 - r), min(nz, z1 + r)
        Wc = orc.warp_fwd_chunk(M, u0, prm, (a, b))
        Fc = np.ascontiguousarray(F[a:b])
        Hc = orc.mi_hist(np.ascontiguousarray(F[z0:z1]), Wc[z0 - a:z1 - a], bins=wl.bins)
        H += Hc
        # cc for centre planes z0..z1 of the sub-stack a..b: zero padding at
        # the sub-stack faces is wrong only within r planes of them, which are
        # exactly the planes outside [z0, z1) unless at the true volume faces
        cc_sum += orc.lncc_sum(Fc, Wc, wl.win, z_range=(z0 - a, z1 - a))
        if z0 % 256 == 0:
            _log("chunk", z0)
    mi, L = orc.mi_finalize(H, N)
    P.scalar(float(st.loss[0]), -mi, what="MI loss")
    P.scalar(float(st.loss[1]), -cc_sum / N, what="LNCC loss")
    _log("losses ok")
    # gradients at sampled voxels
    sel = idx[np.random.default_rng(6).choice(idx.size, 300, replace=False)]
    sel.sort()
    pts = np.stack(np.unravel_index(sel, shape), 1)
    Ws, _, ks = orc.warp_points(M, u0, prm, sel)
    g_mi = orc.mi_grad_values(F.reshape(-1)[sel], Ws, L, bins=wl.bins, N=N)
    g_cc = _lncc_grad_points_c5(orc, F_dev, M, u0, prm, shape, wl.win, pts)
    g_ref = g_mi + g_cc
    si = torch.as_tensor(sel, device=DEV)
    # the slab calls of the backward form the MI gradient from the stored W:
    # gW holds the LNCC part, and the MI gradient sweep completes it here
    assert st.mi_bwd
    gW_step = P.step_gW(st)
    g_gpu = gW_step.reshape(-1)[si].cpu().numpy()
    # sampled: the floor term uses the sample's own scale
    P.elementwise(g_gpu, g_ref, P.RTOL_GRAD, what="gW sampled")
    gu_ref = orc.warp_bwd_points(M, u0, prm, sel, g_ref)
    ok = ks >= P.KINK_BAND
    _check_update(orc, _sampled(st.u, si), _sampled(st.m1, si), _sampled(st.m2, si), gu_ref.T, c.lr, ok,
                  "Adam step sampled")
    gu_all = _gu_at_start(st, gW_step)
    del gW_step
    gu = torch.stack([gu_all[k].reshape(-1)[si] for k in range(3)], 1).cpu().numpy()
    for k in range(3):
        P.elementwise(gu[:, k], gu_ref[:, k], P.RTOL_GRAD, mask=ok, what=f"gu[{k}] sampled")
    del c, st
    _release()
