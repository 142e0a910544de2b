"""Parity of the MI with a choice of the fixed image's Parzen kernel
(ngv_mi_loss_fwd_bwd_order) against the oracle: the box kernel on F with the
cubic B-spline on W (Mattes et al.'s original pair), on ragged sizes, several
bin counts, clamp edges, exact bin edges, and at the full 640 x 768 x 640
workload; the cubic choice against ngv_mi_loss_fwd_bwd, bit for bit.

The oracle puts a fixed sample in bin floor(c + 1/2) of its fp64 bin
coordinate c; the kernel takes the same floor of an fp32 coordinate, which
is within about 5e-6 bin of c. A sample whose c lies within EDGE_BAND of a
half-integer may therefore fall in the neighbouring bin on the GPU: its
gradient uses another row of the log-ratio table, so such voxels are left out
of the elementwise gradient comparison (their count is printed). Each such
sample moves 1/N of the histogram's mass by one bin, which changes the loss by
O(1/N) relative, far below the loss bar at these sizes.
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


EDGE_BAND = 2e-5  # bins


def near_box_edge(F, bins, lo=0.0, hi=1.0):
    """Fixed samples whose fp64 bin coordinate lies within EDGE_BAND of a
    half-integer (a box edge)."""
    c = 2.0 + (np.clip(np.asarray(F, np.float64), lo, hi) - lo) * (bins - 5) / (hi - lo)
    e = (c + 0.5) - np.floor(c + 0.5)
    return (e < EDGE_BAND) | (e > 1.0 - EDGE_BAND)


def _say(*a):
    print("[case]", *a, flush=True)


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x)).to(DEV)


CASES = [
    ("random", (23, 41, 67), 16),
    ("random", (17, 33, 129), 32),
    ("random", (9, 64, 64), 64),
    ("brain", (40, 48, 56), 32),
    ("random", (1, 1, 7), 8),
    ("random", (20, 30, 70), 200),
]


def _inputs(kind, shape, seed=7):
    if kind == "random":
        F = synth.random_volume(shape, seed, 0, -0.05, 1.05).numpy()
        W = (0.6 * F + 0.4 * synth.random_volume(shape, seed, 1).numpy()).astype(np.float32)
        W.reshape(-1)[:4] = [0.0, 1.0, -0.2, 1.3][:W.size]  # clamp edges and beyond
    else:
        c = synth.make_case("c3", shape=shape)
        F, W = c.F.numpy(), c.M.numpy()
    return F, W


@pytest.mark.parametrize("case", range(len(CASES)))
def test_box_fixed_kernel_parity(orc, ngv, case):
    kind, shape, bins = CASES[case]
    _say("mi box/cubic", kind, shape, bins)
    F, W = _inputs(kind, shape)
    loss = torch.empty(1, dtype=torch.float64, device=DEV)
    gW = torch.empty(shape, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd_order(_dev(F), _dev(W), loss, gW, bins=bins, fixed_order=0, weight=1.25)
    torch.cuda.synchronize()
    lo, go, H = orc.mi_loss_grad(F, W.astype(np.float64), bins=bins, weight=1.25, order=3, forder=0)
    P.scalar(float(loss[0]), lo, what="MI loss (box fixed kernel)")
    edge = near_box_edge(F, bins)
    print(f"[info] fixed samples near a box edge: {int(edge.sum())} of {edge.size}", flush=True)
    _, L = orc.mi_finalize(H, F.size)
    mags = [orc.mi_grad_values(F, W.astype(np.float64), L, bins=bins, weight=1.25, N=F.size, order=3, forder=0,
                               mode=m).reshape(F.shape) for m in (1, 2)]
    P.within(P.to_np(gW), go, P.mi_grad_bar(go, *mags, bins), mask=~edge, what="MI gW (box fixed kernel)")


def test_box_fixed_kernel_exact_edges(orc, ngv):
    """37 bins on [0, 1] (bin scale 32): fixed samples exactly half way between
    two bin centres, where the oracle's reading sends them to the upper bin.
    Every step of the kernel's fp32 coordinate is exact for these values, so
    the kernel decides the same and nothing is masked."""
    bins = 37
    shape = (5, 13, 31)
    n = int(np.prod(shape))
    k = 2 + (synth.scalars(21, 0, n) * 32).astype(np.int64)  # 2 .. 33
    on_edge = synth.scalars(21, 1, n) < 0.5
    F = np.where(on_edge, (k - 1.5) / 32.0, (k - 2.0) / 32.0).astype(np.float32).reshape(shape)
    assert np.all(near_box_edge(F, bins).reshape(-1) == on_edge)
    W = synth.random_volume(shape, 21, 2, -0.05, 1.05).numpy()
    _say("mi box/cubic exact edges", shape, bins, int(on_edge.sum()))
    loss = torch.empty(1, dtype=torch.float64, device=DEV)
    gW = torch.empty(shape, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd_order(_dev(F), _dev(W), loss, gW, bins=bins, fixed_order=0)
    torch.cuda.synchronize()
    lo, go, _ = orc.mi_loss_grad(F, W.astype(np.float64), bins=bins, order=3, forder=0)
    P.scalar(float(loss[0]), lo, what="MI loss (box fixed kernel, exact edges)")
    P.elementwise(P.to_np(gW), go, P.RTOL_GRAD, what="MI gW (box fixed kernel, exact edges)")


def test_cubic_choice_is_the_default_call(ngv):
    _say("mi order 3 vs default")
    F, W = _inputs("brain", (33, 40, 50))
    F, W = _dev(F), _dev(W)
    l1 = torch.empty(1, dtype=torch.float64, device=DEV)
    l2 = torch.empty(1, dtype=torch.float64, device=DEV)
    g1 = torch.empty_like(F)
    g2 = torch.empty_like(F)
    ngv.ngv_mi_loss_fwd_bwd(F, W, l1, g1)
    ngv.ngv_mi_loss_fwd_bwd_order(F, W, l2, g2, fixed_order=3)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(g1, g2)


def test_box_fixed_kernel_accumulate_and_determinism(ngv):
    _say("mi box/cubic accumulate")
    F, W = _inputs("brain", (33, 40, 50))
    F, W = _dev(F), _dev(W)
    l1 = torch.empty(1, dtype=torch.float64, device=DEV)
    g1 = torch.empty_like(F)
    ngv.ngv_mi_loss_fwd_bwd_order(F, W, l1, g1, fixed_order=0)
    l2 = torch.empty(1, dtype=torch.float64, device=DEV)
    g2 = torch.empty_like(F)
    ngv.ngv_mi_loss_fwd_bwd_order(F, W, l2, g2, fixed_order=0)
    l3 = torch.full((1,), 0.25, dtype=torch.float64, device=DEV)
    g3 = torch.full_like(F, 0.5)
    ngv.ngv_mi_loss_fwd_bwd_order(F, W, l3, g3, fixed_order=0, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(g1, g2)
    assert abs(float(l3[0]) - (float(l1[0]) + 0.25)) < 1e-12
    assert torch.allclose(g3, g1 + 0.5, atol=1e-6)


@pytest.mark.timeout(900)
def test_box_fixed_kernel_full_size(orc, ngv):
    """The 640 x 768 x 640 layered-cortex workload: F against the affinely
    warped M. The loss against the oracle's histogram of the whole volume
    (accumulated over z-chunks), gW at sampled voxels from the oracle's
    log-ratio table."""
    wl = synth.WORKLOADS["c4"]
    shape = wl.shape
    _say("mi box/cubic full size", shape)
    c = synth.make_case(wl, device=DEV)
    u0 = torch.zeros((3,) + shape, device=DEV)
    W = torch.empty(shape, device=DEV)
    ngv.ngv_warp_fwd(c.M, u0, ngv.make_xform(c.A, c.t), W)
    del u0
    loss = torch.zeros(1, dtype=torch.float64, device=DEV)
    gW = torch.empty(shape, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd_order(c.F, W, loss, gW, bins=wl.bins, fixed_order=0)
    torch.cuda.synchronize()
    F, Wn = P.to_np(c.F), P.to_np(W)
    N = F.size
    H = np.zeros((wl.bins, wl.bins))
    for z in range(0, shape[0], 64):
        orc.mi_hist(F[z:z + 64], Wn[z:z + 64].astype(np.float64), bins=wl.bins, order=3, forder=0, H=H)
    mi, L = orc.mi_finalize(H, N)
    P.scalar(float(loss[0]), -mi, what="MI loss (box fixed kernel)")
    rng = np.random.default_rng(9)
    idx = np.unique(rng.integers(0, N, 200000)).astype(np.int64)
    g_ref = orc.mi_grad_values(F.reshape(-1)[idx], Wn.reshape(-1)[idx], L, bins=wl.bins, N=N, order=3, forder=0)
    g = P.to_np(gW.reshape(-1)[torch.as_tensor(idx, device=DEV)])
    edge = near_box_edge(F.reshape(-1)[idx], wl.bins)
    print(f"[info] sampled fixed samples near a box edge: {int(edge.sum())} of {edge.size}", flush=True)
    P.elementwise(g, g_ref, P.RTOL_GRAD, mask=~edge, what="MI gW sampled (box fixed kernel)")
