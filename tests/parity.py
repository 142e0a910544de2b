"""Shared helpers of the parity tests: tolerances and reporting.

Bars (floating point, fp32 kernels against the fp64 oracle):
  losses                       |a - b| <= 1e-4 |b|
  warped voxels W              |a_i - b_i| <= 1e-4 (|b_i| + 1e-3 max|b|)
  gradients gW, gu             |a_i - b_i| <= 1e-3 (|b_i| + 1e-3 max|b|)
  affine sums dA, dt           |a - b| <= 1e-3 |b| + 1e-6 sum_i |g_p(i)| |x(i)|
The floor term keeps near-zero entries meaningful without letting rounding
of tiny values fail the test. Gradients of the sampler are compared away
from cell faces (kinks of the trilinear form), where the one-sided
derivative may differ by the side an fp32 position rounds to.
"""
import numpy as np

RTOL_LOSS = 1e-4
RTOL_W = 1e-4
RTOL_GRAD = 1e-3
FLOOR = 1e-3
KINK_BAND = 1e-4


def to_np(t):
    return t.detach().cpu().numpy()


def elementwise(a, b, rtol, mask=None, floor=FLOOR, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if mask is not None:
        a = a[mask]
        b = b[mask]
    scale = np.abs(b).max() if b.size else 0.0
    tol = rtol * (np.abs(b) + floor * scale)
    err = np.abs(a - b)
    bad = err > tol
    if bad.any():
        i = int(np.argmax(err / np.maximum(tol, 1e-300)))
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} entries out of tolerance; worst "
                             f"a={a.ravel()[i]!r} b={b.ravel()[i]!r} tol={tol.ravel()[i]!r} (max|b|={scale})")
    return float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0


def scalar(a, b, rtol=RTOL_LOSS, what=""):
    assert abs(a - b) <= rtol * abs(b), f"{what}: {a!r} vs {b!r} (rel {abs(a - b) / max(abs(b), 1e-300):.3e})"


def affine_sums(a, b, mag, what=""):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    err = np.linalg.norm(a - b)
    tol = 1e-3 * np.linalg.norm(b) + 1e-6 * mag
    assert err <= tol, f"{what}: |a-b|={err:.3e} > tol {tol:.3e}; a={a} b={b}"


def off_kink(kink, exact_lattice_ok=False):
    """Voxels whose sample is not within KINK_BAND of a cell face. With
    exact_lattice_ok, samples exactly on the lattice (identity maps, where the
    kernel's offset is exactly zero) count as off-kink."""
    if exact_lattice_ok:
        return (kink == 0.0) | (kink >= KINK_BAND)
    return kink >= KINK_BAND


def step_gW(st):
    """The whole similarity gradient dC/dW of a RegistrationStep's last
    forward. When the MI gradient is formed inside the fused backward, gW
    holds only the other terms' part (or nothing), so the MI part is added
    here by the MI gradient sweep from the table the step left in its
    workspace; otherwise gW itself."""
    import torch

    from non_gemm_voxel_amd import ngv
    if not st.mi_bwd:
        return st.gW
    g = st.gW.clone() if st.win else torch.zeros_like(st.gW)
    ngv.ngv_mi_grad(st.F, st.W, g, bins=st.bins, accumulate=True, ws=st.ws)
    return g


# fp32 values of the optimiser constants as the C ABI receives them (floats);
# the oracle is given the same values widened to fp64, as it is for the
# sampler's parameters
def f32(v):
    return float(np.float32(v))


BETA1, BETA2, EPS_ADAM = f32(0.9), f32(0.999), f32(1e-8)
U32 = 2.0 ** -24  # unit roundoff of fp32


def grad_bar(g):
    """The gradient bar per entry, RTOL_GRAD (|g| + FLOOR max|g|), with the
    maximum taken per component (axis 0) of g."""
    g = np.abs(np.asarray(g, np.float64))
    scale = g.reshape(g.shape[0], -1).max(axis=1).reshape((-1,) + (1,) * (g.ndim - 1))
    return RTOL_GRAD * (g + FLOOR * scale)


def adam_bars(g, m1_prev, m2_prev, step, lr, b1=BETA1, b2=BETA2, eps=EPS_ADAM, g_extra=None):
    """Bars for m1, m2 and the update du = u_new - u after one Adam step from
    (m1_prev, m2_prev) with the oracle's gradient g (fp64), carried through the
    step's arithmetic from the gradient bar (a kernel whose gradient meets
    grad_bar(g) can be off by this much), plus a few fp32 roundings of each
    result. m1 and m2 are linear in g and g^2; du is monotone in m1 and in m2,
    so its bar is the largest change over the corners of the m1, m2 box.
    g_extra: a further per-entry allowance on the gradient, added to its bar.
    Returns (m1, m2, du) references and (t_m1, t_m2, t_du) bars."""
    g = np.asarray(g, np.float64)
    m1p = np.asarray(m1_prev, np.float64)
    m2p = np.asarray(m2_prev, np.float64)
    tg = grad_bar(g)
    if g_extra is not None:
        tg = tg + np.asarray(g_extra, np.float64)
    m1 = b1 * m1p + (1.0 - b1) * g
    m2 = b2 * m2p + (1.0 - b2) * g * g
    t1 = (1.0 - b1) * tg + 4 * U32 * (np.abs(m1) + b1 * np.abs(m1p))
    t2 = (1.0 - b2) * (2.0 * np.abs(g) * tg + tg * tg) + 4 * U32 * (np.abs(m2) + b2 * np.abs(m2p))
    bc1 = 1.0 - b1 ** step
    bc2 = 1.0 - b2 ** step

    def du_of(a, b):
        return -lr * (a / bc1) / (np.sqrt(np.maximum(b, 0.0) / bc2) + eps)

    du = du_of(m1, m2)
    td = np.zeros_like(du)
    for s1 in (-1.0, 1.0):
        for s2 in (-1.0, 1.0):
            td = np.maximum(td, np.abs(du_of(m1 + s1 * t1, m2 + s2 * t2) - du))
    td += 8 * U32 * np.abs(du)
    return (m1, m2, du), (t1, t2, td)


def within(a, b, tol, mask=None, what=""):
    """|a - b| <= tol elementwise (over mask); returns the worst err / tol."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    tol = np.broadcast_to(np.asarray(tol, np.float64), b.shape)
    assert a.shape == b.shape, (a.shape, b.shape)
    if mask is not None:
        a, b, tol = a[mask], b[mask], tol[mask]
    err = np.abs(a - b)
    bad = err > tol
    if bad.any():
        i = int(np.argmax(err / np.maximum(tol, 1e-300)))
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} entries out of tolerance; worst "
                             f"a={a.ravel()[i]!r} b={b.ravel()[i]!r} tol={tol.ravel()[i]!r}")
    return float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0


def check_adam_step(orc, u_new, m1_new, m2_new, u_prev, m1_prev, m2_prev, g_ref, step, lr, mask=None, what="",
                    g_extra=None):
    """One Adam step of the kernels (fp32 states after the step) against the
    oracle's step from the same previous state with the oracle's gradient
    g_ref, within the bars that adam_bars carries from the gradient bar.
    Arrays are (3, ...) per component; mask (broadcast to them) selects the
    entries compared, e.g. off the sampler's kinks."""
    shape = np.shape(g_ref)
    u_prev = np.asarray(u_prev, np.float32)
    ur, m1r, m2r = orc.adam(u_prev, g_ref, m1_prev, m2_prev, step, lr, BETA1, BETA2, EPS_ADAM)
    ur, m1r, m2r = ur.reshape(shape), m1r.reshape(shape), m2r.reshape(shape)
    _, (t1, t2, td) = adam_bars(g_ref, m1_prev, m2_prev, step, lr, g_extra=g_extra)
    m = None if mask is None else np.broadcast_to(mask, shape)
    u_new = np.asarray(u_new, np.float64)
    du = u_new - u_prev
    dur = ur - u_prev
    within(m1_new, m1r, t1, m, what=f"{what} m1")
    within(m2_new, m2r, t2, m, what=f"{what} m2")
    within(du, dur, td + U32 * np.abs(u_new), m, what=f"{what} du")


def mi_grad_bar(g, mag_terms, mag_coord, bins, coord_units=3):
    """Bar for an MI gradient evaluated in fp32: the gradient bar RTOL_GRAD
    (|g| + FLOOR max|g|), or, where larger, the forward error of evaluating
    it in fp32, from the oracle's conditioning scales (orc_mi_grad modes 1
    and 2): the sum of 16 table-weighted terms (4 with the box fixed kernel)
    and the fp32 table contribute up to 32 u32 times the terms' magnitude,
    and the fp32 bin coordinates (up to bins - 3, rounded by a few units)
    move the spline weights by up to coord_units u32 bins times the sum's
    derivative (3 for the coordinate's own rounding; more where W itself
    comes from the kernels' fp32 sampler, a few fp32 units of W, which the
    bin scale (< bins) carries into the coordinate).
    Where the terms cancel (sparse histograms, many bins) the result is far
    smaller than they are and only the second bound can be met in fp32."""
    g = np.abs(np.asarray(g, np.float64))
    fp32 = 32 * U32 * np.asarray(mag_terms, np.float64) + coord_units * U32 * bins * np.asarray(mag_coord, np.float64)
    return np.maximum(RTOL_GRAD * (g + FLOOR * g.max()), fp32)


# The kernels compute W in fp32 (the type in which the boundary carries it):
# a few fp32 units from the oracle's fp64 W, where rounding it to fp32 moves
# it by at most half a unit.
W_ROUND_FACTOR = 16


def rounding_sensitivity(g_fp64_W, g_fp32_W):
    """An allowance for a gradient computed from the kernels' fp32 W rather
    than the oracle's fp64 W: how far the oracle's own gradient moves when
    its W is rounded to fp32 (|g(W) - g(fp32(W))|), as a local maximum over
    each voxel's 3^3 neighbourhood (so that a voxel where the rounding
    happens to cancel takes its neighbours' scale), times W_ROUND_FACTOR.
    Near convergence the LNCC gradient is a small remainder of large
    cancelling window terms, and this is the scale at which fp32 inputs
    determine it."""
    import scipy.ndimage as ndi
    d = np.abs(np.asarray(g_fp64_W, np.float64) - np.asarray(g_fp32_W, np.float64))
    return W_ROUND_FACTOR * ndi.maximum_filter(d, size=3, mode="nearest")


def kink_allowance(orc, M, u, prm, gW, kink, exact_lattice_ok=False):
    """An allowance on gu (3, ...) for samples near a cell face, where the
    trilinear derivative is one-sided and either side is a valid answer (an
    fp32 position may fall on the other side): the spread of the valid
    answers from the oracle (warp_kink_spread with KINK_BAND), zero away from
    faces. With exact_lattice_ok (identity maps, where the kernels' offset is
    exactly zero), samples exactly on the lattice take the floor cell on both
    sides, so they get no allowance."""
    sp = orc.warp_kink_spread(M, u, prm, gW, band=KINK_BAND)
    if exact_lattice_ok:
        sp[:, np.asarray(kink) == 0.0] = 0.0
    return sp
