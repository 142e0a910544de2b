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
