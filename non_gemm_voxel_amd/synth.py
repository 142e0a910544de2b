"""Seeded synthetic volume pairs for the registration step.

This module holds input generation only: analytic phantoms, a smooth random
displacement, noise and the affine set-up. It contains none of the step's
arithmetic (no grid sampling, no Parzen windows, no window sums): the moving
image is made by evaluating the analytic phantom at warped coordinates, never
by resampling a stored volume. Both the HIP path and the oracle take their
inputs from here; nothing here depends on either.

Randomness is counter based, so any voxel's value is a pure function of
(seed, stream, voxel index) and volumes can be generated in z-chunks on the
CPU or on a GPU with the same recipe. The hash is Chris Wellons' "lowbias32"
32-bit integer mixer (published in "Prospecting for Hash Functions"),
evaluated with 16-bit partial products so that every intermediate stays below
2^49 in int64 on every device. Normals use the Box-Muller transform.

Volumes are (nz, ny, nx) float32 with x fastest; voxel coordinates are
(x, y, z) = (fastest ... slowest). The registration frame is the normalised
[-1, 1] cube per axis, voxel centres of the end voxels at -1 and +1.
"""
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

_MASK32 = 0xFFFFFFFF


def _mul32(x, c):
    lo = x * (c & 0xFFFF)
    hi = ((x * (c >> 16)) & 0xFFFF) << 16
    return (lo + hi) & _MASK32


def hash32(x):
    """lowbias32 on an int64 tensor holding values in [0, 2^32)."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _key(seed, stream):
    k = (seed * 0x9E3779B1 + stream * 0x85EBCA77 + 0x27D4EB2F) & _MASK32
    return int(hash32(torch.tensor([k], dtype=torch.int64))[0])


def uniform(seed, stream, idx, dtype=torch.float64):
    """U(0,1) (24-bit, never 0 or 1) for int64 counter tensor idx."""
    k = _key(seed, stream)
    h = hash32(hash32((idx & _MASK32) ^ k) ^ (idx >> 32))
    return ((h >> 8).to(dtype) + 0.5) * (1.0 / 16777216.0)


def normal(seed, stream, idx, dtype=torch.float64):
    u1 = uniform(seed, stream, idx, dtype)
    u2 = uniform(seed, stream + 7919, idx, dtype)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)


def scalars(seed, stream, n, kind="uniform"):
    """n host-side random numbers (float64 numpy) for small parameters."""
    idx = torch.arange(n, dtype=torch.int64)
    f = uniform if kind == "uniform" else normal
    return f(seed, stream, idx).numpy()


# --------------------------------------------------------------------------
# affine helpers (voxel frame)
# --------------------------------------------------------------------------

def euler_rotation(ax, ay, az):
    """R = Rz(az) Ry(ay) Rx(ax) acting on (x, y, z) column vectors (radians)."""
    cx, sx, cy, sy, cz, sz = math.cos(ax), math.sin(ax), math.cos(ay), math.sin(ay), math.cos(az), math.sin(az)
    Rx = np.array([[1, 0, 0], [0, cx, -sx], [0, sx, cx]])
    Ry = np.array([[cy, 0, sy], [0, 1, 0], [-sy, 0, cy]])
    Rz = np.array([[cz, -sz, 0], [sz, cz, 0], [0, 0, 1]])
    return Rz @ Ry @ Rx


def normalised_inverse(L, shape):
    """The affine that undoes x -> c + L (x - c) (c: volume centre), written in
    the normalised frame: A = D^-1 L^-1 D with D = diag((n - 1)/2), t = 0."""
    nz, ny, nx = shape
    D = np.diag([(nx - 1) / 2.0, (ny - 1) / 2.0, (nz - 1) / 2.0])
    return np.linalg.inv(D) @ np.linalg.inv(L) @ D


# --------------------------------------------------------------------------
# smooth random displacement
# --------------------------------------------------------------------------

class SmoothField:
    """A smooth random vector field on a grid, in voxel units: each component
    is a sum of K separable low-frequency cosine modes with N(0,1) amplitudes,
    frequencies U[0.25, fmax] cycles per extent and uniform phases. This is a
    band-limited stand-in for Gaussian-smoothed noise that can be evaluated at
    any voxel in closed form. ``scale`` is set so that the largest Euclidean
    norm over the grid equals ``max_norm``."""

    def __init__(self, shape, seed, stream, max_norm, K=6, fmax=2.0, device="cpu"):
        self.shape = tuple(shape)
        self.K = K
        self.device = device
        nz, ny, nx = shape
        a = scalars(seed, stream, 3 * K, "normal").reshape(3, K)
        f = 0.25 + (fmax - 0.25) * scalars(seed, stream + 1, 3 * K).reshape(3, K)  # per axis, per mode
        ph = 2.0 * math.pi * scalars(seed, stream + 2, 3 * 3 * K).reshape(3, 3, K)  # comp, axis, mode
        self.amp = torch.tensor(a, dtype=torch.float64, device=device)
        self.tab = []  # tab[c][axis]: (K, n_axis) cosine tables
        for c in range(3):
            row = []
            for ax, n in enumerate((nx, ny, nz)):
                i = torch.arange(n, dtype=torch.float64, device=device)
                w = torch.tensor(2.0 * math.pi * f[ax] / max(n, 1), dtype=torch.float64, device=device)
                p = torch.tensor(ph[c, ax], dtype=torch.float64, device=device)
                row.append(torch.cos(w[:, None] * i[None, :] + p[:, None]))
            self.tab.append(row)
        self.scale = 1.0
        if max_norm > 0:
            peak = 0.0
            for z0, z1 in z_chunks(nz, nx * ny):
                d = self.chunk(z0, z1)
                peak = max(peak, float(torch.sqrt((d * d).sum(0)).max()))
            self.scale = max_norm / peak if peak > 0 else 0.0
        else:
            self.scale = 0.0

    def chunk(self, z0, z1):
        """(3, z1-z0, ny, nx) float64 field for planes [z0, z1)."""
        nz, ny, nx = self.shape
        out = torch.zeros((3, z1 - z0, ny, nx), dtype=torch.float64, device=self.device)
        for c in range(3):
            tx, ty, tz = self.tab[c]
            for k in range(self.K):
                out[c] += (self.amp[c, k] * tz[k, z0:z1])[:, None, None] * ty[k][None, :, None] * tx[k][None, None, :]
        return out * self.scale


def z_chunks(nz, plane, budget=1 << 24):
    step = max(1, budget // max(plane, 1))
    return [(z, min(nz, z + step)) for z in range(0, nz, step)]


def _grid(z0, z1, ny, nx, device):
    z = torch.arange(z0, z1, dtype=torch.float64, device=device)[:, None, None]
    y = torch.arange(ny, dtype=torch.float64, device=device)[None, :, None]
    x = torch.arange(nx, dtype=torch.float64, device=device)[None, None, :]
    return x, y, z


def _lin_idx(z0, z1, ny, nx, device):
    return torch.arange(z0 * ny * nx, z1 * ny * nx, dtype=torch.int64, device=device).reshape(z1 - z0, ny, nx)


# --------------------------------------------------------------------------
# analytic phantoms: intensity as a function of continuous voxel position
# --------------------------------------------------------------------------

class Blobs:
    """Sum of Gaussian blobs (centres U[0, n-1]^3, sigma U[3, 10], amplitude
    U[0.3, 1], each cut to zero beyond 4 sigma), divided by the sum's maximum
    over the voxel grid."""

    def __init__(self, shape, seed, nblobs=40, device="cpu"):
        nz, ny, nx = shape
        r = scalars(seed, 10, 6 * nblobs).reshape(nblobs, 6)
        self.c = torch.tensor(np.stack([r[:, 0] * (nx - 1), r[:, 1] * (ny - 1), r[:, 2] * (nz - 1)], 1),
                              device=device)
        self.s = torch.tensor(3.0 + 7.0 * r[:, 3], device=device)
        self.a = torch.tensor(0.3 + 0.7 * r[:, 4], device=device)
        self.norm = 1.0
        peak = 0.0
        for z0, z1 in z_chunks(nz, nx * ny):
            x, y, z = _grid(z0, z1, ny, nx, device)
            peak = max(peak, float(self.raw(x, y, z).max()))
        self.norm = peak

    def raw(self, x, y, z):
        out = torch.zeros(torch.broadcast_shapes(x.shape, y.shape, z.shape), dtype=torch.float64, device=x.device)
        for i in range(self.c.shape[0]):
            d2 = (x - self.c[i, 0]) ** 2 + (y - self.c[i, 1]) ** 2 + (z - self.c[i, 2]) ** 2
            s2 = self.s[i] ** 2
            out += torch.where(d2 <= 16.0 * s2, self.a[i] * torch.exp(-d2 / (2.0 * s2)), torch.zeros_like(d2))
        return out

    def __call__(self, x, y, z):
        return self.raw(x, y, z) / self.norm


def _ell_radius(x, y, z, shape):
    nz, ny, nx = shape
    hx, hy, hz = (nx - 1) / 2.0, (ny - 1) / 2.0, (nz - 1) / 2.0
    X, Y, Z = (x - hx) / hx, (y - hy) / hy, (z - hz) / hz
    return X, Y, Z, torch.sqrt(X * X + Y * Y + Z * Z)


class Brain:
    """Nested ellipsoids (semi-axes 0.90 / 0.82 / 0.60 of the half-extent):
    background 0, CSF 0.25, grey matter 0.55, white matter 0.85. ``label``
    gives the class 0..3, ``levels`` the intensity of each class."""

    def __init__(self, shape, levels=(0.0, 0.25, 0.55, 0.85)):
        self.shape = shape
        self.levels = levels

    def label(self, x, y, z):
        _, _, _, rho = _ell_radius(x, y, z, self.shape)
        lab = torch.zeros_like(rho, dtype=torch.int64)
        lab = torch.where(rho <= 0.90, torch.ones_like(lab), lab)
        lab = torch.where(rho <= 0.82, torch.full_like(lab, 2), lab)
        lab = torch.where(rho <= 0.60, torch.full_like(lab, 3), lab)
        return lab

    def __call__(self, x, y, z, levels=None):
        lv = torch.tensor(levels or self.levels, dtype=torch.float64, device=x.device)
        return lv[self.label(x, y, z)]


class Cortex:
    """Layered-cortex phantom: a brain ellipsoid (0.85 of the half-extent) whose
    radius is folded by (1 + 0.04 sin 6theta sin 5phi); outside it a CSF shell
    (0.25) up to 0.90, background 0 beyond; inside, a cortical band ``band``
    voxels deep made of alternating ``sheet``-voxel sheets (0.45 / 0.65), and
    white matter (0.85) below the band."""

    def __init__(self, shape, band=24.0, sheet=2.0):
        self.shape = shape
        self.band = band
        self.sheet = sheet
        nz, ny, nx = shape
        self.hmin = min(nx - 1, ny - 1, nz - 1) / 2.0

    def __call__(self, x, y, z):
        X, Y, Z, rho = _ell_radius(x, y, z, self.shape)
        theta = torch.acos(torch.clamp(Z / torch.clamp(rho, min=1e-12), -1.0, 1.0))
        phi = torch.atan2(Y, X)
        rf = rho / (1.0 + 0.04 * torch.sin(6.0 * theta) * torch.sin(5.0 * phi))
        depth = (0.85 - rf) * self.hmin
        sheet_idx = torch.floor(depth / self.sheet)
        cortex = torch.where(torch.remainder(sheet_idx, 2.0) == 0, torch.full_like(rf, 0.45),
                             torch.full_like(rf, 0.65))
        out = torch.where(depth >= self.band, torch.full_like(rf, 0.85), cortex)
        out = torch.where(rf > 0.85, torch.full_like(rf, 0.25), out)
        out = torch.where(rf > 0.90, torch.zeros_like(rf), out)
        return out


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    shape: tuple             # (nz, ny, nx)
    seed: int
    phantom: str             # blobs | brain | brain_mm | cortex
    rot_deg: tuple           # fixed Euler angles (x, y, z) or None
    rot_range: float         # |angle| bound for random Euler angles (deg), 0: none
    scale_range: float       # |s - 1| bound for random scales, 0: none
    max_disp: float          # max |d| in voxels
    noise: float             # Gaussian noise sd (F and M), 0: none
    rician: float = 0.0      # Rician noise sd on M (multimodal case)
    band: float = 24.0       # cortex band depth in voxels
    bins: Optional[int] = None   # MI bins, None: no MI term
    win: Optional[int] = None    # LNCC window, None: no LNCC term
    smooth_sigma: float = 0.0    # gradient smoothing before the update
    iters: int = 1
    slabs: int = 1               # z-slabs for the moving image
    affine_start: bool = False   # start from the inverse of the generating affine
    note: str = ""


WORKLOADS = {
    "c1": Workload("c1", (64, 64, 64), 1, "blobs", (0.0, 0.0, 3.0), 0.0, 0.0, 2.0, 0.0,
                   bins=32, win=5, note="64^3 Gaussian blobs, one step of LNCC(w=5) + MI(B=32)"),
    "c2": Workload("c2", (160, 192, 224), 2, "brain", None, 5.0, 0.03, 4.0, 0.02,
                   win=7, smooth_sigma=1.0, iters=200, affine_start=True,
                   note="160x192x224 brain phantom, LNCC(w=7), 200 Adam iterations with smoothing"),
    "c3": Workload("c3", (256, 256, 256), 3, "brain_mm", None, 0.0, 0.0, 6.0, 0.02, rician=0.03,
                   bins=32, iters=100, note="256^3 multimodal pair, MI(B=32), 100 iterations"),
    "c4": Workload("c4", (640, 768, 640), 4, "cortex", None, 5.0, 0.03, 8.0, 0.02, band=24.0,
                   bins=32, win=9, affine_start=True,
                   note="640x768x640 layered cortex, MI(B=32) + LNCC(w=9), one step"),
    "c5": Workload("c5", (1280, 1536, 1280), 5, "cortex", None, 3.0, 0.02, 8.0, 0.02, band=48.0,
                   bins=32, win=9, slabs=8, affine_start=True,
                   note="1280x1536x1280 gigavoxel cortex, MI(B=32) + LNCC(w=9), moving image in 8 z-slabs"),
}


@dataclass
class Case:
    """A generated volume pair with its registration set-up."""
    wl: Workload
    shape: tuple
    F: torch.Tensor
    M: torch.Tensor
    A: np.ndarray            # 3x3 float32, normalised frame
    t: np.ndarray            # 3 float32
    S: np.ndarray = field(default_factory=lambda: np.eye(3, dtype=np.float32))
    xmin: np.ndarray = field(default_factory=lambda: -np.ones(3, dtype=np.float32))
    xmax: np.ndarray = field(default_factory=lambda: np.ones(3, dtype=np.float32))
    L_gen: np.ndarray = None  # generating linear map (voxel frame)
    lr: float = 0.0


def _gen_affine(wl):
    if wl.rot_deg is not None:
        ang = [math.radians(a) for a in wl.rot_deg]
        scl = [1.0, 1.0, 1.0]
    elif wl.rot_range > 0 or wl.scale_range > 0:
        r = scalars(wl.seed, 20, 6)
        ang = [math.radians(wl.rot_range * (2 * r[i] - 1)) for i in range(3)]
        scl = [1.0 + wl.scale_range * (2 * r[3 + i] - 1) for i in range(3)]
    else:
        ang, scl = [0.0, 0.0, 0.0], [1.0, 1.0, 1.0]
    return euler_rotation(*ang) @ np.diag(scl)


def make_case(wl, shape=None, device="cpu", band=None):
    """Generate F and M for workload ``wl`` (a Workload or its name) at its own
    shape or at ``shape`` (same recipe, e.g. a small version for checks).

    M(x) = phantom(psi(x)) with psi(x) = c + L (x - c) + d(x), L = R diag(s),
    c the volume centre, d the smooth displacement; noise is drawn
    independently for F and M (two acquisitions)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    shape = tuple(shape or wl.shape)
    nz, ny, nx = shape
    L = _gen_affine(wl)
    disp = SmoothField(shape, wl.seed, 30, wl.max_disp, device=device)
    if wl.phantom == "blobs":
        ph = Blobs(shape, wl.seed, device=device)
    elif wl.phantom in ("brain", "brain_mm"):
        ph = Brain(shape)
    else:
        scale = min(shape) / min(wl.shape)
        ph = Cortex(shape, band=band if band is not None else max(4.0, wl.band * scale))
    F = torch.empty(shape, dtype=torch.float32, device=device)
    M = torch.empty(shape, dtype=torch.float32, device=device)
    c = torch.tensor([(nx - 1) / 2.0, (ny - 1) / 2.0, (nz - 1) / 2.0], dtype=torch.float64, device=device)
    Lt = torch.tensor(L, dtype=torch.float64, device=device)
    for z0, z1 in z_chunks(nz, nx * ny, 1 << 22):
        x, y, z = _grid(z0, z1, ny, nx, device)
        idx = _lin_idx(z0, z1, ny, nx, device)
        # fixed image
        f = ph(x, y, z)
        if wl.noise > 0:
            f = f + wl.noise * normal(wl.seed, 40, idx)
        F[z0:z1] = torch.clamp(f, 0.0, 1.0).to(torch.float32)
        # moving image: the phantom at psi(x)
        X = x.expand(z1 - z0, ny, nx) - c[0]
        Y = y.expand(z1 - z0, ny, nx) - c[1]
        Z = z.expand(z1 - z0, ny, nx) - c[2]
        d = disp.chunk(z0, z1)
        px = c[0] + Lt[0, 0] * X + Lt[0, 1] * Y + Lt[0, 2] * Z + d[0]
        py = c[1] + Lt[1, 0] * X + Lt[1, 1] * Y + Lt[1, 2] * Z + d[1]
        pz = c[2] + Lt[2, 0] * X + Lt[2, 1] * Y + Lt[2, 2] * Z + d[2]
        if wl.phantom == "brain_mm":
            g = ph(px, py, pz, levels=(0.0, 0.90, 0.35, 0.60))
            n1 = wl.rician * normal(wl.seed, 50, idx)
            n2 = wl.rician * normal(wl.seed, 60, idx)
            m = torch.sqrt((g + n1) ** 2 + n2 ** 2)
        else:
            m = ph(px, py, pz)
            if wl.noise > 0:
                m = m + wl.noise * normal(wl.seed, 70, idx)
        M[z0:z1] = torch.clamp(m, 0.0, 1.0).to(torch.float32)
    if wl.affine_start:
        A = normalised_inverse(L, shape)
    else:
        A = np.eye(3)
    lr = 0.5 / (max(shape) - 1)
    return Case(wl, shape, F, M, A.astype(np.float32), np.zeros(3, np.float32), L_gen=L, lr=lr)


def random_field(shape, seed, stream, max_norm, device="cpu", dtype=torch.float32):
    """A smooth random 3-vector field (3, nz, ny, nx), largest norm max_norm."""
    sf = SmoothField(shape, seed, stream, max_norm, device=device)
    return sf.chunk(0, shape[0]).to(dtype)


def random_volume(shape, seed, stream, lo=0.0, hi=1.0, device="cpu", dtype=torch.float32):
    """i.i.d. U(lo, hi) voxels."""
    n = int(np.prod(shape))
    idx = torch.arange(n, dtype=torch.int64, device=device).reshape(shape)
    return (lo + (hi - lo) * uniform(seed, stream, idx)).to(dtype)
