"""The seeded input generator: determinism and the stated ranges."""
import numpy as np
import torch

from non_gemm_voxel_amd import synth


def test_hash_uniform_range_and_determinism():
    idx = torch.arange(0, 1 << 16, dtype=torch.int64)
    a = synth.uniform(3, 1, idx)
    b = synth.uniform(3, 1, idx)
    assert torch.equal(a, b)
    assert float(a.min()) > 0.0 and float(a.max()) < 1.0
    assert abs(float(a.mean()) - 0.5) < 0.01
    c = synth.uniform(3, 2, idx)
    assert not torch.equal(a, c)
    # indices beyond 2^32 use the high word too
    hi = synth.uniform(3, 1, idx + (1 << 32))
    assert not torch.equal(a, hi)


def test_normal_moments():
    idx = torch.arange(0, 1 << 18, dtype=torch.int64)
    g = synth.normal(7, 0, idx)
    assert abs(float(g.mean())) < 0.01
    assert abs(float(g.std()) - 1.0) < 0.01


def test_chunking_does_not_change_values():
    shape = (9, 10, 11)
    f1 = synth.SmoothField(shape, 5, 30, 2.0)
    full = f1.chunk(0, 9)
    parts = torch.cat([f1.chunk(0, 4), f1.chunk(4, 9)], dim=1)
    assert torch.equal(full, parts)
    assert abs(float(torch.sqrt((full * full).sum(0)).max()) - 2.0) < 1e-12


def test_case_c1_ranges_and_repeatability():
    c = synth.make_case("c1")
    d = synth.make_case("c1")
    assert torch.equal(c.F, d.F) and torch.equal(c.M, d.M)
    assert c.F.shape == (64, 64, 64) and c.F.dtype == torch.float32
    assert float(c.F.min()) >= 0.0 and float(c.F.max()) == 1.0
    assert float(c.M.min()) >= 0.0 and float(c.M.max()) <= 1.0
    assert np.array_equal(c.A, np.eye(3, dtype=np.float32))


def test_small_versions_of_the_phantoms():
    c2 = synth.make_case("c2", shape=(40, 48, 56))
    bg = float((c2.F < 0.1).float().mean())
    assert 0.5 < bg < 0.75  # about 62% background at any size
    c3 = synth.make_case("c3", shape=(32, 32, 32))
    assert float(c3.M.max()) <= 1.0 and float(c3.M.min()) >= 0.0
    c4 = synth.make_case("c4", shape=(48, 56, 48))
    vals = np.round(c4.F.numpy(), 1)
    for level in (0.0, 0.2, 0.4, 0.6, 0.8):  # bg, CSF, sheets, WM
        assert (vals == level).mean() > 0.005
    A = c4.A.astype(np.float64)
    # the start affine undoes the generating one (normalised frame)
    nz, ny, nx = c4.shape
    D = np.diag([(nx - 1) / 2, (ny - 1) / 2, (nz - 1) / 2])
    assert np.abs(D @ A @ np.linalg.inv(D) @ c4.L_gen - np.eye(3)).max() < 1e-6
