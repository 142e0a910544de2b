"""The step driver's choice of call sequence, on the host (no kernels run):
which fused calls RegistrationStep uses for each combination of terms,
smoothing, slabs and options, and how it splits the moving image."""
import pytest
import torch

from non_gemm_voxel_amd.step import RegistrationStep


def _step(shape=(8, 9, 10), **kw):
    F = torch.zeros(shape)
    M = torch.zeros(shape)
    return RegistrationStep(F, M, None, None, **kw)


def test_needs_a_similarity_term():
    with pytest.raises(ValueError):
        _step()


@pytest.mark.parametrize("kw,fused,mi_bwd,fused_mi,fused_step", [
    # the default step: backward fused with Adam; with MI it forms the MI gradient
    (dict(bins=32, win=9), True, True, False, False),
    (dict(win=7, smooth_sigma=1.0), False, False, False, False),  # smoothing: separate Adam
    (dict(bins=32), True, True, False, False),
    (dict(bins=32, win=9, slabs=8), True, True, False, False),  # slabs: the MI gradient from the stored W
    (dict(bins=200, win=9), True, False, False, False),  # the sampler's LDS tables take 128 bins
    (dict(bins=32, win=9, fused=False), False, False, False, False),
    (dict(bins=32, win=9, mi_in_backward=False), True, False, False, False),
    (dict(bins=32, win=9, fused_mi=True), True, True, True, False),
    (dict(bins=200, win=9, fused_mi=True), True, False, False, False),
    # the two-sweep step: an LNCC term, one slab, w <= 11, MI bins <= 128
    (dict(bins=32, win=9, fused_step=True), True, True, False, True),
    (dict(win=7, smooth_sigma=1.0, fused_step=True), False, False, False, True),
    (dict(bins=32, fused_step=True), True, True, False, False),
    (dict(bins=32, win=9, slabs=2, fused_step=True), True, True, False, False),
    (dict(bins=32, win=9, slabs=8, mi_in_backward=False), True, False, False, False),
    (dict(bins=32, win=13, fused_step=True), True, True, False, False),
    (dict(bins=200, win=9, fused_step=True), True, False, False, False),
])
def test_call_sequence_choice(kw, fused, mi_bwd, fused_mi, fused_step):
    st = _step(**kw)
    assert (st.fused, st.mi_bwd, st.fused_mi, st.fused_step) == (fused, mi_bwd, fused_mi, fused_step)


@pytest.mark.parametrize("nz,slabs", [(10, 1), (10, 3), (16, 8), (7, 7)])
def test_slabs_cover_the_moving_image(nz, slabs):
    st = _step(shape=(nz, 4, 5), bins=32, slabs=slabs)
    z = 0
    for (z0, n), view in zip(st.slabs, st.M_views):
        assert z0 == z and n >= 1 and view.shape[0] == n
        z += n
    assert z == nz
    assert (st.zrange is not None) == (slabs > 1)


def test_workspace_holds_the_window():
    from non_gemm_voxel_amd import ngv
    st = _step(win=21)
    assert st.ws.numel() >= ngv.ngv_workspace_bytes(32, 21)
