"""ngv_mi_loss_fwd_bwd_noalloc -- the MI loss and gradient with the library's
fixed per-GPU scratch instead of a caller's workspace -- against
ngv_mi_loss_fwd_bwd with a workspace, bit for bit (the same kernels on the
same inputs), and against the oracle, on calls in a row: the second with a
smaller volume and fewer bins, so that a histogram left in the scratch by the
first call would show, then a loss-only call and an accumulating one.
"""
import numpy as np
import pytest
import torch

from non_gemm_voxel_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(shape, seed):
    F = synth.random_volume(shape, seed, 0, -0.05, 1.05).numpy()
    W = (0.6 * F + 0.4 * synth.random_volume(shape, seed, 1).numpy()).astype(np.float32)
    return torch.as_tensor(F).to(DEV), torch.as_tensor(W).to(DEV)


def _pair(ngv, F, W, bins, with_grad=True, accumulate=False, start=None):
    """(loss, gW) of the workspace call and of the no-allocation call."""
    out = []
    for noalloc in (False, True):
        loss = torch.full((1,), 0.0 if start is None else start[0], dtype=torch.float64, device=DEV)
        gW = None
        if with_grad:
            gW = torch.full_like(F, 0.0 if start is None else start[1])
        if noalloc:
            ngv.ngv_mi_loss_fwd_bwd_noalloc(F, W, loss, gW, bins=bins, weight=1.25, accumulate=accumulate)
        else:
            ngv.ngv_mi_loss_fwd_bwd(F, W, loss, gW, bins=bins, weight=1.25, accumulate=accumulate)
        out.append((loss, gW))
    torch.cuda.synchronize()
    return out


def test_noalloc_mi_matches_the_workspace_call(orc):
    from non_gemm_voxel_amd import ngv
    for shape, bins in (((37, 61, 83), 64), ((9, 20, 31), 32), ((3, 5, 7), 128)):
        print("[case] noalloc mi", shape, bins, flush=True)
        F, W = _inputs(shape, 13 + bins)
        (l_ws, g_ws), (l_na, g_na) = _pair(ngv, F, W, bins)
        assert torch.equal(l_ws, l_na) and torch.equal(g_ws, g_na)
        Fn, Wn = P.to_np(F), P.to_np(W).astype(np.float64)
        lo, go, H = orc.mi_loss_grad(Fn, Wn, bins=bins, weight=1.25)
        P.scalar(float(l_na[0]), lo, what="MI loss (no allocation)")
        _, L = orc.mi_finalize(H, Fn.size)
        mags = [orc.mi_grad_values(Fn, Wn, L, bins=bins, weight=1.25, N=Fn.size, mode=m).reshape(Fn.shape)
                for m in (1, 2)]
        P.within(P.to_np(g_na), go, P.mi_grad_bar(go, *mags, bins), what="MI gW (no allocation)")
    # loss only, then accumulating into a loss and gradient that hold values
    F, W = _inputs((11, 13, 17), 5)
    (l_ws, _), (l_na, _) = _pair(ngv, F, W, 16, with_grad=False)
    assert torch.equal(l_ws, l_na)
    (l_ws, g_ws), (l_na, g_na) = _pair(ngv, F, W, 16, accumulate=True, start=(0.5, -0.25))
    assert torch.equal(l_ws, l_na) and torch.equal(g_ws, g_na)


def test_noalloc_mi_refuses_more_bins_than_its_scratch_holds():
    from non_gemm_voxel_amd import ngv
    F, W = _inputs((4, 4, 4), 3)
    loss = torch.zeros(1, dtype=torch.float64, device=DEV)
    with pytest.raises(ngv.NgvError) as e:
        ngv.ngv_mi_loss_fwd_bwd_noalloc(F, W, loss, None, bins=129)
    assert e.value.code == ngv.NGV_EUNSUPPORTED
