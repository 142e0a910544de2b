"""A whole registration step recorded once as a HIP graph and replayed: every
replay is bit for bit the eager step it stands for (the Adam step number is
advanced on the device), with the program's own eager work and
synchronisations between the replays. Covers the fused path, the smoothed
path (separate backward and update) and the slab sequence."""
import pytest
import torch

from non_gemm_voxel_amd import synth
from non_gemm_voxel_amd.step import RegistrationStep

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("wl_name,shape,slabs", [("c1", None, 1), ("c2", (24, 32, 40), 1),
                                                 ("c5", (40, 48, 40), 4)])
def test_graph_replays_match_eager_steps(wl_name, shape, slabs):
    print("[case] graph", wl_name, shape, slabs, flush=True)
    wl = synth.WORKLOADS[wl_name]
    c = synth.make_case(wl, shape=shape)

    def make():
        return RegistrationStep(c.F.to(DEV), c.M.to(DEV), c.A, c.t, bins=wl.bins, win=wl.win,
                                smooth_sigma=wl.smooth_sigma, lr=c.lr, slabs=slabs)

    a, b = make(), make()
    a.step()
    b.step()
    graph = a.capture()
    torch.cuda.synchronize()
    assert torch.equal(a.u, b.u)  # recording ran nothing
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        x = torch.arange(4096, device=DEV, dtype=torch.float32)  # eager work between replays
        assert float((x * 2).max()) == 8190.0
        b.step()
        torch.cuda.synchronize()
        for name in ("u", "m1", "m2", "W", "gW", "loss", "gA", "gt", "step_dev"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
    assert int(a.step_dev[0]) == 4
