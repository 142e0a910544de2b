"""A whole registration step recorded once as a HIP graph and replayed: every
replay is bit for bit the eager step it stands for (the Adam step number is
advanced on the device), with the program's own eager work and
synchronisations between the replays. Covers the fused path, the smoothed
path (separate backward and update), the slab sequence (its backward forming
the MI gradient from the stored W) and the two-sweep step."""
import pytest
import torch

from non_gemm_voxel_amd import synth
from non_gemm_voxel_amd.step import RegistrationStep

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("wl_name,shape,slabs,fused_step", [("c1", None, 1, False), ("c2", (24, 32, 40), 1, False),
                                                            ("c5", (40, 48, 40), 4, False),
                                                            ("c4", (24, 32, 40), 1, True)])
def test_graph_replays_match_eager_steps(wl_name, shape, slabs, fused_step):
    print("[case] graph", wl_name, shape, slabs, "fused_step" if fused_step else "", flush=True)
    wl = synth.WORKLOADS[wl_name]
    c = synth.make_case(wl, shape=shape)

    def make():
        return RegistrationStep(c.F.to(DEV), c.M.to(DEV), c.A, c.t, bins=wl.bins, win=wl.win,
                                smooth_sigma=wl.smooth_sigma, lr=c.lr, slabs=slabs, fused_step=fused_step)

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
        # (the two-sweep step stores neither W nor gW: it writes gu instead)
        names = ("u", "m1", "m2", "gu", "loss", "gA", "gt", "step_dev") if fused_step else \
            ("u", "m1", "m2", "W", "gW", "loss", "gA", "gt", "step_dev")
        for name in names:
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
    assert int(a.step_dev[0]) == 4
