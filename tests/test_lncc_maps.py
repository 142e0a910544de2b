"""The LNCC kernel's stage-BC and stage-D thread -> task maps (lncc_maps.hpp,
radius 4): every task on exactly one thread, and no two lanes that gfx950
serves in one LDS pass touch the same banks (16-byte reads in the lane groups
GA/GB of a half-wave, 8-byte writes in 16 consecutive lanes)."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "non_gemm_voxel_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_lncc_maps", os.path.join(CSRC, "gen_lncc_maps.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_lane_groups_partition_a_half_wave():
    g = _gen()
    assert sorted(g.GA + g.GB) == list(range(32))
    assert sorted(l for c in g.CELLS for l in c) == list(range(32))
    assert all(len(c) == 8 for c in g.CELLS)


def test_bc_map_is_conflict_free_permutation():
    g = _gen()
    bc, _ = g.read(os.path.join(CSRC, "lncc_maps.hpp"))
    tasks, u, v = g.bc_tasks()
    index = {(bc_, bs): t for t, (bc_, bs) in enumerate(tasks)}
    lanes = [None if e == 0xFFFF else index[(e & 0xFF, e >> 8)] for e in bc]
    g.check(lanes, u, v, len(tasks))


def test_d_map_is_conflict_free_permutation_on_five_waves():
    g = _gen()
    _, d = g.read(os.path.join(CSRC, "lncc_maps.hpp"))
    tasks, u, v = g.d_tasks()
    index = {t_: t for t, t_ in enumerate(tasks)}
    lanes = [None if e == 0xFFFF else index[(e & 0xFF, (e >> 8) & 0xF, e >> 12)] for e in d]
    g.check(lanes, u, v, len(tasks))
    assert all(e == 0xFFFF for e in d[320:])


def test_check_rejects_a_conflict():
    g = _gen()
    tasks, u, v = g.bc_tasks()
    # plain order: the 16-lane read groups that wrap from one row pair to the next collide
    lanes = [t if t < len(tasks) else None for t in range(g.NTHREADS)]
    try:
        g.check(lanes, u, v, len(tasks))
    except AssertionError:
        return
    raise AssertionError("plain order passed the conflict check")
