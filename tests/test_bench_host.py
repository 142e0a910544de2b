"""Host-side pieces of bench.py: the byte model covers every call the step
can time, and a counter summary is used only for the kernel source it was
taken on (no GPU)."""
import os

import bench


def test_call_bytes_cover_every_call():
    for name in bench.CALL_SOURCE:
        assert bench.call_bytes(name, False) > 0
    assert bench.call_bytes("lncc", True) == bench.call_bytes("lncc", False) + 4
    assert bench.call_bytes("warp_bwd_adam", False) < bench.call_bytes("warp_bwd", False) + bench.call_bytes(
        "adam", False)


def test_traffic_summary_tracks_source(tmp_path, monkeypatch):
    root = tmp_path
    (root / "profiles").mkdir()
    (root / "non_gemm_voxel_amd" / "csrc").mkdir(parents=True)
    csrc = root / "non_gemm_voxel_amd" / "csrc"
    names = bench.CALL_SOURCE["lncc"].split()
    assert names[:2] == ["lncc.hip", "lncc_maps.hpp"]
    for n in names:
        (csrc / n).write_text(f"{n} v1\n")
    maps = csrc / "lncc_maps.hpp"
    import hashlib
    # the LNCC call's source: the kernel file and the headers it includes, in that order
    sha = hashlib.sha256(b"".join((csrc / n).read_bytes() for n in names)).hexdigest()
    (root / "profiles" / "lncc_c4_hbm_traffic.txt").write_text(
        f"# header\ncall: lncc\nsource_sha256: {sha}\nbytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.measured_traffic("lncc", "c4") == 1234.0
    maps.write_text("table v2\n")
    assert bench.measured_traffic("lncc", "c4") is None
    maps.write_text("lncc_maps.hpp v1\n")
    assert bench.measured_traffic("lncc", "c4") == 1234.0
    (csrc / "lncc.hip").write_text("kernel v2\n")
    assert bench.measured_traffic("lncc", "c4") is None
    assert bench.measured_traffic("mi", "c4") is None


def test_committed_summaries_parse():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for f in os.listdir(os.path.join(root, "profiles")):
        if f.endswith("_hbm_traffic.txt"):
            text = open(os.path.join(root, "profiles", f)).read()
            assert "source_sha256:" in text and "bytes_per_launch:" in text, f


class _St:
    def __init__(self, slabs, win):
        self.slabs = [(0, 1)] * slabs
        self.zrange = object() if slabs > 1 else None
        self.win = win


class _Timer:
    def __init__(self, st, active, acc):
        self.st, self.active, self.acc = st, active, acc


def test_roofline_is_per_launch_of_the_dominant_kernel():
    """A slab sequence launches its kernel once per slab: the roofline's launch
    is one of those (the call's time, voxels and counter bytes over the slab
    count, the same rate), named as rocprofv3 names it; a one-launch call
    keeps the whole call."""
    active = ["warp_fwd", "mi_fwd", "lncc", "warp_bwd_adam_slab_mi"]
    acc = {"lncc": False, "warp_bwd_adam_slab_mi": True}
    per_call = {"warp_fwd": 30.0, "mi_fwd": 9.0, "lncc": 56.0, "warp_bwd_adam_slab_mi": 59.2}
    nvox = 8 * 10 ** 6
    out = bench.summarise(_Timer(_St(8, 9), active, acc), 0.1542 * 10, per_call, 10, nvox, "nowhere")
    r = out["roofline"]
    assert r["kernel"] == "warp_bwd_adam_slab_mi" and r["kernel_name"] == "warp_bwd_kernel<true, true, true>"
    assert r["launches_per_call"] == 8
    assert abs(r["ms_per_launch"] - 59.2 / 8) < 1e-12 and r["voxels_per_launch"] == nvox / 8
    rate = 88 * nvox / (59.2e-3) / 1e9
    assert abs(r["achieved"] - rate) < 1e-9 * rate and abs(r["frac"] - rate / 8000.0) < 1e-12
    per_call["lncc"] = 60.0
    r = bench.summarise(_Timer(_St(8, 9), active, acc), 1.6, per_call, 10, nvox, "nowhere")["roofline"]
    assert r["kernel"] == "lncc" and r["kernel_name"] == "lncc_kernel<4, false>"
    assert r["launches_per_call"] == 1 and r["ms_per_launch"] == 60.0 and r["voxels_per_launch"] == nvox
    assert "fp64" in r


def test_more_than_one_gpu_is_refused():
    """One GPU only: any other --gpus exits with a message before touching a
    device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU only" in r.stderr and not r.stdout.strip()
