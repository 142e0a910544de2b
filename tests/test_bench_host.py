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
    src = root / "non_gemm_voxel_amd" / "csrc" / "lncc.hip"
    maps = root / "non_gemm_voxel_amd" / "csrc" / "lncc_maps.hpp"
    src.write_text("kernel v1\n")
    maps.write_text("table v1\n")
    import hashlib
    # the LNCC call's source is the kernel file and its lane-map header, in that order
    sha = hashlib.sha256(src.read_bytes() + maps.read_bytes()).hexdigest()
    (root / "profiles" / "lncc_c4_hbm_traffic.txt").write_text(
        f"# header\ncall: lncc\nsource_sha256: {sha}\nbytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.measured_traffic("lncc", "c4") == 1234.0
    maps.write_text("table v2\n")
    assert bench.measured_traffic("lncc", "c4") is None
    maps.write_text("table v1\n")
    src.write_text("kernel v2\n")
    assert bench.measured_traffic("lncc", "c4") is None
    assert bench.measured_traffic("mi", "c4") is None


def test_committed_summaries_parse():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for f in os.listdir(os.path.join(root, "profiles")):
        if f.endswith("_hbm_traffic.txt"):
            text = open(os.path.join(root, "profiles", f)).read()
            assert "source_sha256:" in text and "bytes_per_launch:" in text, f
