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
