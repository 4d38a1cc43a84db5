"""bench.py reports counter-measured HBM traffic only for the kernel source it was measured on."""
import hashlib
import os

import bench


def _write(tmp_path, digest, value=123456):
    (tmp_path / "s.md").write_text(
        "command: rocprofv3 --pmc FETCH_SIZE ...\n"
        f"source sequence_long_context_amd/csrc/api.hip sha256 {digest}\n"
        f"hbm_bytes_per_launch s32k {value}\n")


def test_matching_source_gives_bytes(tmp_path):
    src = os.path.join(bench.ROOT, "sequence_long_context_amd/csrc/api.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    _write(tmp_path, digest)
    got = bench.measured_traffic("s.md", ["sequence_long_context_amd/csrc/api.hip"], str(tmp_path))
    assert got == {"s32k": 123456}


def test_changed_source_gives_none(tmp_path):
    _write(tmp_path, "0" * 64)
    assert bench.measured_traffic("s.md", ["sequence_long_context_amd/csrc/api.hip"],
                                  str(tmp_path)) == {}


def test_source_not_listed_gives_none(tmp_path):
    src = os.path.join(bench.ROOT, "sequence_long_context_amd/csrc/api.hip")
    _write(tmp_path, hashlib.sha256(open(src, "rb").read()).hexdigest())
    assert bench.measured_traffic("s.md", ["sequence_long_context_amd/csrc/api.hip",
                                           "sequence_long_context_amd/csrc/layout.hip"],
                                  str(tmp_path)) == {}
    assert bench.measured_traffic("missing.md", [], str(tmp_path)) == {}
