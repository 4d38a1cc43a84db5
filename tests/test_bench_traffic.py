"""bench.py: counter-measured HBM traffic only for the kernel source it was measured on; the
algorithmic flop and exponential counts; one GPU only."""
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


def test_algorithmic_flops_and_exps():
    """4*D flops per visible (query, key) pair: the 32k rank's causal attention (4 heads) is
    1.0995e12 flop, the 4k rank's 1.718e10; one exponential per visible pair."""
    assert bench.attention_flops(32768, 4, 128, True) == 4 * 128 * 4 * 32768 * 32769 // 2
    assert abs(bench.attention_flops(32768, 4, 128, True) - 1.0995e12) < 1e8
    assert abs(bench.attention_flops(4096, 4, 128, True) - 1.718e10) < 1e7
    assert bench.attention_flops(256, 1, 32, False) == 4 * 32 * 256 * 256
    # sampled rows: causal row i sees i + 1 keys
    assert bench.attention_flops(8, 1, 2, True, rows=[0, 7]) == 4 * 2 * (1 + 8)
    assert bench.PEAK_EXP_PER_S == 256 * 4 * 8 * 2.4e9


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
