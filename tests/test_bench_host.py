"""Host-side logic of bench.py (no GPU): the committed-counter lookup behind the roofline's
`traffic` field, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def write_counters(folder, digest, fetch="113068061546", write="2469923968"):
    path = os.path.join(folder, "dW_gu_large_counters.md")
    with open(path, "w") as fh:
        fh.write("# dW_gu GEMM HBM traffic, large-context workload\n\n")
        fh.write("Some prose: with a colon that is not a key.\n\n")
        fh.write(f"source_sha256: {digest}\n")
        fh.write("workload: large\n")
        if fetch is not None:
            fh.write(f"fetch_bytes_per_launch: {fetch}\n")
        fh.write(f"write_bytes_per_launch: {write}\n")
        fh.write("| table | row: with colon |\n")
    return path


def test_traffic_read_only_for_the_current_sources(tmp_path, monkeypatch):
    """Counters taken on the current library sources are reported; counters whose
    source_sha256 differs (the kernels changed since) give None, as do a missing or
    malformed summary."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.committed_traffic("large", "dW_gu") is None                # missing
    digest = bench.kernel_source_digest()
    write_counters(str(tmp_path), digest)
    assert bench.committed_traffic("large", "dW_gu") == {"fetch": 113068061546.0,
                                                          "write": 2469923968.0}
    write_counters(str(tmp_path), "0" * 64)
    assert bench.committed_traffic("large", "dW_gu") is None                # stale
    write_counters(str(tmp_path), digest, fetch=None)
    assert bench.committed_traffic("large", "dW_gu") is None                # no fetch line
    write_counters(str(tmp_path), digest, fetch="n/a")
    assert bench.committed_traffic("large", "dW_gu") is None                # not a number


def test_digest_is_a_stable_sha256():
    """The digest (a sha256 over the HIP sources and build.py) is 64 hex digits and the same
    on every call."""
    d = bench.kernel_source_digest()
    assert len(d) == 64 and all(c in "0123456789abcdef" for c in d)
    assert bench.kernel_source_digest() == d


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """bench.py measures one GPU's share: more GPUs, or a multi-rank launch, exit with
    status 2 and a message saying so, before anything touches a GPU."""
    e = dict(os.environ)
    e.update(env)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                         capture_output=True, text=True, env=e, timeout=300)
    assert res.returncode == 2
    assert "exactly one GPU" in res.stderr
    assert res.stdout == ""
