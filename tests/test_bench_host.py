"""Host-side checks of bench.py (no GPU): the multi-GPU refusal and the
counter-measured traffic figures, which are valid only for the kernel sources
they were taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("kernel", ["pass1_qres", "pass2_accum", "bwd_dh", "ta_attend"])
def test_traffic_figures_match_current_sources(kernel):
    """Each stored HBM-traffic figure carries the sha256 of the sources it
    was measured on; a kernel edited since reports null traffic, so the
    figure must be measured again (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import bench
    nbytes, digest, names = bench.TRAFFIC[kernel]
    for n in names:
        assert os.path.exists(os.path.join(ROOT, "prototype_attention_compression_amd", "csrc", n)), n
    if bench.sources_digest(names) != digest:
        # the guard: a stale figure is never reported
        assert bench.measured_traffic(kernel) is None
        pytest.skip(f"{kernel}: sources changed since the counters were taken; traffic reports null "
                    "until FETCH_SIZE / WRITE_SIZE are measured again")
    assert bench.measured_traffic(kernel) == nbytes


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
