"""Host-side checks of bench.py that need no GPU: the one-GPU contract, the
workload table and the algorithmic byte counts the roofline divides by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_every_workload_has_kernel_sources():
    import bench
    from gemm_gguf_block_amd import synth
    names = [w for w in synth.WORKLOADS] + list(bench.BATCH_WORKLOADS)
    for w in names:
        for f in bench._sources(w):
            assert os.path.exists(os.path.join(ROOT, "gemm_gguf_block_amd", "csrc", f)), (w, f)
        assert len(bench.kernel_source_hash(w)) == 64


@pytest.mark.parametrize("fmt,n,k,bytes_", [("q4_k", 14336, 4096, 14336 * 16 * 144),
                                            ("q8_0", 4096, 4096, 4096 * 128 * 34),
                                            ("q6_k", 128256, 4096, 128256 * 16 * 210),
                                            ("q4_0", 14336, 4096, 14336 * 128 * 18),
                                            ("q5_0", 14336, 4096, 14336 * 128 * 22),
                                            ("q5_k", 14336, 4096, 14336 * 16 * 176)])
def test_weight_bytes_per_row_match_the_block_layouts(fmt, n, k, bytes_):
    """The GEMV roofline counts every weight byte once: n rows of k/block_elems
    blocks of the format's published size."""
    import gemm_gguf_block_amd as qg
    from gemm_gguf_block_amd import synth
    assert n * qg.row_bytes(fmt, k) == bytes_
    assert n * synth.row_bytes(fmt, k) == bytes_
