"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message (one GPU's share is what is measured; sharding is a
design note), the algorithmic byte counts per parameter, and the gradient-release
buckets of the timing loop."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_parameter():
    sys.path.insert(0, ROOT)
    import bench
    from compressed_adamw_state_amd import workloads as W
    w = W.WORKLOADS["llama31_8b"]
    assert bench.algorithmic_bytes(w) == 98_370_700_288          # 12.25 B/param
    assert bench.algorithmic_bytes(W.WORKLOADS["llama31_8b_lion"]) == 10.125 * w.numel
    assert bench.algorithmic_bytes(W.WORKLOADS["llama31_8b_adamw_fp32"]) == 28 * w.numel


def test_release_buckets_cover_the_list_in_backward_order():
    sys.path.insert(0, ROOT)
    import bench
    from compressed_adamw_state_amd import workloads as W
    assert bench.release_buckets([10, 100, 5, 7], 0) == [(3, 1), (2, 1), (1, 1), (0, 1)]
    assert bench.release_buckets([10, 100, 5, 7], 30) == [(1, 3), (0, 1)]
    assert bench.release_buckets([10, 100, 5, 7], 10 ** 9) == [(0, 4)]
    assert bench.release_buckets([], 64) == []
    sizes = [t.numel for t in W.WORKLOADS["llama2_13b"].tensors]
    b = bench.release_buckets(sizes, 64 << 20)
    assert [i for f, c in reversed(b) for i in range(f, f + c)] == list(range(len(sizes)))
    assert all(2 * sum(sizes[f:f + c]) >= 64 << 20 for f, c in b[:-1])
