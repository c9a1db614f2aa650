"""bench.py's command-line contract that needs no GPU: more than one GPU is refused with a
message and a non-zero status before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_full_and_sampled_on_host():
    """The oracle legs of the benchmark run on host tensors: a full run reports every row, a
    sampled run reports its sample and the extrapolated whole-workload time."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    w = W.WORKLOADS[1]
    q, k, v = W.make_inputs(w, "cpu")
    rec = bench.cpu_baseline(w, q, k, v, 0.0, full=True)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["cores"] >= 1
    assert rec["value"] > 0 and "all 256 query rows" in rec["sample"]
    assert "extrapolated_full_workload_s" not in rec
    small = W.Workload(3, "bf16 causal test shape", 1, 2, 600, 600, 64, W.torch.bfloat16, True)
    q, k, v = W.make_inputs(small, "cpu")
    rec = bench.cpu_baseline(small, q, k, v, 0.05)
    assert rec["value"] > 0 and "of 1200 query rows" in rec["sample"]
    assert rec["extrapolated_full_workload_s"] >= rec["seconds"] * 0.99


def test_visible_keys_counts_the_mask():
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    w = W.Workload(3, "t", 1, 2, 5, 8, 64, W.torch.bfloat16, True)
    # bottom-right causal: query i sees keys 0 .. i + 3
    assert list(bench.visible_keys(w, [0, 1, 4, 5, 9])) == [4, 5, 8, 4, 8]
    w2 = W.Workload(2, "t", 1, 1, 5, 8, 64, W.torch.bfloat16, False)
    assert list(bench.visible_keys(w2, [0, 4])) == [8, 8]
