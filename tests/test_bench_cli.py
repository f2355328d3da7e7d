"""bench.py's command line on the CPU: requests it refuses before touching a GPU,
and the algorithmic byte count its roofline rests on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_reason():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_bad_step_counts_are_refused():
    assert run_bench("--steps", "0").returncode != 0
    assert run_bench("--warmup", "-1").returncode != 0


def test_unknown_weight_layout_is_refused():
    r = run_bench("--weight-layout", "columns")
    assert r.returncode != 0
    assert "weight-layout" in r.stderr


def test_step_bytes_counts_weights_once_and_each_kv_entry_once():
    """The 8B-shaped stack at batch 1 with 512 cached positions: 218.1 M
    parameters per layer in bfloat16 plus two float32 norm gains, 32 layers;
    the 512 cached K/V entries read and the new one written, at 2 x 8 x 128 x 2
    bytes per position per layer (14.027 GB per step in all)."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    w = synth.get_workload("c2_8b_b1")
    by = bench.step_bytes(w, [512])
    H, F, L = 4096, 14336, 32
    params = (6144 * H + H * 4096 + 3 * H * F)
    assert by["weights"] == L * (params * 2 + 2 * H * 4)
    kv_row = 2 * 8 * 128 * 2
    assert by["kv_read"] == 512 * kv_row * L
    assert by["kv_write"] == 1 * kv_row * L
    assert by["total"] == by["weights"] + by["kv_read"] + by["kv_write"] == 14_026_932_224
