"""Host-side behaviour that needs no GPU: the product path refuses to run
without its native library (no fallback), bench.py refuses more than one
GPU, and the bench's percentile helper."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_py(code, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=e, stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=300)


def test_missing_library_raises():
    # the binding's library path pointed at a missing file, as on a tree
    # where the library was never built
    r = run_py("import speculative_verify_attention_amd as s\n"
               "from speculative_verify_attention_amd import _binding\n"
               f"_binding.LIB_PATH = {os.path.join(ROOT, '_no_such_dir', 'libsvattn.so')!r}\n"
               "try:\n"
               "    s.KVCache(1, 64, 4, 1, 2, s.KV_FP32)\n"
               "except RuntimeError as e:\n"
               "    print('raised:', e)\n"
               "else:\n"
               "    print('no error')\n")
    assert "raised:" in r.stdout and "not built" in r.stdout, r.stdout


def test_library_path_is_in_tree():
    sys.path.insert(0, ROOT)
    from speculative_verify_attention_amd import _binding

    assert _binding.LIB_PATH == os.path.join(ROOT, "speculative_verify_attention_amd", "libsvattn.so")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout


def test_percentiles_nearest_rank():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.percentiles([5, 1, 2, 3, 4, 6, 7, 8, 9, 10]) == [1, 5, 9]
    assert bench.percentiles([2.5]) == [2.5, 2.5, 2.5]
