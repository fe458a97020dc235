"""The host core (allocator, tables, rollback, codec constants, n-gram
drafter, verify planner) under AddressSanitizer and UndefinedBehaviorSanitizer:
the host-logic suites run in a child process against libsvattn_core_san.so,
which is built with the planner's invariant checks compiled in, with the
sanitizer runtimes preloaded; any report aborts the child."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "speculative_verify_attention_amd", "libsvattn_core_san.so")
SUITES = ["tests/test_core.py", "tests/test_ngram.py", "tests/test_plan.py"]


def runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_host_core_suites_under_asan_ubsan():
    if shutil.which("g++") is None:
        pytest.skip("g++ (and its sanitizer runtimes) not installed here")
    assert os.path.exists(SAN_LIB), "libsvattn_core_san.so is not built; run python -m speculative_verify_attention_amd.build"
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    assert asan and ubsan, "sanitizer runtimes not found"
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = (
        "import sys\n"
        "from speculative_verify_attention_amd import _binding\n"
        f"_binding.CORE_LIB_PATH = {SAN_LIB!r}\n"
        "import pytest\n"
        f"rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', *{SUITES!r}])\n"
        "maps = open('/proc/self/maps').read()\n"
        "print('sanitized core mapped:', 'libsvattn_core_san.so' in maps, flush=True)\n"
        "sys.exit(int(rc))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=1200)
    tail = r.stdout[-4000:]
    assert r.returncode == 0, tail
    assert "sanitized core mapped: True" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
