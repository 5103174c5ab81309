"""Host code under the sanitizers (CPU only, g++ / gcc builds, no HIP).

- The CPU oracle (oracle/oracle.c, OpenMP loops) built with AddressSanitizer
  and UndefinedBehaviorSanitizer: the oracle's own test files run against it
  in a child process (the runtime preloaded, any report aborts the run).
- The decode-host cache core (csrc/host_tier_core.h: cache state, fetch on a
  pool of worker threads, the dispatcher thread's job queue; the library's
  oasis_host_tier_* entry points are this code plus HIP calls) driven by
  tests/sanitize/host_tier_san.cpp under ASan + UBSan and, separately, under
  ThreadSanitizer: random histories on 1-5 workers, directly and through the
  dispatcher, must give the one-thread result with no sanitizer report.
The cache follows paperpeel v2 §3.2.1 (ii), §3.2.2 and §3.2.3 (union fetch
of whole blocks, union block map, LRU with a protected working set).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_kv_block_quest_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_tier_san.cpp")
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
ORACLE_TESTS = ["test_oracle_attn.py", "test_oracle_summaries_scores.py",
                "test_oracle_topk_plan.py", "test_oracle_host_tier.py"]


def _build(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        if "cannot find" in res.stderr or "sanitize" in res.stderr and "unrecognized" in res.stderr:
            pytest.skip(f"sanitizer runtime not available: {res.stderr[-300:]}")
        raise AssertionError(f"build failed: {' '.join(cmd)}\n{res.stderr}")


def _run(cmd, env=None, timeout=300):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert res.returncode == 0, f"{' '.join(cmd)} failed ({res.returncode}):\n{res.stdout[-3000:]}\n{res.stderr[-6000:]}"
    return res


@pytest.mark.parametrize("flags,opts", [
    (["-fsanitize=address,undefined", "-fno-omit-frame-pointer"],
     {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}),
    (["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1"}),
], ids=["asan_ubsan", "tsan"])
def test_host_tier_core(tmp_path, flags, opts):
    exe = str(tmp_path / "host_tier_san")
    _build(["g++", "-std=c++17", "-O1", "-g", "-fno-sanitize-recover=all", *flags, "-pthread",
            f"-I{CSRC}", DRIVER, "-o", exe])
    env = dict(os.environ, **opts)
    res = _run([exe], env=env)
    assert res.stdout.strip().endswith("ok")
    assert "failed" in res.stdout  # the small-budget case ran and failed as expected


def test_oracle_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboasis_oracle_san.so")
    _build(["gcc", "-std=c11", "-O1", "-g", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
            "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
            "-o", lib, ORACLE_C, "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan.so not found")
    env = dict(os.environ, LD_PRELOAD=asan, OASIS_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",  # the interpreter's own leaks
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", t) for t in ORACLE_TESTS]
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
            "import oracle; oracle._load()\n"
            "maps = open('/proc/self/maps').read()\n"
            "assert %r in maps, 'the sanitized oracle is not the one loaded'\n"
            "import pytest\n"
            "sys.exit(pytest.main(%r + ['-q', '-p', 'no:cacheprovider']))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, tests))
    res = _run([sys.executable, "-c", code], env=env, timeout=600)
    assert " passed" in res.stdout and " failed" not in res.stdout
