"""The host table builders under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/table_fuzz_driver.cpp drives asv_seg_table_build and
asv_block_table_build (host code, no HIP calls) over random valid rounds
(windows of 1-40 rows up to 2,048 rows, keys up to 131,072, 0-3 conv and
attention layers: the size query, the exact blob, a blob one byte short)
and malformed ones (no rows, keys below the rows, a capacity that is not a
multiple of 32, keys past 131,072, more than 2,048 rows, aliasing caches),
each with its expected return code. The builder is compiled here with g++
and the sanitizers; any report fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is needed to build the sanitized driver")
def test_table_builders_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "table_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "table_fuzz_driver.cpp"),
           os.path.join(ROOT, "attention_stream_verify_amd", "csrc", "table.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "400"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout, r.stdout[-4000:]
    assert "400 iterations, 0 failures" in r.stdout
