"""The CPU oracle built with gcc's AddressSanitizer and
UndefinedBehaviorSanitizer (host code only) and run over every entry point
on small shapes, including corrupted headers and invalid widths
(oracle/sanitize_check.c). Any out-of-bounds access, leak, signed overflow
or other undefined behaviour ends the run with a nonzero status."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import codebook

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_check")
    src = os.path.join(ROOT, "oracle", "sanitize_check.c")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"), src, "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    levels, thr = codebook.codec_table()
    args = [float(np.float32(x)).hex() for x in list(levels) + list(thr)]
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe] + args, capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "oracle sanitizer run ok" in res.stdout
