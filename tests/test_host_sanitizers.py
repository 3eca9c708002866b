"""The host prefix-tree manager under AddressSanitizer and UBSan.

tests/host/manager_fuzz.cpp drives random insert / append / batched append /
remove sequences and plan builds (chunk sizes 2..128, tiny vocabularies so
prefixes collide and chunks split everywhere); built with g++ and both
sanitizers, any invalid memory access or undefined behaviour aborts the run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "decode_attention_prefix_tree_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_manager_random_scripts_under_sanitizers(tmp_path):
    exe = str(tmp_path / "manager_fuzz")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", f"-I{CSRC}", os.path.join(HERE, "host", "manager_fuzz.cpp"),
         os.path.join(CSRC, "manager.cpp"), "-o", exe],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe, "120"], capture_output=True, text=True, timeout=300,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1"})
    assert run.returncode == 0, (run.stdout[-1000:], run.stderr[-3000:])
    assert run.stdout.startswith("ok:")
