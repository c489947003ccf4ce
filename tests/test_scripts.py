"""The top-level scripts compile, and bench.py refuses more than one GPU."""
import os
import py_compile
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("path", ["bench.py", "__graft_entry__.py", "tests/golden/make_golden.py",
                                  "tiled_online_softmax_04_amd/build.py"])
def test_compiles(path):
    py_compile.compile(os.path.join(ROOT, path), doraise=True)


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
