"""Host-side guards: the binding refuses to run without the HIP library (no
fallback of any kind), and the benchmark refuses more than one GPU."""

import os
import subprocess
import sys

import pytest

from draft_token_verification_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(ImportError, match="not built"):
        _lib._load()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
