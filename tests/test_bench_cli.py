"""Host checks of bench.py's command line: the one-GPU rule and the workload and mode names (no GPU needed)."""
import os
import subprocess
import sys

import pytest

from dynamic_sparse_attention_decode_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=120):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = _bench("--gpus", str(n))
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")   # no JSON line


def test_help_names_every_workload_and_mode():
    r = _bench("--help")
    assert r.returncode == 0, r.stderr
    text = " ".join(r.stdout.split())
    for name in inputs.WORKLOADS:
        assert name in text, name
    for mode in ("prr_fused", "prr_1stream", "prr_2stream", "serialized", "serialized_fused"):
        assert mode in text, mode


def test_unknown_workload_is_rejected():
    r = _bench("--workload", "no_such_workload")
    assert r.returncode != 0
