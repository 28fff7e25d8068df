"""Host-side checks of bench.py that need no GPU: its command-line contract,
the settle phase's bookkeeping, and the lookup of committed rocprofv3
figures (which must parse and stay plausible for the headline workload)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = run_bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("args", [("--steps", "0"), ("--warmup", "-1")])
def test_bad_step_counts_are_refused(args):
    r = run_bench(*args)
    assert r.returncode == 2 and "--steps" in r.stderr


class _FakeCuda:
    def __init__(self):
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1


class _FakeTorch:
    def __init__(self):
        self.cuda = _FakeCuda()


def test_settle_runs_batches_until_its_time_is_spent():
    calls = []
    torch = _FakeTorch()
    ms, n = bench.settle(lambda: calls.append(1), torch, 5.0)
    assert ms >= 5.0 and n == len(calls) and n >= 10 and n % 10 == 0
    assert torch.cuda.syncs == n // 10  # one synchronisation per batch of ten


def test_settle_off():
    torch = _FakeTorch()
    assert bench.settle(lambda: pytest.fail("no launch expected"), torch, 0.0) == (0.0, 0)
    assert torch.cuda.syncs == 0


def test_profiled_figures_parse_and_are_plausible():
    # B=4 H=16 S=4096 D=64 fp16: 2 bytes x 4 x B*H*S*D plus the fp32 lse
    algorithmic = 2 * 4 * 4 * 16 * 4096 * 64 + 4 * 4 * 16 * 4096
    t = bench.profiled_traffic("multihead_causal")
    if t is not None:  # None only when the kernel sources changed since the profile pass
        assert algorithmic <= t <= 4 * algorithmic
    busy = bench.profiled_busy("multihead_causal")
    for key, val in busy.items():
        assert key.startswith(("mfma_busy_pct_", "valu_active_pct_")) and 0.0 < val <= 100.0


def test_unknown_workload_has_no_profile():
    assert bench.profiled_traffic("no_such_workload") is None
    assert bench.profiled_busy("no_such_workload") == {}
