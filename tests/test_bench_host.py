"""Host logic of bench.py, on the CPU: the cold-weight rotation count, the step-time
percentiles, the digest that ties counter summaries to the kernel sources, the oracle's
thread count, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


class FakeLayer:
    def __init__(self, n_experts, per_expert):
        self.n_experts = n_experts
        self.per = per_expert

    def expert_bytes(self, e):
        return self.per


def test_rotation_copies_closed_form():
    """No weight may come back within 288 MiB of other steps' weights: copies =
    ceil(288 MiB / smallest step) + 1, the smallest step being k + 1 experts (one token,
    k routed and the shared one)."""
    iq2 = 3 * synth.matrix_bytes(synth.QTYPE_IQ2XS, 512, 2048)  # gate, up, down of one expert
    iq1 = 3 * synth.matrix_bytes(synth.QTYPE_IQ1M, 512, 2048)
    assert iq2 == 3 * 286720 and iq1 == 3 * 229376
    # field decode layer, IQ2: 11 experts = 9,461,760 B per step -> 32 steps span 288 MiB
    assert bench.rotation_copies(FakeLayer(512, iq2), 1, 10, 1) == 33
    # 8-token IQ1 layer: the bound uses one token's 11 experts = 7,569,408 B -> 40 steps
    assert bench.rotation_copies(FakeLayer(512, iq1), 8, 10, 1) == 41
    # a tiny layer hits the cap; a huge one still rotates over at least two copies
    assert bench.rotation_copies(FakeLayer(16, 1000), 1, 4, 0) == 64
    assert bench.rotation_copies(FakeLayer(512, 1 << 30), 1, 10, 1) == 2
    assert bench.LLC_REUSE_BYTES == 288 << 20


def test_percentiles_of_a_ramp():
    """101 steps of 1, 2, ..., 101 us: p10 = 11, p50 = 51, p90 = 91 (linear interpolation
    lands on samples exactly), in any input order."""
    samples = [(i + 1) * 1e-3 for i in range(101)][::-1]  # milliseconds
    p = bench.percentiles(samples)
    assert p == {"p10_us": 11.0, "p50_us": 51.0, "p90_us": 91.0, "n": 101}


def test_code_digest_ignores_comments_and_spacing():
    a = "int f(int x) {  // first\n  return x + 1; /* two\n lines */ }\n"
    b = "int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    d = bench.kernel_digest()
    assert len(d) == 64 and d == bench.kernel_digest()


def test_oracle_threads_respect_the_cpu_share(monkeypatch):
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.oracle_threads() == 1
    monkeypatch.setenv("OMP_NUM_THREADS", str(10 * n))
    assert bench.oracle_threads() == n            # never more than the cores this process may use
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.oracle_threads() == n
    info = bench.cpu_info()
    assert info["nproc"] >= 1 and info["affinity"] == n and isinstance(info["cpu_model"], str)


def test_more_than_one_gpu_is_refused():
    """The layer is data-parallel with no exchange: bench.py measures one GPU and says so
    for --gpus N > 1 (before touching any GPU)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", list(bench.WORKLOADS))
def test_workloads_are_described(name):
    banks, T, k, shared, zipf, path, desc = bench.WORKLOADS[name]
    assert path in ("decode", "prefill", "stack") and T >= 1 and 1 <= k <= 16 and desc
