"""bench.py's host-side contract, on the CPU: more than one GPU is refused
with a message, the per-step byte accounting matches the method's algorithmic
bytes, and the workloads are the pages' tensor-parallel message shapes."""
from __future__ import annotations

import os
import subprocess
import sys

import bench
from custom_all_reduce_amd import accounting as acc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr and r.stdout == ""


def test_step_bytes_are_one_gpus_algorithmic_bytes():
    n, S = 8, 128 << 10
    per = bench.step_bytes(n, S)
    assert per["oneshot"] == n * S + S
    # one rank's two-shot: S read by the reduce-scatter (its segment of n inputs), S by the
    # all-gather (all n segments); S/n (its segment) + S (its output) written
    assert per["twoshot"] == 2 * S + S // n + S
    # under LL / LL128 every segment is a wire of its S/n bytes
    for p in ("ll", "ll128"):
        w = acc.wire_bytes(p, S // n)
        assert per["twoshot_" + p] == S + n * w + w + S
    W1, W2 = acc.wire_bytes("ll", S), acc.wire_bytes("ll128", S)
    assert W1 == 2 * S and W2 == 128 * -(-S // 120)
    # LL / LL128 in one launch: own message read, own wire written, n-1 peers' wires read, output written
    assert per["ll"] == S + W1 + (n - 1) * W1 + S
    assert per["ll128"] == S + W2 + (n - 1) * W2 + S
    # = pack (S + W) plus receive (n W + S) less the own wire the receive no longer reads
    assert per["ll"] == acc.total(acc.ll_pack("ll", S)) + acc.total(acc.ll_reduce("ll", n, S)) - W1
    assert set(per) == set(bench.KERNELS)


def test_workloads_are_the_pages_message_shapes():
    n, dt, numel, k, _ = bench.WORKLOADS["decode"]
    assert (n, dt, numel, k) == (8, "bf16", 8 * 8192, "oneshot")  # [8 tokens x hidden 8192]
    n, dt, numel, k, _ = bench.WORKLOADS["prefill"]
    assert (n, dt, numel, k) == (8, "bf16", 512 * 8192, "twoshot")
    for w, bytes_per_rank in (("ll64k", 64 << 10), ("ll1m", 1 << 20)):
        n, dt, numel, _, _ = bench.WORKLOADS[w]
        assert dt == "f32" and numel * 4 == bytes_per_rank


def test_default_workload_is_the_two_shot_prefill_message():
    """With no flags bench.py measures the n = 8, bf16 [512 x 8192] message
    (8 MiB per rank), and the roofline is the two-shot's."""
    import inspect

    src = inspect.getsource(bench.main)
    assert 'ap.add_argument("--workload", default="prefill"' in src
    assert bench.WORKLOADS["prefill"][3] == "twoshot"
    assert bench.KERNEL_LAUNCHES >= 200 and bench.KERNEL_REPLAYS >= 3
    assert bench.CURVE_SIZES == [128 << 10, 1 << 20, 8 << 20, 64 << 20]


def test_oracle_step_bytes_are_what_the_oracle_moves():
    from oracle import model

    n, S = 8, 1 << 20
    want = (n + 1) * S + 2 * n * S + (n + 1) * S
    for p in ("ll", "ll128"):
        W = model.ll_wire_bytes(p, S)
        want += S + W + n * W + S
    assert bench.oracle_step_bytes(n, S) == want


def test_store_path_accounting():
    S, n = 1 << 20, 8
    assert acc.reduce_bcast(n, S, 1) == (S, S)
    assert acc.reduce_bcast(n, S, n) == (n * S, n * S)
    assert acc.push(S, n) == (S, n * S)
    assert acc.push(S, 1) == (S, S)


def test_kernel_hash_ignores_comments_but_not_code():
    """The hash that keeps a kernel's HBM counters valid changes with its
    code, not with its comments."""
    src = 'int f(int a) {  // add one\n    /* block\n comment */ return a + 1;\n}\n'
    assert bench.code_text(src) == bench.code_text(src.replace("add one", "increment"))
    assert bench.code_text(src) == bench.code_text(src.replace("    ", "\t"))
    assert bench.code_text(src) != bench.code_text(src.replace("a + 1", "a + 2"))
    assert "//" not in bench.code_text(src) and "/*" not in bench.code_text(src)


def test_roofline_kernel_is_also_timed_per_call_and_in_batches():
    """The configuration's kernel is also timed per call between events and
    in batches, beside the graph-replay median; the rocprofv3 summary is
    named for the kernel-only durations."""
    import inspect

    src = inspect.getsource(bench.main)
    assert "other_timings = rig.event_timings(config_kernel)" in src
    assert '"other_timings": dict(other_timings or {}' in src
    ev = inspect.getsource(bench.Rig.event_timings)
    assert "warm=20, calls=200, batch=20" in ev
    assert "statistics.median(per)" in ev and "statistics.median(bat)" in ev


def test_nvlink_model_crossover_beside_the_measured_one():
    """The sweep prints the pages' NVLink model crossover beside the measured
    one; bench's formula agrees with the oracle's model (pinned against the
    pages' ~257 KB at n = 8)."""
    from oracle import model

    for n in (8, 16):
        assert abs(bench.nvlink_model_crossover(n) - model.crossover_oneshot_twoshot(n)) < 1e-6 * model.crossover_oneshot_twoshot(n)
    assert round(bench.nvlink_model_crossover(8)) == 257143
    assert round(bench.nvlink_model_crossover(16)) == 102857
