"""GPU parity of exactly what bench.py times: for each of its workloads
(decode: n = 8 bf16 [8 x 8192]; prefill: n = 8 bf16 [512 x 8192]; ll64k and
ll1m: n = 8 fp32, 64 KiB and 1 MiB per rank), the step's four launches --
one-shot, rank 0's fused two-shot, and rank 0's LL and LL128 each sent and
received in one launch -- on bench.py's own buffer sets, with the peers'
shares published the way bench.py publishes them, over several steps.
Every output is compared with the oracle element by element."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from devtensors import bits, first_mismatch, oracle_bits

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")


@pytest.mark.parametrize("workload", sorted(bench.WORKLOADS))
def test_bench_step_matches_the_oracle(workload):
    n, dt_name, numel, _ = bench.WORKLOADS[workload]
    dt = torch.float32 if dt_name == "f32" else torch.bfloat16
    host = synth.rank_inputs(n, numel, dt_name, "normal", config=1)  # bench.py's inputs
    if dt_name == "f32":
        src = [torch.from_numpy(a).cuda() for a in host]
    else:
        src = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in host]
    want = oracle_bits(oracle.oneshot(host, dt_name))
    car.set_poll_timeout_ns(50_000_000)
    try:
        sets = [bench.BufferSet(torch, car, src, n, dt, numel) for _ in range(2)]
        flags = car.new_flags(n)
        calls = [bench.step_calls(car, b, flags) for b in sets]
        for b in sets:
            bench.publish_peers(car, b, flags)
        for step in range(1, 5):
            b = sets[step % 2]
            for t in (b.out, b.outs[bench.ME], b.out_ll, b.out_128):
                t.zero_()
            bench.run_step(calls[step % 2], step)
            torch.cuda.synchronize()
            car.raise_on_status(flags, f"{workload} step {step}")
            for name, t in (("one-shot", b.out), ("two-shot", b.outs[bench.ME]), ("LL", b.out_ll),
                            ("LL128", b.out_128)):
                got = bits(t)
                assert np.array_equal(got, want), f"{workload} step {step} {name}: " + first_mismatch(got, want)
    finally:
        car.set_poll_timeout_ns(0)
