"""GPU parity of exactly what bench.py times: for each of its workloads
(prefill: n = 8 bf16 [512 x 8192]; decode: n = 8 bf16 [8 x 8192]; ll64k and
ll1m: n = 8 fp32, 64 KiB and 1 MiB per rank), the step's six launches --
one-shot; rank 0's fused two-shot with slots, with LL segments and with LL128
segments; rank 0's LL and LL128 each sent and received in one launch -- on
bench.py's own rotated buffer sets, with the peers' shares published the way
bench.py publishes them, over several steps.  Every output is compared with
the oracle element by element."""
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
    import numpy

    n, dt_name, numel, _, _ = bench.WORKLOADS[workload]
    host = synth.rank_inputs(n, numel, dt_name, "normal", config=1)  # bench.py's inputs
    if dt_name == "f32":
        src = [torch.from_numpy(a).cuda() for a in host]
    else:
        src = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in host]
    want = oracle_bits(oracle.oneshot(host, dt_name))
    car.set_poll_timeout_ns(50_000_000)
    try:
        rig = bench.Rig(torch, car, numpy, n, dt_name, numel, 0, src=src)  # two sets
        assert rig.nsets == 2
        for i in range(4):
            b = rig.sets[i % 2]
            for t in b.step_outputs():
                t.zero_()
            rig.run_step(i, rig.next_steps(1))
            torch.cuda.synchronize()
            car.raise_on_status(rig.flags, f"{workload} step {i}")
            for name, t in zip(bench.KERNELS, b.step_outputs()):
                got = bits(t)
                assert np.array_equal(got, want), f"{workload} step {i} {name}: " + first_mismatch(got, want)
    finally:
        car.set_poll_timeout_ns(0)


def test_per_kernel_timing_graph_keeps_the_outputs():
    """A kernel's timing graph (launches over the rotated sets, replayed
    several times with the same step ids) leaves correct outputs."""
    import numpy

    rig = bench.Rig(torch, car, numpy, 8, "bf16", 8 * 4096, 0)
    ref = torch.empty(8 * 4096, dtype=torch.bfloat16, device="cuda")
    car.ar_oneshot(rig.sets[0].ins, ref)
    for name in bench.KERNELS:
        for b in rig.sets:
            for t in b.step_outputs():
                t.zero_()
        us, reps = rig.time_kernel(name, launches=8, replays=3)
        assert us > 0 and len(reps) == 3
        k = bench.KERNELS.index(name)
        for b in rig.sets:
            assert torch.equal(b.step_outputs()[k].view(torch.int16), ref.view(torch.int16)), name
