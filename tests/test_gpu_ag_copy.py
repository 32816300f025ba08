"""GPU parity of the copy-engine all-gather (ar_twoshot_ag_copy) against the
oracle: after a reduce-scatter, a one-workgroup slot wait and n
hipMemcpyAsync copies per output give exactly the one-shot result; with auto
step ids, in a graph, for one rank's share, and with a missing peer (a
reported timeout)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")


class Ranks:
    def __init__(self, n, numel, dt, config):
        self.n = n
        self.host = synth.rank_inputs(n, numel, dt, "normal", config=config)
        self.want = oracle_bits(oracle.oneshot(self.host, dt))
        self.ins = [to_dev(a) for a in self.host]
        tdt = self.ins[0].dtype
        self.segs = [torch.empty(numel // n, dtype=tdt, device="cuda") for _ in range(n)]
        self.outs = [torch.zeros(numel, dtype=tdt, device="cuda") for _ in range(n)]
        self.flags = car.new_flags(n)
        torch.cuda.synchronize()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n", [2, 5, 8, 16])
def test_all_ranks_after_reduce_scatter(n, dt):
    per_vec = 8 if dt == "bf16" else 4
    rk = Ranks(n, n * per_vec * 777, dt, config=700 + n)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, 1)
    car.ar_twoshot_ag_copy(rk.segs, rk.outs, rk.flags, 1)
    torch.cuda.synchronize()
    car.raise_on_status(rk.flags)
    for r in range(n):
        assert np.array_equal(bits(rk.outs[r]), rk.want), f"rank {r}"


def test_one_rank_share():
    n = 8
    rk = Ranks(n, 8 * 8192, "bf16", config=710)
    for r in range(1, n):
        car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, 1 << 31, r0=r, r1=r + 1)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, 5, r0=0, r1=1)
    car.ar_twoshot_ag_copy(rk.segs, [rk.outs[0]] + [None] * (n - 1), rk.flags, 5, r0=0, r1=1)
    torch.cuda.synchronize()
    car.raise_on_status(rk.flags)
    assert np.array_equal(bits(rk.outs[0]), rk.want)
    for r in range(1, n):
        assert not bits(rk.outs[r]).any()  # outputs outside [r0, r1) untouched


def test_auto_steps_in_a_graph():
    n, numel = 4, 4 * 8 * 4096
    data = [synth.rank_inputs(n, numel, "bf16", "normal", config=720 + k) for k in range(2)]
    wants = [oracle_bits(oracle.oneshot(h, "bf16")) for h in data]
    rk = Ranks(n, numel, "bf16", config=720)

    def step():
        car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, 0)
        car.ar_twoshot_ag_copy(rk.segs, rk.outs, rk.flags, 0)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(6):
        for d, a in zip(rk.ins, data[rep % 2]):
            d.copy_(to_dev(a))
        for o in rk.outs:
            o.zero_()
        torch.cuda.synchronize()
        if rep == 3:
            step()  # eager, same flag region
        else:
            g.replay()
        torch.cuda.synchronize()
        car.raise_on_status(rk.flags, f"step {rep}")
        for r in range(n):
            assert np.array_equal(bits(rk.outs[r]), wants[rep % 2]), f"step {rep} rank {r}"


def test_missing_peer_is_a_reported_timeout():
    n = 8
    rk = Ranks(n, 8 * 8192, "bf16", config=730)
    for r in range(n):
        if r != 6:
            car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, 3, r0=r, r1=r + 1)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(50_000_000)
    try:
        car.ar_twoshot_ag_copy(rk.segs, rk.outs, rk.flags, 3)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, phase, rank = car.decode_status(car.read_status(rk.flags)[0])
    assert (code, phase, rank) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG, 6)  # rank 6's slots are missing
    with pytest.raises(car.ArError):
        car.raise_on_status(rk.flags)


def test_synchronous_errors():
    n = 4
    rk = Ranks(n, 4 * 8 * 100, "bf16", config=740)
    # an output too small for the all-gather is refused before anything runs
    with pytest.raises(ValueError):
        car.ar_twoshot_ag_copy(rk.segs, [rk.segs[0]] + rk.outs[1:], rk.flags, 1)
    # an output of the right size that overlaps a segment
    big = torch.zeros(rk.outs[0].numel(), dtype=rk.outs[0].dtype, device="cuda")
    segs = [big[:rk.segs[0].numel()]] + rk.segs[1:]
    with pytest.raises(car.ArError) as e:
        car.ar_twoshot_ag_copy(segs, [big] + rk.outs[1:], rk.flags, 1)
    assert e.value.code == car.AR_ERR_ALIAS
    with pytest.raises(car.ArError) as e:
        car.ar_twoshot_ag_copy(rk.segs, rk.outs, rk.flags, 1, r0=3, r1=3)
    assert e.value.code == car.AR_ERR_ARG
