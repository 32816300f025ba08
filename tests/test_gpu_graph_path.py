"""The graph path and the staging path.

Graph path: a two-shot call captured once into a HIP graph with step 0
(auto), so every replay takes its step id from the per-rank epochs in the
flag region and advances them -- no reset between replays.  Every replay gets
new inputs (eager work between replays) and must match the oracle; a replay
where one rank's reduce-scatter is missing must end in a reported timeout
(stale segments never pass), and a reset recovers.

Staging path: the caller's tensors are copied into registered buffers
(ar_push with one destination) and the reduction writes the result back into
the caller's tensors in place."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

def epochs(flags, n):
    """Rank r's epoch, checked equal in every wavefront's copy (two 4-wave
    workgroups per CU take part in an auto launch; the other copies stay 0)."""
    grid = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    base = 32 + n * car.AR_SLOTS_PER_RANK
    # group w (n words) belongs to wavefront w; word r of it to rank r
    w = flags[base:base + n * car.AR_EPOCH_COPIES].cpu().numpy().astype(np.int64).reshape(-1, n)
    assert (w[grid:, :] == 0).all()
    for r in range(n):
        assert (w[:grid, r] == w[0, r]).all(), f"rank {r}: epoch copies differ"
    return w[0, :].tolist()


class Set:
    def __init__(self, n, numel, dt, configs):
        self.data = [synth.rank_inputs(n, numel, dt, "normal", config=c) for c in configs]
        self.want = [oracle_bits(oracle.oneshot(h, dt)) for h in self.data]
        self.ins = [to_dev(a) for a in self.data[0]]
        tdt = self.ins[0].dtype
        self.segs = [torch.empty(numel // n, dtype=tdt, device="cuda") for _ in range(n)]
        self.outs = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
        self.flags = car.new_flags(n)
        torch.cuda.synchronize()

    def load(self, k):
        for d, a in zip(self.ins, self.data[k]):
            d.copy_(to_dev(a))
        for o in self.outs:
            o.zero_()
        torch.cuda.synchronize()


def capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("n,numel,dt", [(8, 8 * 8192, "bf16"), (5, 5 * 4 * 1000, "f32"), (16, 16 * 8 * 512, "bf16")])
def test_fused_full_emulation_replays_without_reset(n, numel, dt):
    s = Set(n, numel, dt, [600 + k for k in range(3)])
    g = capture(lambda: car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, outs=s.outs))
    for rep in range(9):
        s.load(rep % 3)
        g.replay()
        torch.cuda.synchronize()
        car.raise_on_status(s.flags, f"replay {rep}")
        assert epochs(s.flags, n) == [rep + 1] * n
        for r in range(n):
            assert np.array_equal(bits(s.outs[r]), s.want[rep % 3]), f"replay {rep} rank {r}"


@pytest.mark.parametrize("numel", [8 * 8192, 8 * 8 * 64 * 1024])
def test_one_rank_shares_in_a_graph(numel):
    """Peers' reduce-scatters and rank 0's fused share as separate launches,
    all with auto step ids, in one graph; eager auto calls in between.  At
    decode size (128 KiB per rank) and at 8 MiB per rank."""
    n, dt = 8, "bf16"
    s = Set(n, numel, dt, [610, 611])
    out0 = [s.outs[0]] + [None] * (n - 1)

    def one_step():
        for r in range(1, n):
            car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=r, r1=r + 1)
        car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=0, r1=1, outs=out0)

    g = capture(one_step)
    for rep in range(6):
        s.load(rep % 2)
        if rep % 3 == 2:
            one_step()  # the same calls, eager
        else:
            g.replay()
        torch.cuda.synchronize()
        car.raise_on_status(s.flags, f"step {rep}")
        assert epochs(s.flags, n) == [rep + 1] * n
        assert np.array_equal(bits(s.outs[0]), s.want[rep % 2]), f"step {rep}"


@pytest.mark.parametrize("proto", ["slots", "ll", "ll128"])
def test_auto_steps_with_changing_sizes_on_one_flag_region(proto):
    """Auto step ids on one flag region while the message size changes from
    call to call (every rank's two-shot in one launch): three sizes whose
    tilings differ (64-vector tiles at the two smaller sizes, 128-vector tiles
    at 8 MiB per rank), visited in an order where each follows a different
    one.  The fixed grid keeps every wavefront's epoch copies in step whatever
    the size, so each call must match the oracle, and the epochs must count
    the calls."""
    n, dt = 4, "bf16"
    numels = [4 * 8 * 37, 4 * 8 * 5000, 4 * (4 << 20)]
    data = [synth.rank_inputs(n, k, dt, "normal", config=660 + i) for i, k in enumerate(numels)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in data]
    flags = car.new_flags(n)
    bufs = []
    for k, h in zip(numels, data):
        ins = [to_dev(a) for a in h]
        tdt = ins[0].dtype
        m = k // n
        if proto == "slots":
            segs = [torch.empty(m, dtype=tdt, device="cuda") for _ in range(n)]
        else:
            W = car.ll_wire_bytes(proto, m * 2)
            segs = [torch.zeros(W, dtype=torch.uint8, device="cuda") for _ in range(n)]
        outs = [torch.empty(k, dtype=tdt, device="cuda") for _ in range(n)]
        bufs.append((ins, segs, outs))
    fn = {"slots": car.ar_twoshot_rs, "ll": car.ar_twoshot_ll, "ll128": car.ar_twoshot_ll128}[proto]
    torch.cuda.synchronize()
    order = [0, 2, 1, 2, 0, 1, 1, 2]
    for call, i in enumerate(order):
        ins, segs, outs = bufs[i]
        for o in outs:
            o.fill_(7)
        fn(ins, segs, flags, 0, outs=outs)
        torch.cuda.synchronize()
        car.raise_on_status(flags, f"call {call} (size {numels[i]})")
        for r in range(n):
            assert np.array_equal(bits(outs[r]), wants[i]), f"call {call} size {numels[i]} rank {r}"
    assert epochs(flags, n) == [len(order)] * n


def test_split_rs_then_ag_with_auto_steps():
    n, numel, dt = 4, 4 * 8 * 700, "bf16"
    s = Set(n, numel, dt, [620, 621])

    def one_step():
        car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0)
        car.ar_twoshot_ag(s.segs, s.outs, s.flags, 0)

    g = capture(one_step)
    for rep in range(4):
        s.load(rep % 2)
        g.replay()
        torch.cuda.synchronize()
        car.raise_on_status(s.flags, f"step {rep}")
        assert epochs(s.flags, n) == [rep + 1] * n  # the all-gather does not advance
        for r in range(n):
            assert np.array_equal(bits(s.outs[r]), s.want[rep % 2])


def test_missing_peer_times_out_instead_of_passing_stale_segments():
    """Step 1 completes.  At step 2 rank 3 never reduces: rank 0's share must
    wait for rank 3's slots >= 2, run out of time and report it (not copy the
    step-1 segment).  A reset then starts clean."""
    n, numel, dt = 8, 8 * 8192, "bf16"
    s = Set(n, numel, dt, [630, 631])
    out0 = [s.outs[0]] + [None] * (n - 1)
    for r in range(1, n):
        car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=r, r1=r + 1)
    car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=0, r1=1, outs=out0)
    torch.cuda.synchronize()
    car.raise_on_status(s.flags, "step 1")
    assert np.array_equal(bits(s.outs[0]), s.want[0])

    s.load(1)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(50_000_000)
    try:
        for r in range(1, n):
            if r != 3:
                car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=r, r1=r + 1)
        car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=0, r1=1, outs=out0)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, phase, _ = car.decode_status(car.read_status(s.flags)[0])
    assert (code, phase) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG)
    ep = epochs(s.flags, n)
    assert ep[3] == 1 and all(ep[r] == 2 for r in range(n) if r != 3)

    car.ar_flag_barrier_reset(s.flags, n)
    assert epochs(s.flags, n) == [0] * n
    for r in range(1, n):
        car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=r, r1=r + 1)
    car.ar_twoshot_rs(s.ins, s.segs, s.flags, 0, r0=0, r1=1, outs=out0)
    torch.cuda.synchronize()
    car.raise_on_status(s.flags, "after reset")
    assert np.array_equal(bits(s.outs[0]), s.want[1])


# ------------------------------------------------------------- staging path --
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_staged_in_place_all_reduce(dt):
    """Non-graph path: stage every rank's tensor into its registered buffer,
    then reduce from the registered buffers back into the tensors in place --
    rank 0 by the one-shot, every rank by the reduce-broadcast."""
    n, numel = 8, 8 * 8192 + 5
    host = synth.rank_inputs(n, numel, dt, "normal", config=640)
    want = oracle_bits(oracle.oneshot(host, dt))
    xs = [to_dev(a) for a in host]  # the callers' tensors
    reg = [torch.empty_like(x) for x in xs]  # registered buffers
    car.ar_push(xs, [[r] for r in reg])
    car.ar_oneshot(reg, xs[0])
    torch.cuda.synchronize()
    assert np.array_equal(bits(xs[0]), want)
    for r in range(1, n):
        assert np.array_equal(bits(xs[r]), oracle_bits(host[r]))  # untouched

    xs = [to_dev(a) for a in host]
    car.ar_push(xs, [[r] for r in reg])
    car.ar_reduce_bcast(reg, xs)
    torch.cuda.synchronize()
    for r in range(n):
        assert np.array_equal(bits(xs[r]), want), f"rank {r}"


def test_staged_path_in_a_graph():
    n, numel, dt = 4, 4 * 8192, "bf16"
    datasets = [synth.rank_inputs(n, numel, dt, "normal", config=650 + k) for k in range(2)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in datasets]
    xs = [to_dev(a) for a in datasets[0]]
    reg = [torch.empty_like(x) for x in xs]
    torch.cuda.synchronize()

    def step():
        car.ar_push(xs, [[r] for r in reg])
        car.ar_reduce_bcast(reg, xs)

    g = capture(step)
    for rep in range(4):
        for d, a in zip(xs, datasets[rep % 2]):
            d.copy_(to_dev(a))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(n):
            assert np.array_equal(bits(xs[r]), wants[rep % 2]), f"replay {rep} rank {r}"
