"""GPU parity of the two-shot under the LL and LL128 protocols
(ar_twoshot_ll, ar_twoshot_ll128): the reduced segments travel as LL wires
(4 data bytes and the step id per 8-byte line) or LL128 wires (120 data
bytes and a 64-bit step id per 128-byte line, the data ordered before the
flag), and the all-gather checks the flags of the lines it copies.  Outputs
must equal the oracle's all-reduce bit for bit, and every segment wire the
oracle's LL / LL128 packing of the oracle's reduce-scatter segment."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, filled, first_mismatch, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")
DT = {"f32": torch.float32, "bf16": torch.bfloat16}
ES = {"f32": 4, "bf16": 2}
PROTOS = ["ll", "ll128"]
TSLL = {"ll": car.ar_twoshot_ll, "ll128": car.ar_twoshot_ll128}


class Ranks:
    def __init__(self, host_ins, dt, proto):
        self.n = len(host_ins)
        self.dt = dt
        self.proto = proto
        self.numel = host_ins[0].size
        self.m = self.numel // self.n
        self.W = car.ll_wire_bytes(proto, self.m * ES[dt])
        self.ins = [to_dev(a) for a in host_ins]
        # segment wires zeroed (every flag below the first step, as LL needs
        # before first use), each with a 256-byte guard band after it
        self.wbuf = [torch.full((self.W + 256,), 0xA5, dtype=torch.uint8, device="cuda") for _ in range(self.n)]
        self.segw = [b[:self.W] for b in self.wbuf]
        for w in self.segw:
            w.zero_()
        self.outs = [filled(self.numel, DT[dt]) for _ in range(self.n)]
        self.flags = car.new_flags(self.n)

    def load(self, host_ins):
        for d, a in zip(self.ins, host_ins):
            d.copy_(to_dev(a))


def check(rk, host, step, ranks=None, wires=None):
    segs, _ = oracle.twoshot(host, rk.dt)
    want = oracle_bits(oracle.oneshot(host, rk.dt))
    for r in (range(rk.n) if ranks is None else ranks):
        got = bits(rk.outs[r])
        assert np.array_equal(got, want), f"rank {r}: " + first_mismatch(got, want)
    for j in (range(rk.n) if wires is None else wires):
        got = bits(rk.wbuf[j])
        want_w = oracle.ll_pack(rk.proto, segs[j], step)
        assert np.array_equal(got[:rk.W], want_w), f"segment wire {j}: " + first_mismatch(got[:rk.W], want_w)
        assert np.all(got[rk.W:] == 0xA5), f"wrote past segment wire {j}"


def assert_ok(flags):
    word, detail = car.read_status(flags)
    assert word == 0, f"status {car.decode_status(word)} detail {detail}"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 5, 8, 16])
@pytest.mark.parametrize("seg_vectors", [1, 64, 65, 97, 64 * 1024])
@pytest.mark.parametrize("proto", PROTOS)
def test_full_emulation(proto, n, dt, seg_vectors):
    """Every rank in one persistent launch: the all-gather reads lines other
    wavefronts of the same launch are writing."""
    m = seg_vectors * (16 // ES[dt])
    if n * m * ES[dt] > 64 << 20:
        pytest.skip("keeps the oracle to seconds")
    host = synth.rank_inputs(n, n * m, dt, "normal", config=300 + n)
    rk = Ranks(host, dt, proto)
    TSLL[proto](rk.ins, rk.segw, rk.flags, 5, outs=rk.outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check(rk, host, 5)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n, seg_vectors", [(8, 1024), (8, 64 * 1024), (16, 97), (2, 64 * 1024 + 7)])
@pytest.mark.parametrize("proto", PROTOS)
def test_one_gpu_share_steps_with_changing_data(proto, n, dt, seg_vectors):
    """Rank me's share after the peers' reduce-scatters of the same step,
    three steps on the same buffers with new data each step."""
    m = seg_vectors * (16 // ES[dt])
    datasets = [synth.rank_inputs(n, n * m, dt, "normal", config=320 + k) for k in range(2)]
    rk = Ranks(datasets[0], dt, proto)
    me = n // 2
    outs = [rk.outs[r] if r == me else None for r in range(n)]
    for step in (1, 2, 3):
        host = datasets[step % 2]
        rk.load(host)
        for r in range(n):
            if r != me:
                TSLL[proto](rk.ins, rk.segw, rk.flags, step, r0=r, r1=r + 1)
        TSLL[proto](rk.ins, rk.segw, rk.flags, step, r0=me, r1=me + 1, outs=outs)
        torch.cuda.synchronize()
        assert_ok(rk.flags)
        check(rk, host, step, ranks=[me])


@pytest.mark.parametrize("proto", PROTOS)
def test_many_full_steps_without_reset(proto):
    """Steps 1..30 of every rank in one launch, data alternating: a copy of a
    line left from the previous step would show."""
    n, dt, m = 8, "bf16", 8 * 4096
    datasets = [synth.rank_inputs(n, n * m, dt, "normal", config=330 + k) for k in range(3)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in datasets]
    rk = Ranks(datasets[0], dt, proto)
    for step in range(1, 31):
        rk.load(datasets[step % 3])
        TSLL[proto](rk.ins, rk.segw, rk.flags, step, outs=rk.outs)
        torch.cuda.synchronize()
        assert_ok(rk.flags)
        for r in (0, 5):
            assert np.array_equal(bits(rk.outs[r]), wants[step % 3]), f"step {step} rank {r}"


@pytest.mark.parametrize("seg_vectors", [1024, 64 * 1024])
@pytest.mark.parametrize("proto", PROTOS)
def test_missing_peer_times_out_and_names_its_segment(proto, seg_vectors):
    """Rank 6 reduced the previous step only: rank 0's share must report
    (timeout, all-gather phase, segment 6) and exit; then a full step works."""
    n, dt = 8, "bf16"
    m = seg_vectors * 8
    host = synth.rank_inputs(n, n * m, dt, "normal", config=340)
    rk = Ranks(host, dt, proto)
    TSLL[proto](rk.ins, rk.segw, rk.flags, 1, r0=6, r1=7)
    for r in range(1, n):
        if r != 6:
            TSLL[proto](rk.ins, rk.segw, rk.flags, 2, r0=r, r1=r + 1)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(2_000_000)
    try:
        TSLL[proto](rk.ins, rk.segw, rk.flags, 2, r0=0, r1=1, outs=[rk.outs[0]] + [None] * (n - 1))
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, phase, seg = car.decode_status(car.read_status(rk.flags)[0])
    assert (code, phase, seg) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG, 6)
    car.ar_flag_barrier_reset(rk.flags, n)
    TSLL[proto](rk.ins, rk.segw, rk.flags, 3, outs=rk.outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check(rk, host, 3)


@pytest.mark.parametrize("proto", PROTOS)
def test_in_a_graph_with_increasing_steps(proto):
    """Six full steps with step ids 1..6 captured once, replayed with new
    data.  The ids travel in the lines, so the wires are zeroed between
    replays (outside the graph) to bring every line below step 1 again."""
    n, dt, m = 4, "f32", 4 * 3000
    datasets = [synth.rank_inputs(n, n * m, dt, "normal", config=350 + k) for k in range(2)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in datasets]
    rk = Ranks(datasets[0], dt, proto)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(6):
            TSLL[proto](rk.ins, rk.segw, rk.flags, 1 + k, outs=rk.outs)
    torch.cuda.synchronize()
    for rep in range(4):
        rk.load(datasets[rep % 2])
        for w in rk.segw:
            w.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_ok(rk.flags)
        for r in range(n):
            assert np.array_equal(bits(rk.outs[r]), wants[rep % 2]), f"replay {rep} rank {r}"


# ------------------------------------------------------------ auto step ids --
def epochs(flags, n):
    """Rank r's epoch, equal in every wavefront copy of an auto launch (two
    4-wave workgroups per CU)."""
    grid = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    base = 32 + n * car.AR_SLOTS_PER_RANK
    w = flags[base:base + n * car.AR_EPOCH_COPIES].cpu().numpy().astype(np.int64).reshape(-1, n)
    for r in range(n):
        assert (w[:grid, r] == w[0, r]).all(), f"rank {r}: epoch copies differ"
    return w[0, :].tolist()


@pytest.mark.parametrize("n, dt, seg_vectors", [(8, "bf16", 1024), (5, "f32", 97), (16, "bf16", 64 * 1024)])
@pytest.mark.parametrize("proto", PROTOS)
def test_full_emulation_auto_steps_replayed_without_reset(proto, n, dt, seg_vectors):
    """Every rank in one auto launch, captured once, replayed with new data
    and nothing reset: each replay matches the oracle, its lines carry the
    new epoch, and every epoch advances by one."""
    m = seg_vectors * (16 // ES[dt])
    datasets = [synth.rank_inputs(n, n * m, dt, "normal", config=360 + k) for k in range(3)]
    rk = Ranks(datasets[0], dt, proto)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        TSLL[proto](rk.ins, rk.segw, rk.flags, 0, outs=rk.outs)
    torch.cuda.synchronize()
    for rep in range(6):
        host = datasets[rep % 3]
        rk.load(host)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_ok(rk.flags)
        assert epochs(rk.flags, n) == [rep + 1] * n
        check(rk, host, rep + 1, ranks=[0, n - 1])


@pytest.mark.parametrize("proto", PROTOS)
def test_one_rank_shares_auto_steps_in_a_graph(proto):
    """The peers' reduce-scatters and rank 0's fused share, all auto, in one
    graph; eager auto calls between replays keep the epochs in step."""
    n, dt, m = 8, "bf16", 8 * 4096
    datasets = [synth.rank_inputs(n, n * m, dt, "normal", config=370 + k) for k in range(2)]
    rk = Ranks(datasets[0], dt, proto)
    out0 = [rk.outs[0]] + [None] * (n - 1)

    def one_step():
        for r in range(1, n):
            TSLL[proto](rk.ins, rk.segw, rk.flags, 0, r0=r, r1=r + 1)
        TSLL[proto](rk.ins, rk.segw, rk.flags, 0, r0=0, r1=1, outs=out0)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_step()
    torch.cuda.synchronize()
    for rep in range(6):
        host = datasets[rep % 2]
        rk.load(host)
        if rep % 3 == 2:
            one_step()  # the same calls, eager
        else:
            g.replay()
        torch.cuda.synchronize()
        assert_ok(rk.flags)
        assert epochs(rk.flags, n) == [rep + 1] * n
        check(rk, host, rep + 1, ranks=[0])


@pytest.mark.parametrize("proto", PROTOS)
def test_auto_steps_missing_peer_times_out(proto):
    """Step 1 completes; at step 2 rank 3 does not reduce: rank 0's share
    reports (timeout, all-gather phase, segment 3) instead of copying rank
    3's step-1 lines."""
    n, dt, m = 8, "bf16", 8 * 4096
    host = synth.rank_inputs(n, n * m, dt, "normal", config=380)
    rk = Ranks(host, dt, proto)
    out0 = [rk.outs[0]] + [None] * (n - 1)
    for r in range(1, n):
        TSLL[proto](rk.ins, rk.segw, rk.flags, 0, r0=r, r1=r + 1)
    TSLL[proto](rk.ins, rk.segw, rk.flags, 0, r0=0, r1=1, outs=out0)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    for r in range(1, n):
        if r != 3:
            TSLL[proto](rk.ins, rk.segw, rk.flags, 0, r0=r, r1=r + 1)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(2_000_000)
    try:
        TSLL[proto](rk.ins, rk.segw, rk.flags, 0, r0=0, r1=1, outs=out0)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, phase, seg = car.decode_status(car.read_status(rk.flags)[0])
    assert (code, phase, seg) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG, 3)
