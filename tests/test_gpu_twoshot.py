"""GPU parity of the two-shot path (reduce-scatter, flag barrier, all-gather)
against the CPU oracle, bit for bit, in every launch form."""
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


class Ranks:
    """n emulated ranks on one GPU: inputs, segments, outputs, a flag region."""

    def __init__(self, host_ins, dt):
        self.n = len(host_ins)
        self.dt = dt
        self.numel = host_ins[0].size
        self.m = self.numel // self.n
        self.ins = [to_dev(a) for a in host_ins]
        self.segs = [filled(self.m, DT[dt]) for _ in range(self.n)]
        self.outs = [filled(self.numel, DT[dt]) for _ in range(self.n)]
        self.flags = car.new_flags(self.n)

    def load(self, host_ins):
        for d, a in zip(self.ins, host_ins):
            d.copy_(to_dev(a))


def check_outputs(rk, host_ins, ranks=None):
    segs_w, _ = oracle.twoshot(host_ins, rk.dt)
    want = oracle_bits(oracle.oneshot(host_ins, rk.dt))
    for r in (range(rk.n) if ranks is None else ranks):
        got = bits(rk.outs[r])
        assert np.array_equal(got, want), f"rank {r}: " + first_mismatch(got, want)
    for j in range(rk.n):
        assert np.array_equal(bits(rk.segs[j]), oracle_bits(segs_w[j])), f"segment {j}"


def assert_ok(flags):
    word, detail = car.read_status(flags)
    assert word == 0, f"status {car.decode_status(word)} detail {detail}"


def test_prefill_n8_bf16_512x8192_fused_full_emulation():
    """n = 8 ranks, bf16 [512 x 8192] per rank: one persistent grid does every
    rank's reduce-scatter, the flag barrier and every rank's all-gather."""
    w = synth.WORKLOADS["twoshot_prefill_n8_bf16_512x8192"]
    host = synth.rank_inputs(w["n"], w["numel"], "bf16", "normal", config=w["config"])
    rk = Ranks(host, "bf16")
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, outs=rk.outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 8, 13, 16])
def test_fused_all_rank_counts(n, dt):
    es = 4 if dt == "f32" else 2
    m = (16 // es) * 97  # segments of 97 vectors: one full and one short tile
    host = synth.rank_inputs(n, n * m, dt, "normal", config=30 + n)
    rk = Ranks(host, dt)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, outs=rk.outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 8, 16])
@pytest.mark.parametrize("seg_vectors", [1, 64, 65, 64 * 1024, 64 * 1024 + 64 * 3, 200003])
def test_fused_tilings(n, dt, seg_vectors):
    """Segment sizes around the tile boundaries: 1 vector, exactly one tile,
    one tile plus a vector, 1024 tiles of 64 vectors, and sizes that force
    tiles of 128 vectors with a short last tile."""
    es = 4 if dt == "f32" else 2
    m = seg_vectors * (16 // es)
    if n * m * es > 256 << 20:
        pytest.skip("keeps the oracle to seconds")
    host = synth.rank_inputs(n, n * m, dt, "normal", config=40 + n)
    rk = Ranks(host, dt)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, outs=rk.outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_launches_rs_then_ag(dt):
    n, m = 8, 4096
    host = synth.rank_inputs(n, n * m, dt, "normal", config=50)
    rk = Ranks(host, dt)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1)
    car.ar_twoshot_ag(rk.segs, rk.outs, rk.flags, step=1)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_one_gpu_share_with_peers_published_earlier(dt):
    """Per-rank share: the peers' segments and slots come from an earlier
    reduce-scatter; the timed form is RS of rank `me` fused with its AG."""
    n, m = 8, 8192
    host = synth.rank_inputs(n, n * m, dt, "normal", config=51)
    rk = Ranks(host, dt)
    me = 3
    for r in range(n):
        if r != me:
            car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, r0=r, r1=r + 1)
    outs = [rk.outs[r] if r == me else None for r in range(n)]
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, r0=me, r1=me + 1, outs=outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host, ranks=[me])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n,seg_vectors", [(2, 64 * 1024), (8, 64 * 1024), (16, 32 * 1024), (8, 40017)])
def test_share_at_prefill_sizes(n, dt, seg_vectors):
    """One rank's share at 1024 tiles per segment (4-8 MiB per rank), where
    the persistent grid has fewer wavefronts than items and each wavefront
    holds a reduce-scatter tile and several all-gather tiles.  A short last
    tile (40017 vectors) included; three steps with changing data on the same
    buffers."""
    es = 4 if dt == "f32" else 2
    m = seg_vectors * (16 // es)
    datasets = [synth.rank_inputs(n, n * m, dt, "normal", config=70 + k) for k in range(2)]
    rk = Ranks(datasets[0], dt)
    me = n - 1
    outs = [rk.outs[r] if r == me else None for r in range(n)]
    for step in (1, 2, 3):
        host = datasets[step % 2]
        rk.load(host)
        for r in range(n):
            if r != me:
                car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=step, r0=r, r1=r + 1)
        car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=step, r0=me, r1=me + 1, outs=outs)
        torch.cuda.synchronize()
        assert_ok(rk.flags)
        check_outputs(rk, host, ranks=[me])


def test_share_missing_peer_times_out_at_prefill_size():
    """8 MiB per rank, a peer that never reduces: the share still publishes
    its own tiles, then waits, runs out of time and names the missing
    segment.  A reset then starts clean."""
    n, dt, m = 8, "bf16", 8 * 64 * 1024
    host = synth.rank_inputs(n, n * m, dt, "normal", config=75)
    rk = Ranks(host, dt)
    out0 = [rk.outs[0]] + [None] * (n - 1)
    for r in range(1, n):
        if r != 5:
            car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, r0=r, r1=r + 1)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(2_000_000)
    try:
        car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, r0=0, r1=1, outs=out0)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, phase, rank = car.decode_status(car.read_status(rk.flags)[0])
    assert (code, phase, rank) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG, 5)
    # rank 0 published every tile of its segment before it waited
    ktiles = 1024  # 64 Ki vectors per segment: 1024 tiles of 64
    slots0 = rk.flags[32:32 + ktiles].cpu().numpy().view("uint32")
    assert (slots0 == 1).all()
    # recovery
    car.ar_flag_barrier_reset(rk.flags, n)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, outs=rk.outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host)


def test_many_steps_with_changing_data():
    """Steps 1..40 on the same buffers with new data every step: catches a
    consumer that reads a stale segment after the barrier."""
    n, m, dt = 8, 64 * 1024, "bf16"
    datasets = [synth.rank_inputs(n, n * m, dt, "normal", config=60 + k) for k in range(3)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in datasets]
    rk = Ranks(datasets[0], dt)
    for step in range(1, 41):
        k = step % 3
        rk.load(datasets[k])
        car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=step, outs=rk.outs)
        torch.cuda.synchronize()
        assert_ok(rk.flags)
        for r in range(n):
            got = bits(rk.outs[r])
            assert np.array_equal(got, wants[k]), f"step {step} rank {r}: " + first_mismatch(got, wants[k])


def test_all_outputs_identical_and_equal_to_oneshot():
    n, m, dt = 16, 4096, "f32"
    host = synth.rank_inputs(n, n * m, dt, "normal", config=70)
    rk = Ranks(host, dt)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=7, outs=rk.outs)
    one = torch.empty(n * m, device="cuda")
    car.ar_oneshot(rk.ins, one)
    torch.cuda.synchronize()
    ref = bits(one)
    for r in range(n):
        assert np.array_equal(bits(rk.outs[r]), ref)


def test_reset_zeroes_the_region():
    n = 16
    f = torch.full((car.flag_bytes(n) // 4,), -1, dtype=torch.int32, device="cuda")
    car.ar_flag_barrier_reset(f, n)
    torch.cuda.synchronize()
    assert int(f.abs().sum()) == 0


def test_missing_rank_times_out_and_names_it():
    """Rank 3 never publishes: the all-gather waits on its slots, runs out of
    its (deliberately tiny) budget, records (timeout, phase 1, rank 3) and
    the kernel exits normally."""
    n, m, dt = 8, 4096, "f32"
    host = synth.rank_inputs(n, n * m, dt, "normal", config=80)
    rk = Ranks(host, dt)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(50_000)  # 50 us
    try:
        for r in range(n):
            if r != 3:
                car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, r0=r, r1=r + 1)
        car.ar_twoshot_ag(rk.segs, rk.outs, rk.flags, step=1)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    word, detail = car.read_status(rk.flags)
    code, phase, rank = car.decode_status(word)
    assert (code, phase, rank) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG, 3)
    # recovery: reset, then the next step works
    car.ar_flag_barrier_reset(rk.flags, n)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=1, outs=rk.outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host)


def test_stale_step_times_out():
    """Every slot holds step 4; a consumer of step 5 must not pass."""
    n, m, dt = 4, 1024, "bf16"
    host = synth.rank_inputs(n, n * m, dt, "normal", config=81)
    rk = Ranks(host, dt)
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=4)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(20_000)
    try:
        car.ar_twoshot_ag(rk.segs, rk.outs, rk.flags, step=5)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, phase, _ = car.decode_status(car.read_status(rk.flags)[0])
    assert (code, phase) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG)


def test_synchronous_errors_on_device_buffers():
    n = 4
    host = synth.rank_inputs(n, n * 100, "f32", "normal", config=82)  # 100-float segments: 400 B, ok
    rk = Ranks(host, "f32")
    bad = synth.rank_inputs(3, 3 * 10, "f32", "normal", config=83)  # 10 floats: 40 B, not whole vectors
    rb = Ranks(bad, "f32")
    with pytest.raises(car.ArError) as e:
        car.ar_twoshot_rs(rb.ins, rb.segs, rb.flags, step=1, outs=rb.outs)
    assert e.value.code == car.AR_ERR_DIVISIBLE
    with pytest.raises(car.ArError) as e:
        car.ar_twoshot_rs(rk.ins, [rk.ins[0][:100]] + rk.segs[1:], rk.flags, step=1)
    assert e.value.code == car.AR_ERR_ALIAS


def test_largest_step_id_then_reset_and_restart():
    """Step ids run up to 2^32 - 1; a reset lets them start again at 1
    (every wait passes at >= step, so without the reset step 1 would see the
    old slots as arrived)."""
    n = 4
    host = synth.rank_inputs(n, n * 8 * 300, "bf16", "normal", config=95)
    want = oracle_bits(oracle.oneshot(host, "bf16"))
    rk = Ranks(host, "bf16")
    last = (1 << 32) - 1
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, last, outs=rk.outs)
    torch.cuda.synchronize()
    car.raise_on_status(rk.flags)
    for r in range(n):
        assert np.array_equal(bits(rk.outs[r]), want)
    for proto in ("ll", "ll128"):
        W = car.ll_wire_bytes(proto, host[0].size * 2)
        wires = [torch.empty(W, dtype=torch.uint8, device="cuda") for _ in range(n)]
        out = torch.empty(host[0].size, dtype=rk.ins[0].dtype, device="cuda")
        car.ar_ll_pack(rk.ins, wires, proto, last)
        (car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack)(wires, out, last, rk.flags)
        torch.cuda.synchronize()
        car.raise_on_status(rk.flags, proto)
        assert np.array_equal(bits(out), want), proto
    car.ar_flag_barrier_reset(rk.flags, n)
    for o in rk.outs:
        o.zero_()
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, 1, outs=rk.outs)
    torch.cuda.synchronize()
    car.raise_on_status(rk.flags)
    for r in range(n):
        assert np.array_equal(bits(rk.outs[r]), want)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
@pytest.mark.parametrize("seg_vectors", [1, 63, 64, 65, 255, 257, 64 * 1024 + 64 * 3, 200003])
def test_share_tilings(n, dt, seg_vectors):
    """One rank's share (grid sized to the work: a wavefront per reduce-scatter
    tile, one per all-gather chunk) at segment sizes around the unit, chunk and
    tile boundaries, including tiles of 128 and 256 vectors with a short last
    tile; the rank in the middle of the table, so the all-gather skips an
    inner segment."""
    es = 4 if dt == "f32" else 2
    m = seg_vectors * (16 // es)
    if n * m * es > 256 << 20:
        pytest.skip("keeps the oracle to seconds")
    host = synth.rank_inputs(n, n * m, dt, "normal", config=90 + n)
    rk = Ranks(host, dt)
    me = n // 2
    for r in range(n):
        if r != me:
            car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=3, r0=r, r1=r + 1)
    outs = [rk.outs[r] if r == me else None for r in range(n)]
    car.ar_twoshot_rs(rk.ins, rk.segs, rk.flags, step=3, r0=me, r1=me + 1, outs=outs)
    torch.cuda.synchronize()
    assert_ok(rk.flags)
    check_outputs(rk, host, ranks=[me])
