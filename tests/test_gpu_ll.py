"""GPU parity of the LL and LL128 protocols (pack on the sender, poll +
unpack + reduce on the receiver) against the CPU oracle, bit for bit."""
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


def wires_for(n, numel, dt, proto):
    W = car.ll_wire_bytes(proto, numel * ES[dt])
    # wire buffers padded to 16 bytes plus a guard band of 256 bytes
    bufs = [torch.full((W + 256,), 0xA5, dtype=torch.uint8, device="cuda") for _ in range(n)]
    return bufs, W


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("numel", [1, 2, 3, 5, 29, 30, 31, 59, 60, 61, 240, 1000, 4096 + 7, 65536 + 3])
def test_pack_layout_matches_oracle(proto, dt, numel):
    n = 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=90)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, proto)
    car.ar_ll_pack(srcs, [b[:W] for b in bufs], proto, step=123457)
    torch.cuda.synchronize()
    for r in range(n):
        got = bits(bufs[r])
        want = oracle.ll_pack(proto, host[r], 123457)
        assert np.array_equal(got[:W], want), first_mismatch(got[:W], want)
        assert np.all(got[W:] == 0xA5), "pack wrote past the wire buffer"


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
@pytest.mark.parametrize("numel", [1, 7, 61, 1023, 30 * 64 * 3 + 11, 100000 + 1])
def test_reduce_matches_oracle(proto, dt, n, numel):
    host = synth.rank_inputs(n, numel, dt, "normal", config=91 + n)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    outbuf = filled(numel + 64, DT[dt])
    out = outbuf[:numel]
    car.ar_ll_pack(srcs, wires, proto, step=9)
    fn = car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack
    fn(wires, out, 9, flags)
    torch.cuda.synchronize()
    assert car.read_status(flags)[0] == 0
    got = bits(out)
    want = oracle_bits(oracle.ll_reduce(proto, [oracle.ll_pack(proto, a, 9) for a in host], numel, dt, 9))
    assert np.array_equal(got, want), first_mismatch(got, want)
    assert np.array_equal(want, oracle_bits(oracle.oneshot(host, dt)))
    assert np.array_equal(bits(outbuf[numel:]), bits(filled(64, DT[dt]))), "wrote past the output"


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("kib, steps", [(64, 1000), (1024, 100)])
def test_steps_without_reset(proto, kib, steps):
    """n = 8 ranks, fp32 payload of 64 KiB (steps 1..1000) or 1 MiB (steps
    1..100) per rank; the data alternates between three sets so a receiver
    that reused an old line would produce a wrong sum."""
    n, dt = 8, "f32"
    numel = kib * 1024 // 4
    sets = [synth.rank_inputs(n, numel, dt, "normal", config=95 + k) for k in range(3)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in sets]
    dsets = [[to_dev(a) for a in h] for h in sets]
    bufs, W = wires_for(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    outs = torch.empty((steps, numel), device="cuda")
    fn = car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack
    for step in range(1, steps + 1):
        car.ar_ll_pack(dsets[step % 3], wires, proto, step=step)
        fn(wires, outs[step - 1], step, flags)
    torch.cuda.synchronize()
    assert car.read_status(flags)[0] == 0
    got_all = outs.cpu().numpy().view(np.uint32)
    for step in range(1, steps + 1):
        got = got_all[step - 1]
        assert np.array_equal(got, wants[step % 3]), f"step {step}: " + first_mismatch(got, wants[step % 3])


@pytest.mark.parametrize("proto, phase", [("ll", 2), ("ll128", 3)])
def test_stale_rank_times_out_and_names_it(proto, phase):
    """Rank 5 packed step s-1; the receiver of step s must report (timeout,
    phase, rank 5) after its tiny budget and exit normally."""
    n, numel, dt = 8, 4096, "f32"
    host = synth.rank_inputs(n, numel, dt, "normal", config=99)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    car.ar_ll_pack([s for i, s in enumerate(srcs) if i != 5], [w for i, w in enumerate(wires) if i != 5], proto,
                   step=11)
    car.ar_ll_pack([srcs[5]], [wires[5]], proto, step=10)
    out = torch.empty(numel, device="cuda")
    fn = car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(20_000)
    try:
        fn(wires, out, 11, flags)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    word, detail = car.read_status(flags)
    code, ph, rank = car.decode_status(word)
    assert (code, ph, rank) == (car.AR_ERR_TIMEOUT, phase, 5)
    assert detail < (numel * 4 + 3) // 4
    # the same wires at step 10 are ready for every rank (>= 10)
    car.ar_flag_barrier_reset(flags, n)
    fn(wires, out, 10, flags)
    torch.cuda.synchronize()
    assert car.read_status(flags)[0] == 0
    assert np.array_equal(bits(out), oracle_bits(oracle.oneshot(host, dt)))


def test_wire_sizes_for_the_64KiB_and_1MiB_messages():
    for S in (64 * 1024, 1024 * 1024):
        assert car.ll_wire_bytes("ll", S) == 2 * S
        assert car.ll_wire_bytes("ll128", S) == oracle.ll_wire_bytes("ll128", S)


# The LL receiver has two kernels: one line per lane up to 16 MiB per rank,
# two lines per lane above (whose odd last line is finished by one lane).
# These cases sit on both sides of that boundary, with partial last lines.
ONE_LINE_MAX = 16 << 20


@pytest.mark.parametrize("dt, numel", [("f32", ONE_LINE_MAX // 4), ("f32", ONE_LINE_MAX // 4 + 3),
                                       ("bf16", ONE_LINE_MAX // 2), ("bf16", ONE_LINE_MAX // 2 + 5)])
@pytest.mark.parametrize("n", [2, 3])
def test_ll_reduce_either_side_of_the_kernel_switch(dt, numel, n):
    host = synth.rank_inputs(n, numel, dt, "normal", config=120 + n)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, "ll")
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    outbuf = filled(numel + 64, DT[dt])
    out = outbuf[:numel]
    car.ar_ll_pack(srcs, wires, "ll", step=4)
    car.ar_ll_reduce_unpack(wires, out, 4, flags)
    torch.cuda.synchronize()
    assert car.read_status(flags)[0] == 0
    got = bits(out)
    want = oracle_bits(oracle.oneshot(host, dt))
    assert np.array_equal(got, want), first_mismatch(got, want)
    assert np.array_equal(bits(outbuf[numel:]), bits(filled(64, DT[dt]))), "wrote past the output"


def test_stale_rank_above_the_kernel_switch_times_out():
    """The two-line receiver's bounded wait: rank 1 packed the previous step."""
    n, numel, dt = 2, ONE_LINE_MAX // 4 + 3, "f32"
    host = synth.rank_inputs(n, numel, dt, "normal", config=130)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, "ll")
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    car.ar_ll_pack([srcs[0]], [wires[0]], "ll", step=21)
    car.ar_ll_pack([srcs[1]], [wires[1]], "ll", step=20)
    out = torch.empty(numel, device="cuda")
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(20_000)
    try:
        car.ar_ll_reduce_unpack(wires, out, 21, flags)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    word, detail = car.read_status(flags)
    assert car.decode_status(word) == (car.AR_ERR_TIMEOUT, car.PHASE_LL, 1)
    assert detail < numel
    car.ar_flag_barrier_reset(flags, n)
    car.ar_ll_reduce_unpack(wires, out, 20, flags)
    torch.cuda.synchronize()
    assert car.read_status(flags)[0] == 0
    assert np.array_equal(bits(out), oracle_bits(oracle.oneshot(host, dt)))


# ------------------------------------------------- send + receive, one launch --
def allreduce_case(proto, dt, n, me, numel, step, config):
    """Peers' wires packed beforehand at `step`; rank me's message and the
    reduction in one ar_ll_allreduce launch."""
    host = synth.rank_inputs(n, numel, dt, "normal", config=config)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    peers = [r for r in range(n) if r != me]
    car.ar_ll_pack([srcs[r] for r in peers], [wires[r] for r in peers], proto, step=step)
    flags = car.new_flags(n)
    outbuf = filled(numel + 64, DT[dt])
    out = outbuf[:numel]
    car.ar_ll_allreduce(srcs[me], wires, out, flags, proto, me, step)
    torch.cuda.synchronize()
    return host, bufs, W, flags, outbuf, out


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("numel", [1, 61, 30 * 64 * 3 + 11, 64 * 64 * 4, 100000 + 1])
def test_allreduce_matches_oracle(proto, dt, n, where, numel):
    """Output = the oracle's sum of all n messages; rank me's wire = the
    oracle's packing of its message; nothing written past either."""
    me = {"first": 0, "middle": n // 2, "last": n - 1}[where]
    host, bufs, W, flags, outbuf, out = allreduce_case(proto, dt, n, me, numel, 77, 140 + n)
    assert car.read_status(flags)[0] == 0
    got = bits(out)
    want = oracle_bits(oracle.oneshot(host, dt))
    assert np.array_equal(got, want), first_mismatch(got, want)
    assert np.array_equal(bits(outbuf[numel:]), bits(filled(64, DT[dt]))), "wrote past the output"
    wire = bits(bufs[me])
    want_wire = oracle.ll_pack(proto, host[me], 77)
    assert np.array_equal(wire[:W], want_wire), "own wire: " + first_mismatch(wire[:W], want_wire)
    assert np.all(wire[W:] == 0xA5), "wrote past rank me's wire"


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("kib, steps", [(64, 300), (1024, 40)])
def test_allreduce_steps_without_reset(proto, kib, steps):
    """n = 8, fp32, rank 3's step: every step the peers pack new data, then
    one launch packs rank 3's and reduces; data alternates between three sets."""
    n, dt, me = 8, "f32", 3
    numel = kib * 1024 // 4
    sets = [synth.rank_inputs(n, numel, dt, "normal", config=150 + k) for k in range(3)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in sets]
    dsets = [[to_dev(a) for a in h] for h in sets]
    bufs, W = wires_for(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    outs = torch.empty((steps, numel), device="cuda")
    peers = [r for r in range(n) if r != me]
    for step in range(1, steps + 1):
        d = dsets[step % 3]
        car.ar_ll_pack([d[r] for r in peers], [wires[r] for r in peers], proto, step=step)
        car.ar_ll_allreduce(d[me], wires, outs[step - 1], flags, proto, me, step)
    torch.cuda.synchronize()
    assert car.read_status(flags)[0] == 0
    got_all = outs.cpu().numpy().view(np.uint32)
    for step in range(1, steps + 1):
        got = got_all[step - 1]
        assert np.array_equal(got, wants[step % 3]), f"step {step}: " + first_mismatch(got, wants[step % 3])


@pytest.mark.parametrize("proto, phase", [("ll", 2), ("ll128", 3)])
def test_allreduce_stale_peer_times_out_after_packing(proto, phase):
    """Rank 5 packed the previous step: the launch still writes rank 2's
    wire for step s, then reports (timeout, phase, rank 5) and exits."""
    n, numel, dt, me = 8, 4096, "f32", 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=160)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    car.ar_ll_pack([srcs[r] for r in range(n) if r not in (me, 5)], [wires[r] for r in range(n) if r not in (me, 5)],
                   proto, step=11)
    car.ar_ll_pack([srcs[5]], [wires[5]], proto, step=10)
    out = torch.empty(numel, device="cuda")
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(20_000)
    try:
        car.ar_ll_allreduce(srcs[me], wires, out, flags, proto, me, 11)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, ph, rank = car.decode_status(car.read_status(flags)[0])
    assert (code, ph, rank) == (car.AR_ERR_TIMEOUT, phase, 5)
    assert np.array_equal(bits(bufs[me])[:W], oracle.ll_pack(proto, host[me], 11))


# Above 16 MiB per rank the send-and-receive LL launch takes two lines per
# lane.  Tails: f32 + 3 and bf16 + 5 leave an odd last line (4 and 2 bytes),
# finished by one lane; bf16 + 3 leaves an even line count whose last chunk
# ends in a lone bf16.
@pytest.mark.parametrize("dt, numel, n, me", [("f32", ONE_LINE_MAX // 4, 2, 0), ("f32", ONE_LINE_MAX // 4 + 3, 2, 1),
                                              ("bf16", ONE_LINE_MAX // 2 + 5, 2, 1), ("bf16", ONE_LINE_MAX // 2 + 3, 3, 1),
                                              ("f32", ONE_LINE_MAX // 4 + 3, 3, 2)])
def test_allreduce_ll_either_side_of_the_kernel_switch(dt, numel, n, me):
    host, bufs, W, flags, outbuf, out = allreduce_case("ll", dt, n, me, numel, 5, 170 + n)
    assert car.read_status(flags)[0] == 0
    got, want = bits(out), oracle_bits(oracle.oneshot(host, dt))
    assert np.array_equal(got, want), first_mismatch(got, want)
    assert np.array_equal(bits(outbuf[numel:]), bits(filled(64, DT[dt]))), "wrote past the output"
    wire = bits(bufs[me])
    assert np.array_equal(wire[:W], oracle.ll_pack("ll", host[me], 5)), "own wire"
    assert np.all(wire[W:] == 0xA5), "wrote past rank me's wire"


@pytest.mark.parametrize("dt, numel", [("f32", ONE_LINE_MAX // 4 + 3), ("bf16", ONE_LINE_MAX // 2 + 3)])
def test_allreduce_ll_above_16MiB_auto_steps(dt, numel):
    """Step 0 above the switch: three rounds of the peer's auto pack and rank
    0's auto send-and-receive from zeroed wires, new data each round; every
    output matches the oracle and rank 0's wire is its packing at step 3."""
    n, me = 2, 0
    rounds = [synth.rank_inputs(n, numel, dt, "normal", config=175 + k) for k in range(3)]
    bufs, W = wires_for(n, numel, dt, "ll")
    for b in bufs:
        b[:W].zero_()
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    out = torch.empty(numel, dtype=DT[dt], device="cuda")
    for k, host in enumerate(rounds):
        srcs = [to_dev(a) for a in host]
        car.ar_ll_pack([srcs[1]], [wires[1]], "ll", 0)
        car.ar_ll_allreduce(srcs[me], wires, out, flags, "ll", me, 0)
        torch.cuda.synchronize()
        assert car.read_status(flags)[0] == 0, f"round {k}"
        got, want = bits(out), oracle_bits(oracle.oneshot(host, dt))
        assert np.array_equal(got, want), f"round {k}: " + first_mismatch(got, want)
    assert np.array_equal(bits(bufs[me])[:W], oracle.ll_pack("ll", rounds[-1][me], 3))


def test_allreduce_ll_above_16MiB_stale_peer_times_out_after_packing():
    """Two lines per lane: rank 1 packed the previous step; rank 0's launch
    still writes its wire for step s (odd last line included), then reports
    (timeout, LL, rank 1)."""
    n, numel, dt, me = 2, ONE_LINE_MAX // 4 + 3, "f32", 0
    host = synth.rank_inputs(n, numel, dt, "normal", config=179)
    srcs = [to_dev(a) for a in host]
    bufs, W = wires_for(n, numel, dt, "ll")
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    car.ar_ll_pack([srcs[1]], [wires[1]], "ll", step=30)
    out = torch.empty(numel, device="cuda")
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(20_000)
    try:
        car.ar_ll_allreduce(srcs[me], wires, out, flags, "ll", me, 31)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, ph, rank = car.decode_status(car.read_status(flags)[0])
    assert (code, ph, rank) == (car.AR_ERR_TIMEOUT, car.PHASE_LL, 1)
    assert np.array_equal(bits(bufs[me])[:W], oracle.ll_pack("ll", host[me], 31))


# ------------------------------------------------------------ auto step ids --
def zeroed_wires(n, numel, dt, proto):
    bufs, W = wires_for(n, numel, dt, proto)
    for b in bufs:
        b[:W].zero_()
    return bufs, W


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt, numel", [("f32", 4096 + 3), ("bf16", 61), ("bf16", 30 * 64 * 3 + 11)])
def test_pack_auto_steps_advance_every_line(proto, dt, numel):
    """Step 0: every line's flag becomes its previous flag + 1; after three
    calls from zeroed wires the wire is the oracle's packing at step 3."""
    n = 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=180)
    srcs = [to_dev(a) for a in host]
    bufs, W = zeroed_wires(n, numel, dt, proto)
    for _ in range(3):
        car.ar_ll_pack(srcs, [b[:W] for b in bufs], proto, 0)
    torch.cuda.synchronize()
    for r in range(n):
        got = bits(bufs[r])
        want = oracle.ll_pack(proto, host[r], 3)
        assert np.array_equal(got[:W], want), first_mismatch(got[:W], want)
        assert np.all(got[W:] == 0xA5), "pack wrote past the wire buffer"


@pytest.mark.parametrize("proto", ["ll", "ll128"])
def test_allreduce_auto_steps_with_changing_sizes_on_the_same_wires(proto):
    """One GPU's LL / LL128 step with auto step ids (each line's previous
    flag + 1) on wire buffers sized for the largest message, used as prefixes
    while the message size changes from call to call (bf16: 1000, 70001 and,
    past the LL receiver's one-line limit, 17 MiB per rank).  Lines past a
    smaller message keep their flags; the peers' packs advance the same lines
    as rank me, so every call pairs its lines with the peers' and matches the
    oracle."""
    n, me, dt = 4, 1, "bf16"
    numels = [1000, 70001, (ONE_LINE_MAX + (1 << 20)) // 2]
    data = [synth.rank_inputs(n, k, dt, "normal", config=480 + i) for i, k in enumerate(numels)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in data]
    srcs = [[to_dev(a) for a in h] for h in data]
    Wmax = car.ll_wire_bytes(proto, numels[-1] * 2)
    bufs = [torch.zeros(Wmax, dtype=torch.uint8, device="cuda") for _ in range(n)]
    flags = car.new_flags(n)
    peers = [r for r in range(n) if r != me]
    torch.cuda.synchronize()
    for call, i in enumerate([0, 2, 1, 2, 0, 1]):
        W = car.ll_wire_bytes(proto, numels[i] * 2)
        wires = [b[:W] for b in bufs]
        out = torch.full((numels[i],), 7, dtype=torch.bfloat16, device="cuda")
        car.ar_ll_pack([srcs[i][r] for r in peers], [wires[r] for r in peers], proto, 0)
        car.ar_ll_allreduce(srcs[i][me], wires, out, flags, proto, me, 0)
        torch.cuda.synchronize()
        car.raise_on_status(flags, f"call {call} (numel {numels[i]})")
        got = bits(out)
        assert np.array_equal(got, wants[i]), f"call {call} numel {numels[i]}: " + first_mismatch(got, wants[i])


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt, numel", [("bf16", 8 * 8192), ("f32", 100000 + 1)])
def test_allreduce_auto_steps_replayed_in_a_graph(proto, dt, numel):
    """The peers' packs and rank 3's send-and-receive, all with step 0,
    captured once and replayed with new data and nothing reset in between:
    every replay matches the oracle and advances every line by one."""
    n, me = 8, 3
    datasets = [synth.rank_inputs(n, numel, dt, "normal", config=190 + k) for k in range(3)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in datasets]
    srcs = [to_dev(a) for a in datasets[0]]
    bufs, W = zeroed_wires(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    out = torch.empty(numel, dtype=DT[dt], device="cuda")
    peers = [r for r in range(n) if r != me]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        car.ar_ll_pack([srcs[r] for r in peers], [wires[r] for r in peers], proto, 0)
        car.ar_ll_allreduce(srcs[me], wires, out, flags, proto, me, 0)
    torch.cuda.synchronize()
    for rep in range(6):
        k = rep % 3
        for d, a in zip(srcs, datasets[k]):  # eager work between replays
            d.copy_(to_dev(a))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert car.read_status(flags)[0] == 0, f"replay {rep}"
        got = bits(out)
        assert np.array_equal(got, wants[k]), f"replay {rep}: " + first_mismatch(got, wants[k])
        for r in (me, peers[0]):
            w = bits(bufs[r])[:W]
            assert np.array_equal(w, oracle.ll_pack(proto, datasets[k][r], rep + 1)), f"replay {rep}: wire {r}"


def test_allreduce_ll_two_lines_auto_steps_replayed_in_a_graph():
    """As above with LL above 16 MiB per rank (two lines per lane, odd last
    line): the peers' auto packs and rank 1's auto send-and-receive captured
    once, replayed three times with new data and nothing reset."""
    n, me, dt, numel = 4, 1, "f32", ONE_LINE_MAX // 4 + 3
    datasets = [synth.rank_inputs(n, numel, dt, "normal", config=197 + k) for k in range(3)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in datasets]
    srcs = [to_dev(a) for a in datasets[0]]
    bufs, W = zeroed_wires(n, numel, dt, "ll")
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    out = torch.empty(numel, dtype=DT[dt], device="cuda")
    peers = [r for r in range(n) if r != me]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        car.ar_ll_pack([srcs[r] for r in peers], [wires[r] for r in peers], "ll", 0)
        car.ar_ll_allreduce(srcs[me], wires, out, flags, "ll", me, 0)
    torch.cuda.synchronize()
    for rep in range(3):
        for d, a in zip(srcs, datasets[rep]):  # eager work between replays
            d.copy_(to_dev(a))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert car.read_status(flags)[0] == 0, f"replay {rep}"
        got = bits(out)
        assert np.array_equal(got, wants[rep]), f"replay {rep}: " + first_mismatch(got, wants[rep])
        w = bits(bufs[me])[:W]
        assert np.array_equal(w, oracle.ll_pack("ll", datasets[rep][me], rep + 1)), f"replay {rep}: own wire"


@pytest.mark.parametrize("proto, phase", [("ll", 2), ("ll128", 3)])
def test_allreduce_auto_steps_peer_left_behind_times_out(proto, phase):
    """Two auto steps for every rank, then a third where rank 6 does not
    pack: rank 0's lines move to 3, rank 6's stay at 2, and the launch
    reports (timeout, phase, rank 6)."""
    n, numel, dt, me = 8, 4096, "f32", 0
    host = synth.rank_inputs(n, numel, dt, "normal", config=195)
    srcs = [to_dev(a) for a in host]
    bufs, W = zeroed_wires(n, numel, dt, proto)
    wires = [b[:W] for b in bufs]
    flags = car.new_flags(n)
    out = torch.empty(numel, device="cuda")
    peers = [r for r in range(n) if r != me]
    for _ in range(2):
        car.ar_ll_pack([srcs[r] for r in peers], [wires[r] for r in peers], proto, 0)
        car.ar_ll_allreduce(srcs[me], wires, out, flags, proto, me, 0)
    torch.cuda.synchronize()
    assert car.read_status(flags)[0] == 0
    assert np.array_equal(bits(out), oracle_bits(oracle.oneshot(host, dt)))
    late = [r for r in peers if r != 6]
    car.ar_ll_pack([srcs[r] for r in late], [wires[r] for r in late], proto, 0)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(20_000)
    try:
        car.ar_ll_allreduce(srcs[me], wires, out, flags, proto, me, 0)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    code, ph, rank = car.decode_status(car.read_status(flags)[0])
    assert (code, ph, rank) == (car.AR_ERR_TIMEOUT, phase, 6)
    assert np.array_equal(bits(bufs[me])[:W], oracle.ll_pack(proto, host[me], 3))
