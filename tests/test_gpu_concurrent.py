"""Consumers that start before their data exists.

Each case launches a consumer while the producers it waits on have written
nothing; their buffers (wire lines, segments, arrival slots) live in pinned
host memory, and the host writes them (all data first, then the flags or
slots) after a delay while the kernel polls: the LL / LL128 receivers, one
GPU's LL / LL128 step in one launch, one rank's two-shot share with slots,
under LL and under LL128, and the copy-engine all-gather.  This exercises the
polling paths against a writer that is truly concurrent (two GPU streams may
share one hardware queue, so a second stream would not guarantee that).
Every wait is bounded, so a mistake shows up as a reported timeout, never as
a hang.

(The two-shot barrier's case of consumers polling while producers of the
same launch publish is the fused full-emulation launch exercised throughout
test_gpu_twoshot.py.)"""
from __future__ import annotations

import ctypes
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")


def pinned_device_view(nbytes: int):
    """Zeroed pinned host buffer and its device address."""
    t = torch.zeros(nbytes + 16, dtype=torch.uint8, pin_memory=True)
    hip = ctypes.CDLL("libamdhip64.so.7")
    dp = ctypes.c_void_p()
    assert hip.hipHostGetDevicePointer(ctypes.byref(dp), ctypes.c_void_p(t.data_ptr()), 0) == 0
    off = (-dp.value) % 16  # 16-byte alignment on the device side
    return t, off, dp.value + off


def write_lines(host_buf: np.ndarray, proto: str, msg: np.ndarray, step: int):
    """Host-side sender: every line's data, then (after all data) every flag."""
    raw = msg.view(np.uint8)
    d, lb = (4, 8) if proto == "ll" else (120, 128)
    lines = -(-raw.size // d)
    view = host_buf[: lines * lb].reshape(lines, lb)
    pad = np.zeros(lines * d, np.uint8)
    pad[: raw.size] = raw
    view[:, :d] = pad.reshape(lines, d)
    flag = np.zeros(lb - d, np.uint8)
    flag[:4] = np.frombuffer(np.uint32(step).tobytes(), np.uint8)
    view[:, d:] = flag


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_receiver_polls_until_the_host_writes_the_lines(proto, dt):
    n, numel = 4, 1500 + (1 if dt == "bf16" else 0)
    es = 4 if dt == "f32" else 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=310)
    want = oracle_bits(oracle.oneshot(host, dt))
    W = car.ll_wire_bytes(proto, numel * es)
    bufs = [pinned_device_view(W) for _ in range(n)]
    out = torch.empty(numel, dtype=torch.float32 if dt == "f32" else torch.bfloat16, device="cuda")
    flags = car.new_flags(n)
    torch.cuda.synchronize()
    wires = (ctypes.c_void_p * n)(*[b[2] for b in bufs])
    fn = car.lib.ar_ll_reduce_unpack if proto == "ll" else car.lib.ar_ll128_reduce_unpack
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(3_000_000_000)
    try:
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert fn(wires, n, out.data_ptr(), numel, 0 if dt == "f32" else 1, 9, flags.data_ptr(), st) == 0
        time.sleep(0.05)  # the receiver is polling now
        for r in range(n):
            t, off, _ = bufs[r]
            write_lines(t.numpy()[off:], proto, host[r], 9)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    assert car.read_status(flags)[0] == 0
    assert np.array_equal(bits(out), want)


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_send_and_receive_waits_for_late_peers(proto, dt):
    """One GPU's LL / LL128 step in one launch (ar_ll_allreduce) started while
    its peers' lines are still zero: the peers' wires are pinned host buffers
    the host fills after a delay, so the fold the kernel runs as its first
    loads land is on stale lines and must be redone after the slow path's
    re-read.  Rank me's wire (device memory) must hold its packed message and
    the output the oracle's all-reduce.  The sizes leave a partial last
    wavefront (rank me's bytes loaded word by word) and, in bf16, a lone
    final element."""
    n, me = 4, 2
    numel = 1500 + (1 if dt == "bf16" else 0)
    es = 4 if dt == "f32" else 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=312)
    want = oracle_bits(oracle.oneshot(host, dt))
    W = car.ll_wire_bytes(proto, numel * es)
    bufs = [pinned_device_view(W) if r != me else None for r in range(n)]
    own = torch.zeros(W, dtype=torch.uint8, device="cuda")
    src = to_dev(host[me])
    out = torch.empty(numel, dtype=src.dtype, device="cuda")
    flags = car.new_flags(n)
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    wires = (P * n)(*[own.data_ptr() if r == me else bufs[r][2] for r in range(n)])
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(3_000_000_000)
    try:
        st = P(torch.cuda.current_stream().cuda_stream)
        rc = car.lib.ar_ll_allreduce(src.data_ptr(), wires, n, me, out.data_ptr(), numel, 0 if dt == "f32" else 1,
                                     car.AR_PROTO_LL if proto == "ll" else car.AR_PROTO_LL128, 9, flags.data_ptr(), st)
        assert rc == 0
        time.sleep(0.05)  # the launch is polling now
        for r in range(n):
            if r != me:
                t, off, _ = bufs[r]
                write_lines(t.numpy()[off:], proto, host[r], 9)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    assert car.read_status(flags)[0] == 0
    assert np.array_equal(bits(out), want)
    assert np.array_equal(bits(own), oracle.ll_pack(proto, bits(src), 9))


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_twoshot_share_under_ll_waits_for_the_host_written_peer_segments(proto, dt):
    """Rank 0's two-shot under LL or LL128 with the peers' segment wires in
    pinned host memory, all flags 0 at launch: the all-gather polls the
    flags; the host then writes every peer line's data and afterwards its
    flag.  The output must be the oracle's all-reduce, and rank 0's own
    segment wire the oracle's packing of its segment."""
    n, es = 4, 4 if dt == "f32" else 2
    m = (16 // es) * 150  # 150 vectors: 20 lines per segment, a partial last line
    numel = n * m
    host = synth.rank_inputs(n, numel, dt, "normal", config=311)
    segs, _ = oracle.twoshot(host, dt)
    want = oracle_bits(oracle.oneshot(host, dt))
    W = car.ll_wire_bytes(proto, m * es)
    ins = [to_dev(a) for a in host]
    own = torch.zeros(W, dtype=torch.uint8, device="cuda")
    bufs = [None] + [pinned_device_view(W) for _ in range(1, n)]
    out = torch.empty(numel, dtype=ins[0].dtype, device="cuda")
    flags = car.new_flags(n)
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    in_p = (P * n)(*[t.data_ptr() for t in ins])
    seg_p = (P * n)(own.data_ptr(), *[b[2] for b in bufs[1:]])
    out_p = (P * n)(out.data_ptr(), *([None] * (n - 1)))
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(3_000_000_000)
    try:
        st = P(torch.cuda.current_stream().cuda_stream)
        fn = car.lib.ar_twoshot_ll if proto == "ll" else car.lib.ar_twoshot_ll128
        rc = fn(in_p, n, seg_p, numel, 0 if dt == "f32" else 1, 0, 1, flags.data_ptr(), 7, out_p, st)
        assert rc == 0
        time.sleep(0.05)  # the all-gather is polling now
        for j in range(1, n):
            t, off, _ = bufs[j]
            write_lines(t.numpy()[off:], proto, segs[j], 7)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    assert car.read_status(flags)[0] == 0
    assert np.array_equal(bits(out), want)
    assert np.array_equal(bits(own), oracle.ll_pack(proto, segs[0], 7))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_slot_share_waits_for_host_published_peers(dt):
    """Rank 0's fused two-shot share with arrival slots (one wavefront per
    tile and per all-gather chunk), launched while its peers have published
    nothing: the peers' segments and the flag region are pinned host memory,
    and the host writes every peer segment and afterwards its slots (x86
    store order keeps the data first) while the all-gather polls.  The
    output must be the oracle's all-reduce and rank 0's segment the oracle's
    reduce-scatter."""
    n, es = 4, 4 if dt == "f32" else 2
    m = (16 // es) * 64 * 5 + (16 // es) * 3  # 5 whole 64-vector tiles and a partial one
    numel = n * m
    host = synth.rank_inputs(n, numel, dt, "normal", config=313)
    segs, _ = oracle.twoshot(host, dt)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    own = torch.zeros(m, dtype=ins[0].dtype, device="cuda")
    bufs = [None] + [pinned_device_view(m * es) for _ in range(1, n)]
    fl_t, fl_off, fl_dev = pinned_device_view(car.flag_bytes(n))
    out = torch.empty(numel, dtype=ins[0].dtype, device="cuda")
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    in_p = (P * n)(*[t.data_ptr() for t in ins])
    seg_p = (P * n)(own.data_ptr(), *[b[2] for b in bufs[1:]])
    out_p = (P * n)(out.data_ptr(), *([None] * (n - 1)))
    slots = fl_t.numpy()[fl_off:].view(np.uint32)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(3_000_000_000)
    try:
        st = P(torch.cuda.current_stream().cuda_stream)
        rc = car.lib.ar_twoshot_rs(in_p, n, seg_p, numel, 0 if dt == "f32" else 1, 0, 1, P(fl_dev), 7, out_p, st)
        assert rc == 0
        time.sleep(0.05)  # the all-gather is polling now
        for j in range(1, n):
            t, off, _ = bufs[j]
            t.numpy()[off:off + m * es] = segs[j].view(np.uint8)
        for j in range(1, n):
            base = 32 + j * car.AR_SLOTS_PER_RANK
            slots[base:base + car.AR_SLOTS_PER_RANK] = 7
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    assert slots[0] == 0, car.decode_status(int(slots[0]))
    assert np.array_equal(bits(out), want)
    assert np.array_equal(bits(own), oracle_bits(segs[0]))


def test_copy_engine_all_gather_waits_for_host_published_slots():
    """The copy-engine all-gather (one waiting workgroup, then one copy per
    segment) launched while no peer has published: segments and slots are
    pinned host memory that the host fills after a delay (segments first,
    then slots).  Rank 0's output must be the oracle's all-reduce."""
    n, dt, es = 4, "bf16", 2
    m = 8 * 64 * 3
    numel = n * m
    host = synth.rank_inputs(n, numel, dt, "normal", config=314)
    segs, _ = oracle.twoshot(host, dt)
    want = oracle_bits(oracle.oneshot(host, dt))
    bufs = [pinned_device_view(m * es) for _ in range(n)]
    fl_t, fl_off, fl_dev = pinned_device_view(car.flag_bytes(n))
    out = torch.empty(numel, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    seg_p = (P * n)(*[b[2] for b in bufs])
    out_p = (P * n)(out.data_ptr(), *([None] * (n - 1)))
    slots = fl_t.numpy()[fl_off:].view(np.uint32)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(3_000_000_000)
    try:
        st = P(torch.cuda.current_stream().cuda_stream)
        rc = car.lib.ar_twoshot_ag_copy(seg_p, n, out_p, numel, 1, 0, 1, P(fl_dev), 9, st)
        assert rc == 0
        time.sleep(0.05)  # the wait kernel is polling now
        for j in range(n):
            t, off, _ = bufs[j]
            t.numpy()[off:off + m * es] = segs[j].view(np.uint8)
        for j in range(n):
            base = 32 + j * car.AR_SLOTS_PER_RANK
            slots[base:base + car.AR_SLOTS_PER_RANK] = 9
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    assert slots[0] == 0, car.decode_status(int(slots[0]))
    assert np.array_equal(bits(out), want)
