"""Index arithmetic at large sizes: n = 2 ranks of 2^30 + 5 bf16 elements
(2 GiB and a ragged tail per rank; 2^27 16-byte vectors, LL wires of 4 GiB,
byte offsets past 2^32), through every path: one-shot, reduce-broadcast, LL
and LL128 (receiver and one launch), and the two-shot (every rank with
slots, LL and LL128 segments, and one rank's share).  Small-integer inputs keep every sum exact, so a
wrong index anywhere shows as a wrong value.  Outputs are checked on samples
around the power-of-two boundaries against the oracle run on the sampled
columns."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

N = 2
NUMEL = (1 << 30) + 5


def sample(numel, seed=21):
    rng = np.random.default_rng(seed)
    pick = [np.arange(0, 4096), np.arange(numel - 4096, numel), rng.integers(0, numel, 20000)]
    for e in range(20, 31):
        b = 1 << e
        if b < numel:
            pick.append(np.arange(max(0, b - 40), min(numel, b + 40)))
    return np.unique(np.concatenate(pick))


@pytest.fixture(scope="module")
def data():
    host = synth.rank_inputs(N, NUMEL, "bf16", "int", config=30)
    idx = sample(NUMEL)
    want = oracle_bits(oracle.oneshot([np.ascontiguousarray(a[idx]) for a in host], "bf16"))
    ins = [to_dev(a) for a in host]
    del host
    return ins, idx, want


def check(t, idx, want, what):
    got = bits(t)[idx]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{what}: {bad.size} sampled mismatches, first at element {idx[bad[0]]}"


def test_oneshot_and_reduce_broadcast(data):
    ins, idx, want = data
    out = torch.empty(NUMEL, dtype=torch.bfloat16, device="cuda")
    car.ar_oneshot(ins, out)
    torch.cuda.synchronize()
    check(out, idx, want, "one-shot")
    outs = [out, torch.empty_like(out)]
    car.ar_reduce_bcast(ins, outs)
    torch.cuda.synchronize()
    for j in range(N):
        check(outs[j], idx, want, f"reduce-broadcast out[{j}]")


def test_ll_and_ll128(data):
    ins, idx, want = data
    out = torch.empty(NUMEL, dtype=torch.bfloat16, device="cuda")
    flags = car.new_flags(N)
    for proto in ("ll", "ll128"):
        W = car.ll_wire_bytes(proto, NUMEL * 2)
        wires = [torch.empty(W, dtype=torch.uint8, device="cuda") for _ in range(N)]
        car.ar_ll_pack(ins, wires, proto, 1)
        (car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack)(wires, out, 1, flags)
        torch.cuda.synchronize()
        car.raise_on_status(flags, proto)
        check(out, idx, want, proto)
        del wires
        torch.cuda.empty_cache()


def test_ll_and_ll128_send_and_receive_in_one_launch(data):
    """Rank 1 packs its 2 GiB message and reduces rank 0's 4 GiB LL wire (or
    its LL128 wire) in one launch."""
    ins, idx, want = data
    out = torch.empty(NUMEL, dtype=torch.bfloat16, device="cuda")
    flags = car.new_flags(N)
    for proto in ("ll", "ll128"):
        W = car.ll_wire_bytes(proto, NUMEL * 2)
        wires = [torch.empty(W, dtype=torch.uint8, device="cuda") for _ in range(N)]
        car.ar_ll_pack(ins[:N - 1], wires[:N - 1], proto, 1)
        car.ar_ll_allreduce(ins[N - 1], wires, out, flags, proto, N - 1, 1)
        torch.cuda.synchronize()
        car.raise_on_status(flags, proto)
        check(out, idx, want, proto + " in one launch")
        del wires
        torch.cuda.empty_cache()


def test_two_shot_divisible_prefix(data):
    """The two-shot needs n whole 16-byte segments: the first 2^30 elements."""
    ins, idx, want = data
    m = 1 << 30
    keep = idx < m
    heads = [t[:m] for t in ins]
    segs = [torch.empty(m // N, dtype=torch.bfloat16, device="cuda") for _ in range(N)]
    outs = [torch.empty(m, dtype=torch.bfloat16, device="cuda") for _ in range(N)]
    flags = car.new_flags(N)
    car.ar_twoshot_rs(heads, segs, flags, 0, outs=outs)
    torch.cuda.synchronize()
    car.raise_on_status(flags)
    for r in range(N):
        check(outs[r], idx[keep], want[keep], f"two-shot rank {r}")
    # the same under LL: 1 GiB segments travel as 2 GiB wires (byte offsets past 2^31)
    del segs
    segw = [torch.zeros(car.ll_wire_bytes("ll", m // N * 2), dtype=torch.uint8, device="cuda") for _ in range(N)]
    for o in outs:
        o.zero_()
    car.ar_twoshot_ll(heads, segw, flags, 1, outs=outs)
    torch.cuda.synchronize()
    car.raise_on_status(flags)
    for r in range(N):
        check(outs[r], idx[keep], want[keep], f"two-shot under LL rank {r}")
    # under LL128: 1 GiB segments as 1.07 GiB wires of 128-byte lines
    del segw
    segw = [torch.zeros(car.ll_wire_bytes("ll128", m // N * 2), dtype=torch.uint8, device="cuda") for _ in range(N)]
    for o in outs:
        o.zero_()
    car.ar_twoshot_ll128(heads, segw, flags, 1, outs=outs)
    torch.cuda.synchronize()
    car.raise_on_status(flags)
    for r in range(N):
        check(outs[r], idx[keep], want[keep], f"two-shot under LL128 rank {r}")
    del segw
    # one rank's share with slots (the grid sized to the work) after its peer's
    # reduce-scatter: rank 1, whose segment starts past byte 2^31 of every input
    segs = [torch.empty(m // N, dtype=torch.bfloat16, device="cuda") for _ in range(N)]
    car.ar_twoshot_rs(heads, segs, flags, 2, r0=0, r1=1)
    outs[1].zero_()
    car.ar_twoshot_rs(heads, segs, flags, 2, r0=1, r1=2, outs=[None, outs[1]])
    torch.cuda.synchronize()
    car.raise_on_status(flags)
    check(outs[1], idx[keep], want[keep], "two-shot share of rank 1")
