"""GPU parity at the largest configuration, n = 16 ranks with 64 MiB per rank
(fp32 and bf16), compared with the oracle element by element: the oracle's
one-shot runs on the full arrays (32 Mi bf16 / 16 Mi fp32 elements per
rank) and every output of every path is compared with it in full.  The
two-shot's segments equal the oracle's reduce-scatter, i.e. slices of the
one-shot result (pinned on the CPU: two-shot == one-shot bitwise).  Also
every rank's two-shot in one launch at n = 16, 8 MiB per rank, and the
copy-engine all-gather and auto step ids at 64 MiB."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, first_mismatch, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

N = 16
PEER = 1 << 31


@pytest.fixture(scope="module", params=["bf16", "f32"])
def big(request):
    """Device inputs of 16 ranks x 64 MiB and the oracle's full result."""
    dt = request.param
    es = 4 if dt == "f32" else 2
    numel = (64 << 20) // es
    print(f"fullsize: generating n={N} {dt} {numel} elements per rank", flush=True)
    host = synth.rank_inputs(N, numel, dt, "normal", config=4)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    del host
    yield dt, es, numel, ins, want
    del ins
    torch.cuda.empty_cache()


def same(t, want, what):
    got = bits(t)
    assert got.size == want.size
    assert np.array_equal(got, want), f"{what}: " + first_mismatch(got, want)


def test_oneshot_and_two_shot_shares(big):
    dt, es, numel, ins, want = big
    m = numel // N
    tdt = ins[0].dtype
    car.set_poll_timeout_ns(200_000_000)
    try:
        out = torch.full((numel,), 7, dtype=tdt, device="cuda")
        car.ar_oneshot(ins, out)
        torch.cuda.synchronize()
        same(out, want, "one-shot")
        # two-shot with slots: ranks 0 and 15 each take their share after the peers
        segs = [torch.empty(m, dtype=tdt, device="cuda") for _ in range(N)]
        flags = car.new_flags(N)
        for me in (0, N - 1):
            for r in range(N):
                if r != me:
                    car.ar_twoshot_rs(ins, segs, flags, PEER, r0=r, r1=r + 1)
            out.fill_(7)
            car.ar_twoshot_rs(ins, segs, flags, 1 + me, r0=me, r1=me + 1,
                              outs=[out if r == me else None for r in range(N)])
            torch.cuda.synchronize()
            car.raise_on_status(flags)
            same(out, want, f"two-shot share of rank {me}")
            same(segs[me], want[me * m:(me + 1) * m], f"segment {me}")
        del segs
        # the two-shot under LL and under LL128, rank 3's share
        for proto, fn in (("ll", car.ar_twoshot_ll), ("ll128", car.ar_twoshot_ll128)):
            W = car.ll_wire_bytes(proto, m * es)
            segw = [torch.zeros(W, dtype=torch.uint8, device="cuda") for _ in range(N)]
            fl = car.new_flags(N)
            for r in range(N):
                if r != 3:
                    fn(ins, segw, fl, PEER, r0=r, r1=r + 1)
            out.fill_(7)
            fn(ins, segw, fl, 5, r0=3, r1=4, outs=[out if r == 3 else None for r in range(N)])
            torch.cuda.synchronize()
            car.raise_on_status(fl)
            same(out, want, f"two-shot under {proto}, share of rank 3")
            wire3 = oracle.ll_pack(proto, np.ascontiguousarray(want[3 * m:4 * m]), 5)
            same(segw[3], wire3, f"{proto} segment wire of rank 3")
            del segw
    finally:
        car.set_poll_timeout_ns(0)


def test_ll_and_ll128_receivers_and_one_launch(big):
    """Above 16 MiB per rank the LL receiver and the one-launch LL take two
    lines per lane; both are compared in full here."""
    dt, es, numel, ins, want = big
    tdt = ins[0].dtype
    flags = car.new_flags(N)
    car.set_poll_timeout_ns(200_000_000)
    try:
        out = torch.empty(numel, dtype=tdt, device="cuda")
        for proto in ("ll", "ll128"):
            W = car.ll_wire_bytes(proto, numel * es)
            wires = [torch.zeros(W, dtype=torch.uint8, device="cuda") for _ in range(N)]
            car.ar_ll_pack(ins, wires, proto, 3)
            out.fill_(7)
            (car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack)(wires, out, 3, flags)
            torch.cuda.synchronize()
            car.raise_on_status(flags)
            same(out, want, f"{proto} receiver")
            # rank 9's step in one launch: its wire written, the other 15 read
            # (they carry step 3, so rank 9 runs step 3 too)
            out.fill_(7)
            wires[9].zero_()
            car.ar_ll_allreduce(ins[9], wires, out, flags, proto, 9, 3)
            torch.cuda.synchronize()
            car.raise_on_status(flags)
            same(out, want, f"{proto} sent and received in one launch")
            same(wires[9], oracle.ll_pack(proto, bits(ins[9]), 3), f"{proto} wire of rank 9")
            del wires
    finally:
        car.set_poll_timeout_ns(0)


def test_reduce_broadcast_push_and_no_alloc(big):
    dt, es, numel, ins, want = big
    tdt = ins[0].dtype
    bouts = [torch.full((numel,), 7, dtype=tdt, device="cuda") for _ in range(N)]
    car.ar_reduce_bcast(ins, bouts, 0, 1)
    car.ar_reduce_bcast(ins, bouts, 1, N)
    torch.cuda.synchronize()
    for j in range(N):
        same(bouts[j], want, f"reduce-broadcast out[{j}]")
    car.ar_push([ins[5]], [bouts])
    torch.cuda.synchronize()
    src5 = bits(ins[5])
    for j in (0, 8, N - 1):
        same(bouts[j], src5, f"push to rank {j}")
    for o in bouts:
        o.fill_(7)
    car.ar_twoshot_noalloc(ins, bouts)
    torch.cuda.synchronize()
    for j in (0, 8, N - 1):
        same(bouts[j], want, f"allocation-free two-shot out[{j}]")


def test_n16_8MiB_full_emulation_two_shot():
    """All 16 ranks' two-shot in one persistent grid; every output in full."""
    n, dt = 16, "bf16"
    numel = (8 << 20) // 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=4)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    segs = [torch.empty(numel // n, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    outs = [torch.empty(numel, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    flags = car.new_flags(n)
    car.ar_twoshot_rs(ins, segs, flags, 1, outs=outs)
    torch.cuda.synchronize()
    car.raise_on_status(flags)
    for r in range(n):
        same(outs[r], want, f"rank {r}")


def test_n16_64MiB_copy_engine_all_gather_and_auto_step():
    """One rank's reduce-scatter with auto step ids, then the copy-engine
    all-gather, at 64 MiB per rank; and the fused full emulation with auto
    step ids at 8 MiB, replayed twice without a reset; outputs in full."""
    n, dt = 16, "bf16"
    numel = (64 << 20) // 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=8)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    del host
    segs = [torch.empty(numel // n, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    out = torch.zeros(numel, dtype=ins[0].dtype, device="cuda")
    flags = car.new_flags(n)
    car.set_poll_timeout_ns(200_000_000)
    try:
        for r in range(n):
            car.ar_twoshot_rs(ins, segs, flags, 0, r0=r, r1=r + 1)
        car.ar_twoshot_ag_copy(segs, [out] + [None] * (n - 1), flags, 0, r0=0, r1=1)
        torch.cuda.synchronize()
        car.raise_on_status(flags)
        same(out, want, "copy-engine all-gather")
    finally:
        car.set_poll_timeout_ns(0)
    del ins, segs, out

    numel = (8 << 20) // 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=10)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    segs = [torch.empty(numel // n, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    outs = [torch.zeros(numel, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    flags = car.new_flags(n)
    for rep in range(2):
        car.ar_twoshot_rs(ins, segs, flags, 0, outs=outs)
        torch.cuda.synchronize()
        car.raise_on_status(flags, f"auto step {rep}")
        for r in range(n):
            same(outs[r], want, f"auto step {rep} rank {r}")
