"""Seeded randomized GPU parity across every path.

Each case draws a rank count, a size (ragged for the paths that accept any
size, divisible for the two-shot), a dtype and a value mix -- N(0,1) scaled by
a random power of two per rank, small integers, values near the overflow and
subnormal ranges, and a sprinkling of inf, NaN and -0 -- then compares with
the CPU oracle, bit for bit: the one-shot; the fused two-shot (every rank,
and one rank's share after its peers' reduce-scatters; slots, LL and LL128
segments); the two-shot split into a reduce-scatter and an all-gather on the
compute units or on the copy engines; the allocation-free entry point; the
reduce-broadcast; the push and staging copies; LL and LL128 (pack then
receiver, and one rank's send and receive in one launch).  The cases are
fixed by the seed."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

CASES = 100


def case(k):
    rng = np.random.default_rng(90_000 + k)
    n = int(rng.integers(2, 17))
    dt = "bf16" if rng.random() < 0.5 else "f32"
    per_vec = 8 if dt == "bf16" else 4
    if rng.random() < 0.5:  # divisible: every path including the two-shot
        numel = n * per_vec * int(rng.integers(1, 3000))
    else:  # ragged
        numel = int(rng.integers(1, 200_000))
    ins = synth.rank_inputs(n, numel, dt, "normal", config=900 + k)
    mix = rng.integers(0, 4)
    for r, a in enumerate(ins):
        if dt == "f32":
            if mix == 1:
                a[:] = synth.integers_f32(numel, synth.rank_seed(950 + k, r))
            elif mix == 2:
                a *= np.float32(2.0 ** int(rng.integers(-130, 120)))
            elif mix == 3:
                picks = rng.integers(0, numel, size=max(1, numel // 500))
                a[picks] = rng.choice(np.array([np.inf, -np.inf, np.nan, -0.0, 3.3e38, -3.3e38, 1e-44],
                                               np.float32), size=picks.size)
        else:
            if mix == 2:  # shift exponents up or down, keeping the bf16 bit pattern valid
                e = ((a >> 7) & 0xFF).astype(np.int32) + int(rng.integers(-100, 100))
                e = np.clip(e, 1, 254).astype(np.uint16)
                a[:] = (a & 0x807F) | (e << 7)
            elif mix == 3:
                picks = rng.integers(0, numel, size=max(1, numel // 500))
                a[picks] = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC1, 0x8000, 0x7F7F, 0xFF7F, 0x0001],
                                               np.uint16), size=picks.size)
    return n, dt, numel, ins


@pytest.mark.parametrize("k", range(CASES))
def test_random_case_every_path(k):
    n, dt, numel, host = case(k)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    tdt = ins[0].dtype
    es = 4 if dt == "f32" else 2
    label = f"case {k}: n={n} {dt} numel={numel}"

    out = torch.empty(numel, dtype=tdt, device="cuda")
    car.ar_oneshot(ins, out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), want), label + " one-shot"

    outs = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
    car.ar_reduce_bcast(ins, outs)
    torch.cuda.synchronize()
    for r in range(n):
        assert np.array_equal(bits(outs[r]), want), label + f" reduce-broadcast out[{r}]"

    # push: one rank's message to every output (a bit copy); staging copy: to one
    me = k % n
    car.ar_push([ins[me]], [outs])
    torch.cuda.synchronize()
    for r in range(n):
        assert np.array_equal(bits(outs[r]), oracle_bits(host[me])), label + f" push to out[{r}]"
    out.fill_(7)
    car.ar_push([ins[me]], [[out]])
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle_bits(host[me])), label + " staging copy"

    flags = car.new_flags(n)
    if numel % n == 0 and (numel // n * es) % 16 == 0:
        segs = [torch.empty(numel // n, dtype=tdt, device="cuda") for _ in range(n)]
        car.ar_twoshot_rs(ins, segs, flags, 1, outs=outs)
        torch.cuda.synchronize()
        car.raise_on_status(flags, label)
        for r in range(n):
            assert np.array_equal(bits(outs[r]), want), label + f" two-shot rank {r}"
        segw = [torch.zeros(car.ll_wire_bytes("ll", numel // n * es), dtype=torch.uint8, device="cuda")
                for _ in range(n)]
        car.ar_twoshot_ll(ins, segw, flags, 1, outs=outs)
        torch.cuda.synchronize()
        car.raise_on_status(flags, label)
        for r in range(n):
            assert np.array_equal(bits(outs[r]), want), label + f" two-shot under LL rank {r}"
        segw128 = [torch.zeros(car.ll_wire_bytes("ll128", numel // n * es), dtype=torch.uint8, device="cuda")
                   for _ in range(n)]
        car.ar_twoshot_ll128(ins, segw128, flags, 1, outs=outs)
        torch.cuda.synchronize()
        car.raise_on_status(flags, label)
        for r in range(n):
            assert np.array_equal(bits(outs[r]), want), label + f" two-shot under LL128 rank {r}"
        # one rank's share (the grid sized to the work) after the peers' reduce-scatters
        me = k % n
        for name, fn, seg in (("slots", car.ar_twoshot_rs, segs), ("LL", car.ar_twoshot_ll, segw),
                              ("LL128", car.ar_twoshot_ll128, segw128)):
            for r in range(n):
                if r != me:
                    fn(ins, seg, flags, 3, r0=r, r1=r + 1)
            out.fill_(7)
            fn(ins, seg, flags, 3, r0=me, r1=me + 1, outs=[out if r == me else None for r in range(n)])
            torch.cuda.synchronize()
            car.raise_on_status(flags, label)
            assert np.array_equal(bits(out), want), label + f" two-shot share of rank {me} with {name}"
        # split: every rank's reduce-scatter, then the all-gather on the compute
        # units, then again with the all-gather on the copy engines
        for name, ag in (("all-gather", car.ar_twoshot_ag), ("copy-engine all-gather", car.ar_twoshot_ag_copy)):
            step = 5 if ag is car.ar_twoshot_ag else 6
            for o in outs:
                o.fill_(7)
            car.ar_twoshot_rs(ins, segs, flags, step)
            ag(segs, outs, flags, step)
            torch.cuda.synchronize()
            car.raise_on_status(flags, label)
            for r in range(n):
                assert np.array_equal(bits(outs[r]), want), label + f" split two-shot ({name}) rank {r}"
        for o in outs:
            o.fill_(7)
        car.ar_twoshot_noalloc(ins, outs)
        torch.cuda.synchronize()
        for r in range(n):
            assert np.array_equal(bits(outs[r]), want), label + f" allocation-free two-shot rank {r}"

    for proto in ("ll", "ll128"):
        W = car.ll_wire_bytes(proto, numel * es)
        wires = [torch.empty(W, dtype=torch.uint8, device="cuda") for _ in range(n)]
        car.ar_ll_pack(ins, wires, proto, 2)
        (car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack)(wires, out, 2, flags)
        torch.cuda.synchronize()
        car.raise_on_status(flags, label)
        assert np.array_equal(bits(out), want), label + " " + proto
        # one rank's step in one launch over the same (already packed) peers' wires
        me = k % n
        out.zero_()
        car.ar_ll_allreduce(ins[me], wires, out, flags, proto, me, 2)
        torch.cuda.synchronize()
        car.raise_on_status(flags, label)
        assert np.array_equal(bits(out), want), label + f" {proto} in one launch, rank {me}"
