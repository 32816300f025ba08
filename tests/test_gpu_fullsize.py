"""GPU parity at the largest workload sizes (n = 16 ranks, 64 MiB per rank,
and n = 8 at 8 MiB), in the launch configurations bench.py times.  The oracle
computes sampled output elements one by one (the fold is per element, so the
oracle run on the sampled columns of every rank gives exactly those
outputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")


def sample_indices(numel: int, seed: int = 5) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = [np.arange(0, min(2048, numel)), np.arange(max(0, numel - 2048), numel),
            rng.integers(0, numel, 8192)]
    # around 16-byte-vector and segment boundaries
    for b in (numel // 16, numel // 8, numel // 2, 3 * numel // 4):
        pick.append(np.arange(max(0, b - 9), min(numel, b + 9)))
    return np.unique(np.concatenate(pick))


def expect_at(host, idx, dt):
    cols = [np.ascontiguousarray(a[idx]) for a in host]
    return oracle_bits(oracle.oneshot(cols, dt))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_n16_64MiB_per_rank_all_paths_sampled(dt):
    n = 16
    es = 4 if dt == "f32" else 2
    numel = (64 << 20) // es
    host = synth.rank_inputs(n, numel, dt, "normal", config=4)
    idx = sample_indices(numel)
    want = expect_at(host, idx, dt)
    ins = [to_dev(a) for a in host]
    del host
    tdt = ins[0].dtype
    flags = car.new_flags(n)
    car.set_poll_timeout_ns(200_000_000)
    try:
        out = torch.empty(numel, dtype=tdt, device="cuda")
        car.ar_oneshot(ins, out)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out)[idx], want), "one-shot"

        # two-shot, one rank's share (rank 0) with the peers published first
        segs = [torch.empty(numel // n, dtype=tdt, device="cuda") for _ in range(n)]
        for r in range(1, n):
            car.ar_twoshot_rs(ins, segs, flags, 1 << 31, r0=r, r1=r + 1)
        out.fill_(0)
        car.ar_twoshot_rs(ins, segs, flags, 1, r0=0, r1=1, outs=[out] + [None] * (n - 1))
        torch.cuda.synchronize()
        car.raise_on_status(flags)
        assert np.array_equal(bits(out)[idx], want), "two-shot share"

        for proto in ("ll", "ll128"):
            W = car.ll_wire_bytes(proto, numel * es)
            wires = [torch.empty(W, dtype=torch.uint8, device="cuda") for _ in range(n)]
            car.ar_ll_pack(ins, wires, proto, 3)
            out.fill_(0)
            (car.ar_ll_reduce_unpack if proto == "ll" else car.ar_ll128_reduce_unpack)(wires, out, 3, flags)
            torch.cuda.synchronize()
            car.raise_on_status(flags)
            assert np.array_equal(bits(out)[idx], want), proto
            # rank 9's step in one launch: its wire written, the other 15 read
            out.fill_(0)
            car.ar_ll_allreduce(ins[9], wires, out, flags, proto, 9, 3)
            torch.cuda.synchronize()
            car.raise_on_status(flags)
            assert np.array_equal(bits(out)[idx], want), proto + " in one launch"
            del wires

        # reduce-broadcast, rank 0's share and then the remaining ranks
        bouts = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
        car.ar_reduce_bcast(ins, bouts, 0, 1)
        car.ar_reduce_bcast(ins, bouts, 1, n)
        torch.cuda.synchronize()
        for j in (0, 7, n - 1):
            assert np.array_equal(bits(bouts[j])[idx], want), f"reduce-broadcast out[{j}]"
        # push of rank 5's message to every rank, sampled bytes equal
        car.ar_push([ins[5]], [bouts])
        torch.cuda.synchronize()
        src5 = bits(ins[5])[idx]
        for j in (0, n - 1):
            assert np.array_equal(bits(bouts[j])[idx], src5), f"push dst {j}"
        del bouts
    finally:
        car.set_poll_timeout_ns(0)


def test_n16_8MiB_full_emulation_two_shot_sampled():
    """All 16 ranks' two-shot in one persistent grid; every output sampled."""
    n, dt = 16, "bf16"
    numel = (8 << 20) // 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=4)
    idx = sample_indices(numel, seed=6)
    want = expect_at(host, idx, dt)
    ins = [to_dev(a) for a in host]
    segs = [torch.empty(numel // n, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    outs = [torch.empty(numel, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    flags = car.new_flags(n)
    car.ar_twoshot_rs(ins, segs, flags, 1, outs=outs)
    torch.cuda.synchronize()
    car.raise_on_status(flags)
    for r in range(n):
        assert np.array_equal(bits(outs[r])[idx], want), f"rank {r}"


def test_n16_64MiB_copy_engine_all_gather_and_auto_step_sampled():
    """One rank's reduce-scatter with an auto step id, then the copy-engine
    all-gather, at 64 MiB per rank; and the fused full emulation with auto
    step ids at 8 MiB, replayed twice without a reset."""
    n, dt = 16, "bf16"
    numel = (64 << 20) // 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=8)
    idx = sample_indices(numel, seed=9)
    want = expect_at(host, idx, dt)
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
        assert np.array_equal(bits(out)[idx], want), "copy-engine all-gather"
    finally:
        car.set_poll_timeout_ns(0)
    del ins, segs, out

    numel = (8 << 20) // 2
    host = synth.rank_inputs(n, numel, dt, "normal", config=10)
    idx = sample_indices(numel, seed=11)
    want = expect_at(host, idx, dt)
    ins = [to_dev(a) for a in host]
    segs = [torch.empty(numel // n, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    outs = [torch.zeros(numel, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    flags = car.new_flags(n)
    for rep in range(2):
        car.ar_twoshot_rs(ins, segs, flags, 0, outs=outs)
        torch.cuda.synchronize()
        car.raise_on_status(flags, f"auto step {rep}")
        for r in (0, 5, n - 1):
            assert np.array_equal(bits(outs[r])[idx], want), f"auto step {rep} rank {r}"
