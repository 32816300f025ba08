"""The entry points captured into a HIP graph (as bench.py times them):
replay several times with the program's own eager work in between (new
inputs, synchronisations) and check every replay against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")


def test_graph_replays_of_every_path():
    n, numel, dt = 8, 8 * 8192, "bf16"
    datasets = [synth.rank_inputs(n, numel, dt, "normal", config=200 + k) for k in range(3)]
    wants = [oracle_bits(oracle.oneshot(h, dt)) for h in datasets]
    ins = [to_dev(a) for a in datasets[0]]
    tdt = ins[0].dtype
    S = numel * 2
    flags = car.new_flags(n)
    segs = [torch.empty(numel // n, dtype=tdt, device="cuda") for _ in range(n)]
    outs_full = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
    out_one = torch.empty(numel, dtype=tdt, device="cuda")
    out_share = torch.empty(numel, dtype=tdt, device="cuda")
    w_ll = [torch.empty(car.ll_wire_bytes("ll", S), dtype=torch.uint8, device="cuda") for _ in range(n)]
    w_128 = [torch.empty(car.ll_wire_bytes("ll128", S), dtype=torch.uint8, device="cuda") for _ in range(n)]
    out_ll = torch.empty(numel, dtype=tdt, device="cuda")
    out_128 = torch.empty(numel, dtype=tdt, device="cuda")
    w1_ll = [torch.empty(car.ll_wire_bytes("ll", S), dtype=torch.uint8, device="cuda") for _ in range(n)]
    w1_128 = [torch.empty(car.ll_wire_bytes("ll128", S), dtype=torch.uint8, device="cuda") for _ in range(n)]
    out1_ll = torch.empty(numel, dtype=tdt, device="cuda")
    out1_128 = torch.empty(numel, dtype=tdt, device="cuda")
    bc_full = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
    bc_share = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
    staging = [[torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)] for _ in range(n)]
    out_push = torch.empty(numel, dtype=tdt, device="cuda")
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        car.ar_oneshot(ins, out_one)
        # every rank in one grid: a reset captured first makes each replay's
        # barrier wait for that replay's own reduce-scatter
        car.ar_flag_barrier_reset(flags, n)
        car.ar_twoshot_rs(ins, segs, flags, 1, outs=outs_full)
        # rank 0's share after the peers' reduce-scatter of the same replay
        for r in range(1, n):
            car.ar_twoshot_rs(ins, segs, flags, 2, r0=r, r1=r + 1)
        car.ar_twoshot_rs(ins, segs, flags, 2, r0=0, r1=1, outs=[out_share] + [None] * (n - 1))
        car.ar_ll_pack(ins, w_ll, "ll", 2)
        car.ar_ll_reduce_unpack(w_ll, out_ll, 2, flags)
        car.ar_ll_pack(ins, w_128, "ll128", 2)
        car.ar_ll128_reduce_unpack(w_128, out_128, 2, flags)
        # rank 3's LL / LL128 step in one launch after the peers' packs
        peers = [r for r in range(n) if r != 3]
        car.ar_ll_pack([ins[r] for r in peers], [w1_ll[r] for r in peers], "ll", 2)
        car.ar_ll_allreduce(ins[3], w1_ll, out1_ll, flags, "ll", 3, 2)
        car.ar_ll_pack([ins[r] for r in peers], [w1_128[r] for r in peers], "ll128", 2)
        car.ar_ll_allreduce(ins[3], w1_128, out1_128, flags, "ll128", 3, 2)
        car.ar_reduce_bcast(ins, bc_full)
        for r in range(n):  # every rank's share, one launch each
            car.ar_reduce_bcast(ins, bc_share, r, r + 1)
        # one-shot push: sender i into slot i of every rank's staging buffer
        car.ar_push(ins, [[staging[j][i] for j in range(n)] for i in range(n)])
        car.ar_oneshot(staging[3], out_push)
    torch.cuda.synchronize()

    for rep in range(6):
        k = rep % 3
        for d, a in zip(ins, datasets[k]):  # eager work between replays
            d.copy_(to_dev(a))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert car.read_status(flags)[0] == 0, f"replay {rep}"
        for name, t in [("oneshot", out_one), ("share", out_share), ("ll", out_ll), ("ll128", out_128),
                        ("ll one launch", out1_ll), ("ll128 one launch", out1_128), ("push", out_push)] + [(f"full{r}", outs_full[r]) for r in range(n)] + \
                       [(f"bcast{r}", bc_full[r]) for r in range(n)] + [(f"bshare{r}", bc_share[r]) for r in range(n)]:
            assert np.array_equal(bits(t), wants[k]), f"replay {rep}: {name}"
