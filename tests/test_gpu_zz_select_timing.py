"""The algorithm selector against live timings: at sync cost 0 (all ranks on
one GPU) the algorithm it picks must time within 30% (plus 0.5 us of launch
jitter) of the fastest of the eight, measured here the way its table was
measured (one GPU's share, buffer sets rotated over 512 MiB, graph-replayed
launches)."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

PEER = 1 << 31


def share_calls(n, numel, flags, gen):
    bf = torch.bfloat16
    S = numel * 2
    W1, W2 = car.ll_wire_bytes("ll", S), car.ll_wire_bytes("ll128", S)
    src = [torch.randn(numel, generator=gen, device="cuda").to(bf) for _ in range(n)]
    fp = n * S + 5 * S + n * (W1 + W2) + (3 * n - 1) * S + n * (car.ll_wire_bytes("ll128", S // n) + 2 * S // n)
    calls = {a: [] for a in car.ALGOS}
    keep = []
    for _ in range(max(2, -(-(512 << 20) // fp))):
        ins = [t.clone() for t in src]
        segs = [torch.empty(numel // n, dtype=bf, device="cuda") for _ in range(n)]
        out = torch.empty(numel, dtype=bf, device="cuda")
        w1 = [torch.empty(W1, dtype=torch.uint8, device="cuda") for _ in range(n)]
        w2 = [torch.empty(W2, dtype=torch.uint8, device="cuda") for _ in range(n)]
        slots0 = [torch.empty(numel, dtype=bf, device="cuda") for _ in range(n)]  # rank 0's push targets
        mine = [slots0[0]] + [torch.empty(numel, dtype=bf, device="cuda") for _ in range(1, n)]
        bouts = [out] + [torch.empty(numel, dtype=bf, device="cuda") for _ in range(1, n)]
        segw = [torch.zeros(car.ll_wire_bytes("ll", numel // n * 2), dtype=torch.uint8, device="cuda")
                for _ in range(n)]
        segw128 = [torch.zeros(car.ll_wire_bytes("ll128", numel // n * 2), dtype=torch.uint8, device="cuda")
                   for _ in range(n)]
        keep.append((ins, segs, out, w1, w2, slots0, mine, bouts, segw, segw128))
        for r in range(1, n):
            car.ar_twoshot_rs(ins, segs, flags, PEER, r0=r, r1=r + 1)
            car.ar_twoshot_ll(ins, segw, flags, PEER, r0=r, r1=r + 1)
            car.ar_twoshot_ll128(ins, segw128, flags, PEER, r0=r, r1=r + 1)
        car.ar_ll_pack(ins[1:], w1[1:], "ll", PEER)
        car.ar_ll_pack(ins[1:], w2[1:], "ll128", PEER)
        one = car.prepare_oneshot(ins, out)
        calls["oneshot"].append(lambda s, one=one: one())
        calls["twoshot"].append(car.prepare_twoshot_rs(ins, segs, flags, 0, 1, [out] + [None] * (n - 1)))
        for name, w in (("ll", w1), ("ll128", w2)):
            calls[name].append(car.prepare_ll_allreduce(ins[0], w, out, flags, name, 0))
        ps, po = car.prepare_push([ins[0]], [slots0]), car.prepare_oneshot(mine, out)
        calls["push"].append(lambda s, ps=ps, po=po: (ps(), po()))
        bc = car.prepare_reduce_bcast(ins, bouts, 0, 1)
        calls["bcast"].append(lambda s, bc=bc: bc())
        calls["twoshot_ll"].append(car.prepare_twoshot_ll(ins, segw, flags, 0, 1, [out] + [None] * (n - 1)))
        calls["twoshot_ll128"].append(car.prepare_twoshot_ll128(ins, segw128, flags, 0, 1,
                                                                [out] + [None] * (n - 1)))
    return calls, keep


def time_us(calls, K):
    m = len(calls)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            calls[i % m](1 + i)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e3 / K)
    return best


@pytest.mark.parametrize("n", [4, 8, 16])
@pytest.mark.parametrize("S", [64 << 10, 2 << 20, 16 << 20])
def test_selected_algorithm_is_near_the_fastest(n, S):
    numel = S // 2
    numel -= numel % (8 * n)
    flags = car.new_flags(n)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7 * n + S.bit_length())
    car.set_poll_timeout_ns(50_000_000)
    try:
        calls, keep = share_calls(n, numel, flags, gen)
        torch.cuda.synchronize()
        K = int(min(200, max(16, 0.004 * 4e12 / ((n + 1) * numel * 2))))
        t = {a: time_us(calls[a], K) for a in car.ALGOS}
        car.raise_on_status(flags)
    finally:
        car.set_poll_timeout_ns(0)
    pick = car.select_algo(n, numel, torch.bfloat16)
    print(f"n={n} S={numel * 2}: " + ", ".join(f"{a} {v:.2f} us" for a, v in t.items()) + f"; selected {pick}")
    assert t[pick] <= 1.3 * min(t.values()) + 0.5, (pick, t)
