"""The allocation-free two-shot (ar_twoshot_noalloc), called through the C
ABI, against the allocating fused two-shot (ar_twoshot_rs with outputs, every
rank in one launch) on the same inputs: bit for bit, on calls in a row with
the second smaller than the first and the rank count changing, under graph
replay, and with a message above the scratch limit refused."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import synth
from devtensors import bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")
P = ctypes.c_void_p


def noalloc(ins, outs):
    """The entry point itself, through the C ABI (ctypes, plain pointers)."""
    n = len(ins)
    dt = 0 if ins[0].dtype == torch.float32 else 1
    return car.lib.ar_twoshot_noalloc((P * n)(*[t.data_ptr() for t in ins]), n,
                                      (P * n)(*[o.data_ptr() for o in outs]), ins[0].numel(), dt,
                                      P(torch.cuda.current_stream().cuda_stream))


def allocating(ins):
    """The existing entry point: fused two-shot of every rank, caller-owned
    segments and flag region."""
    n, numel = len(ins), ins[0].numel()
    segs = [torch.empty(numel // n, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    outs = [torch.empty(numel, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    flags = car.new_flags(n)
    car.ar_twoshot_rs(ins, segs, flags, 1, outs=outs)
    torch.cuda.synchronize()
    car.raise_on_status(flags, "allocating two-shot")
    return [bits(o) for o in outs]


def check(n, dt, numel, config):
    host = synth.rank_inputs(n, numel, dt, "normal", config=config)
    ins = [to_dev(a) for a in host]
    want = allocating(ins)
    outs = [torch.full((numel,), 3.0, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    assert noalloc(ins, outs) == car.AR_OK
    torch.cuda.synchronize()
    for r in range(n):
        got = bits(outs[r])
        assert np.array_equal(got, want[r]), f"n={n} {dt} numel={numel} rank {r}"


def test_calls_in_a_row_second_smaller():
    """8 MiB per rank (n = 8, bf16 [512 x 8192]), then 128 KiB per rank, then
    a larger n with fp32, then the largest message the scratch takes."""
    print("noalloc: n=8 bf16 [512 x 8192], then [8 x 8192]", flush=True)
    check(8, "bf16", 512 * 8192, config=900)
    check(8, "bf16", 8 * 8192, config=901)
    print("noalloc: n=16 fp32 1 MiB per rank, n=3 bf16, n=4 fp32 64 MiB per rank", flush=True)
    check(16, "f32", 1 << 18, config=902)
    check(3, "bf16", 3 * 8 * 97, config=903)
    check(4, "f32", (car.AR_NOALLOC_MAX_BYTES // 4) // 16 * 16, config=904)


def test_replayed_in_a_graph():
    """Captured once, replayed with new inputs between replays: every replay
    equals the allocating two-shot on that replay's inputs."""
    n, numel = 8, 8 * 4096
    data = [synth.rank_inputs(n, numel, "bf16", "normal", config=910 + k) for k in range(3)]
    ins = [to_dev(a) for a in data[0]]
    outs = [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    assert noalloc(ins, outs) == car.AR_OK  # first call on the device: eager
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert noalloc(ins, outs) == car.AR_OK
    torch.cuda.synchronize()
    for rep in range(5):
        for d, a in zip(ins, data[rep % 3]):
            d.copy_(to_dev(a))
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = allocating(ins)
        for r in range(n):
            assert np.array_equal(bits(outs[r]), want[r]), f"replay {rep} rank {r}"


def test_above_the_scratch_limit_is_refused():
    n = 2
    numel = car.AR_NOALLOC_MAX_BYTES // 4 + 8 * n
    ins = [torch.zeros(numel, dtype=torch.float32, device="cuda") for _ in range(n)]
    outs = [torch.full((numel,), 5.0, dtype=torch.float32, device="cuda") for _ in range(n)]
    torch.cuda.synchronize()
    assert noalloc(ins, outs) == car.AR_ERR_SIZE
    torch.cuda.synchronize()
    assert all(bool((o == 5.0).all()) for o in outs)
    assert "scratch" in car.lib.ar_status_string(car.AR_ERR_SIZE).decode()
