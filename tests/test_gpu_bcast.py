"""GPU parity of the store-side variants against the CPU oracle, bit for bit:
ar_reduce_bcast (every output = the one-shot sum; a rank's share writes only
its own vector range of every output) and ar_push (every destination = the
source bytes; with ar_oneshot over the staging slots, the one-shot push)."""
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
PER_VEC = {"f32": 4, "bf16": 8}
GUARD = 64


def guarded(numel, dt, count):
    """count outputs, each followed by a guard band, all filled with a pattern."""
    bufs = [filled(numel + GUARD, DT[dt]) for _ in range(count)]
    return bufs, [b[:numel] for b in bufs]


def pattern(numel, dt):
    return bits(filled(numel, DT[dt]))


def owned(numel, dt, n, r0, r1):
    """Element range [lo, hi) that ranks [r0, r1) write: whole 16-byte vectors
    split floor(r * V / n), plus the partial last vector for the last rank."""
    V = numel // PER_VEC[dt]
    lo, hi = V * r0 // n * PER_VEC[dt], V * r1 // n * PER_VEC[dt]
    if r1 == n:
        hi = numel
    return lo, hi


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", list(range(2, 17)))
def test_full_broadcast_every_output_is_the_sum(n, dt):
    numel = 3 * 128 * 8 * n + 5  # several workgroups per rank and a partial vector
    host = synth.rank_inputs(n, numel, dt, "normal", config=400 + n)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    bufs, outs = guarded(numel, dt, n)
    car.ar_reduce_bcast(ins, outs)
    torch.cuda.synchronize()
    for j in range(n):
        got = bits(outs[j])
        assert np.array_equal(got, want), f"out[{j}]: " + first_mismatch(got, want)
        assert np.array_equal(bits(bufs[j][numel:]), pattern(GUARD, dt)), f"out[{j}] guard"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("numel", [1, 3, 7, 8, 9, 15, 16, 17, 100, 1000, 4095, 4096, 4097, 65536 + 3])
def test_sizes_and_tails(numel, dt):
    n = 5
    host = synth.rank_inputs(n, numel, dt, "normal", config=430)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    bufs, outs = guarded(numel, dt, n)
    car.ar_reduce_bcast(ins, outs)
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits(outs[j]), want), f"numel {numel} out[{j}]"
        assert np.array_equal(bits(bufs[j][numel:]), pattern(GUARD, dt))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n,numel", [(8, 8 * 8192), (3, 1000 * 8 + 3), (16, 16 * 8 * 5), (16, 40)])
def test_one_rank_share_writes_only_its_range(n, numel, dt):
    """Each [r, r+1) launch alone writes exactly its owned range of every
    output; the n shares together give the full result."""
    host = synth.rank_inputs(n, numel, dt, "normal", config=440 + n)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    pat = pattern(numel, dt)
    for r in range(n):
        bufs, outs = guarded(numel, dt, n)
        car.ar_reduce_bcast(ins, outs, r, r + 1)
        torch.cuda.synchronize()
        lo, hi = owned(numel, dt, n, r, r + 1)
        for j in range(n):
            got = bits(outs[j])
            assert np.array_equal(got[lo:hi], want[lo:hi]), f"rank {r} out[{j}]"
            assert np.array_equal(got[:lo], pat[:lo]) and np.array_equal(got[hi:], pat[hi:]), \
                f"rank {r} wrote outside [{lo}, {hi}) of out[{j}]"
            assert np.array_equal(bits(bufs[j][numel:]), pattern(GUARD, dt))
    bufs, outs = guarded(numel, dt, n)
    for r in range(n):
        car.ar_reduce_bcast(ins, outs, r, r + 1)
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits(outs[j]), want)


def test_rank_ranges_compose():
    n, numel, dt = 7, 7 * 8 * 300 + 6, "bf16"
    host = synth.rank_inputs(n, numel, dt, "normal", config=450)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    bufs, outs = guarded(numel, dt, n)
    for r0, r1 in [(0, 2), (2, 3), (3, 7)]:
        car.ar_reduce_bcast(ins, outs, r0, r1)
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits(outs[j]), want)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_special_values_match_the_oneshot(dt):
    n, numel = 4, 4096
    host = synth.rank_inputs(n, numel, dt, "normal", config=460)
    for a in host:  # infinities, NaN, -0 and huge values in a few places
        if dt == "f32":
            a[:8] = np.array([np.inf, -np.inf, np.nan, -0.0, 3e38, -3e38, 1e-45, 0.0], np.float32)
        else:
            a[:8] = np.array([0x7F80, 0xFF80, 0x7FC1, 0x8000, 0x7F7F, 0xFF7F, 0x0001, 0x0000], np.uint16)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    bufs, outs = guarded(numel, dt, n)
    car.ar_reduce_bcast(ins, outs)
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits(outs[j]), want)


# ------------------------------------------------------------------ push ------
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("numel", [1, 5, 8, 9, 1000, 4097, 128 * 8 * 3 + 7])
@pytest.mark.parametrize("ndst", [1, 2, 7, 16])
def test_push_copies_bytes_exactly(numel, ndst, dt):
    host = synth.rank_inputs(2, numel, dt, "normal", config=470)
    srcs = [to_dev(a) for a in host]
    rows = [guarded(numel, dt, ndst) for _ in srcs]
    car.ar_push(srcs, [r[1] for r in rows])
    torch.cuda.synchronize()
    for i, (bufs, dsts) in enumerate(rows):
        for j in range(ndst):
            assert np.array_equal(bits(dsts[j]), oracle_bits(host[i])), f"sender {i} dst {j}"
            assert np.array_equal(bits(bufs[j][numel:]), pattern(GUARD, dt))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 5, 8, 16])
def test_oneshot_push_all_reduce(n, dt):
    """Every rank pushes its input into its slot of every rank's staging
    buffer; every rank's one-shot over its own slots gives the sum."""
    numel = 8 * 8192 + 3
    es = 4 if dt == "f32" else 2
    stride = -(-numel * es // 16) * 16 // es  # slots start on 16-byte boundaries
    host = synth.rank_inputs(n, numel, dt, "normal", config=480 + n)
    want = oracle_bits(oracle.oneshot(host, dt))
    ins = [to_dev(a) for a in host]
    staging = [torch.empty(n * stride, dtype=DT[dt], device="cuda") for _ in range(n)]
    slot = lambda j, i: staging[j][i * stride:i * stride + numel]  # noqa: E731
    car.ar_push(ins, [[slot(j, i) for j in range(n)] for i in range(n)])
    outs = [torch.empty(numel, dtype=DT[dt], device="cuda") for _ in range(n)]
    for j in range(n):
        car.ar_oneshot([slot(j, i) for i in range(n)], outs[j])
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits(outs[j]), want), f"rank {j}"


# --------------------------------------------------------- synchronous errors --
def test_errors_are_reported_before_launch():
    n, numel = 4, 4096
    ins = [torch.zeros(numel, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    outs = [torch.zeros(numel, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    with pytest.raises(car.ArError) as e:
        car.ar_reduce_bcast(ins, [ins[0]] + outs[1:])
    assert e.value.code == car.AR_ERR_ALIAS
    with pytest.raises(car.ArError) as e:
        car.ar_reduce_bcast(ins, [outs[0]] * n)
    assert e.value.code == car.AR_ERR_ALIAS
    with pytest.raises(car.ArError) as e:
        car.ar_reduce_bcast(ins, outs, 2, 2)
    assert e.value.code == car.AR_ERR_ARG
    with pytest.raises(car.ArError) as e:
        shifted = torch.zeros(numel + 1, dtype=torch.bfloat16, device="cuda")[1:]
        car.ar_reduce_bcast(ins, [shifted] + outs[1:])
    assert e.value.code == car.AR_ERR_ALIGN
    with pytest.raises(car.ArError) as e:
        car.ar_push([ins[0]], [[outs[0], outs[0]]])
    assert e.value.code == car.AR_ERR_ALIAS
    with pytest.raises(car.ArError) as e:
        car.ar_push([ins[0]], [[]])
    assert e.value.code == car.AR_ERR_ARG
    with pytest.raises(car.ArError) as e:
        car.ar_push([ins[0]], [[outs[0], ins[0]]])
    assert e.value.code == car.AR_ERR_ALIAS
