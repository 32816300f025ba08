"""GPU parity of ar_oneshot against the CPU oracle, bit for bit."""
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


def run_oneshot(host_ins, dt):
    ins = [to_dev(a) for a in host_ins]
    numel = host_ins[0].size
    # output with a guard band of 64 elements after it, filled with a pattern
    buf = filled(numel + 64, DT[dt])
    out = buf[:numel]
    car.ar_oneshot(ins, out)
    torch.cuda.synchronize()
    guard = bits(buf[numel:])
    assert np.array_equal(guard, bits(filled(64, DT[dt]))), "write past the end of the output"
    return bits(out)


def test_small_n2_f32_integers_4096():
    """n = 2 ranks, 4096 fp32 integer values in [-8, 8]."""
    w = synth.WORKLOADS["oneshot_n2_f32_int_4096"]
    ins = synth.rank_inputs(w["n"], w["numel"], "f32", "int", config=w["config"])
    got = run_oneshot(ins, "f32")
    want = oracle_bits(oracle.oneshot(ins, "f32"))
    assert np.array_equal(got, want), first_mismatch(got, want)
    exact = (ins[0].astype(np.int64) + ins[1].astype(np.int64)).astype(np.float32)
    assert np.array_equal(got, exact.view(np.uint32))


def test_decode_n8_bf16_8x8192():
    """n = 8 ranks, bf16 [8 tokens x 8192 hidden] per rank, N(0,1)."""
    w = synth.WORKLOADS["oneshot_decode_n8_bf16_8x8192"]
    ins = synth.rank_inputs(w["n"], w["numel"], "bf16", "normal", config=w["config"])
    got = run_oneshot(ins, "bf16")
    want = oracle_bits(oracle.oneshot(ins, "bf16"))
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", list(range(2, 17)))
def test_all_rank_counts_ragged(n, dt):
    """Several workgroups' worth of vectors plus a partial last vector."""
    numel = 3 * 256 * 8 * 4 + 5
    ins = synth.rank_inputs(n, numel, dt, "normal", config=10 + n)
    got = run_oneshot(ins, dt)
    want = oracle_bits(oracle.oneshot(ins, dt))
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("numel", [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 255, 1024, 2047, 2048 * 8 + 1, 65536 + 7])
def test_sizes_and_tails(numel, dt):
    n = 5
    ins = synth.rank_inputs(n, numel, dt, "normal", config=20)
    got = run_oneshot(ins, dt)
    want = oracle_bits(oracle.oneshot(ins, dt))
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("ngpus", [2, 3, 8, 16])
def test_fill_pattern_closed_form(ngpus):
    """x_g[i] = g + i % 7 sums to ngpus(ngpus-1)/2 + ngpus*(i % 7) ("多 GPU 与 NCCL", NCCL 编程)."""
    numel = 7 * 4096 + 3
    for dt in ("f32", "bf16"):
        ins = synth.rank_inputs(ngpus, numel, dt, "fill", config=0)
        got = run_oneshot(ins, dt)
        i = np.arange(numel)
        expect = (ngpus * (ngpus - 1) / 2 + ngpus * (i % 7)).astype(np.float32)
        want = expect.view(np.uint32) if dt == "f32" else (expect.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(got, want)


def test_negative_zero_column_sums_to_plus_zero():
    ins = [np.full(40, -0.0, np.float32) for _ in range(3)]
    assert np.all(run_oneshot(ins, "f32") == 0)
    insb = [np.full(40, 0x8000, np.uint16) for _ in range(3)]
    assert np.all(run_oneshot(insb, "bf16") == 0)


def test_special_values_match_oracle():
    """Infinities, NaN, overflow to infinity, subnormals and ties in the bf16 rounding."""
    vals = np.array([np.inf, -np.inf, np.nan, 3.0e38, 1.0e-40, -1.0e-40, 1 + 2**-8, 1 + 3 * 2**-8, -0.0, 0.0,
                     2**-126, 65504.0, 1e30, -1e30], dtype=np.float32)
    rng = np.random.default_rng(3)
    numel = 4096
    ins = []
    for r in range(4):
        a = rng.choice(vals, numel).astype(np.float32)
        ins.append(a)
    got = run_oneshot(ins, "f32")
    want = oracle_bits(oracle.oneshot(ins, "f32"))
    nan_w = np.isnan(want.view(np.float32))
    assert np.array_equal(np.isnan(got.view(np.float32)), nan_w)
    assert np.array_equal(got[~nan_w], want[~nan_w])
    # bf16 output: the GPU's rounding must match the oracle's including NaN quieting
    insb = [oracle.f32_to_bf16(a) for a in ins]
    got = run_oneshot(insb, "bf16")
    want = oracle_bits(oracle.oneshot(insb, "bf16"))
    assert np.array_equal(got, want), first_mismatch(got, want)


def _split_into_three_bf16(x):
    """bf16 patterns a, b, c with ((0 + a) + b) + c == x exactly in fp32: a holds
    the top 8 significant bits of x, b the next 8, c the last 8.  Rows where a
    piece would fall below bf16's range are dropped."""
    def trunc(v):
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)

    def widen(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    xd = x.astype(np.float64)
    a = trunc(x)
    r1 = xd - widen(a)
    b = trunc(r1.astype(np.float32))
    r2 = r1 - widen(b)
    c = trunc(r2.astype(np.float32))
    ok = (widen(c) == r2) & (r1.astype(np.float32).astype(np.float64) == r1)
    return a[ok], b[ok], c[ok], x[ok]


def test_bf16_rounding_over_many_bit_patterns():
    """Build bf16 inputs whose fp32 fold equals a chosen fp32 value x, for x
    covering every 6-bit top-of-dropped-half pattern on 4096 mantissa/exponent
    tops (plus the exact ties), so the kernel's final rounding meets every
    rounding case; compare with the oracle bit for bit."""
    hi = np.arange(0x0C00, 0x7F00, 7, dtype=np.uint32)  # positive normal tops, exponent >= 2^-103
    lo = np.concatenate([np.arange(0, 1 << 16, 1024, dtype=np.uint32),
                         np.array([0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x0001], np.uint32)])
    u = (hi[:, None] << 16 | lo[None, :]).reshape(-1).astype(np.uint32)
    u = np.concatenate([u, u | 0x80000000])  # both signs
    x = u.view(np.float32)
    a, b, c, xs = _split_into_three_bf16(x)
    assert xs.size > 0.9 * x.size
    fold = oracle.bf16_to_f32(a) + oracle.bf16_to_f32(b) + oracle.bf16_to_f32(c)
    assert np.array_equal(fold.view(np.uint32), xs.view(np.uint32))  # the split is exact
    got = run_oneshot([a, b, c], "bf16")
    want = oracle_bits(oracle.oneshot([a, b, c], "bf16"))
    assert np.array_equal(got, want), first_mismatch(got, want)


def test_repeat_calls_are_bitwise_identical():
    n, numel = 8, 8 * 8192
    ins = synth.rank_inputs(n, numel, "bf16", "normal", config=1)
    dins = [to_dev(a) for a in ins]
    outs = [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(5)]
    for o in outs:
        car.ar_oneshot(dins, o)
    torch.cuda.synchronize()
    ref = bits(outs[0])
    for o in outs[1:]:
        assert np.array_equal(bits(o), ref)


def test_device_errors_raise():
    a = torch.zeros(1024 + 4, device="cuda")
    b = torch.zeros(1024 + 4, device="cuda")
    out = torch.zeros(1024, device="cuda")
    with pytest.raises(car.ArError) as e:
        car.ar_oneshot([a[1:1025], b[:1024]], out)  # 4-byte offset
    assert e.value.code == car.AR_ERR_ALIGN
    with pytest.raises(car.ArError) as e:
        car.ar_oneshot([a[:1024], b[:1024]], a[4:1028])  # output inside an input
    assert e.value.code == car.AR_ERR_ALIAS


# The one-shot takes 4-byte lanes below 512 KiB per rank and 8-byte lanes
# from there on; these sizes sit on both sides of that switch, with and
# without a partial last vector.
NARROW_MAX = 512 << 10


@pytest.mark.parametrize("dt, numel", [("f32", NARROW_MAX // 4 - 1), ("f32", NARROW_MAX // 4),
                                       ("f32", NARROW_MAX // 4 + 1), ("bf16", NARROW_MAX // 2 - 1),
                                       ("bf16", NARROW_MAX // 2), ("bf16", NARROW_MAX // 2 + 3)])
@pytest.mark.parametrize("n", [3, 16])
def test_either_side_of_the_lane_width_switch(dt, numel, n):
    ins = synth.rank_inputs(n, numel, dt, "normal", config=140 + n)
    got = run_oneshot(ins, dt)
    want = oracle_bits(oracle.oneshot(ins, dt))
    assert np.array_equal(got, want), first_mismatch(got, want)
