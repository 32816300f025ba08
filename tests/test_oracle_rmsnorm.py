"""Pins of the oracle's fused all-reduce + residual add + RMSNorm (O10).

The pages name the fused op without defining it; the oracle's reading is the
usual RMSNorm of the residual stream after the all-reduced sum is added to
it.  Each check here comes from somewhere other than that function's own
code: the one-shot fold (O2, pinned elsewhere) plus a numpy fp32 add for the
residual output, and closed forms for the normalized rows.  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth


def widen(a, dt):
    return a if dt == "f32" else oracle.bf16_to_f32(a)


def narrow(a, dt):
    a = np.asarray(a, np.float32)
    return a if dt == "f32" else oracle.f32_to_bf16(a)


def rows_of(values: np.ndarray, n: int, dt: str):
    """Rank inputs whose one-shot fold is exactly ``values`` (rank 0 carries
    them, the other ranks zeros) and a zero residual."""
    v = narrow(values.reshape(-1), dt)
    ins = [v] + [narrow(np.zeros(v.size), dt) for _ in range(n - 1)]
    return ins, narrow(np.zeros(v.size), dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 5, 8])
def test_residual_out_is_the_oneshot_fold_plus_residual(dt, n):
    hidden, rows = 96, 7
    ins = synth.rank_inputs(n, rows * hidden, dt, "normal", config=40 + n)
    res = synth.rank_inputs(1, rows * hidden, dt, "normal", config=60 + n)[0]
    w = synth.rank_inputs(1, hidden, dt, "normal", config=61)[0]
    got, _ = oracle.oneshot_rmsnorm(ins, res, w, hidden, 1e-6, dt)
    fold = oracle.oneshot([widen(a, dt) for a in ins], "f32")  # the rank-order fp32 fold
    want = narrow(fold + widen(res, dt), dt)                   # one more IEEE fp32 add, one rounding
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("c", [3.0, -0.5, 0.001])
def test_constant_row_normalizes_to_its_sign_times_weight(dt, c):
    hidden, rows = 37, 3
    ins, res = rows_of(np.full(rows * hidden, c), 4, dt)
    w = synth.rank_inputs(1, hidden, dt, "normal", config=62)[0]
    _, y = oracle.oneshot_rmsnorm(ins, res, w, hidden, 0.0, dt)
    want = np.tile(np.sign(c) * widen(w, dt).astype(np.float64), rows)
    assert np.allclose(y, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_eps_inside_the_root(dt):
    # constant row c with eps = c^2: y = sign(c) w / sqrt(2)
    hidden, c = 16, -2.0
    ins, res = rows_of(np.full(hidden, c), 3, dt)
    w = synth.rank_inputs(1, hidden, dt, "normal", config=63)[0]
    _, y = oracle.oneshot_rmsnorm(ins, res, w, hidden, c * c, dt)
    assert np.allclose(y, -widen(w, dt).astype(np.float64) / np.sqrt(2.0), rtol=1e-15, atol=0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_one_hot_row(dt):
    # h = a e_p: the root mean square is |a| / sqrt(H), so y_p = sign(a) sqrt(H) w_p, zeros elsewhere
    hidden, p, a = 50, 17, -6.0
    h = np.zeros(hidden)
    h[p] = a
    ins, res = rows_of(h, 2, dt)
    w = synth.rank_inputs(1, hidden, dt, "normal", config=64)[0]
    _, y = oracle.oneshot_rmsnorm(ins, res, w, hidden, 0.0, dt)
    want = np.zeros(hidden)
    want[p] = -np.sqrt(hidden) * float(widen(w, dt)[p])
    assert np.allclose(y, want, rtol=1e-15, atol=0)


def test_two_hot_row_uses_the_unrounded_sum():
    # bf16 ranks 1 and 2^-10 sum to 1 + 2^-10 in fp32, which bf16 cannot hold:
    # the row is normalized from that fp32 value, not from its rounding
    hidden = 8
    r0 = np.zeros(hidden, np.float32)
    r1 = np.zeros(hidden, np.float32)
    r0[0], r1[0] = 1.0, 2.0**-10
    r0[3] = 2.0
    ins = [oracle.f32_to_bf16(r0), oracle.f32_to_bf16(r1)]
    res = oracle.f32_to_bf16(np.zeros(hidden, np.float32))
    w = oracle.f32_to_bf16(np.ones(hidden, np.float32))
    ro, y = oracle.oneshot_rmsnorm(ins, res, w, hidden, 0.0, "bf16")
    a, b = 1.0 + 2.0**-10, 2.0
    rms = np.sqrt((a * a + b * b) / hidden)
    assert np.allclose(y[[0, 3]], [a / rms, b / rms], rtol=1e-15, atol=0)
    assert oracle.bf16_to_f32(ro)[0] == 1.0  # residual_out: the sum rounded once to bf16


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_normalized_rows_have_unit_rms(dt):
    hidden, rows = 256, 9
    ins = synth.rank_inputs(8, rows * hidden, dt, "normal", config=65)
    res = synth.rank_inputs(1, rows * hidden, dt, "normal", config=66)[0]
    w = narrow(np.ones(hidden), dt)
    _, y = oracle.oneshot_rmsnorm(ins, res, w, hidden, 0.0, dt)
    assert np.allclose((y.reshape(rows, hidden) ** 2).mean(axis=1), 1.0, rtol=1e-12, atol=0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_scaling_every_input_by_two_changes_nothing(dt):
    hidden, rows = 64, 5
    ins = synth.rank_inputs(4, rows * hidden, dt, "normal", config=67)
    res = synth.rank_inputs(1, rows * hidden, dt, "normal", config=68)[0]
    w = synth.rank_inputs(1, hidden, dt, "normal", config=69)[0]
    _, y1 = oracle.oneshot_rmsnorm(ins, res, w, hidden, 0.0, dt)
    dbl = lambda a: narrow(widen(a, dt) * np.float32(2.0), dt)  # exact: a power of two
    ro2, y2 = oracle.oneshot_rmsnorm([dbl(a) for a in ins], dbl(res), w, hidden, 0.0, dt)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_weight_scales_each_column(dt):
    hidden, rows = 40, 6
    ins = synth.rank_inputs(3, rows * hidden, dt, "normal", config=70)
    res = synth.rank_inputs(1, rows * hidden, dt, "normal", config=71)[0]
    w = synth.rank_inputs(1, hidden, dt, "normal", config=72)[0]
    _, y1 = oracle.oneshot_rmsnorm(ins, res, narrow(np.ones(hidden), dt), hidden, 1e-5, dt)
    _, yw = oracle.oneshot_rmsnorm(ins, res, w, hidden, 1e-5, dt)
    want = y1 * np.tile(widen(w, dt).astype(np.float64), rows)
    assert np.array_equal(yw, want)


def test_rows_are_independent():
    hidden, rows = 24, 4
    ins = synth.rank_inputs(2, rows * hidden, "f32", "normal", config=73)
    res = synth.rank_inputs(1, rows * hidden, "f32", "normal", config=74)[0]
    w = synth.rank_inputs(1, hidden, "f32", "normal", config=75)[0]
    ro1, y1 = oracle.oneshot_rmsnorm(ins, res, w, hidden, 1e-6, "f32")
    ins2 = [a.copy() for a in ins]
    ins2[1][2 * hidden:3 * hidden] *= np.float32(7.0)  # change row 2 only
    ro2, y2 = oracle.oneshot_rmsnorm(ins2, res, w, hidden, 1e-6, "f32")
    keep = np.r_[0:2 * hidden, 3 * hidden:rows * hidden]
    assert np.array_equal(y1[keep], y2[keep]) and np.array_equal(ro1[keep], ro2[keep])
    assert not np.array_equal(y1[2 * hidden:3 * hidden], y2[2 * hidden:3 * hidden])


def test_numel_must_be_whole_rows():
    ins = synth.rank_inputs(2, 100, "f32", "normal", config=76)
    with pytest.raises(ValueError):
        oracle.oneshot_rmsnorm(ins, ins[0].copy(), np.ones(30, np.float32), 30, 0.0, "f32")
