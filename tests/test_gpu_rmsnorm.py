"""Parity of the fused one-shot all-reduce + residual add + RMSNorm
(ar_oneshot_rmsnorm) with the oracle (O10).

residual_out is compared bit for bit.  out is fp32 arithmetic on the device
whose sum of squares is taken in another order than the oracle's fp64 sum,
so it is compared with the oracle's unrounded fp64 value y, to a tolerance
derived from that arithmetic: the device's sum of squares is a sequential
sum of at most 32 terms per lane followed by a 6-level shuffle tree and a
4-level workgroup tree, 42 fp32 roundings deep, so its relative error is at
most 42 * 2^-24 = 2.5e-6; the root, the division and the two products add
four more roundings, and the factor's error is half the sum's, so the fp32
result is within about 1.5e-6 of y, relatively.  With REL = 4e-6 (that
bound with a margin):
  bf16: |out - y| <= ulp(out) / 2 + REL |y|, i.e. out is the correctly
        rounded y except where y lies within REL |y| of a rounding midpoint;
  fp32: |out - y| <= REL |y|.
Zeros (a row of zeros) must come out as zeros."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

REL = 4e-6


def host_values(t: torch.Tensor, dt: str) -> np.ndarray:
    b = bits(t)
    return b.view(np.float32).astype(np.float64) if dt == "f32" else \
        (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def check_out(got: np.ndarray, y: np.ndarray, dt: str, what: str):
    err = np.abs(got - y)
    if dt == "f32":
        bound = REL * np.abs(y)
    else:
        # spacing of bf16 values at |got|: 2^(exponent - 7); the smallest normal's below it
        e = np.floor(np.log2(np.maximum(np.abs(got), 2.0**-126)))
        bound = np.exp2(e - 7) / 2 + REL * np.abs(y)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{what}: {bad.size} elements outside the bound, first {bad[0]}: "
                           f"got {got[bad[0]]!r}, oracle {y[bad[0]]!r}")


def run_case(n, dt, rows, hidden, eps, config, in_place=False, ws=None):
    numel = rows * hidden
    host = synth.rank_inputs(n, numel, dt, "normal", config=config)
    res = synth.rank_inputs(1, numel, dt, "normal", config=config + 1000)[0]
    w = synth.rank_inputs(1, hidden, dt, "normal", config=config + 2000)[0]
    want_ro, y = oracle.oneshot_rmsnorm(host, res, w, hidden, eps, dt)
    ins = [to_dev(a) for a in host]
    d_res, d_w = to_dev(res), to_dev(w)
    d_ro = d_res if in_place else torch.empty_like(d_res)
    d_out = torch.empty_like(d_res)
    car.ar_oneshot_rmsnorm(ins, d_res, d_w, d_ro, d_out, eps, workspace=ws)
    torch.cuda.synchronize()
    what = f"n={n} {dt} rows={rows} hidden={hidden} eps={eps}{' in place' if in_place else ''}" \
           f"{' with a workspace' if ws is not None else ''}"
    if ws is not None:
        assert car.read_status(ws) == (0, 0), what
    assert np.array_equal(bits(d_ro), oracle_bits(want_ro)), f"{what}: residual_out differs from the oracle"
    check_out(host_values(d_out, dt), y, dt, what)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
@pytest.mark.parametrize("rows, hidden", [(1, 8), (3, 264), (7, 1000), (5, 4096), (2, 8192)])
def test_matches_the_oracle(n, dt, rows, hidden):
    run_case(n, dt, rows, hidden, 1e-6, config=300 + n)


@pytest.mark.parametrize("dt, hidden", [("bf16", 16384), ("bf16", 32768), ("f32", 8192), ("f32", 16384),
                                        ("bf16", 8200), ("f32", 4100)])
@pytest.mark.parametrize("n", [4, 16])
def test_rows_of_several_vectors_per_lane(n, dt, hidden):
    # more than 1024 vectors per row: two or four per lane
    run_case(n, dt, 3, hidden, 1e-5, config=320 + n)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_residual_updated_in_place(dt):
    run_case(8, dt, 6, 2048, 1e-6, config=330, in_place=True)


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.1, 10.0])
def test_eps(eps):
    run_case(4, "bf16", 4, 512, eps, config=331)


def test_prefill_and_decode_shapes():
    # hidden 8192: the prefill message (512 tokens) and the decode message (8 tokens), n = 8 bf16
    run_case(8, "bf16", 512, 8192, 1e-6, config=340)
    run_case(8, "bf16", 8, 8192, 1e-6, config=341)


def test_more_rows_than_workgroups():
    # above 2^20 rows the workgroups stride over the rows
    run_case(2, "bf16", (1 << 20) + 3, 8, 1e-6, config=342)


def test_zero_rows_stay_zero():
    n, hidden = 3, 64
    ins = [torch.zeros(2 * hidden, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    res = torch.zeros(2 * hidden, dtype=torch.bfloat16, device="cuda")
    res[hidden:] = 1.0  # row 1 constant: normalizes to (1 / sqrt(1 + eps)) * weight, 0.5 in bf16
    w = torch.full((hidden,), 0.5, dtype=torch.bfloat16, device="cuda")
    ro, out = torch.empty_like(res), torch.empty_like(res)
    car.ar_oneshot_rmsnorm(ins, res, w, ro, out, 1e-6)  # row 0: 0 * (1 / sqrt(eps)) = 0
    torch.cuda.synchronize()
    got = out.float().cpu()
    assert torch.equal(got[:hidden], torch.zeros(hidden))
    assert torch.equal(got[hidden:], torch.full((hidden,), 0.5))


def test_size_checks_before_launch():
    x = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        car.ar_oneshot_rmsnorm([x, x[:32]], x, w, torch.empty_like(x), torch.empty_like(x))
    with pytest.raises(ValueError):
        car.ar_oneshot_rmsnorm([x, x], x, torch.zeros(24, dtype=torch.bfloat16, device="cuda"),
                               torch.empty_like(x), torch.empty_like(x))
    with pytest.raises(car.ArError):
        car.ar_oneshot_rmsnorm([x, x], x, torch.zeros(4, dtype=torch.bfloat16, device="cuda"),
                               torch.empty_like(x), torch.empty_like(x))  # 8-byte rows


# ---- the few-rows path: parts of a row on a fixed grid, through a workspace --
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 8, 16])
@pytest.mark.parametrize("rows, hidden", [(1, 8), (3, 264), (7, 1000), (8, 8192), (32, 8192), (5, 32768),
                                          (64, 8192)])
def test_with_a_workspace_matches_the_oracle(n, dt, rows, hidden):
    # the parts path: rows of at least 128 KiB over the n + 1 streams, at most 512 parts
    # (n >= 8 at hidden 8192 bf16 up to 32 rows, fp32 up to 16, hidden 32768 bf16 up to 8);
    # every other case takes a workgroup per row.  The longest fp32 row (64 KiB) is 16384
    # elements.
    if dt == "f32" and hidden == 32768:
        hidden = 16384
    ws = car.new_rmsnorm_workspace()
    run_case(n, dt, rows, hidden, 1e-6, config=350 + n, ws=ws)


def test_workspace_calls_in_a_row_with_changing_shapes():
    # every call advances every workgroup's epoch: calls of any shape, on either
    # kernel, keep the epochs in step
    ws = car.new_rmsnorm_workspace()
    shapes = [(8, 8192), (3, 8192), (64, 8192), (200, 4096), (1, 256), (2, 32768), (8, 8192), (33, 8192), (8, 8192)]
    for i, (rows, hidden) in enumerate(shapes * 3):
        run_case(8, "bf16", rows, hidden, 1e-6, config=360 + i, ws=ws)


def test_workspace_path_replayed_in_a_graph():
    n, rows, hidden, dt = 8, 8, 8192, "bf16"
    ws = car.new_rmsnorm_workspace()
    numel = rows * hidden
    w = synth.rank_inputs(1, hidden, dt, "normal", config=370)[0]
    d_w = to_dev(w)
    ins = [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    d_res, d_ro, d_out = (torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    call = car.prepare_oneshot_rmsnorm(ins, d_res, d_w, d_ro, d_out, 1e-6, workspace=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(6):
        host = synth.rank_inputs(n, numel, dt, "normal", config=371 + rep)
        res = synth.rank_inputs(1, numel, dt, "normal", config=380 + rep)[0]
        for t, a in zip(ins, host):
            t.copy_(to_dev(a))
        d_res.copy_(to_dev(res))
        if rep % 2:
            call()  # an eager call between replays on the same workspace
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_ro, y = oracle.oneshot_rmsnorm(host, res, w, hidden, 1e-6, dt)
        assert np.array_equal(bits(d_ro), oracle_bits(want_ro)), f"replay {rep}"
        check_out(host_values(d_out, dt), y, dt, f"replay {rep}")
    assert car.read_status(ws) == (0, 0)


def test_a_part_whose_siblings_never_reach_its_step_times_out():
    # forced from the host: one workgroup's epoch jumps ahead, so its step id is
    # one its siblings never write; its bounded wait ends and is reported
    n, rows, hidden = 8, 2, 8192  # 16 parts per row; workgroup 21 is part 5 of row 1
    ws = car.new_rmsnorm_workspace()
    ws[32 + 21] = 1000
    numel = rows * hidden
    ins = [torch.ones(numel, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    res, w = torch.zeros(numel, dtype=torch.bfloat16, device="cuda"), torch.ones(hidden, dtype=torch.bfloat16,
                                                                                   device="cuda")
    ro, out = torch.empty_like(res), torch.full_like(res, -1.0)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(1_000_000)
    try:
        car.ar_oneshot_rmsnorm(ins, res, w, ro, out, 1e-6, workspace=ws)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    word, detail = car.read_status(ws)
    code, phase, _ = car.decode_status(word)
    assert (code, phase, detail) == (car.AR_ERR_TIMEOUT, car.PHASE_RMSNORM, 1)
    got = out.float().cpu()
    # row 0 and the other parts of row 1 are normalized (constant 8 -> 1); part 5 of row 1 is not written
    assert torch.equal(got[:hidden], torch.ones(hidden))
    part = got[hidden + 5 * 512: hidden + 6 * 512]
    assert torch.equal(part, torch.full((512,), -1.0))
    rest = torch.cat([got[hidden: hidden + 5 * 512], got[hidden + 6 * 512:]])
    assert torch.equal(rest, torch.ones(rest.numel()))
