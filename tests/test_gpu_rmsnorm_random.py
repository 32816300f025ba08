"""Seeded random cases of the fused all-reduce + residual add + RMSNorm, both
forms: each case draws its rank count, rows (a multiple of the rank count),
row length (whole 16-byte vectors, up to the 64 KiB row), data type, eps, the
value distribution (normal, or small integers whose sums are exact), and,
for the one-shot form, whether residual_out is the residual itself and
whether a workspace is given; the two-shot form runs every rank's
reduce-scatter and then every rank's share with explicit step ids, or, with
auto step ids (step 0: ids kept in the segments, one reduce-scatter per rank
per step), the peers' reduce-scatters and then rank 0's share.  residual_out is compared with
the oracle bit for bit and out with the oracle's fp64 value within the bound
derived in test_gpu_rmsnorm.py; where both forms take the same kind of path
(a workgroup per row, or parts of rows), their outputs must agree bit for
bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev
from test_gpu_rmsnorm import check_out, host_values

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

CASES = 60


def draw(i):
    rng = np.random.default_rng(9000 + i)
    n = int(rng.integers(2, 17))
    dt = "bf16" if rng.random() < 0.6 else "f32"
    per_vec = 8 if dt == "bf16" else 4
    max_vecs = 4096
    vecs = int(rng.choice([1, 3, 33, 64, 100, 512, 1000, 1024, 1025, 2048, 3000, max_vecs]))
    hidden = vecs * per_vec
    groups = int(rng.integers(1, 5))
    rows = n * groups
    eps = float(rng.choice([0.0, 1e-6, 1e-5, 0.5]))
    kind = "int" if rng.random() < 0.3 else "normal"
    in_place = bool(rng.random() < 0.3)
    ws = bool(rng.random() < 0.6)
    auto = bool(rng.random() < 0.5)
    return n, dt, rows, hidden, eps, kind, in_place, ws, auto


@pytest.mark.parametrize("i", range(CASES))
def test_random_case(i):
    n, dt, rows, hidden, eps, kind, in_place, use_ws, auto = draw(i)
    numel = rows * hidden
    what = f"case {i}: n={n} {dt} rows={rows} hidden={hidden} eps={eps} {kind}" \
           f"{' in place' if in_place else ''}{' workspace' if use_ws else ''}{' auto ids' if auto else ''}"
    print(what, flush=True)
    host = synth.rank_inputs(n, numel, dt, kind, config=9100 + i)
    res = synth.rank_inputs(1, numel, dt, kind, config=9200 + i)[0]
    w = synth.rank_inputs(1, hidden, dt, "normal", config=9300 + i)[0]
    if kind == "int" and eps == 0.0:
        eps = 1e-6  # an all-zero integer row would divide by zero
    want_ro, y = oracle.oneshot_rmsnorm(host, res, w, hidden, eps, dt)
    ins = [to_dev(a) for a in host]
    d_w = to_dev(w)

    v = hidden * (4 if dt == "f32" else 2) // 16
    heavy = (n + 1) * v * 16 >= 128 << 10
    one_parts = use_ws and heavy and rows * -(-v // 64) <= 512
    two_parts = heavy and rows // n < 256

    # one-shot form
    d_res = to_dev(res)
    d_ro = d_res if in_place else torch.empty_like(d_res)
    d_out = torch.empty_like(d_res)
    ws = car.new_rmsnorm_workspace() if use_ws else None
    car.ar_oneshot_rmsnorm(ins, d_res, d_w, d_ro, d_out, eps, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(d_ro), oracle_bits(want_ro)), f"{what}: one-shot residual_out"
    one = host_values(d_out, dt)
    check_out(one, y, dt, what + " (one-shot)")
    if ws is not None:
        assert car.read_status(ws) == (0, 0), what

    # two-shot form: every rank's reduce-scatter, then every rank's share
    residuals = [to_dev(res) for _ in range(n)]
    segs = car.new_rmsnorm_segments(n, rows, hidden, ins[0].dtype)
    flags = car.new_flags(n)
    outs = [torch.empty(numel, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    ros = [torch.empty(numel, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    if auto:
        car.ar_twoshot_rmsnorm(ins, residuals, d_w, segs, flags, 0, r0=1, r1=n, eps=eps)
        shares = [0]
    else:
        car.ar_twoshot_rmsnorm(ins, residuals, d_w, segs, flags, 1, r0=0, r1=n, eps=eps)
        shares = range(n)
    for me in shares:
        car.ar_twoshot_rmsnorm(ins, residuals, d_w, segs, flags, 0 if auto else 1, r0=me, r1=me + 1,
                               residual_outs=[ros[r] if r == me else None for r in range(n)],
                               outs=[outs[r] if r == me else None for r in range(n)], eps=eps)
    torch.cuda.synchronize()
    car.raise_on_status(flags, what)
    for me in shares:
        assert np.array_equal(bits(ros[me]), oracle_bits(want_ro)), f"{what}: two-shot residual_out, rank {me}"
        two = host_values(outs[me], dt)
        check_out(two, y, dt, f"{what} (two-shot, rank {me})")
        if one_parts == two_parts:
            assert np.array_equal(two, one), f"{what}: the two forms differ, rank {me}"
