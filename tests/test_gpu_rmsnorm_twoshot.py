"""The fused all-reduce + residual add + RMSNorm in two-shot form
(ar_twoshot_rmsnorm): every rank's reduce-scatter publishes its rows, then
each rank's share (its own rows and the all-gather of its peers') is checked
against the oracle (O10: residual_out bit for bit, out within the bound
derived in test_gpu_rmsnorm.py) and, where both take the same kind of path,
against the one-shot form with a workspace bit for bit: a workgroup per row
in both (the same per-row code), or parts of rows in both (the same
arithmetic in the same shuffle trees).  The two-shot form cuts rows into
parts where a row's n + 1 streams hold at least 128 KiB and a rank owns
fewer than 256 rows; the one-shot form where the same holds for the bytes
and rows * parts <= 512."""
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


class Setup:
    def __init__(self, n, dt, rows, hidden, config, eps=1e-6):
        self.n, self.dt, self.rows, self.hidden, self.eps = n, dt, rows, hidden, eps
        numel = rows * hidden
        self.host = synth.rank_inputs(n, numel, dt, "normal", config=config)
        self.res = synth.rank_inputs(1, numel, dt, "normal", config=config + 1000)[0]
        self.w = synth.rank_inputs(1, hidden, dt, "normal", config=config + 2000)[0]
        self.ins = [to_dev(a) for a in self.host]
        self.residuals = [to_dev(self.res) for _ in range(n)]  # every rank's copy of the residual stream
        self.weight = to_dev(self.w)
        tdt = self.ins[0].dtype
        self.segs = car.new_rmsnorm_segments(n, rows, hidden, tdt)
        self.outs = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
        self.ros = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
        self.flags = car.new_flags(n)

    def want(self):
        return oracle.oneshot_rmsnorm(self.host, self.res, self.w, self.hidden, self.eps, self.dt)

    def vecs(self):
        return self.hidden * (4 if self.dt == "f32" else 2) // 16

    def oneshot_parts(self) -> bool:
        v = self.vecs()
        return self.rows * -(-v // 64) <= 512 and (self.n + 1) * v * 16 >= 128 << 10

    def twoshot_parts(self) -> bool:
        return self.rows // self.n < 256 and (self.n + 1) * self.vecs() * 16 >= 128 << 10

    def oneshot_bits(self):
        # the one-shot form with a workspace (on its parts path where that applies)
        ro, out = torch.empty_like(self.outs[0]), torch.empty_like(self.outs[0])
        car.ar_oneshot_rmsnorm(self.ins, self.residuals[0], self.weight, ro, out, self.eps,
                               workspace=car.new_rmsnorm_workspace())
        torch.cuda.synchronize()
        return bits(ro), bits(out)

    def reduce_scatter(self, step, ranks=None):
        ranks = range(self.n) if ranks is None else ranks
        for r in ranks:
            car.ar_twoshot_rmsnorm(self.ins, self.residuals, self.weight, self.segs, self.flags, step, r0=r,
                                   r1=r + 1, eps=self.eps)

    def share(self, me, step):
        outs = [self.outs[r] if r == me else None for r in range(self.n)]
        ros = [self.ros[r] if r == me else None for r in range(self.n)]
        car.ar_twoshot_rmsnorm(self.ins, self.residuals, self.weight, self.segs, self.flags, step, r0=me,
                               r1=me + 1, residual_outs=ros, outs=outs, eps=self.eps)


def check_rank(s: Setup, me, want_ro, y, one_ro, one_out, what):
    assert np.array_equal(bits(s.ros[me]), oracle_bits(want_ro)), f"{what}: residual_out differs from the oracle"
    check_out(host_values(s.outs[me], s.dt), y, s.dt, what)
    assert np.array_equal(bits(s.ros[me]), one_ro), f"{what}: residual_out differs from the one-shot form"
    if s.oneshot_parts() == s.twoshot_parts():
        assert np.array_equal(bits(s.outs[me]), one_out), f"{what}: out differs from the one-shot form"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
@pytest.mark.parametrize("groups, hidden", [(1, 8), (3, 264), (2, 1000), (4, 8192), (2, 16384)])
def test_every_rank_matches_the_oracle_and_the_one_shot(n, dt, groups, hidden):
    if dt == "f32" and hidden == 16384 and n == 16:
        hidden = 8192  # keep the case small
    s = Setup(n, dt, n * groups, hidden, config=400 + n)
    want_ro, y = s.want()
    one_ro, one_out = s.oneshot_bits()
    s.reduce_scatter(1)  # every rank's rows published (split launches)
    car.ar_twoshot_rmsnorm(s.ins, s.residuals, s.weight, s.segs, s.flags, 1, r0=0, r1=n, eps=s.eps)  # one launch
    for me in range(n):
        s.share(me, 1)
    torch.cuda.synchronize()
    car.raise_on_status(s.flags, "two-shot rmsnorm")
    for me in range(n):
        check_rank(s, me, want_ro, y, one_ro, one_out, f"n={n} {dt} rows={s.rows} hidden={hidden} rank {me}")


@pytest.mark.parametrize("n, rows, hidden", [(2, 2 * 1030, 8), (8, 8 * 300, 8192)])
def test_many_rows_per_rank(n, rows, hidden):
    # more than 1024 rows per rank (two rows per arrival slot), and heavy rows
    # with at least 256 per rank: both take a workgroup per row
    s = Setup(n, "bf16", rows, hidden, config=420)
    want_ro, y = s.want()
    one_ro, one_out = s.oneshot_bits()
    s.reduce_scatter(1)
    for me in (0, n - 1):
        s.share(me, 1)
    torch.cuda.synchronize()
    car.raise_on_status(s.flags, "two-shot rmsnorm")
    for me in (0, n - 1):
        check_rank(s, me, want_ro, y, one_ro, one_out, f"n={n} rows={rows} rank {me}")


def test_steps_in_a_row_with_changing_data():
    n, rows, hidden = 8, 16, 4096
    s = Setup(n, "bf16", rows, hidden, config=430)
    for step in range(1, 6):
        host = synth.rank_inputs(n, rows * hidden, "bf16", "normal", config=431 + step)
        for t, a in zip(s.ins, host):
            t.copy_(to_dev(a))
        s.host = host
        want_ro, y = s.want()
        s.reduce_scatter(step, ranks=[r for r in range(n) if r != 3])
        s.share(3, step)  # rank 3's share publishes its own rows too
        torch.cuda.synchronize()
        car.raise_on_status(s.flags, f"step {step}")
        assert np.array_equal(bits(s.ros[3]), oracle_bits(want_ro)), f"step {step}"
        check_out(host_values(s.outs[3], "bf16"), y, "bf16", f"step {step}")


def test_a_missing_peer_is_reported_as_a_timeout():
    n, rows, hidden = 4, 8, 1024
    s = Setup(n, "bf16", rows, hidden, config=440)
    s.reduce_scatter(1, ranks=[0, 2, 3])  # rank 1 never publishes
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(1_000_000)
    try:
        s.share(0, 1)
        torch.cuda.synchronize()
    finally:
        car.set_poll_timeout_ns(old)
    word, _ = car.read_status(s.flags)
    code, phase, rank = car.decode_status(word)
    assert (code, phase, rank) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG, 1)


def test_argument_errors():
    s = Setup(4, "bf16", 8, 64, config=450)
    f = car.ar_twoshot_rmsnorm
    with pytest.raises(ValueError):  # a rank range past n
        f(s.ins, s.residuals, s.weight, s.segs, s.flags, 1, r0=3, r1=5)
    with pytest.raises(car.ArError):  # the all-gather for two ranks in one launch
        f(s.ins, s.residuals, s.weight, s.segs, s.flags, 1, r0=0, r1=2, residual_outs=s.ros, outs=s.outs)
    with pytest.raises(ValueError):  # residual_outs without outs
        f(s.ins, s.residuals, s.weight, s.segs, s.flags, 1, r0=0, r1=1, residual_outs=s.ros)
    x = [torch.zeros(6 * 64, dtype=torch.bfloat16, device="cuda") for _ in range(4)]  # 6 rows over 4 ranks
    with pytest.raises(car.ArError) as e:
        f(x, x, s.weight, [torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")] * 4, s.flags, 1)
    assert e.value.code == car.AR_ERR_DIVISIBLE


# ---- auto step ids (step 0): each rank's epoch kept in its segment ----------
def epoch_words(s: Setup, r):
    """Rank r's epoch words: (those of its reduce-scatter, those of its
    all-gather).  A segment holds G out rows and G residual_out rows, G P
    partial slots and G P done flags, then (16-byte aligned) a word per
    wavefront: parts of rows, G P for the reduce-scatter and (n - 1) G P for
    the all-gather; a workgroup per row, tiles x wavefronts per workgroup for
    the reduce-scatter and n - 1 times that for the all-gather."""
    V, G = s.vecs(), s.rows // s.n
    P = -(-V // 64)
    if s.twoshot_parts():
        rs = G * P
    else:
        tile = -(-G // 1024)
        vpt = 1 if V <= 1024 else (2 if V <= 2048 else 4)
        rs = -(-G // tile) * -(-(-(-V // vpt)) // 64)
    off = -(-(32 * G * V + 12 * G * P) // 16) * 16
    w = s.segs[r][off: off + 4 * s.n * rs].view(torch.int32).cpu().numpy()
    return w[:rs], w[rs:]


def check_epochs(s: Setup, calls):
    # every reduce-scatter word advanced once per step; only rank 0's all-gather ran
    for r in range(s.n):
        rs, ag = epoch_words(s, r)
        assert (rs == calls).all(), f"rank {r}: reduce-scatter epochs {set(rs.tolist())}, want {calls}"
        assert (ag == (calls if r == 0 else 0)).all(), f"rank {r}: all-gather epochs {set(ag.tolist())}"


def check_share(s: Setup, me, what):
    want_ro, y = s.want()
    assert np.array_equal(bits(s.ros[me]), oracle_bits(want_ro)), f"{what}: residual_out"
    check_out(host_values(s.outs[me], s.dt), y, s.dt, what)


def new_data(s: Setup, config):
    s.host = synth.rank_inputs(s.n, s.rows * s.hidden, s.dt, "normal", config=config)
    for t, a in zip(s.ins, s.host):
        t.copy_(to_dev(a))


# parts of rows (8 and 2 rows per rank), a workgroup per row (300 rows per rank; light rows;
# 1030 rows per rank, two to an arrival slot)
AUTO_CASES = [(8, 64, 8192), (16, 32, 16384), (8, 8 * 300, 8192), (4, 32, 64), (2, 2 * 1030, 8)]


@pytest.mark.parametrize("n, rows, hidden", AUTO_CASES)
def test_auto_step_ids_in_a_row(n, rows, hidden):
    s = Setup(n, "bf16", rows, hidden, config=460)
    for it in range(4):
        new_data(s, 461 + it)
        car.ar_twoshot_rmsnorm(s.ins, s.residuals, s.weight, s.segs, s.flags, 0, r0=1, r1=n, eps=s.eps)
        s.share(0, 0)
        torch.cuda.synchronize()
        car.raise_on_status(s.flags, f"auto step {it}")
        check_share(s, 0, f"n={n} rows={rows} hidden={hidden} auto step {it}")
    check_epochs(s, 4)


@pytest.mark.parametrize("n, rows, hidden", [AUTO_CASES[0], AUTO_CASES[2]])
def test_auto_step_ids_replayed_in_a_graph(n, rows, hidden):
    # the peers' reduce-scatters and rank 0's share captured once; each replay
    # takes the next id, with eager calls on the same segments in between
    s = Setup(n, "bf16", rows, hidden, config=470)
    only0 = (lambda ts: [ts[0]] + [None] * (n - 1))
    peers = car.prepare_twoshot_rmsnorm(s.ins, s.residuals, s.weight, s.segs, s.flags, 1, n, eps=s.eps)
    share = car.prepare_twoshot_rmsnorm(s.ins, s.residuals, s.weight, s.segs, s.flags, 0, 1, only0(s.ros),
                                        only0(s.outs), eps=s.eps)

    def step():
        peers(0)
        share(0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    calls = 1
    for rep in range(6):
        new_data(s, 471 + rep)
        if rep % 2:
            step()  # eager, between replays
            calls += 1
            torch.cuda.synchronize()
        g.replay()
        calls += 1
        torch.cuda.synchronize()
        car.raise_on_status(s.flags, f"replay {rep}")
        check_share(s, 0, f"n={n} rows={rows} replay {rep}")
    check_epochs(s, calls)


@pytest.mark.parametrize("n, rows, hidden", [AUTO_CASES[0], AUTO_CASES[3]])
def test_auto_step_ids_after_a_missing_peer(n, rows, hidden):
    # rank 1's reduce-scatter is skipped for a step: rank 0's share times out naming
    # it, and rank 1's epoch words stay a step behind, so the next step times out
    # too; zeroing the segments (and resetting the flag region) restarts every epoch
    s = Setup(n, "bf16", rows, hidden, config=480)
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(1_000_000)
    try:
        for it, skip in enumerate((True, False)):
            new_data(s, 481 + it)
            car.ar_twoshot_rmsnorm(s.ins, s.residuals, s.weight, s.segs, s.flags, 0, r0=2, r1=n, eps=s.eps)
            if not skip:
                car.ar_twoshot_rmsnorm(s.ins, s.residuals, s.weight, s.segs, s.flags, 0, r0=1, r1=2, eps=s.eps)
            s.share(0, 0)
            torch.cuda.synchronize()
            word, _ = car.read_status(s.flags)
            code, phase, rank = car.decode_status(word)
            assert (code, phase, rank) == (car.AR_ERR_TIMEOUT, car.PHASE_TWOSHOT_AG, 1), f"step {it}"
            car.ar_flag_barrier_reset(s.flags, n)
    finally:
        car.set_poll_timeout_ns(old)
    for t in s.segs:
        t.zero_()
    for it in range(2):
        new_data(s, 483 + it)
        car.ar_twoshot_rmsnorm(s.ins, s.residuals, s.weight, s.segs, s.flags, 0, r0=1, r1=n, eps=s.eps)
        s.share(0, 0)
        torch.cuda.synchronize()
        car.raise_on_status(s.flags, f"after the restart, step {it}")
        check_share(s, 0, f"n={n} rows={rows} after the restart, step {it}")
    check_epochs(s, 2)
