"""Pins for the CPU oracle: each check ties it to something other than itself
(values printed on the pages, closed forms, library routines, invariants,
brute force).  CPU only."""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import synth
from oracle import model
from conftest import golden_kv, read_golden


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------- O1 --
def _check_chunk(lo):
    u = np.arange(lo, lo + (1 << 26), dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    ours = oracle.f32_to_bf16(f)
    ref = _torch_bf16_bits(f)
    nan_in = np.isnan(f)
    ours_nan = ((ours & 0x7F80) == 0x7F80) & ((ours & 0x7F) != 0)
    ok_nan = bool(np.all(ours_nan[nan_in]))
    # NaN: sign kept, quiet bit set, payload truncated (the oracle's stated reading)
    exp_nan = ((u[nan_in] >> 16) | 0x40).astype(np.uint16)
    ok_payload = bool(np.array_equal(ours[nan_in], exp_nan))
    mism = int(np.count_nonzero(ours[~nan_in] != ref[~nan_in]))
    return mism, ok_nan, ok_payload


def test_bf16_rne_exhaustive_against_torch():
    """All 2^32 float32 patterns: round-to-nearest-even must equal PyTorch's
    CPU float32->bfloat16 conversion (a library routine) for every non-NaN
    input; every NaN must stay a quiet NaN with its sign."""
    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(_check_chunk, range(0, 1 << 32, 1 << 26)))
    assert sum(r[0] for r in res) == 0
    assert all(r[1] for r in res)
    assert all(r[2] for r in res)


@pytest.mark.parametrize(
    "x, expect",
    [
        (1.0 + 2.0**-8, 0x3F80),  # exactly half an ulp above 1.0: tie -> even (down)
        (1.0 + 3 * 2.0**-8, 0x3F82),  # tie between 0x3F81 and 0x3F82: -> even (up)
        (1.0 + 2.0**-8 + 2.0**-20, 0x3F81),  # just above the tie: up
        (-(1.0 + 2.0**-8), 0xBF80),  # sign symmetric
        (float(np.finfo(np.float32).max), 0x7F80),  # max finite float32 rounds to +inf
        (float("inf"), 0x7F80),
        (-float("inf"), 0xFF80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float(np.float32(2.0**-130)), 0x0008),  # subnormal 2^-130 = 2^19 * 2^-149: bits 0x00080000
    ],
)
def test_bf16_rne_special_cases(x, expect):
    assert int(oracle.f32_to_bf16(np.array([x], dtype=np.float32))[0]) == expect


def test_bf16_widen_is_exact():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(b)
    fin = np.isfinite(f)
    assert np.array_equal(oracle.f32_to_bf16(f[fin]), b[fin])


# --------------------------------------------------------------------- O2 --
@pytest.mark.parametrize("n", [2, 3, 5, 8, 16])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_oneshot_integer_data_matches_int64_sum(n, dt):
    """Integer-valued data U{-8..8}: every partial sum is an integer below
    2^8 in magnitude, so fp32 accumulation and one bf16 rounding are exact.
    The oracle must equal the int64 sum (a closed form)."""
    numel = 4096 + 37
    ins = synth.rank_inputs(n, numel, dt, "int", config=0)
    out = oracle.oneshot(ins, dt)
    ints = [synth.integers_f32(numel, synth.rank_seed(0, r)).astype(np.int64) for r in range(n)]
    exact = np.sum(ints, axis=0).astype(np.float32)
    got = out if dt == "f32" else oracle.bf16_to_f32(out)
    assert np.array_equal(got, exact)


@pytest.mark.parametrize("ngpus", list(range(2, 17)))
def test_oneshot_fill_closed_form(ngpus):
    """The NCCL program's check: x_g[i] = g + i%7 sums to
    ngpus(ngpus-1)/2 + ngpus*(i%7) (fixture fill_closed_form.txt)."""
    kv = golden_kv("fill_closed_form.txt")
    mod = int(kv["fill_modulus"])
    numel = 7 * 1000 + 3
    for dt in ("f32", "bf16"):
        ins = synth.rank_inputs(ngpus, numel, dt, "fill", config=0)
        out = oracle.oneshot(ins, dt)
        got = out if dt == "f32" else oracle.bf16_to_f32(out)
        i = np.arange(numel)
        expect = ngpus * (ngpus - 1) / 2 + ngpus * (i % mod)
        assert np.array_equal(got.astype(np.float64), expect)


def test_oneshot_rank_permutation_invariant_on_integers():
    n, numel = 8, 3000
    ins = synth.rank_inputs(n, numel, "f32", "int", config=0)
    base = oracle.oneshot(ins, "f32")
    perm = list(np.random.default_rng(7).permutation(n))
    assert np.array_equal(oracle.oneshot([ins[p] for p in perm], "f32"), base)


def test_oneshot_n2_is_one_ieee_add():
    """n = 2: +0 + a is a (for a != -0), then one add: numpy's float32 a+b."""
    a = synth.normal_f32(10000, 1)
    b = synth.normal_f32(10000, 2)
    assert np.array_equal(oracle.oneshot([a, b], "f32"), (a + b).astype(np.float32))


def test_oneshot_is_a_fold_in_rank_order():
    """Non-associative case that exposes the order: ranks 0..2 hold
    (2^24, 1, 1): ((0 + 2^24) + 1) + 1 = 2^24 in fp32 (each +1 rounds away),
    while any order adding the ones first gives 2^24 + 2."""
    ins = [np.array([2.0**24], np.float32), np.array([1.0], np.float32), np.array([1.0], np.float32)]
    assert oracle.oneshot(ins, "f32")[0] == np.float32(2.0**24)
    ins2 = [ins[1], ins[2], ins[0]]
    assert oracle.oneshot(ins2, "f32")[0] == np.float32(2.0**24 + 2)


def test_oneshot_accumulator_starts_at_plus_zero():
    """The accumulator starts at +0 and every rank is added, so a column of
    -0.0 sums to +0.0 (the first rank is not used as the start value)."""
    ins = [np.array([-0.0], np.float32) for _ in range(4)]
    assert _bits(oracle.oneshot(ins, "f32"))[0] == 0x00000000
    insb = [np.array([0x8000], np.uint16) for _ in range(4)]
    assert int(oracle.oneshot(insb, "bf16")[0]) == 0x0000


@pytest.mark.parametrize("n", [2, 8, 16])
def test_oneshot_normal_within_recursive_summation_bound(n):
    """N(0,1) data: |fold - exact| <= gamma_{n} * sum|x| (recursive summation,
    Higham, Accuracy and Stability of Numerical Algorithms, eq. 4.4 with the
    extra +0 start), then bf16 rounding adds at most half a bf16 ulp."""
    numel = 20000
    ins = synth.rank_inputs(n, numel, "f32", "normal", config=5)
    out = oracle.oneshot(ins, "f32").astype(np.float64)
    X = np.stack([a.astype(np.float64) for a in ins])
    exact = X.sum(0)
    u = 2.0**-24
    gamma = n * u / (1 - n * u)
    assert np.all(np.abs(out - exact) <= gamma * np.abs(X).sum(0))
    insb = synth.rank_inputs(n, numel, "bf16", "normal", config=5)
    outb = oracle.bf16_to_f32(oracle.oneshot(insb, "bf16")).astype(np.float64)
    Xb = np.stack([oracle.bf16_to_f32(a).astype(np.float64) for a in insb])
    exb = Xb.sum(0)
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(exb) + 1e-300)[1] - 9)  # 2^(e-1-8): half of bf16 ulp
    assert np.all(np.abs(outb - exb) <= gamma * np.abs(Xb).sum(0) * 1.01 + half_ulp * 1.01 + 1e-40)


# --------------------------------------------------------------------- O3 --
@pytest.mark.parametrize("n", [2, 4, 8, 16])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_twoshot_equals_oneshot_bitwise(n, dt):
    numel = n * 1024
    ins = synth.rank_inputs(n, numel, dt, "normal", config=2)
    segs, outs = oracle.twoshot(ins, dt)
    ref = oracle.oneshot(ins, dt)
    for r in range(n):
        assert np.array_equal(outs[r], ref)
    # all-reduce = reduce-scatter + all-gather: the segments, in order, are the result
    assert np.array_equal(np.concatenate(segs), ref)


def test_twoshot_rejects_non_divisible():
    ins = synth.rank_inputs(3, 100, "f32", "normal", config=2)
    with pytest.raises(ValueError):
        oracle.twoshot(ins, "f32")


# --------------------------------------------------------------------- O4 --
@pytest.mark.parametrize("p", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ring_integer_data_equals_oneshot(p, dt):
    numel = p * 257
    ins = synth.rank_inputs(p, numel, dt, "int", config=0)
    bufs, sent = oracle.ring(ins, dt)
    ref = oracle.oneshot(ins, dt)
    for r in range(p):
        assert np.array_equal(bufs[r], ref)
    es = 4 if dt == "f32" else 2
    S = numel * es
    # each rank sends 2(p-1) chunks of S/p bytes (ring section, "多 GPU 与 NCCL")
    assert all(s == 2 * (p - 1) * S // p for s in sent)
    assert all(s == model.remote_bytes_per_rank("ring", S, p) for s in sent)


def test_ring_normal_data_within_bound():
    p, numel = 8, 8 * 1000
    ins = synth.rank_inputs(p, numel, "f32", "normal", config=4)
    bufs, _ = oracle.ring(ins, "f32")
    X = np.stack([a.astype(np.float64) for a in ins])
    u = 2.0**-24
    gamma = (p - 1) * u / (1 - (p - 1) * u)
    for r in range(p):
        assert np.array_equal(bufs[r], bufs[0])  # all-gather copies: every rank agrees
        assert np.all(np.abs(bufs[r] - X.sum(0)) <= gamma * np.abs(X).sum(0))


def test_ring_by_brute_force_tiny():
    """p = 3, one element per chunk, distinct powers of two so every partial
    sum is exact and the rank holding each chunk can be read off: after the
    ring every rank holds the full sums."""
    ins = [np.array([1, 2, 4], np.float32) * (8.0**r) for r in range(3)]
    bufs, sent = oracle.ring(ins, "f32")
    tot = sum(ins)
    for b in bufs:
        assert np.array_equal(b, tot)
    assert sent == [4 * 4] * 3  # 2(p-1) = 4 messages of one float


# ------------------------------------------------------------------ O5/O6 --
def test_protocol_table_efficiencies():
    rows = {r[0]: [int(v) for v in r[1:]] for r in read_golden("protocol_table.txt")}
    for proto, key in (("ll", "LL"), ("ll128", "LL128")):
        line, data, flag, pct = rows[key]
        assert data + flag == line
        S = 120 * 4 * 1000  # a multiple of both payload sizes: no padding
        eff = S / oracle.ll_wire_bytes(proto, S)
        assert eff == pytest.approx(data / line)
        assert round(100 * eff) == pct


def _check_layout(proto, msg, step):
    wire = oracle.ll_pack(proto, msg, step)
    raw = msg.view(np.uint8)
    d, lb = (4, 8) if proto == "ll" else (120, 128)
    lines = wire.reshape(-1, lb)
    assert lines.shape[0] == -(-raw.size // d)
    pad = np.zeros(lines.shape[0] * d, np.uint8)
    pad[: raw.size] = raw
    assert np.array_equal(lines[:, :d].reshape(-1), pad)
    if proto == "ll":
        assert np.all(lines[:, 4:].copy().view(np.uint32)[:, 0] == step)
    else:
        assert np.all(lines[:, 120:].copy().view(np.uint64)[:, 0] == step)
    return wire


@settings(max_examples=60, deadline=None)
@given(
    proto=st.sampled_from(["ll", "ll128"]),
    nbytes=st.integers(min_value=1, max_value=3000),
    step=st.integers(min_value=1, max_value=2**32 - 1),
    seed=st.integers(0, 2**31),
)
def test_ll_round_trip_and_layout(proto, nbytes, step, seed):
    msg = np.random.default_rng(seed).integers(0, 256, nbytes, dtype=np.uint8)
    wire = _check_layout(proto, msg, step)
    back, ready, bad = oracle.ll_unpack(proto, wire, nbytes, step)
    assert ready and bad is None
    assert np.array_equal(back, msg)
    # a receiver waiting for an earlier step accepts it too (>= step)
    assert oracle.ll_unpack(proto, wire, nbytes, max(1, step - 1))[1]
    if step < 2**32 - 1:
        _, ready2, bad2 = oracle.ll_unpack(proto, wire, nbytes, step + 1)
        assert not ready2 and bad2 == 0


def test_ll_wire_sizes_for_the_64KiB_and_1MiB_messages():
    for S in (64 * 1024, 1024 * 1024):
        assert oracle.ll_wire_bytes("ll", S) == 2 * S == model.ll_wire_bytes("ll", S)
        lines = oracle.ll_lines("ll128", S)
        assert lines * 120 >= S > (lines - 1) * 120
        assert oracle.ll_wire_bytes("ll128", S) == 128 * lines == model.ll_wire_bytes("ll128", S)


# --------------------------------------------------------------------- O7 --
@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ll_reduce_equals_oneshot_of_payloads(proto, dt):
    n, numel = 8, 4096 + 7
    ins = synth.rank_inputs(n, numel, dt, "normal", config=3)
    wires = [oracle.ll_pack(proto, a, 17) for a in ins]
    out = oracle.ll_reduce(proto, wires, numel, dt, 17)
    assert np.array_equal(out, oracle.oneshot(ins, dt))


@pytest.mark.parametrize("proto", ["ll", "ll128"])
def test_ll_reduce_stale_flag_names_the_rank(proto):
    n, numel = 8, 2048
    ins = synth.rank_inputs(n, numel, "f32", "normal", config=3)
    wires = [oracle.ll_pack(proto, a, 5) for a in ins]
    wires[5] = oracle.ll_pack(proto, ins[5], 4)  # rank 5 still on step 4
    with pytest.raises(oracle.OracleTimeout) as e:
        oracle.ll_reduce(proto, wires, numel, "f32", 5)
    assert e.value.rank == 5 and e.value.line == 0


# --------------------------------------------------------------------- O8 --
def test_flag_barrier_steps_withheld_and_reset():
    n = 8
    b = oracle.FlagBarrier(n)
    for s in range(1, 1001):
        assert not b.can_pass(s)
        for r in range(n):
            b.publish(r, s)
        assert b.can_pass(s)
    for r in range(n):
        if r != 3:
            b.publish(r, 1001)
    assert not b.can_pass(1001) and b.first_missing(1001) == 3
    b.publish(3, 1002)  # a rank that moved ahead still counts as arrived
    assert b.can_pass(1001)
    b.reset()
    assert b.flags == [0] * n and not b.can_pass(1)
    with pytest.raises(ValueError):
        b.publish(0, 0)


# --------------------------------------------------------------------- O9 --
def test_alpha_beta_table_reproduces_printed_values():
    names = ["ring", "tree", "one-shot", "two-shot", "NVLS"]
    for row in read_golden("alpha_beta_table.txt"):
        S = int(row[0])
        printed = [float(v) for v in row[1:6]]
        got = [round(model.ALGOS[k](S) * 1e6, 1) for k in names]
        assert got == printed
        best = min((k for k in names if k != "NVLS"), key=lambda k: model.ALGOS[k](S))
        assert best == row[6]


def test_ring_1gib_line():
    kv = golden_kv("ring_1gib.txt")
    S = int(kv["bytes"])
    t = model.t_ring(S)
    assert f"{t * 1e3:.2f}" == kv["ms"]
    assert f"{model.algbw(S, t) / 1e9:.0f}" == kv["algbw_GBps"]
    assert f"{model.busbw(S, t, 8) / 1e9:.0f}" == kv["busbw_GBps"]


def test_exercise_answers():
    kv = golden_kv("exercises.txt")
    n = int(kv["ex1_n"])
    bus = float(kv["ex1_busbw_GBps"]) * 1e9
    S = int(kv["ex1_bytes"])
    alg_ar = bus / model.BUSBW_FACTOR["all-reduce"](n)
    assert round(alg_ar / 1e9, 1) == float(kv["ex1_allreduce_algbw_GBps"])
    assert round(S / alg_ar * 1e3, 1) == float(kv["ex1_allreduce_ms"])
    alg_ag = bus / model.BUSBW_FACTOR["all-gather"](n)
    assert round(alg_ag / 1e9) == float(kv["ex1_allgather_algbw_GBps"])
    assert round(S / alg_ag * 1e3, 2) == float(kv["ex1_allgather_ms"])
    # crossover: "about 257 KB" at n = 8, none at n = 2
    s_star = model.crossover_oneshot_twoshot(int(kv["ex2_n"]))
    assert round(s_star / 1e3) == int(kv["ex2_crossover_KB"])
    assert math.isinf(model.crossover_oneshot_twoshot(2))
    # at the crossover the two model times agree
    assert model.t_oneshot(s_star) == pytest.approx(model.t_twoshot(s_star), rel=1e-12)
    # TP exercise: decode 16 KB (1 token x 8192 x 2 B), prefill 128 MB (8192 tokens)
    hidden = int(kv["ex3_hidden"])
    dec = 1 * hidden * 2
    assert round(dec / 1024) == int(kv["ex3_decode_KB"])
    bw = float(kv["ex3_bw_GBps"]) * 1e9
    assert round(model.remote_bytes_per_rank("ring", dec, 8) / bw * 1e6, 2) == float(kv["ex3_decode_us"])
    pre = 8192 * hidden * 2
    assert round(pre / 2**20) == int(kv["ex3_prefill_MB"])
    sent = model.remote_bytes_per_rank("ring", pre, 8)
    sent_mb = round(sent / 2**20)
    assert sent_mb == int(kv["ex3_prefill_ring_sent_MB"])
    # the page divides the MiB count by 400 GB/s as if it were 10^6 bytes (224 MB -> 0.56 ms)
    assert round(sent_mb * 1e6 / bw * 1e3, 2) == float(kv["ex3_prefill_ms"])


def test_remote_byte_counts():
    S = 1 << 20
    assert model.remote_bytes_per_rank("one-shot", S, 8) == 7 * S
    assert model.remote_bytes_per_rank("two-shot", S, 8) == 2 * 7 / 8 * S
    assert model.busbw(S, 1.0, 8) == S * 2 * 7 / 8


# ------------------------------------------------------ O9: HBM byte model --
class _Counted:
    """A buffer that counts the bytes read from and written to it."""

    def __init__(self, nbytes):
        self.nbytes, self.r, self.w = nbytes, 0, 0

    def read(self, lo, hi):
        assert 0 <= lo <= hi <= self.nbytes
        self.r += hi - lo

    def write(self, lo, hi):
        assert 0 <= lo <= hi <= self.nbytes
        self.w += hi - lo


def _brute_bytes(op, S, n, proto=None, es=2):
    """Walk each operation element by element (line by line for the wires),
    as its steps are written, touching counted buffers; return the totals.
    Independent of model.hbm_bytes: no formula, only the steps."""
    N, m = S // es, S // es // n
    ins = [_Counted(S) for _ in range(n)]
    bufs = list(ins)

    def new(nb):
        b = _Counted(nb)
        bufs.append(b)
        return b

    def lines(nbytes, proto):
        data, line = (4, 8) if proto == "ll" else (120, 128)
        return [(k * data, min((k + 1) * data, nbytes), k * line, (k + 1) * line)
                for k in range((nbytes + data - 1) // data)]

    if op == "oneshot":
        out = new(S)
        for k in range(N):
            for i in range(n):
                ins[i].read(k * es, (k + 1) * es)
            out.write(k * es, (k + 1) * es)
    elif op in ("twoshot_share", "twoshot_full"):
        segs = [new(m * es) for _ in range(n)]
        ranks = range(n) if op == "twoshot_full" else [n // 2]
        for r in ranks:  # reduce-scatter: segment r of every rank's message
            for k in range(m):
                for i in range(n):
                    ins[i].read((r * m + k) * es, (r * m + k + 1) * es)
                segs[r].write(k * es, (k + 1) * es)
        if op == "twoshot_share":  # the peers' segments: other GPUs' work
            for j in range(n):
                if j != n // 2:
                    segs[j].w += m * es
        for r in ranks:  # all-gather: every segment into rank r's output
            out = new(S)
            for j in range(n):
                for k in range(m):
                    segs[j].read(k * es, (k + 1) * es)
                    out.write((j * m + k) * es, (j * m + k + 1) * es)
        if op == "twoshot_share":
            for j in range(n):
                if j != n // 2:
                    segs[j].w -= m * es
    elif op in ("ll_reduce", "ll_pack"):
        L = lines(S, proto)
        W = L[-1][3]
        if op == "ll_pack":
            w = new(W)
            for d0, d1, l0, l1 in L:
                ins[0].read(d0, d1)
                w.write(l0, l1)
            for b in ins[1:]:
                b.r = b.w = 0
        else:
            wires = [new(W) for _ in range(n)]
            out = new(S)
            for d0, d1, l0, l1 in L:
                for w in wires:
                    w.read(l0, l1)
                out.write(d0, d1)
    else:
        raise ValueError(op)
    return sum(b.r for b in bufs), sum(b.w for b in bufs)


@pytest.mark.parametrize("n", [2, 3, 8])
@pytest.mark.parametrize("S", [96, 240, 1920])
def test_hbm_bytes_by_brute_force(n, S):
    """model.hbm_bytes against a step-by-step walk of each operation that
    counts every byte read and written (S divisible by n and by 2 bytes)."""
    if S % (2 * n):
        pytest.skip("two-shot needs whole bf16 segments")
    for op in ("oneshot", "twoshot_share", "twoshot_full"):
        assert model.hbm_bytes(op, S, n) == _brute_bytes(op, S, n), op
    for proto in ("ll", "ll128"):
        assert model.hbm_bytes("ll_pack", S, n, proto) == _brute_bytes("ll_pack", S, n, proto), proto
        assert model.hbm_bytes("ll_reduce", S, n, proto) == _brute_bytes("ll_reduce", S, n, proto), proto


def test_hbm_bytes_at_the_stated_configurations():
    for cfg, op, n, S, r, w in read_golden("hbm_bytes.txt"):
        n, S, r, w = int(n), int(S), int(r), int(w)
        if op.startswith("ll"):
            proto = op.split("_")[0]
            got = model.hbm_bytes("ll_reduce", S, n, proto)
        else:
            got = model.hbm_bytes(op, S, n)
        assert got == (r, w), (cfg, op, n, S, got)


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_hbm_reads_minus_local_reads_are_the_pages_remote_bytes(n):
    """The pages count only the bytes a GPU pulls from its peers: (n-1)S for
    the one-shot and 2(n-1)/n S for the two-shot (算法).  Taking the local
    reads (a rank's own buffer; for the two-shot its own input segment and its
    own reduced segment) out of the HBM reads must give exactly those."""
    S = 1 << 20
    r, _ = model.hbm_bytes("oneshot", S, n)
    assert r - S == model.remote_bytes_per_rank("one-shot", S, n)
    r, _ = model.hbm_bytes("twoshot_share", S, n)
    assert r - 2 * (S // n) == model.remote_bytes_per_rank("two-shot", S, n)
