"""The C-ABI library loads on the CPU, exports every entry point declared in
include/ar.h, and rejects bad arguments synchronously (host logic only: no
call here reaches a kernel launch).  CPU only."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import custom_all_reduce_amd as car
from custom_all_reduce_amd import accounting
from oracle import model

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ar.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^(?:int|size_t|void|uint64_t|double|const char\*)\s+(ar_\w+)\(", text, re.M)))


def test_header_declares_the_seven_path_calls():
    names = declared_functions()
    for required in ("ar_oneshot", "ar_twoshot_rs", "ar_twoshot_ag", "ar_ll_pack", "ar_ll_reduce_unpack",
                     "ar_ll128_reduce_unpack", "ar_flag_barrier_reset"):
        assert required in names


def test_header_declares_the_store_paths_copy_engine_and_selector():
    names = declared_functions()
    for required in ("ar_reduce_bcast", "ar_push", "ar_twoshot_ag_copy", "ar_select_algo", "ar_algo_cost_us",
                     "ar_flag_bytes", "ar_ll_wire_bytes", "ar_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", car.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\sT\s(ar_\w+)$", out.stdout, re.M))
    missing = [f for f in declared_functions() if f not in exported]
    assert missing == []
    for f in declared_functions():
        assert hasattr(car.lib, f)


def test_library_is_gfx950_only():
    """The embedded offload bundle (built here) names the gfx950 target and no other GPU target."""
    blob = open(car.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"hipv4-amdgcn-amd-amdhsa--(gfx[0-9a-f]+)", blob))
    assert targets == {b"gfx950"}


def test_flag_bytes_layout():
    for n in range(2, 17):
        assert car.flag_bytes(n) == 128 + n * (car.AR_SLOTS_PER_RANK + car.AR_EPOCH_COPIES) * 4
    assert car.flag_bytes(1) == 0 and car.flag_bytes(17) == 0


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 119, 120, 121, 240, 65536, 1 << 20, 12345])
def test_wire_bytes_agree_with_oracle_model(S):
    for proto in ("ll", "ll128"):
        assert car.ll_wire_bytes(proto, S) == model.ll_wire_bytes(proto, S) == accounting.wire_bytes(proto, S)


def test_poll_timeout_setting():
    old = car.get_poll_timeout_ns()
    car.set_poll_timeout_ns(12345)
    assert car.get_poll_timeout_ns() == 12345
    car.set_poll_timeout_ns(0)  # back to the default
    assert car.get_poll_timeout_ns() == 1_000_000_000
    car.set_poll_timeout_ns(old)


# ---- synchronous argument checks with fake device addresses (never launched) --
L = car.lib
A = 0x7F0000000000  # 16-byte aligned fake addresses, far apart


def arr(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def fake_ins(n, stride=1 << 30, base=A):
    return arr(*[base + i * stride for i in range(n)])


NUL = ctypes.c_void_p(0)


def test_oneshot_argument_errors():
    ins = fake_ins(4)
    out = A + 100 * (1 << 30)
    assert L.ar_oneshot(ins, 1, out, 16, 0, NUL) == car.AR_ERR_ARG  # n < 2
    assert L.ar_oneshot(fake_ins(17), 17, out, 16, 0, NUL) == car.AR_ERR_ARG  # n > 16
    assert L.ar_oneshot(ins, 4, out, 0, 0, NUL) == car.AR_ERR_ARG  # numel 0
    assert L.ar_oneshot(ins, 4, out, 16, 2, NUL) == car.AR_ERR_ARG  # dtype
    assert L.ar_oneshot(ins, 4, None, 16, 0, NUL) == car.AR_ERR_ARG
    assert L.ar_oneshot(arr(A, 0, A + (2 << 30), A + (3 << 30)), 4, out, 16, 0, NUL) == car.AR_ERR_ARG
    assert L.ar_oneshot(ins, 4, out + 8, 16, 0, NUL) == car.AR_ERR_ALIGN
    assert L.ar_oneshot(arr(A + 4, A + (1 << 30), A + (2 << 30), A + (3 << 30)), 4, out, 16, 0, NUL) == \
        car.AR_ERR_ALIGN
    # output overlapping an input (the reference's non-graph in-place case)
    assert L.ar_oneshot(ins, 4, A + 16, 16, 0, NUL) == car.AR_ERR_ALIAS
    assert L.ar_oneshot(ins, 4, A - 16 * 4 + 16, 16, 0, NUL) == car.AR_ERR_ALIAS
    # touching but not overlapping is fine -> would launch; not called here


def test_size_limit_is_16_GiB_per_rank():
    ins = fake_ins(2, stride=1 << 40)
    out = A + (8 << 40)
    # 2^34 bytes + one element is refused before anything else happens
    assert L.ar_oneshot(ins, 2, out, (1 << 34) // 4 + 1, 0, NUL) == car.AR_ERR_ARG
    assert L.ar_oneshot(ins, 2, out, (1 << 34) // 2 + 1, 1, NUL) == car.AR_ERR_ARG


def test_reduce_bcast_argument_errors():
    n = 4
    ins, outs = fake_ins(n), fake_ins(n, base=A + (64 << 30))
    f = L.ar_reduce_bcast
    assert f(ins, 1, outs, 64, 0, 0, 1, NUL) == car.AR_ERR_ARG  # n < 2
    assert f(ins, n, outs, 0, 0, 0, n, NUL) == car.AR_ERR_ARG  # numel 0
    assert f(ins, n, outs, 64, 2, 0, n, NUL) == car.AR_ERR_ARG  # dtype
    assert f(ins, n, outs, 64, 0, 2, 2, NUL) == car.AR_ERR_ARG  # empty rank range
    assert f(ins, n, outs, 64, 0, 0, n + 1, NUL) == car.AR_ERR_ARG
    assert f(ins, n, None, 64, 0, 0, n, NUL) == car.AR_ERR_ARG
    assert f(ins, n, arr(A + (64 << 30), 0, A + (66 << 30), A + (67 << 30)), 64, 0, 0, n, NUL) == car.AR_ERR_ARG
    assert f(ins, n, arr(A + (64 << 30) + 8, A + (65 << 30), A + (66 << 30), A + (67 << 30)), 64, 0, 0, n, NUL) \
        == car.AR_ERR_ALIGN
    # an output overlapping an input, and two outputs overlapping each other
    assert f(ins, n, arr(A + 16, A + (65 << 30), A + (66 << 30), A + (67 << 30)), 64, 0, 0, n, NUL) == car.AR_ERR_ALIAS
    assert f(ins, n, arr(A + (64 << 30), A + (64 << 30) + 128, A + (66 << 30), A + (67 << 30)), 64, 0, 0, n, NUL) \
        == car.AR_ERR_ALIAS


def test_push_argument_errors():
    src = fake_ins(2)
    dst = fake_ins(4, base=A + (64 << 30))
    f = L.ar_push
    assert f(src, 0, dst, 2, 64, 0, NUL) == car.AR_ERR_ARG  # no sender
    assert f(src, 2, dst, 0, 64, 0, NUL) == car.AR_ERR_ARG  # no destination
    assert f(src, 2, dst, 17, 64, 0, NUL) == car.AR_ERR_ARG
    assert f(src, 2, dst, 2, 0, 0, NUL) == car.AR_ERR_ARG
    assert f(src, 2, None, 2, 64, 0, NUL) == car.AR_ERR_ARG
    assert f(src, 2, arr(A + (64 << 30) + 4, A + (65 << 30), A + (66 << 30), A + (67 << 30)), 2, 64, 0, NUL) \
        == car.AR_ERR_ALIGN
    assert f(src, 2, arr(A + (64 << 30), A + (65 << 30), A + 64, A + (67 << 30)), 2, 64, 0, NUL) == car.AR_ERR_ALIAS
    assert f(src, 2, arr(A + (64 << 30), A + (64 << 30) + 16, A + (66 << 30), A + (67 << 30)), 2, 64, 0, NUL) \
        == car.AR_ERR_ALIAS


def test_ag_copy_argument_errors():
    n = 4
    segs, outs = fake_ins(n), fake_ins(n, base=A + (64 << 30))
    flags = A + (200 << 30)
    g = L.ar_twoshot_ag_copy
    assert g(segs, n, None, 64, 0, 0, n, flags, 1, NUL) == car.AR_ERR_ARG
    assert g(segs, n, outs, 66, 0, 0, n, flags, 1, NUL) == car.AR_ERR_DIVISIBLE
    assert g(segs, n, outs, 64, 0, 3, 3, flags, 1, NUL) == car.AR_ERR_ARG
    assert g(segs, n, outs, 64, 0, 0, n, flags + 4, 1, NUL) == car.AR_ERR_ALIGN


def test_twoshot_argument_errors():
    n = 4
    ins, segs = fake_ins(n), fake_ins(n, base=A + (64 << 30))
    outs = fake_ins(n, base=A + (128 << 30))
    flags = A + (200 << 30)
    f = L.ar_twoshot_rs
    # step 0 is valid (the step id kept in the flag region): not called here
    assert f(ins, n, segs, 64, 0, 2, 2, flags, 1, outs, NUL) == car.AR_ERR_ARG  # empty rank range
    assert f(ins, n, segs, 64, 0, 0, n + 1, flags, 1, outs, NUL) == car.AR_ERR_ARG
    assert f(ins, n, segs, 64, 0, -1, n, flags, 1, outs, NUL) == car.AR_ERR_ARG
    assert f(ins, n, segs, 64, 0, 0, n, None, 1, outs, NUL) == car.AR_ERR_ARG
    assert f(ins, n, segs, 66, 0, 0, n, flags, 1, outs, NUL) == car.AR_ERR_DIVISIBLE  # 66 % 4
    assert f(ins, n, segs, 4 * 6, 0, 0, n, flags, 1, outs, NUL) == car.AR_ERR_DIVISIBLE  # 24-byte segments
    assert f(ins, n, segs, 64, 0, 0, n, flags + 4, 1, outs, NUL) == car.AR_ERR_ALIGN
    # a segment inside an input
    bad_segs = arr(A + 64, A + (65 << 30), A + (66 << 30), A + (67 << 30))
    assert f(ins, n, bad_segs, 64, 0, 0, n, flags, 1, outs, NUL) == car.AR_ERR_ALIAS
    # flags overlapping an output
    assert f(ins, n, segs, 64, 0, 0, n, A + (128 << 30) + 16, 1, outs, NUL) == car.AR_ERR_ALIAS
    g = L.ar_twoshot_ag
    assert g(segs, n, None, 64, 0, 0, n, flags, 1, NUL) == car.AR_ERR_ARG
    # step 0 is valid for the all-gather too (auto): not called here
    assert g(segs, n, arr(A + (128 << 30), A + 8, A + (130 << 30), A + (131 << 30)), 64, 0, 0, n, flags, 1, NUL) \
        == car.AR_ERR_ALIGN


def test_ll_argument_errors():
    n = 3
    srcs, wires = fake_ins(n), fake_ins(n, base=A + (64 << 30))
    assert L.ar_ll_pack(srcs, wires, 0, 10, 0, 0, 1, NUL) == car.AR_ERR_ARG  # count 0
    assert L.ar_ll_pack(srcs, wires, n, 10, 0, 2, 1, NUL) == car.AR_ERR_ARG  # proto
    assert L.ar_ll_pack(srcs, arr(A + (64 << 30) + 8, A + (65 << 30), A + (66 << 30)), n, 10, 0, 0, 1, NUL) == \
        car.AR_ERR_ALIGN
    # wire of 10 fp32 (80 bytes) overlapping the source
    assert L.ar_ll_pack(srcs, arr(A + 32, A + (65 << 30), A + (66 << 30)), n, 10, 0, 0, 1, NUL) == car.AR_ERR_ALIAS
    out, flags = A + (100 << 30), A + (101 << 30)
    for fn in (L.ar_ll_reduce_unpack, L.ar_ll128_reduce_unpack):
        assert fn(wires, 1, out, 10, 0, 1, flags, NUL) == car.AR_ERR_ARG
        assert fn(wires, n, out, 10, 0, 0, flags, NUL) == car.AR_ERR_ARG
        assert fn(wires, n, out, 10, 0, 1, None, NUL) == car.AR_ERR_ARG
        assert fn(wires, n, out + 4, 10, 0, 1, flags, NUL) == car.AR_ERR_ALIGN
        assert fn(wires, n, A + (64 << 30) + 16, 10, 0, 1, flags, NUL) == car.AR_ERR_ALIAS
    assert L.ar_flag_barrier_reset(None, 4, NUL) == car.AR_ERR_ARG
    assert L.ar_flag_barrier_reset(flags, 1, NUL) == car.AR_ERR_ARG
    assert L.ar_flag_barrier_reset(flags + 8, 4, NUL) == car.AR_ERR_ALIGN


def test_twoshot_ll_argument_errors():
    n = 4
    ins = fake_ins(n)
    segw = fake_ins(n, base=A + (64 << 30))
    outs = fake_ins(n, base=A + (128 << 30))
    flags = A + (200 << 30)
    f = L.ar_twoshot_ll
    numel = 4 * 64  # 64 fp32 per segment: 256 data bytes, a 512-byte LL wire
    assert f(None, n, segw, numel, 0, 0, n, flags, 1, outs, NUL) == car.AR_ERR_ARG
    assert f(ins, n, None, numel, 0, 0, n, flags, 1, outs, NUL) == car.AR_ERR_ARG
    assert f(ins, 1, segw, numel, 0, 0, 1, flags, 1, outs, NUL) == car.AR_ERR_ARG
    assert f(ins, n, segw, numel, 0, 2, 1, flags, 1, outs, NUL) == car.AR_ERR_ARG  # r0 >= r1
    assert f(ins, n, segw, 4 * 3, 0, 0, n, flags, 1, outs, NUL) == car.AR_ERR_DIVISIBLE  # 12-byte segments
    assert f(ins, n, arr(A + (64 << 30) + 8, A + (65 << 30), A + (66 << 30), A + (67 << 30)), numel, 0, 0, n,
             flags, 1, outs, NUL) == car.AR_ERR_ALIGN
    # segw[0] is 512 bytes: an input 256 bytes in overlaps its second half (the first 256 would not tell)
    assert f(arr(A + (64 << 30) + 256, A + (1 << 30), A + (2 << 30), A + (3 << 30)), n, segw, numel, 0, 0, n,
             flags, 1, outs, NUL) == car.AR_ERR_ALIAS


def test_ll_allreduce_argument_errors():
    n = 3
    src = A + (90 << 30)
    wires = fake_ins(n, base=A + (64 << 30))  # 1 GiB apart
    out, flags = A + (100 << 30), A + (101 << 30)
    f = L.ar_ll_allreduce
    for proto in (0, 1):
        assert f(src, wires, 1, 0, out, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ARG  # n
        assert f(src, wires, n, -1, out, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ARG  # me
        assert f(src, wires, n, n, out, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ARG
        assert f(src, wires, n, 1, out, 0, 0, proto, 1, flags, NUL) == car.AR_ERR_ARG  # numel 0
        assert f(None, wires, n, 1, out, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ARG
        assert f(src, wires, n, 1, out, 10, 0, proto, 1, None, NUL) == car.AR_ERR_ARG
        assert f(src, wires, n, 1, out, 10, 2, proto, 1, flags, NUL) == car.AR_ERR_ARG  # dtype
        assert f(src + 4, wires, n, 1, out, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ALIGN
        assert f(src, wires, n, 1, out + 8, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ALIGN
        assert f(src, arr(A + (64 << 30), A + (65 << 30) + 4, A + (66 << 30)), n, 1, out, 10, 0, proto, 1, flags,
                 NUL) == car.AR_ERR_ALIGN
        # out (40 bytes) over the source; the source over rank me's (written) wire
        assert f(src, wires, n, 1, src + 16, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ALIAS
        assert f(A + (65 << 30) + 16, wires, n, 1, out, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ALIAS
        # out over a peer's (read) wire
        assert f(src, wires, n, 1, A + (66 << 30) + 16, 10, 0, proto, 1, flags, NUL) == car.AR_ERR_ALIAS
    assert f(src, wires, n, 1, out, 10, 0, 2, 1, flags, NUL) == car.AR_ERR_ARG  # proto


def test_status_strings():
    for code in range(7):
        assert L.ar_status_string(code).decode()
    assert "timed out" in L.ar_status_string(car.AR_ERR_TIMEOUT | (1 << 8) | (3 << 16)).decode()
    assert car.decode_status(5 | (2 << 8) | (7 << 16)) == (5, 2, 7)


def test_accounting_matches_oracle_model():
    for n in (2, 8, 16):
        for S in (16384, 1 << 20):
            assert accounting.oneshot(n, S) == model.hbm_bytes("oneshot", S, n)
            assert accounting.twoshot(n, S, 1) == model.hbm_bytes("twoshot_share", S, n)
            assert accounting.twoshot(n, S, n) == model.hbm_bytes("twoshot_full", S, n)
            assert accounting.twoshot_ll(n, S, 1) == model.hbm_bytes("twoshot_ll_share", S, n)
            assert accounting.twoshot_ll(n, S, 1, "ll128") == model.hbm_bytes("twoshot_ll128_share", S, n)
            # the fused kernel's own count: the rank's own segment is never read back
            kr, kw = accounting.twoshot_kernel(n, S, 1)
            assert (kr + S // n, kw) == accounting.twoshot(n, S, 1)
            for proto in ("ll", "ll128"):
                assert accounting.ll_pack(proto, S) == model.hbm_bytes("ll_pack", S, n, proto)
                assert accounting.ll_reduce(proto, n, S) == model.hbm_bytes("ll_reduce", S, n, proto)
                assert accounting.ll_allreduce(proto, n, S) == model.hbm_bytes("ll_allreduce", S, n, proto)


# ---- algorithm selector (host logic) ------------------------------------------
def _sizes():
    # grid points, points between them, below and above the measured range
    return [1 << 10, 16 << 10, 24 << 10, 200 << 10, 1 << 20, 1_300_000, 3 << 20, 5 << 20, 64 << 20, 100 << 20,
            1 << 30]


@pytest.mark.parametrize("n", list(range(2, 17)))
@pytest.mark.parametrize("sync_us", [0.0, 1.5, 25.0])
def test_selector_picks_the_least_modelled_cost(n, sync_us):
    import torch
    for dt, es in ((torch.bfloat16, 2), (torch.float32, 4)):
        for S in _sizes():
            numel = max(1, S // es)
            costs = {a: car.algo_cost_us(a, n, numel, dt, sync_us) for a in car.ALGOS}
            ok = {a: c for a, c in costs.items() if c is not None}
            want = min(ok, key=lambda a: (ok[a], car.ALGOS.index(a)))
            assert car.select_algo(n, numel, dt, sync_us) == want, (n, S, dt, sync_us, costs)
            assert all(c > 0 for c in ok.values())


def test_selector_cost_model_terms():
    import torch
    bf = torch.bfloat16
    # sync terms: 2 per call for the one-shot, 4 for the two-shot, none for LL / LL128,
    # 2 for the two-shot under LL and LL128 (start and end; the barrier is in the lines)
    assert len(car.ALGOS) == 8
    for a, k in zip(car.ALGOS, (2, 4, 0, 0, 2, 2, 2, 2)):
        assert car.algo_cost_us(a, 8, 1 << 20, bf, 10.0) == pytest.approx(car.algo_cost_us(a, 8, 1 << 20, bf, 0.0) + 10 * k)
    # flat below the grid, increasing in size above it, linear beyond the last point
    for a in car.ALGOS:
        assert car.algo_cost_us(a, 8, 64, bf) == car.algo_cost_us(a, 8, 8 << 10, bf)
        c = [car.algo_cost_us(a, 8, (s << 20) // 2, bf) for s in (64, 128, 192)]
        assert c[2] - c[1] == pytest.approx(c[1] - c[0], rel=1e-6) and c[2] > c[1] > c[0]
    # bf16 and fp32 of the same byte count cost the same
    assert car.algo_cost_us("twoshot", 8, 1 << 20, bf) == car.algo_cost_us("twoshot", 8, 1 << 19, torch.float32)


def test_selector_regimes():
    """What the measured table must show.  With no cross-GPU sync cost (one
    GPU): small messages take the one-shot or the reduce-broadcast (both one
    launch-bound pass), large ones the reduce-broadcast, which moves the
    fewest bytes (S read, S written per rank) with no barrier; two ranks never
    take the two-shot ([NCCL] 练习 2: at n = 2 both move S, and the one-shot
    saves a synchronisation); the push never wins (it is a copy plus the
    one-shot, with the one-shot's synchronisations).  A large sync cost moves
    small messages to a flag protocol."""
    import torch
    bf = torch.bfloat16
    for n in range(2, 17):
        assert car.select_algo(n, 8 << 10, bf) in ("oneshot", "bcast"), n
        big = (64 << 20) // 2
        big -= big % (8 * n)
        assert car.select_algo(n, big, bf) == "bcast", n
        assert car.select_algo(n, 8 << 10, bf, sync_us=20.0) in ("ll", "ll128"), n
        for S in _sizes():
            for sync in (0.0, 1.5, 25.0):
                assert car.select_algo(n, S // 2, bf, sync) != "push"
    for S in _sizes():
        assert car.select_algo(2, S // 2, bf) != "twoshot"


def test_selector_never_picks_an_inapplicable_two_shot():
    import torch
    bf = torch.bfloat16
    assert car.algo_cost_us("twoshot", 8, (16 << 20) // 2 + 1, bf) is None
    assert car.algo_cost_us("twoshot", 16, 16 * 4, bf) is None  # 8-byte segments
    assert car.algo_cost_us("twoshot", 8, (16 << 20) // 2, bf) is not None
    assert car.algo_cost_us("twoshot_ll", 8, (16 << 20) // 2 + 1, bf) is None
    assert car.algo_cost_us("twoshot_ll", 8, (16 << 20) // 2, bf) is not None
    for sync in (0.0, 0.5, 3.0):  # wherever the two-shot would be cheapest, it must not be chosen
        assert car.select_algo(8, (16 << 20) // 2 + 1, bf, sync) not in ("twoshot", "twoshot_ll")
    assert car.lib.ar_select_algo(1, 10, 0, 0.0) == -car.AR_ERR_ARG
    assert car.lib.ar_select_algo(17, 10, 0, 0.0) == -car.AR_ERR_ARG
    assert car.lib.ar_select_algo(8, 0, 0, 0.0) == -car.AR_ERR_ARG
    assert car.lib.ar_select_algo(8, 10, 5, 0.0) == -car.AR_ERR_ARG
    assert car.lib.ar_select_algo(8, 10, 0, -1.0) == -car.AR_ERR_ARG
    assert car.lib.ar_select_algo(8, 10, 0, float("nan")) == -car.AR_ERR_ARG
    assert car.lib.ar_algo_cost_us(7, 8, 10, 0, 0.0) < 0
    assert car.lib.ar_algo_cost_us(-1, 8, 10, 0, 0.0) < 0


def test_import_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: a copy of the package without libar.so refuses to import."""
    import shutil
    import sys as _sys
    pkg = tmp_path / "custom_all_reduce_amd"
    pkg.mkdir()
    src = os.path.join(ROOT, "custom_all_reduce_amd")
    for f in os.listdir(src):
        if f.endswith(".py"):
            shutil.copy(os.path.join(src, f), pkg / f)
    r = subprocess.run([_sys.executable, "-c", "import custom_all_reduce_amd"], cwd=tmp_path, capture_output=True,
                       text=True, timeout=120, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "libar.so is missing" in r.stderr and "no CPU fallback" in r.stderr


def test_overlap_check_finds_one_planted_overlap_anywhere():
    """Random layouts of 2..16 senders x destinations with exactly one planted
    overlap (a destination inside a source, or two destinations sharing bytes)
    are refused wherever the overlap sits in address order.  Every layout
    holds an overlap, so no call here gets past validation."""
    import random
    rnd = random.Random(5)
    S = 4096
    for trial in range(300):
        nsrc, ndst = rnd.randint(1, 16), rnd.randint(2, 16)
        slots = rnd.sample(range(1, 100000), nsrc + nsrc * ndst)  # distinct, far apart (S-byte units * 4)
        addrs = [A + s * 4 * S for s in slots]
        src, dst = addrs[:nsrc], addrs[nsrc:]
        k = rnd.randrange(len(dst))
        if rnd.random() < 0.5:
            dst[k] = rnd.choice(src) + 16 * rnd.randint(0, S // 16 - 1)  # inside a source
        else:
            other = rnd.choice([d for i, d in enumerate(dst) if i != k])
            dst[k] = other + 16 * rnd.randint(0, S // 16 - 1)  # sharing bytes with another destination
        assert L.ar_push(arr(*src), nsrc, arr(*dst), ndst, S // 2, 1, NUL) == car.AR_ERR_ALIAS, trial


# ---- size checks of the binding (host logic, CPU tensors) ----------------------
def test_size_checks_reject_undersized_buffers():
    """The C ABI sees only pointers, so the binding checks every buffer's size
    before a call enqueues anything: undersized segments, segment wires, flag
    regions and wrong-sized outputs raise ValueError; exact sizes pass."""
    import torch

    n, m = 8, 8 * 100
    numel = n * m
    bf = torch.bfloat16
    ins = [torch.zeros(numel, dtype=bf) for _ in range(n)]
    segs = [torch.zeros(m, dtype=bf) for _ in range(n)]
    outs = [torch.zeros(numel, dtype=bf)] + [None] * (n - 1)
    flags = torch.zeros(car.flag_bytes(n) // 4, dtype=torch.int32)
    car._twoshot_sizes(ins, segs, flags, outs)  # exact sizes
    with pytest.raises(ValueError):
        car._twoshot_sizes(ins, segs[:-1] + [torch.zeros(m - 8, dtype=bf)], flags, outs)
    with pytest.raises(ValueError):
        car._twoshot_sizes(ins, segs, flags[:-1], outs)
    with pytest.raises(ValueError):
        car._twoshot_sizes(ins, segs, flags, [torch.zeros(numel - 1, dtype=bf)] + outs[1:])
    with pytest.raises(ValueError):
        car._twoshot_sizes(ins[:-1] + [torch.zeros(numel, dtype=torch.float32)], segs, flags, outs)
    for proto in ("ll", "ll128"):
        W = car.ll_wire_bytes(proto, m * 2)
        wires = [torch.zeros(W, dtype=torch.uint8) for _ in range(n)]
        car._twoshot_sizes(ins, wires, flags, outs, seg_proto=proto)
        with pytest.raises(ValueError):
            car._twoshot_sizes(ins, wires[:-1] + [torch.zeros(W - 1, dtype=torch.uint8)], flags, outs,
                               seg_proto=proto)
    # LL128 wires are larger than LL wires of the same message only past 120 bytes
    assert car.ll_wire_bytes("ll128", m * 2) < car.ll_wire_bytes("ll", m * 2)
    with pytest.raises(ValueError):
        car._need_bytes([torch.zeros(127, dtype=torch.uint8)], car.STATUS_BYTES, "flags")


def test_oneshot_rmsnorm_argument_errors():
    f0 = L.ar_oneshot_rmsnorm

    def f(*a):  # without a workspace (its checks are below)
        return f0(*a[:-1], None, a[-1])

    n, rows, hidden = 4, 8, 4096
    ins = fake_ins(n)
    res, w, ro, out = A + (64 << 30), A + (65 << 30), A + (66 << 30), A + (67 << 30)
    assert f(ins, 1, res, w, ro, out, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ARG  # n < 2
    assert f(ins, n, res, w, ro, out, 0, hidden, 1e-6, 1, NUL) == car.AR_ERR_ARG  # no rows
    assert f(ins, n, res, w, ro, out, rows, 0, 1e-6, 1, NUL) == car.AR_ERR_ARG  # no columns
    assert f(ins, n, res, w, ro, out, rows, hidden, 1e-6, 2, NUL) == car.AR_ERR_ARG  # dtype
    assert f(ins, n, None, w, ro, out, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ARG
    assert f(ins, n, res, None, ro, out, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ARG
    for eps in (-1e-6, float("nan"), float("inf")):
        assert f(ins, n, res, w, ro, out, rows, hidden, eps, 1, NUL) == car.AR_ERR_ARG
    # a row of at most 64 KiB: 32768 bf16 or 16384 fp32 elements
    assert f(ins, n, res, w, ro, out, rows, 32768 + 8, 1e-6, 1, NUL) == car.AR_ERR_ARG
    assert f(ins, n, res, w, ro, out, rows, 16384 + 4, 1e-6, 0, NUL) == car.AR_ERR_ARG
    # the 16 GiB per rank limit
    assert f(ins, n, res, w, ro, out, (1 << 34) // (2 * 8) + 1, 8, 1e-6, 1, NUL) == car.AR_ERR_ARG
    assert f(ins, n, res + 8, w, ro, out, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ALIGN
    assert f(ins, n, res, w + 8, ro, out, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ALIGN
    # a row must be whole 16-byte vectors
    assert f(ins, n, res, w, ro, out, rows, 4100, 1e-6, 1, NUL) == car.AR_ERR_DIVISIBLE
    assert f(ins, n, res, w, ro, out, rows, 4098, 1e-6, 0, NUL) == car.AR_ERR_DIVISIBLE
    # out overlapping an input, the weight or residual_out; residual_out partly over the residual
    assert f(ins, n, res, w, ro, A + 16, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ALIAS
    assert f(ins, n, res, w, ro, w + 64, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ALIAS
    assert f(ins, n, res, w, ro, ro + 1024, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ALIAS
    assert f(ins, n, res, w, res + 1024, out, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ALIAS
    assert f(ins, n, res, w, A + (1 << 30), out, rows, hidden, 1e-6, 1, NUL) == car.AR_ERR_ALIAS
    # the workspace: aligned, and not overlapping any other buffer
    ws = A + (68 << 30)
    assert f0(ins, n, res, w, ro, out, rows, hidden, 1e-6, 1, ws + 4, NUL) == car.AR_ERR_ALIGN
    assert f0(ins, n, res, w, ro, out, rows, hidden, 1e-6, 1, out + 64, NUL) == car.AR_ERR_ALIAS
    assert f0(ins, n, res, w, ro, out, rows, hidden, 1e-6, 1, w, NUL) == car.AR_ERR_ALIAS


def test_twoshot_rmsnorm_argument_errors():
    # every check happens before anything is enqueued, so fake addresses serve
    n, rows, hidden = 4, 8, 4096
    ins = fake_ins(n)
    res = fake_ins(n, base=A + (64 << 30))
    segs = fake_ins(n, base=A + (80 << 30))
    ro = fake_ins(n, base=A + (96 << 30))
    out = fake_ins(n, base=A + (112 << 30))
    w, fl = A + (128 << 30), A + (129 << 30)

    def f(ins=ins, n=n, res=res, w=w, segs=segs, ro=ro, out=out, rows=rows, hidden=hidden, eps=1e-6, dt=1, r0=0,
          r1=1, fl=fl, step=0):
        return L.ar_twoshot_rmsnorm(ins, n, res, w, segs, ro, out, rows, hidden, eps, dt, r0, r1, fl, step, NUL)

    assert f(n=1) == car.AR_ERR_ARG
    assert f(rows=0) == car.AR_ERR_ARG
    assert f(hidden=0) == car.AR_ERR_ARG
    assert f(dt=2) == car.AR_ERR_ARG
    assert f(w=None) == car.AR_ERR_ARG
    assert f(fl=None) == car.AR_ERR_ARG
    assert f(r0=2, r1=2) == car.AR_ERR_ARG
    assert f(r0=3, r1=5, ro=None, out=None) == car.AR_ERR_ARG  # past n
    assert f(r0=0, r1=2) == car.AR_ERR_ARG  # an all-gather for two ranks in one launch
    assert f(ro=None) == car.AR_ERR_ARG  # out without residual_out
    for eps in (-1e-6, float("nan"), float("inf")):
        assert f(eps=eps) == car.AR_ERR_ARG
    assert f(hidden=32768 + 8) == car.AR_ERR_ARG  # a row of more than 64 KiB
    assert f(segs=fake_ins(n, base=A + (80 << 30) + 8)) == car.AR_ERR_ALIGN
    assert f(fl=fl + 4) == car.AR_ERR_ALIGN
    assert f(w=w + 8) == car.AR_ERR_ALIGN
    assert f(rows=6) == car.AR_ERR_DIVISIBLE  # rows split over the ranks
    assert f(hidden=4100) == car.AR_ERR_DIVISIBLE  # whole 16-byte vectors per row
    # overlaps: an output over an input; residual_out over the residual (no in-place
    # update in this form); a peer's segment, read by the all-gather, over the output
    assert f(out=fake_ins(n, base=A + 16)) == car.AR_ERR_ALIAS
    assert f(ro=res) == car.AR_ERR_ALIAS
    assert f(segs=arr(*([segs[0]] + [out[0] + 1024] + list(segs)[2:]))) == car.AR_ERR_ALIAS
    # the flag region over the weight
    assert f(fl=w) == car.AR_ERR_ALIAS


@pytest.mark.parametrize("n, rows, hidden, dt", [(8, 512, 8192, 1), (8, 4096, 8192, 1), (16, 32, 16384, 1),
                                                 (4, 32, 64, 1), (2, 2060, 8, 1), (8, 64, 4096, 0)])
def test_rmsnorm_segment_bytes_cover_the_layout(n, rows, hidden, dt):
    # a rank's segment: G out rows and G residual_out rows, G P 8-byte partial slots and G P
    # done flags, then (16-byte aligned) the auto ids' epoch words: G P per rank for parts of
    # rows, tiles x wavefronts per workgroup per rank for a workgroup per row
    es = 4 if dt == 0 else 2
    V, G = hidden * es // 16, rows // n
    P = -(-V // 64)
    if G < 256 and (n + 1) * V * 16 >= 128 << 10:
        words = n * G * P
    else:
        tile = -(-G // 1024)
        vpt = 1 if V <= 1024 else (2 if V <= 2048 else 4)
        words = n * -(-G // tile) * -(-(-(-V // vpt)) // 64)
    need = -(-(32 * G * V + 12 * G * P) // 16) * 16 + 4 * words
    got = L.ar_rmsnorm_segment_bytes(n, rows, hidden, dt)
    assert got % 16 == 0 and need <= got < need + 16
    assert L.ar_rmsnorm_segment_bytes(n, rows + 1, hidden, dt) == 0  # rows that do not split


def test_rmsnorm_workspace_size():
    # 32 status words, 1024 epochs and 1024 8-byte slots
    assert car.rmsnorm_workspace_bytes() == (32 + 1024 + 2 * 1024) * 4
