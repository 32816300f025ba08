"""Pin strength: plant plausible mistakes in a copy of the C oracle (on the
CPU) and check that the pins catch every one of them.  The clean oracle must
pass the same checks.  CPU only."""
from __future__ import annotations

import os
import tempfile

import numpy as np
import pytest

import oracle
import synth

SRC = os.path.join(os.path.dirname(oracle.__file__), "ar_oracle.c")

# (name, exact text in ar_oracle.c, replacement) -- each one a mistake that a
# careless restatement of the pages could make.
MUTANTS = [
    ("accumulator_starts_at_rank0",
     "        float acc = 0.0f;\n        for (int i = 0; i < n; ++i)\n            acc = acc + load_elem(in[i], k, dtype);\n        store_elem(out, k, dtype, acc);",
     "        float acc = load_elem(in[0], k, dtype);\n        for (int i = 1; i < n; ++i)\n            acc = acc + load_elem(in[i], k, dtype);\n        store_elem(out, k, dtype, acc);"),
    ("truncate_instead_of_round", "        kept += 1u;", "        kept += 0u;"),
    ("ties_away_from_zero", "(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    ("nan_not_quieted", "return (uint16_t)(kept | 0x0040u);", "return (uint16_t)(kept);"),
    ("dropped_last_rank",
     "        for (int i = 0; i < n; ++i)\n            acc = acc + load_elem(in[i], k, dtype);\n        store_elem(out, k, dtype, acc);",
     "        for (int i = 0; i < n - 1; ++i)\n            acc = acc + load_elem(in[i], k, dtype);\n        store_elem(out, k, dtype, acc);"),
    ("rank_added_twice",
     "        for (int i = 0; i < n; ++i)\n            acc = acc + load_elem(in[i], k, dtype);\n        store_elem(out, k, dtype, acc);",
     "        for (int i = 0; i < n; ++i)\n            acc = acc + load_elem(in[i > 0 ? i : 1], k, dtype);\n        store_elem(out, k, dtype, acc);"),
    ("twoshot_wrong_segment", "load_elem(in[i], (size_t)r * m + k, dtype)",
     "load_elem(in[i], (size_t)((r + 1) % n) * m + k, dtype)"),
    ("allgather_transposed", "memcpy((char*)out[r] + (size_t)j * m * es, seg[j], m * es);",
     "memcpy((char*)out[j] + (size_t)r * m * es, seg[(j + 1) % n], m * es);"),
    ("ring_wrong_schedule",
     "            int c = ((r - s) % n + n) % n;\n            size_t lo = (size_t)c * numel / (size_t)n, hi = (size_t)(c + 1) * numel / (size_t)n;\n            memcpy(msg",
     "            int c = ((r + s) % n + n) % n;\n            size_t lo = (size_t)c * numel / (size_t)n, hi = (size_t)(c + 1) * numel / (size_t)n;\n            memcpy(msg"),
    ("ll_flag_first", "            memcpy(line + 4, &f, 4);", "            memcpy(line, &f, 4);"),
    ("ll128_payload_124", "return proto == OR_LL ? 4u : 120u;", "return proto == OR_LL ? 4u : 124u;"),
    ("flag_compare_equal", "if (line_flag(proto, line) < (uint64_t)step) {",
     "if (line_flag(proto, line) != (uint64_t)step) {"),
    ("rms_over_hidden_minus_one", "double ms = sumsq / (double)hidden;", "double ms = sumsq / (double)(hidden - 1);"),
    ("eps_outside_the_root", "double inv = 1.0 / sqrt(ms + eps);", "double inv = 1.0 / (sqrt(ms) + eps);"),
    ("residual_added_first",
     "            float acc = 0.0f;\n            for (int r = 0; r < n; ++r)\n                acc = acc + load_elem(in[r], e, dtype);\n            float h = acc + load_elem(residual, e, dtype);",
     "            float acc = load_elem(residual, e, dtype);\n            for (int r = 0; r < n; ++r)\n                acc = acc + load_elem(in[r], e, dtype);\n            float h = acc;"),
    ("weight_indexed_by_row", "(double)load_elem(weight, k, dtype)", "(double)load_elem(weight, i % hidden, dtype)"),
    ("normalized_from_rounded_sum", "            hrow[k] = (double)h;",
     "            hrow[k] = (double)load_elem(residual_out, e, dtype);"),
]


def _run_pins(lib):
    """A compact pass over the pins of test_oracle_pins.py, on a given build.
    Returns the names of the checks that failed."""
    bad = []
    # O1 special values (round-to-nearest-even, overflow, NaN quiet)
    xs = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, np.finfo(np.float32).max], np.float32)
    if list(oracle.f32_to_bf16(xs, lib)) != [0x3F80, 0x3F82, 0x3F81, 0x7F80]:
        bad.append("rne_special")
    nan = np.array([0x7F800001], np.uint32).view(np.float32)
    if int(oracle.f32_to_bf16(nan, lib)[0]) != 0x7FC0:
        bad.append("nan")
    # O2 integer closed form and the +0 start
    for dt in ("f32", "bf16"):
        ins = synth.rank_inputs(5, 999, dt, "int", config=0)
        got = oracle.oneshot(ins, dt, lib)
        got = got if dt == "f32" else oracle.bf16_to_f32(got)
        ints = [synth.integers_f32(999, synth.rank_seed(0, r)).astype(np.int64) for r in range(5)]
        if not np.array_equal(got, np.sum(ints, 0).astype(np.float32)):
            bad.append("int_sum_" + dt)
    z = [np.array([-0.0], np.float32)] * 3
    if oracle.oneshot(z, "f32", lib).view(np.uint32)[0] != 0:
        bad.append("plus_zero")
    # O3 = O2 bitwise
    ins = synth.rank_inputs(4, 4 * 64, "f32", "normal", config=2)
    segs, outs = oracle.twoshot(ins, "f32", lib)
    ref = oracle.oneshot(ins, "f32", lib)
    if not all(np.array_equal(o, ref) for o in outs) or not np.array_equal(np.concatenate(segs), ref):
        bad.append("twoshot")
    # O4 ring on integers
    ins = synth.rank_inputs(4, 4 * 33, "f32", "int", config=0)
    bufs, sent = oracle.ring(ins, "f32", lib)
    if not all(np.array_equal(b, ref2) for b, ref2 in zip(bufs, [oracle.oneshot(ins, "f32", lib)] * 4)):
        bad.append("ring")
    # O5/O6 layout and >= step
    msg = np.arange(250, dtype=np.uint8)
    for proto, d, lb in (("ll", 4, 8), ("ll128", 120, 128)):
        w = oracle.ll_pack(proto, msg, 9, lib)
        if w.size != lb * -(-250 // d):
            bad.append("size_" + proto)
            continue
        lines = w.reshape(-1, lb)
        pad = np.zeros(lines.shape[0] * d, np.uint8)
        pad[:250] = msg
        if not np.array_equal(lines[:, :d].reshape(-1), pad):
            bad.append("layout_" + proto)
        if not oracle.ll_unpack(proto, w, 250, 8, lib)[1]:
            bad.append("ge_" + proto)
    # O10: residual output = O2 fold + residual; unit RMS; eps in the root; weight per column;
    # the row normalized from the unrounded fp32 sum
    hidden, rows = 40, 3
    ins = synth.rank_inputs(3, rows * hidden, "f32", "normal", config=80)
    res = synth.rank_inputs(1, rows * hidden, "f32", "normal", config=81)[0]
    ro, y = oracle.oneshot_rmsnorm(ins, res, np.ones(hidden, np.float32), hidden, 0.0, "f32", lib)
    if not np.array_equal(ro, oracle.oneshot(ins, "f32", lib) + res):
        bad.append("rmsnorm_residual")
    if not np.allclose((y.reshape(rows, hidden) ** 2).mean(axis=1), 1.0, rtol=1e-12, atol=0):
        bad.append("rmsnorm_unit_rms")
    c = np.full(hidden, -2.0, np.float32)
    zero = np.zeros(hidden, np.float32)
    w = synth.rank_inputs(1, hidden, "f32", "normal", config=82)[0]
    _, y = oracle.oneshot_rmsnorm([c, zero], zero, w, hidden, 4.0, "f32", lib)
    if not np.allclose(y, -w.astype(np.float64) / np.sqrt(2.0), rtol=1e-15, atol=0):
        bad.append("rmsnorm_eps_weight")
    r0, r1 = np.zeros(8, np.float32), np.zeros(8, np.float32)
    r0[0], r1[0], r0[3] = 1.0, 2.0**-10, 2.0
    bz = oracle.f32_to_bf16(np.zeros(8, np.float32), lib)
    _, y = oracle.oneshot_rmsnorm([oracle.f32_to_bf16(r0, lib), oracle.f32_to_bf16(r1, lib)], bz,
                                  oracle.f32_to_bf16(np.ones(8, np.float32), lib), 8, 0.0, "bf16", lib)
    a = 1.0 + 2.0**-10
    if not np.isclose(y[0], a / np.sqrt((a * a + 4.0) / 8), rtol=1e-15, atol=0):
        bad.append("rmsnorm_unrounded")
    return bad


def test_clean_oracle_passes_the_compact_pins():
    assert _run_pins(oracle.load()) == []


@pytest.mark.parametrize("name, old, new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mut.c")
        so = os.path.join(d, f"libmut_{name}.so")
        with open(c, "w", encoding="utf-8") as f:
            f.write(mutated)
        oracle.build(c, so)
        lib = oracle.load(so)
        assert _run_pins(lib) != [], f"planted mistake {name} went unnoticed"
