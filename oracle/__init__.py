"""CPU oracle for the per-GPU custom all-reduce reduction kernel.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``custom_all_reduce_amd``) never imports it and shares no code with
it: the arithmetic lives in ``ar_oracle.c`` (plain C, built with
``-O2 -ffp-contract=off``) and the accounting / alpha-beta model in
``model.py``.

Functions take and return numpy arrays.  float32 data is ``np.float32``;
bfloat16 data is carried as raw ``np.uint16`` bit patterns.

Parity status of each function:
  f32_to_bf16 / bf16_to_f32 (O1)   pinned: exhaustive against torch CPU + special cases
  oneshot (O2)                     pinned: int closed form, fill closed form, fp64 bound
  twoshot (O3)                     pinned: equals O2 bitwise, RS+AG identity
  ring (O4)                        pinned on integer data and byte counts; on real-valued
                                   data its association differs from O2 -> bound only
  ll_pack / ll_unpack (O5, O6)     pinned: round trip, sizes, flag positions, efficiencies
  ll_reduce (O7)                   pinned: equals O2 of payloads; stale flag -> timeout
  FlagBarrier (O8)                 pinned: steps 1..1000, withheld flag, reset
  oneshot_rmsnorm (O10)            pinned: residual_out against O2 + residual on integer
                                   data; y by constant rows, a one-hot row, unit RMS
                                   of the normalized row, scale invariance, eps
  model.* (O9)                     pinned: the printed alpha-beta table and exercises;
                                   hbm_bytes by a byte-counting walk of each operation's
                                   steps, the stated configuration values, and the pages'
                                   remote byte counts
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ar_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
LL, LL128 = 0, 1
_DT = {"f32": F32, "bf16": BF16, F32: F32, BF16: BF16}
_PROTO = {"ll": LL, "ll128": LL128, LL: LL, LL128: LL128}

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC"]


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the C oracle with gcc (no FMA contraction, no fast-math)."""
    cmd = ["gcc", *GCC_FLAGS, *extra, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class OracleTimeout(Exception):
    """A line was not ready: the real receiver would time out here."""

    def __init__(self, rank: int, line: int):
        super().__init__(f"line {line} of rank {rank} not ready")
        self.rank = rank
        self.line = line


def _setup(lib):
    c = ctypes
    vp, sz, i32, u32 = c.c_void_p, c.c_size_t, c.c_int, c.c_uint32
    lib.oracle_f32_to_bf16_array.argtypes = [vp, vp, sz]
    lib.oracle_oneshot.argtypes = [vp, i32, vp, sz, i32]
    lib.oracle_twoshot.argtypes = [vp, i32, vp, vp, sz, i32]
    lib.oracle_ring.argtypes = [vp, i32, vp, sz, i32, vp]
    lib.oracle_ll_lines.argtypes = [i32, sz]
    lib.oracle_ll_lines.restype = sz
    lib.oracle_ll_wire_bytes.argtypes = [i32, sz]
    lib.oracle_ll_wire_bytes.restype = sz
    lib.oracle_ll_pack.argtypes = [i32, vp, sz, vp, u32]
    lib.oracle_ll_unpack.argtypes = [i32, vp, sz, vp, u32, c.POINTER(sz)]
    lib.oracle_ll_unpack.restype = i32
    lib.oracle_ll_reduce.argtypes = [i32, vp, i32, vp, sz, i32, u32, c.POINTER(i32), c.POINTER(sz)]
    lib.oracle_ll_reduce.restype = i32
    lib.oracle_oneshot_rmsnorm.argtypes = [vp, i32, vp, vp, vp, vp, sz, sz, c.c_double, i32]
    return lib


_lib_cache = {}


def load(path: str = _LIB):
    """Load (building first if absent) the oracle shared library."""
    if path in _lib_cache:
        return _lib_cache[path]
    if path == _LIB and not os.path.exists(path):
        build()
    lib = _setup(ctypes.CDLL(path))
    _lib_cache[path] = lib
    return lib


def _np_dtype(dt):
    return np.float32 if _DT[dt] == F32 else np.uint16


def _ptrs(arrays):
    return (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])


def _check(arrays, dt, numel=None):
    want = _np_dtype(dt)
    for a in arrays:
        if a.dtype != want or not a.flags["C_CONTIGUOUS"]:
            raise TypeError(f"expected contiguous {np.dtype(want)} arrays")
        if numel is not None and a.size != numel:
            raise ValueError("rank arrays must all hold numel elements")


# ---------------------------------------------------------------- O1 -------
def f32_to_bf16(x: np.ndarray, lib=None) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (see ar_oracle.c)."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_f32_to_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float32 (exact widening: the bits become the top half)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- O2 -------
def oneshot(ins, dt, lib=None) -> np.ndarray:
    """One-shot all-reduce of the rank arrays ``ins`` (one output)."""
    lib = lib or load()
    n, numel = len(ins), ins[0].size
    _check(ins, dt, numel)
    out = np.empty(numel, dtype=_np_dtype(dt))
    lib.oracle_oneshot(_ptrs(ins), n, out.ctypes.data, numel, _DT[dt])
    return out


# ---------------------------------------------------------------- O3 -------
def twoshot(ins, dt, lib=None):
    """Two-shot all-reduce.  Returns (segments, outputs): n segments of
    numel/n elements (reduce-scatter) and n full outputs (all-gather)."""
    lib = lib or load()
    n, numel = len(ins), ins[0].size
    _check(ins, dt, numel)
    if numel % n:
        raise ValueError("two-shot needs numel divisible by the rank count")
    m = numel // n
    segs = [np.empty(m, dtype=_np_dtype(dt)) for _ in range(n)]
    outs = [np.empty(numel, dtype=_np_dtype(dt)) for _ in range(n)]
    lib.oracle_twoshot(_ptrs(ins), n, _ptrs(segs), _ptrs(outs), numel, _DT[dt])
    return segs, outs


# ---------------------------------------------------------------- O4 -------
def ring(ins, dt, lib=None):
    """Step-by-step ring all-reduce.  Returns (per-rank results, bytes sent per rank)."""
    lib = lib or load()
    n, numel = len(ins), ins[0].size
    _check(ins, dt, numel)
    bufs = [np.empty(numel, dtype=_np_dtype(dt)) for _ in range(n)]
    sent = np.zeros(n, dtype=np.uint64)
    lib.oracle_ring(_ptrs(ins), n, _ptrs(bufs), numel, _DT[dt], sent.ctypes.data)
    return bufs, [int(v) for v in sent]


# ------------------------------------------------------------- O5/O6 -------
def ll_lines(proto, nbytes: int, lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_ll_lines(_PROTO[proto], int(nbytes)))


def ll_wire_bytes(proto, nbytes: int, lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_ll_wire_bytes(_PROTO[proto], int(nbytes)))


def ll_pack(proto, msg: np.ndarray, step: int, lib=None) -> np.ndarray:
    """Pack one rank's message (any contiguous array, taken as bytes)."""
    lib = lib or load()
    msg = np.ascontiguousarray(msg)
    nbytes = msg.nbytes
    wire = np.empty(ll_wire_bytes(proto, nbytes, lib), dtype=np.uint8)
    lib.oracle_ll_pack(_PROTO[proto], msg.ctypes.data, nbytes, wire.ctypes.data, int(step))
    return wire


def ll_unpack(proto, wire: np.ndarray, nbytes: int, step: int, lib=None):
    """Returns (bytes as uint8 array, ready, first not-ready line or None)."""
    lib = lib or load()
    wire = np.ascontiguousarray(wire, dtype=np.uint8)
    dst = np.zeros(int(nbytes), dtype=np.uint8)
    bad = ctypes.c_size_t(0)
    ok = lib.oracle_ll_unpack(_PROTO[proto], wire.ctypes.data, int(nbytes), dst.ctypes.data,
                              int(step), ctypes.byref(bad))
    return dst, bool(ok), (None if ok else int(bad.value))


# ---------------------------------------------------------------- O7 -------
def ll_reduce(proto, wires, numel: int, dt, step: int, lib=None) -> np.ndarray:
    """Poll (once), unpack and reduce n ranks' wire buffers.  Raises
    OracleTimeout naming the first (rank, line) whose flag is behind."""
    lib = lib or load()
    wires = [np.ascontiguousarray(w, dtype=np.uint8) for w in wires]
    out = np.empty(int(numel), dtype=_np_dtype(dt))
    br, bl = ctypes.c_int(0), ctypes.c_size_t(0)
    ok = lib.oracle_ll_reduce(_PROTO[proto], _ptrs(wires), len(wires), out.ctypes.data, int(numel),
                              _DT[dt], int(step), ctypes.byref(br), ctypes.byref(bl))
    if not ok:
        raise OracleTimeout(int(br.value), int(bl.value))
    return out


# ---------------------------------------------------------------- O8 -------
class FlagBarrier:
    """Model of the step-id flag barrier between the two-shot phases.

    Each rank owns one 32-bit flag.  Publishing step s sets it to s.  A rank
    may pass the barrier of step s once every flag is >= s (a peer that has
    already moved on counts as arrived).  Step 0 means never written; reset
    clears every flag so steps can start again at 1.  Follows the start/end
    synchronisation of the kernel shell on "0-custom-all-reduce" (实现 step 6)
    and the semaphore remark in the 协议 section of the NCCL page.
    """

    MAX_STEP = 2**32 - 1

    def __init__(self, n: int):
        self.flags = [0] * n

    def publish(self, rank: int, step: int):
        if not 1 <= step <= self.MAX_STEP:
            raise ValueError("step ids run from 1 to 2**32-1")
        self.flags[rank] = step

    def can_pass(self, step: int) -> bool:
        return all(f >= step for f in self.flags)

    def first_missing(self, step: int):
        for r, f in enumerate(self.flags):
            if f < step:
                return r
        return None

    def reset(self):
        self.flags = [0] * len(self.flags)


# ---------------------------------------------------------------- O10 ------
def oneshot_rmsnorm(ins, residual, weight, hidden: int, eps: float, dt, lib=None):
    """One-shot all-reduce + residual add + RMSNorm (see ar_oracle.c, O10).

    ``ins`` and ``residual`` hold rows * hidden elements each, ``weight``
    hidden.  Returns (residual_out in the data type, y as float64 unrounded)."""
    lib = lib or load()
    n, numel = len(ins), ins[0].size
    _check(list(ins) + [residual], dt, numel)
    _check([weight], dt, hidden)
    if hidden <= 0 or numel % hidden != 0:
        raise ValueError("numel must be a multiple of hidden")
    rows = numel // hidden
    res_out = np.empty(numel, dtype=_np_dtype(dt))
    y = np.empty(numel, dtype=np.float64)
    lib.oracle_oneshot_rmsnorm(_ptrs(ins), n, residual.ctypes.data, weight.ctypes.data, res_out.ctypes.data,
                               y.ctypes.data, rows, hidden, float(eps), _DT[dt])
    return res_out, y
