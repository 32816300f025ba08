"""Python binding of ``libar.so``, the gfx950 custom all-reduce reduction kernels.

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI declared in ``include/ar.h``.  PyTorch supplies the
device memory (tensors) and the stream.  There is no CPU fallback: if the
library is missing, importing this package raises.

Functions mirror the C entry points and take ``torch.Tensor`` arguments:

    ar_oneshot(ins, out)                         one output = sum of ranks
    ar_oneshot_rmsnorm(ins, residual, weight, residual_out, out, eps, workspace=None)
                                                 the same, + residual, then RMSNorm of each row
    ar_twoshot_rmsnorm(ins, residuals, weight, segs, flags, step, r0=0, r1=None,
                       residual_outs=None, outs=None, eps=1e-6)   its two-shot form (rows split by rank)
    ar_twoshot_rs(ins, segs, flags, step, r0=0, r1=None, outs=None)
    ar_twoshot_ag(segs, outs, flags, step, r0=0, r1=None)
    ar_ll_pack(srcs, wires, proto, step)
    ar_ll_reduce_unpack(wires, out, step, flags)
    ar_ll128_reduce_unpack(wires, out, step, flags)
    ar_ll_allreduce(src, wires, out, flags, proto, me, step)   pack + reduce, one launch
    ar_twoshot_ll(ins, segws, flags, step, r0=0, r1=None, outs=None)   two-shot, LL segments
    ar_twoshot_ll128(ins, segws, flags, step, r0=0, r1=None, outs=None) two-shot, LL128 segments
    ar_flag_barrier_reset(flags, n)
    ar_twoshot_noalloc(ins, outs)                two-shot, no allocation (library scratch)

Each call enqueues on ``stream`` (default: torch's current stream) and
raises :class:`ArError` on a synchronous error.  Asynchronous timeouts are
read with :func:`read_status` after synchronising.

The C ABI sees pointers, not sizes, so the ``prepare_*`` helpers check every
tensor's size against what the call will read or write (segments, wires,
flag regions, outputs) and raise ``ValueError`` before anything is enqueued.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import accounting  # noqa: F401  (re-exported helper module)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libar.so")

AR_OK, AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_DIVISIBLE, AR_ERR_ALIAS, AR_ERR_TIMEOUT, AR_ERR_HIP, AR_ERR_SIZE = range(8)
AR_NOALLOC_MAX_BYTES = 64 << 20
AR_F32, AR_BF16 = 0, 1
AR_PROTO_LL, AR_PROTO_LL128 = 0, 1
AR_MAX_RANKS = 16
AR_SLOTS_PER_RANK = 1024
AR_EPOCH_COPIES = 4096
PHASE_TWOSHOT_AG, PHASE_LL, PHASE_LL128, PHASE_RMSNORM = 1, 2, 3, 4

_DTYPES = {torch.float32: AR_F32, torch.bfloat16: AR_BF16}
_PROTOS = {"ll": AR_PROTO_LL, "ll128": AR_PROTO_LL128, AR_PROTO_LL: AR_PROTO_LL, AR_PROTO_LL128: AR_PROTO_LL128}


class ArError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.ar_status_string(code).decode() if _lib is not None else str(code)
        super().__init__(f"{where}: {msg} (status {code})")


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python custom_all_reduce_amd/build.py` from the repository "
            "root (there is no CPU fallback)"
        )
    lib = ctypes.CDLL(path)
    vp, sz, i32, u32, u64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64
    P = ctypes.POINTER(ctypes.c_void_p)
    lib.ar_flag_bytes.argtypes, lib.ar_flag_bytes.restype = [i32], sz
    lib.ar_ll_wire_bytes.argtypes, lib.ar_ll_wire_bytes.restype = [i32, sz], sz
    lib.ar_set_poll_timeout_ns.argtypes, lib.ar_set_poll_timeout_ns.restype = [u64], None
    lib.ar_get_poll_timeout_ns.argtypes, lib.ar_get_poll_timeout_ns.restype = [], u64
    lib.ar_status_string.argtypes, lib.ar_status_string.restype = [i32], ctypes.c_char_p
    lib.ar_oneshot.argtypes, lib.ar_oneshot.restype = [P, i32, vp, sz, i32, vp], i32
    lib.ar_oneshot_rmsnorm.argtypes = [P, i32, vp, vp, vp, vp, sz, sz, ctypes.c_float, i32, vp, vp]
    lib.ar_oneshot_rmsnorm.restype = i32
    lib.ar_rmsnorm_workspace_bytes.argtypes, lib.ar_rmsnorm_workspace_bytes.restype = [], sz
    lib.ar_twoshot_rmsnorm.argtypes = [P, i32, P, vp, P, P, P, sz, sz, ctypes.c_float, i32, i32, i32, vp, u32, vp]
    lib.ar_twoshot_rmsnorm.restype = i32
    lib.ar_rmsnorm_segment_bytes.argtypes, lib.ar_rmsnorm_segment_bytes.restype = [i32, sz, sz, i32], sz
    lib.ar_reduce_bcast.argtypes, lib.ar_reduce_bcast.restype = [P, i32, P, sz, i32, i32, i32, vp], i32
    lib.ar_push.argtypes, lib.ar_push.restype = [P, i32, P, i32, sz, i32, vp], i32
    lib.ar_twoshot_rs.argtypes, lib.ar_twoshot_rs.restype = [P, i32, P, sz, i32, i32, i32, vp, u32, P, vp], i32
    lib.ar_twoshot_ag.argtypes, lib.ar_twoshot_ag.restype = [P, i32, P, sz, i32, i32, i32, vp, u32, vp], i32
    lib.ar_twoshot_ag_copy.argtypes, lib.ar_twoshot_ag_copy.restype = [P, i32, P, sz, i32, i32, i32, vp, u32, vp], i32
    lib.ar_ll_pack.argtypes, lib.ar_ll_pack.restype = [P, P, i32, sz, i32, i32, u32, vp], i32
    lib.ar_ll_reduce_unpack.argtypes, lib.ar_ll_reduce_unpack.restype = [P, i32, vp, sz, i32, u32, vp, vp], i32
    lib.ar_ll128_reduce_unpack.argtypes = [P, i32, vp, sz, i32, u32, vp, vp]
    lib.ar_ll128_reduce_unpack.restype = i32
    lib.ar_ll_allreduce.argtypes = [vp, P, i32, i32, vp, sz, i32, i32, u32, vp, vp]
    lib.ar_ll_allreduce.restype = i32
    lib.ar_twoshot_ll.argtypes, lib.ar_twoshot_ll.restype = [P, i32, P, sz, i32, i32, i32, vp, u32, P, vp], i32
    lib.ar_twoshot_ll128.argtypes = [P, i32, P, sz, i32, i32, i32, vp, u32, P, vp]
    lib.ar_twoshot_ll128.restype = i32
    lib.ar_flag_barrier_reset.argtypes, lib.ar_flag_barrier_reset.restype = [vp, i32, vp], i32
    lib.ar_twoshot_noalloc.argtypes, lib.ar_twoshot_noalloc.restype = [P, i32, P, sz, i32, vp], i32
    lib.ar_select_algo.argtypes, lib.ar_select_algo.restype = [i32, sz, i32, ctypes.c_double], i32
    lib.ar_algo_cost_us.argtypes, lib.ar_algo_cost_us.restype = [i32, i32, sz, i32, ctypes.c_double], ctypes.c_double
    return lib


_lib = None
_lib = _load()
lib = _lib


# ------------------------------------------------------------------ helpers --
def _ptr_array(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16") from None


def _dev_tensor(t: torch.Tensor, what: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor, got {t.device}")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        # every call runs on the current device; another device's memory is not its to touch
        raise ValueError(f"{what} is on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _check(code: int, where: str):
    if code != AR_OK:
        raise ArError(code, where)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need_bytes(ts, nbytes: int, what: str):
    for t in ts:
        if _nbytes(t) < nbytes:
            raise ValueError(f"{what} holds {_nbytes(t)} bytes, the call needs {nbytes}")


def _need_like(ts, dtype, numel: int, what: str):
    for t in ts:
        if t.dtype != dtype or t.numel() != numel:
            raise ValueError(f"{what} must be {numel} elements of {dtype}, got {t.numel()} of {t.dtype}")


# bytes of the status words every flag-waiting call writes (the first line of
# a flag region)
STATUS_BYTES = 128


def _twoshot_sizes(ins, segs, flags, outs, seg_proto=None):
    """Size checks of the two-shot calls: equal inputs, segments of numel/n
    elements (or LL / LL128 wires of them), a whole flag region, outputs of
    numel elements.  A numel the call cannot split is left to the C ABI
    (AR_ERR_DIVISIBLE)."""
    n = len(segs)
    if ins:
        _need_like(ins, ins[0].dtype, ins[0].numel(), "every input")
    _need_bytes([flags], flag_bytes(n), "the flag region")
    ref = ins[0] if ins else segs[0]
    numel = ref.numel() if ins else segs[0].numel() * n
    if numel % n == 0:
        m = numel // n
        if seg_proto is None:
            _need_like(segs, ref.dtype, m, "every segment")
        else:
            _need_bytes(segs, ll_wire_bytes(seg_proto, m * ref.element_size()), "every segment wire")
    if outs is not None:
        _need_like([o for o in outs if o is not None], ref.dtype, numel, "every output")


def flag_bytes(n: int) -> int:
    return int(_lib.ar_flag_bytes(n))


def ll_wire_bytes(proto, nbytes: int) -> int:
    return int(_lib.ar_ll_wire_bytes(_PROTOS[proto], int(nbytes)))


def set_poll_timeout_ns(ns: int):
    _lib.ar_set_poll_timeout_ns(int(ns))


def get_poll_timeout_ns() -> int:
    return int(_lib.ar_get_poll_timeout_ns())


ALGOS = ("oneshot", "twoshot", "ll", "ll128", "push", "bcast", "twoshot_ll", "twoshot_ll128")  # ar_algo 0..7


def _dtype_arg(dtype) -> int:
    if isinstance(dtype, torch.dtype):
        if dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {dtype}: use float32 or bfloat16")
        return _DTYPES[dtype]
    return int(dtype)


def algo_cost_us(algo: str, n: int, numel: int, dtype, sync_us: float = 0.0):
    """Modelled time of one call (ar_algo_cost_us); None where the algorithm
    does not apply (a two-shot the size cannot split)."""
    t = float(_lib.ar_algo_cost_us(ALGOS.index(algo), int(n), int(numel), _dtype_arg(dtype), float(sync_us)))
    return None if t < 0 else t


def select_algo(n: int, numel: int, dtype, sync_us: float = 0.0) -> str:
    """Algorithm of least modelled time for an all-reduce of numel elements of
    dtype (torch dtype or AR_F32/AR_BF16) per rank over n ranks, with sync_us
    per cross-GPU semaphore synchronisation."""
    r = int(_lib.ar_select_algo(int(n), int(numel), _dtype_arg(dtype), float(sync_us)))
    if r < 0:
        raise ArError(-r, "ar_select_algo")
    return ALGOS[r]


def new_flags(n: int, device=None) -> torch.Tensor:
    """Allocate a flag region for n ranks (uint32 words) and reset it on the
    current stream.  Set-up only; not part of the per-step path."""
    words = flag_bytes(n) // 4
    f = torch.empty(words, dtype=torch.int32, device=device or "cuda")
    ar_flag_barrier_reset(f, n)
    return f


def read_status(flags: torch.Tensor):
    """(status word, detail word) of a flag region; synchronises the device."""
    s = flags[:2].cpu().numpy().view("uint32")
    return int(s[0]), int(s[1])


def decode_status(word: int):
    """Split a status word into (code, phase, rank)."""
    return word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFFFF


def raise_on_status(flags: torch.Tensor, where: str = "kernel"):
    word, detail = read_status(flags)
    if word != 0:
        code, phase, rank = decode_status(word)
        err = ArError(code, f"{where} (phase {phase}, rank {rank}, index {detail})")
        err.phase, err.rank, err.detail = phase, rank, detail
        raise err


# ------------------------------------------------------------- entry points --
class Prepared:
    """One entry point with its pointer tables already marshalled.

    ``call(step=None, stream=None)`` enqueues it; only the step id and the
    stream are filled in per call.  Holds references to the tensors so their
    memory outlives the prepared call."""

    __slots__ = ("fn", "args", "step_pos", "name", "keep")

    def __init__(self, fn, args, step_pos, name, keep):
        self.fn, self.args, self.step_pos, self.name, self.keep = fn, list(args), step_pos, name, keep

    def __call__(self, step=None, stream=None):
        args = self.args
        if self.step_pos is not None:
            if step is None:
                raise ValueError(f"{self.name} needs a step id")
            args[self.step_pos] = int(step)
        args[-1] = _stream(stream)
        code = self.fn(*args)
        if code != AR_OK:
            raise ArError(code, self.name)


def prepare_oneshot(ins, out: torch.Tensor) -> Prepared:
    ins = [_dev_tensor(t, "input") for t in ins]
    out = _dev_tensor(out, "out")
    dt = _dtype_code(out)
    for t in ins:
        if t.dtype != out.dtype or t.numel() != out.numel():
            raise ValueError("inputs and output must share dtype and numel")
    args = [_ptr_array([t.data_ptr() for t in ins]), len(ins), out.data_ptr(), out.numel(), dt, None]
    return Prepared(_lib.ar_oneshot, args, None, "ar_oneshot", (ins, out))


def rmsnorm_workspace_bytes() -> int:
    return int(_lib.ar_rmsnorm_workspace_bytes())


def new_rmsnorm_workspace(device=None) -> torch.Tensor:
    """A zeroed workspace for ar_oneshot_rmsnorm's few-rows path (one per call
    site; calls sharing it must be ordered on one stream)."""
    return torch.zeros(rmsnorm_workspace_bytes() // 4, dtype=torch.int32, device=device or "cuda")


def prepare_oneshot_rmsnorm(ins, residual: torch.Tensor, weight: torch.Tensor, residual_out: torch.Tensor,
                            out: torch.Tensor, eps: float = 1e-6, workspace=None) -> Prepared:
    """One-shot all-reduce + residual add + RMSNorm over rows of
    ``weight.numel()`` elements: every input, the residual, residual_out and
    out hold rows * hidden elements (residual_out may be residual itself).
    ``workspace`` (from :func:`new_rmsnorm_workspace`, or None) lets few rows
    spread over the whole device."""
    ins = [_dev_tensor(t, "input") for t in ins]
    residual = _dev_tensor(residual, "residual")
    weight = _dev_tensor(weight, "weight")
    residual_out = _dev_tensor(residual_out, "residual_out")
    out = _dev_tensor(out, "out")
    dt = _dtype_code(out)
    hidden = weight.numel()
    if hidden == 0 or out.numel() % hidden != 0:
        raise ValueError(f"out holds {out.numel()} elements, not whole rows of {hidden}")
    _need_like(ins + [residual, residual_out], out.dtype, out.numel(), "every input, residual and residual_out")
    _need_like([weight], out.dtype, hidden, "weight")
    ws = None
    if workspace is not None:
        workspace = _dev_tensor(workspace, "workspace")
        _need_bytes([workspace], rmsnorm_workspace_bytes(), "the workspace")
        ws = workspace.data_ptr()
    args = [_ptr_array([t.data_ptr() for t in ins]), len(ins), residual.data_ptr(), weight.data_ptr(),
            residual_out.data_ptr(), out.data_ptr(), out.numel() // hidden, hidden, float(eps), dt, ws, None]
    return Prepared(_lib.ar_oneshot_rmsnorm, args, None, "ar_oneshot_rmsnorm",
                    (ins, residual, weight, residual_out, out, workspace))


def rmsnorm_segment_bytes(n: int, rows: int, hidden: int, dtype) -> int:
    """Bytes of one rank's segment in ar_twoshot_rmsnorm (its rows of out and of
    residual_out, the parts' slots and flags, then the epoch words of auto
    step ids); 0 if rows is not a multiple of n."""
    return int(_lib.ar_rmsnorm_segment_bytes(int(n), int(rows), int(hidden), _dtype_arg(dtype)))


def new_rmsnorm_segments(n: int, rows: int, hidden: int, dtype, device=None):
    """n zeroed segments for ar_twoshot_rmsnorm (uint8 tensors)."""
    nb = rmsnorm_segment_bytes(n, rows, hidden, dtype)
    if nb == 0:
        raise ValueError(f"{rows} rows do not split over {n} ranks")
    return [torch.zeros(nb, dtype=torch.uint8, device=device or "cuda") for _ in range(n)]


def prepare_twoshot_rmsnorm(ins, residuals, weight: torch.Tensor, segs, flags: torch.Tensor, r0: int = 0,
                            r1=None, residual_outs=None, outs=None, eps: float = 1e-6) -> Prepared:
    """The fused all-reduce + residual add + RMSNorm in two-shot form (see
    ar_twoshot_rmsnorm in include/ar.h).  outs / residual_outs None: the
    reduce-scatter of ranks [r0, r1) alone; else one rank's share (r1 = r0 + 1),
    with n entries each (None outside [r0, r1)).  Called with the step id."""
    n = len(ins)
    r1 = r0 + 1 if r1 is None else r1
    ins = [_dev_tensor(t, "input") for t in ins]
    ref = ins[0]
    weight = _dev_tensor(weight, "weight")
    hidden = weight.numel()
    dt = _dtype_code(ref)
    if hidden == 0 or ref.numel() % hidden != 0:
        raise ValueError(f"inputs hold {ref.numel()} elements, not whole rows of {hidden}")
    rows = ref.numel() // hidden
    _need_like(ins, ref.dtype, ref.numel(), "every input")
    _need_like([weight], ref.dtype, hidden, "weight")
    if len(residuals) != n or len(segs) != n:
        raise ValueError("residuals and segs need one entry per rank")
    if not 0 <= r0 < r1 <= n:
        raise ValueError(f"ranks [{r0}, {r1}) are not a range within [0, {n})")
    mine = range(r0, r1)
    for r in mine:
        _need_like([_dev_tensor(residuals[r], "residual")], ref.dtype, ref.numel(), "every residual in [r0, r1)")
    segs = [_dev_tensor(t, "segment") for t in segs]
    if rows % n == 0:
        _need_bytes(segs, rmsnorm_segment_bytes(n, rows, hidden, ref.dtype), "every segment")
    _need_bytes([_dev_tensor(flags, "flags")], flag_bytes(n), "the flag region")
    ro_arr = o_arr = None
    if (outs is None) != (residual_outs is None):
        raise ValueError("pass both outs and residual_outs, or neither")
    if outs is not None:
        if len(outs) != n or len(residual_outs) != n:
            raise ValueError("outs and residual_outs need n entries (None outside [r0, r1))")
        for r in mine:
            _need_like([_dev_tensor(outs[r], "out"), _dev_tensor(residual_outs[r], "residual_out")], ref.dtype,
                       ref.numel(), "every output in [r0, r1)")
        o_arr = _ptr_array([outs[r].data_ptr() if r in mine else 0 for r in range(n)])
        ro_arr = _ptr_array([residual_outs[r].data_ptr() if r in mine else 0 for r in range(n)])
    res_arr = _ptr_array([residuals[r].data_ptr() if r in mine else 0 for r in range(n)])
    args = [_ptr_array([t.data_ptr() for t in ins]), n, res_arr, weight.data_ptr(),
            _ptr_array([t.data_ptr() for t in segs]), ro_arr, o_arr, rows, hidden, float(eps), dt, r0, r1,
            flags.data_ptr(), 0, None]
    return Prepared(_lib.ar_twoshot_rmsnorm, args, 14, "ar_twoshot_rmsnorm",
                    (ins, residuals, weight, segs, flags, outs, residual_outs))


def ar_twoshot_rmsnorm(ins, residuals, weight, segs, flags, step: int, r0: int = 0, r1=None, residual_outs=None,
                       outs=None, eps: float = 1e-6, stream=None):
    """ar_twoshot_rmsnorm: the reduce-scatter of ranks [r0, r1) (outs None), or
    one rank's share with the all-gather of its peers' rows.  step 0: ids
    kept in the segments (one auto call per rank per step)."""
    prepare_twoshot_rmsnorm(ins, residuals, weight, segs, flags, r0, r1, residual_outs, outs, eps)(step, stream)


def _same_shape(ts, ref, what):
    for t in ts:
        if t.dtype != ref.dtype or t.numel() != ref.numel():
            raise ValueError(f"{what} must share dtype and numel")


def prepare_reduce_bcast(ins, outs, r0: int = 0, r1=None) -> Prepared:
    n = len(ins)
    r1 = n if r1 is None else r1
    ins = [_dev_tensor(t, "input") for t in ins]
    outs = [_dev_tensor(t, "out") for t in outs]
    if len(outs) != n:
        raise ValueError("need one output per rank")
    _same_shape(ins + outs, ins[0], "inputs and outputs")
    args = [_ptr_array([t.data_ptr() for t in ins]), n, _ptr_array([t.data_ptr() for t in outs]), ins[0].numel(),
            _dtype_code(ins[0]), r0, r1, None]
    return Prepared(_lib.ar_reduce_bcast, args, None, "ar_reduce_bcast", (ins, outs))


def prepare_push(srcs, dsts) -> Prepared:
    """dsts[i] lists sender i's destinations (the same count for every sender)."""
    srcs = [_dev_tensor(t, "src") for t in srcs]
    if len(dsts) != len(srcs) or len({len(d) for d in dsts}) != 1:
        raise ValueError("dsts must hold one equally long list per sender")
    flat = [_dev_tensor(t, "dst") for row in dsts for t in row]
    _same_shape(srcs + flat, srcs[0], "sources and destinations")
    args = [_ptr_array([t.data_ptr() for t in srcs]), len(srcs), _ptr_array([t.data_ptr() for t in flat]),
            len(dsts[0]), srcs[0].numel(), _dtype_code(srcs[0]), None]
    return Prepared(_lib.ar_push, args, None, "ar_push", (srcs, flat))


def prepare_twoshot_rs(ins, segs, flags, r0: int = 0, r1=None, outs=None) -> Prepared:
    n = len(ins)
    r1 = n if r1 is None else r1
    ins = [_dev_tensor(t, "input") for t in ins]
    segs = [_dev_tensor(t, "segment") for t in segs]
    flags = _dev_tensor(flags, "flags")
    if len(segs) != n:
        raise ValueError("need one segment buffer per rank")
    out_arr = None
    if outs is not None:
        if len(outs) != n:
            raise ValueError("outs must hold n entries (None outside [r0, r1))")
        out_arr = _ptr_array([(_dev_tensor(o, "out").data_ptr() if o is not None else 0) for o in outs])
    _twoshot_sizes(ins, segs, flags, outs)
    args = [_ptr_array([t.data_ptr() for t in ins]), n, _ptr_array([t.data_ptr() for t in segs]), ins[0].numel(),
            _dtype_code(ins[0]), r0, r1, flags.data_ptr(), 0, out_arr, None]
    return Prepared(_lib.ar_twoshot_rs, args, 8, "ar_twoshot_rs", (ins, segs, flags, outs))


def _prepare_twoshot_wire(fn, name, proto, ins, segws, flags, r0, r1, outs) -> Prepared:
    n = len(ins)
    r1 = n if r1 is None else r1
    ins = [_dev_tensor(t, "input") for t in ins]
    segws = [_dev_tensor(t, "segment wire") for t in segws]
    flags = _dev_tensor(flags, "flags")
    if len(segws) != n:
        raise ValueError("need one segment wire per rank")
    out_arr = None
    if outs is not None:
        if len(outs) != n:
            raise ValueError("outs must hold n entries (None outside [r0, r1))")
        out_arr = _ptr_array([(_dev_tensor(o, "out").data_ptr() if o is not None else 0) for o in outs])
    _twoshot_sizes(ins, segws, flags, outs, seg_proto=proto)
    args = [_ptr_array([t.data_ptr() for t in ins]), n, _ptr_array([t.data_ptr() for t in segws]), ins[0].numel(),
            _dtype_code(ins[0]), r0, r1, flags.data_ptr(), 0, out_arr, None]
    return Prepared(fn, args, 8, name, (ins, segws, flags, outs))


def prepare_twoshot_ll(ins, segws, flags, r0: int = 0, r1=None, outs=None) -> Prepared:
    """Two-shot with LL segment wires (uint8 tensors of ll_wire_bytes("ll", m * element size))."""
    return _prepare_twoshot_wire(_lib.ar_twoshot_ll, "ar_twoshot_ll", "ll", ins, segws, flags, r0, r1, outs)


def prepare_twoshot_ll128(ins, segws, flags, r0: int = 0, r1=None, outs=None) -> Prepared:
    """Two-shot with LL128 segment wires (uint8 tensors of ll_wire_bytes("ll128", m * element size))."""
    return _prepare_twoshot_wire(_lib.ar_twoshot_ll128, "ar_twoshot_ll128", "ll128", ins, segws, flags, r0, r1,
                                 outs)


def prepare_twoshot_ag(segs, outs, flags, r0: int = 0, r1=None, numel=None) -> Prepared:
    n = len(segs)
    r1 = n if r1 is None else r1
    segs = [_dev_tensor(t, "segment") for t in segs]
    flags = _dev_tensor(flags, "flags")
    numel = segs[0].numel() * n if numel is None else numel
    out_arr = _ptr_array([(_dev_tensor(o, "out").data_ptr() if o is not None else 0) for o in outs])
    if len(outs) != n:
        raise ValueError("outs must hold n entries (None outside [r0, r1))")
    _need_like(segs, segs[0].dtype, segs[0].numel(), "every segment")
    _need_bytes([flags], flag_bytes(n), "the flag region")
    if numel % n == 0:
        _need_like(segs, segs[0].dtype, numel // n, "every segment")
    _need_like([o for o in outs if o is not None], segs[0].dtype, numel, "every output")
    args = [_ptr_array([t.data_ptr() for t in segs]), n, out_arr, numel, _dtype_code(segs[0]), r0, r1,
            flags.data_ptr(), 0, None]
    return Prepared(_lib.ar_twoshot_ag, args, 8, "ar_twoshot_ag", (segs, outs, flags))


def prepare_twoshot_ag_copy(segs, outs, flags, r0: int = 0, r1=None, numel=None) -> Prepared:
    n = len(segs)
    r1 = n if r1 is None else r1
    segs = [_dev_tensor(t, "segment") for t in segs]
    flags = _dev_tensor(flags, "flags")
    numel = segs[0].numel() * n if numel is None else numel
    out_arr = _ptr_array([(_dev_tensor(o, "out").data_ptr() if o is not None else 0) for o in outs])
    if len(outs) != n:
        raise ValueError("outs must hold n entries (None outside [r0, r1))")
    _need_like(segs, segs[0].dtype, segs[0].numel(), "every segment")
    _need_bytes([flags], flag_bytes(n), "the flag region")
    if numel % n == 0:
        _need_like(segs, segs[0].dtype, numel // n, "every segment")
    _need_like([o for o in outs if o is not None], segs[0].dtype, numel, "every output")
    args = [_ptr_array([t.data_ptr() for t in segs]), n, out_arr, numel, _dtype_code(segs[0]), r0, r1,
            flags.data_ptr(), 0, None]
    return Prepared(_lib.ar_twoshot_ag_copy, args, 8, "ar_twoshot_ag_copy", (segs, outs, flags))


def prepare_ll_pack(srcs, wires, proto) -> Prepared:
    srcs = [_dev_tensor(t, "src") for t in srcs]
    wires = [_dev_tensor(t, "wire") for t in wires]
    if len(wires) != len(srcs):
        raise ValueError("need one wire per message")
    _need_like(srcs, srcs[0].dtype, srcs[0].numel(), "every message")
    _need_bytes(wires, ll_wire_bytes(proto, _nbytes(srcs[0])), "every wire")
    args = [_ptr_array([t.data_ptr() for t in srcs]), _ptr_array([t.data_ptr() for t in wires]), len(srcs),
            srcs[0].numel(), _dtype_code(srcs[0]), _PROTOS[proto], 0, None]
    return Prepared(_lib.ar_ll_pack, args, 6, "ar_ll_pack", (srcs, wires))


def prepare_ll_reduce(wires, out, flags, proto) -> Prepared:
    wires = [_dev_tensor(t, "wire") for t in wires]
    out = _dev_tensor(out, "out")
    flags = _dev_tensor(flags, "flags")
    fn, name = ((_lib.ar_ll_reduce_unpack, "ar_ll_reduce_unpack") if _PROTOS[proto] == AR_PROTO_LL
                else (_lib.ar_ll128_reduce_unpack, "ar_ll128_reduce_unpack"))
    _need_bytes(wires, ll_wire_bytes(proto, _nbytes(out)), "every wire")
    _need_bytes([flags], STATUS_BYTES, "the flag region")
    args = [_ptr_array([t.data_ptr() for t in wires]), len(wires), out.data_ptr(), out.numel(), _dtype_code(out), 0,
            flags.data_ptr(), None]
    return Prepared(fn, args, 5, name, (wires, out, flags))


def prepare_ll_allreduce(src, wires, out, flags, proto, me: int) -> Prepared:
    """One GPU's LL / LL128 step in one launch: pack rank ``me``'s message
    ``src`` into ``wires[me]`` and reduce every rank's message into ``out``."""
    src = _dev_tensor(src, "src")
    wires = [_dev_tensor(t, "wire") for t in wires]
    out = _dev_tensor(out, "out")
    flags = _dev_tensor(flags, "flags")
    if src.dtype != out.dtype or src.numel() != out.numel():
        raise ValueError("src and out must share dtype and numel")
    _need_bytes(wires, ll_wire_bytes(proto, _nbytes(src)), "every wire")
    _need_bytes([flags], STATUS_BYTES, "the flag region")
    args = [src.data_ptr(), _ptr_array([t.data_ptr() for t in wires]), len(wires), int(me), out.data_ptr(),
            out.numel(), _dtype_code(out), _PROTOS[proto], 0, flags.data_ptr(), None]
    return Prepared(_lib.ar_ll_allreduce, args, 8, "ar_ll_allreduce", (src, wires, out, flags))


def ar_oneshot(ins, out: torch.Tensor, stream=None):
    """out = sum of ins (fp32 accumulation in rank order, one rounding)."""
    prepare_oneshot(ins, out)(stream=stream)
    return out


def ar_oneshot_rmsnorm(ins, residual, weight, residual_out, out, eps: float = 1e-6, workspace=None, stream=None):
    """h = sum of ins + residual (fp32, rank order); residual_out = h rounded;
    out = h / sqrt(mean of h^2 over its row + eps) * weight, rounded once."""
    prepare_oneshot_rmsnorm(ins, residual, weight, residual_out, out, eps, workspace)(stream=stream)
    return out


def ar_reduce_bcast(ins, outs, r0: int = 0, r1=None, stream=None):
    """Ranks [r0, r1) reduce their 1/n of the vectors into every output."""
    prepare_reduce_bcast(ins, outs, r0, r1)(None, stream)


def ar_push(srcs, dsts, stream=None):
    """Copy srcs[i] into every tensor of dsts[i]."""
    prepare_push(srcs, dsts)(None, stream)


def ar_twoshot_rs(ins, segs, flags, step: int, r0: int = 0, r1=None, outs=None, stream=None):
    """Reduce-scatter for ranks [r0, r1); with ``outs`` also the barrier and
    the all-gather in the same persistent launch."""
    prepare_twoshot_rs(ins, segs, flags, r0, r1, outs)(step, stream)


def ar_twoshot_ag(segs, outs, flags, step: int, r0: int = 0, r1=None, numel=None, stream=None):
    """All-gather for ranks [r0, r1) after waiting on every segment's slots."""
    prepare_twoshot_ag(segs, outs, flags, r0, r1, numel)(step, stream)


def ar_twoshot_ag_copy(segs, outs, flags, step: int, r0: int = 0, r1=None, numel=None, stream=None):
    """All-gather on the copy engines after a one-workgroup slot wait."""
    prepare_twoshot_ag_copy(segs, outs, flags, r0, r1, numel)(step, stream)


def ar_ll_pack(srcs, wires, proto, step: int, stream=None):
    """Pack every message of ``srcs`` into its wire buffer (uint8 tensors)."""
    prepare_ll_pack(srcs, wires, proto)(step, stream)


def ar_ll_reduce_unpack(wires, out, step: int, flags, stream=None):
    prepare_ll_reduce(wires, out, flags, "ll")(step, stream)
    return out


def ar_ll128_reduce_unpack(wires, out, step: int, flags, stream=None):
    prepare_ll_reduce(wires, out, flags, "ll128")(step, stream)
    return out


def ar_twoshot_ll(ins, segws, flags, step: int, r0: int = 0, r1=None, outs=None, stream=None):
    """Two-shot under LL: reduce-scatter into LL segment wires for ranks
    [r0, r1); with ``outs`` also the all-gather in the same launch."""
    prepare_twoshot_ll(ins, segws, flags, r0, r1, outs)(step, stream)


def ar_twoshot_ll128(ins, segws, flags, step: int, r0: int = 0, r1=None, outs=None, stream=None):
    """Two-shot under LL128: reduce-scatter into LL128 segment wires for
    ranks [r0, r1); with ``outs`` also the all-gather in the same launch."""
    prepare_twoshot_ll128(ins, segws, flags, r0, r1, outs)(step, stream)


def ar_ll_allreduce(src, wires, out, flags, proto, me: int, step: int, stream=None):
    prepare_ll_allreduce(src, wires, out, flags, proto, me)(step, stream)
    return out


def ar_twoshot_noalloc(ins, outs, stream=None):
    """Every rank's two-shot in one launch, segments and slots in the
    library's own device array (no allocation; at most AR_NOALLOC_MAX_BYTES
    per rank)."""
    ins = [_dev_tensor(t, "input") for t in ins]
    outs = [_dev_tensor(t, "out") for t in outs]
    if len(outs) != len(ins):
        raise ValueError("need one output per rank")
    _need_like(ins + outs, ins[0].dtype, ins[0].numel(), "every input and output")
    _check(_lib.ar_twoshot_noalloc(_ptr_array([t.data_ptr() for t in ins]), len(ins),
                                   _ptr_array([t.data_ptr() for t in outs]), ins[0].numel(), _dtype_code(ins[0]),
                                   _stream(stream)), "ar_twoshot_noalloc")


def ar_flag_barrier_reset(flags, n: int, stream=None):
    flags = _dev_tensor(flags, "flags")
    if flags.numel() * flags.element_size() < flag_bytes(n):
        raise ValueError("flag region too small for n ranks")
    _check(_lib.ar_flag_barrier_reset(flags.data_ptr(), n, _stream(stream)), "ar_flag_barrier_reset")
