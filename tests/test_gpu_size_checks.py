"""Every prepare_* helper refuses an undersized buffer with ValueError before
anything is enqueued: the C ABI sees only pointers, so an undersized tensor
would otherwise be read or written past its end.  The output tensors (and
the flag region) must be untouched afterwards."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")


def test_undersized_buffers_raise_before_launch():
    n, m = 8, 8 * 64
    numel = n * m
    bf = torch.bfloat16
    ins = [torch.randn(numel, device="cuda").to(bf) for _ in range(n)]
    segs = [torch.zeros(m, dtype=bf, device="cuda") for _ in range(n)]
    short_seg = torch.zeros(m - 8, dtype=bf, device="cuda")
    out = torch.full((numel,), 7.0, dtype=bf, device="cuda")
    outs = [out] + [None] * (n - 1)
    flags = car.new_flags(n)
    torch.cuda.synchronize()
    before = [out.clone(), flags.clone()]
    cases = [
        lambda: car.ar_twoshot_rs(ins, segs[:-1] + [short_seg], flags, 1, 0, 1, outs),
        lambda: car.ar_twoshot_rs(ins, segs, flags[:-1], 1, 0, 1, outs),
        lambda: car.ar_twoshot_rs(ins, segs, flags, 1, 0, 1, [out[:-1]] + outs[1:]),
        lambda: car.ar_twoshot_ag(segs[:-1] + [short_seg], outs, flags, 1, 0, 1),
        lambda: car.ar_twoshot_ag_copy(segs, [out[:-8]] + outs[1:], flags, 1, 0, 1),
    ]
    for proto, fn in (("ll", car.ar_twoshot_ll), ("ll128", car.ar_twoshot_ll128)):
        W = car.ll_wire_bytes(proto, m * 2)
        wires = [torch.zeros(W, dtype=torch.uint8, device="cuda") for _ in range(n)]
        cases.append(lambda fn=fn, wires=wires: fn(ins, wires[:-1] + [wires[-1][:-16]], flags, 1, 0, 1, outs))
        Wm = car.ll_wire_bytes(proto, numel * 2)
        mw = [torch.zeros(Wm, dtype=torch.uint8, device="cuda") for _ in range(n)]
        cases.append(lambda proto=proto, mw=mw: car.ar_ll_pack(ins, mw[:-1] + [mw[-1][:-8]], proto, 1))
        cases.append(lambda proto=proto, mw=mw: car.prepare_ll_reduce(mw[:-1] + [mw[-1][:-8]], out, flags,
                                                                      proto)(1))
        cases.append(lambda proto=proto, mw=mw: car.ar_ll_allreduce(ins[0], mw[:-1] + [mw[-1][:-8]], out, flags,
                                                                    proto, 0, 1))
        cases.append(lambda proto=proto, mw=mw: car.ar_ll_allreduce(ins[0], mw, out, flags[:31], proto, 0, 1))
        cases.append(lambda proto=proto, mw=mw: car.ar_ll_pack([ins[0], ins[1][:-8]], mw[:2], proto, 1))
    # the fused all-reduce + RMSNorm: rows of 64, one-shot and two-shot forms
    hidden = 64
    w = torch.ones(hidden, dtype=bf, device="cuda")
    res = torch.zeros(numel, dtype=bf, device="cuda")
    ws = car.new_rmsnorm_workspace()
    rsegs = car.new_rmsnorm_segments(n, numel // hidden, hidden, bf)
    resid = [res] * n
    cases += [
        lambda: car.ar_oneshot_rmsnorm(ins, res[:-hidden], w, out, out),
        lambda: car.ar_oneshot_rmsnorm(ins, res, w, out[:-hidden], out),
        lambda: car.ar_oneshot_rmsnorm(ins, res, w, out, out[:-8]),
        lambda: car.ar_oneshot_rmsnorm(ins[:-1] + [ins[-1][:-hidden]], res, w, out, out),
        lambda: car.ar_oneshot_rmsnorm(ins, res, w, out, out, workspace=ws[:-1]),
        lambda: car.ar_oneshot_rmsnorm(ins, res, torch.ones(hidden - 8, dtype=bf, device="cuda"), out, out),
        lambda: car.ar_twoshot_rmsnorm(ins, resid, w, rsegs[:-1] + [rsegs[-1][:-16]], flags, 1),
        lambda: car.ar_twoshot_rmsnorm(ins, resid, w, rsegs, flags[:-1], 1),
        lambda: car.ar_twoshot_rmsnorm(ins, [res[:-hidden]] + resid[1:], w, rsegs, flags, 1, 0, 1),
        lambda: car.ar_twoshot_rmsnorm(ins, resid, w, rsegs, flags, 1, 0, 1, residual_outs=outs,
                                       outs=[out[:-hidden]] + outs[1:]),
        lambda: car.ar_twoshot_rmsnorm(ins, resid, w, rsegs, flags, 1, 0, 1, residual_outs=[out[:-hidden]] + outs[1:],
                                       outs=outs),
        lambda: car.ar_twoshot_rmsnorm(ins, resid, w, rsegs, flags, 1, 0, 1, residual_outs=outs),
    ]
    ws_before = ws.clone()
    seg_before = [t.clone() for t in rsegs]
    for k, c in enumerate(cases):
        with pytest.raises(ValueError):
            c()
    torch.cuda.synchronize()
    assert torch.equal(out, before[0]) and torch.equal(flags, before[1])
    assert torch.equal(ws, ws_before) and all(torch.equal(a, b) for a, b in zip(rsegs, seg_before))
