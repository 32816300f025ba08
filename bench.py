"""Benchmark of the per-GPU custom all-reduce reduction kernels on one MI355X.

A step is one pass of the whole hot path, one GPU's share of it, over one
message of the workload, with the n ranks' registered buffers emulated as n
HBM allocations on this GPU; this GPU plays rank `me` = 0:

  1. one-shot: the full output of rank me                (ar_oneshot)
  2. two-shot: reduce-scatter of segment me, flag barrier, all-gather into
     rank me's output, in one launch                     (ar_twoshot_rs, fused, [me, me+1))
  3. the two-shot under LL: the same with the segments as LL wires
                                                         (ar_twoshot_ll, fused, [me, me+1))
  4. the two-shot under LL128: the segments as LL128 wires, each line's data
     ordered before its flag                             (ar_twoshot_ll128, fused, [me, me+1))
  5. LL: pack rank me's message into its wire buffer and poll/unpack/reduce
     the peers' wire buffers, rank me's term from its message, in one launch
                                                         (ar_ll_allreduce)
  6. LL128: the same with 128-byte lines

The peers' shares (their segments and slots, their packed wire buffers) are
other GPUs' work: they are published once before timing with a step id above
every timed one, as a peer that has already moved on would leave them.  Step
ids of the timed steps increase (no flag reset on the path).  Inputs are
resident in HBM before timing starts; caches are kept cold by rotating
through identical buffer sets totalling more than 1 GiB (MI355X has 256 MiB
of memory-side cache).

Timing.
  - The timed region: K steps captured once into a HIP graph and replayed
    once between two events (a decode engine runs this path under graph
    replay); --steps K sets only this.
  - Each kernel alone: a graph of KERNEL_LAUNCHES launches of it over the
    rotated sets, replayed once to warm up and then KERNEL_REPLAYS times;
    its time is the median replay / KERNEL_LAUNCHES.  Independent of --steps.
  - The same per-kernel timing at 128 KiB, 1 MiB, 8 MiB and 64 MiB per rank
    (n = 8, bf16): the metric's curve, in the same JSON line.

Rates use the algorithmic HBM bytes of each operation (oracle/model.py and
custom_all_reduce_amd/accounting.py hold the same counts), against the
published 8 TB/s and against a plain device copy measured in the same run.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "reduce-kernel GB/s and % of HBM peak vs message size/rank, n=8, 1×MI355X"
HBM_PEAK = 8000.0  # GB/s, MI355X HBM3E published peak

WORKLOADS = {
    # name: (n ranks, dtype, elements per rank, the kernel the configuration names, description)
    "prefill": (8, "bf16", 512 * 8192, "twoshot",
                "two-shot prefill message: n=8 ranks, bf16 [512 x 8192] = 8 MiB per rank"),
    "decode": (8, "bf16", 8 * 8192, "oneshot",
               "one-shot decode message: n=8 ranks, bf16 [8 x 8192] = 128 KiB per rank"),
    "ll64k": (8, "f32", 16384, "ll128", "LL / LL128 message: n=8 ranks, fp32 64 KiB per rank"),
    "ll1m": (8, "f32", 262144, "ll128", "LL / LL128 message: n=8 ranks, fp32 1 MiB per rank"),
}
KERNELS = ["oneshot", "twoshot", "twoshot_ll", "twoshot_ll128", "ll", "ll128"]
FUSED_KERNELS = ["oneshot_rmsnorm", "twoshot_rmsnorm"]  # the fused all-reduce + RMSNorm, both forms
KERNEL_SOURCES = {
    "oneshot_rmsnorm": ["rmsnorm.hip"],
    "twoshot_rmsnorm": ["rmsnorm.hip"],
    "oneshot": ["oneshot.hip"],
    "twoshot": ["twoshot.hip", "fastdiv.hpp"],
    "twoshot_ll": ["twoshot.hip", "fastdiv.hpp"],
    "twoshot_ll128": ["twoshot.hip", "fastdiv.hpp"],
    "ll": ["ll.hip"],
    "ll128": ["ll.hip"],
}
KERNEL_LAUNCHES = 200  # launches per per-kernel timing graph
KERNEL_REPLAYS = 5     # timed replays of it (after one warm-up replay); the median counts
CURVE_SIZES = [128 << 10, 1 << 20, 8 << 20, 64 << 20]
ME = 0
PEER_STEP = 1 << 31  # step id of the peers' published shares, above every timed step


def code_text(src: str) -> str:
    """C++ source with comments removed and whitespace collapsed: what the
    compiler sees, so that a comment edit does not count as a kernel change.
    (The kernel sources hold no string literal that contains // or /*.)"""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_src_sha(kernel: str) -> str:
    """Hash of the code (comments excluded) of a kernel's sources, recorded
    beside its HBM counters: the counters count only while it matches."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["ar_device.hpp"]:
        with open(os.path.join(ROOT, "custom_all_reduce_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def kernel_bytes(n, S):
    """Algorithmic (reads, writes) of one launch of each step kernel."""
    from custom_all_reduce_amd import accounting as acc

    return {
        "oneshot": acc.oneshot(n, S),
        "twoshot": acc.twoshot(n, S, 1),
        "twoshot_ll": acc.twoshot_ll(n, S, 1, "ll"),
        "twoshot_ll128": acc.twoshot_ll(n, S, 1, "ll128"),
        "ll": acc.ll_allreduce("ll", n, S),
        "ll128": acc.ll_allreduce("ll128", n, S),
    }


def step_bytes(n, S):
    from custom_all_reduce_amd import accounting as acc

    return {k: acc.total(rw) for k, rw in kernel_bytes(n, S).items()}


class BufferSet:
    """All device buffers of one step for n ranks (rank ME's outputs; every
    rank's with full=True, for the all-rank launches of the sweep)."""

    def __init__(self, torch, car, src, n, dt, numel, full=False):
        es = 4 if dt == torch.float32 else 2
        S, m = numel * es, numel // n
        dev = "cuda"
        self.ins = [t.clone() for t in src]
        self.out = torch.empty(numel, dtype=dt, device=dev)
        self.segs = [torch.empty(m, dtype=dt, device=dev) for _ in range(n)]
        # segment wires of the two-shot under LL / LL128, zeroed (flags below every step)
        self.segw = [torch.zeros(car.ll_wire_bytes("ll", m * es), dtype=torch.uint8, device=dev) for _ in range(n)]
        self.segw128 = [torch.zeros(car.ll_wire_bytes("ll128", m * es), dtype=torch.uint8, device=dev)
                        for _ in range(n)]
        self.outs = [torch.empty(numel, dtype=dt, device=dev) if (full or r == ME) else None for r in range(n)]
        self.out_tsll = torch.empty(numel, dtype=dt, device=dev)
        self.out_ts128 = torch.empty(numel, dtype=dt, device=dev)
        self.w_ll = [torch.empty(car.ll_wire_bytes("ll", S), dtype=torch.uint8, device=dev) for _ in range(n)]
        self.w_128 = [torch.empty(car.ll_wire_bytes("ll128", S), dtype=torch.uint8, device=dev) for _ in range(n)]
        self.out_ll = torch.empty(numel, dtype=dt, device=dev)
        self.out_128 = torch.empty(numel, dtype=dt, device=dev)

    def tensors(self):
        return ([*self.ins, self.out, *self.segs, *self.segw, *self.segw128, self.out_tsll, self.out_ts128,
                 *self.w_ll, *self.w_128, self.out_ll, self.out_128] + [o for o in self.outs if o is not None])

    def footprint(self):
        return sum(t.numel() * t.element_size() for t in self.tensors())

    def step_outputs(self):
        """The output of every step kernel, in KERNELS order."""
        return [self.out, self.outs[ME], self.out_tsll, self.out_ts128, self.out_ll, self.out_128]


def only_me(b, outs):
    return [outs[r] if r == ME else None for r in range(len(b.ins))]


def kernel_calls(car, b, flags):
    """Prepared launches of one buffer set: name -> call(step)."""
    n = len(b.ins)
    one = car.prepare_oneshot(b.ins, b.out)
    ts_outs = only_me(b, b.outs)
    calls = {
        "oneshot": lambda s, one=one: one(),
        "twoshot": car.prepare_twoshot_rs(b.ins, b.segs, flags, ME, ME + 1, ts_outs),
        "twoshot_ll": car.prepare_twoshot_ll(b.ins, b.segw, flags, ME, ME + 1,
                                             only_me(b, [b.out_tsll] * n)),
        "twoshot_ll128": car.prepare_twoshot_ll128(b.ins, b.segw128, flags, ME, ME + 1,
                                                   only_me(b, [b.out_ts128] * n)),
        "ll": car.prepare_ll_allreduce(b.ins[ME], b.w_ll, b.out_ll, flags, "ll", ME),
        "ll128": car.prepare_ll_allreduce(b.ins[ME], b.w_128, b.out_128, flags, "ll128", ME),
    }
    return calls


def publish_peers(car, b, flags):
    """Untimed: the peers' shares as their own GPUs would have left them."""
    n = len(b.ins)
    peers = [r for r in range(n) if r != ME]
    for r in peers:
        car.ar_twoshot_rs(b.ins, b.segs, flags, PEER_STEP, r0=r, r1=r + 1)
        car.ar_twoshot_ll(b.ins, b.segw, flags, PEER_STEP, r0=r, r1=r + 1)
        car.ar_twoshot_ll128(b.ins, b.segw128, flags, PEER_STEP, r0=r, r1=r + 1)
    car.ar_ll_pack([b.ins[r] for r in peers], [b.w_ll[r] for r in peers], "ll", PEER_STEP)
    car.ar_ll_pack([b.ins[r] for r in peers], [b.w_128[r] for r in peers], "ll128", PEER_STEP)


class Rig:
    """Rotated buffer sets of one (n, dtype, numel), the peers published, and
    an increasing step id for every explicit-id launch."""

    def __init__(self, torch, car, np, n, dt_name, numel, rotate_bytes, src=None, warm=False, full=False):
        self.torch, self.car = torch, car
        self.n, self.dt_name, self.numel = n, dt_name, numel
        self.dt = torch.float32 if dt_name == "f32" else torch.bfloat16
        self.es = 4 if dt_name == "f32" else 2
        self.S = numel * self.es
        if src is None:
            gen = torch.Generator(device="cuda")
            gen.manual_seed(1000 * n + self.S.bit_length())
            src = [torch.randn(numel, generator=gen, device="cuda").to(self.dt) for _ in range(n)]
        first = BufferSet(torch, car, src, n, self.dt, numel, full)
        self.fp = first.footprint()
        self.nsets = 1 if warm else max(2, int(np.ceil(rotate_bytes / self.fp)))
        self.sets = [first] + [BufferSet(torch, car, src, n, self.dt, numel, full) for _ in range(self.nsets - 1)]
        self.flags = car.new_flags(n)
        for b in self.sets:
            publish_peers(car, b, self.flags)
        self.calls = [kernel_calls(car, b, self.flags) for b in self.sets]
        self.step = 1
        torch.cuda.synchronize()
        car.raise_on_status(self.flags, "publishing the peers")

    def next_steps(self, k):
        s = self.step
        self.step += k
        return s

    def run_step(self, i, step):
        c = self.calls[i % self.nsets]
        for name in KERNELS:
            c[name](step)

    def time_kernel(self, name, launches=KERNEL_LAUNCHES, replays=KERNEL_REPLAYS):
        """Median per-launch time (us) of `launches` graph-replayed launches
        of one kernel over the rotated sets."""
        torch = self.torch
        s0 = self.next_steps(launches)
        cs = self.calls
        g = graph_of(torch, lambda: [cs[i % self.nsets][name](s0 + i) for i in range(launches)])
        timed_replay(torch, g)  # warm-up replay
        reps = [timed_replay(torch, g) for _ in range(replays)]
        del g
        self.car.raise_on_status(self.flags, f"timing {name}")
        return statistics.median(reps) * 1e3 / launches, [round(r * 1e3 / launches, 3) for r in reps]

    def event_timings(self, name, warm=20, calls=200, batch=20):
        """The two further timings beside the graph-replay median: eager
        launches after `warm` untimed ones, `calls` launches each between two
        events on the launching stream (median per call), then `calls` more in
        batches of `batch` between two events (median batch / batch).  Eager
        per-call figures include the host's launch gaps."""
        torch = self.torch
        cs, ns = self.calls, self.nsets
        s0 = self.next_steps(warm + 2 * calls)
        for i in range(warm):
            cs[i % ns][name](s0 + i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for i, (a, b) in enumerate(ev):
            a.record()
            cs[(warm + i) % ns][name](s0 + warm + i)
            b.record()
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) * 1e3 for a, b in ev]
        nb = calls // batch
        evb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nb)]
        base = warm + calls
        for g, (a, b) in enumerate(evb):
            a.record()
            for j in range(batch):
                i = base + g * batch + j
                cs[i % ns][name](s0 + i)
            b.record()
        torch.cuda.synchronize()
        self.car.raise_on_status(self.flags, f"event timings of {name}")
        bat = [a.elapsed_time(b) * 1e3 / batch for a, b in evb]
        return {"event_per_call_us": round(statistics.median(per), 3), "batched_mean_us": round(statistics.median(bat), 3),
                "calls": calls, "batch": batch, "warmup_calls": warm, "launch": "eager"}

    def check_outputs(self, i):
        """Every step kernel's output of set i equals the one-shot's, bit for bit."""
        torch = self.torch
        b = self.sets[i % self.nsets]
        outs = b.step_outputs()
        iv = torch.int16 if self.es == 2 else torch.int32
        ref = outs[0].view(iv)
        for name, t in zip(KERNELS[1:], outs[1:]):
            assert torch.equal(t.view(iv), ref), f"{name} output differs from the one-shot's"


def graph_of(torch, fn):
    """Capture fn() into a HIP graph (torch.cuda.CUDAGraph on ROCm)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed_replay(torch, g):
    """Replay g once between two events on the current stream; returns ms."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def launch_floor_us(torch, K=KERNEL_LAUNCHES):
    """Per-launch time of a graph-replayed one-element fill, timed like the
    kernels: the floor under every launch."""
    t = torch.zeros(1, device="cuda")
    g = graph_of(torch, lambda: [t.fill_(float(i)) for i in range(K)])
    timed_replay(torch, g)
    return round(statistics.median(timed_replay(torch, g) for _ in range(KERNEL_REPLAYS)) * 1e3 / K, 3)


def copy_gbps(torch, nbytes=1 << 30, copies=10):
    """A plain device-to-device copy of nbytes (torch's copy kernel), graph-
    replayed, median of KERNEL_REPLAYS: read + write bytes per second.  A
    second, measured denominator beside the published peak."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    g = graph_of(torch, lambda: [b.copy_(a) for _ in range(copies)])
    timed_replay(torch, g)
    ms = statistics.median(timed_replay(torch, g) for _ in range(KERNEL_REPLAYS))
    del g, a, b
    torch.cuda.empty_cache()
    return round(2 * nbytes * copies / (ms * 1e-3) / 1e9, 1)


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source: (FETCH_SIZE / WRITE_SIZE scaled
    by a plain copy, the memory-sector count, source); else (None, None, note)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None, None, None
    text = open(path, encoding="utf-8").read()
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)\s+src_sha:\s*([0-9a-f]+)", text)
    rel = os.path.relpath(path, ROOT)
    if not m or m.group(2) != kernel_src_sha(kernel):
        return None, None, rel + " (taken on an older kernel source: not used)"
    sect = re.search(r"\| HBM bytes per launch, sectors \| (\d+) \|", text)
    return int(m.group(1)), (int(sect.group(1)) if sect else None), rel


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return model, os.cpu_count(), usable


def oracle_step_bytes(n, S):
    """HBM bytes the oracle's own step moves: the one-shot, the two-shot of
    every rank (the oracle has no one-rank form), and per protocol the pack
    of rank 0's message plus the reduce of all n wires."""
    from oracle import model

    tot = sum(model.hbm_bytes("oneshot", S, n)) + sum(model.hbm_bytes("twoshot_full", S, n))
    for p in ("ll", "ll128"):
        tot += sum(model.hbm_bytes("ll_pack", S, n, p)) + sum(model.hbm_bytes("ll_reduce", S, n, p))
    return tot


def cpu_baseline(host, dt_name, n, budget_s):
    """The C oracle doing the same message on the host: single-threaded for
    about budget_s / 2 seconds, then with one thread per usable core (element
    ranges of every rank split between the threads; the C calls run without
    Python's lock) for about as long.  Credits the bytes the oracle's step
    actually moves."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    lib = oracle.load()
    numel = host[0].size
    es = 4 if dt_name == "f32" else 2

    def one_step(ins, s):
        oracle.oneshot(ins, dt_name, lib)
        oracle.twoshot(ins, dt_name, lib)
        for proto in ("ll", "ll128"):
            wires = [oracle.ll_pack(proto, a, s, lib) for a in ins[:1]] + peer_wires[id(ins[0])][proto]
            oracle.ll_reduce(proto, wires, ins[0].size, dt_name, s, lib)

    def prep(ins):
        peer_wires[id(ins[0])] = {p: [oracle.ll_pack(p, a, PEER_STEP, lib) for a in ins[1:]] for p in ("ll", "ll128")}

    peer_wires = {}
    prep(host)
    model_name, nproc, usable = host_cpu()
    threads = max(1, min(16, usable))
    # element ranges: whole two-shot segments and whole LL128 lines in every range
    unit = n * 480
    bounds = [min(numel, (numel * t // threads) // unit * unit) for t in range(threads)] + [numel]
    slices = [[a[bounds[t]:bounds[t + 1]].copy() for a in host] for t in range(threads)]
    slices = [s for s in slices if s[0].size > 0]
    for s in slices:
        prep(s)

    def run(fn, budget):
        steps, t0 = 0, time.perf_counter()
        while True:
            fn(steps + 1)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return steps, el

    s1, e1 = run(lambda s: one_step(host, s), budget_s / 2)
    with ThreadPoolExecutor(len(slices)) as ex:
        sT, eT = run(lambda s: list(ex.map(lambda sl: one_step(sl, s), slices)), budget_s / 2)
    per_step = oracle_step_bytes(n, numel * es)
    return {
        "value": round(per_step * sT / eT / 1e9, 4),
        "unit": "GB/s",
        "cores": len(slices),
        "kind": "oracle",
        "sample": f"{sT} steps on the workload's own data with {len(slices)} threads over element ranges, "
                  f"{eT:.1f} s; a step is the oracle's one-shot, its two-shot of all {n} ranks, and per protocol "
                  "the pack of rank 0's message plus the reduce of all n wires (the peers' wires packed once "
                  f"beforehand); credited with the {per_step} HBM bytes that step moves",
        "single_thread": {"value": round(per_step * s1 / e1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "steps": s1, "seconds": round(e1, 1)},
        "host": {"cpu_model": model_name, "nproc": nproc, "usable_cores": usable},
    }


def curve(args, torch, car, np):
    """Per-kernel time and rate at CURVE_SIZES bytes per rank, n = 8, bf16."""
    from custom_all_reduce_amd import accounting as acc

    rows = []
    for S in CURVE_SIZES:
        rig = Rig(torch, car, np, 8, "bf16", S // 2, args.rotate_gib * (1 << 30))
        row = {"bytes_per_rank": S}
        for name in KERNELS:
            us, _ = rig.time_kernel(name, replays=3)
            by = acc.total(kernel_bytes(8, S)[name])
            gbps = by / (us * 1e-6) / 1e9
            row[name] = {"us": round(us, 3), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK, 4)}
        row["ll128_vs_oneshot"] = round(row["ll128"]["GBps"] / row["oneshot"]["GBps"], 3)
        rig.check_outputs(0)
        rows.append(row)
        print("curve " + json.dumps(row), file=sys.stderr, flush=True)
        del rig
        torch.cuda.empty_cache()
    return rows


SWEEP_SIZES = [16 << 10, 256 << 10, 1 << 20, 8 << 20, 64 << 20]


RMS_ROW = 16 << 10  # row bytes of the fused all-reduce + RMSNorm in the sweep and its profile


def add_rmsnorm_calls(torch, car, rig):
    """Add the fused all-reduce + RMSNorm over rows of RMS_ROW bytes to every
    buffer set of a full rig (one with n + 1 outputs per set): the one-shot
    form with a workspace (its few-rows path where that applies), residual,
    residual_out and output in three of the set's other output buffers; where
    the rows split over the ranks, also its two-shot form, rank 0's share, the
    peers' reduce-scatters published once beforehand on a flag region of its
    own, with explicit step ids and (on segments of its own) auto ones.
    Returns (whether the two-shot form was added, the buffers to keep
    alive)."""
    n, es, S = rig.n, rig.es, rig.S
    w = torch.ones(RMS_ROW // es, dtype=rig.dt, device="cuda")
    ws = car.new_rmsnorm_workspace()
    rows = S // RMS_ROW
    two = rows > 0 and rows % n == 0
    fl = car.new_flags(n)
    keep = {}
    for i, b in enumerate(rig.sets):
        c = rig.calls[i]
        rn = car.prepare_oneshot_rmsnorm(b.ins, b.outs[1], w, b.outs[2], b.outs[3], 1e-6, workspace=ws)
        c["oneshot_rmsnorm"] = lambda s, f=rn: f()
        if two:
            segs = car.new_rmsnorm_segments(n, rows, RMS_ROW // es, rig.dt)
            resid = [b.outs[1]] * n
            car.ar_twoshot_rmsnorm(b.ins, resid, w, segs, fl, PEER_STEP, r0=1, r1=n)
            tr = car.prepare_twoshot_rmsnorm(b.ins, resid, w, segs, fl, ME, ME + 1,
                                             only_me(b, b.outs[2:3] * n), only_me(b, b.outs[3:4] * n))
            c["twoshot_rmsnorm"] = lambda s, f=tr: f(s)
            # the same share with auto step ids, on segments of its own (explicit
            # and auto ids do not mix); its peers published at PEER_STEP too
            segs_a = car.new_rmsnorm_segments(n, rows, RMS_ROW // es, rig.dt)
            car.ar_twoshot_rmsnorm(b.ins, resid, w, segs_a, fl, PEER_STEP, r0=1, r1=n)
            ta = car.prepare_twoshot_rmsnorm(b.ins, resid, w, segs_a, fl, ME, ME + 1,
                                             only_me(b, b.outs[2:3] * n), only_me(b, b.outs[3:4] * n))
            c["twoshot_rmsnorm_auto"] = lambda s, f=ta: f(0)
            keep[i] = (segs, segs_a)
    torch.cuda.synchronize()
    car.raise_on_status(fl, "publishing the peers' fused reduce-scatters")
    keep["flags"], keep["weight"], keep["workspace"] = fl, w, ws
    return two, keep


def nvlink_model_crossover(n, alpha=1.5e-6, beta=450e9):
    """Bytes per rank where the pages' alpha-beta model of 8-GPU NVLink ("集合通信：
    NCCL 的算法、协议与推理框架的定制 all-reduce", 算法 and 练习 2; alpha = 1.5 us,
    beta = 450 GB/s) makes the two-shot (4 alpha + 2 (n-1)/n S / beta) as fast as
    the one-shot (2 alpha + (n-1) S / beta): S* = 2 alpha beta / ((n-1)(1 - 2/n))."""
    return 2 * alpha * beta / ((n - 1) * (1 - 2 / n))


def sweep(args, torch, car, np, out_path):
    """Per-kernel GB/s and fraction of HBM peak vs bytes per rank, for n = 8
    and n = 16, fp32 and bf16 (cold caches, graph-replayed launches), for the
    step kernels and the other entry points.  Writes one JSON object per
    (n, dtype, size, kernel) to out_path and returns the one-shot / two-shot
    crossover per (n, dtype)."""
    from custom_all_reduce_amd import accounting as acc

    rows = []
    cross = {}
    cross_hbm = {}
    for n in (8, 16):
        for dt_name in ("bf16", "f32"):
            es = 4 if dt_name == "f32" else 2
            t_one, t_two = {}, {}
            for S in SWEEP_SIZES:
                rig = Rig(torch, car, np, n, dt_name, S // es, args.rotate_gib * (1 << 30), full=True)
                fl = rig.flags
                rms_ts, extra = add_rmsnorm_calls(torch, car, rig)
                for i, b in enumerate(rig.sets):
                    c = rig.calls[i]
                    c["ll_pack"] = car.prepare_ll_pack([b.ins[ME]], [b.w_ll[ME]], "ll")
                    c["ll_reduce"] = car.prepare_ll_reduce(b.w_ll, b.out_ll, fl, "ll")
                    c["ll128_pack"] = car.prepare_ll_pack([b.ins[ME]], [b.w_128[ME]], "ll128")
                    c["ll128_reduce"] = car.prepare_ll_reduce(b.w_128, b.out_128, fl, "ll128")
                    bc1 = car.prepare_reduce_bcast(b.ins, b.outs, ME, ME + 1)
                    bca = car.prepare_reduce_bcast(b.ins, b.outs)
                    push = car.prepare_push([b.ins[ME]], [b.outs])
                    stage = car.prepare_push([b.ins[ME]], [[b.out]])
                    agc = car.prepare_twoshot_ag_copy(b.segs, only_me(b, b.outs), fl, ME, ME + 1)
                    tsa = car.prepare_twoshot_rs(b.ins, b.segs, fl, ME, ME + 1, only_me(b, b.outs))
                    c["bcast"] = lambda s, f=bc1: f()
                    c["bcast_full"] = lambda s, f=bca: f()
                    c["push"] = lambda s, f=push: f()
                    c["stage"] = lambda s, f=stage: f()
                    c["ag_copy"] = lambda s, f=agc: f(1)  # every slot holds a later step by now
                    c["twoshot_auto"] = lambda s, f=tsa: f(0)  # step id from the flag region
                    # the receivers alone: every wire carries flags >= 1 by now
                    for k in ("ll_reduce", "ll128_reduce"):
                        c[k] = (lambda s, f=c[k]: f(1))
                    ful = car.prepare_twoshot_rs(b.ins, b.segs, fl, outs=b.outs)
                    tsll_all = car.prepare_twoshot_ll(b.ins, b.segw, fl, outs=b.outs)
                    ts128_all = car.prepare_twoshot_ll128(b.ins, b.segw128, fl, outs=b.outs)
                    # all-rank launches rewrite every rank's segments: their ids go above
                    # the peers' published step, so nothing the publishing left counts
                    c["twoshot_full"] = lambda s, f=ful: f(PEER_STEP + s)
                    c["twoshot_ll_full"] = lambda s, f=tsll_all: f(PEER_STEP + s)
                    c["twoshot_ll128_full"] = lambda s, f=ts128_all: f(PEER_STEP + s)
                kinds = [(k, kernel_bytes(n, S)[k]) for k in KERNELS] + [
                    ("ll_pack", acc.ll_pack("ll", S, 1)), ("ll_reduce", acc.ll_reduce("ll", n, S)),
                    ("ll128_pack", acc.ll_pack("ll128", S, 1)), ("ll128_reduce", acc.ll_reduce("ll128", n, S)),
                    ("bcast", acc.reduce_bcast(n, S, 1)), ("bcast_full", acc.reduce_bcast(n, S, n)),
                    ("push", acc.push(S, n)), ("stage", acc.push(S, 1)), ("ag_copy", acc.twoshot_ag(n, S, 1)),
                    ("twoshot_auto", acc.twoshot(n, S, 1)),
                    ("oneshot_rmsnorm", acc.oneshot_rmsnorm(n, S, RMS_ROW)),
                    *([("twoshot_rmsnorm", acc.twoshot_rmsnorm(n, S, RMS_ROW)),
                       ("twoshot_rmsnorm_auto", acc.twoshot_rmsnorm(n, S, RMS_ROW))] if rms_ts else []),
                    # the all-rank launches last: they rewrite every rank's segments
                    ("twoshot_full", acc.twoshot(n, S, n)), ("twoshot_ll_full", acc.twoshot_ll(n, S, n, "ll")),
                    ("twoshot_ll128_full", acc.twoshot_ll(n, S, n, "ll128"))]
                K = int(min(KERNEL_LAUNCHES, max(16, 0.02 * 5e12 / (n * S))))
                for name, rw in kinds:
                    us, _ = rig.time_kernel(name, launches=K, replays=3)
                    gbps = acc.total(rw) / (us * 1e-6) / 1e9
                    rows.append({"n": n, "dtype": dt_name, "bytes_per_rank": S, "kernel": name,
                                 "avg_us": round(us, 3), "algorithmic_bytes": acc.total(rw), "GBps": round(gbps, 1),
                                 "frac_of_peak": round(gbps / HBM_PEAK, 4), "launches": K,
                                 "buffer_sets": rig.nsets})
                    print(f"sweep n={n} {dt_name} S={S} {name}: {us:.2f} us {gbps:.0f} GB/s", file=sys.stderr,
                          flush=True)
                    if name == "oneshot":
                        t_one[S] = us
                    elif name == "twoshot":
                        t_two[S] = us
                del rig, extra
                torch.cuda.empty_cache()
            # crossover: first size where two-shot (one rank's share) beats one-shot,
            # log-linear interpolation of the time difference between the bracketing sizes
            xs = None
            for a, b in zip(SWEEP_SIZES, SWEEP_SIZES[1:]):
                da, db = t_two[a] - t_one[a], t_two[b] - t_one[b]
                if da >= 0 > db or (da > 0 and db <= 0):
                    f = da / (da - db)
                    xs = float(np.exp(np.log(a) + f * (np.log(b) - np.log(a))))
                    break
            if xs is None and t_two[SWEEP_SIZES[0]] < t_one[SWEEP_SIZES[0]]:
                xs = float(SWEEP_SIZES[0])
            cross[f"n{n}_{dt_name}"] = None if xs is None else round(xs)
            # the same alpha-beta model on HBM: the two-shot's extra fixed cost at
            # the smallest size over the one-shot's streaming rate at the largest,
            # S* = alpha_gpu * B / (n - 2) (one-shot (n+1) S vs two-shot ~3 S bytes)
            s0, s1 = SWEEP_SIZES[0], SWEEP_SIZES[-1]
            alpha_us = t_two[s0] - t_one[s0]
            b_per_us = (n + 1) * s1 / t_one[s1]
            cross_hbm[f"n{n}_{dt_name}"] = round(max(alpha_us, 0.0) * b_per_us / (n - 2))
    nvlink = {f"n{n}": round(nvlink_model_crossover(n)) for n in (8, 16)}
    with open(out_path, "w", encoding="utf-8") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")
        f.write(json.dumps({"crossover_bytes_per_rank": cross, "hbm_analogue_bytes_per_rank": cross_hbm,
                            "nvlink_model_bytes_per_rank": nvlink}) + "\n")
    return rows, {"measured": cross, "hbm_analogue": cross_hbm, "nvlink_model": nvlink}


SELECT_SIZES = [16 << 10, 32 << 10, 64 << 10, 128 << 10, 256 << 10, 512 << 10, 1 << 20, 3 << 19, 2 << 20,
                3 << 20, 4 << 20, 6 << 20, 8 << 20, 12 << 20, 16 << 20, 32 << 20, 64 << 20]
SELECT_ALGOS = ["oneshot", "twoshot", "ll", "ll128", "push", "bcast", "twoshot_ll", "twoshot_ll128"]


def select_table(args, torch, car, np, out_path):
    """One GPU's share of an all-reduce by each algorithm, n = 2..16, bf16,
    over SELECT_SIZES bytes per rank (cold: buffer sets rotated over >= 1 GiB;
    graph-replayed).  The shares: one-shot; rank 0's fused two-shot (slots,
    LL and LL128 segments) after the peers' reduce-scatter; rank 0's LL /
    LL128 send and receive in one launch (ar_ll_allreduce), the peers' wires
    packed beforehand; rank 0's push plus its one-shot over its staging
    slots; rank 0's reduce-broadcast share.  Each time is the median of
    three replays.  Writes one JSON object per (n, size)."""
    rows = []
    with open(out_path, "w", encoding="utf-8") as f:
        for n in range(2, 17):
            for S in SELECT_SIZES:
                numel = S // 2
                numel -= numel % (8 * n)  # whole 16-byte vectors in every segment
                Sb = numel * 2
                rig = Rig(torch, car, np, n, "bf16", numel, 1 << 30)
                keep = []
                for i, b in enumerate(rig.sets):
                    slots0 = [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
                    mine = [slots0[0]] + [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(1, n)]
                    bouts = [b.out] + [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(1, n)]
                    keep.append((slots0, mine, bouts))
                    ps, po = car.prepare_push([b.ins[0]], [slots0]), car.prepare_oneshot(mine, b.out)
                    bc = car.prepare_reduce_bcast(b.ins, bouts, 0, 1)
                    rig.calls[i]["push"] = lambda s, ps=ps, po=po: (ps(), po())
                    rig.calls[i]["bcast"] = lambda s, bc=bc: bc()
                torch.cuda.synchronize()
                row = {"n": n, "bytes_per_rank": Sb}
                K = int(min(200, max(16, 0.004 * 4e12 / ((n + 1) * Sb))))
                for a in SELECT_ALGOS:
                    us, _ = rig.time_kernel(a, launches=K, replays=3)
                    row[a + "_us"] = round(us, 3)
                rows.append(row)
                f.write(json.dumps(row) + "\n")
                f.flush()
                print("select-table " + " ".join(f"{k}={v}" for k, v in row.items()), file=sys.stderr, flush=True)
                del rig, keep
                torch.cuda.empty_cache()
    return rows


def device_summary(torch):
    """What the run ran on, as the runtime reports it."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "l2_bytes": getattr(p, "L2_cache_size", None), "hbm_bytes": p.total_memory}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="steps in the timed region")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate-gib", type=float, default=1.0, help="total size of the rotated buffer sets")
    ap.add_argument("--warm", action="store_true", help="one buffer set (cache-warm); labelled as such")
    ap.add_argument("--cpu-seconds", type=float, default=16.0, help="oracle budget; 0 skips the CPU baseline")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of one graph replay")
    ap.add_argument("--no-kernel-times", action="store_true", help="skip the per-kernel timing graphs")
    ap.add_argument("--no-curve", action="store_true", help="skip the per-kernel timing at 128 KiB..64 MiB")
    ap.add_argument("--sweep", metavar="OUT.jsonl", help="also run the size sweep (n = 8, 16; fp32, bf16) into a file")
    ap.add_argument("--select-table", metavar="OUT.jsonl",
                    help="only time one GPU's share by each algorithm for n = 2..16 over a size grid, then exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run ten 256 MiB device-to-device copies (reference for HBM byte counters), then exit")
    ap.add_argument("--profile-kernel", choices=KERNELS + FUSED_KERNELS,
                    help="only launch this kernel 20 times on the workload (for counter runs), then exit; "
                         "the fused all-reduce + RMSNorm kernels run over rows of 16 KiB")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the reduction with the ranks emulated on that GPU; "
              f"--gpus {args.gpus} (world size {world}) is not supported: run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.calibrate_copy:
        # A plain copy of known size: FETCH_SIZE and WRITE_SIZE of its kernel
        # should read 256 MiB each; their ratio to that scales the counters.
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 256 << 20, "launches": 10}), flush=True)
        return 0

    import custom_all_reduce_amd as car
    import synth

    torch.cuda.set_device(0)
    # No wait on this path should take more than microseconds: a protocol
    # mistake then shows up as a reported timeout after 50 ms, not 1 s.
    car.set_poll_timeout_ns(50_000_000)

    if args.select_table:
        rows = select_table(args, torch, car, np, args.select_table)
        print(json.dumps({"select_table_rows": len(rows), "file": args.select_table}), flush=True)
        return 0

    n, dt_name, numel, config_kernel, desc = WORKLOADS[args.workload]
    es = 4 if dt_name == "f32" else 2
    S = numel * es
    host = synth.rank_inputs(n, numel, dt_name, "normal", config=1)
    if dt_name == "f32":
        src = [torch.from_numpy(a).cuda() for a in host]
    else:
        src = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in host]

    if args.profile_kernel:
        fused = args.profile_kernel in FUSED_KERNELS
        rig = Rig(torch, car, np, n, dt_name, numel, args.rotate_gib * (1 << 30), src=src, full=fused)
        if fused:
            two, keep = add_rmsnorm_calls(torch, car, rig)
            if args.profile_kernel == "twoshot_rmsnorm" and not two:
                print(f"the rows of {RMS_ROW} bytes of workload {args.workload} do not split over {n} ranks",
                      file=sys.stderr)
                return 2
        s0 = rig.next_steps(20)
        for i in range(20):
            rig.calls[i % rig.nsets][args.profile_kernel](s0 + i)
        torch.cuda.synchronize()
        car.raise_on_status(rig.flags, "profile")
        if fused:
            car.raise_on_status(keep["flags"], "profile")
        print(json.dumps({"profiled_kernel": args.profile_kernel, "launches": 20, "workload": args.workload}),
              flush=True)
        return 0

    rig = Rig(torch, car, np, n, dt_name, numel, args.rotate_gib * (1 << 30), src=src, warm=args.warm)
    nsets, fp = rig.nsets, rig.fp
    per_rw = kernel_bytes(n, S)
    per_bytes = step_bytes(n, S)
    bytes_per_step = sum(per_bytes.values())
    print(f"bench: {args.workload}: {nsets} buffer sets of {fp / 2**20:.1f} MiB ready", file=sys.stderr, flush=True)

    # Untimed warm-up, eager.
    s0 = rig.next_steps(args.warmup)
    for i in range(args.warmup):
        rig.run_step(i, s0 + i)
    torch.cuda.synchronize()
    car.raise_on_status(rig.flags, "warm-up")

    # Timed region: exactly K steps, captured once into a HIP graph (as a
    # decode engine would run them) with fresh step ids, replayed once
    # between a synchronize and two events.
    K = args.steps
    s0 = rig.next_steps(K)

    def k_steps():
        for i in range(K):
            rig.run_step(args.warmup + i, s0 + i)

    if args.eager:
        torch.cuda.synchronize()
        t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        t_a.record()
        k_steps()
        t_b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_total = t_a.elapsed_time(t_b)
    else:
        g = graph_of(torch, k_steps)
        wall0 = time.perf_counter()
        ms_total = timed_replay(torch, g)
        wall = time.perf_counter() - wall0
        del g
    car.raise_on_status(rig.flags, "timed steps")
    ms_per_step = ms_total / K
    # Every output of the last set the timed steps wrote equals the one-shot's (bitwise).
    rig.check_outputs(args.warmup + K - 1)
    print(f"bench: timed {K} steps, {ms_per_step * 1e3:.2f} us per step", file=sys.stderr, flush=True)

    kernels = {}
    copy_rate = None
    floor_us = None
    other_timings = None
    if not args.no_kernel_times:
        for name in KERNELS:
            us, reps = rig.time_kernel(name)
            gb = per_bytes[name] / (us * 1e-6) / 1e9
            kernels[name] = {"us": round(us, 3), "replays_us": reps, "algorithmic_bytes": per_bytes[name],
                             "GBps": round(gb, 1), "frac": round(gb / HBM_PEAK, 4)}
        floor_us = launch_floor_us(torch)
        other_timings = rig.event_timings(config_kernel)
        print(f"bench: kernels {json.dumps(kernels)}", file=sys.stderr, flush=True)
    del rig
    torch.cuda.empty_cache()
    if not args.no_kernel_times:
        copy_rate = copy_gbps(torch)
        for k in kernels.values():
            k["frac_of_copy"] = round(k["GBps"] / copy_rate, 4)

    value = bytes_per_step * K / (ms_total * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic",
        "config": {
            "workload": desc,
            "n_ranks": n,
            "bytes_per_rank": S,
            "arithmetic": f"{dt_name} data, fp32 accumulation in rank order, one rounding to {dt_name}",
            "step": "rank 0's share, six launches: one-shot; two-shot (RS of segment 0 -> barrier -> AG into "
                    "output 0, one launch) with slots, with LL segments and with LL128 segments; LL and LL128 "
                    "(pack own, reduce n; one launch each); the peers' shares published before timing",
            "algorithmic_bytes_per_step": bytes_per_step,
            "cache": "warm (one buffer set)" if args.warm else
                     f"cold: {nsets} rotated buffer sets, {nsets * fp / 2**30:.2f} GiB",
            "timing": ("eager launches" if args.eager else "one HIP-graph replay of the K steps") +
                      f"; kernels: {KERNEL_LAUNCHES} graph-replayed launches, median of {KERNEL_REPLAYS} replays",
            "wall_s": round(wall, 3),
        },
        "kernels": kernels,
        "copy_GBps": copy_rate,
        "launch_floor_us": floor_us,
        "device": device_summary(torch),
    }
    if kernels:
        # the roofline of the kernel the configuration names (the two-shot for the
        # prefill message), with the algorithmic bytes of one launch
        rk = config_kernel
        trace_summary = f"profiles/{args.workload}_step_kernel_trace.md"
        A = kernels[rk]["GBps"]
        tb, tsect, tsrc = read_traffic(rk, args.workload)
        longest = max(kernels, key=lambda k: kernels[k]["us"])
        line["roofline"] = {
            "kernel": rk,
            "bound": "hbm",
            "achieved": A,
            "peak": HBM_PEAK,
            "unit": "GB/s",
            "frac": round(A / HBM_PEAK, 4),
            "traffic": tb,
            "traffic_sectors": tsect,
            "traffic_source": tsrc,
            "algorithmic_bytes_per_launch": per_bytes[rk],
            "reads_writes": list(per_rw[rk]),
            "us": kernels[rk]["us"],
            "frac_of_copy": kernels[rk].get("frac_of_copy"),
            "longest_kernel": {"kernel": longest, "us": kernels[longest]["us"], "frac": kernels[longest]["frac"]},
            # the same kernel timed the other ways: kernel-only durations in the
            # committed rocprofv3 trace summary; eager launches between events here
            "other_timings": dict(other_timings or {}, kernel_trace=trace_summary if os.path.exists(
                os.path.join(ROOT, trace_summary)) else None),
        }
    if not args.no_curve and not args.no_kernel_times:
        line["curve_n8_bf16"] = curve(args, torch, car, np)
        for row in line["curve_n8_bf16"]:
            for k in KERNELS:
                row[k]["frac_of_copy"] = round(row[k]["GBps"] / copy_rate, 4)
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(host, dt_name, n, args.cpu_seconds)
    if args.sweep:
        torch.cuda.empty_cache()
        rows, cross = sweep(args, torch, car, np, args.sweep)
        line["sweep"] = {"file": args.sweep, "crossover_bytes_per_rank": cross}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
