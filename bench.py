"""Benchmark of the per-GPU custom all-reduce reduction kernels on one MI355X.

A step is one pass of the whole hot path, one GPU's share of it, over one
message of the workload, with the n ranks' registered buffers emulated as n
HBM allocations on this GPU; this GPU plays rank `me` = 0:

  1. one-shot: the full output of rank me            (ar_oneshot)
  2. two-shot: reduce-scatter of segment me, flag barrier, all-gather into
     rank me's output, in one persistent launch      (ar_twoshot_rs, fused, [me, me+1))
  3. LL: pack rank me's message into its wire buffer and poll/unpack/reduce
     the peers' wire buffers, rank me's term from its message, in one launch
     (ar_ll_allreduce)
  4. LL128: the same with 128-byte lines

The peers' shares (their segments and slots, their packed wire buffers) are
other GPUs' work: they are published once before timing with a step id above
every timed one, as a peer that has already moved on would leave them.  Step
ids of the timed steps increase (no flag reset on the path).  Inputs are
resident in HBM before timing starts; caches are kept cold by rotating
through identical buffer sets totalling more than 1 GiB (MI355X has 256 MiB
of memory-side cache).

Timing: the K steps are captured once into a HIP graph and replayed once
between two events (a decode engine runs this path under graph replay).
Per-kernel durations: K launches of one kernel, graph-replayed, total / K.

Output: one JSON line with the whole-step throughput (algorithmic HBM bytes
per second, see custom_all_reduce_amd/accounting.py), the roofline of the
dominant kernel, and the CPU oracle's throughput on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "reduce-kernel GB/s and % of HBM peak vs message size/rank, n=8, 1×MI355X"
HBM_PEAK = 8000.0  # GB/s, MI355X HBM3E published peak

WORKLOADS = {
    # name: (n ranks, dtype, elements per rank, description)
    "decode": (8, "bf16", 8 * 8192, "one-shot-sized decode message: n=8 ranks, bf16 [8 x 8192] = 128 KiB per rank"),
    "prefill": (8, "bf16", 512 * 8192, "prefill message: n=8 ranks, bf16 [512 x 8192] = 8 MiB per rank"),
    "ll64k": (8, "f32", 16384, "LL-sized message: n=8 ranks, fp32 64 KiB per rank"),
    "ll1m": (8, "f32", 262144, "n=8 ranks, fp32 1 MiB per rank"),
}
KERNELS = ["oneshot", "twoshot", "ll", "ll128"]
KERNEL_SOURCES = {
    "oneshot": ["oneshot.hip"],
    "twoshot": ["twoshot.hip", "fastdiv.hpp"],
    "ll": ["ll.hip"],
    "ll128": ["ll.hip"],
}


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


def step_bytes(n, S):
    from custom_all_reduce_amd import accounting as acc

    per = {
        "oneshot": acc.total(acc.oneshot(n, S)),
        "twoshot": acc.total(acc.twoshot(n, S, 1)),
        "ll": acc.total(acc.ll_allreduce("ll", n, S)),
        "ll128": acc.total(acc.ll_allreduce("ll128", n, S)),
    }
    return per


class BufferSet:
    """All device buffers of one step for n ranks."""

    def __init__(self, torch, car, src, n, dt, numel):
        self.ins = [t.clone() for t in src]
        self.out = torch.empty(numel, dtype=dt, device="cuda")
        self.segs = [torch.empty(numel // n, dtype=dt, device="cuda") for _ in range(n)]
        # LL segment wires of the two-shot under LL, zeroed (flags below every step)
        es_ = 4 if dt == torch.float32 else 2
        self.segw = [torch.zeros(car.ll_wire_bytes("ll", numel // n * es_), dtype=torch.uint8, device="cuda")
                     for _ in range(n)]
        self.outs = [torch.empty(numel, dtype=dt, device="cuda") for _ in range(n)]
        es = 4 if dt == torch.float32 else 2
        S = numel * es
        self.w_ll = [torch.empty(car.ll_wire_bytes("ll", S), dtype=torch.uint8, device="cuda") for _ in range(n)]
        self.w_128 = [torch.empty(car.ll_wire_bytes("ll128", S), dtype=torch.uint8, device="cuda") for _ in range(n)]
        self.out_ll = torch.empty(numel, dtype=dt, device="cuda")
        self.out_128 = torch.empty(numel, dtype=dt, device="cuda")

    def footprint(self):
        ts = self.ins + [self.out] + self.segs + self.segw + self.outs + self.w_ll + self.w_128 + \
            [self.out_ll, self.out_128]
        return sum(t.numel() * t.element_size() for t in ts)


ME = 0
PEER_STEP = 1 << 31  # step id of the peers' published shares, above every timed step


def step_calls(car, b, flags):
    """The four launches of one step on buffer set b (rank ME's share)."""
    n = len(b.ins)
    outs = [b.outs[r] if r == ME else None for r in range(n)]
    return [
        car.prepare_oneshot(b.ins, b.out),
        car.prepare_twoshot_rs(b.ins, b.segs, flags, r0=ME, r1=ME + 1, outs=outs),
        car.prepare_ll_allreduce(b.ins[ME], b.w_ll, b.out_ll, flags, "ll", ME),
        car.prepare_ll_allreduce(b.ins[ME], b.w_128, b.out_128, flags, "ll128", ME),
    ]


def split_ll_calls(car, b, flags):
    """The LL / LL128 step as two launches each (pack, then receive), for
    the sweep."""
    return {
        "ll_pack": car.prepare_ll_pack([b.ins[ME]], [b.w_ll[ME]], "ll"),
        "ll_reduce": car.prepare_ll_reduce(b.w_ll, b.out_ll, flags, "ll"),
        "ll128_pack": car.prepare_ll_pack([b.ins[ME]], [b.w_128[ME]], "ll128"),
        "ll128_reduce": car.prepare_ll_reduce(b.w_128, b.out_128, flags, "ll128"),
    }


def publish_peers(car, b, flags):
    """Untimed: the peers' shares as their own GPUs would have left them."""
    n = len(b.ins)
    peers = [r for r in range(n) if r != ME]
    for r in peers:
        car.ar_twoshot_rs(b.ins, b.segs, flags, PEER_STEP, r0=r, r1=r + 1)
        car.ar_twoshot_ll(b.ins, b.segw, flags, PEER_STEP, r0=r, r1=r + 1)
    car.ar_ll_pack([b.ins[r] for r in peers], [b.w_ll[r] for r in peers], "ll", PEER_STEP)
    car.ar_ll_pack([b.ins[r] for r in peers], [b.w_128[r] for r in peers], "ll128", PEER_STEP)


def run_step(calls, step):
    calls[0]()
    for c in calls[1:]:
        c(step)


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


def launch_floor_us(torch, K):
    """Average time of one graph-replayed launch that does almost nothing (a
    one-element fill), timed like the kernels: the floor under every launch."""
    t = torch.zeros(1, device="cuda")
    g = graph_of(torch, lambda: [t.fill_(float(i)) for i in range(K)])
    timed_replay(torch, g)
    return round(timed_replay(torch, g) * 1e3 / K, 3)


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)\s+src_sha:\s*([0-9a-f]+)", text)
    if not m or m.group(2) != kernel_src_sha(kernel):
        return None
    return int(m.group(1))


def cpu_baseline(host, dt_name, n, numel, per_kernel_bytes, budget_s):
    """The C oracle doing the same step (rank 0's share) on the host, single
    thread, for about budget_s seconds of work.  The peers' wire buffers are
    packed once outside the timed loop, as on the GPU."""
    import oracle

    lib = oracle.load()
    peer_wires = {p: [oracle.ll_pack(p, a, 1 << 31, lib) for a in host] for p in ("ll", "ll128")}
    steps = 0
    t0 = time.perf_counter()
    while True:
        s = steps + 1
        oracle.oneshot(host, dt_name, lib)
        oracle.twoshot(host, dt_name, lib)  # the oracle's two-shot computes every rank's RS and AG
        for proto in ("ll", "ll128"):
            wires = list(peer_wires[proto])
            wires[0] = oracle.ll_pack(proto, host[0], s, lib)
            oracle.ll_reduce(proto, wires, numel, dt_name, s, lib)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    total = sum(per_kernel_bytes.values()) * steps
    return {
        "value": round(total / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{steps} steps of the same workload and data (one-shot; two-shot, where the oracle computes all "
                  f"{n} ranks' RS+AG; pack of rank 0 + reduce of {n} wires for LL and LL128), {el:.1f} s, "
                  "single-threaded C oracle; bytes credited as for rank 0's share",
    }


SWEEP_SIZES = [16 << 10, 256 << 10, 1 << 20, 8 << 20, 64 << 20]


def sweep(args, torch, car, np, out_path):
    """Per-kernel GB/s and fraction of HBM peak vs bytes per rank, for n = 8
    and n = 16, fp32 and bf16 (cold caches, graph-replayed launches).  Writes
    one JSON object per (n, dtype, size, kernel) to out_path and returns the
    one-shot / two-shot crossover per (n, dtype)."""
    import synth
    from custom_all_reduce_amd import accounting as acc

    rows = []
    cross = {}
    for n in (8, 16):
        for dt_name in ("bf16", "f32"):
            dt = torch.float32 if dt_name == "f32" else torch.bfloat16
            es = 4 if dt_name == "f32" else 2
            t_one, t_two = {}, {}
            for S in SWEEP_SIZES:
                numel = S // es
                host = synth.rank_inputs(n, numel, dt_name, "normal", config=4)
                if dt_name == "f32":
                    src = [torch.from_numpy(a).cuda() for a in host]
                else:
                    src = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in host]
                fp = (n * 2 + 5) * S + n * (acc.wire_bytes("ll", S) + acc.wire_bytes("ll128", S))
                nsets = max(2, int(np.ceil((1 << 30) / fp)))
                sets = [BufferSet(torch, car, src, n, dt, numel) for _ in range(nsets)]
                flags = car.new_flags(n)
                calls = [step_calls(car, b, flags) for b in sets]
                full = [car.prepare_twoshot_rs(b.ins, b.segs, flags, outs=b.outs) for b in sets]
                bc_one = [car.prepare_reduce_bcast(b.ins, b.outs, ME, ME + 1) for b in sets]
                bc_all = [car.prepare_reduce_bcast(b.ins, b.outs) for b in sets]
                push = [car.prepare_push([b.ins[ME]], [b.outs]) for b in sets]
                stage = [car.prepare_push([b.ins[ME]], [[b.out]]) for b in sets]
                ag_copy = [car.prepare_twoshot_ag_copy(b.segs, [b.outs[r] if r == ME else None for r in range(n)],
                                                       flags, ME, ME + 1) for b in sets]
                ts_auto = [car.prepare_twoshot_rs(b.ins, b.segs, flags, r0=ME, r1=ME + 1,
                                                  outs=[b.outs[r] if r == ME else None for r in range(n)])
                           for b in sets]
                split = [split_ll_calls(car, b, flags) for b in sets]
                tsll_one = [car.prepare_twoshot_ll(b.ins, b.segw, flags, ME, ME + 1,
                                                   [b.outs[r] if r == ME else None for r in range(n)]) for b in sets]
                tsll_all = [car.prepare_twoshot_ll(b.ins, b.segw, flags, outs=b.outs) for b in sets]
                for b in sets:
                    publish_peers(car, b, flags)
                run_step(calls[0], 1)
                torch.cuda.synchronize()
                car.raise_on_status(flags, "sweep warm-up")
                # K launches per timing: enough for ~20 ms at 5 TB/s, within [16, 400]
                K = int(min(400, max(16, 0.02 * 5e12 / (n * S))))
                step = 3
                # the full emulation rewrites every rank's slots, so it goes last
                kinds = [("oneshot", 0, acc.oneshot(n, S)), ("twoshot", 1, acc.twoshot(n, S, 1)),
                         ("ll", 2, acc.ll_allreduce("ll", n, S)), ("ll128", 3, acc.ll_allreduce("ll128", n, S)),
                         ("ll_pack", "split", acc.ll_pack("ll", S, 1)),
                         ("ll_reduce", "split", acc.ll_reduce("ll", n, S)),
                         ("ll128_pack", "split", acc.ll_pack("ll128", S, 1)),
                         ("ll128_reduce", "split", acc.ll_reduce("ll128", n, S)),
                         ("bcast", "bc_one", acc.reduce_bcast(n, S, 1)),
                         ("bcast_full", "bc_all", acc.reduce_bcast(n, S, n)),
                         ("push", "push", acc.push(S, n)),
                         ("stage", "stage", acc.push(S, 1)),
                         ("ag_copy", "ag_copy", acc.twoshot_ag(n, S, 1)),
                         ("twoshot_auto", "ts_auto", acc.twoshot(n, S, 1)),
                         ("twoshot_ll", "tsll_one", acc.twoshot_ll(n, S, 1)),
                         ("twoshot_ll_full", "tsll_all", acc.twoshot_ll(n, S, n)),
                         ("twoshot_full", None, acc.twoshot(n, S, n))]
                extra = {"bc_one": bc_one, "bc_all": bc_all, "push": push, "stage": stage, "ts_auto": ts_auto,
                         "ag_copy": ag_copy}
                for name, ki, rw in kinds:
                    base = step

                    def launches(ki=ki, base=base, name=name):
                        for i in range(K):
                            if ki is None:
                                full[i % nsets](base + i)
                            elif ki == "ts_auto":
                                extra[ki][i % nsets](0)  # step id from the flag region
                            elif ki == "ag_copy":
                                extra[ki][i % nsets](1)  # every slot holds a later step by now
                            elif ki == "split" and name.endswith("reduce"):
                                split[i % nsets][name](1)  # every wire carries flags >= 1 by now
                            elif ki == "split":
                                split[i % nsets][name](base + i)
                            elif ki == "tsll_all":
                                # above the peers' published step, so no line
                                # left by the publishing counts as arrived
                                tsll_all[i % nsets](PEER_STEP + base + i)
                            elif ki == "tsll_one":
                                tsll_one[i % nsets](base + i)
                            elif isinstance(ki, str):
                                extra[ki][i % nsets]()
                            elif name == "oneshot":
                                calls[i % nsets][0]()
                            else:
                                calls[i % nsets][ki](base + i)

                    g = graph_of(torch, launches)
                    ms = timed_replay(torch, g)
                    del g
                    step = base + K
                    us = ms * 1e3 / K
                    gbps = acc.total(rw) / (us * 1e-6) / 1e9
                    row = {"n": n, "dtype": dt_name, "bytes_per_rank": S, "kernel": name, "avg_us": round(us, 3),
                           "algorithmic_bytes": acc.total(rw), "GBps": round(gbps, 1),
                           "frac_of_peak": round(gbps / HBM_PEAK, 4), "launches": K, "buffer_sets": nsets}
                    rows.append(row)
                    car.raise_on_status(flags, f"sweep {name} n={n} {dt_name} S={S}")
                    print(f"sweep n={n} {dt_name} S={S} {name}: {us:.2f} us {gbps:.0f} GB/s", file=sys.stderr,
                          flush=True)
                    if name == "oneshot":
                        t_one[S] = us
                    elif name == "twoshot":
                        t_two[S] = us
                car.raise_on_status(flags, "sweep")
                del sets, calls, full, src, extra, bc_one, bc_all, push, stage, ts_auto, ag_copy, split
                del tsll_one, tsll_all
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
    with open(out_path, "w", encoding="utf-8") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")
        f.write(json.dumps({"crossover_bytes_per_rank": cross}) + "\n")
    return rows, cross


SELECT_SIZES = [16 << 10, 32 << 10, 64 << 10, 128 << 10, 256 << 10, 512 << 10, 1 << 20, 3 << 19, 2 << 20,
                3 << 20, 4 << 20, 6 << 20, 8 << 20, 12 << 20, 16 << 20, 32 << 20, 64 << 20]
SELECT_ALGOS = ["oneshot", "twoshot", "ll", "ll128", "push", "bcast", "twoshot_ll"]


def select_table(args, torch, car, np, out_path):
    """One GPU's share of an all-reduce by each algorithm, n = 2..16, bf16,
    over SELECT_SIZES bytes per rank (cold: buffer sets rotated over >= 1 GiB;
    graph-replayed).  The shares: one-shot; rank 0's fused two-shot after the
    peers' reduce-scatter; rank 0's LL / LL128 send and receive in one launch
    (ar_ll_allreduce), the peers' wires packed beforehand.  Each time
    is the median of three replays.  Writes one JSON object per (n, size)."""
    rows = []
    gen = torch.Generator(device="cuda")
    with open(out_path, "w", encoding="utf-8") as f:
        for n in range(2, 17):
            for S in SELECT_SIZES:
                numel = S // 2
                numel -= numel % (8 * n)  # whole 16-byte vectors in every segment
                Sb = numel * 2
                W1, W2 = car.ll_wire_bytes("ll", Sb), car.ll_wire_bytes("ll128", Sb)
                fp = n * Sb + 5 * Sb + n * (W1 + W2) + (2 * n - 1) * Sb + n * Sb
                nsets = max(2, int(np.ceil((1 << 30) / fp)))
                gen.manual_seed(1000 * n + S.bit_length())
                src = [torch.randn(numel, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(n)]
                flags = car.new_flags(n)
                calls = {a: [] for a in SELECT_ALGOS}
                keep = []
                for _ in range(nsets):
                    ins = [t.clone() for t in src]
                    segs = [torch.empty(numel // n, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
                    out = torch.empty(numel, dtype=torch.bfloat16, device="cuda")
                    w1 = [torch.empty(W1, dtype=torch.uint8, device="cuda") for _ in range(n)]
                    w2 = [torch.empty(W2, dtype=torch.uint8, device="cuda") for _ in range(n)]
                    # push: rank 0's slot in every rank's staging buffer, and rank 0's
                    # staging buffer (slot 0 is its own push target)
                    slots0 = [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
                    mine = [slots0[0]] + [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(1, n)]
                    bouts = [out] + [torch.empty(numel, dtype=torch.bfloat16, device="cuda") for _ in range(1, n)]
                    segw = [torch.zeros(car.ll_wire_bytes("ll", numel // n * 2), dtype=torch.uint8, device="cuda")
                            for _ in range(n)]
                    keep.append((ins, segs, out, w1, w2, slots0, mine, bouts, segw))
                    for r in range(1, n):
                        car.ar_twoshot_rs(ins, segs, flags, PEER_STEP, r0=r, r1=r + 1)
                        car.ar_twoshot_ll(ins, segw, flags, PEER_STEP, r0=r, r1=r + 1)
                    car.ar_ll_pack(ins[1:], w1[1:], "ll", PEER_STEP)
                    car.ar_ll_pack(ins[1:], w2[1:], "ll128", PEER_STEP)
                    one = car.prepare_oneshot(ins, out)
                    calls["oneshot"].append(lambda s, one=one: one())
                    calls["twoshot"].append(car.prepare_twoshot_rs(ins, segs, flags, 0, 1, [out] + [None] * (n - 1)))
                    for name, w in (("ll", w1), ("ll128", w2)):
                        calls[name].append(car.prepare_ll_allreduce(ins[0], w, out, flags, name, 0))
                    ps, po = car.prepare_push([ins[0]], [slots0]), car.prepare_oneshot(mine, out)
                    calls["push"].append(lambda s, ps=ps, po=po: (ps(), po()))
                    bc = car.prepare_reduce_bcast(ins, bouts, 0, 1)
                    calls["bcast"].append(lambda s, bc=bc: bc())
                    calls["twoshot_ll"].append(car.prepare_twoshot_ll(ins, segw, flags, 0, 1,
                                                                      [out] + [None] * (n - 1)))
                del src
                torch.cuda.synchronize()
                row = {"n": n, "bytes_per_rank": Sb}
                K = int(min(200, max(16, 0.004 * 4e12 / ((n + 1) * Sb))))
                for a in SELECT_ALGOS:
                    cs = calls[a]
                    g = graph_of(torch, lambda cs=cs: [cs[i % nsets](1 + i) for i in range(K)])
                    timed_replay(torch, g)
                    # median of three replays: one disturbed replay does not move the table
                    reps = sorted(timed_replay(torch, g) for _ in range(3))
                    row[a + "_us"] = round(reps[1] * 1e3 / K, 3)
                    del g
                car.raise_on_status(flags, f"select-table n={n} S={Sb}")
                rows.append(row)
                f.write(json.dumps(row) + "\n")
                f.flush()
                print("select-table " + " ".join(f"{k}={v}" for k, v in row.items()), file=sys.stderr, flush=True)
                del calls, keep
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
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate-gib", type=float, default=1.0, help="total size of the rotated buffer sets")
    ap.add_argument("--warm", action="store_true", help="one buffer set (cache-warm); labelled as such")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle budget; 0 skips the CPU baseline")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of one graph replay")
    ap.add_argument("--no-kernel-times", action="store_true", help="skip the per-kernel timing graphs")
    ap.add_argument("--sweep", metavar="OUT.jsonl", help="also run the size sweep (n = 8, 16; fp32, bf16) into a file")
    ap.add_argument("--select-table", metavar="OUT.jsonl",
                    help="only time one GPU's share by each algorithm for n = 2..16 over a size grid, then exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run ten 256 MiB device-to-device copies (reference for HBM byte counters), then exit")
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

    if args.select_table:
        torch.cuda.set_device(0)
        car.set_poll_timeout_ns(50_000_000)
        rows = select_table(args, torch, car, np, args.select_table)
        print(json.dumps({"select_table_rows": len(rows), "file": args.select_table}), flush=True)
        return 0

    n, dt_name, numel, desc = WORKLOADS[args.workload]
    dt = torch.float32 if dt_name == "f32" else torch.bfloat16
    es = 4 if dt_name == "f32" else 2
    S = numel * es
    torch.cuda.set_device(0)
    # No wait on this path should take more than microseconds: a protocol
    # mistake then shows up as a reported timeout after 50 ms, not 1 s.
    car.set_poll_timeout_ns(50_000_000)

    host = synth.rank_inputs(n, numel, dt_name, "normal", config=1)
    if dt_name == "f32":
        src = [torch.from_numpy(a).cuda() for a in host]
    else:
        src = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in host]

    first = BufferSet(torch, car, src, n, dt, numel)
    fp = first.footprint()
    nsets = 1 if args.warm else max(2, int(np.ceil(args.rotate_gib * (1 << 30) / fp)))
    sets = [first] + [BufferSet(torch, car, src, n, dt, numel) for _ in range(nsets - 1)]
    flags = car.new_flags(n)
    calls = [step_calls(car, b, flags) for b in sets]
    for b in sets:
        publish_peers(car, b, flags)
    torch.cuda.synchronize()

    per_bytes = step_bytes(n, S)
    bytes_per_step = sum(per_bytes.values())
    print(f"bench: {args.workload}: {nsets} buffer sets of {fp / 2**20:.1f} MiB ready", file=sys.stderr, flush=True)

    # Untimed warm-up, eager.
    step = 1
    for i in range(args.warmup):
        run_step(calls[i % nsets], step)
        step += 1
    torch.cuda.synchronize()
    car.raise_on_status(flags, "warm-up")

    # Timed region: exactly K steps, captured once into a HIP graph (as a
    # decode engine would run them) with fresh step ids, replayed once
    # between a synchronize and two events.
    K = args.steps
    s0 = step

    def k_steps():
        for i in range(K):
            run_step(calls[(args.warmup + i) % nsets], s0 + i)

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
    step = s0 + K
    car.raise_on_status(flags, "timed steps")
    ms_per_step = ms_total / K

    # Every output of the last set must equal the one-shot output (bitwise).
    last = sets[(args.warmup + K - 1) % nsets]
    ref = last.out.view(torch.int16 if es == 2 else torch.int32)
    for t in [last.outs[ME], last.out_ll, last.out_128]:
        assert torch.equal(t.view(ref.dtype), ref), "outputs of the step disagree"

    # Per-kernel launch durations: K launches of one kernel, rotating sets,
    # captured into a graph and replayed between two events; average = total / K.
    kernels = {}
    if not args.no_kernel_times:
        for ki, name in enumerate(KERNELS):
            base = step

            def k_launches(ki=ki, base=base, name=name):
                for i in range(K):
                    c = calls[i % nsets][ki]
                    if name == "oneshot":
                        c()
                    else:
                        c(base + i)

            g = graph_of(torch, k_launches)
            ms = timed_replay(torch, g)
            del g
            if name != "oneshot":
                step = base + K
            us = ms * 1e3 / K
            kernels[name] = {
                "avg_us": round(us, 3),
                "bytes": per_bytes[name],
                "GBps": round(per_bytes[name] / (us * 1e-6) / 1e9, 1),
            }
        car.raise_on_status(flags, "per-kernel timing")
    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"]) if kernels else None
    floor_us = launch_floor_us(torch, K) if kernels else None
    print(f"bench: timed {K} steps, {ms_per_step * 1e3:.2f} us per step; kernels {kernels}", file=sys.stderr,
          flush=True)

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
            "step": "rank 0's share: oneshot + twoshot(RS seg 0 -> barrier -> AG out 0, fused) + "
                    "LL(pack own, reduce n; one launch) + LL128(same); peers' shares published before timing",
            "algorithmic_bytes_per_step": bytes_per_step,
            "cache": "warm (one buffer set)" if args.warm else
                     f"cold: {nsets} rotated buffer sets, {nsets * fp / 2**30:.2f} GiB",
            "timing": "eager launches" if args.eager else "one HIP-graph replay of the K steps",
            "wall_s": round(wall, 3),
        },
        "kernels": kernels,
        "device": device_summary(torch),
    }
    if dominant:
        A = kernels[dominant]["GBps"]
        tb = read_traffic(dominant, args.workload)
        line["roofline"] = {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": A,
            "peak": HBM_PEAK,
            "unit": "GB/s",
            "frac": round(A / HBM_PEAK, 4),
            "traffic": tb,
            "algorithmic_bytes_per_launch": per_bytes[dominant],
            "avg_us": kernels[dominant]["avg_us"],
            "launch_floor_us": floor_us,
        }
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(host, dt_name, n, numel, per_bytes, args.cpu_seconds)
    if args.sweep:
        del sets, calls
        torch.cuda.empty_cache()
        rows, cross = sweep(args, torch, car, np, args.sweep)
        best = max((r for r in rows if r["bytes_per_rank"] >= (1 << 20) and r["n"] == 8),
                   key=lambda r: r["frac_of_peak"])
        line["sweep"] = {"file": args.sweep, "crossover_bytes_per_rank": cross,
                         "best_n8_at_or_above_1MiB": {k: best[k] for k in ("kernel", "dtype", "bytes_per_rank",
                                                                            "GBps", "frac_of_peak")}}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
