"""Independent all-reduces on two streams at once, issued from two host
threads: each has its own buffers and flag region, and both must come out
exactly as the oracle says on every step (auto step ids, so the flag regions'
epochs advance independently).  Streams keep the default priority."""
from __future__ import annotations

import threading

import numpy as np
import pytest
import torch

import oracle
import synth
from devtensors import bits, oracle_bits, to_dev

pytestmark = pytest.mark.gpu

car = pytest.importorskip("custom_all_reduce_amd")

STEPS = 12


class Job:
    def __init__(self, n, numel, config):
        self.n = n
        host = synth.rank_inputs(n, numel, "bf16", "normal", config=config)
        self.want = oracle_bits(oracle.oneshot(host, "bf16"))
        self.ins = [to_dev(a) for a in host]
        tdt = self.ins[0].dtype
        self.segs = [torch.empty(numel // n, dtype=tdt, device="cuda") for _ in range(n)]
        self.outs = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
        self.one = torch.empty(numel, dtype=tdt, device="cuda")
        self.bc = [torch.empty(numel, dtype=tdt, device="cuda") for _ in range(n)]
        self.flags = car.new_flags(n)
        self.stream = torch.cuda.Stream()  # default priority
        self.error = None

    def run(self):
        try:
            with torch.cuda.stream(self.stream):
                for _ in range(STEPS):
                    car.ar_oneshot(self.ins, self.one)
                    car.ar_twoshot_rs(self.ins, self.segs, self.flags, 0, outs=self.outs)
                    car.ar_reduce_bcast(self.ins, self.bc)
            self.stream.synchronize()
        except Exception as e:  # reported by the main thread
            self.error = e


def test_two_streams_from_two_threads():
    torch.cuda.synchronize()
    jobs = [Job(8, 8 * 8192, 800), Job(5, 5 * 8 * 4000, 801)]
    torch.cuda.synchronize()
    threads = [threading.Thread(target=j.run) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    for k, j in enumerate(jobs):
        assert j.error is None, f"job {k}: {j.error}"
        car.raise_on_status(j.flags, f"job {k}")
        assert np.array_equal(bits(j.one), j.want), f"job {k} one-shot"
        for r in range(j.n):
            assert np.array_equal(bits(j.outs[r]), j.want), f"job {k} two-shot rank {r}"
            assert np.array_equal(bits(j.bc[r]), j.want), f"job {k} reduce-broadcast out[{r}]"
        base = 32 + j.n * car.AR_SLOTS_PER_RANK
        # wavefront 0's group of epoch copies, one word per rank
        ep = j.flags[base:base + j.n * car.AR_EPOCH_COPIES].cpu().numpy().reshape(-1, j.n)[0, :]
        assert (ep == STEPS).all(), f"job {k} epochs {ep}"
