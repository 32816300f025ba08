"""Byte accounting and the alpha-beta cost model (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The cost model follows the alpha-beta comparison on "集合通信：NCCL 的算法、协议与
推理框架的定制 all-reduce" (anrans.github.io serving/comm/nccl, 算法 section):
every algorithm pays a fixed cost alpha per synchronised step and moves its
per-GPU bytes at link bandwidth beta.  The bandwidth conventions (algbw,
busbw and the busbw factors per collective) follow the "读懂 nccl-tests"
section of the same page and the algbw/busbw section of "多 GPU 与 NCCL".
The per-rank byte counts follow the one-shot / two-shot bullets (算法) and
the ring section of "多 GPU 与 NCCL".
"""
from __future__ import annotations

import math

# The page's 8-GPU NVLink example: 8 GPUs, 450 GB/s per GPU per direction,
# 1.5 microseconds of fixed cost per step.
PAGE_N = 8
PAGE_BETA = 450e9
PAGE_ALPHA = 1.5e-6


def t_ring(S, n=PAGE_N, alpha=PAGE_ALPHA, beta=PAGE_BETA):
    """Ring: 2(n-1) steps; each GPU sends 2(n-1)/n of S."""
    return 2 * (n - 1) * alpha + 2 * (n - 1) / n * S / beta


def t_tree(S, n=PAGE_N, alpha=PAGE_ALPHA, beta=PAGE_BETA):
    """Double binary tree: 2 log2(n) steps, about 2S per GPU."""
    return 2 * math.log2(n) * alpha + 2 * S / beta


def t_oneshot(S, n=PAGE_N, alpha=PAGE_ALPHA, beta=PAGE_BETA):
    """One-shot: two synchronisations; each GPU reads the other n-1 full buffers."""
    return 2 * alpha + (n - 1) * S / beta


def t_twoshot(S, n=PAGE_N, alpha=PAGE_ALPHA, beta=PAGE_BETA):
    """Two-shot: four fixed costs; reads 2(n-1)/n of S per GPU."""
    return 4 * alpha + 2 * (n - 1) / n * S / beta


def t_nvls(S, n=PAGE_N, alpha=PAGE_ALPHA, beta=PAGE_BETA):
    """In-switch reduction: each GPU sends one copy and receives one copy."""
    return 2 * alpha + S / beta


ALGOS = {"ring": t_ring, "tree": t_tree, "one-shot": t_oneshot, "two-shot": t_twoshot, "NVLS": t_nvls}


def algbw(S, t):
    """Algorithm bandwidth: bytes per GPU over time."""
    return S / t


BUSBW_FACTOR = {
    "all-reduce": lambda n: 2 * (n - 1) / n,
    "all-gather": lambda n: (n - 1) / n,
    "reduce-scatter": lambda n: (n - 1) / n,
    "broadcast": lambda n: 1.0,
}


def busbw(S, t, n, collective="all-reduce"):
    """Bus bandwidth: algbw times the collective's correction factor."""
    return algbw(S, t) * BUSBW_FACTOR[collective](n)


def crossover_oneshot_twoshot(n=PAGE_N, alpha=PAGE_ALPHA, beta=PAGE_BETA):
    """Message size where the one-shot and two-shot model times are equal.

    Setting 2a + (n-1)S/b = 4a + 2(n-1)/n S/b gives S* = 2ab / ((n-1)(1-2/n)).
    At n = 2 the denominator vanishes: both read S, one-shot saves a sync and is
    never slower, so there is no crossover (returns inf)."""
    den = (n - 1) * (1 - 2 / n)
    if den == 0:
        return math.inf
    return 2 * alpha * beta / den


def remote_bytes_per_rank(algo, S, n):
    """Bytes each GPU pulls from its peers (the model's link traffic)."""
    if algo == "one-shot":
        return (n - 1) * S
    if algo in ("two-shot", "ring"):
        return 2 * (n - 1) / n * S
    if algo == "NVLS":
        return S
    raise ValueError(algo)


def ll_wire_bytes(proto, S):
    """Bytes on the wire for an S-byte message: LL packs 4 data bytes per
    8-byte line, LL128 packs 120 data bytes per 128-byte line."""
    if proto == "ll":
        return 8 * math.ceil(S / 4)
    if proto == "ll128":
        return 128 * math.ceil(S / 120)
    raise ValueError(proto)


def hbm_bytes(op, S, n, proto=None):
    """HBM bytes (reads, writes) the method moves on one GPU when the n ranks'
    buffers are n allocations on that GPU: every read of a rank buffer,
    segment or wire buffer and every write, each byte once.

    Written from the steps of each operation, not from any kernel:
    one-shot -- read every rank's message, write the sum (算法, one-shot).
    Two-shot, one rank's share -- the reduce-scatter reads segment r of all
    n messages (S bytes) and writes the reduced segment (S/n); the
    all-gather reads all n reduced segments (S) and writes the output (S)
    (算法, two-shot: reduce-scatter then all-gather; "多 GPU 与 NCCL", 集合通信).
    All n ranks: n times that.  LL / LL128 -- the sender reads its message
    and writes its wire; the receiver reads n wires and writes the sum
    (协议 table: 4 data bytes per 8-byte line, 120 per 128-byte line).  The
    two-shot under LL carries each segment as an LL wire of twice its bytes.
    A kernel may move fewer bytes than this (the fused two-shot writes its
    own segment of the output from registers and never reads it back); that
    saving is the kernel's, not the method's, and is not counted here."""
    if op == "oneshot":
        return n * S, S
    if op == "twoshot_share":
        return 2 * S, S // n + S
    if op == "twoshot_full":
        return 2 * n * S, (n + 1) * S
    if op == "ll_pack":
        return S, ll_wire_bytes(proto, S)
    if op == "ll_reduce":
        return n * ll_wire_bytes(proto, S), S
    if op == "ll_allreduce":
        # one rank's step: its message read and its wire written (the pack),
        # the n-1 peers' wires read and the sum written (the receiver; its own
        # term is its message, already read)
        return S + (n - 1) * ll_wire_bytes(proto, S), ll_wire_bytes(proto, S) + S
    if op == "twoshot_ll_share":
        # as twoshot_share, with every segment an LL wire of its S/n bytes
        w = ll_wire_bytes("ll", S // n)
        return S + n * w, w + S
    if op == "twoshot_ll128_share":
        w = ll_wire_bytes("ll128", S // n)
        return S + n * w, w + S
    raise ValueError(op)
