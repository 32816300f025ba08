"""Algorithmic HBM bytes of each kernel, for throughput and roofline figures.

Counts what the method must move on one GPU when the n ranks' buffers are n
allocations on that GPU: every read of a rank buffer, segment or wire buffer
and every write, each byte once.  S = numel * element size (bytes per rank).

  oneshot                 reads n*S               writes S
  twoshot, one rank       reads S (RS: segment r of n inputs) + S (AG: all n segments)
                          writes S/n (segment) + S (output)
  twoshot, all n ranks    n times the above
  twoshot RS only / AG only, per rank: reads S / S, writes S/n / S
  twoshot under LL, one   reads S (RS) + n*2S/n (AG: all n LL segment wires)
    rank                  writes 2S/n (its segment wire) + S (output)
  twoshot under LL128     as under LL with LL128 segment wires W(S/n)
  reduce_bcast, one rank  reads S (its 1/n of n inputs)   writes S (1/n into n outputs)
  reduce_bcast, all n     reads n*S               writes n*S
  push, one sender        reads S                 writes ndst*S
  LL / LL128 pack, each   reads S                 writes W(S)
  LL / LL128 reduce       reads n*W(S)            writes S
  LL / LL128 send and     reads S (own message) + (n-1)*W(S) (the peers' wires)
    receive, one launch   writes W(S) (own wire) + S
  one-shot + residual +   reads n*S + S (residual) + one row (the weight)
    RMSNorm               writes S (residual_out) + S (output)
  two-shot + residual +   reads S (its rows of n inputs) + S/n (residual) + one row
    RMSNorm, one rank       + 2(n-1)S/n (the peers' rows of both results)
                          writes 2S/n (own rows) + 2S/n (segment) + 2(n-1)S/n

The fused two-shot kernel writes rank r's own segment of its output straight
from the reduce-scatter's registers and never reads it back, so it moves
S/n (S/n wire bytes under LL) fewer reads per rank than the method's count;
twoshot_kernel() gives that kernel count, which is reported beside the
algorithmic one but never used for a rate.  W(S) = 8*ceil(S/4) for LL (4 data bytes per 8-byte line) and
128*ceil(S/120) for LL128 (120 data bytes per 128-byte line) -- the line
formats of the protocol table on "集合通信：NCCL 的算法、协议与推理框架的定制
all-reduce".  The flag region (a few KiB) is left out.
"""
from __future__ import annotations

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak


def wire_bytes(proto: str, S: int) -> int:
    if proto == "ll":
        return 8 * ((S + 3) // 4)
    if proto == "ll128":
        return 128 * ((S + 119) // 120)
    raise ValueError(proto)


def oneshot(n: int, S: int):
    return n * S, S


def oneshot_rmsnorm(n: int, S: int, row_bytes: int):
    """One-shot all-reduce + residual add + RMSNorm over rows of row_bytes:
    the n inputs and the residual once, the weight (one row) once; residual_out
    and the output once."""
    return n * S + S + row_bytes, 2 * S


def twoshot_rmsnorm(n: int, S: int, row_bytes: int):
    """One rank's share of the two-shot fused all-reduce + RMSNorm."""
    peers = 2 * (n - 1) * (S // n)
    return S + S // n + row_bytes + peers, 4 * (S // n) + peers


def twoshot(n: int, S: int, ranks: int):
    """Fused two-shot; ranks = how many emulated ranks the launch computes (1 or n)."""
    return ranks * 2 * S, ranks * (S // n) + ranks * S


def twoshot_kernel(n: int, S: int, ranks: int):
    """What the fused two-shot kernel itself moves: the all-gather does not
    read back the rank's own segment (it is stored from registers)."""
    return ranks * (S + (n - 1) * (S // n)), ranks * (S // n) + ranks * S


def twoshot_ll(n: int, S: int, ranks: int, proto: str = "ll"):
    """Fused two-shot with LL (or LL128) segment wires."""
    w = wire_bytes(proto, S // n)
    return ranks * (S + n * w), ranks * (w + S)


def twoshot_rs(n: int, S: int, ranks: int):
    return ranks * S, ranks * (S // n)


def twoshot_ag(n: int, S: int, ranks: int):
    return ranks * S, ranks * S


def reduce_bcast(n: int, S: int, ranks: int):
    """ranks = how many emulated ranks' shares the launch computes; each
    share reads its 1/n of every input and writes it into every output."""
    return ranks * S, ranks * S


def push(S: int, ndst: int, count: int = 1):
    return count * S, count * ndst * S


def ll_pack(proto: str, S: int, count: int = 1):
    return count * S, count * wire_bytes(proto, S)


def ll_reduce(proto: str, n: int, S: int):
    return n * wire_bytes(proto, S), S


def ll_allreduce(proto: str, n: int, S: int):
    """One GPU's LL / LL128 step in one launch: its own term comes from its
    message, not from its wire buffer."""
    W = wire_bytes(proto, S)
    return S + (n - 1) * W, W + S


def total(rw) -> int:
    return int(rw[0] + rw[1])
