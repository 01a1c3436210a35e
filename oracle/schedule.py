"""Recursive-doubling all-gather schedule, written from page 1 ("All-gather:
parameters land at their final address") and page 3 Figure 5(a).

TEST INFRASTRUCTURE ONLY (plain Python, small inputs): the library's own
schedule generator is checked against this, and this against the pages'
worked facts (M = 5 takes 3 rounds; M = 8 takes 3 where a ring takes 7).

The schedule as implemented here: machines 0..M-1 start with one piece
each (their own). Round d = 0, 1, ... pairs every machine with a receiver
2^d below it and a sender 2^d above it (indices mod M); it passes on the
oldest min(2^d, M - 2^d) pieces it holds and takes in as many. So the pieces
moved per round double until the final round, which, when M is not a power
of two, carries only the pieces still missing; no piece is received twice,
and after ceil(log2 M) rounds every machine holds all M. Each transfer is cut
into a small head and the remainder (the tail), the heads of a round adding
up to at most `head_bytes` (8 MiB by default, page 1), and the next round
waits for the heads to be confirmed.
"""
from typing import Dict, List


def rd_rounds(M: int) -> int:
    """Number of rounds: the smallest d with 2^d >= M (0 for M = 1)."""
    d = 0
    while (1 << d) < M:
        d += 1
    return d


def rd_schedule(M: int, n: int, piece_bytes: int = 0, head_bytes: int = 8 << 20) -> List[Dict]:
    """Node n's transfers, one dict per round:
    round, send_to, recv_from, count (pieces), send_slots (held slots sent),
    recv_slots (where the received pieces go), head, tail (bytes of the send).
    Slot k of node n's stage holds the piece of node (n + k) mod M."""
    out = []
    held = 1
    for d in range(rd_rounds(M)):
        step = 1 << d
        count = min(step, M - step)
        nbytes = count * piece_bytes
        head = min(nbytes, head_bytes)
        out.append({
            "round": d,
            "send_to": (n - step) % M,
            "recv_from": (n + step) % M,
            "count": count,
            "send_slots": list(range(0, count)),
            "recv_slots": list(range(held, held + count)),
            "head": head,
            "tail": nbytes - head,
        })
        held += count
    return out


def rd_simulate(M: int) -> List[List[int]]:
    """Run every node's schedule; return each node's stage as the list of
    node ids held in slot order. Each sent piece is the sender's slot, read
    before that round's receives land (all sends of a round use the holdings
    from the end of the previous round)."""
    stage = [[n] for n in range(M)]
    for d in range(rd_rounds(M)):
        before = [list(s) for s in stage]
        for n in range(M):
            sched = rd_schedule(M, n)[d]
            src = sched["recv_from"]
            for k, slot in zip(sched["send_slots"], sched["recv_slots"]):
                # node src sends its slot k (its send_slots) to node n
                assert slot == len(stage[n]), "receive slots must be filled in order"
                stage[n].append(before[src][k])
    return stage


def ring_rounds(M: int) -> int:
    return max(M - 1, 0)
