"""Recursive-doubling all-gather schedule and stage-order placement (no GPU):
the oracle against the pages' facts, and the library against the oracle."""
import json
import math
import os

import numpy as np
import pytest

from oracle.schedule import rd_rounds, rd_schedule, rd_simulate, ring_rounds
from workloads import host_rank_major_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_pages_round_counts():
    with open(os.path.join(GOLDEN, "recursive_doubling.json")) as f:
        g = json.load(f)
    for fact in g["facts"]:
        assert rd_rounds(fact["machines"]) == fact["rounds"]
        assert len(rd_schedule(fact["machines"], 0)) == fact["rounds"]
        if "ring_rounds" in fact:
            assert ring_rounds(fact["machines"]) == fact["ring_rounds"]


@pytest.mark.parametrize("M", list(range(1, 70)))
def test_simulation_gathers_everything_once(M):
    stage = rd_simulate(M)
    assert rd_rounds(M) == (0 if M == 1 else math.ceil(math.log2(M)))
    for n, s in enumerate(stage):
        assert len(s) == M and sorted(s) == list(range(M))      # all pieces, none twice
        assert s == [(n + k) % M for k in range(M)]               # slot k: node n + k
    # pieces moved = M - 1 per node (nothing redundant)
    assert sum(r["count"] for r in rd_schedule(M, 0)) == M - 1


def test_heads_and_tails():
    for M in (2, 5, 8, 13, 64):
        for piece in (0, 1000, 3 << 20, 5 << 20):
            for r in rd_schedule(M, 1, piece, 8 << 20):
                assert r["head"] == min(r["count"] * piece, 8 << 20)
                assert r["head"] + r["tail"] == r["count"] * piece


@pytest.fixture(scope="module")
def tide():
    import mixed_precision_rs_amd as t
    return t


def test_library_schedule_equals_oracle(tide):
    for M in range(1, 70):
        for n in range(M):
            for piece, head in ((0, 0), (3 << 20, 0), (7 << 20, 1 << 20)):
                lib = tide.rd_schedule(M, n, piece, head)
                orc = rd_schedule(M, n, piece, head or (8 << 20))
                assert len(lib) == len(orc)
                for a, b in zip(lib, orc):
                    assert a["round"] == b["round"]
                    assert (a["send_to"], a["recv_from"], a["count"]) == \
                        (b["send_to"], b["recv_from"], b["count"])
                    assert list(range(a["send_slot"], a["send_slot"] + a["count"])) == b["send_slots"]
                    assert list(range(a["recv_slot"], a["recv_slot"] + a["count"])) == b["recv_slots"]
                    assert (a["head_bytes"], a["tail_bytes"]) == (b["head"], b["tail"])


def test_library_schedule_rejects(tide):
    from mixed_precision_rs_amd import TideError
    for args in ((0, 0), (5, 5), (5, -1)):
        with pytest.raises(TideError):
            tide.rd_schedule(*args)
    with pytest.raises(TideError):
        tide.rd_schedule(8, 0, -1)


def test_stage_placement_oracle_pins(orc):
    """Placing from a stage in arrival order equals placing from the
    rank-major buffer the stage is a rotation of (np.roll by whole shards);
    first_rank = 0 is the plain placement."""
    shapes, N = [(13, 6), (2, 1), (40, 3), (1, 1), (6, 9)], 6
    S = orc.layout(shapes, N)["S"]
    for stride in (S, S + 3):
        rm = host_rank_major_bits(N * stride, seed=9)
        want = orc.allgather_place(shapes, N, rm, shard_stride=stride)
        for first in range(N):
            stage = np.roll(rm.reshape(N, stride), -first, axis=0).reshape(-1)
            got = orc.allgather_place_stage(shapes, N, stage, first, shard_stride=stride)
            for a, b in zip(got, want):
                assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        orc.allgather_place_stage(shapes, N, rm, N)


def test_stage_placement_rejects_bad_first_rank(tide):
    plan = tide.plan_create([(8, 4)], 4, 2)
    with pytest.raises(tide.TideError) as e:
        tide.allgather_place_stage(plan, 0x7f0000000000, 4, [0x7f0000100000], stream=0)
    assert e.value.status_name == "TIDE_ERR_INVALID_ARG"
