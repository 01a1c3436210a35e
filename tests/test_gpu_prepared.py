"""Prepared calls (tide_prepare_*, tide_call_enqueue) against the oracle, and
captured into a HIP graph.

  * a prepared reduce-scatter, placement (rank-major and rotated stage order)
    and staging, enqueued repeatedly while the contents of their buffers
    change, match the oracle every time, full grid and budgeted, with rank
    ranges;
  * enqueueing allocates no device memory;
  * one training-step-like sequence (stage, reduce from the slots, place) of
    prepared calls is captured into a graph and replayed four times with new
    gradient and shard values written eagerly between the replays; every
    replay equals the oracle.
"""
import numpy as np
import pytest
import torch

from gpu_util import bits_of, dev, same_f32, same_u16, say, to_dev_bf16
from workloads import host_grads, host_rank_major_bits

pytestmark = pytest.mark.gpu

SHAPES = [(300, 100), (17, 40), (1, 1), (500, 64), (9, 7)]
N, L = 16, 4


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _write_grads(g_dev, grads):
    for c, row in enumerate(g_dev):
        for p, t in enumerate(row):
            t.view(-1).view(torch.int16).copy_(
                torch.from_numpy(grads[c][p].view(np.int16).copy()).to(dev()))


@pytest.mark.parametrize("kind", ["full", "budgeted"])
@pytest.mark.parametrize("rr", [(0, N), (3, 11)])
def test_prepared_calls_match_oracle(tide, orc, kind, rr):
    plan = tide.plan_create(SHAPES, N, L)
    S = plan.S
    launch = (tide.Launch(rank_begin=rr[0], rank_end=rr[1]) if kind == "full" else
              tide.budgeted(max_launch_us=3, rank_begin=rr[0], rank_end=rr[1]))
    g_dev = [[torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
             for _ in range(L)]
    out = torch.full((N * S,), 7.0, device=dev())
    sh = torch.empty(N * S, dtype=torch.bfloat16, device=dev())
    params = [torch.zeros((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    rot = [torch.zeros((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    slots = [torch.zeros(N * S, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    rs = tide.prepare_reduce_scatter_bf16_fp32(plan, g_dev, out, launch=launch)
    ag = tide.prepare_allgather_place(plan, sh, params, launch=launch)
    ag_rot = tide.prepare_allgather_place(plan, sh, rot, first_rank=N // 2, launch=launch)
    st = tide.prepare_stage_grads_bf16(plan, g_dev, slots, launch=launch)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for it in range(3):
        grads = host_grads(SHAPES, L, seed=it)
        _write_grads(g_dev, grads)
        bits = host_rank_major_bits(N * S, seed=50 + it)
        sh.view(torch.int16).copy_(torch.from_numpy(bits.view(np.int16).copy()).to(dev()))
        for call in (rs, ag, ag_rot, st):
            call.enqueue()
        torch.cuda.synchronize()
        say("prepared %s ranks %s iteration %d" % (kind, rr, it))
        want = np.full(N * S, 7.0, np.float32)
        orc.reduce_scatter(SHAPES, N, L, grads, rank_range=rr, out=want)
        same_f32(bits_of(out), want, "reduce-scatter")
        want_p = orc.allgather_place(SHAPES, N, bits, rank_range=rr)
        # placement: compare the rows of the range (other rows keep earlier values)
        for p, (t, k) in enumerate(SHAPES):
            R = -(-t // N)
            lo, hi = rr[0] * R * k, min(rr[1] * R * k, t * k)
            if hi > lo:
                exp = np.asarray(want_p[p]).reshape(-1)[lo:hi]
                same_u16(bits_of(params[p])[lo:hi], exp, "placement p=%d" % p)
        # `sh` read as a stage buffer: slot k holds rank (N/2 + k) mod N
        want_r = orc.allgather_place_stage(SHAPES, N, bits, N // 2, rank_range=rr)
        for p, (t, k) in enumerate(SHAPES):
            R = -(-t // N)
            lo, hi = rr[0] * R * k, min(rr[1] * R * k, t * k)
            if hi > lo:
                same_u16(bits_of(rot[p])[lo:hi], np.asarray(want_r[p]).reshape(-1)[lo:hi],
                         "rotated placement p=%d" % p)
        want_s = orc.stage_grads(SHAPES, N, L, grads, slots=[bits_of(x).copy() for x in slots],
                                 rank_range=rr)
        for c in range(L):
            same_u16(bits_of(slots[c]), want_s[c], "slot %d" % c)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, "enqueue allocated device memory"
    for call in (rs, ag, ag_rot, st):
        call.close()


@pytest.mark.parametrize("kind", ["full", "budgeted"])
def test_prepared_step_in_a_graph(tide, orc, kind):
    """Stage into the slots, reduce from the slots, place: captured once,
    replayed four times with new inputs written eagerly in between."""
    plan = tide.plan_create(SHAPES, N, L)
    S = plan.S
    launch = tide.Launch() if kind == "full" else tide.budgeted(max_launch_us=3)
    g_dev = [[torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
             for _ in range(L)]
    slots = [torch.zeros(N * S, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    out = torch.empty(N * S, device=dev())
    sh = torch.empty(N * S, dtype=torch.bfloat16, device=dev())
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    st = tide.prepare_stage_grads_bf16(plan, g_dev, slots, launch=launch)
    rs = tide.prepare_reduce_scatter_bf16_fp32(plan, tide.slot_grads_table(plan, slots), out,
                                               launch=launch)
    ag = tide.prepare_allgather_place(plan, sh, params, launch=launch)
    _write_grads(g_dev, host_grads(SHAPES, L, seed=0))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for call in (st, rs, ag):                    # warm-up outside the capture
            call.enqueue()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.enqueue()
        rs.enqueue()
        ag.enqueue()
    for rep in range(4):
        grads = host_grads(SHAPES, L, seed=100 + rep)
        _write_grads(g_dev, grads)
        bits = host_rank_major_bits(N * S, seed=200 + rep)
        sh.view(torch.int16).copy_(torch.from_numpy(bits.view(np.int16).copy()).to(dev()))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("prepared step graph (%s) replay %d" % (kind, rep))
        same_f32(bits_of(out), orc.reduce_scatter(SHAPES, N, L, grads).reshape(-1),
                 "replay %d reduce-scatter" % rep)
        want_p = orc.allgather_place(SHAPES, N, bits)
        for p in range(len(SHAPES)):
            same_u16(bits_of(params[p]), want_p[p], "replay %d placement %d" % (rep, p))
    del g
    for call in (st, rs, ag):
        call.close()


def test_tile_cache_eviction_keeps_prepared_calls(tide, orc):
    """More distinct rank ranges than the per-device tile-table cache holds
    (256): older tables are freed after the device drains, while the table of
    a live prepared call is kept. Every result equals the oracle's."""
    shapes = [(130, 8), (17, 3), (64, 1)]
    N, L = 64, 2
    grads = host_grads(shapes, L, seed=8)
    plan = tide.plan_create(shapes, N, L)
    S = plan.S
    g = [[to_dev_bf16(grads[c][p], (t, k)) for p, (t, k) in enumerate(shapes)] for c in range(L)]
    want = orc.reduce_scatter(shapes, N, L, grads).reshape(-1)
    pinned_out = torch.full((N * S,), float("nan"), device=dev())
    call = tide.prepare_reduce_scatter_bf16_fp32(plan, g, pinned_out,
                                                 launch=tide.Launch(rank_begin=5, rank_end=40))
    ranges = [(a, b) for a in range(N) for b in range(a + 1, N + 1)][:300]
    out = torch.full((N * S,), float("nan"), device=dev())
    say("tile cache: %d distinct rank ranges" % len(ranges))
    for i, (a, b) in enumerate(ranges):
        tide.reduce_scatter_bf16_fp32(plan, g, out, launch=tide.Launch(rank_begin=a, rank_end=b))
        if i % 50 == 49:
            torch.cuda.synchronize()
            got = bits_of(out)
            assert np.array_equal(got[a * S: b * S].view(np.uint32), want[a * S: b * S].view(np.uint32))
    torch.cuda.synchronize()
    call.enqueue()
    torch.cuda.synchronize()
    got = bits_of(pinned_out)
    assert np.array_equal(got[5 * S: 40 * S].view(np.uint32), want[5 * S: 40 * S].view(np.uint32))
    assert np.all(np.isnan(got[: 5 * S])) and np.all(np.isnan(got[40 * S:]))
    call.close()
