"""HIP graph capture.

The calls that read a per-call pointer table (reduce-scatter; placement and
staging with the kernel engine) refuse a capturing stream with
TIDE_ERR_UNSUPPORTED and enqueue nothing. The calls that pass everything by
value (the landing sum, full grid and budgeted; the runtime-copy placement)
are captured and replayed several times, with eager work and
synchronisations between the replays, and every replay must equal the eager
result for the inputs of that moment.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, say
from workloads import device_grads, device_rank_major_bits

pytestmark = pytest.mark.gpu

SHAPES = [(300, 1000), (17, 4096), (1, 1), (5000, 64)]
N, L = 16, 4


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def test_table_calls_refuse_capture(tide):
    plan = tide.plan_create(SHAPES, N, L)
    grads = device_grads(SHAPES, L, seed=1)
    out = torch.full((N * plan.S,), 3.0, device=dev())
    sh = device_rank_major_bits(N * plan.S, seed=2)
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    slots = [torch.zeros(N * plan.S, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    tide.reduce_scatter_bf16_fp32(plan, grads, out)          # warm the plan's device state
    torch.cuda.synchronize()
    out.fill_(3.0)
    calls = {"reduce": lambda: tide.reduce_scatter_bf16_fp32(plan, grads, out),
             "placement": lambda: tide.allgather_place(plan, sh, params),
             "staging": lambda: tide.stage_grads_bf16(plan, grads, slots)}
    for name, fn in calls.items():
        g = torch.cuda.CUDAGraph()
        with pytest.raises(tide.TideError) as e:
            with torch.cuda.graph(g):
                fn()
        assert e.value.status_name == "TIDE_ERR_UNSUPPORTED", name
        del g
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    assert all(torch.all(s_.view(torch.int16) == 0) for s_ in slots)
    # the same calls still work eagerly afterwards
    tide.reduce_scatter_bf16_fp32(plan, grads, out)
    torch.cuda.synchronize()
    assert not torch.all(out == 3.0)


@pytest.mark.parametrize("budgeted", [False, True])
def test_landing_graph_replays(tide, budgeted):
    Lg, M, S = 8, 5, 100003
    C = -(-S // Lg)
    launch = tide.budgeted(max_launch_us=20) if budgeted else tide.Launch()
    inb = [torch.randn(Lg * Lg * C, device=dev()) for _ in range(Lg)]
    shards = [torch.empty(S, device=dev()) for _ in range(Lg)]
    ref = [torch.empty(S, device=dev()) for _ in range(Lg)]
    tide.landing_sum_fp32(Lg, M, S, inb, shards, launch=launch)    # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tide.landing_sum_fp32(Lg, M, S, inb, shards, launch=launch)
    for rep in range(4):
        for t in inb:                     # eager work between the replays: new inputs
            t.normal_()
        torch.cuda.synchronize()
        g.replay()
        tide.landing_sum_fp32(Lg, M, S, inb, ref, launch=launch)
        torch.cuda.synchronize()
        for b in range(Lg):
            assert torch.equal(shards[b].view(torch.int32), ref[b].view(torch.int32)), (rep, b)
        say("landing graph replay %d ok (budgeted=%s)" % (rep, budgeted))


def test_runtime_copy_placement_graph_replays(tide):
    plan = tide.plan_create(SHAPES, N, 1)
    sh = device_rank_major_bits(N * plan.S, seed=5)
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    ref = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    tide.allgather_place(plan, sh, params, engine="runtime")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tide.allgather_place(plan, sh, params, engine="runtime")
    for rep in range(4):
        sh.copy_(device_rank_major_bits(N * plan.S, seed=10 + rep))
        torch.cuda.synchronize()
        g.replay()
        tide.allgather_place(plan, sh, ref)                 # kernel engine, eager
        torch.cuda.synchronize()
        for p in range(len(SHAPES)):
            assert torch.equal(params[p].view(torch.int16), ref[p].view(torch.int16)), (rep, p)
