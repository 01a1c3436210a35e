"""Placement from a recursive-doubling stage buffer on the GPU, through the C
ABI, against the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import SENTINEL_BF16, bits_of, same_u16, say, to_dev_bf16
from oracle.schedule import rd_simulate
from workloads import host_rank_major_bits
from workloads.configs import padding_stress_shapes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


@pytest.mark.parametrize("engine", ["kernel", "runtime"])
def test_stage_placement(tide, orc, engine):
    groups = [([(8, 4), (4, 4), (12, 4)], 4),
              ([(37, 3), (5, 16), (640, 64), (3, 1), (100, 4096)], 8),
              (padding_stress_shapes(11, count=20, max_rows=300, ks=(1, 64, 4096)), 48)]
    for gi, (shapes, N) in enumerate(groups):
        plan = tide.plan_create(shapes, N, 1)
        for stride_extra, off in ((0, 0), (3, 1)):
            stride = plan.S + stride_extra
            stage = host_rank_major_bits(N * stride, seed=gi)
            sh = to_dev_bf16(stage, (N * stride,), off)
            for first in sorted({0, 1, N // 2, N - 1}):
                for rr in ((0, N), (min(1, N - 1), N - 1)):
                    if rr[1] <= rr[0]:
                        continue
                    say("stage %s group %d first=%d ranks=%s" % (engine, gi, first, rr))
                    want = [np.full(t * k, SENTINEL_BF16, np.uint16) for t, k in shapes]
                    orc.allgather_place_stage(shapes, N, stage, first, shard_stride=stride,
                                              rank_range=rr, params=want)
                    params = [to_dev_bf16(np.full(t * k, SENTINEL_BF16, np.uint16), (t, k))
                              for t, k in shapes]
                    tide.allgather_place_stage(plan, sh, first, params, shard_stride=stride,
                                               engine=engine,
                                               launch=tide.Launch(rank_begin=rr[0], rank_end=rr[1]))
                    torch.cuda.synchronize()
                    for p in range(len(shapes)):
                        same_u16(bits_of(params[p]), want[p], "param %d" % p)


def test_recursive_doubling_end_to_end(tide, orc):
    """M nodes of L ranks: each node's stage, filled by simulating the
    schedule, placed with first_rank = n * L, gives every node the same
    parameters as placing the rank-major buffer."""
    M, L = 5, 4
    N = M * L
    shapes = [(330, 64), (17, 1), (90, 520)]
    plan = tide.plan_create(shapes, N, 1)
    S = plan.S
    rm = host_rank_major_bits(N * S, seed=3)
    want = orc.allgather_place(shapes, N, rm)
    node_pieces = rm.reshape(M, L * S)            # node m's piece = its L shards
    for n, slots in enumerate(rd_simulate(M)):
        stage = np.concatenate([node_pieces[m] for m in slots])
        params = [torch.empty((t, k), dtype=torch.bfloat16, device="cuda") for t, k in shapes]
        tide.allgather_place_stage(plan, to_dev_bf16(stage, (N * S,)), n * L, params)
        torch.cuda.synchronize()
        for p in range(len(shapes)):
            same_u16(bits_of(params[p]), want[p], "node %d param %d" % (n, p))


@pytest.mark.parametrize("name", ["llama70b_layer", "qwen3_moe_layer"])
def test_stage_placement_full_size(tide, orc, name):
    """Stage-order placement at the benchmark's size, half the ranks rotated
    (stage slot k holds rank (N/2 + k) mod N): every parameter equals the
    torch view of the unrotated shards; one parameter also against the oracle."""
    from gpu_util import dev
    from workloads import device_rank_major_bits
    from workloads.configs import CONFIGS
    cfg = CONFIGS[name]
    N = cfg.N
    plan = tide.plan_create(cfg.shapes, N, 1)
    S = plan.S
    lay = orc.layout(cfg.shapes, N)
    rank_major = device_rank_major_bits(N * S, seed=3)
    first = N // 2
    stage = torch.roll(rank_major.view(N, S), shifts=-first, dims=0).contiguous().view(-1)
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in cfg.shapes]
    say("%s: stage-order placement, first rank %d" % (name, first))
    tide.allgather_place_stage(plan, stage, first, params)
    torch.cuda.synchronize()
    v = rank_major.view(N, S)
    for p, (t, k) in enumerate(cfg.shapes):
        o, s = int(lay["o"][p]), int(lay["s"][p])
        want = v[:, o:o + s].reshape(-1)[:t * k]
        assert torch.equal(params[p].reshape(-1).view(torch.int16), want.view(torch.int16)), p
    p = int(np.argmin([t * k for t, k in cfg.shapes]))
    sub = [cfg.shapes[p]]
    o, s = int(lay["o"][p]), int(lay["s"][p])
    sub_stage = bits_of(stage.view(N, S)[:, o:o + s].contiguous())
    want = orc.allgather_place_stage(sub, N, sub_stage, first)[0]
    same_u16(bits_of(params[p]), want, "%s param %d vs oracle" % (name, p))
