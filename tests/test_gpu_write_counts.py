"""Every output element lands exactly once: the debug write counts
(tide_launch.write_counts) of the reduce-scatter, the placement, the staging
and the landing sum, against the oracle's own write counts (reduce-scatter)
and against the index sets the layout defines (the rest).

Several writes of one element with the same value, or a write outside the
call's range, would pass a value check but not this one.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, say, to_dev_bf16
from workloads import host_grads, host_rank_major_bits
from workloads.configs import padding_stress_shapes

pytestmark = pytest.mark.gpu

GROUPS = [
    ([(8, 4), (4, 4), (12, 4)], 4, 2),
    ([(5, 3), (1, 7), (9, 1), (16, 2), (0, 5)], 4, 3),
    ([(3, 5)], 8, 2),
    ([(300, 1000), (17, 4096), (1, 1), (5000, 64)], 64, 8),
    (padding_stress_shapes(5, count=24, max_rows=400, ks=(1, 3, 64, 4096)), 48, 4),
    # Reduce tile order: 50 small pieces (24,576 elements each, 1.2 M per rank)
    # form one long group walked rank by rank; a 131,072-element piece closes
    # it; 50 more small pieces and a tiny one follow.
    ([(768, 256)] * 50 + [(2048, 512)] + [(768, 256)] * 50 + [(7, 3)], 8, 2),
]


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _launches(tide, rb=0, re=0):
    return {"full": tide.Launch(rank_begin=rb, rank_end=re),
            "budgeted": tide.budgeted(max_launch_us=2, rank_begin=rb, rank_end=re),
            "scalar": tide.Launch(flags=tide.FLAG_SCALAR_PATH, rank_begin=rb, rank_end=re)}


def _param_major_expected(lay, shapes, N, rb, re):
    """1 at N * o_p + f for every element f of parameter p held by ranks [rb, re)."""
    want = np.zeros(N * int(lay["S"]), np.int32)
    for p, (t, k) in enumerate(shapes):
        s, o = int(lay["s"][p]), int(lay["o"][p])
        lo, hi = rb * s, min(re * s, t * k)
        if hi > lo:
            want[N * o + lo:N * o + hi] = 1
    return want


@pytest.mark.parametrize("gi", range(len(GROUPS)))
def test_each_element_lands_once(tide, orc, gi):
    shapes, N, L = GROUPS[gi]
    plan = tide.plan_create(shapes, N, L)
    S = plan.S
    lay = orc.layout(shapes, N)
    grads = host_grads(shapes, L, seed=gi)
    g_dev = [[to_dev_bf16(grads[c][p], (t, k), (c + p) % 2) for p, (t, k) in enumerate(shapes)]
             for c in range(L)]
    ranges = [(0, N)] + ([(1, N - 1)] if N > 2 else [])
    for rb, re in ranges:
        for kind, launch in _launches(tide, rb, re).items():
            say("write counts group %d %s ranks [%d, %d)" % (gi, kind, rb, re))
            # reduce-scatter, stride S + 3: the gaps between shards must stay 0
            stride = S + 3
            out = torch.empty(N * stride, dtype=torch.float32, device=dev())
            cnt = torch.zeros(N * stride, dtype=torch.int32, device=dev())
            tide.reduce_scatter_bf16_fp32(plan, g_dev, out, out_stride=stride,
                                          launch=tide.counted(launch, cnt))
            torch.cuda.synchronize()
            _, want = orc.reduce_scatter(shapes, N, L, grads, out_stride=stride,
                                         rank_range=(rb, re), count_writes=True)
            assert np.array_equal(cnt.cpu().numpy(), want.reshape(-1).astype(np.int32)), \
                "reduce-scatter write counts (%s, [%d, %d))" % (kind, rb, re)

            # placement, in rank-major and in rotated stage order
            sh = to_dev_bf16(host_rank_major_bits(N * S, seed=gi), (N * S,))
            want_p = _param_major_expected(lay, shapes, N, rb, re)
            for first in sorted({0, N // 2}):
                params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev())
                          for t, k in shapes]
                cnt = torch.zeros(N * S, dtype=torch.int32, device=dev())
                tide.allgather_place_stage(plan, sh, first, params,
                                           launch=tide.counted(launch, cnt))
                torch.cuda.synchronize()
                assert np.array_equal(cnt.cpu().numpy(), want_p), \
                    "placement write counts (%s, first %d)" % (kind, first)

            # staging into L slots
            slots = [torch.empty(N * S, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
            cnt = torch.zeros(L * N * S, dtype=torch.int32, device=dev())
            tide.stage_grads_bf16(plan, g_dev, slots, launch=tide.counted(launch, cnt))
            torch.cuda.synchronize()
            assert np.array_equal(cnt.cpu().numpy(), np.tile(want_p, L)), \
                "staging write counts (%s)" % kind


def test_landing_each_element_once(tide):
    for L, M, S in ((4, 3, 5003), (8, 8, 4096), (3, 1, 7)):
        C = -(-S // L)
        inb = [torch.randn(L * L * C, device=dev()) for _ in range(L)]
        for kind, launch in _launches(tide).items():
            shards = [torch.empty(S, device=dev()) for _ in range(L)]
            cnt = torch.zeros(L * S, dtype=torch.int32, device=dev())
            tide.landing_sum_fp32(L, M, S, inb, shards, launch=tide.counted(launch, cnt))
            torch.cuda.synchronize()
            assert torch.all(cnt == 1), "landing write counts (L=%d M=%d S=%d %s)" % (L, M, S, kind)


def test_counts_array_too_small_is_refused(tide):
    shapes, N, L = GROUPS[1]
    plan = tide.plan_create(shapes, N, L)
    g = [[torch.zeros((t, k), dtype=torch.bfloat16, device=dev()) for t, k in shapes]
         for _ in range(L)]
    out = torch.full((N * plan.S,), 5.0, device=dev())
    cnt = torch.zeros(N * plan.S - 1, dtype=torch.int32, device=dev())
    with pytest.raises(tide.TideError):
        tide.reduce_scatter_bf16_fp32(plan, g, out, launch=tide.counted(tide.Launch(), cnt))
    sh = torch.zeros(N * plan.S, dtype=torch.bfloat16, device=dev())
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in shapes]
    big = torch.zeros(N * plan.S, dtype=torch.int32, device=dev())
    with pytest.raises(tide.TideError):
        tide.allgather_place(plan, sh, params, engine="runtime",
                             launch=tide.counted(tide.Launch(), big))
    torch.cuda.synchronize()
    assert torch.all(out == 5.0) and torch.all(cnt == 0) and torch.all(big == 0)
