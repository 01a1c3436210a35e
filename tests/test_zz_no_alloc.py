"""The allocation-free reduce-scatter (tide_reduce_scatter_bf16_fp32_noalloc)
against the eager entry point it varies, bit for bit over the whole output
buffer, through the C ABI: two calls in a row on one GPU, the second with a
smaller group, in full-grid and budgeted launches and on a rank subset; the
smaller case is also checked against the CPU oracle."""
import numpy as np
import pytest
import torch

from gpu_util import bits_of, dev, say, to_dev_bf16
from workloads import device_grads, host_grads
from workloads.configs import padding_stress_shapes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _pair(tide, plan, grads, launch, stride_extra=0):
    """Output buffers (NaN-filled, one extra shard of slack) of the eager call
    and of the allocation-free call on the same inputs."""
    stride = plan.S + stride_extra
    n = plan.N * stride + 64
    a = torch.full((n,), float("nan"), dtype=torch.float32, device=dev())
    b = torch.full((n,), float("nan"), dtype=torch.float32, device=dev())
    tide.reduce_scatter_bf16_fp32(plan, grads, a, out_stride=stride, launch=launch)
    tide.reduce_scatter_bf16_fp32_noalloc(plan, grads, b, out_stride=stride, launch=launch)
    torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    ga, gb = bits_of(a).view(np.uint32), bits_of(b).view(np.uint32)
    bad = np.flatnonzero(ga != gb)
    assert bad.size == 0, "%s: %d elements differ, first at %d" % (what, bad.size, bad[0])


@pytest.mark.parametrize("mode", ["full", "budgeted"])
def test_two_calls_second_smaller(tide, orc, mode):
    launch = tide.Launch() if mode == "full" else tide.budgeted()
    # First call: a ragged padding-stress-shaped group, 48 ranks, 8 contributors.
    big = padding_stress_shapes(7, count=60, max_rows=700, ks=(1, 64, 4096))
    say("noalloc %s: first call, P=%d, N=48, L=8" % (mode, len(big)))
    p1 = tide.plan_create(big, 48, 8)
    g1 = device_grads(big, 8, seed=3, outlier_frac=0.01)
    a, b = _pair(tide, p1, g1, launch, stride_extra=3)
    _same(a, b, "first call (%s)" % mode)
    # Second call right after: a smaller group, also checked against the oracle.
    small = padding_stress_shapes(8, count=9, max_rows=90, ks=(1, 3, 64))
    say("noalloc %s: second call, P=%d, N=7, L=3" % (mode, len(small)))
    p2 = tide.plan_create(small, 7, 3)
    hg = host_grads(small, 3, seed=5)
    g2 = [[to_dev_bf16(hg[c][p], (t, k)) for p, (t, k) in enumerate(small)] for c in range(3)]
    a, b = _pair(tide, p2, g2, launch)
    _same(a, b, "second call (%s)" % mode)
    want = orc.reduce_scatter(small, 7, 3, hg).reshape(-1)
    got = bits_of(b)[: 7 * p2.S]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_rank_subset_and_repeat(tide):
    """A rank subset, then the same call again (its tables are not uploaded a
    second time), then a different group of the same size: all equal to the
    eager call."""
    shapes = [(300, 64), (77, 1), (129, 257), (5, 4096), (1000, 8)]
    plan = tide.plan_create(shapes, 16, 4)
    grads = device_grads(shapes, 4, seed=9)
    lr = tide.Launch(rank_begin=3, rank_end=11)
    for rep in range(2):
        say("noalloc: ranks [3, 11), call %d" % rep)
        a, b = _pair(tide, plan, grads, lr)
        _same(a, b, "rank subset, call %d" % rep)
    other = device_grads(shapes, 4, seed=10)
    a, b = _pair(tide, plan, other, tide.Launch())
    _same(a, b, "other gradients")
