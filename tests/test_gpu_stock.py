"""The stock FSDP2 path (torch._chunk_cat pack into fp32 per contributor,
summed in contributor order; split_with_sizes_copy for the all-gather
copy-out) computes the same bits as this library's reduce-scatter and
placement (on the GPU, at a multi-tile size)."""
import numpy as np
import pytest
import torch

from gpu_util import dev
from workloads import device_grads, device_rank_major_bits
from workloads.configs import padding_stress_shapes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def test_stock_path_equals_ours(tide):
    shapes = padding_stress_shapes(5, count=25, max_rows=400, ks=(1, 64, 4096))
    N, L = 48, 8
    plan = tide.plan_create(shapes, N, L)
    S = plan.S
    grads = device_grads(shapes, L, seed=5, sigma=1.0, outlier_frac=0.01)
    acc = torch.empty((N, S), dtype=torch.float32, device=dev())
    tmp = torch.empty_like(acc)
    torch._chunk_cat(grads[0], dim=0, num_chunks=N, out=acc)
    for c in range(1, L):
        torch._chunk_cat(grads[c], dim=0, num_chunks=N, out=tmp)
        acc.add_(tmp)
    out = torch.empty(N * S, dtype=torch.float32, device=dev())
    tide.reduce_scatter_bf16_fp32(plan, grads, out)
    torch.cuda.synchronize()
    assert torch.equal(acc.view(-1).view(torch.int32), out.view(torch.int32))

    sh = device_rank_major_bits(N * S, seed=6)
    sizes = [-(-t // N) * k for t, k in shapes]
    padded = [torch.empty((N, sz), dtype=torch.bfloat16, device=dev()) for sz in sizes]
    torch.split_with_sizes_copy(sh.view(N, S), sizes, dim=1, out=padded)
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in shapes]
    tide.allgather_place(plan, sh, params)
    torch.cuda.synchronize()
    for (t, k), pad, got in zip(shapes, padded, params):
        want = pad.reshape(-1)[:t * k]
        assert torch.equal(got.reshape(-1).view(torch.int16), want.view(torch.int16))
