"""The bandwidth-ceiling kernels (tide_diag_stream) do what the benchmark
says they measure: copy and write move the bytes, and the reduce-pattern
kernel gives the fixed-order fp32 sum of its sources (exact here: small
integers, whose sums binary32 represents exactly in any order)."""
import numpy as np
import pytest
import torch

from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def test_copy_write_read(tide):
    n = 2048 * 300
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device=dev())
    dst = torch.full((n // 4,), 7, dtype=torch.int32, device=dev())
    tide.diag_stream(2, [src], dst, n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    tide.diag_stream(1, [], dst, n)
    torch.cuda.synchronize()
    assert int(dst.abs().sum()) == 0
    tide.diag_stream(0, [src], dst, n)           # reads only
    dst.fill_(7)
    tide.diag_stream(2, [src], dst, n, workgroups=3)   # 1024-thread workgroups
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("nsrc", [1, 3, 8])
def test_reduce_pattern(tide, nsrc):
    n = 1024 * 257
    g = torch.Generator(device=dev())
    g.manual_seed(nsrc)
    srcs = [torch.randint(-256, 257, (n,), generator=g, device=dev()).to(torch.float32)
            .to(torch.bfloat16) for _ in range(nsrc)]
    want = sum(s.float().cpu().numpy().astype(np.float64) for s in srcs)
    for wg in (0, 5):
        dst = torch.full((n,), float("nan"), device=dev())
        tide.diag_stream(3, srcs, dst, n, workgroups=wg)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy().astype(np.float64), want)


def test_rejects(tide):
    x = torch.zeros(4096, dtype=torch.float32, device=dev())
    with pytest.raises(tide.TideError):
        tide.diag_stream(4, [x], x, 2048)
    with pytest.raises(tide.TideError):
        tide.diag_stream(2, [x], x, 1000)        # not a whole unit
    with pytest.raises(tide.TideError):
        tide.diag_stream(3, [x] * 9, x, 1024)    # too many sources
