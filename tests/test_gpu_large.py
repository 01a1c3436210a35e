"""Offsets beyond 2^31 elements: one parameter larger than 2^31 elements and a
second whose rank-major pieces start beyond 2^31 in the output, through the
reduce-scatter, the placement, and the Slot-Reuse staging; and one reduce of
more than 2^34 elements, whose tiles outnumber the full grid's workgroups.

Checks: sampled pieces against the oracle (bit for bit), the identical-
contributor whole-output closed form (2 * f32(g) in every true element, +0
in padding), the placement against a torch view of the shards, and the
staged slot against the gradients (torch on the device).
"""
import gc

import numpy as np
import pytest
import torch

from gpu_util import bits_of, dev, same_f32, say
from workloads import device_grads, device_rank_major_bits

pytestmark = pytest.mark.gpu

# 262,201 x 8192 = 2,147,950,592 elements (> 2^31); N = 8 pads it by 7 rows.
SHAPES = [(262_201, 8192), (19, 3)]
N, L = 8, 2


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def test_beyond_int32(tide, orc):
    assert SHAPES[0][0] * SHAPES[0][1] > 2 ** 31
    plan = tide.plan_create(SHAPES, N, L)
    S = plan.S
    lay = orc.layout(SHAPES, N)
    assert S == int(lay["S"]) and (N - 1) * S + int(lay["o"][1]) > 2 ** 31
    say("large: generating %d x %d grads (%.1f GB)" % (L, len(SHAPES), L * 2 * sum(t * k for t, k in SHAPES) / 1e9))
    grads = device_grads(SHAPES, L, seed=3)
    out = torch.empty(N * S, dtype=torch.float32, device=dev())
    out.view(torch.int32).fill_(0x7FC0DEAD)
    tide.reduce_scatter_bf16_fp32(plan, grads, out)
    torch.cuda.synchronize()
    say("large: checking sampled pieces against the oracle")
    for r, p in [(0, 0), (N - 1, 0), (3, 1), (N - 1, 1)]:
        first, n = orc.piece_rows(SHAPES, N, r, p)
        rows = [bits_of(grads[c][p][first:first + n]) for c in range(L)]
        want = orc.reduce_piece(SHAPES, N, L, r, p, rows)
        o, s = int(lay["o"][p]), int(lay["s"][p])
        same_f32(bits_of(out[r * S + o: r * S + o + s]), want, "piece (r=%d, p=%d)" % (r, p))
    del out, grads
    _free()

    say("large: identical contributors, whole output")
    g0 = device_grads(SHAPES, 1, seed=4)[0]
    out = torch.empty(N * S, dtype=torch.float32, device=dev())
    tide.reduce_scatter_bf16_fp32(plan, [g0] * L, out)
    torch.cuda.synchronize()
    o2 = out.view(N, S)
    for p, (t, k) in enumerate(SHAPES):
        R, o, s = int(lay["R"][p]), int(lay["o"][p]), int(lay["s"][p])
        got = o2[:, o:o + s].reshape(N * R, k)
        assert torch.equal(got[:t].view(torch.int32),
                           (g0[p].float() * float(L)).view(torch.int32)), p
        assert torch.all(got[t:].view(torch.int32) == 0), p
    del out, o2

    say("large: Slot-Reuse staging")
    slots = [torch.empty(N * S, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    tide.stage_grads_bf16(plan, [g0] * L, slots)
    torch.cuda.synchronize()
    for c in range(L):
        for p, (t, k) in enumerate(SHAPES):
            at = N * int(lay["o"][p])
            assert torch.equal(slots[c][at:at + t * k].view(torch.int16),
                               g0[p].reshape(-1).view(torch.int16)), (c, p)
    del slots, g0
    _free()

    say("large: placement")
    sh = device_rank_major_bits(N * S, seed=6)
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    tide.allgather_place(plan, sh, params)
    torch.cuda.synchronize()
    v = sh.view(N, S)
    for p, (t, k) in enumerate(SHAPES):
        o, s = int(lay["o"][p]), int(lay["s"][p])
        want = v[:, o:o + s].reshape(-1)[:t * k]
        assert torch.equal(params[p].reshape(-1).view(torch.int16), want.view(torch.int16)), p
    del sh, params, v
    _free()
    say("large: ok")


# 2,097,160 x 8192 = 17,179,934,720 elements (> 2^34): 16,777,280 reduce
# tiles, 64 more than the full grid's 2^24 workgroups, so the last tiles are
# reached through the workgroups' loop. N = 8 divides T: no padding.
HUGE = [(2_097_160, 8192)]


def test_full_grid_cap_and_beyond_2_34(tide):
    """One reduce over more tiles than the full grid has workgroups, with
    element offsets beyond 2^34 (byte offsets beyond 2^36). Two identical
    contributors give the closed form out = 2 * f32(g) in every element
    (doubling is exact in binary32; a bf16 near its maximum doubles to inf on
    both sides). About 103 GB of device memory."""
    (t, k), = HUGE
    n = t * k
    free, _ = torch.cuda.mem_get_info()
    if free < 6 * n + (16 << 30):
        pytest.skip("needs %.0f GB of free device memory, %.0f GB free" % ((6 * n + (16 << 30)) / 1e9, free / 1e9))
    plan = tide.plan_create(HUGE, 8, 2)
    assert plan.S * 8 == n and n > 2 ** 34
    tiles = plan.trace_records(0)
    assert tiles == 1 << 24 and n // 1024 > tiles
    say("huge: drawing %d bf16 values (%.1f GB)" % (n, 2 * n / 1e9))
    g = torch.empty((t, k), dtype=torch.bfloat16, device=dev())
    flat = g.view(-1)
    gen = torch.Generator(device=dev())
    gen.manual_seed(11)
    chunk = 1 << 30
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        flat[a:b] = torch.randn(b - a, generator=gen, device=dev(), dtype=torch.float32).to(torch.bfloat16)
    out = torch.empty(n, dtype=torch.float32, device=dev())
    out.view(torch.int32).fill_(0x7FC0DEAD)
    say("huge: reduce-scatter")
    tide.reduce_scatter_bf16_fp32(plan, [[g], [g]], out)
    torch.cuda.synchronize()
    say("huge: checking every element in %d chunks" % ((n + chunk - 1) // chunk))
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        want = flat[a:b].float().mul_(2.0)
        assert torch.equal(out[a:b].view(torch.int32), want.view(torch.int32)), (a, b)
        del want
    del g, flat, out
    _free()
    say("huge: ok")
