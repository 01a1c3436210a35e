"""The DMA-engine (SDMA) path of the placement and of the Slot-Reuse staging
against the CPU oracle, bit for bit, through the C ABI.

The engine path is host-synchronous (it waits for the stream, runs linear
copies spread over the GPU's DMA engines and returns once they are done), so
these tests also check the ordering both ways: a source written by a kernel
just before the call, and destinations a kernel read just before and reads
just after it.
"""
import numpy as np
import pytest
import torch

from gpu_util import SENTINEL_BF16, bits_of, dev, same_u16, say, to_dev_bf16
from workloads import host_grads, host_rank_major_bits
from workloads.configs import CONFIGS, padding_stress_shapes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _params_in_one_buffer(shapes, offs, gap=5):
    """All parameters as views of one sentinel-filled bf16 buffer, parameter p
    starting offs[p] elements past a gap, so that every element a call must
    not write can be checked."""
    sizes = [t * k for t, k in shapes]
    starts, pos = [], gap
    for n, o in zip(sizes, offs):
        pos += o
        starts.append(pos)
        pos += n + gap
    buf = torch.full((pos + gap,), 0, dtype=torch.int16, device=dev())
    buf.fill_(int(np.int16(SENTINEL_BF16.view(np.int16))))
    bbuf = buf.view(torch.bfloat16)
    views = [bbuf[a:a + n].view(t, k) for a, n, (t, k) in zip(starts, sizes, shapes)]
    return bbuf, views, starts


def _expect_buffer(total, starts, want_p):
    e = np.full(total, SENTINEL_BF16, np.uint16)
    for a, w in zip(starts, want_p):
        e[a:a + w.size] = w
    return e


def test_engine_count(tide):
    n = tide.dma_engine_count(0)
    say("DMA engines for copies inside device 0: %d" % n)
    assert 1 <= n <= 32


@pytest.mark.parametrize("seed", range(8))
def test_placement_fuzz(tide, orc, seed):
    """Random ragged groups: strides above S, sources at 2 mod 4 bytes,
    parameters at odd element offsets, rank subsets and rotated stage order;
    the SDMA path writes exactly the oracle's bytes and nothing else."""
    rng = np.random.default_rng(1000 + seed)
    shapes = padding_stress_shapes(seed, count=int(rng.integers(1, 14)), max_rows=90,
                                   ks=(1, 3, 64, 257))
    N = int(rng.integers(1, 12))
    plan = tide.plan_create(shapes, N, 1)
    S = plan.S
    stride = S + int(rng.integers(0, 4))
    shard_off = int(rng.integers(0, 2))
    first = int(rng.integers(0, N))
    rb = int(rng.integers(0, N))
    re = int(rng.integers(rb, N + 1))
    offs = [int(x) for x in rng.integers(0, 4, len(shapes))]
    say("sdma placement fuzz seed %d: P=%d N=%d stride=S+%d shard_off=%d first=%d ranks [%d,%d)"
        % (seed, len(shapes), N, stride - S, shard_off, first, rb, re))
    bits = host_rank_major_bits(N * stride, seed=seed + 7)
    sh = to_dev_bf16(bits, (N * stride,), shard_off)
    buf, views, starts = _params_in_one_buffer(shapes, offs)
    want_p = [np.full(t * k, SENTINEL_BF16, np.uint16) for t, k in shapes]
    if re > rb:
        orc.allgather_place_stage(shapes, N, bits, first, shard_stride=stride,
                                  rank_range=(rb, re), params=want_p)
    launch = tide.Launch(rank_begin=rb, rank_end=re) if re > rb else tide.Launch(rank_begin=N, rank_end=N)
    tide.allgather_place_stage(plan, sh, first, views, shard_stride=stride, engine="sdma",
                               launch=launch)
    torch.cuda.synchronize()
    same_u16(bits_of(buf), _expect_buffer(buf.numel(), starts, want_p), "sdma placement")


def test_placement_equals_kernel_engine_on_wan_group(tide):
    """The Wan2.2 DiT block group at full size (1.4 GB placed, its 6 x 5120
    modulation padded to one row per rank): the SDMA engine and the kernel
    engine write the same bytes."""
    cfg = CONFIGS["wan22_dit_block"]
    plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
    g = torch.Generator(device=dev())
    g.manual_seed(3)
    sh = torch.randint(-32768, 32767, (cfg.N * plan.S,), dtype=torch.int16, device=dev(),
                       generator=g).view(torch.bfloat16)
    a = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in cfg.shapes]
    b = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in cfg.shapes]
    tide.allgather_place(plan, sh, a, engine="kernel")
    tide.allgather_place(plan, sh, b, engine="sdma")
    torch.cuda.synchronize()
    for p in range(plan.P):
        assert torch.equal(a[p].view(torch.int16), b[p].view(torch.int16)), p


def test_ordering_against_kernels(tide, orc):
    """A kernel writes the shards and another reads the parameters right
    before the call (nothing synchronised in between); kernels read the
    parameters right after it. Repeated with new contents each time, so stale
    data from an earlier round would show."""
    shapes = [(300, 64), (77, 1), (129, 257), (5, 4096)]
    N = 8
    plan = tide.plan_create(shapes, N, 1)
    S = plan.S
    params = [torch.zeros((t, k), dtype=torch.bfloat16, device=dev()) for t, k in shapes]
    src = torch.empty(N * S, dtype=torch.int16, device=dev())
    sh = torch.empty(N * S, dtype=torch.int16, device=dev())
    for rnd in range(4):
        bits = host_rank_major_bits(N * S, seed=50 + rnd)
        want = orc.allgather_place(shapes, N, bits)
        src.copy_(torch.from_numpy(bits.view(np.int16)).to(dev()))
        torch.cuda.synchronize()
        sh.copy_(src)                                  # kernel producer, not synchronised
        before = [p.float().sum() for p in params]     # kernel readers of the old contents
        tide.allgather_place(plan, sh.view(torch.bfloat16), params, engine="sdma")
        want_dev = [torch.from_numpy(w.view(np.int16)).to(dev()) for w in want]
        for p in range(plan.P):
            assert torch.equal(params[p].view(torch.int16).reshape(-1), want_dev[p]), (rnd, p)
        del before


@pytest.mark.parametrize("seed", range(4))
def test_staging_then_reduce(tide, orc, seed):
    """Slot-Reuse staging on the DMA engines, then the reduce reading the slots
    through the table tide_plan_slot_grads builds: equal to the oracle's
    staging and to its reduce of the original gradients."""
    rng = np.random.default_rng(seed)
    shapes = padding_stress_shapes(seed + 20, count=int(rng.integers(2, 10)), max_rows=60,
                                   ks=(1, 5, 64))
    N, L = int(rng.integers(1, 9)), int(rng.integers(1, 5))
    plan = tide.plan_create(shapes, N, L)
    NS = N * plan.S
    grads = host_grads(shapes, L, seed=seed + 3)
    offs = rng.integers(0, 3, (L, len(shapes)))
    g_dev = [[to_dev_bf16(grads[c][p], (t, k), int(offs[c][p])) for p, (t, k) in enumerate(shapes)]
             for c in range(L)]
    slot_off = int(rng.integers(0, 2))
    slots = [to_dev_bf16(np.full(NS, SENTINEL_BF16, np.uint16), (NS,), slot_off) for _ in range(L)]
    rb = int(rng.integers(0, N))
    re = int(rng.integers(rb + 1, N + 1))
    say("sdma staging seed %d: P=%d N=%d L=%d ranks [%d,%d)" % (seed, len(shapes), N, L, rb, re))
    tide.stage_grads_bf16(plan, g_dev, slots, engine="sdma",
                          launch=tide.Launch(rank_begin=rb, rank_end=re))
    want_slots = orc.stage_grads(shapes, N, L, grads,
                                 slots=[np.full(NS, SENTINEL_BF16, np.uint16) for _ in range(L)],
                                 rank_range=(rb, re))
    for c in range(L):
        same_u16(bits_of(slots[c]), want_slots[c], "slot %d" % c)
    # Whole range staged, then the reduce from the slots.
    tide.stage_grads_bf16(plan, g_dev, slots, engine="sdma")
    out = torch.full((NS,), float("nan"), dtype=torch.float32, device=dev())
    tide.reduce_scatter_bf16_fp32(plan, tide.slot_grads_table(plan, slots), out)
    torch.cuda.synchronize()
    want = orc.reduce_scatter(shapes, N, L, grads).reshape(-1)
    assert np.array_equal(bits_of(out).view(np.uint32), want.view(np.uint32))


def test_refused_while_capturing(tide):
    shapes = [(8, 4), (4, 4)]
    plan = tide.plan_create(shapes, 2, 1)
    sh = torch.zeros(2 * plan.S, dtype=torch.bfloat16, device=dev())
    params = [torch.zeros(s, dtype=torch.bfloat16, device=dev()) for s in shapes]
    g = torch.cuda.CUDAGraph()
    with pytest.raises(tide.TideError) as ei:
        with torch.cuda.graph(g):
            tide.allgather_place(plan, sh, params, engine="sdma")
    assert ei.value.status_name == "TIDE_ERR_UNSUPPORTED"
    torch.cuda.synchronize()
