"""Slot-Reuse staging through the C ABI against the CPU oracle, bit for bit.

  * every slot element is compared with the oracle's staging of the same
    bits into a sentinel-filled slot (so padding rows and the bytes around
    the slot must keep their sentinel);
  * the reduce-scatter that reads the staged slots (slot_grads_table) must
    equal the oracle's reduce-scatter of the original gradients;
  * rank-range pipelining (stage a range, reduce it, next range) covers the
    whole output;
  * the ordering the pages describe for the mode (page 1 "When gradients can
    be freed also needs planning"; page 3 Figure 7) on two streams: the slot
    is refilled only after the gradients were copied in (the all-gather
    vacated it), the gradient memory is released right after the staging
    call, and the next all-gather refills the slot only after the reduce has
    read it;
  * full-size workloads: every staged parameter equals its gradient (torch on
    the device), and sampled reduced pieces equal the oracle's.
"""
import gc

import numpy as np
import pytest
import torch

from gpu_util import SENTINEL_BF16, SENTINEL_F32, bits_of, dev, same_f32, same_u16, say, to_dev_bf16
from workloads import device_grads, host_grads, host_rank_major_bits, host_special_grads
from workloads.configs import CONFIGS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _sentinel_slots(L, n, off):
    bufs = [torch.empty(n + off + 8, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    for b in bufs:
        b.view(torch.int16).fill_(int(np.int16(np.uint16(SENTINEL_BF16).view(np.int16))))
    return bufs, [b[off:off + n] for b in bufs]


def run_stage(tide, orc, shapes, N, L, grads, *, grad_offs=None, slot_off=0, engine="kernel",
              launch=None, rank_range=None, check_reduce=True):
    plan = tide.plan_create(shapes, N, L)
    S = plan.S
    n = N * S
    rb, re = (0, N) if rank_range is None else rank_range
    if launch is None:
        launch = tide.Launch()
    launch.rank_begin, launch.rank_end = (rb, re) if re > rb else (N, N)
    g_dev = [[to_dev_bf16(grads[c][p], (t, k), 0 if grad_offs is None else grad_offs[c][p])
              for p, (t, k) in enumerate(shapes)] for c in range(L)]
    bufs, slots = _sentinel_slots(L, n, slot_off)
    tide.stage_grads_bf16(plan, g_dev, slots, engine=engine, launch=launch)
    torch.cuda.synchronize()
    want = [np.full(n, SENTINEL_BF16, np.uint16) for _ in range(L)]
    if re > rb:
        orc.stage_grads(shapes, N, L, grads, slots=want, rank_range=(rb, re))
    for c in range(L):
        full = np.concatenate([np.full(slot_off, SENTINEL_BF16, np.uint16), want[c],
                               np.full(8, SENTINEL_BF16, np.uint16)])
        same_u16(bits_of(bufs[c]), full, "slot %d (%s)" % (c, engine))
    if check_reduce and (rb, re) == (0, N):
        out = torch.full((n,), float(SENTINEL_F32), dtype=torch.float32, device=dev())
        tide.reduce_scatter_bf16_fp32(plan, tide.slot_grads_table(plan, slots), out)
        torch.cuda.synchronize()
        same_f32(bits_of(out), orc.reduce_scatter(shapes, N, L, grads), "reduce from slots")


GROUPS = [
    ([(8, 4), (4, 4), (12, 4)], 4, 2),                    # the worked example's group
    ([(5, 3), (1, 7), (9, 1), (16, 2), (6, 6)], 4, 3),
    ([(3, 5)], 8, 2),                                     # T < N
    ([(7, 1), (7, 2), (7, 3)], 3, 1),                     # odd N: odd N * o_p offsets
    ([(13, 6), (2, 1), (0, 4), (40, 3), (1, 1), (6, 9)], 6, 4),
    ([(300, 1000), (17, 4096), (1, 1), (5000, 64)], 64, 8),
    ([(11, 11)], 1, 5),
]


@pytest.mark.parametrize("engine", ["kernel", "runtime", "sdma"])
@pytest.mark.parametrize("gi", range(len(GROUPS)))
def test_stage_groups(tide, orc, gi, engine):
    shapes, N, L = GROUPS[gi]
    say("stage group %d (%s): %s N=%d L=%d" % (gi, engine, shapes, N, L))
    grads = host_grads(shapes, L, seed=gi)
    run_stage(tide, orc, shapes, N, L, grads, engine=engine)
    if engine == "kernel":
        run_stage(tide, orc, shapes, N, L, grads, launch=tide.budgeted(place_blocks=3,
                                                                        max_launch_us=1))
        run_stage(tide, orc, shapes, N, L, grads, launch=tide.Launch(flags=tide.FLAG_SCALAR_PATH))


def test_stage_special_values(tide, orc):
    shapes, N, L = [(37, 3), (5, 16), (64, 8), (3, 1)], 8, 8
    run_stage(tide, orc, shapes, N, L, host_special_grads(shapes, L, seed=3))


@pytest.mark.parametrize("case", range(4))
def test_stage_misaligned(tide, orc, case):
    """Gradient and slot addresses at 2-byte (scalar path) and 4-byte but not
    16-byte (dword-aligned vector path) offsets."""
    shapes, N, L = [(33, 64), (5, 1), (128, 40), (7, 3)], 8, 3
    grads = host_grads(shapes, L, seed=40 + case)
    goff = [[[0, 1, 2, 3][(case + c + p) % 4] for p in range(len(shapes))] for c in range(L)]
    say("misaligned %d: grad offsets %s, slot offset %d" % (case, goff, case))
    run_stage(tide, orc, shapes, N, L, grads, grad_offs=goff, slot_off=case)


@pytest.mark.parametrize("case", range(16))
def test_stage_fuzz(tide, orc, case):
    rng = np.random.default_rng(5000 + case)
    P = int(rng.integers(1, 9))
    N = int(rng.choice([1, 2, 3, 5, 8, 16, 48, 64]))
    L = int(rng.choice([1, 2, 3, 4, 8, 8, 11]))
    shapes = [(int(rng.integers(0, max(2, min(4 * N + 9, 100000 // k)))), k)
              for k in [int(rng.choice([1, 2, 3, 8, 24, 100, 1000, 4096])) for _ in range(P)]]
    grads = host_grads(shapes, L, seed=case)
    mode = int(rng.integers(0, 3))
    launch = [tide.Launch(), tide.budgeted(place_blocks=int(rng.integers(1, 5)), max_launch_us=1),
              tide.Launch(flags=tide.FLAG_SCALAR_PATH)][mode]
    rr = None
    if N > 1 and rng.random() < 0.4:
        a = int(rng.integers(0, N))
        rr = (a, int(rng.integers(a, N + 1)))
    goff = [[int(rng.choice([0, 0, 1, 2, 8])) for _ in shapes] for _ in range(L)]
    engine = str(rng.choice(["kernel", "kernel", "runtime", "sdma"]))
    say("stage fuzz %d: N=%d L=%d shapes=%s mode=%d ranks=%s %s" % (case, N, L, shapes, mode,
                                                                    rr, engine))
    run_stage(tide, orc, shapes, N, L, grads, grad_offs=goff, slot_off=int(rng.choice([0, 1, 2])),
              engine=engine, launch=launch, rank_range=rr)


def test_stage_then_reduce_by_rank_range(tide, orc):
    """Stage ranks [a, b), reduce ranks [a, b), next range: the whole output."""
    shapes, N, L = [(300, 1000), (17, 4096), (1, 1), (5000, 64), (9, 7)], 16, 4
    grads = host_grads(shapes, L, seed=9)
    plan = tide.plan_create(shapes, N, L)
    S = plan.S
    g_dev = [[to_dev_bf16(grads[c][p], (t, k)) for p, (t, k) in enumerate(shapes)]
             for c in range(L)]
    _, slots = _sentinel_slots(L, N * S, 0)
    out = torch.full((N * S,), float(SENTINEL_F32), dtype=torch.float32, device=dev())
    tab = tide.slot_grads_table(plan, slots)
    for a, b in [(0, 3), (3, 4), (4, 11), (11, 16)]:
        tide.stage_grads_bf16(plan, g_dev, slots, launch=tide.Launch(rank_begin=a, rank_end=b))
        tide.reduce_scatter_bf16_fp32(plan, tab, out, launch=tide.Launch(rank_begin=a, rank_end=b))
    torch.cuda.synchronize()
    same_f32(bits_of(out), orc.reduce_scatter(shapes, N, L, grads), "pipelined slot reduce")


def test_slot_release_ordering(tide, orc):
    """Two streams, the order of the pages' Slot-Reuse mode. The all-gather
    stream places layer i's shards out of the slots and records `vacated`;
    the reduce stream waits for it, stages the gradients into the slots, lets
    go of the gradient tensors at once (their memory is handed out again and
    overwritten on the current stream), reduces from the slots and records
    `read`; the all-gather stream waits for `read` before it refills the
    slots with layer i-1's shards and places them. Every result must equal the
    oracle's."""
    shapes, N, L = [(4096, 1024), (77, 4096), (3, 1), (1000, 512)], 8, 4
    plan = tide.plan_create(shapes, N, L)
    S = plan.S
    n = N * S
    grads_h = host_grads(shapes, L, seed=21)
    stage_a = [host_rank_major_bits(n, seed=30 + c) for c in range(L)]
    stage_b = [host_rank_major_bits(n, seed=40 + c) for c in range(L)]
    a_dev = [to_dev_bf16(x, (n,)) for x in stage_a]
    b_dev = [to_dev_bf16(x, (n,)) for x in stage_b]
    slots = [torch.empty(n, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    params_a = [[torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in shapes]
                for _ in range(L)]
    params_b = [[torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in shapes]
                for _ in range(L)]
    out = torch.empty(n, dtype=torch.float32, device=dev())
    s_ag = torch.cuda.Stream()
    s_rs = torch.cuda.Stream()
    vacated = torch.cuda.Event()
    read = torch.cuda.Event()
    s_ag.wait_stream(torch.cuda.current_stream())
    s_rs.wait_stream(torch.cuda.current_stream())
    g_dev = [[to_dev_bf16(grads_h[c][p], (t, k)) for p, (t, k) in enumerate(shapes)]
             for c in range(L)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s_ag):
        for c in range(L):
            slots[c].copy_(a_dev[c])                  # the all-gather lands in the slot
            tide.allgather_place(plan, slots[c], params_a[c], stream=s_ag)
        vacated.record(s_ag)
    with torch.cuda.stream(s_rs):
        s_rs.wait_event(vacated)
        tide.stage_grads_bf16(plan, g_dev, slots, stream=s_rs)
    del g_dev                                         # released right after the staging call
    junk = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()).fill_(-3.0)
            for t, k in shapes for _ in range(L)]
    with torch.cuda.stream(s_rs):
        tide.reduce_scatter_bf16_fp32(plan, tide.slot_grads_table(plan, slots), out, stream=s_rs)
        read.record(s_rs)
    with torch.cuda.stream(s_ag):
        s_ag.wait_event(read)
        for c in range(L):
            slots[c].copy_(b_dev[c])                  # the next all-gather reuses the slot
            tide.allgather_place(plan, slots[c], params_b[c], stream=s_ag)
    torch.cuda.synchronize()
    del junk
    same_f32(bits_of(out), orc.reduce_scatter(shapes, N, L, grads_h), "reduce from slots")
    for c in range(L):
        wa = orc.allgather_place(shapes, N, stage_a[c])
        wb = orc.allgather_place(shapes, N, stage_b[c])
        for p in range(len(shapes)):
            same_u16(bits_of(params_a[c][p]), wa[p], "layer i placement c=%d p=%d" % (c, p))
            same_u16(bits_of(params_b[c][p]), wb[p], "layer i-1 placement c=%d p=%d" % (c, p))


BIG = ["llama70b_layer", "qwen3_moe_layer", "padding_stress", "wan22_dit_block"]


@pytest.mark.parametrize("name", BIG)
def test_stage_full_size(tide, orc, name):
    cfg = CONFIGS[name]
    say("%s: slot-reuse full size" % name)
    grads = device_grads(cfg.shapes, cfg.L, seed=cfg.seed, sigma=cfg.sigma,
                         outlier_frac=cfg.outlier_frac)
    plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
    S = plan.S
    n = cfg.N * S
    slots = [torch.empty(n, dtype=torch.bfloat16, device=dev()) for _ in range(cfg.L)]
    g_tab = tide.grads_table(plan, grads)
    tide.stage_grads_bf16(plan, g_tab, slots)
    torch.cuda.synchronize()
    lay = orc.layout(cfg.shapes, cfg.N)
    for c in range(cfg.L):
        for p, (t, k) in enumerate(cfg.shapes):
            at = cfg.N * int(lay["o"][p])
            assert torch.equal(slots[c][at:at + t * k].view(torch.int16),
                               grads[c][p].reshape(-1).view(torch.int16)), (name, c, p)
    say("%s: staged slots equal the gradients; reducing from the slots" % name)
    out = torch.empty(n, dtype=torch.float32, device=dev())
    out.view(torch.int32).fill_(0x7FC0DEAD)
    tide.reduce_scatter_bf16_fp32(plan, tide.slot_grads_table(plan, slots), out)
    torch.cuda.synchronize()
    ref = torch.empty_like(out)
    tide.reduce_scatter_bf16_fp32(plan, g_tab, ref)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), name
    from test_gpu_fullsize import _check_pieces, _sample_pieces
    _check_pieces(orc, cfg, grads, out, S, _sample_pieces(cfg, np.random.default_rng(7)))
    if name == "wan22_dit_block":
        say("%s: budgeted, runtime-copy and DMA-engine staging" % name)
        for kw in ({"launch": tide.budgeted()}, {"engine": "runtime"}, {"engine": "sdma"}):
            s2 = [torch.zeros(n, dtype=torch.bfloat16, device=dev()) for _ in range(cfg.L)]
            tide.stage_grads_bf16(plan, g_tab, s2, **kw)
            torch.cuda.synchronize()
            for c in range(cfg.L):
                for p, (t, k) in enumerate(cfg.shapes):
                    at = cfg.N * int(lay["o"][p])
                    assert torch.equal(s2[c][at:at + t * k].view(torch.int16),
                                       grads[c][p].reshape(-1).view(torch.int16)), (kw, c, p)
            del s2
    del grads, slots, out, ref, g_tab
    gc.collect()
    torch.cuda.empty_cache()
    say("%s: ok" % name)
