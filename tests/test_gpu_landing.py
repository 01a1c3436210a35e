"""Level-2 landing sum on the GPU, through the C ABI, against the oracle; and
the two-level reduce-scatter (level 1 per source node, Latin-square routing,
landing) against the oracle's and against a flat reduce-scatter."""
import numpy as np
import pytest
import torch

from gpu_util import bits_of, dev, same_f32, say, to_dev_bf16
from workloads import fp32_to_bf16_bits, host_grads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def f32_dev(a, off=0):
    buf = torch.empty(a.size + off + 4, dtype=torch.float32, device=dev())
    t = buf[off:off + a.size]
    t.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev()))
    return t


CASES = [(4, 4, 37), (8, 8, 4096), (8, 5, 10000), (8, 1, 333), (3, 2, 2), (8, 8, 7),
         (16, 11, 20000), (2, 2, 1), (8, 3, 123457)]


@pytest.mark.parametrize("L,M,S", CASES)
def test_landing_vs_oracle(tide, orc, L, M, S):
    rng = np.random.default_rng(L * 1000 + M * 10 + S % 97)
    C = -(-S // L)
    inb = [rng.standard_normal(L * L * C).astype(np.float32) for _ in range(L)]
    init = [rng.standard_normal(S).astype(np.float32) for _ in range(L)]
    for accumulate in (False, True):
        for launch_kind in ("full", "budgeted", "scalar"):
            launch = {"full": tide.Launch(), "budgeted": tide.budgeted(max_launch_us=5),
                      "scalar": tide.Launch(flags=tide.FLAG_SCALAR_PATH)}[launch_kind]
            off = (L + M + int(accumulate)) % 3
            say("landing L=%d M=%d S=%d acc=%s %s off=%d" % (L, M, S, accumulate, launch_kind, off))
            d_in = [f32_dev(a, off) for a in inb]
            d_sh = [f32_dev(a, (off + 1) % 3) for a in init]
            tide.landing_sum_fp32(L, M, S, d_in, d_sh, accumulate=accumulate, launch=launch)
            torch.cuda.synchronize()
            want = orc.landing_sum(L, M, S, inb, shards=[a.copy() for a in init],
                                   accumulate=accumulate)
            for b in range(L):
                same_f32(bits_of(d_sh[b]), want[b], "shard %d" % b)


def test_landing_rejects(tide):
    from mixed_precision_rs_amd import TideError
    with pytest.raises(TideError):
        tide.landing_sum_fp32(4, 5, 10, [0x7f0000000000] * 4, [0x7f0010000000] * 4, stream=0)
    with pytest.raises(TideError):
        tide.landing_sum_fp32(65, 1, 10, [0x7f0000000000] * 65, [0x7f0010000000] * 65, stream=0)
    ib = [0x7f0000000000 + i * 0x100000 for i in range(2)]
    with pytest.raises(TideError):          # shards overlap each other
        tide.landing_sum_fp32(2, 2, 10, ib, [0x7f0010000000, 0x7f0010000004], stream=0)
    with pytest.raises(TideError):          # shard inside an inbox
        tide.landing_sum_fp32(2, 2, 10, ib, [ib[0] + 8, 0x7f0010000000], stream=0)
    with pytest.raises(TideError):          # misaligned
        tide.landing_sum_fp32(2, 2, 10, ib, [0x7f0010000002, 0x7f0011000000], stream=0)


def gpu_two_level(tide, shapes, M, L, grads_by_node_dev, dst):
    """Level 1 with the reduce kernel on each source node (ranks of node dst),
    the slices routed to dst's inboxes by the Latin square, then landing."""
    N = M * L
    plan = tide.plan_create(shapes, N, L)
    S = plan.S
    C = -(-S // L)
    inboxes = [torch.zeros(L * L * C, dtype=torch.float32, device=dev()) for _ in range(L)]
    part = torch.empty(N * S, dtype=torch.float32, device=dev())
    for src in range(M):
        tide.reduce_scatter_bf16_fp32(plan, grads_by_node_dev[src], part,
                                      launch=tide.Launch(rank_begin=dst * L, rank_end=dst * L + L))
        p2 = part.view(N, S)[dst * L: dst * L + L]
        c, slice_of, gpu_of = tide.latin_square(M, L, dst, src)
        for j in range(L):                      # source GPU j sends slice (j + c) mod L on rail j
            s = slice_of[j]
            g = gpu_of[s]
            n = max(0, min(C, S - s * C))
            for b in range(L):
                inboxes[g][(s * L + b) * C:(s * L + b) * C + n].copy_(p2[b, s * C: s * C + n])
    shards = [torch.empty(S, dtype=torch.float32, device=dev()) for _ in range(L)]
    tide.landing_sum_fp32(L, M, S, inboxes, shards)
    torch.cuda.synchronize()
    return shards, S


def test_two_level_pipeline(tide, orc):
    import pins_landing
    for shapes, M, L, integer in (([(40, 3), (7, 1), (65, 2)], 3, 4, False),
                                  ([(512, 64), (30, 1), (100, 130)], 4, 8, False),
                                  ([(512, 64), (30, 1), (100, 130)], 4, 8, True)):
        rng = np.random.default_rng(M * L)
        N = M * L
        if integer:
            gbn = [[[fp32_to_bf16_bits(rng.integers(-64, 65, t * k).astype(np.float32))
                     for (t, k) in shapes] for _ in range(L)] for _ in range(M)]
        else:
            gbn = [host_grads(shapes, L, seed=100 + n) for n in range(M)]
        gdev = [[[to_dev_bf16(gbn[n][c][p], (t, k)) for p, (t, k) in enumerate(shapes)]
                 for c in range(L)] for n in range(M)]
        for dst in range(M):
            say("two-level M=%d L=%d dst=%d integer=%s" % (M, L, dst, integer))
            shards, S = gpu_two_level(tide, shapes, M, L, gdev, dst)
            want = pins_landing.two_level(orc, shapes, M, L, gbn, dst)
            for b in range(L):
                same_f32(bits_of(shards[b]), want[b], "dst %d shard %d" % (dst, b))
            if integer:
                flat = orc.reduce_scatter(shapes, N, M * L, [row for node in gbn for row in node])
                for b in range(L):
                    same_f32(bits_of(shards[b]), flat[dst * L + b], "flat dst %d shard %d" % (dst, b))


def test_landing_full_size(tide, orc):
    """The landing sum at the size the benchmark times: L = M = 8 partials of
    the Llama-3.1-70B layer group's shard (S = 13,369,600), full grid and
    budgeted, every element against the oracle."""
    from workloads.configs import CONFIGS
    cfg = CONFIGS["llama70b_layer"]
    L = M = cfg.L
    S = int(orc.layout(cfg.shapes, cfg.N)["S"])
    C = -(-S // L)
    g = torch.Generator(device=dev())
    g.manual_seed(11)
    inb = [torch.randn(L * L * C, generator=g, device=dev()) for _ in range(L)]
    h_in = [t.cpu().numpy() for t in inb]
    say("landing full size: oracle over %d x %d floats" % (L, L * L * C))
    want = orc.landing_sum(L, M, S, h_in)
    for kind, launch in (("full", tide.Launch()), ("budgeted", tide.budgeted())):
        shards = [torch.empty(S, dtype=torch.float32, device=dev()) for _ in range(L)]
        tide.landing_sum_fp32(L, M, S, inb, shards, launch=launch)
        torch.cuda.synchronize()
        for b in range(L):
            same_f32(bits_of(shards[b]), want[b], "%s shard %d" % (kind, b))
        del shards
