"""The four large workloads at full size, in the launch configuration the
benchmark times (full grid), plus the CU-budgeted mode on the DiT block.

Checks, per workload:
  * the whole output: every shard of the reduce-scatter (distinct
    contributors, so a fold-order mistake would show) and every parameter the
    placement wrote, against the oracle on the same bits, streamed by rank
    range (oracle/check.py);
  * sampled pieces: for ranks {0, 1, N/2, N-1, two random} and a sample of
    parameters, the oracle recomputes the piece from the same input rows
    (fetched from the GPU at the oracle's own piece addresses) and the GPU's
    piece must match bit for bit;
  * every padded row of every shard is +0.0f (oracle layout, torch compare);
  * identical contributors: with all L gradient sets the same tensors, every
    output element equals L * f32(g) exactly in any summation order, so the
    WHOLE output is checked against a torch expression (pad + view) built from
    the oracle's layout;
  * placement, kernel, runtime-copy and DMA engines: every parameter equals
    the split-with-sizes view of the rank-major shards at the oracle's offsets.
"""
import gc

import numpy as np
import pytest
import torch

from gpu_util import bits_of, dev, same_f32, same_u16, say
from workloads import device_grads, device_rank_major_bits
from workloads.configs import CONFIGS

pytestmark = pytest.mark.gpu

BIG = ["llama70b_layer", "qwen3_moe_layer", "padding_stress", "wan22_dit_block"]


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _sample_pieces(cfg, rng):
    N, P = cfg.N, len(cfg.shapes)
    ranks = sorted({0, 1, N // 2, N - 1, int(rng.integers(0, N)), int(rng.integers(0, N))})
    if P <= 16:
        params = list(range(P))
    else:
        params = sorted(set([0, 1, 2, P - 7, P - 6, P - 5, P - 4, P - 3, P - 2, P - 1] +
                            [int(x) for x in rng.integers(0, P, 12)]))
    pieces = [(r, p) for r in ranks for p in params]
    # bound the host traffic of the biggest workloads
    big = [(r, p) for r, p in pieces if cfg.shapes[p][1] * -(-cfg.shapes[p][0] // N) > 1 << 20]
    if len(big) > 24:
        keep = set(map(tuple, rng.permutation(np.array(big))[:24].tolist()))
        pieces = [(r, p) for r, p in pieces if (r, p) not in big or (r, p) in keep]
    return pieces


def _check_pieces(orc, cfg, grads, out, S, pieces):
    lay = orc.layout(cfg.shapes, cfg.N)
    for (r, p) in pieces:
        first, n = orc.piece_rows(cfg.shapes, cfg.N, r, p)
        rows = [bits_of(grads[c][p][first:first + n]) for c in range(cfg.L)]
        want = orc.reduce_piece(cfg.shapes, cfg.N, cfg.L, r, p, rows)
        o, s = int(lay["o"][p]), int(lay["s"][p])
        got = bits_of(out[r * S + o: r * S + o + s])
        same_f32(got, want, "%s piece (r=%d, p=%d)" % (cfg.name, r, p))


def _check_padding(orc, cfg, out, S):
    lay = orc.layout(cfg.shapes, cfg.N)
    o2 = out.view(cfg.N, S)
    for p, (t, k) in enumerate(cfg.shapes):
        R, o, s = int(lay["R"][p]), int(lay["o"][p]), int(lay["s"][p])
        if R * cfg.N == t:
            continue
        pad = torch.zeros(cfg.N * R * k, dtype=torch.bool, device=dev())
        pad[t * k:] = True
        region = o2[:, o:o + s].reshape(-1)[pad]
        assert torch.all(region.view(torch.int32) == 0), "%s param %d: padding not +0" % (cfg.name, p)


def _check_identical(tide, orc, cfg, grads0):
    """All L contributors = grads0: out must be exactly pad(L * f32(g))."""
    plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
    S = plan.S
    out = torch.empty(cfg.N * S, dtype=torch.float32, device=dev())
    tide.reduce_scatter_bf16_fp32(plan, [grads0] * cfg.L, out)
    lay = orc.layout(cfg.shapes, cfg.N)
    o2 = out.view(cfg.N, S)
    for p, (t, k) in enumerate(cfg.shapes):
        R, o, s = int(lay["R"][p]), int(lay["o"][p]), int(lay["s"][p])
        want = torch.zeros((cfg.N * R, k), dtype=torch.float32, device=dev())
        want[:t] = grads0[p].float() * float(cfg.L)
        got = o2[:, o:o + s].reshape(cfg.N * R, k)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), \
            "%s param %d: identical-contributor sum differs" % (cfg.name, p)
    del out
    _free()


def _check_place(tide, orc, cfg, engine, launch=None):
    plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
    S = plan.S
    sh = device_rank_major_bits(cfg.N * S, seed=5)
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in cfg.shapes]
    for x in params:
        x.view(torch.int16).fill_(-4369)   # 0xEEEF sentinel
    tide.allgather_place(plan, sh, params, engine=engine, launch=launch)
    torch.cuda.synchronize()
    lay = orc.layout(cfg.shapes, cfg.N)
    v = sh.view(cfg.N, S)
    for p, (t, k) in enumerate(cfg.shapes):
        o, s = int(lay["o"][p]), int(lay["s"][p])
        want = v[:, o:o + s].reshape(-1)[:t * k]
        assert torch.equal(params[p].reshape(-1).view(torch.int16), want.view(torch.int16)), \
            "%s: placement (%s) of param %d differs" % (cfg.name, engine, p)
    # a sampled parameter also through the oracle's own placement
    p = int(np.argmax([t * k for t, k in cfg.shapes]))
    sub = [cfg.shapes[p]]
    o, s = int(lay["o"][p]), int(lay["s"][p])
    sub_shards = bits_of(v[:, o:o + s].contiguous())
    want = orc.allgather_place(sub, cfg.N, sub_shards)[0]
    same_u16(bits_of(params[p]), want, "%s placement (%s) param %d vs oracle" % (cfg.name, engine, p))
    del sh, params
    _free()


@pytest.mark.parametrize("name", BIG)
def test_full_size(tide, orc, name):
    cfg = CONFIGS[name]
    rng = np.random.default_rng(42)
    say("%s: generating %d x %d params" % (name, cfg.L, len(cfg.shapes)))
    grads = device_grads(cfg.shapes, cfg.L, seed=cfg.seed, sigma=cfg.sigma,
                         outlier_frac=cfg.outlier_frac)
    plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
    S = plan.S
    out = torch.empty(cfg.N * S, dtype=torch.float32, device=dev())
    out.view(torch.int32).fill_(0x7FC0DEAD)
    tide.reduce_scatter_bf16_fp32(plan, grads, out)
    torch.cuda.synchronize()
    say("%s: reduce-scatter done; whole output and placement vs the oracle" % name)
    from oracle import check
    sh = device_rank_major_bits(cfg.N * S, seed=6)
    params = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in cfg.shapes]
    tide.allgather_place(plan, sh, params)
    torch.cuda.synchronize()
    chk = check.whole_output(orc, cfg, S, grads, out, sh, params)
    assert chk["reduce_scatter_bit_exact"] and chk["placement_bit_exact"], chk["first_mismatch"]
    del sh, params
    say("%s: checking sampled pieces" % name)
    _check_pieces(orc, cfg, grads, out, S, _sample_pieces(cfg, rng))
    say("%s: checking padding" % name)
    _check_padding(orc, cfg, out, S)
    if name == "wan22_dit_block":
        say("%s: budgeted 16+4 mode vs full grid" % name)
        out2 = torch.empty_like(out)
        tide.reduce_scatter_bf16_fp32(plan, grads, out2, launch=tide.budgeted())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
        del out2
    grads0 = grads[0]
    del out, grads
    _free()
    say("%s: identical-contributor whole-output check" % name)
    _check_identical(tide, orc, cfg, grads0)
    del grads0
    _free()
    for eng in ("kernel", "runtime", "sdma"):
        say("%s: placement %s" % (name, eng))
        _check_place(tide, orc, cfg, eng)
    if name == "wan22_dit_block":
        _check_place(tide, orc, cfg, "kernel", launch=tide.budgeted())
    say("%s: ok" % name)
