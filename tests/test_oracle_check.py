"""oracle/check.py's whole-output comparison, on the host (no GPU): the
benchmark's "whole output bit-exact" and the full-size GPU tests rest on it,
so it must pass a correct output and catch, and place, a single wrong bit in
any rank range of the reduce-scatter or in any parameter of the placement.
The "GPU" output here is the oracle's own, as torch CPU tensors."""
import numpy as np
import pytest
import torch

from oracle import check
from workloads import host_grads, host_rank_major_bits
from workloads.configs import Config, padding_stress_shapes


def _case(orc, N=20, L=3):
    shapes = padding_stress_shapes(9, count=10, max_rows=70, ks=(1, 3, 16)) + [(1, 4), (0, 3)]
    cfg = Config("check", tuple(shapes), N=N, L=L, sigma=1.0)
    lay = orc.layout(shapes, N)
    S = int(lay["S"])
    grads = host_grads(shapes, L, seed=17)
    g_t = [[torch.from_numpy(grads[c][p].view(np.int16)).view(torch.bfloat16).view(t, k)
            for p, (t, k) in enumerate(shapes)] for c in range(L)]
    out = torch.from_numpy(orc.reduce_scatter(shapes, N, L, grads).reshape(-1).copy())
    bits = host_rank_major_bits(N * S, seed=5)
    shards = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    placed = orc.allgather_place(shapes, N, bits)
    params = [torch.from_numpy(w.view(np.int16).copy()).view(torch.bfloat16).view(t, k)
              for w, (t, k) in zip(placed, shapes)]
    return cfg, lay, S, g_t, out, shards, params


def test_correct_output_passes(orc):
    cfg, _, S, g, out, sh, params = _case(orc)
    r = check.whole_output(orc, cfg, S, g, out, sh, params)
    assert r["reduce_scatter_bit_exact"] and r["placement_bit_exact"], r
    assert r["first_mismatch"] is None
    # every rank was covered: bytes = 2 L valid + 4 N S + 4 valid
    valid = sum(t * k for t, k in cfg.shapes)
    assert r["bytes"] == 2 * cfg.L * valid + 4 * cfg.N * S + 4 * valid


@pytest.mark.parametrize("rank", [0, 9, 19])
def test_one_wrong_bit_in_the_reduce_scatter_is_caught(orc, rank):
    cfg, _, S, g, out, sh, params = _case(orc)
    bad = out.clone()
    i = rank * S + S // 2
    bad.view(torch.int32)[i] ^= 1            # the lowest mantissa bit of one element
    r = check.whole_output(orc, cfg, S, g, bad, sh, params)
    assert not r["reduce_scatter_bit_exact"] and r["placement_bit_exact"]
    first, last = [int(x) for x in r["first_mismatch"].split("ranks ")[1].split("-")]
    assert first <= rank <= last, r["first_mismatch"]


def test_one_wrong_element_in_the_placement_is_caught(orc):
    cfg, lay, S, g, out, sh, params = _case(orc)
    p = max(range(len(cfg.shapes)), key=lambda q: cfg.shapes[q][0] * cfg.shapes[q][1])
    bad = [x.clone() for x in params]
    flat = bad[p].view(-1).view(torch.int16)
    flat[flat.numel() - 1] ^= 1              # the last element, held by the last rank that holds p
    r = check.whole_output(orc, cfg, S, g, out, sh, bad)
    assert r["reduce_scatter_bit_exact"] and not r["placement_bit_exact"]
    assert r["first_mismatch"].startswith("placement, parameter %d," % p), r["first_mismatch"]


def test_padding_must_be_positive_zero(orc):
    """A -0.0 in a padded row differs from the oracle's +0.0 only in the sign
    bit: the comparison is by bits, not by value."""
    cfg, lay, S, g, out, sh, params = _case(orc)
    N = cfg.N
    p = next(q for q, (t, k) in enumerate(cfg.shapes)
             if int(lay["R"][q]) * N > t and k > 0)      # a parameter with padded rows
    t, k = cfg.shapes[p]
    R, o = int(lay["R"][p]), int(lay["o"][p])
    r_last = N - 1                                        # the last rank holds padding of p
    j = (R - 1) * k                                       # its last row's first element
    assert r_last * R + R - 1 >= t
    bad = out.clone()
    bad[r_last * S + o + j] = -0.0
    r = check.whole_output(orc, cfg, S, g, bad, sh, params)
    assert not r["reduce_scatter_bit_exact"]
