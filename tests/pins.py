"""Pins: checks that tie the CPU oracle to something other than itself.

Each pin takes an oracle handle and raises AssertionError when the oracle
disagrees with the pages, with mathematics, or with a library routine that
defines the operation. The same pins run against deliberately broken copies
of the oracle (test_oracle_mutants.py) to show that each plausible mistake is
caught by at least one of them.

Sources the pins use, none of which is the oracle's code:
  * the worked example on page 1 ("What problem is it actually solving?"),
    stored in tests/golden/worked_example.json;
  * torch._chunk_cat, the routine FSDP2 packs reduce-scatter inputs with
    (slice along dim 0 into N chunks, zero-pad each to the first chunk's
    rows, concatenate rank-major, optionally into an fp32 `out`): the stock
    pack page 1 describes (slicing, zero padding and the fp32 upcast);
  * torch.split_with_sizes, FSDP2's all-gather copy-out (page 1; page 3
    Table 7: its copy-out rows add split_with_sizes_copy);
  * closed forms: sums that are exact in binary32 regardless of order;
  * the error bound of recursive binary32 summation against the exact sum;
  * hand-derived results of crafted inputs whose value depends on the order.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from workloads import fp32_to_bf16_bits, host_grads, host_special_grads, host_rank_major_bits
from workloads.configs import padding_stress_shapes

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

U24 = 2.0 ** -24


def _f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _widen(bits):
    """bf16 bits -> float32 values (for building expected values in tests)."""
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_tensor(bits, t, k):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy()
                            ).view(torch.bfloat16).reshape(t, k)


def _same_bits(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.dtype == np.float32:
        # NaN compared as a class (payloads may differ), everything else bitwise.
        an, bn = np.isnan(a), np.isnan(b)
        assert np.array_equal(an, bn), "NaN positions differ"
        ab, bb = _f32_bits(a), _f32_bits(b)
        bad = np.flatnonzero((ab != bb) & ~an)
        assert bad.size == 0, "first mismatch at %d: %r vs %r" % (
            bad[0], a.reshape(-1)[bad[0]], b.reshape(-1)[bad[0]])
    else:
        bad = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
        assert bad.size == 0, "first mismatch at %d" % bad[0]


# Small groups that exercise the layout's corner cases: T_p < N (ranks holding
# only padding), T_p a multiple of N (no padding), K_p = 1 (1-D tensors),
# odd sizes, and a parameter with a single row.
SMALL_GROUPS = [
    ([(8, 4), (4, 4), (12, 4)], 4),                 # the worked example's group
    ([(5, 3), (1, 7), (9, 1), (16, 2)], 4),
    ([(3, 5)], 8),                                   # T < N
    ([(7, 1), (7, 2), (7, 3)], 3),
    ([(13, 6), (2, 1), (40, 3), (1, 1), (6, 9)], 6),
    ([(11, 11)], 1),                                 # a single rank
]


def pin_worked_example(orc):
    """Page 1's worked example: GPU 1's piece of the 2nd parameter starts at
    8 MB in the rank-major buffer and at 9 MB in parameter-major order."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    N = g["N"]
    pieces = g["pieces_per_rank"]
    for K in (1, 4):                       # K=1: the example's MB units; K=4: config 1
        shapes = [(N * n, K) for n in pieces]
        lay = orc.layout(shapes, N)
        assert lay["S"] == g["per_rank_total"] * K
        rm, pm, pmg = orc.piece_start(shapes, N, g["rank"], g["param"])
        assert rm == g["rank_major_start"] * K, rm
        assert pmg == g["param_major_start"] * K, pmg
        # The same fact through data movement: tag each element with a unique
        # small integer, reduce with L = 1 and find where the tagged piece lands.
        tags, base = [], 0
        for (t, k) in shapes:
            tags.append(fp32_to_bf16_bits(np.arange(base, base + t * k, dtype=np.float32)))
            base += t * k
        out = orc.reduce_scatter(shapes, N, 1, [tags]).reshape(-1)
        r, p = g["rank"], g["param"]
        first_row = r * pieces[p]                  # rank r holds rows r*R_p.. of param p
        first_tag = float(sum(t * k for t, k in shapes[:p]) + first_row * K)
        assert out[g["rank_major_start"] * K] == first_tag
        # Placement: gather the rank-major buffer into parameters laid end to end.
        placed = orc.allgather_place(shapes, N, (out.view(np.uint32) >> 16).astype(np.uint16))
        group = np.concatenate(placed)
        assert _widen(group[g["param_major_start"] * K]) == first_tag


def _chunk_cat_fp32(bits_per_param, shapes, N):
    ts = [_bf16_tensor(b, t, k) for b, (t, k) in zip(bits_per_param, shapes)]
    S = sum(-(-t // N) * k for t, k in shapes)
    out = torch.empty((N, S), dtype=torch.float32)
    torch._chunk_cat(ts, dim=0, num_chunks=N, out=out)
    return out


def pin_chunk_cat_single_contributor(orc):
    """L = 1 is FSDP2's stock pack: torch._chunk_cat into fp32."""
    for i, (shapes, N) in enumerate(SMALL_GROUPS):
        grads = host_grads(shapes, 1, seed=100 + i)
        want = _chunk_cat_fp32(grads[0], shapes, N).numpy()
        got = orc.reduce_scatter(shapes, N, 1, grads)
        _same_bits(got, want)


def pin_chunk_cat_fold(orc):
    """General L: pack every contributor with torch._chunk_cat into fp32 and
    add the packed buffers elementwise in contributor order (torch float32
    adds are binary32 round-to-nearest-even)."""
    cases = SMALL_GROUPS + [(padding_stress_shapes(7, count=12, max_rows=60, ks=(1, 3, 8, 16)), 5)]
    for i, (shapes, N) in enumerate(cases):
        for L in (2, 3, 8):
            grads = host_grads(shapes, L, seed=200 + 10 * i + L)
            acc = _chunk_cat_fp32(grads[0], shapes, N)
            for c in range(1, L):
                acc = acc + _chunk_cat_fp32(grads[c], shapes, N)
            got = orc.reduce_scatter(shapes, N, L, grads)
            _same_bits(got, acc.numpy())


def pin_error_bound(orc):
    """Recursive binary32 summation of L terms is within (L-1) * 2^-24 *
    sum|x_c| of the exact sum (plus subnormal spacing slack). Checked against
    the exact rational sum for random and adversarial finite inputs."""
    shapes, N = [(9, 5), (4, 3), (17, 1)], 4
    for L in (2, 5, 8):
        for gen in ("normal", "special"):
            if gen == "normal":
                grads = host_grads(shapes, L, seed=300 + L, sigma=1.0)
            else:
                grads = host_special_grads(shapes, L, seed=300 + L, allow_inf=False)
            out = orc.reduce_scatter(shapes, N, L, grads)
            lay = orc.layout(shapes, N)
            for p, (t, k) in enumerate(shapes):
                vals = [_widen(grads[c][p]).astype(np.float64) for c in range(L)]
                for e in range(t * k):
                    row, col = divmod(e, k)
                    r, i = divmod(row, int(lay["R"][p]))
                    got = float(out[r, lay["o"][p] + i * k + col])
                    xs = [vals[c][e] for c in range(L)]
                    exact = sum((Fraction(x) for x in xs), Fraction(0))
                    mag = sum(abs(x) for x in xs)
                    if math.isinf(got):
                        # overflow only when the exact sum is at binary32's edge
                        assert abs(exact) > Fraction(3.4e38) or mag > 3.4e38
                        continue
                    err = abs(Fraction(got) - exact)
                    bound = Fraction((L - 1) * U24 * mag) + Fraction(L * 2.0 ** -149)
                    assert err <= bound, (p, e, got, float(exact))


def pin_closed_forms(orc):
    """Results fixed by mathematics alone, in any summation order."""
    shapes, N = [(6, 4), (3, 1), (10, 2)], 3
    P = len(shapes)
    lay = orc.layout(shapes, N)
    rng = np.random.default_rng(5)

    def value_at(out, p, e):
        k = shapes[p][1]
        row, col = divmod(e, k)
        r, i = divmod(row, int(lay["R"][p]))
        return out[r, lay["o"][p] + i * k + col]

    for L in (1, 2, 4, 8):
        # (a) identical contributors: every partial sum j*g needs <= 11
        # significant bits, so the result is exactly L*g.
        g = [fp32_to_bf16_bits(rng.standard_normal(t * k).astype(np.float32) * 3.0)
             for t, k in shapes]
        out = orc.reduce_scatter(shapes, N, L, [g] * L)
        for p in range(P):
            for e in range(shapes[p][0] * shapes[p][1]):
                want = np.float32(L * float(_widen(g[p][e])))
                assert _f32_bits(value_at(out, p, e)) == _f32_bits(want)
        # (b) small integers: all partial sums are exact integers.
        ints = [[rng.integers(-256, 257, t * k) for t, k in shapes] for _ in range(L)]
        gi = [[fp32_to_bf16_bits(a.astype(np.float32)) for a in row] for row in ints]
        out = orc.reduce_scatter(shapes, N, L, gi)
        for p in range(P):
            for e in range(shapes[p][0] * shapes[p][1]):
                assert value_at(out, p, e) == float(sum(int(ints[c][p][e]) for c in range(L)))
        # (c) one non-zero contributor: the result is that contributor's value.
        for who in range(L):
            gz = [[np.zeros(t * k, np.uint16) for t, k in shapes] for _ in range(L)]
            gz[who] = [fp32_to_bf16_bits(rng.standard_normal(t * k).astype(np.float32) + 4.0)
                       for t, k in shapes]
            out = orc.reduce_scatter(shapes, N, L, gz)
            for p in range(P):
                for e in range(shapes[p][0] * shapes[p][1]):
                    assert _f32_bits(value_at(out, p, e)) == _f32_bits(_widen(gz[who][p][e]))
    # (d) signed zeros: the fold starts from contributor 0's value, so an
    # all -0.0 input sums to -0.0; any +0.0 term makes it +0.0 (IEEE RNE).
    one = [(1, 1)]
    for L in (1, 2, 8):
        out = orc.reduce_scatter(one, 1, L, [[np.array([0x8000], np.uint16)]] * L)
        assert _f32_bits(out[0, 0]) == 0x80000000
    if True:
        L = 4
        mixed = [[np.array([0x8000], np.uint16)]] * 3 + [[np.array([0x0000], np.uint16)]]
        out = orc.reduce_scatter(one, 1, L, mixed)
        assert _f32_bits(out[0, 0]) == 0x00000000


def pin_contributor_order(orc):
    """Crafted inputs whose binary32 sum depends on the order, with results
    derived by hand for a left fold over c = 0, 1, ..., L-1.

    [1, 2^-24 x 7]: each 1 + 2^-24 is a tie and rounds to even (1.0), so the
    left fold gives exactly 1.0 (a reversed or tree order would not).
    [2^-24 x 7, 1]: the tiny terms add exactly to 7*2^-24 = 3.5*2^-23, and
    1 + 3.5*2^-23 is a tie between 1 + 3*2^-23 and 1 + 4*2^-23 that rounds to
    the even one, 1 + 4*2^-23 = 1 + 2^-21.
    """
    one = [(1, 1)]
    b1 = fp32_to_bf16_bits(np.array([1.0], np.float32))
    tiny = fp32_to_bf16_bits(np.array([2.0 ** -24], np.float32))
    L = 8
    out = orc.reduce_scatter(one, 1, L, [[b1]] + [[tiny]] * 7)
    assert out[0, 0] == np.float32(1.0)
    out = orc.reduce_scatter(one, 1, L, [[tiny]] * 7 + [[b1]])
    assert out[0, 0] == np.float32(1.0 + 2.0 ** -21)


def pin_coverage_and_padding(orc):
    """Every element of [0, S) in every shard is written exactly once, nothing
    in [S, stride) is written, padded rows are +0.0f bit for bit, and every
    true element of every parameter is placed exactly once."""
    for i, (shapes, N) in enumerate(SMALL_GROUPS):
        lay = orc.layout(shapes, N)
        S = lay["S"]
        for stride in (S, S + 3):
            L = 3
            grads = host_special_grads(shapes, L, seed=400 + i)
            out, cnt = orc.reduce_scatter(shapes, N, L, grads, out_stride=stride, count_writes=True)
            assert np.all(cnt[:, :S] == 1)
            assert np.all(cnt[:, S:] == 0)
            assert np.all(np.isnan(out[:, S:]))           # untouched sentinel
            for p, (t, k) in enumerate(shapes):
                R = int(lay["R"][p])
                for r in range(N):
                    for i_ in range(R):
                        if r * R + i_ >= t:
                            seg = out[r, lay["o"][p] + i_ * k: lay["o"][p] + (i_ + 1) * k]
                            assert np.all(_f32_bits(seg) == 0)
            shards = host_rank_major_bits(N * stride, seed=500 + i)
            placed, pc = orc.allgather_place(shapes, N, shards, shard_stride=stride,
                                             count_writes=True)
            for c in pc:
                assert np.all(c == 1)


def pin_split_with_sizes(orc):
    """Placement equals FSDP2's copy-out: split the (N, S) rank-major buffer
    into per-parameter column blocks of s_p, view each as (N * R_p, K_p) and
    keep the first T_p rows."""
    for i, (shapes, N) in enumerate(SMALL_GROUPS):
        S = sum(-(-t // N) * k for t, k in shapes)
        for stride in (S, S + 5):
            shards = host_rank_major_bits(N * stride, seed=600 + i)
            buf = torch.from_numpy(shards.view(np.int16).copy()).view(N, stride)[:, :S]
            sizes = [-(-t // N) * k for t, k in shapes]
            blocks = torch.split_with_sizes(buf, sizes, dim=1)
            placed = orc.allgather_place(shapes, N, shards, shard_stride=stride)
            for (t, k), blk, got in zip(shapes, blocks, placed):
                want = blk.reshape(-1, k)[:t].reshape(-1).numpy().view(np.uint16)
                _same_bits(got, want)


def pin_round_trip(orc):
    """Placing the (bf16-truncated) L = 1 reduce-scatter output restores the
    parameters exactly, for any shard stride."""
    for i, (shapes, N) in enumerate(SMALL_GROUPS):
        params = host_grads(shapes, 1, seed=700 + i)[0]
        S = orc.layout(shapes, N)["S"]
        stride = S + 2
        out = orc.reduce_scatter(shapes, N, 1, [params], out_stride=stride)
        shards = (np.nan_to_num(out, nan=0.0).reshape(-1).view(np.uint32) >> 16).astype(np.uint16)
        placed = orc.allgather_place(shapes, N, shards, shard_stride=stride)
        for a, b in zip(placed, params):
            _same_bits(a, b)


def pin_rank_subset_and_piece(orc):
    """A rank range writes exactly those shards, equal to the full result; the
    piece-at-a-time reduction equals the full reduction piece by piece."""
    shapes, N, L = [(13, 6), (2, 1), (40, 3), (1, 1), (6, 9)], 6, 4
    grads = host_grads(shapes, L, seed=800)
    full = orc.reduce_scatter(shapes, N, L, grads)
    part = orc.reduce_scatter(shapes, N, L, grads, rank_range=(2, 5))
    _same_bits(part[2:5], full[2:5])
    assert np.all(np.isnan(part[:2])) and np.all(np.isnan(part[5:]))
    lay = orc.layout(shapes, N)
    for r in range(N):
        for p, (t, k) in enumerate(shapes):
            first, n = orc.piece_rows(shapes, N, r, p)
            rows = [grads[c][p][first * k:(first + n) * k] for c in range(L)]
            got = orc.reduce_piece(shapes, N, L, r, p, rows)
            _same_bits(got, full[r, lay["o"][p]: lay["o"][p] + lay["s"][p]])


ALL_PINS = [
    pin_worked_example,
    pin_chunk_cat_single_contributor,
    pin_chunk_cat_fold,
    pin_error_bound,
    pin_closed_forms,
    pin_contributor_order,
    pin_coverage_and_padding,
    pin_split_with_sizes,
    pin_round_trip,
    pin_rank_subset_and_piece,
]
