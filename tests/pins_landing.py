"""Pins of the oracle's level-2 landing sum and Latin-square seating.

Sources, none of them the oracle's code: the 4-GPU hand calculation on page 1
(tests/golden/latin_square.json), the defining property of a Latin square,
closed forms exact in binary32, the recursive-summation error bound, and the
two-level pipeline against the oracle's flat reduce-scatter on integer
gradients (every sum exact, so the two must agree bit for bit).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np

from workloads import fp32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _inboxes(L, S, rng, kind="normal", M=None):
    C = -(-S // L)
    out = []
    for _ in range(L):
        if kind == "normal":
            a = rng.standard_normal(L * L * C).astype(np.float32)
        elif kind == "int":
            a = rng.integers(-1000, 1001, L * L * C).astype(np.float32)
        out.append(a)
    return out, C


def pin_latin_hand_example(orc):
    with open(os.path.join(GOLDEN, "latin_square.json")) as f:
        g = json.load(f)
    L, M = g["L"], g["M"]
    node = {"D": 0}
    for name, c in g["relative_index"].items():
        node[name] = (node["D"] - c) % M
    for name, gpu in g["lands_on_gpu"].items():
        c, slice_of, gpu_of = orc.latin_square(M, L, node["D"], node[name])
        assert c == g["relative_index"][name]
        assert gpu_of[g["slice"]] == gpu, (name, gpu_of)


def pin_latin_property(orc):
    """For M = L the seating is a Latin square: every destination GPU receives
    every slice from exactly one source and every source once per slice."""
    for L in (1, 2, 3, 4, 5, 8):
        M = L
        for dst in range(M):
            table = {}                                  # (gpu, slice) -> source
            for src in range(M):
                c, slice_of, gpu_of = orc.latin_square(M, L, dst, src)
                for j in range(L):                      # source GPU j sends over rail j to GPU j
                    s = slice_of[j]
                    assert gpu_of[s] == j
                    assert (j, s) not in table
                    table[(j, s)] = src
            assert len(table) == L * L
            for j in range(L):
                assert sorted(table[(j, s)] for s in range(L)) == list(range(M))
                assert sorted(table[(g, j)] for g in range(L)) == list(range(M))


def _value(inboxes, L, C, g, s, b, e):
    return inboxes[g][(s * L + b) * C + e]


def pin_landing_closed_forms(orc):
    rng = np.random.default_rng(21)
    for L, M, S in ((4, 4, 37), (8, 5, 100), (3, 1, 10), (8, 8, 64)):
        C = -(-S // L)
        # identical bf16-representable partials: M * x exactly, in any order
        x = (np.asarray(fp32_to_bf16_bits(rng.standard_normal(L * L * C).astype(np.float32) * 5),
                        dtype=np.uint32) << 16).view(np.float32)
        shards = orc.landing_sum(L, M, S, [x] * L)
        for b in range(L):
            for f in range(S):
                s, e = divmod(f, C)
                want = np.float32(M * float(x[(s * L + b) * C + e]))
                assert shards[b][f].view(np.uint32) == want.view(np.uint32)
        # integers: exact sums through the Latin square
        ib, C = _inboxes(L, S, rng, "int")
        shards = orc.landing_sum(L, M, S, ib)
        for b in range(L):
            for f in range(S):
                s, e = divmod(f, C)
                want = sum(float(_value(ib, L, C, (s - c) % L, s, b, e)) for c in range(M))
                assert shards[b][f] == want
        # accumulate adds to the shard's value
        init = [np.full(S, 3.0, np.float32) for _ in range(L)]
        acc = orc.landing_sum(L, M, S, ib, shards=init, accumulate=True)
        for b in range(L):
            assert np.array_equal(acc[b], shards[b] + np.float32(3.0))


def pin_landing_error_bound(orc):
    rng = np.random.default_rng(22)
    L, M, S = 8, 8, 50
    ib, C = _inboxes(L, S, rng, "normal")
    shards = orc.landing_sum(L, M, S, ib)
    for b in range(L):
        for f in range(S):
            s, e = divmod(f, C)
            xs = [float(_value(ib, L, C, (s - c) % L, s, b, e)) for c in range(M)]
            exact = sum((Fraction(v) for v in xs), Fraction(0))
            err = abs(Fraction(float(shards[b][f])) - exact)
            assert err <= Fraction((M - 1) * 2.0 ** -24 * sum(abs(v) for v in xs))


def pin_landing_order(orc):
    """[1, 2^-24 x 7] over c = 0..7 is 1.0 for a left fold in source order."""
    L = M = 8
    S = L
    C = 1
    ib = [np.zeros(L * L * C, np.float32) for _ in range(L)]
    # element (b = 0, slice 0): source c sits on GPU (0 - c) mod L at offset 0
    for c in range(M):
        ib[(-c) % L][0] = 1.0 if c == 0 else 2.0 ** -24
    assert orc.landing_sum(L, M, S, ib)[0][0] == np.float32(1.0)
    for c in range(M):
        ib[(-c) % L][0] = 1.0 if c == M - 1 else 2.0 ** -24
    assert orc.landing_sum(L, M, S, ib)[0][0] == np.float32(1.0 + 2.0 ** -21)


def two_level(orc, shapes, M, L, grads_by_node, dst):
    """Level 1 on every source node for destination node dst, routed by the
    Latin square into dst's inboxes, then the landing sum. Returns dst's L
    shards (rank dst * L + b)."""
    N = M * L
    S = orc.layout(shapes, N)["S"]
    C = -(-S // L)
    inboxes = [np.full(L * L * C, np.nan, np.float32) for _ in range(L)]
    for src in range(M):
        part = orc.reduce_scatter(shapes, N, L, grads_by_node[src],
                                  rank_range=(dst * L, dst * L + L))[dst * L: dst * L + L]
        c, slice_of, gpu_of = orc.latin_square(M, L, dst, src)
        for j in range(L):                       # source GPU j: slice (j + c) mod L, rail j
            s = slice_of[j]
            g = gpu_of[s]
            assert g == j
            n = max(0, min(C, S - s * C))
            for b in range(L):
                inboxes[g][(s * L + b) * C:(s * L + b) * C + n] = part[b, s * C: s * C + n]
    return orc.landing_sum(L, M, S, inboxes)


def pin_two_level_equals_flat(orc):
    """With integer gradients every sum is exact, so level 1 + Latin-square
    routing + landing must equal one flat reduce-scatter over all M * L
    contributors, bit for bit (and the zero padding must survive)."""
    rng = np.random.default_rng(23)
    for shapes, M, L in (([(40, 3), (7, 1), (65, 2)], 3, 4), ([(31, 5)], 4, 4), ([(9, 2), (100, 1)], 2, 8)):
        N = M * L
        grads_by_node = []
        for _ in range(M):
            grads_by_node.append([[fp32_to_bf16_bits(rng.integers(-64, 65, t * k).astype(np.float32))
                                   for (t, k) in shapes] for _ in range(L)])
        flat_grads = [row for node in grads_by_node for row in node]          # M * L contributors
        flat = orc.reduce_scatter(shapes, N, M * L, flat_grads)
        for dst in range(M):
            shards = two_level(orc, shapes, M, L, grads_by_node, dst)
            for b in range(L):
                assert np.array_equal(shards[b].view(np.uint32), flat[dst * L + b].view(np.uint32))


ALL_PINS = [pin_latin_hand_example, pin_latin_property, pin_landing_closed_forms,
            pin_landing_error_bound, pin_landing_order, pin_two_level_equals_flat]
