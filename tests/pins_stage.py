"""Pins of the oracle's Slot-Reuse staging (gradients copied into a vacated
all-gather slot, in the group's parameter-major padded layout).

Sources, none of them the oracle's code:
  * the worked example on page 1 ("What problem is it actually solving?",
    tests/golden/worked_example.json): rank 1's piece of parameter 1 (0-based)
    starts at the "9 MB" parameter-major address;
  * the parameter-major slot built by numpy from its definition: every
    parameter zero-extended (here: sentinel-extended) to the smallest row
    count that is a multiple of N, then the parameters concatenated in order
    (np.pad + np.concatenate);
  * when every T_p is a multiple of N there is no padding, and the slot is
    the plain concatenation of the gradients (np.concatenate);
  * staging followed by the reduce-scatter from the slot equals the
    reduce-scatter from the original gradients (the reduce only sees values).
"""
import json
import os

import numpy as np

from workloads.configs import padding_stress_shapes

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SENTINEL = 0x7FC1        # a bf16 NaN pattern no gradient below uses


def _grads(shapes, L, rng):
    # Distinct values per contributor and parameter (never the sentinel).
    return [[rng.integers(0, 0x7F00, t * k, dtype=np.uint16) for (t, k) in shapes]
            for _ in range(L)]


def _padded_rows(T, N):
    """Smallest multiple of N that is not below T (found by counting up)."""
    rows = T
    while rows % N:
        rows += 1
    return rows


def _slot_by_definition(shapes, N, grads_c, fill=SENTINEL):
    parts = []
    for (t, k), g in zip(shapes, grads_c):
        a = np.asarray(g, np.uint16).reshape(t, k)
        parts.append(np.pad(a, ((0, _padded_rows(t, N) - t), (0, 0)),
                            constant_values=fill).reshape(-1))
    return np.concatenate(parts) if parts else np.zeros(0, np.uint16)


def _filled(n, L):
    return [np.full(n, SENTINEL, np.uint16) for _ in range(L)]


def pin_stage_worked_example(orc):
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    N, pieces = g["N"], g["pieces_per_rank"]
    # One row per rank (R_p = 1): parameter p is N rows of pieces[p] elements.
    shapes = [(N, k) for k in pieces]
    rng = np.random.default_rng(11)
    grads = _grads(shapes, 2, rng)
    n = N * g["per_rank_total"]
    slots = orc.stage_grads(shapes, N, 2, grads, slots=_filled(n, 2))
    r, p = g["rank"], g["param"]
    at = g["param_major_start"]
    for c in range(2):
        want = grads[c][p][r * pieces[p]:(r + 1) * pieces[p]]
        assert np.array_equal(slots[c][at:at + pieces[p]], want), c
        assert not np.any(slots[c] == SENTINEL), "no padding in this group"


def pin_stage_pad_concat(orc):
    rng = np.random.default_rng(12)
    cases = [
        ([(5, 3), (1, 7), (9, 1), (16, 2), (6, 6)], 4, 3),   # (6, 6): square
        ([(3, 5)], 8, 2),                          # T < N: ranks with only padding
        ([(7, 1), (7, 2), (7, 3)], 3, 1),
        ([(13, 6), (2, 1), (0, 4), (40, 3), (1, 1), (6, 9)], 6, 4),
        (padding_stress_shapes(3, 12, 40, [1, 3, 8]), 5, 2),
    ]
    for shapes, N, L in cases:
        grads = _grads(shapes, L, rng)
        n = _slot_by_definition(shapes, N, grads[0]).size
        slots = orc.stage_grads(shapes, N, L, grads, slots=_filled(n, L))
        for c in range(L):
            want = _slot_by_definition(shapes, N, grads[c])
            assert np.array_equal(slots[c], want), (shapes, N, c)


def pin_stage_no_padding_is_concat(orc):
    rng = np.random.default_rng(13)
    shapes, N, L = [(8, 4), (4, 4), (12, 4), (4, 1)], 4, 3
    grads = _grads(shapes, L, rng)
    n = sum(t * k for t, k in shapes)
    slots = orc.stage_grads(shapes, N, L, grads, slots=_filled(n, L))
    for c in range(L):
        assert np.array_equal(slots[c], np.concatenate(grads[c])), c


def pin_stage_rank_ranges(orc):
    """Staging ranks [0, k) and then [k, N) writes the same slot as staging
    all ranks; staging one rank r writes exactly rows [r R_p, (r + 1) R_p)."""
    rng = np.random.default_rng(14)
    shapes, N, L = [(13, 6), (2, 1), (40, 3), (1, 1), (6, 9)], 6, 2
    grads = _grads(shapes, L, rng)
    n = _slot_by_definition(shapes, N, grads[0]).size
    full = orc.stage_grads(shapes, N, L, grads, slots=_filled(n, L))
    for k in (0, 1, 4, 6):
        two = _filled(n, L)
        orc.stage_grads(shapes, N, L, grads, slots=two, rank_range=(0, k))
        orc.stage_grads(shapes, N, L, grads, slots=two, rank_range=(k, N))
        for c in range(L):
            assert np.array_equal(two[c], full[c]), (k, c)
    for r in range(N):
        one = orc.stage_grads(shapes, N, L, grads, slots=_filled(n, L), rank_range=(r, r + 1))
        for c in range(L):
            # Expected: the definition's slot with every row outside rank r's
            # block of padded rows replaced by the sentinel.
            want_parts = []
            for (t, k), g in zip(shapes, grads[c]):
                pr = _padded_rows(t, N)
                a = np.full((pr, k), SENTINEL, np.uint16)
                a[:t] = np.asarray(g).reshape(t, k)
                per = pr // N
                keep = np.full((pr, k), SENTINEL, np.uint16)
                keep[r * per:(r + 1) * per] = a[r * per:(r + 1) * per]
                want_parts.append(keep.reshape(-1))
            assert np.array_equal(one[c], np.concatenate(want_parts)), (r, c)


def pin_stage_then_reduce(orc):
    """The reduce-scatter of the staged slots, read at each parameter's
    position in the definition's layout, equals the reduce-scatter of the
    original gradients bit for bit."""
    rng = np.random.default_rng(15)
    shapes, N, L = [(5, 3), (1, 7), (9, 1), (16, 2), (0, 5)], 4, 3
    grads = _grads(shapes, L, rng)
    n = _slot_by_definition(shapes, N, grads[0]).size
    slots = orc.stage_grads(shapes, N, L, grads, slots=_filled(n, L))
    starts = np.cumsum([0] + [_padded_rows(t, N) * k for t, k in shapes])
    views = [[slots[c][starts[p]:starts[p] + t * k] for p, (t, k) in enumerate(shapes)]
             for c in range(L)]
    a = orc.reduce_scatter(shapes, N, L, grads)
    b = orc.reduce_scatter(shapes, N, L, views)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


ALL_PINS = [pin_stage_worked_example, pin_stage_pad_concat, pin_stage_no_padding_is_concat,
            pin_stage_rank_ranges, pin_stage_then_reduce]
