"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutant is a textual edit of oracle/tide_oracle.c compiled into its own
library under pytest's tmp_path; the real oracle is never modified. All
mutants keep every memory access in bounds.
"""
import os

import pytest

import pins
import pins_landing
import pins_stage
from oracle import Oracle
from oracle import build as obuild

RS_FOLD = (
    "v = widen_bf16(grads[0 * (int64_t)P + p][t * K + k]);\n"
    "                        for (int32_t c = 1; c < L; ++c)\n"
    "                            v = v + widen_bf16(grads[(int64_t)c * P + p][t * K + k]);")

LANDING_MUTANTS = {
    # slice from index c seated on GPU (s + c) instead of (s - c)
    "landing_wrong_seat": ("const int32_t g = (int32_t)(((s - c) % L + L) % L);",
                           "const int32_t g = (int32_t)(((s + c) % L + L) % L);"),
    # the last source dropped
    "landing_drop_source": ("for (int32_t c = 1; c < M; ++c) {\n                    const int32_t g",
                            "for (int32_t c = 1; c < M - 1; ++c) {\n                    const int32_t g"),
    # slot and block swapped in the inbox offset
    "landing_block_slot_swapped": ("const int64_t at = (s * L + b) * C + e;",
                                   "const int64_t at = (b * L + s) * C + e;"),
    # every destination GPU reads block 0 of the slice
    "landing_ignores_block": ("const int64_t at = (s * L + b) * C + e;",
                              "const int64_t at = (s * L + 0 * b) * C + e;"),
    # the accumulate flag ignored
    "landing_accumulate_ignored": ("shards[b][f] = accumulate ? shards[b][f] + v : v;",
                                   "shards[b][f] = v;"),
    # Latin square with c = (src - dst) mod M
    "latin_sign": ("*c = ((dst - src) % M + M) % M;", "*c = ((src - dst) % M + M) % M;"),
}

STAGE_MUTANTS = {
    # staged at o_p (the rank-major offset) instead of N * o_p
    "stage_offset_unscaled": ("slots[c][(int64_t)N * lay.o[p] + t * row_len[p] + k] =",
                              "slots[c][lay.o[p] + t * row_len[p] + k] ="),
    # slot c receives the next contributor's gradients
    "stage_wrong_contributor": ("grads[(int64_t)c * P + p][t * row_len[p] + k];",
                                "grads[(int64_t)((c + 1) % L) * P + p][t * row_len[p] + k];"),
    # the last row of every parameter left out
    "stage_drops_last_row": ("const int64_t t1 = t0 + lay.R[p] < rows[p] ? t0 + lay.R[p] : rows[p];",
                             "const int64_t t1 = t0 + lay.R[p] < rows[p] - 1 ? t0 + lay.R[p] : rows[p] - 1;"),
    # the rank range applied to rows as if R_p were 1
    "stage_range_by_row": ("const int64_t t0 = (int64_t)r * lay.R[p];",
                           "const int64_t t0 = (int64_t)r;"),
    # rows transposed with columns (row-major order lost)
    "stage_transposed": ("slots[c][(int64_t)N * lay.o[p] + t * row_len[p] + k] =",
                         "slots[c][(int64_t)N * lay.o[p] + ((rows[p] == row_len[p]) ? k * rows[p] + t : t * row_len[p] + k)] ="),
}

MUTANTS = {
    # the fold drops the last contributor
    "drop_last_contributor": (RS_FOLD, RS_FOLD.replace("c < L;", "c < L - 1;")),
    # subtracts instead of adds
    "wrong_sign": (RS_FOLD, RS_FOLD.replace("v = v + widen", "v = v - widen")),
    # sums in reverse contributor order
    "reverse_order": (RS_FOLD, RS_FOLD.replace(
        "grads[0 * (int64_t)P + p]", "grads[(int64_t)(L - 1) * P + p]").replace(
        "for (int32_t c = 1; c < L; ++c)", "for (int32_t c = L - 2; c >= 0; --c)")),
    # floor instead of ceil for the padded rows per rank
    "rows_floor": ("Rp = rows[p] / N + (rows[p] % N != 0);", "Rp = rows[p] / N + (rows[p] % N > 1);"),
    # always one extra padded row
    "rows_plus_one": ("Rp = rows[p] / N + (rows[p] % N != 0);", "Rp = rows[p] / N + 1;"),
    # prefix offset of the last parameter off by one element
    "offset_off_by_one": ("o[p] = acc;", "o[p] = (p + 1 == P && acc > 0) ? acc - 1 : acc;"),
    # padding written as -0.0 instead of +0.0
    "negative_zero_pad": ("v = 0.0f;                             /* zero-padded row */",
                          "v = -0.0f;                            /* zero-padded row */"),
    # output laid out parameter-major (the 9 MB order) instead of rank-major
    "param_major_output": ("const int64_t d = (int64_t)r * out_stride + lay.o[p] + i * K + k;",
                           "const int64_t d = (int64_t)N * lay.o[p] + (int64_t)r * lay.s[p] + i * K + k;"),
    # shard stride ignored in the reduce-scatter (packed S used instead)
    "rs_ignores_stride": ("const int64_t d = (int64_t)r * out_stride + lay.o[p] + i * K + k;",
                          "const int64_t d = (int64_t)r * lay.S + lay.o[p] + i * K + k;"),
    # shard stride ignored in the placement
    "ag_ignores_stride": ("const int64_t src = (int64_t)r * shard_stride + lay.o[p] + i * K + k;",
                          "const int64_t src = (int64_t)r * lay.S + lay.o[p] + i * K + k;"),
    # placement reads the row of the wrong rank's piece (rank-major order lost)
    "ag_wrong_piece": ("const int64_t src = (int64_t)r * shard_stride + lay.o[p] + i * K + k;",
                       "const int64_t src = (int64_t)(N - 1 - r) * shard_stride + lay.o[p] + i * K + k;"),
    # rounding bit set while widening bf16
    "widen_rounds": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = ((uint32_t)h << 16) | 0x8000u;"),
    # widening that flushes subnormals to zero
    "widen_ftz": ("uint32_t u = (uint32_t)h << 16;",
                  "uint32_t u = (((uint32_t)h >> 7) & 0xFFu) ? ((uint32_t)h << 16) : (((uint32_t)h & 0x8000u) << 16);"),
    # rows transposed with columns inside a piece
    "row_col_transposed": ("v = v + widen_bf16(grads[(int64_t)c * P + p][t * K + k]);\n",
                           "v = v + widen_bf16(grads[(int64_t)c * P + p][(K > 1 && k < T && t < K) ? k * K + t : t * K + k]);\n"),
}


def _build_mutant(tmp_path, name, old, new):
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, "anchor of mutant %s not found in the oracle" % name
    mutated = src.replace(old, new, 1)
    assert mutated != src
    path = os.path.join(str(tmp_path), "mut_%s.c" % name)
    with open(path, "w") as f:
        f.write(mutated)
    lib = os.path.join(str(tmp_path), "libmut_%s.so" % name)
    obuild.build(src=path, out=lib, extra=["-Wno-error"])
    return Oracle(lib)


ALL_MUTANTS = {**MUTANTS, **LANDING_MUTANTS, **STAGE_MUTANTS}


@pytest.mark.parametrize("name", sorted(ALL_MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = ALL_MUTANTS[name]
    orc = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in pins.ALL_PINS + pins_landing.ALL_PINS + pins_stage.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, "no pin catches the planted mistake %r" % name
