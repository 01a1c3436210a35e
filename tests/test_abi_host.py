"""The C-ABI library on the host (no GPU): it loads, exports every symbol that
include/tide.h declares, plans layouts identical to the oracle's, and rejects
bad arguments before touching the GPU. No compute call is made here."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tide():
    import mixed_precision_rs_amd as t
    return t


def header_functions():
    with open(os.path.join(ROOT, "include", "tide.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tide_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(tide):
    declared = header_functions()
    assert set(declared) == set(tide.EXPORTS), declared
    lib = ctypes.CDLL(tide.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(tide):
    lib = tide.lib()
    for code, name in tide._lib.STATUS_NAMES.items():
        assert lib.tide_status_string(code).decode() == name
    assert lib.tide_status_string(99).decode() == "TIDE_ERR_UNKNOWN"
    assert tide.version() >> 16 == 1


def test_layout_equals_oracle(tide, orc):
    from workloads.configs import CONFIGS, padding_stress_shapes
    groups = [(c.shapes, c.N) for c in CONFIGS.values()]
    groups += [(padding_stress_shapes(s, count=30, max_rows=40, ks=(1, 2, 3, 7)), n)
               for s, n in [(1, 5), (2, 16), (3, 1)]]
    for shapes, N in groups:
        plan = tide.plan_create(shapes, N, 8)
        lay = orc.layout(shapes, N)
        assert plan.S == lay["S"]
        for p, (t, k) in enumerate(shapes):
            T, K, R, s, o = plan.param(p)
            assert (T, K, R, s, o) == (t, k, lay["R"][p], lay["s"][p], lay["o"][p])
        for r in sorted({0, min(1, N - 1), N // 2, N - 1}):
            for p in range(0, len(shapes), max(1, len(shapes) // 7)):
                rm, pm, valid = plan.map(r, p)
                orm, _, opmg = orc.piece_start(shapes, N, r, p)
                assert (rm, pm) == (orm, opmg)
                _, nrows = orc.piece_rows(shapes, N, r, p)
                assert valid == nrows * shapes[p][1]


def test_worked_example_map(tide):
    with open(os.path.join(ROOT, "tests", "golden", "worked_example.json")) as f:
        g = json.load(f)
    N = g["N"]
    plan = tide.plan_create([(N * n, 1) for n in g["pieces_per_rank"]], N, 4)
    rm, pm, valid = plan.map(g["rank"], g["param"])
    assert (rm, pm) == (g["rank_major_start"], g["param_major_start"])
    assert plan.S == g["per_rank_total"]


def _status(fn):
    try:
        fn()
    except Exception as e:  # noqa: BLE001
        return getattr(e, "status_name", type(e).__name__)
    return "TIDE_OK"


def test_plan_create_rejects(tide):
    assert _status(lambda: tide.plan_create([(4, 1)], 0, 1)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: tide.plan_create([(4, 1)], 2, 0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: tide.plan_create([(4, 1)], 2, 65)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: tide.plan_create([(-1, 1)], 2, 1)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: tide.plan_create([(4, 0)], 2, 1)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: tide.plan_create([(1 << 40, 1 << 30)], 2, 1)) == "TIDE_ERR_OVERFLOW"
    assert _status(lambda: tide.plan_create([(1 << 31, 1 << 31)], 1, 1)) == "TIDE_ERR_OVERFLOW"
    assert _status(lambda: tide.plan_create([(1 << 31, 1 << 30)] * 3, 1, 1)) == "TIDE_ERR_OVERFLOW"
    lib = tide.lib()
    assert lib.tide_plan_create(None, None, 1, 2, 1, ctypes.byref(ctypes.c_void_p())) == 1
    assert lib.tide_plan_create(None, None, 0, 2, 1, None) == 1
    # An empty group and zero-row parameters are valid.
    assert tide.plan_create([], 4, 2).S == 0
    p = tide.plan_create([(0, 7), (5, 2)], 4, 2)
    assert p.param(0)[2:] == (0, 0, 0) and p.S == 4
    assert _status(lambda: p.param(2)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: p.map(4, 0)) == "TIDE_ERR_INVALID_ARG"
    tide.lib().tide_plan_destroy(None)          # NULL-safe


def test_launch_count(tide):
    from workloads.configs import CONFIGS
    cfg = CONFIGS["wan22_dit_block"]
    plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
    assert plan.launch_count(0) == 1 and plan.launch_count(1) == 1
    b = plan.launch_count(0, tide.budgeted())
    assert b > 4
    assert plan.launch_count(0, tide.budgeted(max_launch_us=3000)) < b
    assert plan.launch_count(0, tide.Launch(rank_begin=3, rank_end=3)) == 0
    # Staging (op 2) walks the placement tiling once per contributor.
    assert plan.launch_count(2) == 1
    assert plan.launch_count(2, tide.budgeted()) >= plan.launch_count(1, tide.budgeted())
    assert _status(lambda: plan.launch_count(3)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: plan.launch_count(0, tide.Launch(mode=7))) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: plan.launch_count(0, tide.Launch(rank_begin=5, rank_end=2))) == \
        "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: plan.launch_count(0, tide.Launch(flags=0x10))) == "TIDE_ERR_INVALID_ARG"


FAKE = 0x7f0000000000    # addresses are never dereferenced: validation fails first


def test_compute_calls_validate_before_enqueue(tide):
    shapes = [(8, 4), (4, 4), (12, 4)]
    plan = tide.plan_create(shapes, 4, 2)
    S = plan.S
    grads = [[FAKE + 0x100000 * (c * 3 + p) for p in range(3)] for c in range(2)]
    out = FAKE + 0x10000000
    rs = tide.reduce_scatter_bf16_fp32
    assert _status(lambda: rs(plan, grads, out, out_stride=S - 1, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: rs(plan, grads, out + 2, stream=0)) == "TIDE_ERR_ALIGNMENT"
    assert _status(lambda: rs(plan, grads, 0, stream=0)) == "TIDE_ERR_INVALID_ARG"
    bad = [list(g) for g in grads]
    bad[1][2] = 0
    assert _status(lambda: rs(plan, bad, out, stream=0)) == "TIDE_ERR_INVALID_ARG"
    bad[1][2] = FAKE + 1
    assert _status(lambda: rs(plan, bad, out, stream=0)) == "TIDE_ERR_ALIGNMENT"
    bad[1][2] = out + 8                      # reads overlap the written output
    assert _status(lambda: rs(plan, bad, out, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: rs(plan, grads, out, stream=0, launch=tide.Launch(mode=3))) == \
        "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: rs(plan, grads, out, stream=0, launch=tide.Launch(rank_begin=-1))) == \
        "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: rs(plan, grads, out, out_stride=1 << 62, stream=0)) == "TIDE_ERR_OVERFLOW"
    # An empty rank range enqueues nothing and succeeds without a GPU.
    assert _status(lambda: rs(plan, grads, out, stream=0,
                              launch=tide.Launch(rank_begin=2, rank_end=2))) == "TIDE_OK"

    ag = tide.allgather_place
    shards = FAKE + 0x20000000
    params = [FAKE + 0x30000000 + 0x100000 * p for p in range(3)]
    assert _status(lambda: ag(plan, shards, params, shard_stride=S - 1, stream=0)) == \
        "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: ag(plan, shards + 1, params, stream=0)) == "TIDE_ERR_ALIGNMENT"
    assert _status(lambda: ag(plan, shards, params, stream=0, engine=5)) == "TIDE_ERR_INVALID_ARG"
    # The DMA-engine path validates the same way before it touches the GPU;
    # with valid arguments it needs one (here: TIDE_ERR_HIP, nothing copied).
    assert _status(lambda: ag(plan, shards, params, stream=0, engine="sdma")) == "TIDE_ERR_HIP"
    assert _status(lambda: ag(plan, shards, [params[0], params[0], params[2]], stream=0,
                              engine="sdma")) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: ag(plan, shards + 1, params, stream=0, engine="sdma")) == \
        "TIDE_ERR_ALIGNMENT"
    assert _status(lambda: ag(plan, shards, [params[0], params[0], params[2]], stream=0)) == \
        "TIDE_ERR_INVALID_ARG"                # two parameters overlap
    assert _status(lambda: ag(plan, shards, [shards + 4, params[1], params[2]], stream=0)) == \
        "TIDE_ERR_INVALID_ARG"                # a parameter overlaps the shards
    assert _status(lambda: ag(plan, shards, [params[0], 0, params[2]], stream=0)) == \
        "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: ag(plan, shards, [params[0], params[1] + 1, params[2]], stream=0)) == \
        "TIDE_ERR_ALIGNMENT"


def test_stage_validates_before_enqueue(tide):
    shapes = [(8, 4), (4, 4), (12, 4)]
    plan = tide.plan_create(shapes, 4, 2)
    NS = plan.N * plan.S
    grads = [[FAKE + 0x100000 * (c * 3 + p) for p in range(3)] for c in range(2)]
    slots = [FAKE + 0x10000000, FAKE + 0x10000000 + 2 * NS]
    st = tide.stage_grads_bf16
    assert _status(lambda: st(plan, grads, [slots[0], slots[0] + 2], stream=0)) == \
        "TIDE_ERR_INVALID_ARG"                # the two slots overlap
    assert _status(lambda: st(plan, grads, [slots[0], slots[1] + 1], stream=0)) == \
        "TIDE_ERR_ALIGNMENT"
    assert _status(lambda: st(plan, grads, [slots[0], 0], stream=0)) == "TIDE_ERR_INVALID_ARG"
    bad = [list(g) for g in grads]
    bad[0][1] = slots[1] + 64                 # a gradient inside a slot
    assert _status(lambda: st(plan, bad, slots, stream=0)) == "TIDE_ERR_INVALID_ARG"
    bad[0][1] = FAKE + 3
    assert _status(lambda: st(plan, bad, slots, stream=0)) == "TIDE_ERR_ALIGNMENT"
    bad[0][1] = 0
    assert _status(lambda: st(plan, bad, slots, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: st(plan, grads, slots, stream=0, engine=7)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: st(plan, grads, slots, stream=0, launch=tide.Launch(rank_end=9))) == \
        "TIDE_ERR_INVALID_ARG"
    # An empty rank range enqueues nothing and succeeds without a GPU.
    assert _status(lambda: st(plan, grads, slots, stream=0,
                              launch=tide.Launch(rank_begin=1, rank_end=1))) == "TIDE_OK"
    # The reduce's table over the slots: slots[c] + N * o_p, in bytes.
    tab = tide.slot_grads_table(plan, slots)
    o = [plan.param(p)[4] for p in range(3)]
    assert [tab.arr[i] for i in range(6)] == [slots[c] + 2 * 4 * o[p] for c in range(2)
                                              for p in range(3)]
    with pytest.raises(ValueError):
        st(plan, grads, slots[:1], stream=0)


def test_trace_record_counts_and_flags(tide):
    from workloads.configs import CONFIGS
    cfg = CONFIGS["wan22_dit_block"]
    plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
    # Full grid: one launch, one workgroup per tile.
    full = plan.trace_records(0)
    assert full > 1000 and plan.launch_count(0) == 1
    # Budgeted: every launch has at most reduce_blocks (placement: place_blocks) workgroups.
    b = tide.budgeted()
    n_rs, l_rs = plan.trace_records(0, b), plan.launch_count(0, b)
    assert (l_rs - 1) * 16 < n_rs <= l_rs * 16
    n_ag, l_ag = plan.trace_records(1, b), plan.launch_count(1, b)
    assert (l_ag - 1) * 4 < n_ag <= l_ag * 4
    assert plan.trace_records(2, b) <= plan.launch_count(2, b) * 4
    # The fence flag is accepted and changes no count; unknown flags are not.
    nf = tide.budgeted(flags=tide.FLAG_NO_LDS_FENCE)
    assert plan.trace_records(0, nf) == n_rs
    assert _status(lambda: plan.trace_records(0, tide.Launch(flags=0x4))) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: plan.trace_records(3)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: plan.trace_records(0, tide.Launch(trace_capacity=-1))) == \
        "TIDE_ERR_INVALID_ARG"
    S = plan.S
    assert tide.landing_trace_records(8, 8, S) >= 1
    lb = tide.landing_trace_records(8, 8, S, launch=tide.budgeted())
    assert lb > 4 and lb % 4 in (0, 1, 2, 3)
    assert _status(lambda: tide.landing_trace_records(8, 9, S)) == "TIDE_ERR_INVALID_ARG"


def test_grid_stays_within_one_dispatch(tide):
    """A dispatch holds fewer than 2^32 work-items: a group with more tiles
    than the full grid's cap gets the capped grid (its workgroups loop over
    the rest), and budgeted block counts are bounded."""
    plan = tide.plan_create([(1 << 22, 8192)], 64, 1)      # 2^35 elements, 2^25 reduce tiles
    cap = plan.trace_records(0)
    assert cap == 1 << 24 and cap * 128 < 1 << 32
    assert plan.launch_count(0) == 1
    assert plan.trace_records(1) == 1 << 24
    b = tide.budgeted(reduce_blocks=65536, place_blocks=65536)
    assert plan.trace_records(0, b) <= plan.launch_count(0, b) * 65536
    for bad in (tide.budgeted(reduce_blocks=65537), tide.budgeted(place_blocks=1 << 30)):
        assert _status(lambda: plan.launch_count(0, bad)) == "TIDE_ERR_INVALID_ARG"


def test_diag_occupy_validates(tide):
    occ = tide.diag_occupy
    assert _status(lambda: occ(0, 256, 0, 10, FAKE, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: occ(4, 65, 0, 10, FAKE, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: occ(4, 2048, 0, 10, FAKE, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: occ(4, 256, 200 * 1024, 10, FAKE, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: occ(4, 256, 0, 10 ** 9, FAKE, stream=0)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: occ(4, 256, 0, 10, 0, stream=0)) == "TIDE_ERR_INVALID_ARG"


def test_prepared_calls_validate_before_allocating(tide):
    shapes = [(8, 4), (4, 4), (12, 4)]
    plan = tide.plan_create(shapes, 4, 2)
    S = plan.S
    grads = [[FAKE + 0x100000 * (c * 3 + p) for p in range(3)] for c in range(2)]
    out = FAKE + 0x10000000
    pr = tide.prepare_reduce_scatter_bf16_fp32
    assert _status(lambda: pr(plan, grads, out, out_stride=S - 1)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: pr(plan, grads, out + 2)) == "TIDE_ERR_ALIGNMENT"
    bad = [list(g) for g in grads]
    bad[0][0] = out + 4
    assert _status(lambda: pr(plan, bad, out)) == "TIDE_ERR_INVALID_ARG"
    shards = FAKE + 0x20000000
    params = [FAKE + 0x30000000 + 0x100000 * p for p in range(3)]
    pa = tide.prepare_allgather_place
    assert _status(lambda: pa(plan, shards, params, first_rank=4)) == "TIDE_ERR_INVALID_ARG"
    assert _status(lambda: pa(plan, shards + 1, params)) == "TIDE_ERR_ALIGNMENT"
    slots = [FAKE + 0x40000000, FAKE + 0x40000000 + 2 * 4 * S]
    ps = tide.prepare_stage_grads_bf16
    assert _status(lambda: ps(plan, grads, [slots[0], slots[0]])) == "TIDE_ERR_INVALID_ARG"
    # A NULL call handle is refused by every call entry point.
    lib = tide.lib()
    assert lib.tide_call_enqueue(None, None) == 1
    lib.tide_call_destroy(None)


def test_struct_layouts_match_the_header(tide, tmp_path):
    """The ctypes mirrors of tide_launch, tide_rd_step and tide_trace_rec have
    the C header's sizes and field offsets (compiled with the host C compiler)."""
    import subprocess
    specs = {"tide_launch": tide.Launch, "tide_rd_step": tide._lib.RdStep}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tide.h"', 'int main(void) {']
    for cname, cls in specs.items():
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append('printf("tide_trace_rec size %zu\\n", sizeof(tide_trace_rec));')
    lines.append('return 0; }')
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Werror", "-I", inc, str(src), "-o", str(exe)])
    got = dict(line.rsplit(" ", 1) for line in subprocess.check_output([str(exe)]).decode().splitlines())
    for cname, cls in specs.items():
        assert int(got["%s size" % cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got["%s.%s" % (cname, f)]) == getattr(cls, f).offset, (cname, f)
    assert int(got["tide_trace_rec size"]) == tide._lib.TRACE_REC_BYTES


def test_binding_checks_tensor_arguments(tide):
    """The library sees only pointers, so the binding checks each tensor's
    dtype, contiguity, size and device before passing its address (raw
    integer addresses are the caller's and pass unchecked)."""
    import torch
    shapes = [(8, 4), (4, 4), (12, 4)]
    plan = tide.plan_create(shapes, 4, 2)
    N, S = plan.N, plan.S
    out = torch.zeros(N * S, dtype=torch.float32)

    def grads_with(c, p, t):
        """Raw addresses everywhere but (c, p), which holds tensor t."""
        g = [[FAKE + 0x100000 * (i * 3 + j) for j in range(3)] for i in range(2)]
        g[c][p] = t
        return g

    with pytest.raises(TypeError):
        tide.grads_table(plan, grads_with(1, 2, torch.zeros((12, 4), dtype=torch.float16)))
    with pytest.raises(ValueError, match="not contiguous"):
        tide.grads_table(plan, grads_with(0, 1, torch.zeros((4, 8), dtype=torch.bfloat16)[:, ::2]))
    with pytest.raises(ValueError, match="not contiguous"):   # a broadcast view spans one row
        tide.grads_table(plan, grads_with(0, 0, torch.zeros(4, dtype=torch.bfloat16).expand(8, 4)))
    with pytest.raises(ValueError, match="expected 48"):
        tide.grads_table(plan, grads_with(1, 2, torch.zeros((11, 4), dtype=torch.bfloat16)))
    with pytest.raises(ValueError, match="not a GPU tensor"):
        tide.grads_table(plan, grads_with(1, 0, torch.zeros((8, 4), dtype=torch.bfloat16)))
    with pytest.raises(ValueError, match="params\\[1\\]"):
        tide.params_table(plan, [FAKE, torch.zeros((4, 5), dtype=torch.bfloat16), FAKE + 4096])
    tab = tide.PointerTable([FAKE] * (2 * 3))
    with pytest.raises(ValueError, match="at least %d" % (N * S)):
        tide.reduce_scatter_bf16_fp32(plan, tab, out[1:], stream=0)
    with pytest.raises(ValueError, match="at least %d" % (3 * S + S + 5 * 3)):
        tide.reduce_scatter_bf16_fp32(plan, tab, out, out_stride=S + 5, stream=0)
    with pytest.raises(TypeError):
        tide.reduce_scatter_bf16_fp32(plan, tab, out.view(torch.int32), stream=0)
    ptab = tide.PointerTable([FAKE] * 3)
    with pytest.raises(ValueError, match="shards"):
        tide.allgather_place(plan, torch.zeros(N * S - 1, dtype=torch.bfloat16), ptab, stream=0)
    with pytest.raises(ValueError, match="slots\\[1\\]"):
        tide.stage_grads_bf16(plan, tab, [FAKE, torch.zeros(N * S - 1, dtype=torch.bfloat16)],
                              stream=0)
    with pytest.raises(ValueError, match="inboxes\\[0\\]"):
        tide.landing_sum_fp32(2, 2, 7, [torch.zeros(15), FAKE], [FAKE, FAKE + 4096], stream=0)
    # Trace and count buffers: dtype, and no capacity beyond the buffer.
    buf = torch.zeros(3 * 10, dtype=torch.int64)
    with pytest.raises(ValueError, match="holds 10 records"):
        tide.traced(tide.Launch(), buf, records=11)
    with pytest.raises(TypeError):
        tide.traced(tide.Launch(), buf.view(torch.float64))
    with pytest.raises(TypeError):
        tide.counted(tide.Launch(), torch.zeros(8, dtype=torch.int64))
    with pytest.raises(ValueError, match="at least 33"):
        tide.diag_occupy(11, 64, 0, 10, buf, stream=0)


def test_slot_grads_table(tide):
    """tide_plan_slot_grads: entry c * P + p is slots[c] + N * o_p (bytes: 2 per element)."""
    shapes = [(8, 4), (4, 4), (12, 4), (3, 5)]
    N, L = 4, 3
    plan = tide.plan_create(shapes, N, L)
    slots = [FAKE + 0x10000000 * c for c in range(L)]
    lib = tide.lib()
    import ctypes
    sa = (ctypes.c_void_p * L)(*slots)
    arr = (ctypes.c_void_p * (L * plan.P))()
    assert lib.tide_plan_slot_grads(plan.handle, sa, arr) == 0
    o = [plan.param(p)[4] for p in range(plan.P)]
    assert o == [0, 2 * 4, 3 * 4, 6 * 4]          # R_p * K_p prefix: 2, 1, 3 rows of 4
    for c in range(L):
        for p in range(plan.P):
            assert arr[c * plan.P + p] == slots[c] + N * o[p] * 2
    sa[1] = None
    assert lib.tide_plan_slot_grads(plan.handle, sa, arr) == 1      # INVALID_ARG


def test_noalloc_refuses_groups_beyond_its_scratch(tide):
    """The allocation-free reduce-scatter keeps its tables in a fixed 1 MiB
    device array: a group that needs more is refused on the host, before
    anything touches the GPU; a small group passes validation (and then needs
    a GPU: TIDE_ERR_HIP here)."""
    big = [(2, 3)] * 3000                           # 3000 * (44 + 8 * 40) bytes > 1 MiB
    plan = tide.plan_create(big, 2, 40)
    grads = [[FAKE + 0x100000 * (c * 3000 + p) for p in range(3000)] for c in range(40)]
    out = FAKE - 0x10000000
    rs = tide.reduce_scatter_bf16_fp32_noalloc
    assert _status(lambda: rs(plan, grads, out, stream=0)) == "TIDE_ERR_INVALID_ARG"
    small = tide.plan_create([(8, 4), (4, 4)], 4, 2)
    g2 = [[FAKE + 0x100000 * (c * 2 + p) for p in range(2)] for c in range(2)]
    assert _status(lambda: rs(small, g2, out, stream=0)) == "TIDE_ERR_HIP"
    assert _status(lambda: rs(small, g2, out + 2, stream=0)) == "TIDE_ERR_ALIGNMENT"
