"""Workgroup traces (tide_launch.trace) and the diagnostic occupant.

  * a traced call writes exactly the output of an untraced one, and one valid
    record per workgroup, for the reduce, the placement, the staging and the
    landing sum, full grid and budgeted;
  * with the LDS reservation, the workgroups of one budgeted launch sit on
    distinct CUs (two 128 KiB reservations do not fit one CU's 160 KiB);
  * a trace array that is too small is refused before anything is enqueued;
  * the occupant's records are valid and its wait ends.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, say
from workloads import device_grads, device_rank_major_bits

pytestmark = pytest.mark.gpu

SHAPES = [(300, 1000), (17, 4096), (1, 1), (5000, 64), (9, 7)]
N, L = 16, 4


@pytest.fixture(scope="module")
def tide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_rs_amd as t
    return t


def _check_records(tide, buf, n):
    rec = tide.decode_trace(buf, n)
    assert np.all(rec["t_end"] >= rec["t_begin"]) and np.all(rec["t_begin"] > 0)
    assert np.all(rec["xcc"] < 8)
    # nothing written past the records the call needs
    assert torch.all(buf[n * 3:] == 0)
    return rec


@pytest.mark.parametrize("budgeted", [False, True])
def test_traced_calls_match_untraced(tide, budgeted):
    plan = tide.plan_create(SHAPES, N, L)
    S = plan.S
    grads = device_grads(SHAPES, L, seed=1)
    base = tide.budgeted(max_launch_us=20) if budgeted else tide.Launch()
    ref = torch.empty(N * S, dtype=torch.float32, device=dev())
    out = torch.empty_like(ref)
    tide.reduce_scatter_bf16_fp32(plan, grads, ref, launch=base)
    n = plan.trace_records(0, base)
    buf = tide.trace_buffer(n + 5)
    tide.reduce_scatter_bf16_fp32(plan, grads, out, launch=tide.traced(base, buf))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    rec = _check_records(tide, buf, n)
    say("reduce %s: %d records on %d CUs" % ("budgeted" if budgeted else "full", n,
                                               len(set(rec["cu"].tolist()))))
    if budgeted:
        for k in range(0, n, 16):
            cus = rec["cu"][k:k + 16]
            assert len(set(cus.tolist())) == len(cus), "two fenced workgroups share a CU"

    sh = device_rank_major_bits(N * S, seed=2)
    p_ref = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    p_out = [torch.empty((t, k), dtype=torch.bfloat16, device=dev()) for t, k in SHAPES]
    tide.allgather_place(plan, sh, p_ref, launch=base)
    n = plan.trace_records(1, base)
    buf = tide.trace_buffer(n + 5)
    tide.allgather_place(plan, sh, p_out, launch=tide.traced(base, buf))
    torch.cuda.synchronize()
    for a, b in zip(p_ref, p_out):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    _check_records(tide, buf, n)

    slots_ref = [torch.zeros(N * S, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    slots_out = [torch.zeros(N * S, dtype=torch.bfloat16, device=dev()) for _ in range(L)]
    tide.stage_grads_bf16(plan, grads, slots_ref, launch=base)
    n = plan.trace_records(2, base)
    buf = tide.trace_buffer(n + 5)
    tide.stage_grads_bf16(plan, grads, slots_out, launch=tide.traced(base, buf))
    torch.cuda.synchronize()
    for a, b in zip(slots_ref, slots_out):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    _check_records(tide, buf, n)

    Lg, Mg, Sg = 4, 3, 5003
    C = -(-Sg // Lg)
    inb = [torch.randn(Lg * Lg * C, device=dev()) for _ in range(Lg)]
    s_ref = [torch.empty(Sg, device=dev()) for _ in range(Lg)]
    s_out = [torch.empty(Sg, device=dev()) for _ in range(Lg)]
    tide.landing_sum_fp32(Lg, Mg, Sg, inb, s_ref, launch=base)
    n = tide.landing_trace_records(Lg, Mg, Sg, launch=base)
    buf = tide.trace_buffer(n + 5)
    tide.landing_sum_fp32(Lg, Mg, Sg, inb, s_out, launch=tide.traced(base, buf))
    torch.cuda.synchronize()
    for a, b in zip(s_ref, s_out):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    _check_records(tide, buf, n)


def test_trace_too_small_is_refused(tide):
    plan = tide.plan_create(SHAPES, N, L)
    grads = device_grads(SHAPES, L, seed=1)
    out = torch.full((N * plan.S,), 7.0, dtype=torch.float32, device=dev())
    b = tide.budgeted(max_launch_us=20)
    n = plan.trace_records(0, b)
    buf = tide.trace_buffer(n)
    with pytest.raises(tide.TideError) as e:
        tide.reduce_scatter_bf16_fp32(plan, grads, out, launch=tide.traced(b, buf, records=n - 1))
    assert e.value.status_name == "TIDE_ERR_INVALID_ARG"
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(buf == 0)


def test_occupant(tide):
    n = 128
    buf = tide.trace_buffer(n)
    tide.diag_occupy(n, 256, 42496, 20000, buf)
    torch.cuda.synchronize()
    rec = _check_records(tide, buf, n)
    span = rec["t_end"] - rec["t_begin"]
    assert np.all(span >= 20000)
    say("occupant: %d workgroups on %d CUs, median span %d ticks" % (
        n, len(set(rec["cu"].tolist())), int(np.median(span))))
