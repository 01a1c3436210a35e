"""The oracle's range-by-range wrappers (used to check very large groups with
bounded host memory) give the same bits as the whole-group calls (no GPU)."""
import numpy as np
import pytest

from workloads import host_grads, host_rank_major_bits
from workloads.configs import padding_stress_shapes


@pytest.mark.parametrize("chunk", [1, 3, 7])
def test_rows_equal_whole(orc, chunk):
    # Ragged group: K = 1 params, pieces that are all padding on the last ranks.
    shapes = padding_stress_shapes(5, count=12, max_rows=40, ks=(1, 3, 8)) + [(2, 5), (0, 4)]
    N, L = 9, 3
    grads = host_grads(shapes, L, seed=11)
    lay = orc.layout(shapes, N)
    S = lay["S"]
    whole = orc.reduce_scatter(shapes, N, L, grads).reshape(-1)
    shards = host_rank_major_bits(N * S, seed=4)
    whole_p = orc.allgather_place(shapes, N, shards)
    for rb in range(0, N, chunk):
        re = min(N, rb + chunk)
        rows = [[grads[c][p][min(t, rb * int(lay["R"][p])) * k: min(t, re * int(lay["R"][p])) * k]
                 for p, (t, k) in enumerate(shapes)] for c in range(L)]
        out = np.full((re - rb) * S, np.nan, np.float32)
        orc.reduce_scatter_rows(shapes, N, L, rows, (rb, re), out)
        assert np.array_equal(out.view(np.uint32), whole[rb * S: re * S].view(np.uint32))
        pr = [np.zeros((min(t, re * int(lay["R"][p])) - min(t, rb * int(lay["R"][p]))) * k, np.uint16)
              for p, (t, k) in enumerate(shapes)]
        orc.allgather_place_rows(shapes, N, shards[rb * S: re * S], (rb, re), pr)
        for p, (t, k) in enumerate(shapes):
            a, b = min(t, rb * int(lay["R"][p])) * k, min(t, re * int(lay["R"][p])) * k
            assert np.array_equal(pr[p], whole_p[p][a:b]), (rb, p)


def test_rows_reject_wrong_sizes(orc):
    shapes = [(5, 2), (3, 1)]
    N, L = 2, 2
    g = host_grads(shapes, L, seed=1)
    S = orc.layout(shapes, N)["S"]
    with pytest.raises(ValueError):
        orc.reduce_scatter_rows(shapes, N, L, g, (0, 1), np.zeros(S, np.float32))
    with pytest.raises(ValueError):
        orc.allgather_place_rows(shapes, N, np.zeros(S, np.uint16), (0, 1),
                                 [np.zeros(1, np.uint16), np.zeros(2, np.uint16)])
