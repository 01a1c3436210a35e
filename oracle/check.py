"""Whole-output comparison of one GPU step with the CPU oracle, streamed by
rank range so that host memory stays bounded by one range's gradients.

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by the GPU
tests and by the benchmark's CPU-baseline leg (which also times the oracle
here). The GPU tensors are only copied to the host; every value compared
against them is computed by the unchanged oracle.
"""
import os
import statistics
import time

import numpy as np


def _run_threads(fn, a, b, nthreads):
    """fn(x, y) on up to `nthreads` host threads over disjoint rank slices of
    [a, b) (the oracle's C calls release the interpreter lock); wall seconds."""
    import threading
    cuts = [a + round(i * (b - a) / nthreads) for i in range(nthreads + 1)]
    slices = [(x, y) for x, y in zip(cuts, cuts[1:]) if y > x]
    th = [threading.Thread(target=fn, args=sl) for sl in slices]
    t0 = time.perf_counter()
    for t in th:
        t.start()
    for t in th:
        t.join()
    return time.perf_counter() - t0, len(slices)


def whole_output(orc, cfg, S, grads, out, shards, params, one_thread_reps=0):
    """The whole output of one step against the CPU oracle, bit for bit: every
    shard of the reduce-scatter and every parameter the placement wrote, from
    the same bits copied from the GPU. Streamed by rank range (as many ranks
    at a time as host threads), so host memory stays bounded by one range's
    gradients. The oracle runs unchanged, one host thread per rank slice.
    With one_thread_reps > 0, the first range is also timed on one thread
    (median of that many runs)."""
    import torch
    N, L, shapes = cfg.N, cfg.L, list(cfg.shapes)
    R = [int(x) for x in orc.layout(shapes, N)["R"]]
    cores = len(os.sched_getaffinity(0))
    chunk = max(8, min(cores, N))
    t_rs = t_ag = 0.0
    used = 1
    ok_rs = ok_ag = True
    first_bad = None
    one = None
    nbytes = 0
    for a in range(0, N, chunk):
        b = min(N, a + chunk)
        lo = [min(t, a * R[p]) for p, (t, _) in enumerate(shapes)]
        hi = [min(t, b * R[p]) for p, (t, _) in enumerate(shapes)]
        h_g = [[grads[c][p].view(-1)[lo[p] * k: hi[p] * k].view(torch.int16).cpu().numpy()
                .view(np.uint16) for p, (_, k) in enumerate(shapes)] for c in range(L)]
        h_sh = shards[a * S: b * S].view(torch.int16).cpu().numpy().view(np.uint16)
        h_out = np.empty((b - a) * S, np.float32)
        h_par = [np.empty((hi[p] - lo[p]) * k, np.uint16) for p, (_, k) in enumerate(shapes)]
        valid = sum((hi[p] - lo[p]) * k for p, (_, k) in enumerate(shapes))
        cbytes = 2 * L * valid + 4 * (b - a) * S + 4 * valid
        nbytes += cbytes

        def rows_of(arrs, x, y):
            return [arr[(min(t, x * R[p]) - lo[p]) * k: (min(t, y * R[p]) - lo[p]) * k]
                    for p, ((t, k), arr) in enumerate(zip(shapes, arrs))]

        def rs(x, y):
            orc.reduce_scatter_rows(shapes, N, L, [rows_of(h_g[c], x, y) for c in range(L)],
                                    (x, y), h_out[(x - a) * S: (y - a) * S])

        def ag(x, y):
            orc.allgather_place_rows(shapes, N, h_sh[(x - a) * S: (y - a) * S], (x, y),
                                     rows_of(h_par, x, y))
        if one_thread_reps and a == 0:
            t1 = [(_run_threads(rs, a, b, 1)[0], _run_threads(ag, a, b, 1)[0])
                  for _ in range(one_thread_reps)]
            t1r = statistics.median(x for x, _ in t1)
            t1a = statistics.median(y for _, y in t1)
            one = {"ranks": "0-%d" % (b - 1), "reps": one_thread_reps, "reduce_s": round(t1r, 3),
                   "placement_s": round(t1a, 3), "GBps": round(cbytes / (t1r + t1a) / 1e9, 4)}
        dt, n = _run_threads(rs, a, b, cores)
        used = max(used, n)
        t_rs += dt
        dt, _ = _run_threads(ag, a, b, cores)
        t_ag += dt
        g_out = out[a * S: b * S].cpu().numpy()
        if not np.array_equal(g_out.view(np.uint32), h_out.view(np.uint32)):
            ok_rs = False
            first_bad = first_bad or "reduce-scatter, ranks %d-%d" % (a, b - 1)
        for p, (_, k) in enumerate(shapes):
            g_p = params[p].view(-1)[lo[p] * k: hi[p] * k].view(torch.int16).cpu().numpy()
            if not np.array_equal(g_p.view(np.uint16), h_par[p]):
                ok_ag = False
                first_bad = first_bad or "placement, parameter %d, ranks %d-%d" % (p, a, b - 1)
        del h_g, h_sh, h_out, h_par
    return {"reduce_scatter_bit_exact": ok_rs, "placement_bit_exact": ok_ag,
            "first_mismatch": first_bad, "bytes": nbytes, "reduce_s": t_rs, "placement_s": t_ag,
            "threads": used, "ranks_per_range": chunk, "one_thread": one}
