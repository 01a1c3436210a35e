#!/usr/bin/env python3
"""Benchmark of the one-GPU hot path of TIDE's layout-aware FSDP2 collectives
on MI355X: the level-1 bf16 -> fp32 reduce-scatter into padded rank-major
shards, then the all-gather placement into parameter storage.

One step = one reduce-scatter + one placement (HIP kernel engine) of one
parameter group, back to back on one stream, inputs already in HBM. The
default group is the padding-stress group (the largest); the Llama, Qwen and
Wan groups follow in a per_config block, with the Wan GEMM-victim protocol.
value = algorithmic bytes per step / median time per step:
    reduce-scatter: 2 * L * valid (bf16 reads) + 4 * N * S (fp32 writes,
                    padding included), placement: 2 * valid + 2 * valid.

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--placement-engine kernel|sdma|runtime] [--parts] [--victim] [--stock]
                  [--slot-reuse] [--occupancy] [--graph] [--fence-study] [--offsets]
                  [--no-cpu-baseline] [--no-per-config]
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "effective HBM GB/s (and % of 8 TB/s) for bf16->fp32 layout RS + AG placement"
# The kernels and the host code that decides their launch shape and tile
# order: counter summaries are valid only for the code they were taken on.
KERNEL_SOURCES = [os.path.join(ROOT, "mixed_precision_rs_amd", "csrc", f)
                  for f in ("kernels.hip", "tide_internal.hpp", "plan.cpp")]
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C++ source without its comments and blank-line or trailing-space noise:
    what the compiler sees (the kernel sources hold no string literals with
    comment markers)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """sha256 of the kernel and launch-policy sources' code (comments
    excluded): counter summaries taken on other code are not used."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()


def counter_traffic(workload: str):
    """HBM bytes per reduce launch measured with rocprofv3 counters, if a
    summary for this workload exists and was taken on the current kernels."""
    path = os.path.join(PROFILES, "reduce_kernel_%s_counters.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return int(m_bytes.group(1))


def group_bytes(cfg, S):
    valid = sum(t * k for t, k in cfg.shapes)
    rs = 2 * cfg.L * valid + 4 * cfg.N * S
    ag = 4 * valid
    return rs, ag, valid


def cpu_baseline(chk, cfg):
    """The oracle timed on the host cores, from a whole-output check
    (oracle/check.py) over the whole group, on the same bits the GPU used."""
    one = chk["one_thread"]
    return {
        "value": round(chk["bytes"] / (chk["reduce_s"] + chk["placement_s"]) / 1e9, 4),
        "unit": "GB/s",
        "cores": chk["threads"],
        "kind": "oracle",
        "sample": "the whole %s group (all %d ranks, %d params): reduce-scatter + placement by the "
                  "unchanged oracle on %d host threads, one rank slice each, %d ranks at a time, "
                  "from the same bits the GPU used: %.2f s + %.2f s; one thread on ranks %s: "
                  "%.2f s + %.2f s = %.2f GB/s (median of %d runs)"
                  % (cfg.name, cfg.N, len(cfg.shapes), chk["threads"], chk["ranks_per_range"],
                     chk["reduce_s"], chk["placement_s"], one["ranks"], one["reduce_s"],
                     one["placement_s"], one["GBps"], one["reps"]),
        "value_one_thread": one["GBps"],
        "gpu_shards_bit_exact_on_sample": chk["reduce_scatter_bit_exact"] and chk["placement_bit_exact"],
        "gpu_reduce_scatter_bit_exact": chk["reduce_scatter_bit_exact"],
        "gpu_placement_bit_exact": chk["placement_bit_exact"],
        "host": host_info(),
    }


def host_info():
    """The host the CPU baseline ran on: CPU model and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0))}


def under_profiler() -> bool:
    """True when rocprofv3 launched this process (its tool library is preloaded)."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "") or any(
        k.startswith("ROCPROF_") for k in os.environ)


def gpu_clocks():
    """Current GPU clock state as rocm-smi reports it (None if it cannot be read).
    Skipped under the profiler: there the child process would carry the
    profiler's preloaded GPU state into rocm-smi's interpreter."""
    import subprocess
    if under_profiler():
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        if r.returncode != 0:
            return None
        d = json.loads(r.stdout)
        card = d.get("card0") or next(iter(d.values()))
        return {k: v for k, v in card.items() if "clock" in k.lower()}
    except Exception:  # noqa: BLE001 - a missing or failing tool only drops this field
        return None


def ceilings(torch, tide, nbytes=4 << 30, nsrc=8, reps=5):
    """Practical HBM ceilings from the library's own streaming kernels
    (tide_diag_stream; 128-thread workgroups, non-temporal accesses, the
    reduce's launch shape): pure read, pure write, copy, and the reduce's own
    access pattern with no layout logic (8 separately allocated bf16 sources
    read with 8-byte loads, the fp32 sum stored with 16-byte stores: 4 bytes
    read per byte written at L = 8). GB/s of bytes moved, median of `reps`."""
    a = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    b = torch.empty_like(a)
    n3 = nbytes // (2 * nsrc) // 1024 * 1024           # elements per source
    srcs = [torch.zeros(n3, dtype=torch.bfloat16, device="cuda") for _ in range(nsrc)]
    d3 = torch.empty(n3, dtype=torch.float32, device="cuda")
    cases = {"read": (0, [a], b, nbytes, nbytes), "write": (1, [], b, nbytes, nbytes),
             "copy": (2, [a], b, nbytes, 2 * nbytes),
             "reduce_pattern": (3, srcs, d3, n3, (2 * nsrc + 4) * n3)}
    res = {}

    def timed(kind, ss, dst, n, wg=0):
        tide.diag_stream(kind, ss, dst, n, workgroups=wg)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            tide.diag_stream(kind, ss, dst, n, workgroups=wg)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)
    for name, (kind, ss, dst, n, moved) in cases.items():
        res[name + "_GBps"] = round(moved / (timed(kind, ss, dst, n) / 1e3) / 1e9, 1)
    # Per CU, in the budgeted kernels' shape: 16 workgroups of 1024 threads on
    # 16 CUs, 1/16 of the buffers (read, and the reduce's pattern).
    nr, n3s = nbytes // 16 // 2048 * 2048, n3 // 16 // 1024 * 1024
    res["per_cu_read_GBps"] = round(nr / (timed(0, [a], b, nr, 16) / 1e3) / 1e9 / 16, 1)
    res["per_cu_reduce_pattern_GBps"] = round(
        (2 * nsrc + 4) * n3s / (timed(3, srcs, d3, n3s, 16) / 1e3) / 1e9 / 16, 1)
    del a, b, srcs, d3
    torch.cuda.empty_cache()
    return res


class SidePair:
    """Two side streams, `gs` for a GEMM (or occupant) and `cs` for the
    collective, that run at the same time. HIP maps streams onto a few
    hardware queues (GPU_MAX_HW_QUEUES), and two streams on one queue run their
    work one after the other. On MI355X a pair that ran concurrently when it
    was made ran every GEMM of the victim protocol after the collective had
    ended, minutes later in the same process. So `ensure()` checks the pair
    again before each measurement and replaces it once it has become serial.
    The check: a tiny kernel on gs completes while a 2 ms occupant
    (tide_diag_occupy, one workgroup) still runs on cs. Under counter
    collection, which serialises every kernel, no pair passes; after one
    failed search `concurrent` stays False and no more streams are made."""

    def __init__(self, torch, tide, tries=8, spin_us=2000):
        self.torch, self.tide, self.tries, self.spin_us = torch, tide, tries, spin_us
        self.trace = torch.zeros(3, dtype=torch.int64, device="cuda")
        self.x = torch.zeros(1024, device="cuda")
        self.x.add_(1.0)                         # kernels loaded before any timing
        tide.diag_occupy(1, 64, 0, 100, self.trace)
        torch.cuda.synchronize()
        self.gs = self.cs = None
        self.concurrent = False
        self.searched_in_vain = False
        self.pairs_made = 0
        self.ensure()

    def lag_ms(self):
        torch = self.torch
        lags = []
        for _ in range(2):
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.cs)
            self.tide.diag_occupy(1, 64, 0, self.spin_us * 100, self.trace, stream=self.cs)
            with torch.cuda.stream(self.gs):
                self.x.add_(1.0)
                e1.record(self.gs)
            torch.cuda.synchronize()
            lags.append(e0.elapsed_time(e1))
        return min(lags)          # a pair on one queue lags by the whole occupant every time

    def ensure(self):
        limit = 0.5 * self.spin_us / 1e3
        if self.gs is not None and (self.searched_in_vain or self.lag_ms() < limit):
            return self.concurrent
        for _ in range(self.tries):
            self.gs, self.cs = self.torch.cuda.Stream(), self.torch.cuda.Stream()
            self.pairs_made += 1
            lag = self.lag_ms()
            if lag < limit:
                log("bench: side stream pair %d runs concurrently (other stream done %.3f ms after "
                    "the occupant started)" % (self.pairs_made - 1, lag))
                self.concurrent = True
                return True
            log("bench: side stream pair %d runs serially (%.3f ms)" % (self.pairs_made - 1, lag))
        log("bench: no concurrent pair of side streams in %d tries (kernels serialised, e.g. by "
            "counter collection); GEMM-victim results will show streams_concurrent = false" % self.tries)
        self.concurrent = False
        self.searched_in_vain = True
        return False


def victim_slowdown(torch, tide, plan, grads, out, shards, params, launch, pair, reps=3, nb=4,
                    M=256, attempts=3):
    """Slowdown of an Mx8192x8192 bf16 GEMM (M = 256: the pages' victim, which
    hipBLASLt runs as 128 workgroups, half the CUs) while the reduce-scatter +
    placement run on another stream (median GEMM time, concurrent vs alone).

    The GEMMs cycle through `nb` different B matrices (nb * 128 MiB, more than
    the 256 MB Infinity Cache), so neither measurement finds B cached from the
    previous GEMM: both read it from HBM, as a training step's GEMMs do."""
    A = torch.randn(M, 8192, device="cuda", dtype=torch.bfloat16)
    Bs = [torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16) for _ in range(nb)]
    C = torch.empty(M, 8192, device="cuda", dtype=torch.bfloat16)
    for i in range(20):
        torch.matmul(A, Bs[i % nb], out=C)
    torch.cuda.synchronize()

    def gemm_times(n):
        gs = pair.gs
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        with torch.cuda.stream(gs):
            for i, (a, b) in enumerate(evs):
                a.record(gs)
                torch.matmul(A, Bs[i % nb], out=C)
                b.record(gs)
        return evs

    pair.ensure()
    alone = gemm_times(200)
    torch.cuda.synchronize()
    t_alone = statistics.median(a.elapsed_time(b) for a, b in alone)
    # Concurrent: the collective on cs, GEMMs back to back on gs. Count the
    # GEMMs that run entirely inside the collective's window; if none does
    # (a full-grid collective is shorter than its queueing delay), count those
    # that overlap the window at all.
    # When a repetition's first GEMM starts late (in the second half of the
    # window), the pair is checked again: if it has become serial it is
    # replaced and the repetition repeated; if it still runs concurrently, the
    # GEMMs waited for CUs (as beside the full grid) and the repetition counts.
    res = []
    tries = 0
    for _ in range(reps):
        for _ in range(attempts):
            tries += 1
            pair.ensure()
            cs = pair.cs
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            cs.wait_stream(torch.cuda.current_stream())
            c0.record(cs)
            tide.reduce_scatter_bf16_fp32(plan, grads, out, stream=cs, launch=launch)
            tide.allgather_place(plan, shards, params, stream=cs, launch=launch)
            c1.record(cs)
            evs = gemm_times(400)
            torch.cuda.synchronize()
            win = c0.elapsed_time(c1)
            spans = [(c0.elapsed_time(a_), c0.elapsed_time(b_)) for a_, b_ in evs]
            overlapped = pair.concurrent
            if spans[0][0] < 0.5 * win or not pair.concurrent:
                break
            made = pair.pairs_made
            pair.ensure()
            if pair.pairs_made == made:
                break
            overlapped = False           # this repetition ran on the pair just replaced
            log("bench: victim repetition ran on a serial stream pair (first GEMM at %.2f ms of a "
                "%.2f ms window); repeated on a new pair" % (spans[0][0], win))
        inside = [e - s for s, e in spans if s >= 0 and e <= win]
        kind = "inside"
        if not inside:
            inside = [e - s for s, e in spans if s < win and e > 0]
            kind = "overlapping"
        if inside:
            res.append((statistics.median(inside), win, len(inside), kind, overlapped))
    del A, Bs, C
    if not res:
        return {"gemm_ms_alone": round(t_alone, 4), "note": "no GEMM overlapped the collective"}
    conc = statistics.median(r[0] for r in res)
    return {"gemm_ms_alone": round(t_alone, 4), "gemm_ms_concurrent": round(conc, 4),
            "slowdown_pct": round(100.0 * (conc / t_alone - 1.0), 2),
            "collective_ms": round(statistics.median(r[1] for r in res), 3),
            "gemms_counted": int(statistics.median(r[2] for r in res)),
            "gemms_counted_are": res[0][3] + " the collective window",
            "streams_concurrent": all(r[4] for r in res), "repetitions_run": tries}


def fence_study(torch, tide, plan, grads, out, shards, params, pair):
    """GEMM-victim slowdown under budgeted launch variants (workgroup lifetime
    300 / 100 / 50 us, LDS fence on and off), for the pages' victim (M = 256:
    128 hipBLASLt workgroups, half the CUs) and for one that fills the GPU in
    one wave (M = 4096: 256 persistent workgroups of 256 threads, one per CU,
    66.5 KB of LDS and 256 VGPRs each), with each variant's collective time
    alone (median of 3)."""
    variants = {"full_grid": tide.Launch()}
    for us in (300, 100, 50):
        variants["budgeted_16_4_%dus_fence" % us] = tide.budgeted(max_launch_us=us)
        variants["budgeted_16_4_%dus_no_fence" % us] = tide.budgeted(
            max_launch_us=us, flags=tide.FLAG_NO_LDS_FENCE)
    res = {}
    for name, launch in variants.items():
        ts = []
        for _ in range(4):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            tide.reduce_scatter_bf16_fp32(plan, grads, out, launch=launch)
            tide.allgather_place(plan, shards, params, launch=launch)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        entry = {"collective_ms_alone": round(statistics.median(ts[1:]), 3),
                 "launches": plan.launch_count(0, launch) + plan.launch_count(1, launch)}
        for M in (256, 4096):
            log("bench: fence study M=%d %s" % (M, name))
            entry["victim_M%d" % M] = victim_slowdown(torch, tide, plan, grads, out, shards, params,
                                                       launch, pair, M=M)
        res[name] = entry
    return res


def occupancy_probe(torch, tide, plan, grads, out, shards, params, pair, probes=500,
                    probe_wgs=128, probe_threads=256, probe_lds=42496, probe_us=40):
    """Where the budgeted collective's workgroups run, how long they live, and
    whether GEMM-shaped occupants (the 256x8192x8192 GEMM's hipBLASLt kernel
    runs 128 workgroups of 256 threads with 42,496 B of LDS) land on a CU that
    a collective workgroup holds at the same time: the one-GPU analog of the
    pages' SM-id probe. Both with the LDS reservation and without it."""
    import numpy as np
    cal = tide.trace_buffer(1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tide.diag_occupy(1, 64, 0, 1000, cal)
    torch.cuda.synchronize()
    e0.record()
    tide.diag_occupy(1, 64, 0, 10_000_000, cal)
    e1.record()
    torch.cuda.synchronize()
    ticks_per_us = 1e7 / (e0.elapsed_time(e1) * 1e3)
    spin = int(probe_us * ticks_per_us)
    res = {"counter_ticks_per_us": round(ticks_per_us, 2),
           "occupant": {"workgroups": probe_wgs, "threads": probe_threads, "lds_bytes": probe_lds,
                        "spin_us": probe_us, "launches": probes}}
    for name, flags in (("with_lds_reservation", 0), ("without_lds_reservation",
                                                      tide.FLAG_NO_LDS_FENCE)):
        b = tide.budgeted(flags=flags)
        n_rs, n_ag = plan.trace_records(0, b), plan.trace_records(1, b)
        t_rs, t_ag = tide.trace_buffer(n_rs), tide.trace_buffer(n_ag)
        t_pr = tide.trace_buffer(probes * probe_wgs)
        pair.ensure()
        gs, cs = pair.gs, pair.cs
        torch.cuda.synchronize()
        cs.wait_stream(torch.cuda.current_stream())
        gs.wait_stream(torch.cuda.current_stream())
        tide.reduce_scatter_bf16_fp32(plan, grads, out, stream=cs, launch=tide.traced(b, t_rs))
        tide.allgather_place(plan, shards, params, stream=cs, launch=tide.traced(b, t_ag))
        for k in range(probes):
            tide.diag_occupy(probe_wgs, probe_threads, probe_lds, spin,
                             t_pr[k * probe_wgs * 3:], stream=gs)
        torch.cuda.synchronize()
        rs, ag = tide.decode_trace(t_rs, n_rs), tide.decode_trace(t_ag, n_ag)
        pr = tide.decode_trace(t_pr, probes * probe_wgs)
        cu = np.concatenate([rs["cu"], ag["cu"]])
        cb = np.concatenate([rs["t_begin"], ag["t_begin"]]).astype(np.int64)
        ce = np.concatenate([rs["t_end"], ag["t_end"]]).astype(np.int64)
        w0, w1 = cb.min(), ce.max()
        by_cu = {}
        for c, a, z in zip(cu.tolist(), cb.tolist(), ce.tolist()):
            by_cu.setdefault(c, []).append((a, z))
        pb, pe = pr["t_begin"].astype(np.int64), pr["t_end"].astype(np.int64)
        inside = (pb >= w0) & (pe <= w1)
        shared = 0
        for c, a, z in zip(pr["cu"][inside].tolist(), pb[inside].tolist(), pe[inside].tolist()):
            if any(x < z and a < y for x, y in by_cu.get(c, ())):
                shared += 1
        n_in = int(inside.sum())
        life = (ce - cb) / ticks_per_us
        per_launch = [len(set(rs["cu"][k:k + b.reduce_blocks].tolist()))
                      for k in range(0, n_rs, b.reduce_blocks)]
        res[name] = {
            "collective_ms": round((w1 - w0) / ticks_per_us / 1e3, 3),
            "collective_workgroups": int(n_rs + n_ag),
            "collective_distinct_cus": len(by_cu),
            "reduce_launch_distinct_cus_median": float(np.median(per_launch)),
            "collective_workgroup_life_us_median": round(float(np.median(life)), 1),
            "collective_workgroup_life_us_p90": round(float(np.percentile(life, 90)), 1),
            "occupant_workgroups_inside_window": n_in,
            "occupant_workgroups_sharing_a_cu": shared,
            "occupant_share_pct": round(100.0 * shared / max(n_in, 1), 2),
            "occupant_life_us_median": round(float(np.median((pe - pb)[inside])) / ticks_per_us, 1)
            if n_in else None,
        }
    # Full grid, for contrast.
    n_full = plan.trace_records(0)
    t_full = tide.trace_buffer(n_full)
    tide.reduce_scatter_bf16_fp32(plan, grads, out, launch=tide.traced(tide.Launch(), t_full))
    torch.cuda.synchronize()
    fr = tide.decode_trace(t_full, n_full)
    fl = (fr["t_end"].astype(np.int64) - fr["t_begin"].astype(np.int64)) / ticks_per_us
    res["full_grid_reduce"] = {"workgroups": int(n_full),
                               "distinct_cus": len(set(fr["cu"].tolist())),
                               "workgroup_life_us_median": round(float(np.median(fl)), 2)}
    return res


def graph_parts(torch, tide, plan, g_tab, out, shards, p_tab, rs_bytes, ag_bytes, iters=10):
    """The step (reduce-scatter + placement) as prepared calls: enqueued eagerly,
    and captured once into a HIP graph and replayed; full grid and budgeted.
    Host time per step (enqueue only) and GPU time per step."""
    res = {}
    for name, launch in (("full_grid", tide.Launch()), ("budgeted_16_4", tide.budgeted())):
        rs = tide.prepare_reduce_scatter_bf16_fp32(plan, g_tab, out, launch=launch)
        ag = tide.prepare_allgather_place(plan, shards, p_tab, launch=launch)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            rs.enqueue()
            ag.enqueue()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record()
        for _ in range(iters):
            rs.enqueue()
            ag.enqueue()
        e1.record()
        h_eager = (time.perf_counter() - h0) / iters
        torch.cuda.synchronize()
        t_eager = e0.elapsed_time(e1) / iters
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rs.enqueue()
            ag.enqueue()
        g.replay()
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        e0.record()
        for _ in range(iters):
            g.replay()
        e1.record()
        h_graph = (time.perf_counter() - h0) / iters
        torch.cuda.synchronize()
        t_graph = e0.elapsed_time(e1) / iters
        res[name] = {"launches_per_step": plan.launch_count(0, launch) + plan.launch_count(1, launch),
                     "prepared_eager_ms": round(t_eager, 4),
                     "prepared_eager_host_ms": round(h_eager * 1e3, 4),
                     "graph_replay_ms": round(t_graph, 4),
                     "graph_replay_host_ms": round(h_graph * 1e3, 4),
                     "graph_GBps": round((rs_bytes + ag_bytes) / (t_graph / 1e3) / 1e9, 1)}
        del g
        rs.close()
        ag.close()
    return res


def stock_fsdp2(torch, tide, plan, cfg, grads, shards, out, p_tab, iters=3):
    """The stock FSDP2 path on one GPU, for comparison: every contributor's
    gradients packed with torch._chunk_cat into an fp32 rank-major buffer (the
    pack FSDP2 runs before its reduce-scatter), the L packed buffers summed in
    contributor order, and the all-gather's rank-major output copied out with
    split_with_sizes_copy into padded parameter storage. Returns times, the
    bytes that path moves, and whether its shards equal ours bit for bit."""
    N, L, S = cfg.N, cfg.L, plan.S
    valid = sum(t * k for t, k in cfg.shapes)
    acc = torch.empty((N, S), dtype=torch.float32, device="cuda")
    tmp = torch.empty((N, S), dtype=torch.float32, device="cuda")

    def rs():
        torch._chunk_cat(grads[0], dim=0, num_chunks=N, out=acc)
        for c in range(1, L):
            torch._chunk_cat(grads[c], dim=0, num_chunks=N, out=tmp)
            acc.add_(tmp)

    sizes = [-(-t // N) * k for t, k in cfg.shapes]
    padded = [torch.empty((N, sz), dtype=torch.bfloat16, device="cuda") for sz in sizes]
    src = shards.view(N, S)

    def ag():
        torch.split_with_sizes_copy(src, sizes, dim=1, out=padded)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    rs_ms, ag_ms = timed(rs), timed(ag)
    tide.reduce_scatter_bf16_fp32(plan, tide.grads_table(plan, grads), out)
    torch.cuda.synchronize()
    exact = bool(torch.equal(acc.view(-1).view(torch.int32), out.view(torch.int32)))
    # bytes: L packs (2 V read, 4 N S written) + (L - 1) adds (8 N S read, 4 N S written)
    rs_bytes = L * (2 * valid + 4 * N * S) + (L - 1) * 12 * N * S
    ag_bytes = 2 * N * S * 2
    del acc, tmp, padded
    torch.cuda.empty_cache()
    return {"reduce_ms": round(rs_ms, 3), "placement_ms": round(ag_ms, 3),
            "reduce_bytes": rs_bytes, "placement_bytes": ag_bytes,
            "shards_equal_ours_bit_for_bit": exact}


def slot_reuse_parts(torch, tide, plan, cfg, g_tab, out, valid, in_place_ms, iters=5, chunks=8):
    """Slot-Reuse mode on this group: the staging copy of the L contributors'
    gradients into vacated slots (kernel and runtime-copy engines), the reduce
    reading the slots, and both together (whole group, and pipelined over
    rank ranges), against the in-place reduce."""
    n = cfg.N * plan.S
    slots = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.L)]
    s_tab = tide.slot_grads_table(plan, slots)
    stage_bytes = 2 * cfg.L * valid * 2

    def timed(fn, k=iters):
        fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(k):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / k

    st_k = timed(lambda: tide.stage_grads_bf16(plan, g_tab, slots))
    st_s = timed(lambda: tide.stage_grads_bf16(plan, g_tab, slots, engine="runtime"), 3)
    st_d = timed(lambda: tide.stage_grads_bf16(plan, g_tab, slots, engine="sdma"), 1)
    rd = timed(lambda: tide.reduce_scatter_bf16_fp32(plan, s_tab, out))

    def both():
        tide.stage_grads_bf16(plan, g_tab, slots)
        tide.reduce_scatter_bf16_fp32(plan, s_tab, out)
    tot = timed(both)
    bounds = [round(i * cfg.N / chunks) for i in range(chunks + 1)]
    ranges = [(a, b) for a, b in zip(bounds, bounds[1:]) if b > a]
    launches = [tide.Launch(rank_begin=a, rank_end=b) for a, b in ranges]

    def piped():
        for lc in launches:
            tide.stage_grads_bf16(plan, g_tab, slots, launch=lc)
            tide.reduce_scatter_bf16_fp32(plan, s_tab, out, launch=lc)
    pip = timed(piped)
    del slots, s_tab
    torch.cuda.empty_cache()
    return {"stage_kernel_ms": round(st_k, 4),
            "stage_kernel_GBps": round(stage_bytes / (st_k / 1e3) / 1e9, 1),
            "stage_runtime_copy_ms": round(st_s, 4),
            "stage_runtime_copy_GBps": round(stage_bytes / (st_s / 1e3) / 1e9, 1),
            "stage_dma_engines_ms": round(st_d, 4),
            "stage_dma_engines_GBps": round(stage_bytes / (st_d / 1e3) / 1e9, 1),
            "stage_bytes": stage_bytes,
            "reduce_from_slots_ms": round(rd, 4),
            "stage_plus_reduce_ms": round(tot, 4),
            "stage_plus_reduce_pipelined_ms": round(pip, 4),
            "pipeline_rank_ranges": len(ranges),
            "in_place_reduce_ms": round(in_place_ms, 4),
            "slot_reuse_over_in_place": round(tot / in_place_ms, 3)}


class Group:
    """One parameter group's inputs and outputs on the GPU, the pointer tables
    marshalled once (the buffers persist across steps, as FSDP's do)."""

    def __init__(self, torch, tide, cfg):
        from workloads import device_grads, device_rank_major_bits
        self.cfg = cfg
        self.plan = tide.plan_create(cfg.shapes, cfg.N, cfg.L)
        S = self.plan.S
        self.grads = device_grads(cfg.shapes, cfg.L, seed=cfg.seed, sigma=cfg.sigma,
                                  outlier_frac=cfg.outlier_frac,
                                  progress=lambda c: log("bench: %s: contributor %d of %d drawn"
                                                         % (cfg.name, c + 1, cfg.L)))
        self.out = torch.empty(cfg.N * S, dtype=torch.float32, device="cuda")
        self.shards = device_rank_major_bits(cfg.N * S, seed=1)
        self.params = [torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
                       for t, k in cfg.shapes]
        self.rs_bytes, self.ag_bytes, self.valid = group_bytes(cfg, S)
        self.g_tab = tide.grads_table(self.plan, self.grads)
        self.p_tab = tide.params_table(self.plan, self.params)
        torch.cuda.synchronize()

    def free(self, torch):
        for name in ("grads", "out", "shards", "params", "g_tab", "p_tab"):
            setattr(self, name, None)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def time_steps(torch, tide, grp, launch, steps, warmup, engine="kernel"):
    """`warmup` untimed steps, then `steps` timed ones; one step = reduce-scatter
    then placement on the current stream. HIP events on that stream bracket
    each part of each step; the wall clock brackets all timed steps."""
    stream = torch.cuda.current_stream()
    plan = grp.plan

    def step(ev):
        ev[0].record(stream)
        tide.reduce_scatter_bf16_fp32(plan, grp.g_tab, grp.out, stream=stream, launch=launch)
        ev[1].record(stream)
        tide.allgather_place(plan, grp.shards, grp.p_tab, stream=stream, launch=launch,
                             engine=engine)
        ev[2].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(warmup + steps)]
    for i in range(warmup):
        step(evs[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[warmup + i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    timed = evs[warmup:]
    rs = [a.elapsed_time(b) for a, b, _ in timed]
    ag = [b.elapsed_time(c) for _, b, c in timed]
    st = [a.elapsed_time(c) for a, _, c in timed]
    tot = grp.rs_bytes + grp.ag_bytes
    return {
        "step_ms_median": statistics.median(st), "step_ms_wall_mean": wall,
        "reduce_ms_mean": statistics.mean(rs), "reduce_ms_median": statistics.median(rs),
        "reduce_ms_min": min(rs), "placement_ms_mean": statistics.mean(ag),
        "placement_ms_median": statistics.median(ag),
        "GBps": tot / (statistics.median(st) / 1e3) / 1e9,
        "reduce_GBps": grp.rs_bytes / (statistics.median(rs) / 1e3) / 1e9,
        "reduce_GBps_mean": grp.rs_bytes / (statistics.mean(rs) / 1e3) / 1e9,
        "placement_GBps": grp.ag_bytes / (statistics.median(ag) / 1e3) / 1e9,
    }


def offset_rates(torch, tide, grp, offsets=(0, 1, 2, 3), reps=8):
    """Reduce rate with every gradient moved to `off` bf16 elements past an
    allocation's start (2 mod 4 bytes for odd `off`: the realigning loads),
    and whether each output equals the aligned call's bit for bit. One copy
    of the gradients is held at a time."""
    plan = grp.plan
    tide.reduce_scatter_bf16_fp32(plan, grp.g_tab, grp.out)
    ref = grp.out.clone()
    res = {}
    for off in offsets:
        views = []
        for c in range(grp.cfg.L):
            row = []
            for p, (t, k) in enumerate(grp.cfg.shapes):
                buf = torch.empty(t * k + 8, dtype=torch.bfloat16, device="cuda")
                v = buf[off:off + t * k].view(t, k)
                v.copy_(grp.grads[c][p])
                row.append(v)
            views.append(row)
        tab = tide.grads_table(plan, views)
        grp.out.fill_(float("nan"))
        tide.reduce_scatter_bf16_fp32(plan, tab, grp.out)
        torch.cuda.synchronize()
        same = bool(torch.equal(grp.out.view(torch.int32), ref.view(torch.int32)))
        ts = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            tide.reduce_scatter_bf16_fp32(plan, tab, grp.out)
            e[1].record()
            torch.cuda.synchronize()
            ts.append(e[0].elapsed_time(e[1]))
        ms = statistics.median(ts)
        res["+%d" % off] = {"reduce_ms_median": round(ms, 4),
                            "reduce_GBps": round(grp.rs_bytes / (ms / 1e3) / 1e9, 1),
                            "equals_aligned_output": same}
        log("bench: gradients at +%d elements: %s" % (off, json.dumps(res["+%d" % off])))
        del views, tab
        torch.cuda.empty_cache()
    return res


def one_gpu_share(torch, tide, grp, reps=10):
    """The reduce one GPU of an L-GPU node runs: its N / L ranks (here ranks
    [0, N / L)), full grid, median of `reps` calls between HIP events on the
    stream. (The placement is the whole group on every GPU, as in the step.)"""
    cfg, plan = grp.cfg, grp.plan
    share = max(1, cfg.N // cfg.L)
    launch = tide.Launch(rank_begin=0, rank_end=share)
    valid = sum(min(t * k, share * plan.param(p)[3]) for p, (t, k) in enumerate(cfg.shapes))
    nbytes = 2 * cfg.L * valid + 4 * share * plan.S
    tide.reduce_scatter_bf16_fp32(plan, grp.g_tab, grp.out, launch=launch)
    ts = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        tide.reduce_scatter_bf16_fp32(plan, grp.g_tab, grp.out, launch=launch)
        e[1].record()
        torch.cuda.synchronize()
        ts.append(e[0].elapsed_time(e[1]))
    ms = statistics.median(ts)
    return {"ranks": [0, share], "reduce_bytes": nbytes, "reduce_ms_median": round(ms, 4),
            "reduce_GBps": round(nbytes / (ms / 1e3) / 1e9, 1)}


def sdma_placement(torch, tide, grp, reps=3):
    """Host wall time of the placement on the DMA engines (the call returns
    once its copies are done; median of `reps` calls)."""
    tide.allgather_place(grp.plan, grp.shards, grp.p_tab, engine="sdma")
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tide.allgather_place(grp.plan, grp.shards, grp.p_tab, engine="sdma")
        ts.append(time.perf_counter() - t0)
    ms = statistics.median(ts) * 1e3
    return {"ms": round(ms, 3), "GBps": round(grp.ag_bytes / (ms / 1e3) / 1e9, 1),
            "engines": tide.dma_engine_count(torch.cuda.current_device())}


def per_config_line(torch, tide, orc, name, args, pair):
    from oracle import check as oracle_check
    """Full-grid step, SDMA placement and the whole-output oracle check of one
    more group; for the Wan2.2 block also the budgeted GEMM-victim protocol."""
    from workloads.configs import CONFIGS
    cfg = CONFIGS[name]
    log("bench: per-config %s: generating inputs" % name)
    grp = Group(torch, tide, cfg)
    t = time_steps(torch, tide, grp, tide.Launch(), args.steps, args.warmup)
    res = {"GBps": round(t["GBps"], 1), "pct_of_8TBps": round(100.0 * t["GBps"] / HBM_PEAK_GBPS, 2),
           "step_ms_median": round(t["step_ms_median"], 4),
           "reduce_GBps": round(t["reduce_GBps"], 1),
           "reduce_frac_by_mean": round(t["reduce_GBps_mean"] / HBM_PEAK_GBPS, 4),
           "placement_GBps": round(t["placement_GBps"], 1),
           "bytes_per_step": grp.rs_bytes + grp.ag_bytes}
    log("bench: per-config %s: %.1f GB/s fused, reduce %.1f, placement %.1f"
        % (name, t["GBps"], t["reduce_GBps"], t["placement_GBps"]))
    res["placement_sdma"] = sdma_placement(torch, tide, grp)
    if name == "wan22_dit_block":
        log("bench: per-config %s: GEMM victim" % name)
        res["victim_gemm_256x8192x8192"] = {
            "budgeted_16_4": victim_slowdown(torch, tide, grp.plan, grp.grads, grp.out, grp.shards,
                                             grp.params, tide.budgeted(), pair),
            "full_grid": victim_slowdown(torch, tide, grp.plan, grp.grads, grp.out, grp.shards,
                                         grp.params, tide.Launch(), pair)}
    if orc is not None:
        # The step's outputs are re-made with the kernel engine before the check.
        tide.reduce_scatter_bf16_fp32(grp.plan, grp.g_tab, grp.out)
        tide.allgather_place(grp.plan, grp.shards, grp.p_tab)
        torch.cuda.synchronize()
        log("bench: per-config %s: whole output vs the oracle" % name)
        chk = oracle_check.whole_output(orc, cfg, grp.plan.S, grp.grads, grp.out, grp.shards,
                                        grp.params)
        res["oracle_bit_exact"] = chk["reduce_scatter_bit_exact"] and chk["placement_bit_exact"]
        if chk["first_mismatch"]:
            res["first_mismatch"] = chk["first_mismatch"]
    grp.free(torch)
    log("bench: per-config %s: %s" % (name, json.dumps(res)))
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="padding_stress",
                    choices=["llama70b_layer", "qwen3_moe_layer", "padding_stress", "wan22_dit_block"])
    ap.add_argument("--mode", default="full", choices=["full", "budgeted"])
    ap.add_argument("--placement-engine", default="kernel", choices=["kernel", "sdma", "runtime"],
                    help="engine of the placement in the timed step (default: the kernel)")
    ap.add_argument("--parts", action="store_true",
                    help="also time the runtime-copy placement, the stage placement and the "
                         "landing sum")
    ap.add_argument("--victim", action="store_true",
                    help="GEMM-victim slowdown of this workload, budgeted and full grid")
    ap.add_argument("--stock", action="store_true",
                    help="also time the stock FSDP2 path (chunk_cat pack + sum, split_with_sizes_copy)")
    ap.add_argument("--slot-reuse", action="store_true",
                    help="also time the Slot-Reuse staging and the reduce reading the slots")
    ap.add_argument("--fence-study", action="store_true",
                    help="GEMM-victim slowdown for budgeted variants (LDS fence on/off, shorter "
                         "launches) with a half-GPU and a full-GPU victim")
    ap.add_argument("--occupancy", action="store_true",
                    help="trace where budgeted workgroups run, beside GEMM-shaped occupants")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step as prepared calls, eager and replayed from a HIP graph")
    ap.add_argument("--offsets", action="store_true",
                    help="also time the reduce with all gradients at 0-3 elements past an "
                         "allocation's start")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (timing and whole-output checks)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other large groups (Llama, Qwen, Wan and the Wan GEMM victim)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark runs on one GPU only (it measures one GPU's share of "
              "the collective); --gpus %d is not supported." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import mixed_precision_rs_amd as tide
    from workloads.configs import CONFIGS

    cfg = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    log("bench: %s, generating inputs" % cfg.name)
    grp = Group(torch, tide, cfg)
    plan, grads, out, shards, params = grp.plan, grp.grads, grp.out, grp.shards, grp.params
    g_tab, p_tab = grp.g_tab, grp.p_tab
    rs_bytes, ag_bytes, valid = grp.rs_bytes, grp.ag_bytes, grp.valid
    S = plan.S
    launch = tide.Launch() if args.mode == "full" else tide.budgeted()

    log("bench: %d warmup + %d timed steps" % (args.warmup, args.steps))
    t = time_steps(torch, tide, grp, launch, args.steps, args.warmup, engine=args.placement_engine)
    value = t["GBps"]
    achieved = t["reduce_GBps_mean"]
    rs_avg, ag_avg = t["reduce_ms_mean"], t["placement_ms_mean"]
    log("bench: %.3f ms/step (median), %.1f GB/s; reduce %.3f ms mean (%.1f GB/s), placement "
        "%.3f ms mean; wall %.3f ms/step"
        % (t["step_ms_median"], value, rs_avg, achieved, ag_avg, t["step_ms_wall_mean"]))

    parts = {
        "step_ms_wall_mean": round(t["step_ms_wall_mean"], 4),
        "GBps_by_wall_mean": round((rs_bytes + ag_bytes) / (t["step_ms_wall_mean"] / 1e3) / 1e9, 1),
        "reduce_ms_mean": round(rs_avg, 4), "reduce_ms_median": round(t["reduce_ms_median"], 4),
        "reduce_ms_min": round(t["reduce_ms_min"], 4),
        "placement_ms_mean": round(ag_avg, 4),
        "placement_ms_median": round(t["placement_ms_median"], 4),
        "reduce_GBps": round(t["reduce_GBps"], 1),
        "placement_GBps": round(t["placement_GBps"], 1),
        "reduce_bytes": rs_bytes, "placement_bytes": ag_bytes,
        "pct_of_8TBps": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "reduce_launches_per_call": plan.launch_count(0, launch),
        "placement_launches_per_call": plan.launch_count(1, launch),
    }
    parts["one_gpu_share"] = one_gpu_share(torch, tide, grp)
    log("bench: one GPU's share %s" % json.dumps(parts["one_gpu_share"]))
    if args.placement_engine != "sdma":
        parts["placement_sdma"] = sdma_placement(torch, tide, grp)
        log("bench: SDMA placement %s" % json.dumps(parts["placement_sdma"]))
    if args.parts:
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        tide.allgather_place(plan, shards, params, engine="runtime")
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(5):
            tide.allgather_place(plan, shards, params, engine="runtime")
        e[1].record()
        torch.cuda.synchronize()
        sd = e[0].elapsed_time(e[1]) / 5
        # Placement from a recursive-doubling stage buffer (rotated by half the ranks).
        e2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        tide.allgather_place_stage(plan, shards, cfg.N // 2, p_tab)
        torch.cuda.synchronize()
        e2[0].record()
        for _ in range(5):
            tide.allgather_place_stage(plan, shards, cfg.N // 2, p_tab)
        e2[1].record()
        torch.cuda.synchronize()
        st = e2[0].elapsed_time(e2[1]) / 5
        parts["placement_stage_rotated_GBps"] = round(ag_bytes / (st / 1e3) / 1e9, 1)
        # Level-2 landing sum of one node (M = L source partials of this
        # group's shard size): M * L * S * 4 bytes read, L * S * 4 written.
        Lg = Mg = cfg.L
        Cg = -(-S // Lg)
        inb = [torch.empty(Lg * Lg * Cg, dtype=torch.float32, device="cuda").normal_()
               for _ in range(Lg)]
        shd = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(Lg)]
        tide.landing_sum_fp32(Lg, Mg, S, inb, shd)
        torch.cuda.synchronize()
        e3 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e3[0].record()
        for _ in range(5):
            tide.landing_sum_fp32(Lg, Mg, S, inb, shd)
        e3[1].record()
        torch.cuda.synchronize()
        lt = e3[0].elapsed_time(e3[1]) / 5
        lb = (Mg * Lg * S + Lg * S) * 4
        parts["landing_ms"] = round(lt, 4)
        parts["landing_GBps"] = round(lb / (lt / 1e3) / 1e9, 1)
        del inb, shd
        parts["placement_runtime_copy_ms"] = round(sd, 4)
        parts["placement_runtime_copy_GBps"] = round(ag_bytes / (sd / 1e3) / 1e9, 1)
        log("bench: runtime-copy placement %.3f ms" % sd)
    # Practical ceilings in the same run, from the library's streaming kernels.
    parts["ceilings"] = ceilings(torch, tide)
    parts["ceilings"]["reduce_over_its_pattern"] = round(
        t["reduce_GBps_mean"] / parts["ceilings"]["reduce_pattern_GBps"], 4)
    log("bench: ceilings %s" % json.dumps(parts["ceilings"]))

    # Two side streams, a GEMM (or occupant) stream and a collective stream,
    # checked to run concurrently before every measurement that needs them.
    pair = SidePair(torch, tide)
    parts["side_streams_concurrent"] = pair.concurrent
    graph = None
    if args.graph:
        log("bench: prepared calls and graph replay")
        graph = graph_parts(torch, tide, plan, g_tab, out, shards, p_tab, rs_bytes, ag_bytes)
        log("bench: graph %s" % json.dumps(graph))

    occ = None
    if args.occupancy:
        log("bench: occupancy probe")
        occ = occupancy_probe(torch, tide, plan, grads, out, shards, params, pair)
        log("bench: occupancy %s" % json.dumps(occ))

    slot = None
    if args.slot_reuse:
        log("bench: slot-reuse staging")
        slot = slot_reuse_parts(torch, tide, plan, cfg, g_tab, out, valid, rs_avg)
        log("bench: slot-reuse %s" % json.dumps(slot))

    stock = None
    if args.stock:
        log("bench: stock FSDP2 path")
        stock = stock_fsdp2(torch, tide, plan, cfg, grads, shards, out, p_tab)
        stock["reduce_speedup_of_ours"] = round(stock["reduce_ms"] / rs_avg, 2)
        stock["placement_speedup_of_ours"] = round(stock["placement_ms"] / ag_avg, 2)
        log("bench: stock %s" % json.dumps(stock))

    victim = None
    if args.victim:
        log("bench: GEMM victim, budgeted")
        victim = {"budgeted_16_4": victim_slowdown(torch, tide, plan, grads, out, shards, params,
                                                   tide.budgeted(), pair),
                  "budgeted_16_4_without_lds_reservation": victim_slowdown(
                      torch, tide, plan, grads, out, shards, params,
                      tide.budgeted(flags=tide.FLAG_NO_LDS_FENCE), pair),
                  "full_grid": victim_slowdown(torch, tide, plan, grads, out, shards, params,
                                               tide.Launch(), pair)}
        log("bench: victim %s" % json.dumps(victim))

    offs = None
    if args.offsets:
        log("bench: gradient offsets")
        offs = offset_rates(torch, tide, grp)

    fence = None
    if args.fence_study:
        fence = fence_study(torch, tide, plan, grads, out, shards, params, pair)
        log("bench: fence study %s" % json.dumps(fence))

    cpu = None
    orc = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.load()
        # The outputs of one full-grid step with the kernel engine are checked.
        tide.reduce_scatter_bf16_fp32(plan, g_tab, out)
        tide.allgather_place(plan, shards, p_tab)
        torch.cuda.synchronize()
        log("bench: whole output vs the CPU oracle, all %d ranks" % cfg.N)
        from oracle import check as oracle_check
        chk = oracle_check.whole_output(orc, cfg, plan.S, grads, out, shards, params,
                                        one_thread_reps=3)
        cpu = cpu_baseline(chk, cfg)
        if chk["first_mismatch"]:
            cpu["first_mismatch"] = chk["first_mismatch"]
        log("bench: cpu %s" % json.dumps(cpu))
    del grads, out, shards, params, g_tab, p_tab
    grp.free(torch)

    per_config = None
    if not args.no_per_config:
        per_config = {}
        for name in ("llama70b_layer", "qwen3_moe_layer", "wan22_dit_block"):
            if name != cfg.name:
                per_config[name] = per_config_line(torch, tide, orc, name, args, pair)
        per_config["all_at_least_70pct"] = all(
            v["pct_of_8TBps"] >= 70.0 for v in per_config.values() if isinstance(v, dict)) and \
            100.0 * value / HBM_PEAK_GBPS >= 70.0
        wv = per_config.get("wan22_dit_block", {}).get("victim_gemm_256x8192x8192")
        if wv and "slowdown_pct" in wv["budgeted_16_4"]:
            per_config["wan22_budgeted_gemm_slowdown_pct"] = wv["budgeted_16_4"]["slowdown_pct"]
            per_config["wan22_victim_streams_concurrent"] = wv["budgeted_16_4"]["streams_concurrent"]
        if orc is not None:
            per_config["all_oracle_bit_exact"] = all(
                v.get("oracle_bit_exact", False) for v in per_config.values() if isinstance(v, dict))

    parts["side_stream_pairs_made"] = pair.pairs_made
    traffic = counter_traffic(cfg.name)
    clocks = gpu_clocks()
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["step_ms_median"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "params": len(cfg.shapes), "N": cfg.N, "L": cfg.L,
                   "S": S, "valid_elements": valid, "bytes_per_step": rs_bytes + ag_bytes,
                   "launch": args.mode, "placement_engine": args.placement_engine,
                   "statistic": "median of the per-step times (HIP events on the stream)",
                   "inputs": "bf16 grads %s, seeded on device" % (
                       "N(0,%g)" % cfg.sigma + (" + %g outliers" % cfg.outlier_frac
                                                if cfg.outlier_frac else ""))},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "reduce_kernel<%d>" % cfg.L},
        "cpu_baseline": cpu,
        "parts": parts,
        "per_config": per_config,
        "gpu_clocks_after_run": clocks,
    }
    if victim is not None:
        line["victim_gemm_256x8192x8192"] = victim
    if stock is not None:
        line["stock_fsdp2_same_gpu"] = stock
    if slot is not None:
        line["slot_reuse"] = slot
    if occ is not None:
        line["occupancy_probe"] = occ
    if fence is not None:
        line["fence_study"] = fence
    if offs is not None:
        line["gradient_offsets"] = offs
    if graph is not None:
        line["prepared_and_graph"] = graph
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
