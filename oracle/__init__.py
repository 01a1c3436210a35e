"""CPU oracle of TIDE's level-1 mixed-precision reduce-scatter and all-gather
placement (ctypes wrapper around tide_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and by
the benchmark's CPU-baseline leg, never by the library. It shares no code with
the HIP path. Every function below takes the group as a list of (T_p, K_p)
shapes and re-derives the layout in C.
"""
import ctypes
import os
import time
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import build as _build

_I64P = ctypes.POINTER(ctypes.c_int64)
_U16P = ctypes.POINTER(ctypes.c_uint16)
_U32P = ctypes.POINTER(ctypes.c_uint32)
_F32P = ctypes.POINTER(ctypes.c_float)


class Oracle:
    """Handle on one build of the oracle library (the default build, or a
    variant compiled by a test from modified source)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        lib.oracle_layout.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                      _I64P, _I64P, _I64P, _I64P]
        lib.oracle_piece_start.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, _I64P, _I64P, _I64P]
        lib.oracle_reduce_scatter.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.POINTER(_U16P), _F32P,
                                              ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              _U32P]
        lib.oracle_piece_rows.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, _I64P, _I64P]
        lib.oracle_reduce_piece.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(_U16P), _F32P]
        lib.oracle_allgather_place.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                               _U16P, ctypes.c_int64, ctypes.POINTER(_U16P),
                                               ctypes.c_int32, ctypes.c_int32,
                                               ctypes.POINTER(_U32P)]
        lib.oracle_allgather_place_stage.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                                     _U16P, ctypes.c_int64, ctypes.c_int32,
                                                     ctypes.POINTER(_U16P), ctypes.c_int32,
                                                     ctypes.c_int32]
        lib.oracle_landing_sum.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                           ctypes.POINTER(_F32P), ctypes.POINTER(_F32P),
                                           ctypes.c_int32]
        lib.oracle_latin_square.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32)]
        lib.oracle_stage_grads.argtypes = [ctypes.c_int32, _I64P, _I64P, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(_U16P),
                                           ctypes.POINTER(_U16P)]
        for f in ("oracle_layout", "oracle_piece_start", "oracle_reduce_scatter",
                  "oracle_piece_rows", "oracle_reduce_piece", "oracle_allgather_place",
                  "oracle_allgather_place_stage", "oracle_landing_sum", "oracle_latin_square",
                  "oracle_stage_grads"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path
        self.last_call_s = 0.0     # wall time of the last C compute call alone

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _shape_arrays(shapes: Sequence[Tuple[int, int]]):
        rows = np.ascontiguousarray([t for t, _ in shapes], dtype=np.int64)
        rlen = np.ascontiguousarray([k for _, k in shapes], dtype=np.int64)
        if rows.size == 0:
            rows = np.zeros(1, np.int64)[:0]
            rlen = np.zeros(1, np.int64)[:0]
        return rows, rlen

    @staticmethod
    def _p(a, t):
        return a.ctypes.data_as(t)

    # -- layout --------------------------------------------------------------
    def layout(self, shapes, N):
        """Return dict with arrays R, s, o (per parameter) and S."""
        rows, rlen = self._shape_arrays(shapes)
        P = len(shapes)
        R = np.zeros(max(P, 1), np.int64)
        s = np.zeros(max(P, 1), np.int64)
        o = np.zeros(max(P, 1), np.int64)
        S = ctypes.c_int64(0)
        rc = self.lib.oracle_layout(P, self._p(rows, _I64P), self._p(rlen, _I64P), N,
                                    self._p(R, _I64P), self._p(s, _I64P), self._p(o, _I64P),
                                    ctypes.byref(S))
        if rc != 0:
            raise ValueError("oracle_layout rejected the group")
        return {"R": R[:P], "s": s[:P], "o": o[:P], "S": int(S.value)}

    def piece_start(self, shapes, N, r, p):
        rows, rlen = self._shape_arrays(shapes)
        a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        rc = self.lib.oracle_piece_start(len(shapes), self._p(rows, _I64P), self._p(rlen, _I64P),
                                         N, r, p, ctypes.byref(a), ctypes.byref(b),
                                         ctypes.byref(c))
        if rc != 0:
            raise ValueError("oracle_piece_start rejected its arguments")
        return int(a.value), int(b.value), int(c.value)

    def piece_rows(self, shapes, N, r, p):
        rows, rlen = self._shape_arrays(shapes)
        a, b = ctypes.c_int64(), ctypes.c_int64()
        rc = self.lib.oracle_piece_rows(len(shapes), self._p(rows, _I64P), self._p(rlen, _I64P),
                                        N, r, p, ctypes.byref(a), ctypes.byref(b))
        if rc != 0:
            raise ValueError("oracle_piece_rows rejected its arguments")
        return int(a.value), int(b.value)

    # -- reduce-scatter ------------------------------------------------------
    def reduce_scatter(self, shapes, N, L, grads: List[List[np.ndarray]],
                       out_stride: Optional[int] = None, rank_range=None,
                       out: Optional[np.ndarray] = None, count_writes=False):
        """grads[c][p]: flat uint16 bf16 bits. Returns out as (N, out_stride)
        float32 (and the per-element write counts if count_writes)."""
        rows, rlen = self._shape_arrays(shapes)
        P = len(shapes)
        S = self.layout(shapes, N)["S"]
        stride = S if out_stride is None else out_stride
        rb, re = (0, N) if rank_range is None else rank_range
        if out is None:
            out = np.full(N * stride, np.nan, dtype=np.float32)
        arrs = [np.ascontiguousarray(grads[c][p], dtype=np.uint16)
                for c in range(L) for p in range(P)]
        ptrs = (_U16P * max(len(arrs), 1))(*[self._p(a, _U16P) for a in arrs])
        counts = np.zeros(N * stride, np.uint32) if count_writes else None
        t0 = time.perf_counter()
        rc = self.lib.oracle_reduce_scatter(
            P, self._p(rows, _I64P), self._p(rlen, _I64P), N, L, ptrs,
            self._p(out, _F32P), stride, rb, re,
            self._p(counts, _U32P) if counts is not None else None)
        self.last_call_s = time.perf_counter() - t0
        if rc != 0:
            raise ValueError("oracle_reduce_scatter rejected its arguments")
        out2 = out.reshape(N, stride) if stride > 0 else out.reshape(N, 0)
        if count_writes:
            return out2, counts.reshape(N, stride)
        return out2

    def reduce_scatter_rows(self, shapes, N, L, grads_rows: List[List[np.ndarray]],
                            rank_range: Tuple[int, int], out_rows: np.ndarray):
        """reduce_scatter over ranks [rb, re) from inputs that hold only those
        ranks' rows, so a very large group can be checked range by range with
        bounded host memory. grads_rows[c][p] holds rows
        [rb * R_p, min(T_p, re * R_p)) of contributor c's gradient (flat uint16);
        out_rows (float32, (re - rb) * S elements) receives shards rb .. re - 1.
        The unchanged C routine is called with every base pointer moved back by
        the rows (and shards) the arrays leave out, so its own indexing, which
        only touches rows and shards of the range, lands inside them."""
        rows, rlen = self._shape_arrays(shapes)
        P = len(shapes)
        lay = self.layout(shapes, N)
        S = lay["S"]
        rb, re = rank_range
        if not (0 <= rb <= re <= N) or out_rows.dtype != np.float32 or \
                out_rows.size < (re - rb) * S or not out_rows.flags.c_contiguous:
            raise ValueError("reduce_scatter_rows: bad range or output")
        keep, ptrs = [], []
        for c in range(L):
            for p in range(P):
                t, k = shapes[p]
                first = min(t, rb * int(lay["R"][p]))
                a = np.ascontiguousarray(grads_rows[c][p], dtype=np.uint16)
                if a.size != (min(t, re * int(lay["R"][p])) - first) * k:
                    raise ValueError("grads_rows[%d][%d] holds %d elements" % (c, p, a.size))
                keep.append(a)
                ptrs.append(a.ctypes.data - first * k * 2 if a.size else 0)
        parr = (_U16P * max(len(ptrs), 1))(*[ctypes.cast(ctypes.c_void_p(x), _U16P)
                                              for x in ptrs])
        out_base = ctypes.cast(ctypes.c_void_p(out_rows.ctypes.data - rb * S * 4), _F32P)
        t0 = time.perf_counter()
        rc = self.lib.oracle_reduce_scatter(P, self._p(rows, _I64P), self._p(rlen, _I64P), N, L,
                                            parr, out_base, S, rb, re, None)
        self.last_call_s = time.perf_counter() - t0
        if rc != 0:
            raise ValueError("oracle_reduce_scatter rejected its arguments")
        return out_rows

    def allgather_place_rows(self, shapes, N, shards_rows: np.ndarray,
                             rank_range: Tuple[int, int], params_rows: List[np.ndarray]):
        """allgather_place over ranks [rb, re) with only those ranks' data in
        memory: shards_rows holds shards rb .. re - 1 ((re - rb) * S uint16,
        stride S); params_rows[p] receives rows [rb * R_p, min(T_p, re * R_p))
        of parameter p. Base pointers are moved back as in reduce_scatter_rows."""
        rows, rlen = self._shape_arrays(shapes)
        P = len(shapes)
        lay = self.layout(shapes, N)
        S = lay["S"]
        rb, re = rank_range
        shards_rows = np.ascontiguousarray(shards_rows, dtype=np.uint16)
        if not (0 <= rb <= re <= N) or shards_rows.size < (re - rb) * S:
            raise ValueError("allgather_place_rows: bad range or shards")
        ptrs = []
        for p in range(P):
            t, k = shapes[p]
            first = min(t, rb * int(lay["R"][p]))
            a = params_rows[p]
            if a.dtype != np.uint16 or not a.flags.c_contiguous or \
                    a.size != (min(t, re * int(lay["R"][p])) - first) * k:
                raise ValueError("params_rows[%d] has the wrong size or type" % p)
            ptrs.append(a.ctypes.data - first * k * 2 if a.size else 0)
        parr = (_U16P * max(P, 1))(*[ctypes.cast(ctypes.c_void_p(x), _U16P) for x in ptrs])
        sh_base = ctypes.cast(ctypes.c_void_p(shards_rows.ctypes.data - rb * S * 2), _U16P)
        t0 = time.perf_counter()
        rc = self.lib.oracle_allgather_place(P, self._p(rows, _I64P), self._p(rlen, _I64P), N,
                                             sh_base, S, parr, rb, re, None)
        self.last_call_s = time.perf_counter() - t0
        if rc != 0:
            raise ValueError("oracle_allgather_place rejected its arguments")
        return params_rows

    def reduce_piece(self, shapes, N, L, r, p, rank_rows: List[np.ndarray]) -> np.ndarray:
        rows, rlen = self._shape_arrays(shapes)
        lay = self.layout(shapes, N)
        dst = np.empty(int(lay["s"][p]), np.float32)
        arrs = [np.ascontiguousarray(a, dtype=np.uint16) for a in rank_rows]
        ptrs = (_U16P * L)(*[self._p(a, _U16P) for a in arrs])
        rc = self.lib.oracle_reduce_piece(len(shapes), self._p(rows, _I64P),
                                          self._p(rlen, _I64P), N, L, r, p, ptrs,
                                          self._p(dst, _F32P))
        if rc != 0:
            raise ValueError("oracle_reduce_piece rejected its arguments")
        return dst

    # -- all-gather placement ------------------------------------------------
    def allgather_place(self, shapes, N, shards: np.ndarray, shard_stride=None,
                        rank_range=None, params: Optional[List[np.ndarray]] = None,
                        count_writes=False):
        """shards: flat uint16 rank-major buffer (N * shard_stride). Returns the
        list of flat uint16 parameter arrays (and write counts if asked)."""
        rows, rlen = self._shape_arrays(shapes)
        P = len(shapes)
        S = self.layout(shapes, N)["S"]
        stride = S if shard_stride is None else shard_stride
        rb, re = (0, N) if rank_range is None else rank_range
        shards = np.ascontiguousarray(shards, dtype=np.uint16)
        if params is None:
            params = [np.zeros(t * k, np.uint16) for t, k in shapes]
        pp = (_U16P * max(P, 1))(*[self._p(a, _U16P) for a in params])
        counts = [np.zeros(t * k, np.uint32) for t, k in shapes] if count_writes else None
        cp = (_U32P * max(P, 1))(*[self._p(a, _U32P) for a in counts]) if counts else None
        t0 = time.perf_counter()
        rc = self.lib.oracle_allgather_place(
            P, self._p(rows, _I64P), self._p(rlen, _I64P), N, self._p(shards, _U16P),
            stride, pp, rb, re, cp)
        self.last_call_s = time.perf_counter() - t0
        if rc != 0:
            raise ValueError("oracle_allgather_place rejected its arguments")
        if count_writes:
            return params, counts
        return params


    def allgather_place_stage(self, shapes, N, stage: np.ndarray, first_rank: int,
                              shard_stride=None, rank_range=None,
                              params: Optional[List[np.ndarray]] = None):
        """Placement from a stage buffer whose position k holds rank
        (first_rank + k) mod N."""
        rows, rlen = self._shape_arrays(shapes)
        P = len(shapes)
        S = self.layout(shapes, N)["S"]
        stride = S if shard_stride is None else shard_stride
        rb, re = (0, N) if rank_range is None else rank_range
        stage = np.ascontiguousarray(stage, dtype=np.uint16)
        if params is None:
            params = [np.zeros(t * k, np.uint16) for t, k in shapes]
        pp = (_U16P * max(P, 1))(*[self._p(a, _U16P) for a in params])
        rc = self.lib.oracle_allgather_place_stage(
            P, self._p(rows, _I64P), self._p(rlen, _I64P), N, self._p(stage, _U16P), stride,
            first_rank, pp, rb, re)
        if rc != 0:
            raise ValueError("oracle_allgather_place_stage rejected its arguments")
        return params


    def landing_sum(self, L, M, S, inboxes: List[np.ndarray], shards=None, accumulate=False):
        """inboxes[g]: float32 arrays of L*L*ceil(S/L); returns the L shards."""
        ib = [np.ascontiguousarray(a, dtype=np.float32) for a in inboxes]
        if shards is None:
            shards = [np.zeros(S, np.float32) for _ in range(L)]
        ip = (_F32P * L)(*[self._p(a, _F32P) for a in ib])
        sp = (_F32P * L)(*[self._p(a, _F32P) for a in shards])
        t0 = time.perf_counter()
        rc = self.lib.oracle_landing_sum(L, M, S, ip, sp, 1 if accumulate else 0)
        self.last_call_s = time.perf_counter() - t0
        if rc != 0:
            raise ValueError("oracle_landing_sum rejected its arguments")
        return shards

    def stage_grads(self, shapes, N, L, grads, slots: Optional[List[np.ndarray]] = None,
                    rank_range: Optional[Tuple[int, int]] = None):
        """Slot-Reuse staging of contributors' bf16 gradients (grads[c][p], uint16
        bits) into L slots of N * S elements (zero-filled when not given);
        returns the slots. rank_range limits the copy to those ranks' rows."""
        rows, rlen = self._shape_arrays(shapes)
        P = len(shapes)
        S = self.layout(shapes, N)["S"]
        if slots is None:
            slots = [np.zeros(N * S, np.uint16) for _ in range(L)]
        if len(slots) != L or any(a.dtype != np.uint16 or a.size < N * S for a in slots):
            raise ValueError("stage_grads needs L uint16 slots of at least N * S elements")
        arrs = [np.ascontiguousarray(grads[c][p], dtype=np.uint16)
                for c in range(L) for p in range(P)]
        gp = (_U16P * max(len(arrs), 1))(*[self._p(a, _U16P) for a in arrs])
        sp = (_U16P * L)(*[self._p(a, _U16P) for a in slots])
        rb, re = rank_range if rank_range is not None else (0, N)
        t0 = time.perf_counter()
        rc = self.lib.oracle_stage_grads(P, self._p(rows, _I64P), self._p(rlen, _I64P), N, L,
                                         rb, re, gp, sp)
        self.last_call_s = time.perf_counter() - t0
        if rc != 0:
            raise ValueError("oracle_stage_grads rejected its arguments")
        return slots

    def latin_square(self, M, L, dst, src):
        """(c, slice handled by each source GPU, destination GPU of each slice)."""
        c = ctypes.c_int32()
        a = (ctypes.c_int32 * L)()
        b = (ctypes.c_int32 * L)()
        rc = self.lib.oracle_latin_square(M, L, dst, src, ctypes.byref(c), a, b)
        if rc != 0:
            raise ValueError("oracle_latin_square rejected its arguments")
        return int(c.value), list(a), list(b)


_default: Optional[Oracle] = None


def load(rebuild: bool = False) -> Oracle:
    """The default oracle build (compiled on first use if missing)."""
    global _default
    if _default is None or rebuild:
        if rebuild or not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default
