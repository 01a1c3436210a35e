"""ctypes binding of libtide.so (declared in include/tide.h).

Argument marshalling only: every step of the reduce-scatter and of the
placement runs in the HIP library. PyTorch supplies device memory and streams.
The binding refuses to work without the built library; there is no fallback.
"""
import ctypes
import os
from typing import List, Optional, Sequence, Tuple, Union

HERE = os.path.dirname(os.path.abspath(__file__))
# TIDE_LIBRARY may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("TIDE_LIBRARY") or os.path.join(HERE, "libtide.so")

TIDE_OK = 0
STATUS_NAMES = {0: "TIDE_OK", 1: "TIDE_ERR_INVALID_ARG", 2: "TIDE_ERR_ALIGNMENT",
                3: "TIDE_ERR_OVERFLOW", 4: "TIDE_ERR_UNSUPPORTED", 5: "TIDE_ERR_NO_MEMORY",
                6: "TIDE_ERR_HIP"}
ENGINE_KERNEL = 0
ENGINE_RUNTIME = 1
ENGINE_SDMA = 2
ENGINES = {"kernel": 0, "runtime": 1, "sdma": 2}
LAUNCH_FULL = 0
LAUNCH_BUDGETED = 1
FLAG_SCALAR_PATH = 0x1
FLAG_NO_LDS_FENCE = 0x2

# Every symbol include/tide.h declares.
EXPORTS = ["tide_plan_create", "tide_plan_destroy", "tide_plan_dims", "tide_plan_param",
           "tide_plan_map", "tide_reduce_scatter_bf16_fp32", "tide_allgather_place",
           "tide_plan_launch_count", "tide_status_string", "tide_last_error_detail",
           "tide_version", "tide_allgather_place_stage", "tide_rd_schedule",
           "tide_landing_sum_fp32", "tide_latin_square", "tide_stage_grads_bf16",
           "tide_plan_trace_records", "tide_landing_trace_records", "tide_diag_occupy",
           "tide_plan_event_count", "tide_prepare_reduce_scatter_bf16_fp32",
           "tide_prepare_allgather_place_stage", "tide_prepare_stage_grads_bf16",
           "tide_call_enqueue", "tide_call_destroy", "tide_plan_slot_grads",
           "tide_dma_engine_count", "tide_reduce_scatter_bf16_fp32_noalloc", "tide_diag_stream"]


class TideError(RuntimeError):
    def __init__(self, status: int, detail: str, call: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, "TIDE_ERR_%d" % status)
        self.detail = detail
        super().__init__("%s failed: %s: %s" % (call, self.status_name, detail))


class RdStep(ctypes.Structure):
    """tide_rd_step."""
    _fields_ = [("round", ctypes.c_int32), ("send_to", ctypes.c_int32),
                ("recv_from", ctypes.c_int32), ("count", ctypes.c_int32),
                ("send_slot", ctypes.c_int32), ("recv_slot", ctypes.c_int32),
                ("head_bytes", ctypes.c_int64), ("tail_bytes", ctypes.c_int64)]


class Launch(ctypes.Structure):
    """tide_launch. All-zero = full grid, all ranks. `trace` is a device
    address (see trace_buffer) or None."""
    _fields_ = [("mode", ctypes.c_int32), ("reduce_blocks", ctypes.c_int32),
                ("place_blocks", ctypes.c_int32), ("max_launch_us", ctypes.c_int32),
                ("rank_begin", ctypes.c_int32), ("rank_end", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("trace", ctypes.c_void_p), ("trace_capacity", ctypes.c_int64),
                ("write_counts", ctypes.c_void_p), ("write_counts_elems", ctypes.c_int64)]


TRACE_REC_BYTES = 24          # sizeof(tide_trace_rec)


def trace_buffer(records: int):
    """A zeroed device buffer for `records` tide_trace_rec entries (int64 x 3 each)."""
    import torch
    return torch.zeros(max(records, 1) * 3, dtype=torch.int64, device="cuda")


def traced(launch: Launch, buf, records: Optional[int] = None) -> Launch:
    """Copy of `launch` that writes its workgroup records into `buf`."""
    out = Launch()
    ctypes.pointer(out)[0] = launch
    cap = buf.numel() // 3
    if records is not None and int(records) > cap:
        raise ValueError("trace buffer holds %d records, %d requested" % (cap, int(records)))
    _tensor_arg(buf, "int64", "trace buffer")
    out.trace = _ptr(buf)
    out.trace_capacity = cap if records is None else int(records)
    return out


def counted(launch: Launch, counts) -> Launch:
    """Copy of `launch` that adds one per written element into `counts` (a
    zeroed int32 device tensor; see tide_launch.write_counts for the indices)."""
    out = Launch()
    ctypes.pointer(out)[0] = launch
    _tensor_arg(counts, "int32", "write counts")
    out.write_counts = _ptr(counts)
    out.write_counts_elems = counts.numel()
    return out


def decode_trace(buf, records: int):
    """Host copy of the first `records` entries: dict of numpy arrays
    (cu: a chip-wide CU key from XCC_ID and HW_ID's CU / shader-array /
    shader-engine fields; xcc; t_begin; t_end in real-time counter ticks)."""
    import numpy as np
    a = buf[: records * 3].view(-1, 3).cpu().numpy()
    w0 = a[:, 0].view(np.uint64)
    hw = (w0 & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    xcc = ((w0 >> np.uint64(32)) & np.uint64(0xF)).astype(np.uint32)
    cu = (xcc << np.uint32(8)) | ((hw >> np.uint32(8)) & np.uint32(0xFF))
    return {"cu": cu, "xcc": xcc, "hw_id": hw, "t_begin": a[:, 1].view(np.uint64),
            "t_end": a[:, 2].view(np.uint64)}


def budgeted(reduce_blocks=16, place_blocks=4, max_launch_us=50, **kw) -> Launch:
    return Launch(mode=LAUNCH_BUDGETED, reduce_blocks=reduce_blocks, place_blocks=place_blocks,
                  max_launch_us=max_launch_us, **kw)


_I64P = ctypes.POINTER(ctypes.c_int64)
_I32P = ctypes.POINTER(ctypes.c_int32)
_VPP = ctypes.POINTER(ctypes.c_void_p)
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libtide.so is not built (%s). Build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python mixed_precision_rs_amd/_build.py`." % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.tide_plan_create.argtypes = [_I64P, _I64P, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    lib.tide_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.tide_plan_destroy.restype = None
    lib.tide_plan_dims.argtypes = [ctypes.c_void_p, _I32P, _I32P, _I32P, _I64P]
    lib.tide_plan_param.argtypes = [ctypes.c_void_p, ctypes.c_int32, _I64P, _I64P, _I64P,
                                    _I64P, _I64P]
    lib.tide_plan_map.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _I64P,
                                  _I64P, _I64P]
    lib.tide_reduce_scatter_bf16_fp32.argtypes = [ctypes.c_void_p, _VPP, ctypes.c_void_p,
                                                  ctypes.c_int64, ctypes.c_void_p,
                                                  ctypes.POINTER(Launch)]
    lib.tide_allgather_place.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         _VPP, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.POINTER(Launch)]
    lib.tide_plan_launch_count.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.POINTER(Launch), _I64P]
    lib.tide_allgather_place_stage.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_int32, _VPP, ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.POINTER(Launch)]
    lib.tide_rd_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.POINTER(RdStep), ctypes.c_int32,
                                     _I32P]
    lib.tide_landing_sum_fp32.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _VPP,
                                          _VPP, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.POINTER(Launch)]
    lib.tide_latin_square.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, _I32P, _I32P, _I32P]
    lib.tide_stage_grads_bf16.argtypes = [ctypes.c_void_p, _VPP, _VPP, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.POINTER(Launch)]
    lib.tide_plan_trace_records.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.POINTER(Launch), _I64P]
    lib.tide_landing_trace_records.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.POINTER(Launch), _I64P]
    lib.tide_plan_event_count.argtypes = [ctypes.c_void_p, _I64P]
    lib.tide_prepare_reduce_scatter_bf16_fp32.argtypes = [
        ctypes.c_void_p, _VPP, ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(Launch),
        ctypes.POINTER(ctypes.c_void_p)]
    lib.tide_prepare_allgather_place_stage.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, _VPP,
        ctypes.POINTER(Launch), ctypes.POINTER(ctypes.c_void_p)]
    lib.tide_prepare_stage_grads_bf16.argtypes = [
        ctypes.c_void_p, _VPP, _VPP, ctypes.POINTER(Launch), ctypes.POINTER(ctypes.c_void_p)]
    lib.tide_call_enqueue.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.tide_call_destroy.argtypes = [ctypes.c_void_p]
    lib.tide_call_destroy.restype = None
    lib.tide_diag_occupy.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.tide_plan_slot_grads.argtypes = [ctypes.c_void_p, _VPP, _VPP]
    lib.tide_reduce_scatter_bf16_fp32_noalloc.argtypes = [ctypes.c_void_p, _VPP, ctypes.c_void_p,
                                                          ctypes.c_int64, ctypes.c_void_p,
                                                          ctypes.POINTER(Launch)]
    lib.tide_dma_engine_count.argtypes = [ctypes.c_int32, _I32P]
    lib.tide_diag_stream.argtypes = [ctypes.c_int32, _VPP, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    lib.tide_status_string.argtypes = [ctypes.c_int]
    lib.tide_status_string.restype = ctypes.c_char_p
    lib.tide_last_error_detail.argtypes = []
    lib.tide_last_error_detail.restype = ctypes.c_char_p
    lib.tide_version.argtypes = []
    lib.tide_version.restype = ctypes.c_int32
    for f in ("tide_plan_create", "tide_plan_dims", "tide_plan_param", "tide_plan_map",
              "tide_reduce_scatter_bf16_fp32", "tide_allgather_place", "tide_plan_launch_count",
              "tide_allgather_place_stage", "tide_rd_schedule", "tide_landing_sum_fp32",
              "tide_latin_square", "tide_stage_grads_bf16", "tide_plan_trace_records",
              "tide_landing_trace_records", "tide_diag_occupy", "tide_plan_event_count",
              "tide_prepare_reduce_scatter_bf16_fp32", "tide_prepare_allgather_place_stage",
              "tide_prepare_stage_grads_bf16", "tide_call_enqueue", "tide_plan_slot_grads",
              "tide_dma_engine_count", "tide_reduce_scatter_bf16_fp32_noalloc",
              "tide_diag_stream"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def lib():
    return _load()


def _check(status: int, call: str):
    if status != TIDE_OK:
        detail = _load().tide_last_error_detail().decode(errors="replace")
        raise TideError(status, detail, call)


def _ptr(x) -> int:
    """Device address of a tensor (or a raw integer address)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _tensor_arg(t, dtype_name: str, what: str, numel: Optional[int] = None,
                min_numel: Optional[int] = None) -> None:
    """Check a tensor argument before its address goes to the library, which
    sees only pointers: dtype, contiguity, size, and that it is on the GPU.
    Raw integer addresses are the caller's responsibility and pass unchecked."""
    if t is None or isinstance(t, int):
        return
    import torch
    dtype = getattr(torch, dtype_name)
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (what, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s is not contiguous" % what)
    n = t.numel()
    if numel is not None and n != numel:
        raise ValueError("%s holds %d elements, expected %d" % (what, n, numel))
    if min_numel is not None and n < min_numel:
        raise ValueError("%s holds %d elements, at least %d needed" % (what, n, min_numel))
    if not t.is_cuda:
        raise ValueError("%s is not a GPU tensor" % what)


def _check_many(tensors, dtype_name: str, numels, what) -> None:
    """_tensor_arg over many tensors of exact sizes, with the common case (a
    contiguous GPU tensor of the right dtype and size) tested in one pass;
    `what(i)` names tensor i in an error."""
    import torch
    dtype = getattr(torch, dtype_name)
    for i, (t, n) in enumerate(zip(tensors, numels)):
        if t is None or isinstance(t, int):
            continue
        if t.dtype is not dtype or not t.is_cuda or t.numel() != n or not t.is_contiguous():
            _tensor_arg(t, dtype_name, what(i), numel=n)


def _shards_elems(plan: "Plan", stride: int) -> int:
    """Elements N shards of S, `stride` apart, span."""
    return 0 if plan.S == 0 else (plan.N - 1) * stride + plan.S


def _stream_handle(stream) -> Tuple[int, object]:
    import torch
    if stream is None:
        s = torch.cuda.current_stream()
    elif isinstance(stream, int):
        return stream, None
    else:
        s = stream
    return int(s.cuda_stream), s


class Plan:
    """A parameter group's layout (tide_plan_create); freed on close()/GC."""

    def __init__(self, shapes: Sequence[Tuple[int, int]], N: int, L: int):
        lib_ = _load()
        self.shapes = [(int(t), int(k)) for t, k in shapes]
        P = len(self.shapes)
        rows = (ctypes.c_int64 * max(P, 1))(*[t for t, _ in self.shapes])
        rlen = (ctypes.c_int64 * max(P, 1))(*[k for _, k in self.shapes])
        h = ctypes.c_void_p()
        _check(lib_.tide_plan_create(rows, rlen, P, N, L, ctypes.byref(h)), "tide_plan_create")
        self._h = h
        self.P, self.N, self.L = P, N, L
        S = ctypes.c_int64()
        _check(lib_.tide_plan_dims(h, None, None, None, ctypes.byref(S)), "tide_plan_dims")
        self.S = int(S.value)

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _load().tide_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def param(self, p: int):
        """(T_p, K_p, R_p, s_p, o_p)."""
        v = [ctypes.c_int64() for _ in range(5)]
        _check(_load().tide_plan_param(self._h, p, *[ctypes.byref(x) for x in v]),
               "tide_plan_param")
        return tuple(int(x.value) for x in v)

    def map(self, r: int, p: int):
        """(rank_major, param_major, valid) of rank r's piece of parameter p."""
        v = [ctypes.c_int64() for _ in range(3)]
        _check(_load().tide_plan_map(self._h, r, p, *[ctypes.byref(x) for x in v]),
               "tide_plan_map")
        return tuple(int(x.value) for x in v)

    def event_count(self) -> int:
        """HIP events the plan holds (tide_plan_event_count)."""
        n = ctypes.c_int64()
        _check(_load().tide_plan_event_count(self._h, ctypes.byref(n)), "tide_plan_event_count")
        return int(n.value)

    def trace_records(self, op: int, launch: Optional[Launch] = None) -> int:
        """Workgroups (trace records) a call of op 0 / 1 / 2 launches."""
        n = ctypes.c_int64()
        _check(_load().tide_plan_trace_records(self._h, op,
                                               ctypes.byref(launch) if launch is not None else None,
                                               ctypes.byref(n)), "tide_plan_trace_records")
        return int(n.value)

    def launch_count(self, op: int, launch: Optional[Launch] = None) -> int:
        n = ctypes.c_int64()
        _check(_load().tide_plan_launch_count(
            self._h, op, ctypes.byref(launch) if launch is not None else None, ctypes.byref(n)),
            "tide_plan_launch_count")
        return int(n.value)


def plan_create(shapes: Sequence[Tuple[int, int]], N: int, L: int) -> Plan:
    return Plan(shapes, N, L)


class PointerTable:
    """Device addresses marshalled once into a ctypes array, for callers whose
    tensors persist across calls (reading `data_ptr()` of thousands of tensors
    costs far more host time than the library's own per-call work). Keeps the
    tensors alive."""

    def __init__(self, tensors: Sequence[object]):
        self.refs = list(tensors)
        self.n = len(self.refs)
        self.arr = (ctypes.c_void_p * max(self.n, 1))(*[_ptr(t) for t in self.refs])


def grads_table(plan: Plan, grads: Sequence[Sequence[object]]) -> PointerTable:
    """grads[c][p] -> the L*P table tide_reduce_scatter_bf16_fp32 reads (c-major)."""
    if len(grads) != plan.L or any(len(g) != plan.P for g in grads):
        raise ValueError("grads must be L=%d lists of P=%d tensors" % (plan.L, plan.P))
    flat = [grads[c][p] for c in range(plan.L) for p in range(plan.P)]
    _check_many(flat, "bfloat16", [t * k for t, k in plan.shapes] * plan.L,
                lambda i: "grads[%d][%d]" % divmod(i, plan.P))
    return PointerTable(flat)


def params_table(plan: Plan, params: Sequence[object]) -> PointerTable:
    if len(params) != plan.P:
        raise ValueError("params must hold P=%d tensors" % plan.P)
    _check_many(params, "bfloat16", [t * k for t, k in plan.shapes], lambda i: "params[%d]" % i)
    return PointerTable(params)


def _record(tensors, stream_obj) -> bool:
    """Tell torch's caching allocator that the tensors are used on a
    non-default stream, so their memory is not handed out again before that
    stream's work on them has run (tensors are assumed to be allocated on the
    default stream; a caller that allocates on other streams records them
    itself). Returns False when nothing could be recorded because the stream
    is capturing a graph (the graph keeps its own references)."""
    import torch
    if stream_obj is None:
        return True
    if stream_obj == torch.cuda.default_stream(stream_obj.device):
        return True
    with torch.cuda.stream(stream_obj):
        if torch.cuda.is_current_stream_capturing():
            return False
    for t in tensors:
        if t is not None and not isinstance(t, int):
            t.record_stream(stream_obj)
    return True


def reduce_scatter_bf16_fp32(plan: Plan, grads: Sequence[Sequence[object]], out,
                             out_stride: Optional[int] = None, stream=None,
                             launch: Optional[Launch] = None) -> None:
    """grads[c][p]: bf16 (T_p, K_p) device tensors (or raw addresses), or a
    PointerTable from grads_table(); out: fp32 device tensor holding N shards
    of out_stride elements (default S)."""
    tab = grads if isinstance(grads, PointerTable) else grads_table(plan, grads)
    if tab.n != plan.L * plan.P:
        raise ValueError("pointer table holds %d entries, expected L*P=%d" % (tab.n, plan.L * plan.P))
    flat, arr = tab.refs, tab.arr
    stride = plan.S if out_stride is None else int(out_stride)
    _tensor_arg(out, "float32", "out", min_numel=_shards_elems(plan, stride))
    sh, sobj = _stream_handle(stream)
    st = _load().tide_reduce_scatter_bf16_fp32(
        plan.handle, arr, _ptr(out), stride, sh,
        ctypes.byref(launch) if launch is not None else None)
    _check(st, "tide_reduce_scatter_bf16_fp32")
    _record(flat + [out], sobj)


def reduce_scatter_bf16_fp32_noalloc(plan: Plan, grads: Sequence[Sequence[object]], out,
                                     out_stride: Optional[int] = None, stream=None,
                                     launch: Optional[Launch] = None) -> None:
    """reduce_scatter_bf16_fp32 through the entry point that allocates no
    device memory (tide_reduce_scatter_bf16_fp32_noalloc). The binding only
    marshals; tensors passed in were allocated by the caller beforehand."""
    tab = grads if isinstance(grads, PointerTable) else grads_table(plan, grads)
    if tab.n != plan.L * plan.P:
        raise ValueError("pointer table holds %d entries, expected L*P=%d" % (tab.n, plan.L * plan.P))
    stride = plan.S if out_stride is None else int(out_stride)
    _tensor_arg(out, "float32", "out", min_numel=_shards_elems(plan, stride))
    sh, sobj = _stream_handle(stream)
    st = _load().tide_reduce_scatter_bf16_fp32_noalloc(
        plan.handle, tab.arr, _ptr(out), stride, sh,
        ctypes.byref(launch) if launch is not None else None)
    _check(st, "tide_reduce_scatter_bf16_fp32_noalloc")
    _record(tab.refs + [out], sobj)


def allgather_place(plan: Plan, shards, params: Sequence[object],
                    shard_stride: Optional[int] = None, stream=None,
                    engine: Union[int, str] = ENGINE_KERNEL,
                    launch: Optional[Launch] = None) -> None:
    """shards: bf16 device tensor of N rank-major shards (shard_stride elements
    apart, default S); params[p]: bf16 (T_p, K_p) device tensors, or a
    PointerTable from params_table()."""
    tab = params if isinstance(params, PointerTable) else params_table(plan, params)
    if tab.n != plan.P:
        raise ValueError("pointer table holds %d entries, expected P=%d" % (tab.n, plan.P))
    if isinstance(engine, str):
        engine = ENGINES[engine]
    arr = tab.arr
    stride = plan.S if shard_stride is None else int(shard_stride)
    _tensor_arg(shards, "bfloat16", "shards", min_numel=_shards_elems(plan, stride))
    sh, sobj = _stream_handle(stream)
    st = _load().tide_allgather_place(plan.handle, _ptr(shards), stride, arr, sh, int(engine),
                                      ctypes.byref(launch) if launch is not None else None)
    _check(st, "tide_allgather_place")
    _record(tab.refs + [shards], sobj)


def allgather_place_stage(plan: Plan, stage, first_rank: int, params: Sequence[object],
                          shard_stride: Optional[int] = None, stream=None,
                          engine: Union[int, str] = ENGINE_KERNEL,
                          launch: Optional[Launch] = None) -> None:
    """Placement from a stage buffer whose position k holds rank
    (first_rank + k) mod N (recursive-doubling arrival order)."""
    tab = params if isinstance(params, PointerTable) else params_table(plan, params)
    if tab.n != plan.P:
        raise ValueError("pointer table holds %d entries, expected P=%d" % (tab.n, plan.P))
    if isinstance(engine, str):
        engine = ENGINES[engine]
    stride = plan.S if shard_stride is None else int(shard_stride)
    _tensor_arg(stage, "bfloat16", "stage", min_numel=_shards_elems(plan, stride))
    sh, sobj = _stream_handle(stream)
    st = _load().tide_allgather_place_stage(plan.handle, _ptr(stage), stride, int(first_rank),
                                            tab.arr, sh, int(engine),
                                            ctypes.byref(launch) if launch is not None else None)
    _check(st, "tide_allgather_place_stage")
    _record(tab.refs + [stage], sobj)


def stage_grads_bf16(plan: Plan, grads: Sequence[Sequence[object]], slots: Sequence[object],
                     stream=None, engine: Union[int, str] = ENGINE_KERNEL,
                     launch: Optional[Launch] = None) -> None:
    """Slot-Reuse staging (tide_stage_grads_bf16): contributor c's gradients
    grads[c][p] (or a grads_table()) are copied into slots[c], a bf16 device
    tensor of N * S elements, at each parameter's offset N * o_p."""
    tab = grads if isinstance(grads, PointerTable) else grads_table(plan, grads)
    if tab.n != plan.L * plan.P:
        raise ValueError("pointer table holds %d entries, expected L*P=%d" % (tab.n, plan.L * plan.P))
    _slots_arg(plan, slots)
    if isinstance(engine, str):
        engine = ENGINES[engine]
    sa = (ctypes.c_void_p * plan.L)(*[_ptr(t) for t in slots])
    sh, sobj = _stream_handle(stream)
    st = _load().tide_stage_grads_bf16(plan.handle, tab.arr, sa, sh, int(engine),
                                       ctypes.byref(launch) if launch is not None else None)
    _check(st, "tide_stage_grads_bf16")
    _record(tab.refs + list(slots), sobj)


def _slots_arg(plan: Plan, slots: Sequence[object]) -> None:
    if len(slots) != plan.L:
        raise ValueError("need L=%d slots" % plan.L)
    for c, t in enumerate(slots):
        _tensor_arg(t, "bfloat16", "slots[%d]" % c, min_numel=plan.N * plan.S)


def slot_grads_table(plan: Plan, slots: Sequence[object]) -> PointerTable:
    """The reduce's L*P gradient table reading the staged slots, as
    tide_plan_slot_grads builds it (keeps the slot tensors alive)."""
    _slots_arg(plan, slots)
    sa = (ctypes.c_void_p * plan.L)(*[_ptr(t) for t in slots])
    n = plan.L * plan.P
    arr = (ctypes.c_void_p * max(n, 1))()
    _check(_load().tide_plan_slot_grads(plan.handle, sa, arr), "tide_plan_slot_grads")
    tab = PointerTable([])
    tab.refs, tab.n, tab.arr = list(slots), n, arr
    return tab


def dma_engine_count(device: int = 0) -> int:
    """DMA engines the SDMA engine path spreads its copies over (tide_dma_engine_count)."""
    n = ctypes.c_int32()
    _check(_load().tide_dma_engine_count(int(device), ctypes.byref(n)), "tide_dma_engine_count")
    return int(n.value)


class Call:
    """A prepared call (tide_call): buffers validated once, its pointer table
    on the device; enqueue() launches its kernels only, so it may be captured
    into a graph. Holds the plan and the buffers alive."""

    def __init__(self, plan: Plan, handle: int, refs):
        self.plan = plan
        self._h = handle
        self.refs = refs
        self._recorded = set()      # streams the buffers are already recorded on

    def enqueue(self, stream=None) -> None:
        sh, sobj = _stream_handle(stream)
        _check(_load().tide_call_enqueue(self._h, sh), "tide_call_enqueue")
        # The call holds its buffers for its whole life, so one record per
        # stream covers every later enqueue on it (a gradient table of
        # thousands of tensors would otherwise cost milliseconds per enqueue).
        if sh not in self._recorded and _record(self.refs, sobj):
            self._recorded.add(sh)

    def close(self):
        if self._h:
            _load().tide_call_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


def _prepared(plan: Plan, fn, name: str, args, refs) -> Call:
    h = ctypes.c_void_p()
    _check(fn(*args, ctypes.byref(h)), name)
    return Call(plan, h.value, refs)


def prepare_reduce_scatter_bf16_fp32(plan: Plan, grads, out, out_stride: Optional[int] = None,
                                     launch: Optional[Launch] = None) -> Call:
    """Prepared form of reduce_scatter_bf16_fp32 (tide_prepare_reduce_scatter_bf16_fp32)."""
    tab = grads if isinstance(grads, PointerTable) else grads_table(plan, grads)
    stride = plan.S if out_stride is None else int(out_stride)
    _tensor_arg(out, "float32", "out", min_numel=_shards_elems(plan, stride))
    return _prepared(plan, _load().tide_prepare_reduce_scatter_bf16_fp32,
                     "tide_prepare_reduce_scatter_bf16_fp32",
                     (plan.handle, tab.arr, _ptr(out), stride,
                      ctypes.byref(launch) if launch is not None else None), tab.refs + [out])


def prepare_allgather_place(plan: Plan, shards, params, shard_stride: Optional[int] = None,
                            first_rank: int = 0, launch: Optional[Launch] = None) -> Call:
    """Prepared form of allgather_place_stage (kernel engine)."""
    tab = params if isinstance(params, PointerTable) else params_table(plan, params)
    stride = plan.S if shard_stride is None else int(shard_stride)
    _tensor_arg(shards, "bfloat16", "shards", min_numel=_shards_elems(plan, stride))
    return _prepared(plan, _load().tide_prepare_allgather_place_stage,
                     "tide_prepare_allgather_place_stage",
                     (plan.handle, _ptr(shards), stride, int(first_rank), tab.arr,
                      ctypes.byref(launch) if launch is not None else None), tab.refs + [shards])


def prepare_stage_grads_bf16(plan: Plan, grads, slots, launch: Optional[Launch] = None) -> Call:
    """Prepared form of stage_grads_bf16 (kernel engine)."""
    tab = grads if isinstance(grads, PointerTable) else grads_table(plan, grads)
    _slots_arg(plan, slots)
    sa = (ctypes.c_void_p * plan.L)(*[_ptr(t) for t in slots])
    return _prepared(plan, _load().tide_prepare_stage_grads_bf16, "tide_prepare_stage_grads_bf16",
                     (plan.handle, tab.arr, sa, ctypes.byref(launch) if launch is not None else None),
                     tab.refs + list(slots))


def rd_schedule(M: int, node: int, piece_bytes: int = 0, head_bytes: int = 0):
    """Node's recursive-doubling rounds as a list of dicts (tide_rd_schedule)."""
    cap = 64
    steps = (RdStep * cap)()
    n = ctypes.c_int32()
    _check(_load().tide_rd_schedule(M, node, piece_bytes, head_bytes, steps, cap,
                                    ctypes.byref(n)), "tide_rd_schedule")
    return [{f: getattr(steps[i], f) for f, _ in RdStep._fields_} for i in range(n.value)]


def landing_sum_fp32(L: int, M: int, S: int, inboxes: Sequence[object], shards: Sequence[object],
                     accumulate: bool = False, stream=None,
                     launch: Optional[Launch] = None) -> None:
    """Level-2 landing sum of one destination node (tide_landing_sum_fp32).
    inboxes[g]: fp32 device tensors of L*L*ceil(S/L); shards[b]: fp32 of S."""
    if len(inboxes) != L or len(shards) != L:
        raise ValueError("need L=%d inboxes and L shards" % L)
    C = -(-int(S) // L) if L > 0 else 0
    for g in range(L):
        _tensor_arg(inboxes[g], "float32", "inboxes[%d]" % g, min_numel=L * L * C)
        _tensor_arg(shards[g], "float32", "shards[%d]" % g, min_numel=int(S))
    ia = (ctypes.c_void_p * L)(*[_ptr(t) for t in inboxes])
    sa = (ctypes.c_void_p * L)(*[_ptr(t) for t in shards])
    sh, sobj = _stream_handle(stream)
    st = _load().tide_landing_sum_fp32(L, M, S, ia, sa, 1 if accumulate else 0, sh,
                                       ctypes.byref(launch) if launch is not None else None)
    _check(st, "tide_landing_sum_fp32")
    _record(list(inboxes) + list(shards), sobj)


def landing_trace_records(L: int, M: int, S: int, accumulate: bool = False,
                          launch: Optional[Launch] = None) -> int:
    n = ctypes.c_int64()
    _check(_load().tide_landing_trace_records(L, M, S, 1 if accumulate else 0,
                                              ctypes.byref(launch) if launch is not None else None,
                                              ctypes.byref(n)), "tide_landing_trace_records")
    return int(n.value)


def diag_occupy(workgroups: int, threads: int, lds_bytes: int, spin_ticks: int, trace,
                stream=None) -> None:
    """tide_diag_occupy: a GEMM-shaped occupant that records where it ran."""
    _tensor_arg(trace, "int64", "trace", min_numel=3 * max(int(workgroups), 0))
    sh, sobj = _stream_handle(stream)
    _check(_load().tide_diag_occupy(workgroups, threads, lds_bytes, spin_ticks, _ptr(trace), sh),
           "tide_diag_occupy")
    _record([trace], sobj)


def diag_stream(kind: int, srcs: Sequence[object], dst, n: int, workgroups: int = 0,
                stream=None) -> None:
    """tide_diag_stream: bandwidth-ceiling kernels (0 read, 1 write, 2 copy,
    3 the reduce's access pattern over len(srcs) bf16 sources); workgroups > 0
    runs that many 1024-thread workgroups instead of the full grid."""
    sa = (ctypes.c_void_p * max(len(srcs), 1))(*[_ptr(t) for t in srcs])
    sh, sobj = _stream_handle(stream)
    _check(_load().tide_diag_stream(int(kind), sa, len(srcs), _ptr(dst), int(n),
                                    int(workgroups), sh), "tide_diag_stream")
    _record(list(srcs) + [dst], sobj)


def latin_square(M: int, L: int, dst_node: int, src_node: int):
    """(c, slice handled by each source GPU, destination GPU of each slice)."""
    c = ctypes.c_int32()
    a = (ctypes.c_int32 * L)()
    b = (ctypes.c_int32 * L)()
    _check(_load().tide_latin_square(M, L, dst_node, src_node, ctypes.byref(c), a, b),
           "tide_latin_square")
    return int(c.value), list(a), list(b)


def version() -> int:
    return int(_load().tide_version())
