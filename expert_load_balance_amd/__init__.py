"""Python binding of libmoe.so, the MI355X (gfx950) MoE-layer hot path.

Argument marshalling only: every function here has the name of a C entry
point declared in ``include/moe.h``, checks that the tensors it is given have
the documented dtype, device and contiguity, and passes their device pointers
and the current HIP stream through ctypes. All arithmetic runs in the HIP
kernels; there is no CPU path. If the library has not been built, every call
raises ``RuntimeError``.

Build with ``python -m expert_load_balance_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MOE_F32", "MOE_BF16", "MoeError", "Shape", "StatsT", "lib_path", "load",
    "moe_status_str", "moe_check_shape", "moe_plan_layout", "moe_plan_bytes", "moe_plan_bind",
    "moe_workspace_bytes", "moe_route", "moe_count", "moe_count_noalloc", "moe_plan", "moe_count_plan", "moe_permute",
    "moe_grouped_gemm",
    "moe_gemm_schedule", "moe_gemm_gateup", "moe_gemm_down", "moe_combine", "moe_stats",
    "moe_capacity_rows", "moe_capacity_dispatch", "moe_capacity_plan", "moe_capacity_combine",
    "moe_repack", "capacity_shape", "moe_router_workspace_bytes", "moe_router", "moe_bias_update", "plan_tables",
    "bind", "moe_pool_bytes", "moe_prefetch_replicas", "moe_grouped_gemm_slots",
    "moe_backward_workspace_bytes", "moe_combine_backward", "moe_ffn_backward",
    "moe_permute_backward", "moe_route_backward", "moe_grouped_gemm_train",
    "moe_replica_grad_bytes", "moe_ffn_backward_replicas", "moe_probe_mfma",
    "moe_probe_copy", "moe_probe_read", "EXPORTED_SYMBOLS",
]

MOE_F32 = 0
MOE_BF16 = 1
ERR_NONFINITE, ERR_RANGE, ERR_REPEAT = 1, 2, 4

EXPORTED_SYMBOLS = (
    "moe_status_str", "moe_check_shape", "moe_plan_layout", "moe_workspace_bytes", "moe_route",
    "moe_count", "moe_plan", "moe_permute", "moe_grouped_gemm", "moe_gemm_schedule",
    "moe_gemm_gateup", "moe_gemm_down", "moe_combine", "moe_stats", "moe_capacity_rows",
    "moe_capacity_dispatch", "moe_capacity_plan", "moe_capacity_combine", "moe_repack",
    "moe_router_workspace_bytes", "moe_router", "moe_bias_update", "moe_pool_bytes",
    "moe_prefetch_replicas", "moe_grouped_gemm_slots", "moe_backward_workspace_bytes",
    "moe_combine_backward", "moe_ffn_backward", "moe_permute_backward", "moe_route_backward",
    "moe_grouped_gemm_train", "moe_replica_grad_bytes", "moe_ffn_backward_replicas",
    "moe_count_noalloc", "moe_probe_mfma", "moe_probe_copy", "moe_probe_read", "moe_count_plan",
    "moe_plan_bytes", "moe_plan_bind",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe.so")
_lib = None


def lib_path() -> str:
    return _LIB_PATH


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_str(status)} (status {status})")


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "E", "k", "F", "R", "S", "dtype")]

    def __init__(self, T, H, E, k, F, R, S, dtype=MOE_BF16):
        super().__init__(T, H, E, k, F, R, S, dtype)

    def replace(self, **kw):
        d = {n: getattr(self, n) for n, _ in self._fields_}
        d.update(kw)
        return Shape(**d)

    @property
    def N(self) -> int:
        return self.T * self.k

    def __repr__(self):
        return "Shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class PlanLayoutT(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "quota", "win_off", "seg_num", "seg_expert", "seg_row", "seg_cnt", "slots_needed",
        "slot_expert", "donor", "piece_num", "piece_rank", "piece_row", "piece_cnt", "total")]


PLAN_T_FIELDS = ("quota", "win_off", "seg_expert", "seg_row", "seg_cnt", "seg_num", "slot_expert",
                 "slots_needed", "piece_rank", "piece_row", "piece_cnt", "piece_num", "donor")


class PlanT(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PLAN_T_FIELDS]


class StatsT(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("E", ctypes.c_int32), ("R", ctypes.c_int32),
        ("max_count", ctypes.c_int32), ("min_count", ctypes.c_int32),
        ("active_experts", ctypes.c_int32),
        ("maxvio_expert", ctypes.c_double), ("balancedness_expert", ctypes.c_double),
        ("home_max", ctypes.c_int32),
        ("maxvio_rank_home", ctypes.c_double), ("balancedness_rank_home", ctypes.c_double),
        ("mapped_max", ctypes.c_int32),
        ("maxvio_rank_mapped", ctypes.c_double), ("balancedness_rank_mapped", ctypes.c_double),
        ("planned_max", ctypes.c_int32), ("planned_min", ctypes.c_int32),
        ("maxvio_rank_planned", ctypes.c_double), ("balancedness_rank_planned", ctypes.c_double),
        ("capacity", ctypes.c_int32),
        ("processed", ctypes.c_int64), ("overflow", ctypes.c_int64), ("padding", ctypes.c_int64),
        ("remote_home", ctypes.c_int64), ("remote_mapped", ctypes.c_int64),
        ("remote_planned", ctypes.c_int64),
        ("replica_pieces", ctypes.c_int32), ("max_slots_needed", ctypes.c_int32),
        ("ranks_over_slots", ctypes.c_int32), ("nonlocal_rows", ctypes.c_int64),
        ("err", ctypes.c_int32),
    ]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_VP = ctypes.c_void_p
_SP = ctypes.POINTER(Shape)


def load():
    """Loads libmoe.so (once). Raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libmoe.so is not built ({_LIB_PATH}); run "
                           "`python -m expert_load_balance_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    st = ctypes.c_int
    sig = {
        "moe_status_str": (ctypes.c_char_p, [st]),
        "moe_check_shape": (st, [_SP]),
        "moe_plan_layout": (st, [_SP, ctypes.POINTER(PlanLayoutT)]),
        "moe_workspace_bytes": (ctypes.c_size_t, [_SP]),
        "moe_plan_bytes": (ctypes.c_size_t, [_SP]),
        "moe_plan_bind": (st, [_SP, _VP, ctypes.POINTER(PlanT)]),
        "moe_route": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "moe_count": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
        "moe_count_noalloc": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "moe_probe_mfma": (st, [ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_size_t, _VP]),
        "moe_probe_copy": (st, [_VP, _VP, ctypes.c_size_t, ctypes.c_int32, _VP]),
        "moe_probe_read": (st, [_VP, ctypes.c_size_t, ctypes.c_int32, _VP, ctypes.c_size_t, _VP]),
        "moe_plan": (st, [_SP, _VP, _VP, _VP]),
        "moe_count_plan": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP, _VP]),
        "moe_permute": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "moe_grouped_gemm": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
        "moe_gemm_schedule": (st, [_SP, _VP, _VP, ctypes.c_size_t, _VP]),
        "moe_gemm_gateup": (st, [_SP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
        "moe_gemm_down": (st, [_SP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
        "moe_combine": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "moe_stats": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_double, _VP,
                           ctypes.c_size_t, ctypes.POINTER(StatsT), _VP, _VP]),
        "moe_capacity_rows": (ctypes.c_int32, [_SP, ctypes.c_double]),
        "moe_capacity_dispatch": (st, [_SP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "moe_capacity_plan": (st, [_SP, ctypes.c_int32, _VP, _VP]),
        "moe_capacity_combine": (st, [_SP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP]),
        "moe_repack": (st, [_SP, _VP, _VP, _VP]),
        "moe_router_workspace_bytes": (ctypes.c_size_t, [_SP]),
        "moe_router": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
        "moe_bias_update": (st, [_SP, _VP, _VP, ctypes.c_float, _VP]),
        "moe_pool_bytes": (ctypes.c_size_t, [_SP]),
        "moe_backward_workspace_bytes": (ctypes.c_size_t, [_SP]),
        "moe_combine_backward": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "moe_ffn_backward": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                  ctypes.c_size_t, _VP]),
        "moe_grouped_gemm_train": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                        ctypes.c_size_t, _VP]),
        "moe_replica_grad_bytes": (ctypes.c_size_t, [_SP]),
        "moe_ffn_backward_replicas": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                           _VP, _VP, ctypes.c_size_t, _VP, ctypes.c_size_t, _VP]),
        "moe_permute_backward": (st, [_SP, _VP, _VP, _VP, _VP]),
        "moe_route_backward": (st, [_SP, _VP, _VP, _VP, _VP, _VP]),
        "moe_prefetch_replicas": (st, [_SP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
        "moe_grouped_gemm_slots": (st, [_SP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP,
                                        _VP, ctypes.c_size_t, _VP]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ------------------------------------------------------------- marshalling --

def _ptr(t, dtype=None, name="tensor", numel=None, nullable=False):
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} must not be None")
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr() or None


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _act_dtype(shape):
    import torch

    return torch.bfloat16 if shape.dtype == MOE_BF16 else torch.float32


def _ok(status, where):
    if status != 0:
        raise MoeError(status, where)


# entry points that only compute on the host (sizes, layouts, checks)
_HOST_ONLY = frozenset(("moe_status_str", "moe_check_shape", "moe_plan_layout",
                        "moe_workspace_bytes", "moe_router_workspace_bytes", "moe_capacity_rows",
                        "moe_pool_bytes", "moe_backward_workspace_bytes",
                        "moe_replica_grad_bytes"))


class _Recorder:
    """Stands in for the loaded library while bind() runs a wrapper: records
    each launching C call and its marshalled arguments instead of making it
    (host-only queries go through)."""

    def __init__(self, lib):
        self.lib, self.calls = lib, []

    def __getattr__(self, name):
        fn = getattr(self.lib, name)
        if name in _HOST_ONLY:
            return fn

        def record(*args):
            self.calls.append((name, fn, args))
            return 0

        return record


def bind(wrapper, *args, **kwargs):
    """Marshals the arguments of one launch-only wrapper call (moe_permute,
    moe_router, ...) once and returns a callable that repeats only its C
    call(s). For timing loops, where the per-call checks and ctypes
    conversions would otherwise cost more host time than a small kernel takes
    on the device. The tensors passed must stay alive while the callable is
    used."""
    global _lib
    real = load()
    rec = _Recorder(real)
    _lib = rec
    try:
        wrapper(*args, **kwargs)
    finally:
        _lib = real
    calls = tuple(rec.calls)

    def run():
        for name, fn, a in calls:
            _ok(fn(*a), name)

    return run


def moe_status_str(status: int) -> str:
    return load().moe_status_str(int(status)).decode()


def moe_check_shape(shape: Shape) -> int:
    return load().moe_check_shape(ctypes.byref(shape))


def moe_plan_layout(shape: Shape) -> dict:
    out = PlanLayoutT()
    _ok(load().moe_plan_layout(ctypes.byref(shape), ctypes.byref(out)), "moe_plan_layout")
    return {n: getattr(out, n) for n, _ in out._fields_}


def moe_plan_bytes(shape: Shape) -> int:
    return int(load().moe_plan_bytes(ctypes.byref(shape)))


def moe_plan_bind(shape: Shape, block_addr: int) -> dict:
    """Table name -> address inside the plan block at `block_addr` (an
    integer address; the block is never dereferenced)."""
    out = PlanT()
    _ok(load().moe_plan_bind(ctypes.byref(shape), ctypes.c_void_p(block_addr), ctypes.byref(out)),
        "moe_plan_bind")
    return {n: getattr(out, n) for n in PLAN_T_FIELDS}


def moe_workspace_bytes(shape: Shape) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(shape)))


def moe_route(shape, logits, bias, ids, w, err, stream=None):
    import torch

    T, E, k = shape.T, shape.E, shape.k
    args = (ctypes.byref(shape), _ptr(logits, torch.float32, "logits", T * E),
            _ptr(bias, torch.float32, "bias", E, nullable=True),
            _ptr(ids, torch.int32, "ids", T * k), _ptr(w, torch.float32, "w", T * k),
            _ptr(err, torch.int32, "err", 1), _stream(stream))
    _ok(load().moe_route(*args), "moe_route")


def moe_count(shape, ids, counts, offsets, eidx, rank_load, err, ws, stream=None):
    import torch

    i32 = torch.int32
    args = (ctypes.byref(shape), _ptr(ids, i32, "ids", shape.N), _ptr(counts, i32, "counts", shape.E),
            _ptr(offsets, i32, "offsets", shape.E + 1), _ptr(eidx, i32, "eidx", shape.N),
            _ptr(rank_load, i32, "rank_load", shape.R), _ptr(err, i32, "err", 1),
            _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _ok(load().moe_count(*args), "moe_count")


def moe_probe_mfma(workgroups, iters, sink, stream=None):
    """The calibration probe: workgroups x 4 waves x 4 * iters bf16 MFMAs
    (32x32x16) on registers only; sink: float32 tensor of at least
    workgroups * 256 elements."""
    import torch

    args = (int(workgroups), int(iters), _ptr(sink, torch.float32, "sink"), sink.numel(),
            _stream(stream))
    _ok(load().moe_probe_mfma(*args), "moe_probe_mfma")


def moe_probe_copy(src, dst, workgroups, stream=None):
    """The HBM calibration probe: copies src into dst (same byte size, a
    multiple of 16) with `workgroups` workgroups."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    args = (_ptr(src, None, "src"), _ptr(dst, None, "dst"), nbytes, int(workgroups), _stream(stream))
    _ok(load().moe_probe_copy(*args), "moe_probe_copy")


def moe_probe_read(src, workgroups, sink, stream=None):
    """The HBM read probe: reads src (a multiple of 16 bytes) in `workgroups`
    contiguous chunks; sink: int32 tensor of at least workgroups * 256
    elements (per-thread XOR of the vectors read)."""
    import torch

    nbytes = src.numel() * src.element_size()
    args = (_ptr(src, None, "src"), nbytes, int(workgroups), _ptr(sink, torch.int32, "sink"),
            sink.numel(), _stream(stream))
    _ok(load().moe_probe_read(*args), "moe_probe_read")


def moe_count_noalloc(shape, ids, counts, offsets, eidx, rank_load, err, stream=None):
    """moe_count without a workspace (the library's fixed device scratch)."""
    import torch

    i32 = torch.int32
    args = (ctypes.byref(shape), _ptr(ids, i32, "ids", shape.N), _ptr(counts, i32, "counts", shape.E),
            _ptr(offsets, i32, "offsets", shape.E + 1), _ptr(eidx, i32, "eidx", shape.N),
            _ptr(rank_load, i32, "rank_load", shape.R), _ptr(err, i32, "err", 1), _stream(stream))
    _ok(load().moe_count_noalloc(*args), "moe_count_noalloc")


def moe_plan(shape, counts, plan, stream=None):
    import torch

    total = moe_plan_layout(shape)["total"]
    _ok(load().moe_plan(ctypes.byref(shape), _ptr(counts, torch.int32, "counts", shape.E),
                        _ptr(plan, torch.int32, "plan", total), _stream(stream)), "moe_plan")


def moe_count_plan(shape, ids, counts, offsets, eidx, rank_load, err, ws, plan, stream=None):
    """moe_count then moe_plan on its counts (one launch up to 16384
    assignments)."""
    import torch

    i32 = torch.int32
    total = moe_plan_layout(shape)["total"]
    args = (ctypes.byref(shape), _ptr(ids, i32, "ids", shape.N), _ptr(counts, i32, "counts", shape.E),
            _ptr(offsets, i32, "offsets", shape.E + 1), _ptr(eidx, i32, "eidx", shape.N),
            _ptr(rank_load, i32, "rank_load", shape.R), _ptr(err, i32, "err", 1),
            _ptr(ws, None, "ws"), ws.numel() * ws.element_size(),
            _ptr(plan, i32, "plan", total), _stream(stream))
    _ok(load().moe_count_plan(*args), "moe_count_plan")


def moe_permute(shape, x, ids, eidx, plan, buf, dest_row, row_src, stream=None):
    import torch

    i32, act = torch.int32, _act_dtype(shape)
    args = (ctypes.byref(shape), _ptr(x, act, "x", shape.T * shape.H), _ptr(ids, i32, "ids", shape.N),
            _ptr(eidx, i32, "eidx", shape.N), _ptr(plan, i32, "plan"),
            _ptr(buf, act, "buf", shape.N * shape.H), _ptr(dest_row, i32, "dest_row", shape.N),
            _ptr(row_src, i32, "row_src", shape.N), _stream(stream))
    _ok(load().moe_permute(*args), "moe_permute")


def _weights(shape, w_gate, w_up, w_down):
    act = _act_dtype(shape)
    n = shape.E * shape.F * shape.H
    return (_ptr(w_gate, act, "w_gate", n) if w_gate is not None else None,
            _ptr(w_up, act, "w_up", n) if w_up is not None else None,
            _ptr(w_down, act, "w_down", n) if w_down is not None else None)


def moe_grouped_gemm(shape, a, plan, w_gate, w_up, w_down, y, ws, stream=None):
    import torch

    act = _act_dtype(shape)
    g, u, d = _weights(shape, w_gate, w_up, w_down)
    args = (ctypes.byref(shape), _ptr(a, act, "a", shape.N * shape.H),
            _ptr(plan, torch.int32, "plan"), g, u, d, _ptr(y, act, "y", shape.N * shape.H),
            _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _ok(load().moe_grouped_gemm(*args), "moe_grouped_gemm")


def moe_gemm_schedule(shape, plan, ws, stream=None):
    import torch

    args = (ctypes.byref(shape), _ptr(plan, torch.int32, "plan"), _ptr(ws, None, "ws"),
            ws.numel() * ws.element_size(), _stream(stream))
    _ok(load().moe_gemm_schedule(*args), "moe_gemm_schedule")


def moe_gemm_gateup(shape, a, plan, w_gate, w_up, ws, stream=None):
    import torch

    act = _act_dtype(shape)
    g, u, _ = _weights(shape, w_gate, w_up, None)
    args = (ctypes.byref(shape), _ptr(a, act, "a", shape.N * shape.H),
            _ptr(plan, torch.int32, "plan"), g, u, _ptr(ws, None, "ws"),
            ws.numel() * ws.element_size(), _stream(stream))
    _ok(load().moe_gemm_gateup(*args), "moe_gemm_gateup")


def moe_gemm_down(shape, plan, w_down, y, ws, stream=None):
    import torch

    act = _act_dtype(shape)
    _, _, d = _weights(shape, None, None, w_down)
    args = (ctypes.byref(shape), _ptr(plan, torch.int32, "plan"), d,
            _ptr(y, act, "y", shape.N * shape.H), _ptr(ws, None, "ws"),
            ws.numel() * ws.element_size(), _stream(stream))
    _ok(load().moe_gemm_down(*args), "moe_gemm_down")


def moe_combine(shape, y, dest_row, w, shared_y, out, stream=None):
    import torch

    act = _act_dtype(shape)
    args = (ctypes.byref(shape), _ptr(y, act, "y", shape.N * shape.H),
            _ptr(dest_row, torch.int32, "dest_row", shape.N), _ptr(w, torch.float32, "w", shape.N),
            _ptr(shared_y, act, "shared_y", shape.T * shape.H, nullable=True),
            _ptr(out, act, "out", shape.T * shape.H), _stream(stream))
    _ok(load().moe_combine(*args), "moe_combine")


def moe_stats(shape, counts, ids, plan, ws, dest_row=None, mapping=None, origin=None, err=None,
              capacity_factor=1.0, stream=None, check=True):
    """Synchronises the stream. Returns (stats dict, rank_loads [3][R] list).
    With check=True a set device error word raises MoeError(MOE_EDATA)."""
    import torch

    i32 = torch.int32
    out = StatsT()
    loads = (ctypes.c_int32 * (3 * shape.R))()
    st = load().moe_stats(
        ctypes.byref(shape), _ptr(counts, i32, "counts", shape.E), _ptr(ids, i32, "ids", shape.N),
        _ptr(plan, i32, "plan"), _ptr(dest_row, i32, "dest_row", shape.N, nullable=True),
        _ptr(mapping, i32, "mapping", shape.E, nullable=True),
        _ptr(origin, i32, "origin", shape.T, nullable=True),
        _ptr(err, i32, "err", 1, nullable=True), float(capacity_factor), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size(), ctypes.byref(out), ctypes.cast(loads, _VP),
        _stream(stream))
    if st != 0 and (check or st != 4):
        raise MoeError(st, "moe_stats")
    R = shape.R
    flat = list(loads)
    return out.as_dict(), [flat[:R], flat[R:2 * R], flat[2 * R:]]


def plan_tables(plan, shape) -> dict:
    """Views of the plan block's tables (by the layout moe_plan_layout reports)."""
    L = moe_plan_layout(shape)
    R, E = shape.R, shape.E
    n = E // R
    sizes = dict(quota=(R,), win_off=(R + 1,), seg_num=(R,), seg_expert=(R, 2 * n),
                 seg_row=(R, 2 * n), seg_cnt=(R, 2 * n), slots_needed=(R,), slot_expert=(R, n),
                 donor=(R,), piece_num=(E,), piece_rank=(E, R), piece_row=(E, R),
                 piece_cnt=(E, R))
    out = {}
    for name, shp in sizes.items():
        cnt = 1
        for s in shp:
            cnt *= s
        out[name] = plan[L[name]:L[name] + cnt].view(*shp)
    return out


# -------------------------------------------------- baselines of the plan --

def moe_capacity_rows(shape, capacity_factor) -> int:
    """Per-expert capacity ceil(N / E * factor); -1 for invalid input."""
    return int(load().moe_capacity_rows(ctypes.byref(shape), float(capacity_factor)))


def capacity_shape(shape, cap):
    """The shape moe_grouped_gemm takes over the [E*cap] capacity buffer."""
    return shape.replace(T=shape.E * cap, k=1)


def moe_capacity_dispatch(shape, cap, counts, x, ids, eidx, buf, dest_row, stream=None):
    import torch

    i32, act = torch.int32, _act_dtype(shape)
    args = (ctypes.byref(shape), int(cap), _ptr(counts, i32, "counts", shape.E),
            _ptr(x, act, "x", shape.T * shape.H), _ptr(ids, i32, "ids", shape.N),
            _ptr(eidx, i32, "eidx", shape.N), _ptr(buf, act, "buf", shape.E * cap * shape.H),
            _ptr(dest_row, i32, "dest_row", shape.N), _stream(stream))
    _ok(load().moe_capacity_dispatch(*args), "moe_capacity_dispatch")


def moe_capacity_plan(shape, cap, plan, stream=None):
    import torch

    total = moe_plan_layout(shape)["total"]
    _ok(load().moe_capacity_plan(ctypes.byref(shape), int(cap),
                                 _ptr(plan, torch.int32, "plan", total), _stream(stream)),
        "moe_capacity_plan")


def moe_capacity_combine(shape, cap, y, dest_row, w, shared_y, out, stream=None):
    import torch

    act = _act_dtype(shape)
    args = (ctypes.byref(shape), int(cap), _ptr(y, act, "y", shape.E * cap * shape.H),
            _ptr(dest_row, torch.int32, "dest_row", shape.N), _ptr(w, torch.float32, "w", shape.N),
            _ptr(shared_y, act, "shared_y", shape.T * shape.H, nullable=True),
            _ptr(out, act, "out", shape.T * shape.H), _stream(stream))
    _ok(load().moe_capacity_combine(*args), "moe_capacity_combine")


def moe_repack(shape, counts, mapping, stream=None):
    import torch

    _ok(load().moe_repack(ctypes.byref(shape), _ptr(counts, torch.int32, "counts", shape.E),
                          _ptr(mapping, torch.int32, "mapping", shape.E), _stream(stream)),
        "moe_repack")


# ------------------------------------------------------------------ router --

def moe_router_workspace_bytes(shape: Shape) -> int:
    return int(load().moe_router_workspace_bytes(ctypes.byref(shape)))


def moe_router(shape, x, w_router, bias, logits, ids, w, err, ws=None, stream=None):
    """ws: a uint8 device tensor of at least moe_router_workspace_bytes(shape)
    bytes, or None when that is 0."""
    import torch

    act, i32 = _act_dtype(shape), torch.int32
    need = moe_router_workspace_bytes(shape)
    args = (ctypes.byref(shape), _ptr(x, act, "x", shape.T * shape.H),
            _ptr(w_router, act, "w_router", shape.E * shape.H),
            _ptr(bias, torch.float32, "bias", shape.E, nullable=True),
            _ptr(logits, torch.float32, "logits", shape.T * shape.E),
            _ptr(ids, i32, "ids", shape.N), _ptr(w, torch.float32, "w", shape.N),
            _ptr(err, i32, "err", 1), _ptr(ws, torch.uint8, "ws", need, nullable=need == 0),
            ws.numel() if ws is not None else 0, _stream(stream))
    _ok(load().moe_router(*args), "moe_router")


def moe_bias_update(shape, counts, bias, gamma, stream=None):
    import torch

    _ok(load().moe_bias_update(ctypes.byref(shape), _ptr(counts, torch.int32, "counts", shape.E),
                               _ptr(bias, torch.float32, "bias", shape.E), float(gamma),
                               _stream(stream)), "moe_bias_update")


def moe_pool_bytes(shape: Shape) -> int:
    return int(load().moe_pool_bytes(ctypes.byref(shape)))


def moe_prefetch_replicas(shape, plan, w_gate, w_up, w_down, pool, stream=None):
    """pool: a device tensor of at least moe_pool_bytes(shape) bytes (any
    dtype), or None when that is 0."""
    import torch

    act = _act_dtype(shape)
    need = moe_pool_bytes(shape)
    n = shape.E * shape.F * shape.H
    _ok(load().moe_prefetch_replicas(
        ctypes.byref(shape), _ptr(plan, torch.int32, "plan"), _ptr(w_gate, act, "w_gate", n),
        _ptr(w_up, act, "w_up", n), _ptr(w_down, act, "w_down", n),
        _ptr(pool, None, "pool", nullable=need == 0), _nbytes(pool), _stream(stream)),
        "moe_prefetch_replicas")


def moe_grouped_gemm_slots(shape, a, plan, w_gate, w_up, w_down, pool, y, ws, stream=None):
    import torch

    act = _act_dtype(shape)
    need = moe_pool_bytes(shape)
    n = shape.E * shape.F * shape.H
    _ok(load().moe_grouped_gemm_slots(
        ctypes.byref(shape), _ptr(a, act, "a", shape.N * shape.H), _ptr(plan, torch.int32, "plan"),
        _ptr(w_gate, act, "w_gate", n), _ptr(w_up, act, "w_up", n), _ptr(w_down, act, "w_down", n),
        _ptr(pool, None, "pool", nullable=need == 0), _nbytes(pool),
        _ptr(y, act, "y", shape.N * shape.H), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_grouped_gemm_slots")


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ---- backward ----------------------------------------------------------------

def moe_backward_workspace_bytes(shape: Shape) -> int:
    return int(load().moe_backward_workspace_bytes(ctypes.byref(shape)))


def moe_combine_backward(shape, dout, y, dest_row, w, dy, dw, stream=None):
    import torch

    act, N = _act_dtype(shape), shape.N
    _ok(load().moe_combine_backward(
        ctypes.byref(shape), _ptr(dout, act, "dout", shape.T * shape.H), _ptr(y, act, "y", N * shape.H),
        _ptr(dest_row, torch.int32, "dest_row", N), _ptr(w, torch.float32, "w", N),
        _ptr(dy, act, "dy", N * shape.H), _ptr(dw, torch.float32, "dw", N), _stream(stream)),
        "moe_combine_backward")


def moe_ffn_backward(shape, buf, plan, w_gate, w_up, w_down, dy, dbuf, dw_gate, dw_up, dw_down,
                     ws, gu=None, stream=None):
    """ws: a uint8 device tensor of at least moe_backward_workspace_bytes(shape);
    gu: None (recompute g | u) or moe_grouped_gemm_train's buffer."""
    import torch

    act, N = _act_dtype(shape), shape.N
    n = shape.E * shape.F * shape.H
    f32 = torch.float32
    _ok(load().moe_ffn_backward(
        ctypes.byref(shape), _ptr(buf, act, "buf", N * shape.H), _ptr(plan, torch.int32, "plan"),
        _ptr(w_gate, act, "w_gate", n), _ptr(w_up, act, "w_up", n), _ptr(w_down, act, "w_down", n),
        _ptr(gu, act, "gu", N * 2 * shape.F, nullable=True), _ptr(dy, act, "dy", N * shape.H), _ptr(dbuf, act, "dbuf", N * shape.H),
        _ptr(dw_gate, f32, "dw_gate", n), _ptr(dw_up, f32, "dw_up", n),
        _ptr(dw_down, f32, "dw_down", n), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
        "moe_ffn_backward")


def moe_permute_backward(shape, dbuf, dest_row, dx, stream=None):
    import torch

    act = _act_dtype(shape)
    _ok(load().moe_permute_backward(
        ctypes.byref(shape), _ptr(dbuf, act, "dbuf", shape.N * shape.H),
        _ptr(dest_row, torch.int32, "dest_row", shape.N), _ptr(dx, act, "dx", shape.T * shape.H),
        _stream(stream)), "moe_permute_backward")


def moe_route_backward(shape, ids, w, dw, dlogits, stream=None):
    import torch

    N = shape.N
    _ok(load().moe_route_backward(
        ctypes.byref(shape), _ptr(ids, torch.int32, "ids", N), _ptr(w, torch.float32, "w", N),
        _ptr(dw, torch.float32, "dw", N), _ptr(dlogits, torch.float32, "dlogits", shape.T * shape.E),
        _stream(stream)), "moe_route_backward")


def moe_grouped_gemm_train(shape, a, plan, w_gate, w_up, w_down, y, gu, ws, stream=None):
    """moe_grouped_gemm that also keeps g | u (bf16 [N][2F], expert order) in gu."""
    import torch

    act, N = _act_dtype(shape), shape.N
    n = shape.E * shape.F * shape.H
    _ok(load().moe_grouped_gemm_train(
        ctypes.byref(shape), _ptr(a, act, "a", N * shape.H), _ptr(plan, torch.int32, "plan"),
        _ptr(w_gate, act, "w_gate", n), _ptr(w_up, act, "w_up", n), _ptr(w_down, act, "w_down", n),
        _ptr(y, act, "y", N * shape.H),
        _ptr(gu, act, "gu", N * 2 * shape.F, nullable=shape.dtype != MOE_BF16),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "moe_grouped_gemm_train")


def moe_replica_grad_bytes(shape: Shape) -> int:
    return int(load().moe_replica_grad_bytes(ctypes.byref(shape)))


def moe_ffn_backward_replicas(shape, buf, plan, w_gate, w_up, w_down, dy, dbuf, dw_gate, dw_up,
                              dw_down, rgrad, ws, gu=None, stream=None):
    """moe_ffn_backward with per-replica gradients in rgrad (float32, at least
    moe_replica_grad_bytes(shape) bytes) reduced into the home experts."""
    import torch

    act, N = _act_dtype(shape), shape.N
    n = shape.E * shape.F * shape.H
    f32 = torch.float32
    _ok(load().moe_ffn_backward_replicas(
        ctypes.byref(shape), _ptr(buf, act, "buf", N * shape.H), _ptr(plan, torch.int32, "plan"),
        _ptr(w_gate, act, "w_gate", n), _ptr(w_up, act, "w_up", n), _ptr(w_down, act, "w_down", n),
        _ptr(gu, act, "gu", N * 2 * shape.F, nullable=True), _ptr(dy, act, "dy", N * shape.H),
        _ptr(dbuf, act, "dbuf", N * shape.H), _ptr(dw_gate, f32, "dw_gate", n),
        _ptr(dw_up, f32, "dw_up", n), _ptr(dw_down, f32, "dw_down", n),
        _ptr(rgrad, f32, "rgrad"), _nbytes(rgrad), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_ffn_backward_replicas")
