"""Plain single-threaded CPU oracle for one MoE layer's hot path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP library (``expert_load_balance_amd``) and the library never falls
back to it.

The arithmetic lives in ``oracle.c`` (built with gcc, no fast-math, no FP
contraction); this module only marshals numpy arrays through ctypes. Each
function names the page passage it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

I32P = ctypes.POINTER(ctypes.c_int32)
F32P = ctypes.POINTER(ctypes.c_float)
F64P = ctypes.POINTER(ctypes.c_double)


class Stats(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64),
        ("E", ctypes.c_int32), ("R", ctypes.c_int32),
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
        ("ranks_over_slots", ctypes.c_int32),
        ("nonlocal_rows", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
            "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.orc_route.restype = ctypes.c_int
        lib.orc_count.restype = ctypes.c_int
        lib.orc_plan.restype = ctypes.c_int
        lib.orc_permute.restype = None
        lib.orc_ffn_rows.restype = None
        lib.orc_combine.restype = None
        lib.orc_stats.restype = None
        lib.orc_capacity.restype = ctypes.c_int32
        lib.orc_capacity.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_double]
        lib.orc_hot_share.restype = ctypes.c_double
        lib.orc_capacity_dispatch.restype = None
        lib.orc_repack.restype = None
        lib.orc_router_logits.restype = None
        lib.orc_bias_update.restype = None
        lib.orc_slot_sources.restype = None
        for fn in ("orc_combine_backward", "orc_ffn_backward_rows", "orc_permute_backward",
                   "orc_route_backward"):
            getattr(lib, fn).restype = None
        _lib = lib
    return _lib


def _p(a, typ):
    if a is None:
        return ctypes.cast(None, typ)
    return a.ctypes.data_as(typ)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def route(logits, bias, k):
    """Top-k ids (selection by logit+bias in fp32, ties to the lower id) and
    softmax weights over the selected raw logits, in double. -> (ids, w, err)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    err = _load().orc_route(T, E, k, _p(lg, F32P), _p(b, F32P), _p(ids, I32P), _p(w, F64P))
    return ids, w, err


def count(ids, E, R):
    """Demand counts, exclusive offsets, stable within-expert index and home
    rank loads. -> dict(counts, offsets, eidx, rank_load, err)."""
    ids = _i32(ids)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    eidx = np.empty(T * k, np.int32)
    rank_load = np.empty(R, np.int32)
    err = _load().orc_count(T, k, E, R, _p(ids, I32P), _p(counts, I32P), _p(offsets, I32P),
                            _p(eidx, I32P), _p(rank_load, I32P))
    return dict(counts=counts, offsets=offsets, eidx=eidx, rank_load=rank_load, err=err)


PLAN_TABLES = ("quota", "win_off", "seg_num", "seg_expert", "seg_row", "seg_cnt",
               "slots_needed", "slot_expert", "donor", "piece_num", "piece_rank",
               "piece_row", "piece_cnt")


def plan(counts, R):
    """Equal-load replica plan from the expert demand vector. -> dict of tables."""
    counts = _i32(counts)
    E = counts.shape[0]
    if R <= 0 or E % R:
        raise ValueError("E must be a multiple of R")
    n = E // R
    t = dict(
        quota=np.empty(R, np.int32), win_off=np.empty(R + 1, np.int32),
        seg_num=np.empty(R, np.int32), seg_expert=np.empty((R, 2 * n), np.int32),
        seg_row=np.empty((R, 2 * n), np.int32), seg_cnt=np.empty((R, 2 * n), np.int32),
        slots_needed=np.empty(R, np.int32), slot_expert=np.empty((R, n), np.int32),
        donor=np.empty(R, np.int32), piece_num=np.empty(E, np.int32),
        piece_rank=np.empty((E, R), np.int32), piece_row=np.empty((E, R), np.int32),
        piece_cnt=np.empty((E, R), np.int32),
    )
    rc = _load().orc_plan(E, R, _p(counts, I32P), *[_p(t[name], I32P) for name in PLAN_TABLES])
    if rc != 0:
        raise ValueError("oracle plan rejected its arguments")
    return t


def permute(x, ids, eidx, pl):
    """Row placement of every assignment into the plan's buffer, byte for byte.
    x: [T, H] array of any dtype. -> (buf [N, H], dest_row [T, k], row_src [N])."""
    x = np.ascontiguousarray(x)
    ids = _i32(ids)
    T, k = ids.shape
    E, R = pl["piece_row"].shape
    N = T * k
    buf = np.zeros((N,) + x.shape[1:], x.dtype)
    dest_row = np.empty((T, k), np.int32)
    row_src = np.full(N, -1, np.int32)
    row_bytes = x.strides[0] if x.ndim > 1 else x.itemsize
    _load().orc_permute(T, k, E, R, ctypes.c_size_t(row_bytes), x.ctypes.data_as(ctypes.c_void_p),
                        _p(ids, I32P), _p(_i32(eidx), I32P), _p(_i32(pl["piece_num"]), I32P),
                        _p(_i32(pl["piece_row"]), I32P), _p(_i32(pl["piece_cnt"]), I32P),
                        buf.ctypes.data_as(ctypes.c_void_p), _p(dest_row, I32P), _p(row_src, I32P))
    return buf, dest_row, row_src


def ffn_rows(x, w_gate, w_up, w_down):
    """SwiGLU expert FFN in double on rows x [n, H]; w_gate/w_up [F, H],
    w_down [H, F] (float32 values). -> y [n, H] float64."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    wg = np.ascontiguousarray(w_gate, dtype=np.float32)
    wu = np.ascontiguousarray(w_up, dtype=np.float32)
    wd = np.ascontiguousarray(w_down, dtype=np.float32)
    nrows, H = x.shape
    F = wg.shape[0]
    assert wg.shape == (F, H) and wu.shape == (F, H) and wd.shape == (H, F)
    y = np.empty((nrows, H), np.float64)
    _load().orc_ffn_rows(nrows, H, F, _p(x, F32P), _p(wg, F32P), _p(wu, F32P), _p(wd, F32P),
                         _p(y, F64P))
    return y


def combine(y, dest_row, w, shared=None):
    """out[t] = sum_j w[t,j] * y[dest_row[t,j]] (+ shared[t]), in double."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    dest_row = _i32(dest_row)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, k = dest_row.shape
    H = y.shape[1]
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.float64)
    out = np.empty((T, H), np.float64)
    _load().orc_combine(T, k, H, _p(y, F64P), _p(dest_row, I32P), _p(w, F64P), _p(sh, F64P),
                        _p(out, F64P))
    return out


def router_logits(x, w_router):
    """logit[t][e] = sum_h x[t][h] * W_r[e][h], in double from float inputs."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w_router, dtype=np.float32)
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), np.float64)
    _load().orc_router_logits(T, E, H, _p(x, F32P), _p(w, F32P), _p(out, F64P))
    return out


def bias_update(counts, bias, gamma, N=None):
    """Sign-rule bias update (an assumption; see oracle.c) around the mean
    demand N / E (N defaults to the sum of counts). -> new fp32 bias."""
    c = _i32(counts)
    b = np.array(bias, dtype=np.float32, copy=True)
    n = int(c.sum()) if N is None else int(N)
    _load().orc_bias_update(c.shape[0], ctypes.c_int64(n), _p(c, I32P),
                            ctypes.c_float(gamma), _p(b, F32P))
    return b


def capacity_dispatch(x, ids, eidx, E, cap):
    """Fixed-capacity dispatch: buf [E*cap][...] (padding rows zero) and
    dest_row (-1 where the assignment is dropped), byte-exact rows."""
    x = np.ascontiguousarray(x)
    ids = _i32(ids)
    eidx = _i32(eidx).reshape(ids.shape)
    T, k = ids.shape
    row_bytes = x.strides[0] if x.ndim > 1 else x.itemsize
    buf = np.empty((E * cap,) + x.shape[1:], x.dtype)
    dest_row = np.empty((T, k), np.int32)
    _load().orc_capacity_dispatch(T, k, E, cap, ctypes.c_size_t(row_bytes),
                                  x.ctypes.data_as(ctypes.c_void_p), _p(ids, I32P), _p(eidx, I32P),
                                  buf.ctypes.data_as(ctypes.c_void_p), _p(dest_row, I32P))
    return buf, dest_row


def repack(counts, R):
    """Greedy balanced packing of experts onto R ranks (n = E/R each):
    mapping[e] = rank."""
    c = _i32(counts)
    mapping = np.empty(c.shape[0], np.int32)
    _load().orc_repack(c.shape[0], int(R), _p(c, I32P), _p(mapping, I32P))
    return mapping


def capacity(N, E, factor):
    """Per-expert capacity ceil(N / E * factor), evaluated in that order."""
    return int(_load().orc_capacity(int(N), int(E), float(factor)))


def hot_share(counts, g):
    """Share of the g hottest experts over their even share g/E."""
    c = _i32(counts)
    return float(_load().orc_hot_share(c.shape[0], _p(c, I32P), int(g)))


def stats(ids, counts, R, S=0, mapping=None, origin=None, dest_row=None, pl=None,
          capacity_factor=1.0):
    """Load statistics (maxvio, balancedness, capacity ledger sums, remote
    routes, replica/slot figures). -> dict."""
    ids = _i32(ids)
    T, k = ids.shape
    counts = _i32(counts)
    E = counts.shape[0]
    mp = None if mapping is None else _i32(mapping)
    og = None if origin is None else _i32(origin)
    dr = None if dest_row is None else _i32(dest_row)
    tabs = {}
    if pl is not None:
        for name in ("win_off", "seg_num", "seg_expert", "seg_cnt", "slots_needed", "slot_expert"):
            tabs[name] = _i32(pl[name])
    out = Stats()
    home = np.zeros(R, np.int32)
    mapped = np.zeros(R, np.int32)
    planned = np.zeros(R, np.int32)
    _load().orc_stats(T, k, E, R, S, _p(counts, I32P), _p(ids, I32P), _p(mp, I32P), _p(og, I32P),
                      _p(dr, I32P), _p(tabs.get("win_off"), I32P), _p(tabs.get("seg_num"), I32P),
                      _p(tabs.get("seg_expert"), I32P), _p(tabs.get("seg_cnt"), I32P),
                      _p(tabs.get("slots_needed"), I32P), _p(tabs.get("slot_expert"), I32P),
                      ctypes.c_double(capacity_factor), _p(home, I32P), _p(mapped, I32P),
                      _p(planned, I32P), ctypes.byref(out))
    d = out.as_dict()
    d["home_load"] = home
    d["mapped_load"] = mapped if mapping is not None else None
    d["planned_load"] = planned if pl is not None else None
    return d


def ledgers(counts, cap):
    """Per-expert processed / overflow / padding vectors at capacity cap."""
    c = np.asarray(counts, dtype=np.int64)
    return np.minimum(c, cap), np.maximum(c - cap, 0), np.maximum(cap - c, 0)


def slot_sources(pl, S):
    """Weight source of every plan segment under S replica slots per rank:
    src [R, 2n] int32 = slot index j, -1 for the home expert's weights, -2
    past the rank's segment count. (orc_slot_sources)"""
    R, n = pl["slot_expert"].shape
    src = np.empty((R, 2 * n), np.int32)
    _load().orc_slot_sources(R * n, R, int(S), _p(_i32(pl["seg_num"]), I32P),
                             _p(_i32(pl["seg_expert"]), I32P), _p(_i32(pl["slot_expert"]), I32P),
                             _p(src, I32P))
    return src


def prefetch(pl, S, w_gate, w_up, w_down):
    """The replica slot pool: pool[r, j] holds copies of (W_gate, W_up, W_down)
    of rank r's j-th replica expert, flattened, for j < min(S, n) and
    slot_expert[r, j] >= 0; slots without an expert stay zero.
    w_gate, w_up: [E, F, H]; w_down: [E, H, F] (any dtype). -> [R, Sm, 3, F*H]."""
    R, n = pl["slot_expert"].shape
    Sm = min(int(S), n)
    E, F, H = w_gate.shape
    pool = np.zeros((R, Sm, 3, F * H), w_gate.dtype)
    for r in range(R):
        for j in range(Sm):
            e = int(pl["slot_expert"][r, j])
            if e >= 0:
                pool[r, j, 0] = w_gate[e].ravel()
                pool[r, j, 1] = w_up[e].ravel()
                pool[r, j, 2] = w_down[e].ravel()
    return pool


def slot_ffn(buf, pl, S, w_gate, w_up, w_down, pool):
    """The expert FFN of every buffer row, segment by segment, with each
    segment's weights taken from its source (slot_sources): home weights or
    pool[r, j] (whatever that slot holds). buf [N, H] -> y [N, H] double."""
    R, n = pl["slot_expert"].shape
    E, F, H = w_gate.shape
    src = slot_sources(pl, S)
    y = np.zeros((buf.shape[0], H))
    for r in range(R):
        for i in range(int(pl["seg_num"][r])):
            e, row, cnt = (int(pl[t][r, i]) for t in ("seg_expert", "seg_row", "seg_cnt"))
            if cnt == 0:
                continue
            j = int(src[r, i])
            if j >= 0:
                wg, wu, wd = (pool[r, j, q].reshape(shp) for q, shp in
                              ((0, (F, H)), (1, (F, H)), (2, (H, F))))
            else:
                wg, wu, wd = w_gate[e], w_up[e], w_down[e]
            y[row:row + cnt] = ffn_rows(buf[row:row + cnt], wg, wu, wd)
    return y


# ---- backward (the chain rule of the forward functions above, in double) ----

def combine_backward(dout, y, dest_row, w):
    """dy [nrows, H] (w * dout scattered to the assignment rows) and dw [T, k]
    (<dout[t], y[dest]>). (orc_combine_backward)"""
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    dest_row = _i32(dest_row)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, k = dest_row.shape
    nrows, H = y.shape
    dy = np.empty((nrows, H), np.float64)
    dw = np.empty((T, k), np.float64)
    _load().orc_combine_backward(T, k, H, ctypes.c_int64(nrows), _p(dout, F64P), _p(y, F64P),
                                 _p(dest_row, I32P), _p(w, F64P), _p(dy, F64P), _p(dw, F64P))
    return dy, dw


def ffn_backward_rows(x, dy, w_gate, w_up, w_down):
    """SwiGLU FFN backward on rows x [n, H] of one expert given dy [n, H].
    -> (dx [n, H], dW_gate [F, H], dW_up [F, H], dW_down [H, F]), double.
    (orc_ffn_backward_rows)"""
    x = np.ascontiguousarray(x, dtype=np.float32)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    wg = np.ascontiguousarray(w_gate, dtype=np.float32)
    wu = np.ascontiguousarray(w_up, dtype=np.float32)
    wd = np.ascontiguousarray(w_down, dtype=np.float32)
    n, H = x.shape
    F = wg.shape[0]
    dx = np.empty((n, H), np.float64)
    dwg = np.zeros((F, H), np.float64)
    dwu = np.zeros((F, H), np.float64)
    dwd = np.zeros((H, F), np.float64)
    _load().orc_ffn_backward_rows(n, H, F, _p(x, F32P), _p(dy, F64P), _p(wg, F32P), _p(wu, F32P),
                                  _p(wd, F32P), _p(dx, F64P), _p(dwg, F64P), _p(dwu, F64P),
                                  _p(dwd, F64P))
    return dx, dwg, dwu, dwd


def permute_backward(dbuf, dest_row):
    """dx [T, H] = sum_j dbuf[dest[t, j]]. (orc_permute_backward)"""
    dbuf = np.ascontiguousarray(dbuf, dtype=np.float64)
    dest_row = _i32(dest_row)
    T, k = dest_row.shape
    nrows, H = dbuf.shape
    dx = np.empty((T, H), np.float64)
    _load().orc_permute_backward(T, k, H, ctypes.c_int64(nrows), _p(dbuf, F64P),
                                 _p(dest_row, I32P), _p(dx, F64P))
    return dx


def route_backward(ids, w, dw, E):
    """dlogits [T, E] of the gate weights' softmax over the selected raw
    logits. (orc_route_backward)"""
    ids = _i32(ids)
    T, k = ids.shape
    w = np.ascontiguousarray(w, dtype=np.float64)
    dw = np.ascontiguousarray(dw, dtype=np.float64)
    dl = np.empty((T, E), np.float64)
    _load().orc_route_backward(T, E, k, _p(ids, I32P), _p(w, F64P), _p(dw, F64P), _p(dl, F64P))
    return dl


def expert_ffn_backward(buf, dy, pl, w_gate, w_up, w_down):
    """The grouped FFN backward over the plan: every expert's rows (all of
    its pieces, home and replicas) through ffn_backward_rows; each expert's
    weight gradient is the sum over all of its rows -- the replicas'
    contributions reduced into the home expert.
    -> (dbuf [N, H], dW_gate [E, F, H], dW_up [E, F, H], dW_down [E, H, F])."""
    E, F, H = w_gate.shape
    dbuf = np.zeros((buf.shape[0], H))
    dwg = np.zeros((E, F, H))
    dwu = np.zeros((E, F, H))
    dwd = np.zeros((E, H, F))
    for e in range(E):
        rows = []
        for p in range(int(pl["piece_num"][e])):
            r0, c = int(pl["piece_row"][e, p]), int(pl["piece_cnt"][e, p])
            rows.extend(range(r0, r0 + c))
        if not rows:
            continue
        rows = np.array(rows)
        dx, dwg[e], dwu[e], dwd[e] = ffn_backward_rows(buf[rows], dy[rows], w_gate[e], w_up[e],
                                                       w_down[e])
        dbuf[rows] = dx
    return dbuf, dwg, dwu, dwd


def replica_backward(buf, dy, pl, w_gate, w_up, w_down):
    """The replica-gradient reduction written out (MoonEP article, paragraph
    3: replica gradients are reduced into the home expert): each expert's home
    piece gives the home part of its gradient; each replica piece (rank r,
    slot j of slot_expert[r]) gives a slot gradient from its own rows; the
    expert's gradient is the home part plus its slots in rank order.
    -> (dW_gate, dW_up, dW_down reduced, slots {(r, j): (g, u, d)})."""
    E, F, H = w_gate.shape
    R, n = pl["slot_expert"].shape
    dwg = np.zeros((E, F, H))
    dwu = np.zeros((E, F, H))
    dwd = np.zeros((E, H, F))
    slots = {}
    parts = {e: [] for e in range(E)}
    for e in range(E):
        for p in range(int(pl["piece_num"][e])):
            r = int(pl["piece_rank"][e, p])
            r0, c = int(pl["piece_row"][e, p]), int(pl["piece_cnt"][e, p])
            if c == 0:
                continue
            _, g, u, d = ffn_backward_rows(buf[r0:r0 + c], dy[r0:r0 + c], w_gate[e], w_up[e],
                                           w_down[e])
            if r == e // n:
                dwg[e] += g
                dwu[e] += u
                dwd[e] += d
            else:
                j = int(np.where(pl["slot_expert"][r] == e)[0][0])
                slots[(r, j)] = (g, u, d)
                parts[e].append((r, j))
    for e in range(E):
        for r, j in sorted(parts[e]):
            g, u, d = slots[(r, j)]
            dwg[e] += g
            dwu[e] += u
            dwd[e] += d
    return dwg, dwu, dwd, slots
