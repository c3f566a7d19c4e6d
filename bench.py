#!/usr/bin/env python3
"""One MoE layer forward (route -> count -> plan -> permute -> grouped SwiGLU
GEMM -> combine) on one MI355X, timed over K steps after W warm-up steps.

Default workload: the DeepSeek-V3-shaped layer in bf16 (T=8192 tokens,
H=7168, 256 routed experts top-8 plus one always-on shared expert, SwiGLU
width 2048, R=32 virtual ranks, S=8) at router skew maxvio 20, with the same
layer at maxvio 0 reported beside it. Inputs are seeded and synthetic and
already resident in HBM when timing starts.

Timing: before every timed step a 512 MB device write evicts the L2 and the
Infinity Cache; each step is bracketed by HIP events on the layer's stream,
and the K steps by synchronisations. `value` = T / mean step time.

Prints ONE JSON line. `roofline` describes the dominant kernel group, the
routed grouped GEMM (schedule + gate/up + down calls): algorithmic bytes
(active experts' weights once + buffer rows read + output rows written) or
flops per call, whichever bound is tighter, over its HIP-event duration;
`cpu_baseline` times the CPU oracle, pinned to one core, on the same
workload (a baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/s at maxvio 0/1/20; grouped-GEMM MFMA % and permute HBM %"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--maxvio", type=float, default=None,
                    help="router skew target (default: the workload's first)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the other workloads / skews reported beside the headline")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only the layer (skip the isolated router, replica-slot and "
                         "fixed-capacity measurements, which launch the same GEMM kernels); "
                         "for kernel traces and counters of the layer alone")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the training step of the workload: the training forward (g|u "
                         "kept) and the backward chain, --steps times; one JSON line of its "
                         "figures (for kernel traces of the backward)")
    ap.add_argument("--cpu-ffn-rows", type=int, default=None,
                    help="buffer rows in the oracle's timed FFN sample (default: 256 * k, "
                         "256 tokens' worth of assignments)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (a known "
                         "byte count for calibrating HBM counters), then exit")
    return ap.parse_args()


def kernel_src_sha():
    p = os.path.join(ROOT, "expert_load_balance_amd", "csrc", "gemm.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traffic_for(workload, maxvio):
    """HBM bytes per call of the routed grouped GEMM (its kernels' launches,
    summed) from committed counter runs, or None if absent or taken on a
    different kernel source."""
    p = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    rec = d.get(f"{workload}@{maxvio:g}")
    if not rec or rec.get("kernel_src_sha") != kernel_src_sha():
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(name, maxvio, lg, bias, x, wts, shared, n_ffn_rows=None, n_shared_tokens=64):
    """The oracle, as it stands, on the same workload, single-threaded and
    pinned to one host core. Route, count, plan, permute and combine run on
    every token; the SwiGLU FFN runs on the first `n_ffn_rows` rows of the
    buffer (by default 256 * k: 256 tokens' worth of assignments, about 30 s
    on the DeepSeek-V3 shape; all rows when they fit) and the shared expert
    on the first `n_shared_tokens` tokens; both are extrapolated per row to
    the whole layer (every row costs the same 3*H*F multiply-adds). Host
    copies of the inputs are made before the clock starts."""
    import numpy as np

    import oracle
    from synth.workloads import WORKLOADS

    w = WORKLOADS[name]
    T, H, E, k, F, R = (w[c] for c in ("T", "H", "E", "k", "F", "R"))
    N = T * k
    n_rows = max(1, min(N, n_ffn_rows or 256 * k))
    xs = x.float().cpu().numpy()
    ids0, _, _ = oracle.route(lg, bias, k)
    c0 = oracle.count(ids0, E, R)
    pl0 = oracle.plan(c0["counts"], R)
    # experts owning the first n_rows buffer rows (window order), and their weights
    seg = []
    for r in range(R):
        for i in range(int(pl0["seg_num"][r])):
            seg.append((int(pl0["seg_row"][r, i]), int(pl0["seg_cnt"][r, i]),
                        int(pl0["seg_expert"][r, i])))
    seg.sort()
    take = [(r0, min(cnt, n_rows - r0), e) for r0, cnt, e in seg if r0 < n_rows and cnt > 0]
    used = sorted({e for _, _, e in take})
    wh = {e: tuple(t[e].float().cpu().numpy() for t in wts) for e in used}
    sh = tuple(t[0].float().cpu().numpy() for t in shared) if shared is not None else None
    n_sh = min(T, max(1, n_shared_tokens)) if shared is not None else 0

    prev = os.sched_getaffinity(0)
    core = min(prev)
    os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        ids, gw, _ = oracle.route(lg, bias, k)
        c = oracle.count(ids, E, R)
        pl = oracle.plan(c["counts"], R)
        buf, dest_row, _ = oracle.permute(xs, ids, c["eidx"], pl)
        t1 = time.perf_counter()
        y = np.zeros((N, H))
        for r0, cnt, e in take:
            y[r0:r0 + cnt] = oracle.ffn_rows(buf[r0:r0 + cnt], *wh[e])
        t2 = time.perf_counter()
        if n_sh:
            oracle.ffn_rows(xs[:n_sh], *sh)
        t3 = time.perf_counter()
        oracle.combine(y, dest_row, gw)
        t4 = time.perf_counter()
    finally:
        os.sched_setaffinity(0, prev)
    t_ffn_row = (t2 - t1) / n_rows
    t_sh_row = (t3 - t2) / n_sh if n_sh else 0.0
    t_layer = (t1 - t0) + (t4 - t3) + t_ffn_row * N + t_sh_row * (T if shared is not None else 0)
    extrap = n_rows < N or (shared is not None and n_sh < T)
    sample = (f"route, count, plan, permute and combine on all {T} tokens "
              f"({(t1 - t0) + (t4 - t3):.1f} s); SwiGLU FFN on the first {n_rows} of {N} buffer rows "
              f"({t2 - t1:.1f} s)"
              + (f" and the shared expert on {n_sh} of {T} tokens ({t3 - t2:.1f} s)" if n_sh else "")
              + (", extrapolated per row to the whole layer" if extrap else "")
              + f"; plain single-threaded C in double, pinned to core {core}")
    return dict(value=T / t_layer, unit="tokens/s", cores=1, kind="oracle", sample=sample,
                ffn_extrapolated=extrap, seconds_measured=t4 - t0,
                cpu_model=cpu_model(), nproc=os.cpu_count(), affinity_cores=len(prev))


class Flusher:
    """Writes a 512 MB device buffer, then reads another one: more than the
    256 MB Infinity Cache and the L2s, so the next kernel reads its operands
    from HBM. The read evicts the written lines, so their write-back happens
    here and not inside the next kernel."""

    def __init__(self, nbytes=512 << 20):
        import torch

        self.buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
        self.rbuf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
        self.wg = 4 * torch.cuda.get_device_properties(0).multi_processor_count
        self.sink = torch.empty(self.wg * 256, dtype=torch.int32, device="cuda")
        self.v = 0

    def __call__(self):
        import expert_load_balance_amd as moe

        self.v ^= 0x5A5A5A5A
        self.buf.fill_(self.v)
        moe.moe_probe_read(self.rbuf, self.wg, self.sink)


def time_back_to_back(fn, reps=50):
    """Mean duration of one call when `reps` calls run back to back on the
    current stream (launch gaps amortised, caches warm), in seconds."""
    import torch

    for _ in range(5):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / reps


def time_flushed(fn, flush, reps=30):
    """Mean HIP-event duration of one call on the current stream with the
    caches flushed before each call, in seconds."""
    import torch

    for _ in range(3):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) * 1e-3 / reps


def measured_peaks():
    """Measured counterparts of the spec peaks: the bf16 MFMA rate of the
    library's calibration probe (four workgroups per CU, registers only,
    operands that change from one MFMA to the next), the faster of two
    2 GiB device-to-device copies (the runtime's and the library's streaming
    copy probe) and the library's read probe over 4 GiB, with the caches
    flushed before each copy and read."""
    import torch

    import expert_load_balance_amd as moe

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg, iters = 4 * cus, 2048
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def probe():
        moe.moe_probe_mfma(wg, iters, sink, stream=stream)

    t_settle = time.perf_counter() + 0.2
    while time.perf_counter() < t_settle:
        probe()
        torch.cuda.synchronize()
    t_mfma = time_back_to_back(probe, reps=20)
    flops = wg * 4 * 4 * iters * 2.0 * 32 * 32 * 16
    flush = Flusher()
    # 4 GiB: long enough that the launch, the ramp and the write-back of the
    # flush's dirty lines weigh little (a flushed 1 GiB read measured about
    # 20 % below a flushed 4 GiB one)
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    half = big.numel() // 2
    a, b = big[:half], big[half:]
    t_rt = time_flushed(lambda: b.copy_(a), flush, reps=5)
    t_probe = time_flushed(lambda: moe.moe_probe_copy(a, b, 8 * cus, stream=stream), flush, reps=5)
    rsink = torch.empty(4 * cus * 256, dtype=torch.int32, device="cuda")
    t_read = time_flushed(lambda: moe.moe_probe_read(big, 4 * cus, rsink, stream=stream), flush, reps=5)
    del a, b, big, flush, sink, rsink
    torch.cuda.empty_cache()
    rt, pr = 2.0 * half / t_rt / 1e9, 2.0 * half / t_probe / 1e9
    rd = 2.0 * half / t_read / 1e9
    return {"mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1),
            "hbm_copy_gbs": round(max(rt, pr), 1),
            "hbm_copy_runtime_gbs": round(rt, 1), "hbm_copy_probe_gbs": round(pr, 1),
            "hbm_read_gbs": round(rd, 1),
            "how": f"moe_probe_mfma: {wg} workgroups x 4 waves x {4 * iters} "
                   "v_mfma_f32_32x32x16_bf16, back to back; 2 GiB device copy (2 GiB read + "
                   "2 GiB written) by the runtime and by moe_probe_copy "
                   f"({8 * cus} workgroups), the faster one; 4 GiB read by moe_probe_read "
                   f"({4 * cus} workgroups, one contiguous chunk each); 512 MB flush before "
                   "each copy and read"}


def time_capacity_layer(shape, lg, bias, x, wts, cf, steps, warmup, L=None, shared=None):
    """The same layer through the fixed-capacity baseline: route, count,
    dispatch into [E][cap] (drop and pad), the expert FFN over the whole
    static buffer, (the shared expert, through L's buffers,) combine. Returns
    tokens/s and the drop / padding figures."""
    import torch

    import expert_load_balance_amd as moe
    from expert_load_balance_amd.layer import alloc

    s = shape
    i32 = torch.int32
    act = x.dtype
    cap = moe.moe_capacity_rows(s, cf)
    cs = moe.capacity_shape(s, cap)
    ws = alloc((moe.moe_workspace_bytes(s),), torch.uint8, "cuda")
    ws2 = alloc((moe.moe_workspace_bytes(cs),), torch.uint8, "cuda")
    ids, w = alloc((s.T, s.k), i32, "cuda"), alloc((s.T, s.k), torch.float32, "cuda")
    err = torch.zeros(1, dtype=i32, device="cuda")
    counts, offsets = alloc((s.E,), i32, "cuda"), alloc((s.E + 1,), i32, "cuda")
    eidx, rank_load = alloc((s.N,), i32, "cuda"), alloc((s.R,), i32, "cuda")
    buf, y = alloc((s.E * cap, s.H), act, "cuda"), alloc((s.E * cap, s.H), act, "cuda")
    dest, out = alloc((s.T, s.k), i32, "cuda"), alloc((s.T, s.H), act, "cuda")
    plan = alloc((moe.moe_plan_layout(cs)["total"],), i32, "cuda")
    moe.moe_capacity_plan(s, cap, plan)      # static: the layout does not depend on the routing

    def step():
        moe.moe_route(s, lg, bias, ids, w, err)
        moe.moe_count(s, ids, counts, offsets, eidx, rank_load, err, ws)
        moe.moe_capacity_dispatch(s, cap, counts, x, ids, eidx, buf, dest)
        moe.moe_grouped_gemm(cs, buf, plan, *wts, y, ws2)
        sy = None
        if shared is not None:
            moe.moe_grouped_gemm(L.shared_shape, x, L.shared_plan, *shared, L.shared_y, L.shared_ws)
            sy = L.shared_y
        moe.moe_capacity_combine(s, cap, y, dest, w, sy, out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    c = counts.cpu()
    kept = int(torch.minimum(c, torch.tensor(cap)).sum())
    return {"capacity_factor": cf, "capacity": cap, "tokens_per_s": s.T / dt,
            "ms_per_step": dt * 1e3, "dropped_assignments": s.N - kept,
            "padding_rows": s.E * cap - kept, "gemm_rows": s.E * cap}


def time_router(shape, x, bias, seed, act, stream, flush):
    """The router's scores + top-k (x read once; W_r is E x H), caches flushed
    before each call. Returns (seconds per call, algorithmic bytes)."""
    import torch

    import expert_load_balance_amd as moe
    import synth

    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    dev = "cuda"
    wr = synth.device_normal((E, H), synth.weight_std(H), seed * 10 + 9, act, dev)
    r_logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    r_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    r_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    r_err = torch.zeros(1, dtype=torch.int32, device=dev)
    r_ws = torch.empty(max(1, moe.moe_router_workspace_bytes(shape)), dtype=torch.uint8, device=dev)
    t = time_flushed(moe.bind(moe.moe_router, shape, x, wr, bias, r_logits, r_ids, r_w,
                              r_err, r_ws, stream=stream), flush)
    nbytes = (T * H + E * H) * (2 if shape.dtype == moe.MOE_BF16 else 4) + T * E * 4 * 2
    return t, nbytes


def time_backward(shape, L, lg, bias, x, wts, shared, seed, stream):
    """The layer's backward from a seeded dout: combine, the expert FFN
    (dgrad + wgrad, from the g | u a training forward kept; and with the
    recompute), dispatch and gate backward, each back to back on the stream;
    the whole chain; and a training step = the training forward + the chain."""
    import torch

    import expert_load_balance_amd as moe
    import synth

    T, H, E, k, F = shape.T, shape.H, shape.E, shape.k, shape.F
    N = T * k
    dev = "cuda"
    act = torch.bfloat16
    dout = synth.device_normal((T, H), 1.0, seed * 10 + 7, act, dev)
    dy = torch.empty((N, H), dtype=act, device=dev)
    dw = torch.empty((T, k), dtype=torch.float32, device=dev)
    dbuf = torch.empty((N, H), dtype=act, device=dev)
    dx = torch.empty((T, H), dtype=act, device=dev)
    dl = torch.empty((T, E), dtype=torch.float32, device=dev)
    dW = [torch.empty((E, F, H), dtype=torch.float32, device=dev),
          torch.empty((E, F, H), dtype=torch.float32, device=dev),
          torch.empty((E, H, F), dtype=torch.float32, device=dev)]
    ws = torch.empty(moe.moe_backward_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    gu = torch.empty((N, 2 * F), dtype=act, device=dev)
    L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream, gu=gu)
    c_comb = moe.bind(moe.moe_combine_backward, shape, dout, L.y, L.dest_row, L.w, dy, dw,
                      stream=stream)
    c_ffn = moe.bind(moe.moe_ffn_backward, shape, L.buf, L.plan, *wts, dy, dbuf, *dW, ws, gu=gu,
                     stream=stream)
    c_ffn_re = moe.bind(moe.moe_ffn_backward, shape, L.buf, L.plan, *wts, dy, dbuf, *dW, ws,
                        stream=stream)
    rgrad = torch.empty(moe.moe_replica_grad_bytes(shape) // 4, dtype=torch.float32, device=dev)
    c_ffn_rep = moe.bind(moe.moe_ffn_backward_replicas, shape, L.buf, L.plan, *wts, dy, dbuf, *dW,
                         rgrad, ws, gu=gu, stream=stream)
    c_perm = moe.bind(moe.moe_permute_backward, shape, dbuf, L.dest_row, dx, stream=stream)
    c_route = moe.bind(moe.moe_route_backward, shape, L.ids, L.w, dw, dl, stream=stream)

    def chain():
        c_comb()
        c_ffn()
        c_perm()
        c_route()

    def step():
        L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream, gu=gu)
        chain()

    t_comb = time_back_to_back(c_comb, reps=20)
    t_ffn = time_back_to_back(c_ffn, reps=5)
    t_ffn_re = time_back_to_back(c_ffn_re, reps=5)
    t_ffn_rep = time_back_to_back(c_ffn_rep, reps=5)
    del rgrad
    t_perm = time_back_to_back(c_perm, reps=20)
    t_route = time_back_to_back(c_route, reps=20)
    t_all = time_back_to_back(chain, reps=5)
    t_step = time_back_to_back(step, reps=5)
    flops = 12.0 * N * H * F      # dh 2, dx 4, dW_down 2, dW_gate|up 4 (x N H F)
    del dW, ws, gu
    return dict(ms=t_all * 1e3, combine_backward_us=t_comb * 1e6, ffn_backward_ms=t_ffn * 1e3,
                permute_backward_us=t_perm * 1e6, route_backward_us=t_route * 1e6,
                ffn_backward_tflops=flops / t_ffn / 1e12,
                ffn_backward_mfma_frac=flops / t_ffn / 1e12 / PEAK_BF16_TFLOPS,
                ffn_backward_recompute_ms=t_ffn_re * 1e3,
                ffn_backward_replica_slots_ms=t_ffn_rep * 1e3,
                train_step_ms=t_step * 1e3, train_step_tokens_per_s=T / t_step)


def time_slots(shape, L, lg, bias, x, wts, shared, steps, stream):
    """Replica slots: the prefetch copy of every filled slot, the grouped GEMM
    by plan segment reading them beside the expert-grouped GEMM, and the whole
    layer with both."""
    import torch

    import expert_load_balance_amd as moe

    T, H, E, F, R, S = shape.T, shape.H, shape.E, shape.F, shape.R, shape.S
    pool_bytes = moe.moe_pool_bytes(shape)
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    n = E // R
    se = moe.plan_tables(L.plan, shape)["slot_expert"].cpu().numpy()[:, :min(S, n)]
    filled = int((se >= 0).sum())
    t_pref = time_back_to_back(moe.bind(moe.moe_prefetch_replicas, shape, L.plan, *wts, pool,
                                        stream=stream), reps=10)
    t_gs = time_back_to_back(moe.bind(moe.moe_grouped_gemm_slots, shape, L.buf, L.plan, *wts,
                                      pool, L.y, L.ws, stream=stream), reps=10)
    t_ge = time_back_to_back(moe.bind(moe.moe_grouped_gemm, shape, L.buf, L.plan, *wts, L.y,
                                      L.ws, stream=stream), reps=10)
    moved = 2.0 * filled * 3 * F * H * (2 if shape.dtype == moe.MOE_BF16 else 4)  # read + write
    for _ in range(2):
        L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream, pool=pool)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream, pool=pool)
    torch.cuda.synchronize()
    t_layer = (time.perf_counter() - t1) / steps
    del pool
    return dict(S=S, slots_filled=filled, pool_gb=pool_bytes / 1e9,
                prefetch_us=t_pref * 1e6, prefetch_gbs=moved / t_pref / 1e9,
                prefetch_hbm_frac=moved / t_pref / 1e9 / PEAK_HBM_GBS,
                gemm_slots_ms=t_gs * 1e3, gemm_experts_ms=t_ge * 1e3,
                layer_tokens_per_s=T / t_layer, layer_ms_per_step=t_layer * 1e3)


def run_workload(name, maxvio, steps, warmup, capacity_factor=None, extras=True):
    """Builds one workload on the GPU, runs `warmup` + `steps` layer steps and
    returns its measurements (plus the inputs, for the CPU baseline); with a
    capacity factor, also the fixed-capacity baseline on the same inputs."""
    import torch

    import expert_load_balance_amd as moe
    from expert_load_balance_amd.layer import STAGES, MoeLayerBuffers
    import synth
    from synth import workloads as wl

    w = wl.WORKLOADS[name]
    dtype = moe.MOE_BF16 if w["dtype"] == "bf16" else moe.MOE_F32
    act = torch.bfloat16 if dtype == moe.MOE_BF16 else torch.float32
    T, H, E, k, F, R, S = (w[c] for c in ("T", "H", "E", "k", "F", "R", "S"))
    shape = moe.Shape(T, H, E, k, F, R, S, dtype)
    dev = "cuda"

    lg_np, bias_np = wl.logits_and_bias(name, maxvio)
    lg = torch.from_numpy(lg_np).to(dev)
    bias = None if bias_np is None else torch.from_numpy(bias_np).to(dev)
    x = synth.device_normal((T, H), 1.0, w["seed"] * 7 + 1, act, dev)
    wts = (synth.device_normal((E, F, H), synth.weight_std(H), w["seed"] * 10 + 1, act, dev),
           synth.device_normal((E, F, H), synth.weight_std(H), w["seed"] * 10 + 2, act, dev),
           synth.device_normal((E, H, F), synth.weight_std(F), w["seed"] * 10 + 3, act, dev))
    shared_F = w.get("shared_F")
    shared = None
    if shared_F:
        shared = (synth.device_normal((1, shared_F, H), synth.weight_std(H), w["seed"] * 10 + 501, act, dev),
                  synth.device_normal((1, shared_F, H), synth.weight_std(H), w["seed"] * 10 + 502, act, dev),
                  synth.device_normal((1, H, shared_F), synth.weight_std(shared_F), w["seed"] * 10 + 503, act, dev))
    L = MoeLayerBuffers(shape, dev, shared_F=shared_F)
    stream = torch.cuda.current_stream()

    flush = Flusher()

    def fwd(marks=None):
        L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream, marks=marks)

    # Untimed: the GPU's clocks settle over the first ~10 steps of load (the
    # first steps after idle run 5-15 % slower), so the layer runs in batches
    # of steps for about 0.2 s before the counted warm-up steps.
    t_settle = time.perf_counter() + 0.2
    while time.perf_counter() < t_settle:
        for _ in range(10):
            fwd()
        torch.cuda.synchronize()
    for _ in range(warmup):
        flush()
        fwd()
    torch.cuda.synchronize()
    print(f"[bench] {name}@{maxvio:g} warm-up done", file=sys.stderr, flush=True)

    # Timed steps: caches flushed before each, the step and its routed grouped
    # GEMM bracketed by HIP events on the layer's stream.
    def ev():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    step_ev = [ev() for _ in range(steps)]
    gemm_ev = [ev() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        step_ev[i][0].record(stream)
        fwd(marks={"gemm": gemm_ev[i]})
        step_ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def dist(pairs):
        v = sorted(a.elapsed_time(b) for a, b in pairs)
        return dict(mean=sum(v) / len(v), median=v[len(v) // 2], p10=v[len(v) // 10],
                    p90=v[(len(v) * 9) // 10])

    step_ms = dist(step_ev)
    gemm_ms = dist(gemm_ev)

    # the same steps back to back without flushes (warm caches, no events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    warm_s = (time.perf_counter() - t1) / steps

    # per-stage breakdown: a second flushed pass with events between stages
    marks = [{s: ev() for s in STAGES} for _ in range(steps)]
    for i in range(steps):
        flush()
        fwd(marks=marks[i])
    torch.cuda.synchronize()
    stage_ms = {}
    for s in STAGES:
        if s == "shared" and shared is None:
            continue
        stage_ms[s] = dist([m[s] for m in marks])

    # the row moves and the top-k alone, caches flushed before each launch
    t_perm = time_flushed(moe.bind(moe.moe_permute, shape, x, L.ids, L.eidx, L.plan, L.buf,
                                   L.dest_row, L.row_src, stream=stream), flush)
    sy = L.shared_y if shared else None
    t_comb = time_flushed(moe.bind(moe.moe_combine, shape, L.y, L.dest_row, L.w, sy, L.out,
                                   stream=stream), flush)
    # the runtime's device-to-device copy of as many bytes as the dispatch
    # moves (half read, half written), timed the same way: the ceiling of a
    # row move of this size, launch and ramp included
    half = (T + T * k) * H * (2 if dtype == moe.MOE_BF16 else 4) // 2
    cp_src = torch.empty(half, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    t_copy = time_flushed(lambda: cp_dst.copy_(cp_src), flush)
    del cp_src, cp_dst
    route_ids = torch.empty_like(L.ids)
    route_w = torch.empty_like(L.w)
    route_err = torch.zeros_like(L.err)
    t_route = time_flushed(moe.bind(moe.moe_route, shape, lg, bias, route_ids, route_w, route_err,
                                    stream=stream), flush)
    del route_ids, route_w, route_err

    t_router = router_bytes = None
    if extras:
        t_router, router_bytes = time_router(shape, x, bias, w["seed"], act, stream, flush)

    slots = None
    if extras and moe.moe_pool_bytes(shape):
        slots = time_slots(shape, L, lg, bias, x, wts, shared, steps, stream)

    bwd = None
    if extras and dtype == moe.MOE_BF16:
        bwd = time_backward(shape, L, lg, bias, x, wts, shared, w["seed"], stream)

    cap_res = None
    if capacity_factor is not None and extras:
        cap_res = time_capacity_layer(shape, lg, bias, x, wts, capacity_factor, steps, warmup,
                                      L=L, shared=shared)
    del flush

    st, _ = moe.moe_stats(shape, L.counts, L.ids, L.plan, L.ws, dest_row=L.dest_row,
                          err=L.err, capacity_factor=w.get("capacity_factor", 1.0))
    N = T * k
    b = 2 if dtype == moe.MOE_BF16 else 4
    gu_s = stage_ms["gemm_gateup"]["mean"] * 1e-3
    dn_s = stage_ms["gemm_down"]["mean"] * 1e-3
    gemm_s = gemm_ms["mean"] * 1e-3
    gemm_flops = 6.0 * N * H * F
    # algorithmic bytes of the routed grouped GEMM: every active expert's three
    # projections read once, the buffer rows read once, the output rows
    # written once (the h round trip between the two calls is not counted)
    gemm_bytes = st["active_experts"] * 3.0 * F * H * b + 2.0 * N * H * b
    perm_bytes = (T + N) * H * b
    comb_bytes = (N + T) * H * b + (T * H * b if shared else 0)
    route_bytes = T * E * 4 + (E * 4 if bias is not None else 0) + T * k * 8
    res = dict(
        name=name, maxvio=maxvio, shape=(T, H, E, k, F, R, S), shared_F=shared_F, dtype=dtype,
        tokens_per_s=T / (step_ms["mean"] * 1e-3), ms_per_step=step_ms["mean"], step_ms=step_ms,
        wall_s=wall, warm_tokens_per_s=T / warm_s, warm_ms_per_step=warm_s * 1e3,
        stage_ms=stage_ms, gemm_ms=gemm_ms,
        gemm_flops=gemm_flops, gemm_bytes=gemm_bytes,
        gemm_tflops=gemm_flops / gemm_s / 1e12, gemm_gbs=gemm_bytes / gemm_s / 1e9,
        gemm_mfma_frac=gemm_flops / gemm_s / 1e12 / PEAK_BF16_TFLOPS,
        gemm_hbm_frac=gemm_bytes / gemm_s / 1e9 / PEAK_HBM_GBS,
        gemm_bound="hbm" if gemm_bytes / PEAK_HBM_GBS > gemm_flops / 1e3 / PEAK_BF16_TFLOPS
        else "mfma",
        gu_tflops=4.0 * N * H * F / gu_s / 1e12, dn_tflops=2.0 * N * H * F / dn_s / 1e12,
        permute_us=t_perm * 1e6, combine_us=t_comb * 1e6, route_us=t_route * 1e6,
        copy_same_bytes_us=t_copy * 1e6,
        permute_hbm_frac=perm_bytes / t_perm / 1e9 / PEAK_HBM_GBS,
        combine_hbm_frac=comb_bytes / t_comb / 1e9 / PEAK_HBM_GBS,
        route_hbm_frac=route_bytes / t_route / 1e9 / PEAK_HBM_GBS,
        permute_hbm_frac_in_layer=perm_bytes / (stage_ms["permute"]["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        combine_hbm_frac_in_layer=comb_bytes / (stage_ms["combine"]["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        stats=st, inputs=(lg_np, bias_np, x, wts, shared), capacity=cap_res, slots=slots,
        backward=bwd,
        shared_gemm=None if shared is None else {
            "ms": stage_ms["shared"]["mean"],
            "mfma_frac": 6.0 * T * H * shared_F / (stage_ms["shared"]["mean"] * 1e-3) / 1e12
            / PEAK_BF16_TFLOPS},
        router=None if t_router is None else {
            "us": t_router * 1e6, "tflops": 2.0 * T * E * H / t_router / 1e12,
            "hbm_frac": router_bytes / t_router / 1e9 / PEAK_HBM_GBS})
    return res


# Every other shape and skew point of the workload list, reported beside the
# headline (layer tokens/s, grouped-GEMM fractions, permute / combine / route
# HBM fractions); decode at the feasible maximum skew (15) for the maxvio-20
# request.
SWEEP = (("mixtral", 0.2), ("a3b", 0.0), ("a3b", 0.2), ("a3b", 1.0),
         ("decode64", 1.0), ("decode64", 20.0), ("decode256", 1.0), ("decode256", 20.0),
         ("decode1024", 1.0), ("decode1024", 20.0))


def summary(q):
    """The per-point figures of a run_workload result (rounded)."""
    def r4(v):
        return None if v is None else round(v, 4)

    out = {
        "tokens_per_s": round(q["tokens_per_s"]), "ms_per_step": r4(q["ms_per_step"]),
        "step_ms_p10_p90": [r4(q["step_ms"]["p10"]), r4(q["step_ms"]["p90"])],
        "warm_tokens_per_s": round(q["warm_tokens_per_s"]),
        "maxvio_realised": r4(q["stats"]["maxvio_expert"]),
        "active_experts": q["stats"]["active_experts"],
        "gemm_ms": r4(q["gemm_ms"]["mean"]), "gemm_bound": q["gemm_bound"],
        "gemm_hbm_frac": r4(q["gemm_hbm_frac"]), "grouped_gemm_mfma_frac": r4(q["gemm_mfma_frac"]),
        "gemm_gateup_tflops": round(q["gu_tflops"], 1), "gemm_down_tflops": round(q["dn_tflops"], 1),
        "permute_hbm_frac": r4(q["permute_hbm_frac"]), "combine_hbm_frac": r4(q["combine_hbm_frac"]),
        "route_hbm_frac": r4(q["route_hbm_frac"]),
        "permute_us": round(q["permute_us"], 2), "combine_us": round(q["combine_us"], 2),
        "copy_same_bytes_as_permute_us": round(q["copy_same_bytes_us"], 2),
        "route_us": round(q["route_us"], 2),
        "plan": {k_: q["stats"][k_] for k_ in ("planned_max", "planned_min", "replica_pieces",
                                               "max_slots_needed", "ranks_over_slots")},
        "stages_ms": {s_: r4(v["mean"]) for s_, v in q["stage_ms"].items()},
    }
    if q["shared_gemm"] is not None:
        out["shared_gemm"] = {k_: r4(v_) for k_, v_ in q["shared_gemm"].items()}
    if q["router"] is not None:
        out["router_us"] = round(q["router"]["us"], 2)
    if q["backward"] is not None:
        out["backward"] = {k_: round(v_, 3) for k_, v_ in q["backward"].items()}
    if q["slots"] is not None:
        out["replica_slots"] = {k_: round(v_, 3) if isinstance(v_, float) else v_
                                for k_, v_ in q["slots"].items()}
    if q["capacity"] is not None:
        cq = q["capacity"]
        out["fixed_capacity_cf1.25"] = {"tokens_per_s": round(cq["tokens_per_s"]),
                                        "dropped_assignments": cq["dropped_assignments"],
                                        "padding_rows": cq["padding_rows"]}
    return out


def run_backward_only(args):
    """The workload's training step alone: warm-up, then --steps training
    forwards (keeping g|u) each followed by the backward chain (combine, FFN
    from the kept g|u, dispatch, gate), bracketed by synchronisations."""
    import torch

    import expert_load_balance_amd as moe
    from expert_load_balance_amd.layer import MoeLayerBuffers
    import synth
    from synth import workloads as wl

    name = args.workload
    w = wl.WORKLOADS[name]
    maxvio = args.maxvio if args.maxvio is not None else w["maxvio"][0]
    T, H, E, k, F, R, S = (w[c] for c in ("T", "H", "E", "k", "F", "R", "S"))
    shape = moe.Shape(T, H, E, k, F, R, S, moe.MOE_BF16)
    dev, act = "cuda", torch.bfloat16
    lg_np, bias_np = wl.logits_and_bias(name, maxvio)
    lg = torch.from_numpy(lg_np).to(dev)
    bias = None if bias_np is None else torch.from_numpy(bias_np).to(dev)
    x = synth.device_normal((T, H), 1.0, w["seed"] * 7 + 1, act, dev)
    wts = (synth.device_normal((E, F, H), synth.weight_std(H), w["seed"] * 10 + 1, act, dev),
           synth.device_normal((E, F, H), synth.weight_std(H), w["seed"] * 10 + 2, act, dev),
           synth.device_normal((E, H, F), synth.weight_std(F), w["seed"] * 10 + 3, act, dev))
    L = MoeLayerBuffers(shape, dev)
    N = T * k
    gu = torch.empty((N, 2 * F), dtype=act, device=dev)
    dout = synth.device_normal((T, H), 1.0, w["seed"] * 10 + 7, act, dev)
    dy = torch.empty((N, H), dtype=act, device=dev)
    dw = torch.empty((T, k), dtype=torch.float32, device=dev)
    dbuf = torch.empty((N, H), dtype=act, device=dev)
    dx = torch.empty((T, H), dtype=act, device=dev)
    dl = torch.empty((T, E), dtype=torch.float32, device=dev)
    dW = [torch.empty((E, F, H), dtype=torch.float32, device=dev),
          torch.empty((E, F, H), dtype=torch.float32, device=dev),
          torch.empty((E, H, F), dtype=torch.float32, device=dev)]
    ws = torch.empty(moe.moe_backward_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        L.forward(lg, bias, x, *wts, stream=stream, gu=gu)
        moe.moe_combine_backward(shape, dout, L.y, L.dest_row, L.w, dy, dw, stream=stream)
        moe.moe_ffn_backward(shape, L.buf, L.plan, *wts, dy, dbuf, *dW, ws, gu=gu, stream=stream)
        moe.moe_permute_backward(shape, dbuf, L.dest_row, dx, stream=stream)
        moe.moe_route_backward(shape, L.ids, L.w, dw, dl, stream=stream)

    # untimed clock settling, as in run_workload
    t_settle = time.perf_counter() + 0.2
    while time.perf_counter() < t_settle:
        for _ in range(3):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / args.steps
    return {"metric": "MoE-layer training step (forward + backward) tokens/s", "value": T / t,
            "unit": "tokens/s", "steps": args.steps, "warmup": args.warmup, "ms_per_step": t * 1e3,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{name} T={T} H={H} E={E} k={k} F={F} R={R} S={S}",
                       "maxvio_target": maxvio}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this layer is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        a = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": 2 * a.numel() * a.element_size()}))
        return

    import expert_load_balance_amd as moe
    from synth import workloads as wl

    moe.load()
    if args.backward_only:
        print(json.dumps(run_backward_only(args)), flush=True)
        return
    name = args.workload
    w = wl.WORKLOADS[name]
    maxvio = args.maxvio if args.maxvio is not None else w["maxvio"][0]
    r = run_workload(name, maxvio, args.steps, args.warmup, capacity_factor=1.25,
                     extras=not args.layer_only)
    T, H, E, k, F, R, S = r["shape"]
    shared_F = r["shared_F"]
    st = r["stats"]
    hbm = r["gemm_bound"] == "hbm"
    rec = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if r["dtype"] == moe.MOE_BF16 else "f32",
        "data": "synthetic (seeded N(0,1) router logits + Zipf expert bias, N(0,1) activations, "
                "N(0,1/sqrt(fan_in)) weights)",
        "config": {"workload": f"{name} T={T} H={H} E={E} k={k} F={F} R={R} S={S}"
                               + (f" shared_F={shared_F}" if shared_F else ""),
                   "maxvio_target": maxvio, "maxvio_realised": st["maxvio_expert"],
                   "global_batch": T, "parallelism": "1 GPU, R virtual ranks"},
        "timing": "HIP events per step on the layer's stream, 512 MB cache flush before each "
                  "step; value = T / mean step",
        "step_ms": {k_: round(v_, 4) for k_, v_ in r["step_ms"].items()},
        "warm_back_to_back": {"tokens_per_s": r["warm_tokens_per_s"],
                              "ms_per_step": r["warm_ms_per_step"]},
        "roofline": {"bound": r["gemm_bound"],
                     "achieved": r["gemm_gbs"] if hbm else r["gemm_tflops"],
                     "peak": PEAK_HBM_GBS if hbm else PEAK_BF16_TFLOPS,
                     "unit": "GB/s" if hbm else "TFLOP/s",
                     "frac": r["gemm_hbm_frac"] if hbm else r["gemm_mfma_frac"],
                     "traffic": traffic_for(name, maxvio),
                     "kernel": "routed grouped GEMM: schedule_kernel + gemm_bf16_kernel<0> + "
                               "fixup_kernel<0> + gemm_bf16_kernel<1> + fixup_kernel<1>",
                     "ms_per_call": r["gemm_ms"]["mean"],
                     "bytes_per_call": r["gemm_bytes"], "flops_per_call": r["gemm_flops"],
                     "mfma_frac": r["gemm_mfma_frac"], "hbm_frac": r["gemm_hbm_frac"]},
    }
    rec.update({k_: v_ for k_, v_ in summary(r).items()
                if k_ not in ("tokens_per_s", "ms_per_step")})
    rec["gemm_src_sha16"] = kernel_src_sha()
    if not args.layer_only:
        mp = measured_peaks()
        rec["measured_peaks"] = mp
        rec["roofline"]["frac_of_measured_peak"] = (
            r["gemm_gbs"] / mp["hbm_copy_gbs"] if hbm else r["gemm_tflops"] / mp["mfma_bf16_tflops"])
        rec["roofline"]["mfma_frac_of_measured_peak"] = r["gemm_tflops"] / mp["mfma_bf16_tflops"]
        if hbm:  # the GEMM's bytes are mostly weight reads: against a plain read stream too
            rec["roofline"]["frac_of_measured_read_peak"] = r["gemm_gbs"] / mp["hbm_read_gbs"]
    if not args.no_cpu_baseline:
        lg_np, bias_np, x, wts, shared = r["inputs"]
        rec["cpu_baseline"] = cpu_baseline(name, maxvio, lg_np, bias_np, x, wts, shared,
                                           n_ffn_rows=args.cpu_ffn_rows)
    del r
    torch.cuda.empty_cache()
    # the workload's other skew points beside the headline (dsv3: maxvio 0)
    others = [m for m in w["maxvio"] if m is not None and m != maxvio]
    if others and args.maxvio is None:
        comp = {}
        for m in others:
            q = run_workload(name, m, args.steps, args.warmup, capacity_factor=1.25,
                             extras=not args.layer_only)
            comp[f"{name}@{m:g}"] = summary(q)
            comp[f"{name}@{m:g}"]["gemm_traffic"] = traffic_for(name, m)
            del q
            torch.cuda.empty_cache()
        rec["companion"] = comp
    if not args.no_sweep and not args.layer_only:
        sweep = {}
        for sname, smv in SWEEP:
            if sname == name:
                continue
            q = run_workload(sname, smv, 10, 3, capacity_factor=1.25)
            sweep[f"{sname}@{smv:g}"] = summary(q)
            del q
            torch.cuda.empty_cache()
        rec["sweep"] = sweep
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
