#!/usr/bin/env python3
"""One MoE layer forward (route -> count -> plan -> permute -> grouped SwiGLU
GEMM -> combine) on one MI355X, timed over K steps after W warm-up steps.

Default workload: the Mixtral-style coarse layer in bf16 (T=2048 tokens,
H=4096, E=8 experts, top-2, SwiGLU width 14336, R=8 virtual ranks, S=1),
router skew maxvio 0.2 (N(0,1) logits plus a tuned Zipf bias). Inputs are
seeded and synthetic and already resident in HBM when timing starts.

Prints ONE JSON line. `value` is whole-layer tokens/s; `roofline` describes
the dominant kernel (the gate/up half of the grouped GEMM), timed with HIP
events on the stream it runs on; `cpu_baseline` times the CPU oracle on a
bounded token sample of the same workload (a baseline, not a target).
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
    ap.add_argument("--workload", default="mixtral")
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
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens in the oracle's timed sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (a known "
                         "byte count for calibrating HBM counters), then exit")
    return ap.parse_args()


def kernel_src_sha():
    p = os.path.join(ROOT, "expert_load_balance_amd", "csrc", "gemm.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(workload, maxvio):
    """HBM bytes per launch of the gate/up kernel from committed counter runs,
    or None if absent or taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "gemm_gateup_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    rec = d.get(f"{workload}@{maxvio:g}")
    if not rec or rec.get("kernel_src_sha") != kernel_src_sha():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(name, maxvio, lg, bias, x, wts, ntok):
    """The oracle, as it stands, on the first `ntok` tokens of the workload.
    Host copies of the inputs (only the experts those tokens use) are made
    before the clock starts."""
    import numpy as np

    import oracle
    from synth.workloads import WORKLOADS

    w = WORKLOADS[name]
    E, k, R = w["E"], w["k"], w["R"]
    xs = x[:ntok].float().cpu().numpy()
    used = sorted(set(oracle.route(lg[:ntok], bias, k)[0].ravel().tolist()))
    wg, wu, wd = ({e: t[e].float().cpu().numpy() for e in used} for t in wts)
    t0 = time.perf_counter()
    ids, gw, _ = oracle.route(lg[:ntok], bias, k)
    c = oracle.count(ids, E, R)
    pl = oracle.plan(c["counts"], R)
    buf, dest_row, row_src = oracle.permute(xs, ids, c["eidx"], pl)
    y = np.zeros((ntok * k, xs.shape[1]))
    for e in range(E):
        rows = []
        for p in range(pl["piece_num"][e]):
            rows.extend(range(pl["piece_row"][e, p], pl["piece_row"][e, p] + pl["piece_cnt"][e, p]))
        if rows:
            y[rows] = oracle.ffn_rows(buf[rows], wg[e], wu[e], wd[e])
    oracle.combine(y, dest_row, gw)
    dt = time.perf_counter() - t0
    return dict(value=ntok / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"first {ntok} of {w['T']} tokens of the same workload, full layer "
                       f"(route, count, plan, permute, SwiGLU FFN, combine), "
                       f"single-threaded C in double, {dt:.1f} s")


def time_back_to_back(fn, reps=50):
    """Mean duration of one call when `reps` calls run back to back on the
    current stream (launch gaps amortised), in seconds."""
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


def time_router(shape, x, bias, seed, act, stream):
    """The router's scores + top-k (x read once; W_r is E x H), back to back.
    Returns (seconds per call, algorithmic bytes)."""
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
    t = time_back_to_back(moe.bind(moe.moe_router, shape, x, wr, bias, r_logits, r_ids, r_w,
                                   r_err, r_ws, stream=stream))
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

    # Untimed: the GPU's clocks settle over the first ~10 steps of load (the
    # first steps after idle run 5-15 % slower), so the layer runs in batches
    # of steps for about 0.2 s before the counted warm-up steps.
    t_settle = time.perf_counter() + 0.2
    while time.perf_counter() < t_settle:
        for _ in range(10):
            L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream)
        torch.cuda.synchronize()
    for _ in range(warmup):
        L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream)
    torch.cuda.synchronize()
    print(f"[bench] {name}@{maxvio:g} warm-up done", file=sys.stderr, flush=True)

    # the timed steps carry no event records (those sit between kernels in
    # the queue); a second pass with per-stage events gives the breakdown
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    marks = [{s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for s in STAGES} for _ in range(steps)]
    for i in range(steps):
        L.forward(lg, bias, x, *wts, shared_w=shared, stream=stream, marks=marks[i])
    torch.cuda.synchronize()

    stage_ms = {}
    for s in STAGES:
        if s == "shared" and shared is None:
            continue
        v = sorted(m[s][0].elapsed_time(m[s][1]) for m in marks)
        stage_ms[s] = dict(mean=sum(v) / len(v), p10=v[len(v) // 10], p90=v[(len(v) * 9) // 10])

    # the two row moves alone, back to back (their in-layer stage times also
    # hold a launch gap each)
    t_perm = time_back_to_back(moe.bind(moe.moe_permute, shape, x, L.ids, L.eidx, L.plan, L.buf,
                                        L.dest_row, L.row_src, stream=stream))
    sy = L.shared_y if shared else None
    t_comb = time_back_to_back(moe.bind(moe.moe_combine, shape, L.y, L.dest_row, L.w, sy, L.out,
                                        stream=stream))

    t_router = router_bytes = None
    if extras:
        t_router, router_bytes = time_router(shape, x, bias, w["seed"], act, stream)

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

    st, _ = moe.moe_stats(shape, L.counts, L.ids, L.plan, L.ws, dest_row=L.dest_row,
                          err=L.err, capacity_factor=w.get("capacity_factor", 1.0))
    N = T * k
    b = 2 if dtype == moe.MOE_BF16 else 4
    gu_s = stage_ms["gemm_gateup"]["mean"] * 1e-3
    dn_s = stage_ms["gemm_down"]["mean"] * 1e-3
    gu_flops = 4.0 * N * H * F
    dn_flops = 2.0 * N * H * F
    perm_bytes = (T + N) * H * b
    comb_bytes = (N + T) * H * b + (T * H * b if shared else 0)
    res = dict(
        name=name, maxvio=maxvio, shape=(T, H, E, k, F, R, S), shared_F=shared_F, dtype=dtype,
        tokens_per_s=T * steps / elapsed, ms_per_step=elapsed * 1e3 / steps, stage_ms=stage_ms,
        gu_flops=gu_flops, gu_tflops=gu_flops / gu_s / 1e12, dn_tflops=dn_flops / dn_s / 1e12,
        gemm_mfma_frac=(gu_flops + dn_flops) / (gu_s + dn_s) / 1e12 / PEAK_BF16_TFLOPS,
        permute_us=t_perm * 1e6, combine_us=t_comb * 1e6,
        permute_hbm_frac=perm_bytes / t_perm / 1e9 / PEAK_HBM_GBS,
        combine_hbm_frac=comb_bytes / t_comb / 1e9 / PEAK_HBM_GBS,
        permute_hbm_frac_in_layer=perm_bytes / (stage_ms["permute"]["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        combine_hbm_frac_in_layer=comb_bytes / (stage_ms["combine"]["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        stats=st, inputs=(lg_np, bias_np, x, wts), capacity=cap_res, slots=slots, backward=bwd,
        # weight-streaming view of the two GEMM calls: every active expert's
        # three projections read once (the bound when rows per expert are few)
        gemm_weight_hbm_frac=st["active_experts"] * 3.0 * F * H * b / (gu_s + dn_s) / 1e9
        / PEAK_HBM_GBS,
        router=None if t_router is None else {
            "us": t_router * 1e6, "tflops": 2.0 * T * E * H / t_router / 1e12,
            "hbm_frac": router_bytes / t_router / 1e9 / PEAK_HBM_GBS})
    return res


# Other workloads and skews reported beside the headline line (layer tokens/s,
# grouped-GEMM MFMA fraction, permute / combine HBM fractions); decode at the
# feasible maximum skew (15) for the maxvio-20 request.
SWEEP = (("a3b", 0.0), ("a3b", 0.2), ("a3b", 1.0), ("dsv3", 20.0), ("dsv3", 0.0),
         ("decode64", 1.0), ("decode256", 20.0), ("decode1024", 1.0), ("decode1024", 20.0))


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
    traffic = traffic_for(name, maxvio)
    achieved = r["gu_tflops"]
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
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "kernel": "gemm_bf16_kernel<0> (gate/up call)",
                     "flops_per_launch": r["gu_flops"]},
        "stages_ms": {s: round(v["mean"], 4) for s, v in r["stage_ms"].items()},
        "gemm_down_tflops": r["dn_tflops"],
        "grouped_gemm_mfma_frac": r["gemm_mfma_frac"],
        "permute_hbm_frac": r["permute_hbm_frac"],
        "combine_hbm_frac": r["combine_hbm_frac"],
        "permute_us": r["permute_us"],
        "combine_us": r["combine_us"],
        "permute_hbm_frac_in_layer": r["permute_hbm_frac_in_layer"],
        "combine_hbm_frac_in_layer": r["combine_hbm_frac_in_layer"],
        "plan": {"planned_max": st["planned_max"], "planned_min": st["planned_min"],
                 "replica_pieces": st["replica_pieces"], "max_slots_needed": st["max_slots_needed"],
                 "ranks_over_slots": st["ranks_over_slots"]},
        "fixed_capacity_baseline": r["capacity"],
        "router_scores_topk": r["router"],
        "replica_slots": r["slots"],
        "backward": r["backward"],
        "gemm_weight_hbm_frac": r["gemm_weight_hbm_frac"],
    }
    if not args.no_cpu_baseline:
        # about 5e10 multiply-adds of FFN work: 10-30 s for the plain C oracle
        ntok = args.cpu_tokens or max(1, min(T, int(5e10 / (k * 3 * H * F))))
        lg_np, bias_np, x, wts = r["inputs"]
        rec["cpu_baseline"] = cpu_baseline(name, maxvio, lg_np, bias_np, x, wts, ntok)
    del r
    torch.cuda.empty_cache()
    if not args.no_sweep and not args.layer_only:
        sweep = {}
        for sname, smv in SWEEP:
            q = run_workload(sname, smv, 10, 3, capacity_factor=1.25)
            cq = q["capacity"]
            sweep[f"{sname}@{smv:g}"] = {
                "tokens_per_s": round(q["tokens_per_s"]), "ms_per_step": round(q["ms_per_step"], 4),
                "maxvio_realised": round(q["stats"]["maxvio_expert"], 4),
                "grouped_gemm_mfma_frac": round(q["gemm_mfma_frac"], 4),
                "gemm_gateup_tflops": round(q["gu_tflops"], 1),
                "gemm_down_tflops": round(q["dn_tflops"], 1),
                "permute_hbm_frac": round(q["permute_hbm_frac"], 4),
                "combine_hbm_frac": round(q["combine_hbm_frac"], 4),
                "router_us": round(q["router"]["us"], 2),
                "gemm_weight_hbm_frac": round(q["gemm_weight_hbm_frac"], 4),
                "backward": None if q["backward"] is None else {
                    k_: round(v_, 3) for k_, v_ in q["backward"].items()},
                "replica_slots": None if q["slots"] is None else {
                    k_: round(v_, 3) if isinstance(v_, float) else v_
                    for k_, v_ in q["slots"].items()},
                "fixed_capacity_cf1.25": {"tokens_per_s": round(cq["tokens_per_s"]),
                                          "dropped_assignments": cq["dropped_assignments"],
                                          "padding_rows": cq["padding_rows"]}}
            del q
            torch.cuda.empty_cache()
        rec["sweep"] = sweep
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
