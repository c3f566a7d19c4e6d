"""GPU parity of the router's scores (a linear layer, the plain reading of
"DeepEP-on-EFA Guidance, section 1", phase (a)) with the top-k step, and of
the balancing-bias update (an assumed rule: the pages print none) against
the CPU oracle.

Where floating point decides an integer, both sides decide in the same
precision: the GPU's fp32 logits are checked against the oracle's double
logits within the fp32 bar (max|d| <= 1e-5 max|ref|), and the expert ids
against the oracle's top-k applied to those same fp32 logits (bit-exact).
"""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

torch = pytest.importorskip("torch")
import expert_load_balance_amd as moe  # noqa: E402
from expert_load_balance_amd.layer import alloc  # noqa: E402

from test_gpu_parity import DEV, assert_tol, host  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_router(shape, x, wr, bias):
    logits = alloc((shape.T, shape.E), torch.float32, DEV)
    ids = alloc((shape.T, shape.k), torch.int32, DEV)
    w = alloc((shape.T, shape.k), torch.float32, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = alloc((moe.moe_router_workspace_bytes(shape),), torch.uint8, DEV)
    moe.moe_router(shape, x, wr, bias, logits, ids, w, err, ws)
    torch.cuda.synchronize()
    return host(logits), host(ids), host(w), int(err.item())


def check_topk(shape, gl, ids, w, bias_np):
    rid, rw, rerr = oracle.route(gl.astype(np.float32), bias_np, shape.k)
    assert rerr == 0
    np.testing.assert_array_equal(ids, rid)
    assert_tol(w, rw, moe.MOE_F32, "gate weights")


CASES = [
    # T, H, E, k, dtype, bias strength
    (1, 64, 8, 2, moe.MOE_BF16, 0.0),
    (33, 128, 13, 3, moe.MOE_BF16, 0.5),
    (100, 256, 64, 8, moe.MOE_BF16, 0.3),
    (300, 128, 128, 8, moe.MOE_BF16, 0.0),
    (70, 64, 200, 8, moe.MOE_BF16, 1.0),
    (129, 512, 256, 8, moe.MOE_BF16, 0.2),
    # K longer than the LDS ring (15 / 10 / 6 / 3 stages for 32 / 64 / 128 /
    # 256 expert rows): the ring wraps several times
    (40, 2048, 8, 2, moe.MOE_BF16, 0.0),
    (50, 1024, 40, 4, moe.MOE_BF16, 0.2),
    (33, 1280, 100, 4, moe.MOE_BF16, 0.0),
    (16, 64, 8, 2, moe.MOE_F32, 0.0),
    (50, 96, 24, 4, moe.MOE_F32, 0.4),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}H{c[1]}E{c[2]}k{c[3]}{'bf16' if c[4] else 'f32'}"
                                             for c in CASES])
def test_router_small(case):
    T, H, E, k, dtype, sb = case
    _say(f"[case] router T={T} H={H} E={E} k={k}")
    shape = moe.Shape(T, H, E, k, 64, 1, 0, dtype)
    act = torch.bfloat16 if dtype == moe.MOE_BF16 else torch.float32
    x = synth.device_normal((T, H), 1.0, 61, act, DEV)
    wr = synth.device_normal((E, H), synth.weight_std(H), 62, act, DEV)
    bias_np = synth.zipf_bias(E, sb, 63).astype(np.float32) if sb else None
    bias = None if bias_np is None else torch.from_numpy(bias_np).to(DEV)
    gl, ids, w, err = run_router(shape, x, wr, bias)
    assert err == 0
    assert_tol(gl, oracle.router_logits(host(x), host(wr)), moe.MOE_F32, "logits")
    check_topk(shape, gl, ids, w, bias_np)


@pytest.mark.parametrize("name", ["mixtral", "dsv3"])
def test_router_full_size(name):
    _say(f"[case] router full {name}")
    w_ = wl.WORKLOADS[name]
    T, H, E, k = w_["T"], w_["H"], w_["E"], w_["k"]
    shape = moe.Shape(T, H, E, k, 64, 1, 0, moe.MOE_BF16)
    torch.cuda.empty_cache()
    x = synth.device_normal((T, H), 1.0, w_["seed"] * 7 + 1, torch.bfloat16, DEV)
    wr = synth.device_normal((E, H), synth.weight_std(H), w_["seed"] * 10 + 9, torch.bfloat16, DEV)
    gl, ids, w, err = run_router(shape, x, wr, None)
    assert err == 0
    toks = np.unique(np.linspace(0, T - 1, 24).astype(int))
    ref = oracle.router_logits(host(x[toks]), host(wr))
    assert_tol(gl[toks], ref, moe.MOE_F32, "logits (sampled tokens)")
    check_topk(shape, gl, ids, w, None)


def test_bias_update_bit_exact_and_closed_loop():
    T, E, k = 1024, 64, 4
    shape = moe.Shape(T, 64, E, k, 64, 8, 1, moe.MOE_BF16)
    rng = np.random.default_rng(3)
    counts = rng.integers(0, 2 * T * k // E, E).astype(np.int32)
    counts[5] = T * k // E                           # exactly at the mean
    b0 = rng.standard_normal(E).astype(np.float32)
    d_b = torch.from_numpy(b0.copy()).to(DEV)
    moe.moe_bias_update(shape, torch.from_numpy(counts).to(DEV), d_b, 0.0625)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(d_b), oracle.bias_update(counts, b0, 0.0625, N=T * k))
    # closed loop on fixed logits: route -> count -> update, 60 times, on both
    # sides; every step is exact, so the biases agree bit for bit
    lg = synth.router_logits(T, E, 9)
    bias = synth.zipf_bias(E, 0.8, 9).astype(np.float32)
    d_lg = torch.from_numpy(lg).to(DEV)
    d_b = torch.from_numpy(bias.copy()).to(DEV)
    ids = alloc((T, k), torch.int32, DEV)
    w = alloc((T, k), torch.float32, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    cnt = alloc((E,), torch.int32, DEV)
    off = alloc((E + 1,), torch.int32, DEV)
    eidx = alloc((T * k,), torch.int32, DEV)
    rl = alloc((shape.R,), torch.int32, DEV)
    ws = alloc((moe.moe_workspace_bytes(shape),), torch.uint8, DEV)
    ref_b = bias.copy()
    for _ in range(60):
        moe.moe_route(shape, d_lg, d_b, ids, w, err)
        moe.moe_count(shape, ids, cnt, off, eidx, rl, err, ws)
        moe.moe_bias_update(shape, cnt, d_b, 0.01)
        rid, _, _ = oracle.route(lg, ref_b, k)
        ref_b = oracle.bias_update(oracle.count(rid, E, shape.R)["counts"], ref_b, 0.01, N=T * k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(d_b), ref_b)
    c = host(cnt)
    first = oracle.count(oracle.route(lg, bias, k)[0], E, 8)["counts"]
    assert c.max() < first.max()                     # the loop evens out demand


def test_bind_repeats_the_same_call():
    """bind() marshals a wrapper's arguments once; the callable it returns
    makes the same C call(s), here on changed input data."""
    T, H, E, k = 70, 1024, 24, 4
    shape = moe.Shape(T, H, E, k, 64, 1, 0, moe.MOE_BF16)
    assert moe.moe_router_workspace_bytes(shape) > 0  # K split into partial planes
    x = synth.device_normal((T, H), 1.0, 71, torch.bfloat16, DEV)
    wr = synth.device_normal((E, H), synth.weight_std(H), 72, torch.bfloat16, DEV)
    logits = alloc((T, E), torch.float32, DEV)
    ids = alloc((T, k), torch.int32, DEV)
    w = alloc((T, k), torch.float32, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    logits.fill_(float("nan"))
    ws = alloc((moe.moe_router_workspace_bytes(shape),), torch.uint8, DEV)
    run = moe.bind(moe.moe_router, shape, x, wr, None, logits, ids, w, err, ws)
    torch.cuda.synchronize()
    assert np.isnan(host(logits)).all()              # binding launched nothing
    x.copy_(synth.device_normal((T, H), 1.0, 73, torch.bfloat16, DEV))
    run()
    torch.cuda.synchronize()
    gl, gi, gw, e2 = run_router(shape, x, wr, None)
    np.testing.assert_array_equal(host(logits), gl)
    np.testing.assert_array_equal(host(ids), gi)
    np.testing.assert_array_equal(host(w), gw)
    assert e2 == 0
