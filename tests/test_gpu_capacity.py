"""GPU parity of the two baselines the equal-load plan replaces -- the
fixed-capacity dispatch (drop and pad) with the expert FFN over the static
[E][cap] buffer, and the greedy repacking of experts onto ranks -- against
the CPU oracle ("MoE Load Balancing: Find Expert Hotspots", sections "Make
expert capacity, overflow, and padding explicit" and "Separate expert demand
from rank placement").

Bar as in test_gpu_parity: bit-exact for dest_row, the buffer (padding rows
included), the capacity plan tables and the mapping; max|d| <= 2e-2 max|ref|
(bf16) or 1e-5 max|ref| (fp32) for the FFN and combine outputs.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

torch = pytest.importorskip("torch")
import expert_load_balance_amd as moe  # noqa: E402
from expert_load_balance_amd.layer import alloc  # noqa: E402

from test_gpu_parity import DEV, assert_tol, host, make_weights, raw_bits  # noqa: E402

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _say(msg):
    print(msg, flush=True)


class CapacityRun:
    """route -> count -> capacity dispatch -> FFN over [E*cap] -> combine, and
    the repacking, all through the C ABI."""

    def __init__(self, shape, lg, bias, x, wts, cf):
        s = shape
        i32 = torch.int32
        act = torch.bfloat16 if s.dtype == moe.MOE_BF16 else torch.float32
        self.shape = s
        ws = alloc((moe.moe_workspace_bytes(s),), torch.uint8, DEV)
        self.ids = alloc((s.T, s.k), i32, DEV)
        self.w = alloc((s.T, s.k), torch.float32, DEV)
        self.err = torch.zeros(1, dtype=i32, device=DEV)
        self.counts = alloc((s.E,), i32, DEV)
        offsets = alloc((s.E + 1,), i32, DEV)
        self.eidx = alloc((s.N,), i32, DEV)
        rank_load = alloc((s.R,), i32, DEV)
        lgd = alloc(lg.shape, torch.float32, DEV)
        lgd.copy_(torch.from_numpy(lg))
        bd = None if bias is None else torch.from_numpy(bias).to(DEV)
        moe.moe_route(s, lgd, bd, self.ids, self.w, self.err)
        moe.moe_count(s, self.ids, self.counts, offsets, self.eidx, rank_load, self.err, ws)
        self.cap = cap = moe.moe_capacity_rows(s, cf)
        assert cap >= 1
        self.buf = alloc((s.E * cap, s.H), act, DEV)
        self.dest = alloc((s.T, s.k), i32, DEV)
        moe.moe_capacity_dispatch(s, cap, self.counts, x, self.ids, self.eidx, self.buf, self.dest)
        cs = moe.capacity_shape(s, cap)
        self.plan = alloc((moe.moe_plan_layout(cs)["total"],), i32, DEV)
        self.plan.fill_(-7)
        moe.moe_capacity_plan(s, cap, self.plan)
        ws2 = alloc((moe.moe_workspace_bytes(cs),), torch.uint8, DEV)
        self.y = alloc((s.E * cap, s.H), act, DEV)
        moe.moe_grouped_gemm(cs, self.buf, self.plan, *wts, self.y, ws2)
        self.out = alloc((s.T, s.H), act, DEV)
        moe.moe_capacity_combine(s, cap, self.y, self.dest, self.w, None, self.out)
        self.mapping = alloc((s.E,), i32, DEV)
        moe.moe_repack(s, self.counts, self.mapping)
        torch.cuda.synchronize()
        assert int(self.err.item()) == 0


def bits_to_f64(bits):
    """Raw bf16 (int16) or fp32 (int32) bits as float64 values."""
    if bits.dtype == np.int16:
        return (bits.astype(np.int32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float32).astype(np.float64)


def check_dispatch_and_plan(run, x_bits, lg, bias):
    """Bit-exact against the oracle's route, count, capacity dispatch and
    repacking on the same inputs. Returns the oracle's (dest_row, buf as
    float64, ids, gate weights, counts)."""
    s, cap = run.shape, run.cap
    ids, w, _ = oracle.route(lg, bias, s.k)
    c = oracle.count(ids, s.E, s.R)
    np.testing.assert_array_equal(host(run.ids), ids, err_msg="ids")
    np.testing.assert_array_equal(host(run.eidx), c["eidx"], err_msg="eidx")
    np.testing.assert_array_equal(host(run.counts), c["counts"], err_msg="counts")
    buf, dest = oracle.capacity_dispatch(x_bits, ids, c["eidx"], s.E, cap)
    np.testing.assert_array_equal(host(run.dest), dest, err_msg="dest_row")
    np.testing.assert_array_equal(host(raw_bits(run.buf)), buf, err_msg="buf (padding included)")
    # the capacity plan: expert e home on rank e / n, one piece of cap rows at e * cap
    n = s.E // s.R
    t = moe.plan_tables(run.plan, s)
    e = np.arange(s.E)
    np.testing.assert_array_equal(host(t["quota"]), np.full(s.R, n * cap))
    np.testing.assert_array_equal(host(t["win_off"]), np.arange(s.R + 1) * n * cap)
    np.testing.assert_array_equal(host(t["piece_num"]), np.ones(s.E))
    np.testing.assert_array_equal(host(t["piece_row"])[:, 0], e * cap)
    np.testing.assert_array_equal(host(t["piece_cnt"])[:, 0], np.full(s.E, cap))
    np.testing.assert_array_equal(host(t["piece_rank"])[:, 0], e // n)
    np.testing.assert_array_equal(host(t["slots_needed"]), np.zeros(s.R))
    np.testing.assert_array_equal(host(t["seg_num"]), np.full(s.R, n))
    np.testing.assert_array_equal(host(t["seg_expert"])[:, :n], e.reshape(s.R, n))
    assert not (host(run.plan) == -7).any()
    np.testing.assert_array_equal(host(run.mapping), oracle.repack(c["counts"], s.R),
                                  err_msg="mapping")
    return dest, bits_to_f64(buf), ids, w, c["counts"]


SMALL = [
    # name, T, H, E, k, F, R, dtype, bias strength, capacity factor
    ("f32_drops", 60, 64, 8, 2, 96, 4, moe.MOE_F32, 0.8, 0.75),
    ("bf16_drops", 300, 128, 16, 4, 192, 4, moe.MOE_BF16, 0.6, 1.0),
    ("bf16_pads", 200, 256, 8, 2, 128, 2, moe.MOE_BF16, 0.0, 2.0),
    ("bf16_fine_grained", 256, 128, 64, 8, 128, 16, moe.MOE_BF16, 0.4, 1.25),
    ("bf16_tiny_cap", 40, 64, 8, 2, 64, 8, moe.MOE_BF16, 1.0, 0.1),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_capacity_path_small(case):
    name, T, H, E, k, F, R, dtype, s_bias, cf = case
    _say(f"[case] capacity {name}")
    shape = moe.Shape(T, H, E, k, F, R, 1, dtype)
    lg = synth.router_logits(T, E, 31)
    bias = synth.zipf_bias(E, s_bias, 31) if s_bias else None
    act = torch.bfloat16 if dtype == moe.MOE_BF16 else torch.float32
    x = synth.device_normal((T, H), 1.0, 41, act, DEV)
    wts = make_weights(E, F, H, dtype, 6)
    run = CapacityRun(shape, lg, bias, x, wts, cf)
    dest, bufh, ids, w, _ = check_dispatch_and_plan(run, host(raw_bits(x)), lg, bias)
    # the FFN over every row of the static buffer (padding rows give zeros)
    wg, wu, wd = (host(t) for t in wts)
    y_ref = np.concatenate([oracle.ffn_rows(bufh[e * run.cap:(e + 1) * run.cap], wg[e], wu[e], wd[e])
                            for e in range(E)])
    assert_tol(host(run.y), y_ref, dtype, "y")
    pad = np.abs(bufh).sum(1) == 0
    assert not host(run.y)[pad].any()
    out_ref = oracle.combine(y_ref, dest, w)
    assert_tol(host(run.out), out_ref, dtype, "out")
    if cf < 1.0:
        assert (dest < 0).any()          # the case really drops


def test_capacity_fixture_fp32():
    """The 16-token hotspot fixture at capacity factor 1.25 (cap 5)."""
    with open(os.path.join(GOLD, "fixture16.json")) as f:
        fix = json.load(f)
    shape = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_F32)
    lg, bias = wl.fixture()
    x = synth.device_normal((16, 64), 1.0, 5, torch.float32, DEV)
    wts = make_weights(8, 128, 64, moe.MOE_F32, 1)
    run = CapacityRun(shape, lg, bias, x, wts, 1.25)
    assert run.cap == fix["capacity"] == 5
    dest, bufh, ids, _, _ = check_dispatch_and_plan(run, host(raw_bits(x)), lg, bias)
    kept = np.bincount(ids.ravel()[dest.ravel() >= 0], minlength=8)
    np.testing.assert_array_equal(kept, fix["processed"])
    assert (dest < 0).sum() == sum(fix["overflow"]) == 5
    pad = (np.abs(bufh).sum(1) == 0).reshape(8, 5).sum(1)
    np.testing.assert_array_equal(pad, fix["padding"])
    # the page's repacking and its rank demand
    np.testing.assert_array_equal(host(run.mapping), [0, 1, 2, 3, 3, 2, 1, 0])
    L_ws = alloc((moe.moe_workspace_bytes(shape),), torch.uint8, DEV)
    plan = alloc((moe.moe_plan_layout(shape)["total"],), torch.int32, DEV)
    moe.moe_plan(shape, run.counts, plan)
    st, loads = moe.moe_stats(shape, run.counts, run.ids, plan, L_ws, mapping=run.mapping,
                              capacity_factor=1.25)
    assert loads[1] == fix["rank_demand_proposed"] == [10, 8, 7, 7]
    assert (st["capacity"], st["processed"], st["overflow"], st["padding"]) == (5, 27, 5, 13)


@pytest.mark.parametrize("E,R", [(8, 4), (8, 8), (16, 2), (128, 16), (256, 32), (256, 1), (64, 64)])
def test_repack_bit_exact(E, R):
    rng = np.random.default_rng(E * 7 + R)
    shape = moe.Shape(1, 64, E, 1, 64, R, 1, moe.MOE_BF16)
    mapping = alloc((E,), torch.int32, DEV)
    for trial in range(10):
        counts = (rng.zipf(1.3, E).clip(max=5000) if trial % 2 else rng.integers(0, 50, E))
        counts = counts.astype(np.int32)
        if trial == 0:
            counts[:] = 3          # all equal: ties everywhere
        moe.moe_repack(shape, torch.from_numpy(counts).to(DEV), mapping)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(mapping), oracle.repack(counts, R), err_msg=f"trial {trial}")


FULL = [("mixtral", 0.2, 1.0), ("decode256", 20, 1.25), ("a3b", 1, 1.25)]


@pytest.mark.parametrize("name,maxvio,cf", FULL, ids=[f"{n}@{m}cf{c}" for n, m, c in FULL])
def test_capacity_full_size_sampled(name, maxvio, cf):
    _say(f"[case] capacity full {name}@{maxvio} cf {cf}")
    w = wl.WORKLOADS[name]
    shape = moe.Shape(w["T"], w["H"], w["E"], w["k"], w["F"], w["R"], w["S"], moe.MOE_BF16)
    lg, bias = wl.logits_and_bias(name, maxvio)
    torch.cuda.empty_cache()
    x = synth.device_normal((w["T"], w["H"]), 1.0, w["seed"] * 7 + 1, torch.bfloat16, DEV)
    wts = make_weights(w["E"], w["F"], w["H"], moe.MOE_BF16, w["seed"])
    run = CapacityRun(shape, lg, bias, x, wts, cf)
    dest, _, ids, wgt, c = check_dispatch_and_plan(run, host(raw_bits(x)), lg, bias)
    st = oracle.stats(ids, c, shape.R, capacity_factor=cf)
    assert (dest < 0).sum() == st["overflow"]
    # FFN on sampled rows of the hottest and coldest non-empty expert and a
    # padding row; combine on sampled tokens
    xh = host(x)
    y = host(run.y)
    nz = np.nonzero(c)[0]
    for e in sorted({int(np.argmax(c)), int(nz[np.argmin(c[nz])])}):
        kept = min(int(c[e]), run.cap)
        pick = np.unique([0, kept // 2, kept - 1])
        rows = e * run.cap + pick
        src = np.array([np.nonzero(dest.ravel() == r)[0][0] // shape.k for r in rows])
        ref = oracle.ffn_rows(xh[src], host(wts[0][e]), host(wts[1][e]), host(wts[2][e]))
        assert_tol(y[rows], ref, moe.MOE_BF16, f"y expert {e}")
        if kept < run.cap:
            assert not y[e * run.cap + kept].any()     # a padding row
    # the kept rows of the sampled tokens, from the oracle's FFN of their x rows
    toks = np.unique(np.linspace(0, shape.T - 1, 6).astype(int))
    d = dest[toks]
    keep = d >= 0
    yr = np.zeros((d.size, shape.H))
    flat = d.ravel()
    src = np.repeat(toks, shape.k)
    for e in sorted({int(r) // run.cap for r in flat[flat >= 0]}):
        sel = np.nonzero((flat >= 0) & (flat // run.cap == e))[0]
        yr[sel] = oracle.ffn_rows(xh[src[sel]], host(wts[0][e]), host(wts[1][e]), host(wts[2][e]))
    out_ref = oracle.combine(yr, np.where(keep, np.arange(d.size).reshape(d.shape), -1),
                             wgt[toks].astype(np.float64))
    assert_tol(host(run.out)[toks], out_ref, moe.MOE_BF16, "out")
