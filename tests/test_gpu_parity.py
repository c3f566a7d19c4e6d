"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: bit-exact for ids, counts, offsets, eidx, rank loads, every plan table,
dest_row, row_src, the permuted buffer and the statistics; for floating
point, max|gpu - ref| <= 2e-2 * max|ref| in bf16 and <= 1e-5 * max|ref| in
fp32, with the tolerance applied per output tensor (route weights are fp32
in both modes). Full-size shapes check the integer path whole and the FFN
and combine on sampled experts / tokens the oracle can afford.
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
from expert_load_balance_amd.layer import MoeLayerBuffers, alloc  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {moe.MOE_BF16: 2e-2, moe.MOE_F32: 1e-5}
GOLD = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float32) \
        else t.detach().cpu().numpy()


def assert_tol(gpu, ref, dtype, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, what
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(gpu - ref).max() if ref.size else 0.0
    assert err <= TOL[dtype] * scale, f"{what}: max|d|={err:.3e} > {TOL[dtype]:g} * {scale:.3e}"


def make_weights(E, F, H, dtype, seed):
    act = torch.bfloat16 if dtype == moe.MOE_BF16 else torch.float32
    wg = synth.device_normal((E, F, H), synth.weight_std(H), seed * 10 + 1, act, DEV)
    wu = synth.device_normal((E, F, H), synth.weight_std(H), seed * 10 + 2, act, DEV)
    wd = synth.device_normal((E, H, F), synth.weight_std(F), seed * 10 + 3, act, DEV)
    return wg, wu, wd


def run_layer(shape, lg, bias, x, wts, shared_w=None, shared_F=None):
    L = MoeLayerBuffers(shape, DEV, shared_F=shared_F)
    lgd = alloc(lg.shape, torch.float32, DEV)       # non-null even for T = 0
    lgd.copy_(torch.from_numpy(lg))
    bd = None if bias is None else torch.from_numpy(bias).to(DEV)
    L.forward(lgd, bd, x, *wts, shared_w=shared_w)
    torch.cuda.synchronize()
    return L


def check_integer_path(L, lg, bias, x_host):
    """route ids/weights, count, plan, permute, bit-exact against the oracle."""
    s = L.shape
    ids, w, err = oracle.route(lg, bias, s.k)
    assert err == 0
    np.testing.assert_array_equal(host(L.ids), ids, err_msg="ids")
    assert_tol(host(L.w), w, moe.MOE_F32, "gate weights")
    c = oracle.count(ids, s.E, s.R)
    np.testing.assert_array_equal(host(L.counts), c["counts"], err_msg="counts")
    np.testing.assert_array_equal(host(L.offsets), c["offsets"], err_msg="offsets")
    np.testing.assert_array_equal(host(L.eidx), c["eidx"], err_msg="eidx")
    np.testing.assert_array_equal(host(L.rank_load), c["rank_load"], err_msg="rank_load")
    pl = oracle.plan(c["counts"], s.R)
    gt = moe.plan_tables(L.plan, s)
    for name in oracle.PLAN_TABLES:
        np.testing.assert_array_equal(host(gt[name]), pl[name], err_msg=name)
    if x_host is not None:
        buf, dest_row, row_src = oracle.permute(x_host, ids, c["eidx"], pl)
        np.testing.assert_array_equal(host(L.dest_row), dest_row, err_msg="dest_row")
        np.testing.assert_array_equal(host(L.row_src), row_src, err_msg="row_src")
        gbuf = L.buf.view(torch.int16 if L.buf.dtype == torch.bfloat16 else torch.int32)
        np.testing.assert_array_equal(host(gbuf), buf, err_msg="buf")
    assert int(L.err.item()) == 0
    return ids, w, c, pl


def raw_bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def expert_rows(pl, e):
    """buf rows of expert e, in virtual-row order (pieces in rank order)."""
    rows = []
    for p in range(pl["piece_num"][e]):
        r0, c = pl["piece_row"][e, p], pl["piece_cnt"][e, p]
        rows.extend(range(r0, r0 + c))
    return np.array(rows, np.int64)


# ------------------------------------------------------------- small, full ---

SMALL = [
    # name, T, H, E, k, F, R, S, dtype, bias strength
    ("tiny_f32_random", 16, 64, 8, 2, 128, 4, 2, moe.MOE_F32, 0.0),
    ("f32_multi_tile", 150, 96, 8, 2, 100, 4, 2, moe.MOE_F32, 0.4),
    ("bf16_multi_tile", 700, 256, 8, 2, 384, 4, 2, moe.MOE_BF16, 0.5),
    ("bf16_ragged_h", 200, 192, 16, 4, 128, 8, 2, moe.MOE_BF16, 0.8),
    ("bf16_fine_grained", 512, 128, 128, 8, 64, 16, 3, moe.MOE_BF16, 0.3),
    ("bf16_one_rank", 97, 128, 4, 2, 64, 1, 0, moe.MOE_BF16, 0.0),
    ("bf16_dense_one_expert", 65, 128, 1, 1, 128, 1, 1, moe.MOE_BF16, 0.0),
    ("bf16_all_experts", 33, 64, 8, 8, 64, 2, 4, moe.MOE_BF16, 0.2),
    ("bf16_fewer_rows_than_ranks", 1, 64, 8, 2, 64, 4, 2, moe.MOE_BF16, 0.0),
    ("bf16_odd_k_split", 300, 128, 8, 2, 192, 4, 2, moe.MOE_BF16, 0.3),
    ("bf16_two_experts_wide", 520, 512, 2, 1, 256, 2, 1, moe.MOE_BF16, 0.0),
    # experts around 32 rows: skinny (<= 32 rows) and 256-row tiles in one launch,
    # 16 K-stages through the skinny kernel's 4-stage ring
    ("bf16_skinny_boundary", 64, 1024, 4, 2, 256, 2, 1, moe.MOE_BF16, 0.0),
    # skinny tiles with 1 and 2 K-stages (gate/up K = 64, down K = 128)
    ("bf16_skinny_short_k", 40, 64, 8, 2, 128, 4, 2, moe.MOE_BF16, 0.5),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_layer_small_full_parity(case):
    name, T, H, E, k, F, R, S, dtype, s_bias = case
    _say(f"[case] {name}")
    shape = moe.Shape(T, H, E, k, F, R, S, dtype)
    lg = synth.router_logits(T, E, 17)
    bias = synth.zipf_bias(E, s_bias, 17) if s_bias else None
    act = torch.bfloat16 if dtype == moe.MOE_BF16 else torch.float32
    x = synth.device_normal((T, H), 1.0, 99, act, DEV)
    wts = make_weights(E, F, H, dtype, 3)
    L = run_layer(shape, lg, bias, x, wts)
    xh = host(x)
    ids, w, c, pl = check_integer_path(L, lg, bias, host(raw_bits(x)))
    # FFN per expert on its rows, oracle in double from the same rounded inputs
    wg, wu, wd = (host(t) for t in wts)
    buf_ref = xh[host(L.row_src)]
    y_ref = np.zeros((T * k, H))
    for e in range(E):
        rows = expert_rows(pl, e)
        if rows.size:
            y_ref[rows] = oracle.ffn_rows(buf_ref[rows], wg[e], wu[e], wd[e])
    assert_tol(host(L.y), y_ref, dtype, "y")
    out_ref = oracle.combine(y_ref, host(L.dest_row), w)
    assert_tol(host(L.out), out_ref, dtype, "out (end to end)")


def test_fixture_layer_fp32():
    """The 16-token hotspot fixture end to end in fp32 (E=8, k=2, R=4)."""
    with open(os.path.join(GOLD, "fixture16.json")) as f:
        fix = json.load(f)
    with open(os.path.join(GOLD, "fixture16_plan_derived.json")) as f:
        der = json.load(f)
    shape = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_F32)
    lg, bias = wl.fixture()
    x = synth.device_normal((16, 64), 1.0, 5, torch.float32, DEV)
    wts = make_weights(8, 128, 64, moe.MOE_F32, 1)
    L = run_layer(shape, lg, bias, x, wts)
    pairs = np.array([[int(p[0]), int(p[1])] for p in fix["pairs"].split(",")])
    np.testing.assert_array_equal(host(L.ids), pairs)
    np.testing.assert_array_equal(host(L.counts), fix["demand"])
    np.testing.assert_array_equal(host(L.rank_load), fix["rank_demand_home"])
    np.testing.assert_array_equal(host(L.dest_row), der["dest_row"])
    check_integer_path(L, lg, bias, host(raw_bits(x)))
    mapping = torch.tensor([0, 1, 2, 3, 3, 2, 1, 0], dtype=torch.int32, device=DEV)
    st, loads = moe.moe_stats(shape, L.counts, L.ids, L.plan, L.ws, dest_row=L.dest_row,
                              mapping=mapping, err=L.err, capacity_factor=1.25)
    assert st["balancedness_expert"] == 4 / 9 and st["maxvio_expert"] == 1.25
    assert st["balancedness_rank_home"] == 8 / 15
    assert st["balancedness_rank_mapped"] == 0.8
    assert loads[0] == fix["rank_demand_home"] and loads[1] == fix["rank_demand_proposed"]
    assert loads[2] == [8, 8, 8, 8]
    assert (st["capacity"], st["processed"], st["overflow"], st["padding"]) == (5, 27, 5, 13)
    assert (st["remote_home"], st["remote_mapped"]) == (22, 25)


def test_route_ties_and_signed_zero():
    T, E, k = 300, 64, 8
    rng = np.random.default_rng(4)
    lg = (rng.integers(-3, 4, size=(T, E)) * 0.5).astype(np.float32)
    lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    bias = (rng.integers(-1, 2, size=E) * 0.5).astype(np.float32)
    # every group width of the top-k kernel: 1, 2, 4, 8, 16, 32 lanes per
    # token, and 64 lanes with 1 to 4 experts per lane
    for e_, k_ in [(64, 8), (13, 5), (256, 64), (200, 8), (2, 2), (32, 8), (20, 3), (8, 2),
                   (5, 4), (4, 1), (1, 1), (128, 8), (150, 6)]:
        shape = moe.Shape(T, 64, e_, k_, 64, 1, 0, moe.MOE_BF16)
        lgx = np.ascontiguousarray(np.tile(lg, (1, 4))[:, :e_])
        bx = np.ascontiguousarray(np.tile(bias, 4)[:e_])
        ids = alloc((T, k_), torch.int32, DEV)
        w = alloc((T, k_), torch.float32, DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        moe.moe_route(shape, torch.from_numpy(lgx).to(DEV), torch.from_numpy(bx).to(DEV), ids, w, err)
        torch.cuda.synchronize()
        rid, rw, rerr = oracle.route(lgx, bx, k_)
        np.testing.assert_array_equal(host(ids), rid)
        assert_tol(host(w), rw, moe.MOE_F32, "w")
        assert int(err.item()) == 0 == rerr


def test_route_flags_nonfinite_logits():
    T, E, k = 40, 32, 4
    for bad in (float("nan"), float("inf")):
        lg = synth.router_logits(T, E, 2)
        lg[7, 9] = bad
        shape = moe.Shape(T, 64, E, k, 64, 4, 1, moe.MOE_BF16)
        ids = alloc((T, k), torch.int32, DEV)
        w = alloc((T, k), torch.float32, DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        moe.moe_route(shape, torch.from_numpy(lg).to(DEV), None, ids, w, err)
        torch.cuda.synchronize()
        assert int(err.item()) & moe.ERR_NONFINITE
        got = host(ids)
        assert ((got >= 0) & (got < E)).all()    # outputs stay in range


def test_count_flags_bad_ids():
    T, k, E, R = 64, 2, 8, 4
    shape = moe.Shape(T, 64, E, k, 64, R, 1, moe.MOE_BF16)
    base = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], 1).astype(np.int32)
    for mutate, bit in [((3, 1, 9), moe.ERR_RANGE), ((5, 1, -2), moe.ERR_RANGE),
                        ((6, 1, None), moe.ERR_REPEAT)]:
        ids = base.copy()
        t, j, v = mutate
        ids[t, j] = ids[t, 0] if v is None else v
        L = MoeLayerBuffers(shape, DEV)
        d_ids = torch.from_numpy(ids).to(DEV)
        moe.moe_count(shape, d_ids, L.counts, L.offsets, L.eidx, L.rank_load, L.err, L.ws)
        torch.cuda.synchronize()
        assert int(L.err.item()) & bit
        c = oracle.count(ids, E, R)
        assert c["err"] & bit
        np.testing.assert_array_equal(host(L.counts), c["counts"])
        np.testing.assert_array_equal(host(L.eidx), c["eidx"])


def test_count_repeats_across_chunks():
    # k = 7 does not divide 64: tokens straddle the 64-assignment rounds and
    # the per-wavefront chunks of the one-workgroup count (N = 9100: chunks of
    # 576). Token 9 (assignments 63..69) repeats across a round, token 82
    # (574..580) across two chunks; the clean ids must raise nothing.
    T, k, E, R = 1300, 7, 16, 4
    shape = moe.Shape(T, 64, E, k, 64, R, 1, moe.MOE_BF16)
    base = ((np.arange(T)[:, None] + np.arange(k)[None, :]) % E).astype(np.int32)
    for t, j in [(None, None), (9, 2), (82, 5), (1299, 6)]:
        ids = base.copy()
        if t is not None:
            ids[t, j] = ids[t, 0]
        L = MoeLayerBuffers(shape, DEV)
        d_ids = torch.from_numpy(ids).to(DEV)
        moe.moe_count(shape, d_ids, L.counts, L.offsets, L.eidx, L.rank_load, L.err, L.ws)
        torch.cuda.synchronize()
        c = oracle.count(ids, E, R)
        assert (int(L.err.item()) & moe.ERR_REPEAT) == (c["err"] & moe.ERR_REPEAT), (t, j)
        assert bool(c["err"] & moe.ERR_REPEAT) == (t is not None)
        np.testing.assert_array_equal(host(L.counts), c["counts"])
        np.testing.assert_array_equal(host(L.eidx), c["eidx"])


PLAN_VECTORS = [
    ("fixture", [9, 6, 5, 4, 3, 2, 2, 1], 4),
    ("balanced", [7] * 16, 8),
    ("one_hot", [0] * 37 + [5000] + [0] * 90, 16),
    ("n_below_r", [1, 0, 0, 0, 1, 0, 0, 0], 4),
    ("empty", [0] * 32, 8),
    ("single_rank", [3, 1, 4, 1, 5, 9, 2, 6], 1),
    ("max_ranks", list(range(128)), 64),
]


@pytest.mark.parametrize("case", PLAN_VECTORS, ids=[c[0] for c in PLAN_VECTORS])
def test_plan_tables_bit_exact(case):
    name, counts, R = case
    E = len(counts)
    shape = moe.Shape(max(1, sum(counts)), 64, E, 1, 64, R, 1, moe.MOE_BF16)
    d_counts = torch.tensor(counts, dtype=torch.int32, device=DEV)
    plan = alloc((moe.moe_plan_layout(shape)["total"],), torch.int32, DEV)
    plan.fill_(-7)
    moe.moe_plan(shape, d_counts, plan)
    torch.cuda.synchronize()
    ref = oracle.plan(np.array(counts), R)
    got = moe.plan_tables(plan, shape)
    for t in oracle.PLAN_TABLES:
        np.testing.assert_array_equal(host(got[t]), ref[t], err_msg=t)
    assert not (host(plan) == -7).any()     # the whole block is written


def test_plan_random_skew_bit_exact():
    rng = np.random.default_rng(12)
    for trial in range(40):
        E, R = [(8, 4), (8, 8), (128, 16), (256, 32), (64, 64), (256, 2)][trial % 6]
        counts = (rng.zipf(1.2 + 0.1 * (trial % 5), E).clip(max=20000)
                  if trial % 2 else rng.integers(0, 300, E)).astype(np.int32)
        shape = moe.Shape(int(counts.sum()) or 1, 64, E, 1, 64, R, 1, moe.MOE_BF16)
        plan = alloc((moe.moe_plan_layout(shape)["total"],), torch.int32, DEV)
        moe.moe_plan(shape, torch.from_numpy(counts).to(DEV), plan)
        torch.cuda.synchronize()
        ref = oracle.plan(counts, R)
        got = moe.plan_tables(plan, shape)
        for t in oracle.PLAN_TABLES:
            np.testing.assert_array_equal(host(got[t]), ref[t], err_msg=f"{t} trial {trial}")


def test_empty_batch():
    shape = moe.Shape(0, 128, 8, 2, 128, 4, 2, moe.MOE_BF16)
    x = alloc((0, 128), torch.bfloat16, DEV)
    wts = make_weights(8, 128, 128, moe.MOE_BF16, 2)
    L = run_layer(shape, np.zeros((0, 8), np.float32), None, x, wts)
    assert host(L.counts).sum() == 0
    gt = moe.plan_tables(L.plan, shape)
    assert host(gt["quota"]).sum() == 0 and host(gt["seg_num"]).sum() == 0


def test_deterministic_bitwise():
    shape = moe.Shape(700, 256, 16, 4, 256, 8, 2, moe.MOE_BF16)
    lg = synth.router_logits(700, 16, 8)
    bias = synth.zipf_bias(16, 0.7, 8)
    x = synth.device_normal((700, 256), 1.0, 7, torch.bfloat16, DEV)
    wts = make_weights(16, 256, 256, moe.MOE_BF16, 4)
    a = run_layer(shape, lg, bias, x, wts)
    b = run_layer(shape, lg, bias, x, wts)
    for name in ("ids", "w", "counts", "eidx", "plan", "dest_row", "row_src", "buf", "y", "out"):
        ta, tb = getattr(a, name), getattr(b, name)
        if ta.dtype == torch.bfloat16:
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), name


def test_host_rejects_before_launch():
    s = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_BF16)
    assert moe.moe_check_shape(s.replace(E=6)) == 1           # E % R != 0
    assert moe.moe_check_shape(s.replace(H=96)) == 2           # bf16 needs H % 64 == 0
    assert moe.moe_check_shape(s.replace(k=9)) == 1
    assert moe.moe_check_shape(s.replace(R=3)) == 1
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)        # far too small
    L = MoeLayerBuffers(s, DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_count(s, L.ids, L.counts, L.offsets, L.eidx, L.rank_load, L.err, ws)


# ------------------------------------------------------- full-size, sampled --

FULL = [("mixtral", 0.2), ("a3b", 0), ("a3b", 1), ("dsv3", 20), ("dsv3", 0),
        ("decode64", 1), ("decode1024", 20), ("decode256", 20)]

_WEIGHT_CACHE = {}


def _workload_tensors(name):
    w = wl.WORKLOADS[name]
    if _WEIGHT_CACHE.get("name") != name:
        _WEIGHT_CACHE.clear()
        torch.cuda.empty_cache()
        dtype = moe.MOE_BF16
        _WEIGHT_CACHE["name"] = name
        _WEIGHT_CACHE["x"] = synth.device_normal((w["T"], w["H"]), 1.0, w["seed"] * 7 + 1,
                                                 torch.bfloat16, DEV)
        _WEIGHT_CACHE["wts"] = make_weights(w["E"], w["F"], w["H"], dtype, w["seed"])
        if w.get("shared_F"):
            sw = make_weights(1, w["shared_F"], w["H"], dtype, w["seed"] + 50)
            _WEIGHT_CACHE["shared"] = sw
    return _WEIGHT_CACHE


def _sample_experts(counts, pl):
    nz = [e for e in range(len(counts)) if counts[e] > 0]
    hot = int(np.argmax(counts))
    cold = min(nz, key=lambda e: (counts[e], e))
    split = [e for e in nz if pl["piece_num"][e] > 1]
    picks = [hot, cold] + split[:1]
    return sorted(set(picks))


@pytest.mark.parametrize("name,maxvio", FULL, ids=[f"{n}@{m}" for n, m in FULL])
def test_full_size_sampled(name, maxvio):
    _say(f"[case] full {name}@{maxvio}")
    w = wl.WORKLOADS[name]
    shape = moe.Shape(w["T"], w["H"], w["E"], w["k"], w["F"], w["R"], w["S"], moe.MOE_BF16)
    lg, bias = wl.logits_and_bias(name, maxvio)
    cache = _workload_tensors(name)
    x, wts = cache["x"], cache["wts"]
    shared = cache.get("shared")
    L = run_layer(shape, lg, bias, x, wts, shared_w=shared, shared_F=w.get("shared_F"))
    ids, wgt, c, pl = check_integer_path(L, lg, bias, host(raw_bits(x)))
    # statistics, bit-exact against the oracle's
    st, loads = moe.moe_stats(shape, L.counts, L.ids, L.plan, L.ws, dest_row=L.dest_row,
                              err=L.err, capacity_factor=w.get("capacity_factor", 1.0))
    ref = oracle.stats(ids, c["counts"], shape.R, S=shape.S, dest_row=host(L.dest_row), pl=pl,
                       capacity_factor=w.get("capacity_factor", 1.0))
    for key_ in ("N", "max_count", "min_count", "active_experts", "maxvio_expert",
                 "balancedness_expert", "home_max", "maxvio_rank_home", "planned_max",
                 "planned_min", "maxvio_rank_planned", "capacity", "processed", "overflow",
                 "padding", "remote_home", "remote_planned", "replica_pieces",
                 "max_slots_needed", "ranks_over_slots", "nonlocal_rows"):
        assert st[key_] == ref[key_], key_
    assert st["planned_max"] - st["planned_min"] <= 1          # equal load
    if shape.S >= shape.E // shape.R:
        assert st["ranks_over_slots"] == 0
    # FFN on sampled experts (a few rows each) and combine on sampled tokens
    xh = host(x)
    wg, wu, wd = wts
    y = host(L.y)
    for e in _sample_experts(c["counts"], pl):
        rows = expert_rows(pl, e)
        pick = np.unique(np.concatenate([rows[:3], rows[-3:], rows[len(rows) // 2:][:2]]))
        src = host(L.row_src)[pick]
        ref_y = oracle.ffn_rows(xh[src], host(wg[e]), host(wu[e]), host(wd[e]))
        assert_tol(y[pick], ref_y, moe.MOE_BF16, f"y expert {e}")
    toks = np.unique(np.linspace(0, shape.T - 1, 6).astype(int))
    dr = host(L.dest_row)[toks]
    sh = None
    if shared is not None:
        sg, su, sd = (host(t[0]) for t in shared)
        sh = oracle.ffn_rows(xh[toks], sg, su, sd)
        assert_tol(host(L.shared_y)[toks], sh, moe.MOE_BF16, "shared expert")
    out_ref = oracle.combine(y[dr.ravel()].reshape(-1, shape.H), np.arange(dr.size).reshape(dr.shape),
                             host(L.w)[toks].astype(np.float64), sh)
    assert_tol(host(L.out)[toks], out_ref, moe.MOE_BF16, "out")
