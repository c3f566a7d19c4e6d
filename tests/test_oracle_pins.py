"""Pins for the CPU oracle against what the pages and the mathematics fix.

Sources: "MoE Load Balancing: Find Expert Hotspots" (the 16-token fixture and
its printed demand, balancedness, rank demand, capacity ledgers and remote
routes), "MoE load balancing: 90/10 routing in production" (the nine-times
share and the bias kept out of the gate), the MoonEP news article (maxvio is
zero when balanced; equal per-rank load however skewed; slots = experts per
rank keeps every touched expert local).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _pairs(g):
    return np.array([[int(p[0]), int(p[1])] for p in g["pairs"].split(",")], np.int32)


FIX = _gold("fixture16.json")
DER = _gold("fixture16_plan_derived.json")


def _mapping(groups, E):
    m = np.empty(E, np.int32)
    for r, grp in enumerate(groups):
        for e in grp:
            m[e] = r
    return m


# ---------------------------------------------------------------- router ----

def test_fixture_logits_route_to_page_pairs():
    ids, w, err = oracle.route(synth.fixture_logits(), None, 2)
    assert err == 0
    np.testing.assert_array_equal(ids, _pairs(FIX))


def test_fixture_weights_closed_form():
    # logits 2 and 1 -> weights e/(e+1) and 1/(e+1) = logistic(1), logistic(-1)
    _, w, _ = oracle.route(synth.fixture_logits(), None, 2)
    np.testing.assert_allclose(w[:, 0], 0.7310585786300049, rtol=0, atol=1e-15)
    np.testing.assert_allclose(w[:, 1], 0.2689414213699951, rtol=0, atol=1e-15)


def test_bias_moves_selection_not_weights():
    # A bias of +5 on every token's second expert reorders the pair; each
    # expert keeps the weight its raw logit earns (bias outside the gate).
    lg = synth.fixture_logits()
    pairs = _pairs(FIX)
    for t in range(16):
        bias = np.zeros(8, np.float32)
        bias[pairs[t, 1]] = 5.0
        ids, w, err = oracle.route(lg[t:t + 1], bias, 2)
        assert err == 0
        assert list(ids[0]) == [pairs[t, 1], pairs[t, 0]]
        assert w[0, 0] == pytest.approx(0.2689414213699951, abs=1e-15)
        assert w[0, 1] == pytest.approx(0.7310585786300049, abs=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_route_matches_full_stable_sort(seed):
    rng = np.random.default_rng(seed)
    T, E = 64, [8, 13, 64, 128, 256, 5][seed]
    k = min(E, [2, 3, 8, 8, 8, 5][seed])
    # coarse values so that ties (including -0 vs +0) are frequent
    lg = (rng.integers(-4, 5, size=(T, E)) * 0.5).astype(np.float32)
    lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    bias = (rng.integers(-2, 3, size=E) * 0.25).astype(np.float32) if seed % 2 else None
    ids, w, err = oracle.route(lg, bias, k)
    assert err == 0
    for t in range(T):
        s = lg[t] + (bias if bias is not None else np.float32(0))
        s = s.astype(np.float32)
        order = sorted(range(E), key=lambda e: (-float(s[e]), e))[:k]
        assert list(ids[t]) == order
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (w >= 0).all()


def test_route_single_expert_weight_is_one():
    lg = synth.router_logits(32, 16, 7)
    _, w, _ = oracle.route(lg, None, 1)
    np.testing.assert_array_equal(w, 1.0)


def test_route_weights_equal_renormalised_full_softmax():
    # softmax over the top-k == full softmax restricted to the top-k, renormalised
    lg = synth.router_logits(16, 32, 3)
    ids, w, _ = oracle.route(lg, None, 4)
    full = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)


def test_route_negative_zero_ties_lower_id():
    lg = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    ids, _, _ = oracle.route(lg, None, 3)
    assert list(ids[0]) == [0, 1, 3]


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_route_flags_nonfinite(bad):
    lg = synth.router_logits(4, 8, 1)
    lg[2, 5] = bad
    assert oracle.route(lg, None, 2)[2] & 1
    bias = np.zeros(8, np.float32)
    bias[3] = bad
    assert oracle.route(synth.router_logits(4, 8, 1), bias, 2)[2] & 1


# ---------------------------------------------------------------- counts ----

def test_fixture_demand_and_rank_demand():
    c = oracle.count(_pairs(FIX), 8, 4)
    assert c["err"] == 0
    np.testing.assert_array_equal(c["counts"], FIX["demand"])
    assert c["counts"].sum() == FIX["assignments"] == FIX["T"] * FIX["k"]
    np.testing.assert_array_equal(c["rank_load"], FIX["rank_demand_home"])
    np.testing.assert_array_equal(c["offsets"], np.concatenate([[0], np.cumsum(FIX["demand"])]))


@pytest.mark.parametrize("seed", range(4))
def test_eidx_is_a_stable_sort(seed):
    # offsets[e] + eidx == position of the assignment in a stable sort by expert
    rng = np.random.default_rng(100 + seed)
    T, E, k = 200, [8, 16, 128, 256][seed], [2, 4, 8, 8][seed]
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    c = oracle.count(ids, E, [4, 4, 16, 32][seed])
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")
    pos = np.empty_like(order)
    pos[order] = np.arange(flat.size)
    np.testing.assert_array_equal(c["offsets"][flat] + c["eidx"], pos)
    np.testing.assert_array_equal(c["counts"], np.bincount(flat, minlength=E))


def test_count_flags_range_and_repeats():
    ids = _pairs(FIX).copy()
    ids[3, 1] = 8
    assert oracle.count(ids, 8, 4)["err"] & 2
    ids = _pairs(FIX).copy()
    ids[5, 1] = ids[5, 0]
    assert oracle.count(ids, 8, 4)["err"] & 4
    ids = _pairs(FIX).copy()
    ids[0, 0] = -1
    assert oracle.count(ids, 8, 4)["err"] & 2


# ----------------------------------------------------------------- stats ----

def test_fixture_statistics():
    ids = _pairs(FIX)
    c = oracle.count(ids, 8, 4)
    prop = _mapping(FIX["proposed_mapping"], 8)
    st = oracle.stats(ids, c["counts"], 4, mapping=prop, capacity_factor=FIX["capacity_factor"])
    a, b = FIX["balancedness_expert"]
    assert st["balancedness_expert"] == a / b
    assert st["balancedness_expert"] == pytest.approx(0.444444, abs=5e-7)
    # maxvio read as max/mean - 1: 9/4 - 1
    assert st["maxvio_expert"] == 1.25
    a, b = FIX["balancedness_rank_home"]
    assert st["balancedness_rank_home"] == a / b
    assert st["balancedness_rank_home"] == pytest.approx(0.533333, abs=5e-7)
    np.testing.assert_array_equal(st["home_load"], FIX["rank_demand_home"])
    np.testing.assert_array_equal(st["mapped_load"], FIX["rank_demand_proposed"])
    a, b = FIX["balancedness_rank_proposed"]
    assert st["balancedness_rank_mapped"] == a / b == 0.8
    assert st["capacity"] == FIX["capacity"]
    assert st["processed"] == FIX["processed_sum"]
    assert st["overflow"] == FIX["overflow_sum"]
    assert st["padding"] == FIX["padding_sum"]
    assert st["remote_home"] == FIX["remote_home"]
    assert st["remote_mapped"] == FIX["remote_proposed"]
    assert st["remote_home"] / st["N"] == FIX["remote_share_home"]
    assert st["remote_mapped"] / st["N"] == FIX["remote_share_proposed"]


def test_fixture_capacity_ledgers():
    cap = oracle.capacity(32, 8, 1.25)
    assert cap == FIX["capacity"]
    proc, over, pad = oracle.ledgers(FIX["demand"], cap)
    np.testing.assert_array_equal(proc, FIX["processed"])
    np.testing.assert_array_equal(over, FIX["overflow"])
    np.testing.assert_array_equal(pad, FIX["padding"])
    # processed + padding fills every expert's capacity; processed + overflow is raw demand
    assert proc.sum() + pad.sum() == 8 * cap
    np.testing.assert_array_equal(proc + over, FIX["demand"])


def test_survivorship_traps_change_the_numbers():
    # the page's three traps each produce a different (wrong) value
    d = np.array(FIX["demand"])
    proc, _, _ = oracle.ledgers(d, 5)
    st_raw = oracle.stats(_pairs(FIX), d, 4)
    assert st_raw["max_count"] == 9 and proc.max() == 5            # demand after dropping overflow
    assert st_raw["balancedness_expert"] != (16 / 8) / 9            # tokens instead of assignments
    assert st_raw["balancedness_expert"] != 9 / 4                   # max/mean instead of mean/max


@pytest.mark.parametrize("seed", range(20))
def test_maxvio_zero_iff_equal(seed):
    rng = np.random.default_rng(seed)
    E, R = 8, 4
    if seed % 2:
        counts = np.full(E, int(rng.integers(1, 20)), np.int32)
    else:
        counts = rng.integers(0, 20, E).astype(np.int32)
        if (counts == counts[0]).all():
            counts[0] += 1
    ids = np.zeros((1, 1), np.int32)
    st = oracle.stats(ids, counts, R)
    assert (st["maxvio_expert"] == 0.0) == bool((counts == counts[0]).all())
    assert st["maxvio_expert"] >= 0


def test_nine_times_share():
    # 90% of the assignments on 26 of 256 experts: 0.9 / (26/256) ~ 8.86
    counts = np.array([1035] * 26 + [13] * 230, np.int32)
    assert counts[:26].sum() == 0.9 * counts.sum()
    assert oracle.hot_share(counts, 26) == pytest.approx(0.9 / (26 / 256), rel=1e-12)
    assert round(oracle.hot_share(counts, 26)) == 9


def test_empty_load_statistics():
    st = oracle.stats(np.zeros((0, 2), np.int32), np.zeros(8, np.int32), 4)
    assert st["maxvio_expert"] == 0.0 and st["balancedness_expert"] == 1.0


# ------------------------------------------------------------------ plan ----

def check_plan_invariants(counts, R, pl):
    counts = np.asarray(counts, np.int64)
    E = counts.size
    n = E // R
    N = int(counts.sum())
    q = pl["quota"]
    assert q.sum() == N
    assert set(q.tolist()) <= {N // R, -(-N // R)}
    assert pl["win_off"][0] == 0
    np.testing.assert_array_equal(np.diff(pl["win_off"]), q)
    per_expert = np.zeros(E, np.int64)
    receivers = 0
    for r in range(R):
        ns = pl["seg_num"][r]
        ex = pl["seg_expert"][r, :ns]
        rows = pl["seg_row"][r, :ns]
        cnt = pl["seg_cnt"][r, :ns]
        assert (pl["seg_expert"][r, ns:] == -1).all()
        assert (cnt > 0).all()
        assert cnt.sum() == q[r]                                   # equal load
        assert (np.diff(ex) > 0).all()                             # expert id ascending
        if ns:
            assert rows[0] == pl["win_off"][r]
            np.testing.assert_array_equal(rows[1:], rows[:-1] + cnt[:-1])
        for e, c in zip(ex, cnt):
            per_expert[e] += c
        foreign = [e for e in ex if e // n != r]
        assert len(foreign) == pl["slots_needed"][r] <= n          # <= n replicas per rank
        assert sorted(foreign) == [e for e in pl["slot_expert"][r] if e >= 0]
        if foreign:
            receivers += 1
            donors = {e // n for e in foreign}
            assert donors == {pl["donor"][r]}                      # a single donor rank
    np.testing.assert_array_equal(per_expert, counts)              # exactly once
    assert receivers <= max(R - 1, 0)
    home = np.array([counts[r * n:(r + 1) * n].sum() for r in range(R)])
    balanced = bool((home == q).all())
    assert balanced == (pl["slots_needed"].sum() == 0)             # replicas only when needed
    # pieces: rank ascending, consistent with segments
    for e in range(E):
        np_ = pl["piece_num"][e]
        ranks = pl["piece_rank"][e, :np_]
        assert (np.diff(ranks) > 0).all()
        assert pl["piece_cnt"][e, :np_].sum() == counts[e]
        for r, row, c in zip(ranks, pl["piece_row"][e, :np_], pl["piece_cnt"][e, :np_]):
            i = list(pl["seg_expert"][r, :pl["seg_num"][r]]).index(e)
            assert pl["seg_row"][r, i] == row and pl["seg_cnt"][r, i] == c


def test_fixture_plan_derived_golden():
    pl = oracle.plan(FIX["demand"], 4)
    np.testing.assert_array_equal(pl["quota"], DER["quota"])
    np.testing.assert_array_equal(pl["win_off"], DER["win_off"])
    for r in range(4):
        segs = [[int(pl["seg_expert"][r, i]), int(pl["seg_row"][r, i]), int(pl["seg_cnt"][r, i])]
                for i in range(pl["seg_num"][r])]
        assert segs == DER["segments"][str(r)]
    np.testing.assert_array_equal(pl["slot_expert"], DER["slot_expert"])
    np.testing.assert_array_equal(pl["donor"], DER["donor"])
    check_plan_invariants(FIX["demand"], 4, pl)


def test_plan_exhaustive_small():
    seen = 0
    for E, R in [(1, 1), (2, 1), (2, 2), (3, 3), (4, 2), (4, 4), (6, 2), (6, 3), (6, 6)]:
        hi = 4 if E <= 4 else 3
        for counts in itertools.product(range(hi + 1), repeat=E):
            if sum(counts) > 12:
                continue
            check_plan_invariants(counts, R, oracle.plan(counts, R))
            seen += 1
    assert seen > 3000


@pytest.mark.parametrize("E,R", [(8, 4), (8, 8), (128, 16), (256, 32), (128, 1), (64, 64)])
def test_plan_random_skew(E, R):
    rng = np.random.default_rng(E * 1000 + R)
    for trial in range(300 if E <= 8 else 60):
        kind = trial % 3
        if kind == 0:
            counts = rng.integers(0, 50, E)
        elif kind == 1:
            counts = rng.zipf(1.5, E).clip(max=5000)
        else:
            counts = np.zeros(E, np.int64)
            counts[rng.integers(0, E)] = rng.integers(1, 5000)
        check_plan_invariants(counts, R, oracle.plan(counts, R))


def test_plan_slots_equal_experts_per_rank_keeps_everything_local():
    # with S = n slots every replica fits a slot, so no row is non-local
    rng = np.random.default_rng(5)
    for _ in range(50):
        counts = rng.zipf(1.3, 128).clip(max=4000).astype(np.int32)
        pl = oracle.plan(counts, 16)
        ids = np.zeros((1, 1), np.int32)
        st = oracle.stats(ids, counts, 16, S=8, pl=pl)
        assert st["ranks_over_slots"] == 0 and st["nonlocal_rows"] == 0
        assert st["planned_max"] - st["planned_min"] <= 1
        assert st["maxvio_rank_planned"] <= (-(-counts.sum() // 16) * 16 - counts.sum()) / counts.sum()


def test_plan_balanced_input_has_no_replicas():
    pl = oracle.plan(np.full(128, 256, np.int32), 16)
    assert pl["slots_needed"].sum() == 0 and (pl["donor"] == -1).all()


# --------------------------------------------------------------- permute ----

def test_fixture_permutation_derived_golden():
    ids = _pairs(FIX)
    c = oracle.count(ids, 8, 4)
    pl = oracle.plan(c["counts"], 4)
    x = synth.host_normal((16, 64), 1.0, 11)
    buf, dest_row, row_src = oracle.permute(x, ids, c["eidx"], pl)
    np.testing.assert_array_equal(dest_row, DER["dest_row"])
    np.testing.assert_array_equal(buf, x[row_src])


@pytest.mark.parametrize("seed", range(3))
def test_permutation_is_a_bijection_into_local_windows(seed):
    rng = np.random.default_rng(seed)
    T, E, k, R = 300, 64, 6, 8
    n = E // R
    lg = synth.router_logits(T, E, seed)
    bias = synth.zipf_bias(E, 0.6, seed)
    ids, _, _ = oracle.route(lg, bias, k)
    c = oracle.count(ids, E, R)
    pl = oracle.plan(c["counts"], R)
    x = rng.integers(0, 1 << 15, size=(T, 8)).astype(np.uint16)
    buf, dest_row, row_src = oracle.permute(x, ids, c["eidx"], pl)
    flat = dest_row.ravel()
    np.testing.assert_array_equal(np.sort(flat), np.arange(T * k))
    np.testing.assert_array_equal(row_src[flat], np.repeat(np.arange(T), k))
    np.testing.assert_array_equal(buf, x[row_src])
    for d, e in zip(flat, ids.ravel()):
        r = int(np.searchsorted(pl["win_off"], d, side="right") - 1)
        assert e // n == r or e in pl["slot_expert"][r]
    # k = 1, w = 1: combine returns x exactly
    ids1 = ids[:, :1].copy()
    c1 = oracle.count(ids1, E, R)
    pl1 = oracle.plan(c1["counts"], R)
    xf = synth.host_normal((T, 16), 1.0, seed)
    buf1, dr1, _ = oracle.permute(xf, ids1, c1["eidx"], pl1)
    out = oracle.combine(buf1.astype(np.float64), dr1, np.ones((T, 1)))
    np.testing.assert_array_equal(out, xf.astype(np.float64))


# ------------------------------------------------------------------- FFN ----

def test_ffn_scalar_closed_form():
    # H = F = 1, all weights 1, x = 1: y = silu(1) * 1 = logistic(1)
    one = np.ones((1, 1), np.float32)
    y = oracle.ffn_rows(one, one, one, one)
    assert y[0, 0] == pytest.approx(0.7310585786300049, abs=1e-15)
    y = oracle.ffn_rows(-one, one, one, one)          # silu(-1) * (-1) = logistic(-1)
    assert y[0, 0] == pytest.approx(0.2689414213699951, abs=1e-15)


def test_ffn_dense_reduces_to_matmul():
    # one expert, k = 1: the layer is a dense SwiGLU FFN (library matmul check)
    H, F, n = 24, 40, 7
    x = synth.host_normal((n, H), 1.0, 1)
    wg = synth.host_normal((F, H), H ** -0.5, 2)
    wu = synth.host_normal((F, H), H ** -0.5, 3)
    wd = synth.host_normal((H, F), F ** -0.5, 4)
    y = oracle.ffn_rows(x, wg, wu, wd)
    X, G, U, D = (a.astype(np.float64) for a in (x, wg, wu, wd))
    g = X @ G.T
    ref = ((g / (1 + np.exp(-g))) * (X @ U.T)) @ D.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    # linear in W_down, zero gate gives zero output
    np.testing.assert_allclose(oracle.ffn_rows(x, wg, wu, 2 * wd), 2 * y, rtol=1e-12, atol=1e-13)
    assert not oracle.ffn_rows(x, np.zeros_like(wg), wu, wd).any()


# --------------------------------------------------------------- combine ----

def test_combine_one_hot_and_order():
    rng = np.random.default_rng(3)
    T, k, H = 10, 3, 5
    y = rng.standard_normal((T * k, H))
    dest = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    w = np.zeros((T, k))
    w[np.arange(T), rng.integers(0, k, T)] = 1.0
    out = oracle.combine(y, dest, w)
    np.testing.assert_array_equal(out, y[dest[np.arange(T), w.argmax(1)]])
    w = rng.random((T, k))
    perm = rng.permutation(k)
    a = oracle.combine(y, dest, w)
    b = oracle.combine(y, dest[:, perm], w[:, perm])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    sh = rng.standard_normal((T, H))
    np.testing.assert_allclose(oracle.combine(y, dest, w, sh), a + sh, rtol=1e-13, atol=1e-15)


# ------------------------------------------------- fixed capacity, repack ----
# "MoE Load Balancing: Find Expert Hotspots", "Make expert capacity, overflow,
# and padding explicit" (cap 5 for the fixture; processed 27, overflow 5,
# padding 13) and "Separate expert demand from rank placement" (the mapping
# {0,7},{1,6},{2,5},{3,4} takes rank demand to [10,8,7,7]).

def test_fixture_capacity_dispatch_ledgers():
    ids = _pairs(FIX)
    T, k = ids.shape
    c = oracle.count(ids, 8, 4)
    cap = FIX["capacity"]
    x = np.arange(T * 3, dtype=np.float32).reshape(T, 3) + 1.0   # no zero rows in x
    buf, dest = oracle.capacity_dispatch(x, ids, c["eidx"], 8, cap)
    kept = np.bincount(ids.ravel()[dest.ravel() >= 0], minlength=8)
    np.testing.assert_array_equal(kept, FIX["processed"])
    assert (dest < 0).sum() == sum(FIX["overflow"])
    pad = (np.abs(buf).sum(1) == 0).reshape(8, cap).sum(1)
    np.testing.assert_array_equal(pad, FIX["padding"])
    assert kept.sum() == 27 and (dest < 0).sum() == 5 and pad.sum() == 13


@pytest.mark.parametrize("seed", range(3))
def test_capacity_dispatch_brute_force(seed):
    # an assignment is kept iff fewer than cap earlier assignments (flat order)
    # went to its expert; it then sits at row e*cap + (that number)
    rng = np.random.default_rng(700 + seed)
    T, E, k = 60, [8, 16, 32][seed], [2, 4, 8][seed]
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    cap = int(rng.integers(1, 2 * T * k // E))
    x = rng.standard_normal((T, 5)).astype(np.float32)
    buf, dest = oracle.capacity_dispatch(x, ids, oracle.count(ids, E, 1)["eidx"], E, cap)
    seen = {}
    want_buf = np.zeros((E * cap, 5), np.float32)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            v = seen.get(e, 0)
            seen[e] = v + 1
            if v < cap:
                assert dest[t, j] == e * cap + v
                want_buf[e * cap + v] = x[t]
            else:
                assert dest[t, j] == -1
    np.testing.assert_array_equal(buf, want_buf)


def test_combine_skips_dropped_assignments():
    rng = np.random.default_rng(5)
    T, k, H = 8, 2, 4
    y = rng.standard_normal((T * k, H))
    dest = np.arange(T * k, dtype=np.int32).reshape(T, k)
    w = rng.random((T, k))
    full = oracle.combine(y, dest, w)
    dropped = dest.copy()
    dropped[::2, 1] = -1
    w0 = w.copy()
    w0[::2, 1] = 0.0
    np.testing.assert_allclose(oracle.combine(y, dropped, w), oracle.combine(y, dest, w0),
                               rtol=1e-15, atol=0)
    assert not np.allclose(oracle.combine(y, dropped, w), full)


def test_fixture_repack_reproduces_page_mapping():
    m = oracle.repack(np.array(FIX["demand"], np.int32), 4)
    np.testing.assert_array_equal(m, _mapping([[0, 7], [1, 6], [2, 5], [3, 4]], 8))
    np.testing.assert_array_equal(np.bincount(m, weights=FIX["demand"], minlength=4), [10, 8, 7, 7])
    st = oracle.stats(_pairs(FIX), np.array(FIX["demand"], np.int32), 4, mapping=m)
    np.testing.assert_array_equal(st["mapped_load"], [10, 8, 7, 7])


@pytest.mark.parametrize("counts, R, groups", [
    ([5, 5, 1, 1], 2, [[0, 2], [1, 3]]),
    ([7, 1, 1, 1, 1, 1], 3, [[0, 5], [1, 3], [2, 4]]),
    ([3, 3, 3, 3], 4, [[0], [1], [2], [3]]),
    ([0, 0, 0, 0, 0, 0, 0, 0], 2, [[0, 1, 2, 3], [4, 5, 6, 7]]),   # equal load: lower rank first
])
def test_repack_hand_examples(counts, R, groups):
    np.testing.assert_array_equal(oracle.repack(np.array(counts, np.int32), R),
                                  _mapping(groups, len(counts)))


@pytest.mark.parametrize("seed", range(4))
def test_repack_invariants_and_brute_force_bounds(seed):
    rng = np.random.default_rng(900 + seed)
    E, R = 8, [2, 4, 2, 4][seed]
    n = E // R
    for _ in range(50):
        c = rng.integers(0, 40, E).astype(np.int32)
        m = oracle.repack(c, R)
        np.testing.assert_array_equal(np.bincount(m, minlength=R), np.full(R, n))
        got = np.bincount(m, weights=c, minlength=R).max()
        # brute force over every balanced placement: the greedy rule is a
        # heuristic, so only the bounds every balanced placement obeys hold
        best = min(max(sum(c[list(g)]) for g in parts) for parts in _balanced_partitions(E, R))
        assert best <= got <= np.sort(c)[::-1][:n].sum()


def _balanced_partitions(E, R):
    n = E // R

    def rec(left, groups):
        if not left:
            yield groups
            return
        first = left[0]
        for rest in itertools.combinations(left[1:], n - 1):
            g = (first,) + rest
            yield from rec([e for e in left if e not in g], groups + [g])

    yield from rec(list(range(E)), [])


# ------------------------------------------------------ router, bias update ----
# "DeepEP-on-EFA Guidance, section 1", phase (a): the router scores every
# expert for every token (read: a linear layer); "MoE load balancing: 90/10
# routing in production": a per-expert bias kept out of the gate. The bias
# update rule is not on the pages (a labelled assumption: the sign rule).

def test_router_logits_special_cases():
    rng = np.random.default_rng(11)
    T, H, E = 7, 16, 16
    x = rng.standard_normal((T, H)).astype(np.float32)
    # identity router: the logits are the first E features, exactly
    np.testing.assert_array_equal(oracle.router_logits(x, np.eye(E, H, dtype=np.float32)), x[:, :E])
    assert not oracle.router_logits(x, np.zeros((E, H), np.float32)).any()
    # small integers: exact in double, so equal to the integer matrix product
    xi = rng.integers(-5, 6, (T, H)).astype(np.float32)
    wi = rng.integers(-5, 6, (E, H)).astype(np.float32)
    want = xi.astype(np.int64) @ wi.astype(np.int64).T
    np.testing.assert_array_equal(oracle.router_logits(xi, wi), want)
    # one-hot rows pick single weights: logit[t][e] = W[e][h_t]
    hs = rng.integers(0, H, T)
    oh = np.zeros((T, H), np.float32)
    oh[np.arange(T), hs] = 1.0
    w = rng.standard_normal((E, H)).astype(np.float32)
    np.testing.assert_array_equal(oracle.router_logits(oh, w), w[:, hs].T)


def test_bias_update_sign_rule():
    counts = np.array([9, 6, 5, 4, 3, 2, 2, 1], np.int32)      # fixture demand, mean 4
    b0 = np.linspace(-1, 1, 8).astype(np.float32)
    g = np.float32(0.125)
    b1 = oracle.bias_update(counts, b0, g)
    np.testing.assert_array_equal(b1[:3], b0[:3] - g)          # above the mean
    assert b1[3] == b0[3]                                       # at the mean
    np.testing.assert_array_equal(b1[4:], b0[4:] + g)          # below the mean
    # balanced demand keeps every bias
    np.testing.assert_array_equal(oracle.bias_update(np.full(8, 4, np.int32), b0, g), b0)


def test_bias_update_closed_loop_reduces_maxvio():
    # route -> count -> update on fixed logits: the assumed rule drives the
    # expert-level maxvio towards zero (the page's aim), starting from a skew
    T, E, k = 512, 16, 2
    lg = synth.router_logits(T, E, 21)
    bias = synth.zipf_bias(E, 0.8, 21).astype(np.float32)
    first = None
    for _ in range(200):
        ids, _, _ = oracle.route(lg, bias, k)
        c = oracle.count(ids, E, 4)["counts"]
        mv = (c.max() * E - T * k) / (T * k)
        first = mv if first is None else first
        bias = oracle.bias_update(c, bias, 0.01)
    assert first > 0.8 and mv < 0.25


# ---- replica weight slots (MoonEP news article, paragraphs 3-4) ----------

def _fixture_plan():
    c = oracle.count(_pairs(FIX), 8, 4)["counts"]
    assert c.tolist() == [9, 6, 5, 4, 3, 2, 2, 1]
    return oracle.plan(c, 4)


def test_fixture_slot_sources():
    """The derived fixture plan: ranks 0, 2, 3 each hold one replica (expert
    2, 0, 0), so with S >= 1 those segments read slot 0 and every other
    segment the home weights; with S = 0 every segment reads home weights."""
    pl = _fixture_plan()
    assert pl["slot_expert"].tolist() == DER["slot_expert"]
    want = [[-1, -1, 0, -2], [-1, -1, -2, -2], [0, -1, -1, -2], [0, -1, -1, -2]]
    assert oracle.slot_sources(pl, 2).tolist() == want
    assert oracle.slot_sources(pl, 1).tolist() == want
    no = [[-1 if v != -2 else -2 for v in row] for row in want]
    assert oracle.slot_sources(pl, 0).tolist() == no


@pytest.mark.parametrize("seed", range(6))
def test_slot_sources_invariants(seed):
    """Every local slot is read by exactly the segment of its expert; home
    segments never read a slot; with S >= n every replica segment is local
    (the slots = experts-per-rank guarantee); the rows read from home weights
    by replica segments are exactly the stats' non-local rows."""
    rng = np.random.default_rng(seed)
    R = int(rng.choice([2, 4, 8]))
    n = int(rng.integers(1, 5))
    E, k, T = R * n, min(R * n, int(rng.integers(1, 4))), int(rng.integers(20, 200))
    lg = synth.router_logits(T, E, seed + 30)
    bias = synth.zipf_bias(E, float(rng.uniform(0, 2)), seed + 30).astype(np.float32)
    ids, _, _ = oracle.route(lg, bias, k)
    c = oracle.count(ids, E, R)
    pl = oracle.plan(c["counts"], R)
    for S in range(0, n + 2):
        src = oracle.slot_sources(pl, S)
        nonlocal_rows = 0
        for r in range(R):
            used = []
            for i in range(2 * n):
                if i >= pl["seg_num"][r]:
                    assert src[r, i] == -2
                    continue
                e = pl["seg_expert"][r, i]
                if e // n == r:
                    assert src[r, i] == -1
                elif src[r, i] >= 0:
                    assert pl["slot_expert"][r, src[r, i]] == e and src[r, i] < S
                    used.append(int(src[r, i]))
                else:
                    assert S < n
                    nonlocal_rows += int(pl["seg_cnt"][r, i])
            assert sorted(used) == list(range(min(S, int(pl["slots_needed"][r]))))
        st = oracle.stats(ids, c["counts"], R, S=S, pl=pl)
        assert st["nonlocal_rows"] == nonlocal_rows


def test_fixture_prefetch_pool():
    """The pool holds bit-exact copies of the slot experts' three projections
    (rank 0 slot 0: expert 2; ranks 2 and 3 slot 0: expert 0); rank 1 has no
    replica and its slot stays empty."""
    pl = _fixture_plan()
    rng = np.random.default_rng(5)
    E, F, H = 8, 6, 4
    wg = rng.standard_normal((E, F, H)).astype(np.float32)
    wu = rng.standard_normal((E, F, H)).astype(np.float32)
    wd = rng.standard_normal((E, H, F)).astype(np.float32)
    pool = oracle.prefetch(pl, 2, wg, wu, wd)
    assert pool.shape == (4, 2, 3, F * H)
    for r, e in ((0, 2), (2, 0), (3, 0)):
        assert np.array_equal(pool[r, 0, 0], wg[e].ravel())
        assert np.array_equal(pool[r, 0, 1], wu[e].ravel())
        assert np.array_equal(pool[r, 0, 2], wd[e].ravel())
    assert not pool[1].any() and not pool[:, 1].any()


def test_slot_ffn_reads_the_slots():
    """With the prefetched pool the slot-reading FFN equals the home-weight
    FFN exactly; doubling W_down in one slot doubles exactly the rows of the
    segment that reads it (the FFN is linear in W_down) and nothing else."""
    pl = _fixture_plan()
    rng = np.random.default_rng(6)
    E, F, H = 8, 6, 4
    wg = rng.standard_normal((E, F, H))
    wu = rng.standard_normal((E, F, H))
    wd = rng.standard_normal((E, H, F))
    buf = rng.standard_normal((32, H))
    pool = oracle.prefetch(pl, 2, wg, wu, wd)
    home = oracle.slot_ffn(buf, pl, 0, wg, wu, wd, pool)
    y = oracle.slot_ffn(buf, pl, 2, wg, wu, wd, pool)
    assert np.array_equal(y, home)
    for r in range(4):
        for i in range(int(pl["seg_num"][r])):
            e, row, cnt = (int(pl[t][r, i]) for t in ("seg_expert", "seg_row", "seg_cnt"))
            assert np.array_equal(home[row:row + cnt], oracle.ffn_rows(buf[row:row + cnt], wg[e],
                                                                       wu[e], wd[e]))
    pool2 = pool.copy()
    pool2[2, 0, 2] *= 2.0                        # rank 2's slot: expert 0, rows 16..18
    y2 = oracle.slot_ffn(buf, pl, 2, wg, wu, wd, pool2)
    assert np.array_equal(y2[16:19], 2.0 * y[16:19])
    assert np.array_equal(np.delete(y2, [16, 17, 18], 0), np.delete(y, [16, 17, 18], 0))


# ---- backward: central differences of the forward functions ---------------

def _grid(rng, shape, bits=6):
    """Values m * 2^-bits in [-1, 1]: exact in float32, and so are their
    +- 2^-12 neighbours used by the central differences below."""
    return (rng.integers(-(1 << bits), (1 << bits) + 1, size=shape) / (1 << bits)).astype(np.float64)


def test_ffn_backward_matches_central_differences():
    """Every entry of dx, dW_gate, dW_up and dW_down against
    (L(+eps) - L(-eps)) / 2 eps of L = <dy, ffn_rows(x, W)>, eps = 2^-12
    (an independent path: the forward oracle, evaluated in double)."""
    rng = np.random.default_rng(11)
    n, H, F = 3, 4, 5
    x = _grid(rng, (n, H))
    wg, wu = _grid(rng, (F, H)), _grid(rng, (F, H))
    wd = _grid(rng, (H, F))
    dy = rng.standard_normal((n, H))
    dx, dwg, dwu, dwd = oracle.ffn_backward_rows(x, dy, wg, wu, wd)
    eps = 2.0 ** -12

    def loss(x_, wg_, wu_, wd_):
        return float((dy * oracle.ffn_rows(x_, wg_, wu_, wd_)).sum())

    def fd(arr, which):
        out = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            vals = []
            for sgn in (1, -1):
                a = arr.copy()
                a[idx] += sgn * eps
                args = [x, wg, wu, wd]
                args[which] = a
                vals.append(loss(*args))
            out[idx] = (vals[0] - vals[1]) / (2 * eps)
        return out

    for got, arr, which in ((dx, x, 0), (dwg, wg, 1), (dwu, wu, 2), (dwd, wd, 3)):
        ref = fd(arr, which)
        assert np.abs(got - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max()), which


def test_combine_backward_is_the_adjoint():
    """L = <dout, combine(y, dest, w)> is linear in y and in w, so dy and dw
    are fixed exactly by <dy, y'> = L(y') and <dw, w'> = L(w') for any y',
    w'; dropped assignments (dest -1) get dw = 0 and their rows stay 0."""
    rng = np.random.default_rng(12)
    T, k, H, nrows = 6, 3, 5, 20
    dest = rng.permutation(nrows)[:T * k].reshape(T, k).astype(np.int32)
    dest[2, 1] = -1
    y = rng.standard_normal((nrows, H))
    w = rng.random((T, k))
    dout = rng.standard_normal((T, H))
    dy, dw = oracle.combine_backward(dout, y, dest, w)
    for _ in range(3):
        y2 = rng.standard_normal((nrows, H))
        assert np.isclose((dy * y2).sum(), (dout * oracle.combine(y2, dest, w)).sum(), rtol=1e-12)
        w2 = rng.random((T, k))
        assert np.isclose((dw * w2).sum(), (dout * oracle.combine(y, dest, w2)).sum(), rtol=1e-12)
    assert dw[2, 1] == 0.0
    unused = np.setdiff1d(np.arange(nrows), dest[dest >= 0])
    assert not dy[unused].any()


def test_permute_backward_is_the_adjoint():
    """<permute(x), dbuf> = <x, permute_backward(dbuf)> on the fixture plan."""
    pl = _fixture_plan()
    ids = _pairs(FIX)
    c = oracle.count(ids, 8, 4)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((16, 7))
    buf, dest, _ = oracle.permute(x, ids, c["eidx"], pl)
    dbuf = rng.standard_normal(buf.shape)
    dx = oracle.permute_backward(dbuf, dest)
    assert np.isclose((buf * dbuf).sum(), (x * dx).sum(), rtol=1e-12)


def test_route_backward_matches_central_differences():
    """dlogits against central differences of L = <dw, w(logits)> through the
    forward top-k + softmax; logits on a 2^-8 grid with distinct values, so a
    2^-14 step never changes the selection. Unselected experts get 0."""
    rng = np.random.default_rng(14)
    T, E, k = 4, 9, 3
    lg = np.stack([rng.permutation(np.arange(E) - E // 2) for _ in range(T)]) / 8.0
    lg = (lg + rng.integers(-3, 4, size=(T, E)) / 256.0).astype(np.float32)
    ids, w, _ = oracle.route(lg, None, k)
    dw = rng.standard_normal((T, k))
    dl = oracle.route_backward(ids, w, dw, E)
    eps = 2.0 ** -14
    for t in range(T):
        for e in range(E):
            vals = []
            for sgn in (1, -1):
                l2 = lg.copy()
                l2[t, e] += np.float32(sgn * eps)
                i2, w2, _ = oracle.route(l2, None, k)
                assert np.array_equal(i2, ids)
                vals.append(float((dw * w2).sum()))
            ref = (vals[0] - vals[1]) / (2 * eps)
            assert abs(dl[t, e] - ref) <= 1e-6, (t, e)
            if e not in ids[t]:
                assert dl[t, e] == 0.0


def test_expert_backward_reduces_replicas_into_home():
    """On the fixture plan expert 0 has a home piece and two replica pieces:
    its weight gradient is the sum of the per-piece gradients (the replicas'
    contributions reduced into the home expert), equal to one call over all
    of its rows."""
    pl = _fixture_plan()
    rng = np.random.default_rng(15)
    E, H, F, N = 8, 4, 6, 32
    buf = _grid(rng, (N, H))
    dy = rng.standard_normal((N, H))
    wg, wu = _grid(rng, (E, F, H)), _grid(rng, (E, F, H))
    wd = _grid(rng, (E, H, F))
    dbuf, dwg, dwu, dwd = oracle.expert_ffn_backward(buf, dy, pl, wg, wu, wd)
    assert int(pl["piece_num"][0]) == 3
    parts = [oracle.ffn_backward_rows(buf[r0:r0 + c], dy[r0:r0 + c], wg[0], wu[0], wd[0])
             for r0, c in zip(pl["piece_row"][0][:3], pl["piece_cnt"][0][:3])]
    for q, got in ((1, dwg[0]), (2, dwu[0]), (3, dwd[0])):
        assert np.allclose(got, sum(p[q] for p in parts), rtol=1e-12, atol=1e-12)


def test_replica_backward_reduction_equals_the_expert_sum():
    """Home part plus replica slots (rank order) equals the gradient over all
    of an expert's rows, for every expert of a skewed random plan; every slot
    of the plan holds exactly its replica piece's gradient."""
    rng = np.random.default_rng(16)
    T, E, k, R, H, F = 60, 8, 2, 4, 4, 6
    lg = synth.router_logits(T, E, 16)
    bias = synth.zipf_bias(E, 1.5, 16).astype(np.float32)
    ids, _, _ = oracle.route(lg, bias, k)
    c = oracle.count(ids, E, R)
    pl = oracle.plan(c["counts"], R)
    assert (pl["slot_expert"] >= 0).sum() >= 2               # replicas exist
    N = T * k
    buf = _grid(rng, (N, H))
    dy = rng.standard_normal((N, H))
    wg, wu = _grid(rng, (E, F, H)), _grid(rng, (E, F, H))
    wd = _grid(rng, (E, H, F))
    dwg, dwu, dwd, slots = oracle.replica_backward(buf, dy, pl, wg, wu, wd)
    _, eg, eu, ed = oracle.expert_ffn_backward(buf, dy, pl, wg, wu, wd)
    for a_, b_ in ((dwg, eg), (dwu, eu), (dwd, ed)):
        assert np.allclose(a_, b_, rtol=1e-12, atol=1e-12)
    assert set(slots) == {(r, j) for r in range(R) for j in range(E // R)
                          if pl["slot_expert"][r, j] >= 0}
