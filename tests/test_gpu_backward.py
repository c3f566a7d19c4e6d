"""GPU parity of the layer's backward (the chain rule of the forward: combine,
SwiGLU expert FFN with the replicas' weight gradients summed into the home
expert, dispatch, gate) against the CPU oracle, whose backward is pinned by
central differences of the forward.

Each backward entry point is fed the same inputs as the oracle's step: the
oracle's forward integers, permuted rows and gate weights (uploaded to the
device) and seeded upstream gradients. The whole chain is also run on the
device from the GPU forward's own buffers and compared with the oracle's
chain from the layer's inputs.

Bar (bf16 layers): bf16 outputs (dy, dbuf, dx) and the weight gradients --
fp32 stores, but computed through the bf16-rounded g, u, dg, du and h --
within 2e-2 * max|ref|; dw and dlogits (fp32 from identical inputs) within
1e-5 * max|ref|; the chain within 2e-2 * max|ref|. fp32 layers (the hotspot
fixture and a random small shape): everything within 1e-5 * max|ref|.
Full-size shapes check sampled rows of dbuf and sampled columns f of every
weight gradient (the FFN splits over f, so the oracle on those columns gives
the exact entries).
"""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl

torch = pytest.importorskip("torch")
import expert_load_balance_amd as moe  # noqa: E402
from expert_load_balance_amd.layer import alloc  # noqa: E402

from test_gpu_parity import (DEV, assert_tol, host, make_weights, oracle_forward,  # noqa: E402
                             run_layer, upload_bits, upload_plan)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


class Backward:
    """The forward on the device (for the chain), the oracle's forward, and
    every backward entry point on inputs both sides share."""

    def __init__(self, shape, lg, bias, seed):
        s = shape
        self.shape = s
        act = torch.bfloat16 if s.dtype == moe.MOE_BF16 else torch.float32
        self.act = act
        self.x = synth.device_normal((s.T, s.H), 1.0, seed, act, DEV)
        self.wts = make_weights(s.E, s.F, s.H, s.dtype, seed)
        self.L = run_layer(s, lg, bias, self.x, self.wts)
        o = oracle_forward(s, lg, bias, self.x)
        self.o, self.pl = o, o["pl"]
        # the oracle's forward on the device, and seeded upstream gradients
        self.d_ids = torch.from_numpy(o["ids"]).to(DEV)
        self.w32 = o["w"].astype(np.float32)
        self.d_w = torch.from_numpy(self.w32).to(DEV)
        self.d_dest = torch.from_numpy(o["dest"]).to(DEV)
        self.d_buf = upload_bits(o["buf_bits"], act)
        self.d_plan = upload_plan(o["pl"], s)
        self.dout = synth.device_normal((s.T, s.H), 1.0, seed + 100, act, DEV)
        self.y_in = synth.device_normal((s.N, s.H), 0.5, seed + 101, act, DEV)
        self.dy_in = synth.device_normal((s.N, s.H), 1.0, seed + 102, act, DEV)
        self.dbuf_in = synth.device_normal((s.N, s.H), 1.0, seed + 103, act, DEV)
        self.dw_in = synth.device_normal((s.T, s.k), 1.0, seed + 104, torch.float32, DEV)
        # the four steps
        self.dy = alloc((s.N, s.H), act, DEV)
        self.dw = alloc((s.T, s.k), torch.float32, DEV)
        moe.moe_combine_backward(s, self.dout, self.y_in, self.d_dest, self.d_w, self.dy, self.dw)
        self.dbuf = alloc((s.N, s.H), act, DEV)
        self.dW = self.new_grads()
        self.ws = alloc((moe.moe_backward_workspace_bytes(s),), torch.uint8, DEV)
        moe.moe_ffn_backward(s, self.d_buf, self.d_plan, *self.wts, self.dy_in, self.dbuf,
                             *self.dW, self.ws)
        self.dx = alloc((s.T, s.H), act, DEV)
        moe.moe_permute_backward(s, self.dbuf_in, self.d_dest, self.dx)
        self.dlogits = alloc((s.T, s.E), torch.float32, DEV)
        moe.moe_route_backward(s, self.d_ids, self.d_w, self.dw_in, self.dlogits)
        torch.cuda.synchronize()

    def new_grads(self):
        s = self.shape
        dW = [alloc((s.E, s.F, s.H), torch.float32, DEV), alloc((s.E, s.F, s.H), torch.float32, DEV),
              alloc((s.E, s.H, s.F), torch.float32, DEV)]
        for t in dW:
            t.fill_(float("nan"))                     # every entry must be written
        return dW

    def chain(self):
        """The whole backward on the device from dout, through the GPU
        forward's own y, rows, plan and gate weights."""
        s, L = self.shape, self.L
        dy = alloc((s.N, s.H), self.act, DEV)
        dw = alloc((s.T, s.k), torch.float32, DEV)
        moe.moe_combine_backward(s, self.dout, L.y, L.dest_row, L.w, dy, dw)
        dbuf = alloc((s.N, s.H), self.act, DEV)
        dW = self.new_grads()
        moe.moe_ffn_backward(s, L.buf, L.plan, *self.wts, dy, dbuf, *dW, self.ws)
        dx = alloc((s.T, s.H), self.act, DEV)
        moe.moe_permute_backward(s, dbuf, L.dest_row, dx)
        dl = alloc((s.T, s.E), torch.float32, DEV)
        moe.moe_route_backward(s, L.ids, L.w, dw, dl)
        torch.cuda.synchronize()
        return dx, dl, dW


SMALL = [
    # name, T, H, E, k, F, R, bias strength
    ("ragged_f", 300, 128, 8, 2, 192, 4, 0.6),
    ("multi_tile", 700, 256, 8, 2, 384, 4, 0.5),
    ("idle_experts", 100, 256, 16, 4, 128, 4, 3.0),
    ("k1_tiny", 64, 64, 4, 1, 64, 2, 0.0),
    ("many_experts", 512, 128, 64, 8, 64, 16, 0.8),
    # 2F / 64 = 16 stages and few tiles: the dx GEMM splits K in two parts
    ("dx_k_split", 300, 256, 2, 1, 512, 2, 0.0),
]


SMALL_F32 = [
    ("f32_random", 150, 96, 8, 2, 100, 4, 0.4, moe.MOE_F32),
    ("f32_hotspot_fixture", 16, 64, 8, 2, 128, 4, None, moe.MOE_F32),
]
SMALL = [c + (moe.MOE_BF16,) for c in SMALL] + SMALL_F32


def _f64(t):
    return host(t).astype(np.float64)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small(case):
    name, T, H, E, k, F, R, sb, dtype = case
    _say(f"[case] backward {name}")
    shape = moe.Shape(T, H, E, k, F, R, 1, dtype)
    if sb is None:                                  # the page's 16 tokens
        lg, bias = synth.fixture_logits(), None
    else:
        lg = synth.router_logits(T, E, 51)
        bias = synth.zipf_bias(E, sb, 51).astype(np.float32) if sb else None
    act_tol = dtype                                 # bf16 outputs: bf16 bar; fp32: fp32 bar
    b = Backward(shape, lg, bias, 52)
    o = b.o
    w = b.w32.astype(np.float64)
    # combine backward
    dy_ref, dw_ref = oracle.combine_backward(_f64(b.dout), _f64(b.y_in), o["dest"], w)
    assert_tol(host(b.dy), dy_ref, act_tol, "dy")
    assert_tol(host(b.dw), dw_ref, moe.MOE_F32, "dw")
    # FFN backward
    wh = [_f64(t) for t in b.wts]
    dbuf_ref, dwg, dwu, dwd = oracle.expert_ffn_backward(o["buf"], _f64(b.dy_in), o["pl"], *wh)
    assert_tol(host(b.dbuf), dbuf_ref, act_tol, "dbuf")
    for got, ref, nm in zip(b.dW, (dwg, dwu, dwd), ("dW_gate", "dW_up", "dW_down")):
        g = host(got)
        assert np.isfinite(g).all(), nm
        assert_tol(g, ref, act_tol, nm)
    idle = np.where(o["c"]["counts"] == 0)[0]
    for e in idle:                                   # experts nobody chose: zero gradients
        assert not host(b.dW[0][e]).any() and not host(b.dW[2][e]).any()
    # dispatch and gate backward
    assert_tol(host(b.dx), oracle.permute_backward(_f64(b.dbuf_in), o["dest"]), act_tol, "dx")
    dl_ref = oracle.route_backward(o["ids"], w, _f64(b.dw_in), E)
    assert_tol(host(b.dlogits), dl_ref, moe.MOE_F32, "dlogits")
    if name == "idle_experts":
        assert len(idle) > 0


def test_backward_chain_against_the_oracle_layer():
    """The whole chain from dout on the device (from the GPU forward) against
    every step in the oracle (double, from the layer's inputs): dx, dlogits
    and the weight gradients."""
    T, H, E, k, F, R = 256, 128, 8, 2, 128, 4
    shape = moe.Shape(T, H, E, k, F, R, 1, moe.MOE_BF16)
    lg = synth.router_logits(T, E, 53)
    bias = synth.zipf_bias(E, 0.7, 53).astype(np.float32)
    b = Backward(shape, lg, bias, 54)
    o = b.o
    ids, w, pl, dest, buf = o["ids"], o["w"], o["pl"], o["dest"], o["buf"]
    wh = [_f64(t) for t in b.wts]
    y = np.zeros((T * k, H))
    for e in range(E):
        rows = [r for p in range(pl["piece_num"][e])
                for r in range(pl["piece_row"][e, p], pl["piece_row"][e, p] + pl["piece_cnt"][e, p])]
        if rows:
            y[rows] = oracle.ffn_rows(buf[rows], wh[0][e], wh[1][e], wh[2][e])
    dy, dw = oracle.combine_backward(_f64(b.dout), y, dest, w)
    dbuf, dwg, dwu, dwd = oracle.expert_ffn_backward(buf, dy, pl, *wh)
    dx, dl, dW = b.chain()
    assert_tol(host(dx), oracle.permute_backward(dbuf, dest), moe.MOE_BF16, "dx (chain)")
    assert_tol(host(dl), oracle.route_backward(ids, w, dw, E), moe.MOE_BF16, "dlogits (chain)")
    for got, ref, nm in zip(dW, (dwg, dwu, dwd), ("dW_gate", "dW_up", "dW_down")):
        assert_tol(host(got), ref, moe.MOE_BF16, nm + " (chain)")


@pytest.mark.parametrize("name,maxvio", [("mixtral", 0.2), ("a3b", 1)])
def test_backward_full_size(name, maxvio):
    _say(f"[case] backward full {name}@{maxvio}")
    torch.cuda.empty_cache()
    w_ = wl.WORKLOADS[name]
    T, H, E, k, F, R, S = (w_[c] for c in ("T", "H", "E", "k", "F", "R", "S"))
    shape = moe.Shape(T, H, E, k, F, R, S, moe.MOE_BF16)
    lg, bias = wl.logits_and_bias(name, maxvio)
    b = Backward(shape, lg, bias, w_["seed"])
    pl = b.pl
    counts = b.o["c"]["counts"]
    for t, nm in zip(b.dW, ("dW_gate", "dW_up", "dW_down")):
        assert bool(torch.isfinite(t).all()), nm
    rng = np.random.default_rng(9)
    e = int(np.argmax(counts))                      # the hottest expert: home + replica pieces
    rows = np.array([r for p in range(pl["piece_num"][e])
                     for r in range(pl["piece_row"][e, p], pl["piece_row"][e, p] + pl["piece_cnt"][e, p])])
    assert pl["piece_num"][e] >= 1 and len(rows) == counts[e]
    xr = b.o["buf"][rows]
    dyr = host(b.dy_in[torch.from_numpy(rows).to(DEV)]).astype(np.float64)
    wg, wu, wd = (host(t[e]).astype(np.float64) for t in b.wts)
    # sampled columns f of the weight gradients (exact: the FFN splits over f)
    fs = np.sort(rng.choice(F, 6, replace=False))
    _, g_s, u_s, d_s = oracle.ffn_backward_rows(xr, dyr, wg[fs], wu[fs], wd[:, fs])
    assert_tol(host(b.dW[0][e])[fs], g_s, moe.MOE_BF16, "dW_gate (sampled f)")
    assert_tol(host(b.dW[1][e])[fs], u_s, moe.MOE_BF16, "dW_up (sampled f)")
    assert_tol(host(b.dW[2][e])[:, fs], d_s, moe.MOE_BF16, "dW_down (sampled f)")
    # sampled rows of dbuf (full F)
    pick = rng.choice(len(rows), 3, replace=False)
    dx_s, _, _, _ = oracle.ffn_backward_rows(xr[pick], dyr[pick], wg, wu, wd)
    assert_tol(host(b.dbuf[torch.from_numpy(rows[pick]).to(DEV)]), dx_s, moe.MOE_BF16,
               "dbuf (sampled rows)")
    # experts with no rows have zero gradients
    for e0 in np.where(counts == 0)[0][:2]:
        assert not bool(b.dW[2][int(e0)].any())


@pytest.mark.parametrize("case", [c for c in SMALL if c[-1] == moe.MOE_BF16][:3] + [
    ("mixtral_like", 300, 256, 4, 2, 1024, 4, 0.5, moe.MOE_BF16)], ids=lambda c: c[0])
def test_backward_with_saved_gate_up(case):
    """The training forward keeps g | u (moe_grouped_gemm_train): its y is
    bit-identical to the plain forward's, and the backward fed with the saved
    g | u (no recompute) meets the same oracle bar as the recomputing one."""
    name, T, H, E, k, F, R, sb, dtype = case
    _say(f"[case] backward with saved g|u {name}")
    shape = moe.Shape(T, H, E, k, F, R, 1, dtype)
    lg = synth.router_logits(T, E, 55)
    bias = synth.zipf_bias(E, sb, 55).astype(np.float32) if sb else None
    b = Backward(shape, lg, bias, 56)
    L = b.L
    y2 = alloc((shape.N, H), torch.bfloat16, DEV)
    gu = alloc((shape.N, 2 * F), torch.bfloat16, DEV)
    moe.moe_grouped_gemm_train(shape, b.d_buf, b.d_plan, *b.wts, y2, gu, L.ws)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), L.y.view(torch.int16))
    dbuf2 = alloc((shape.N, H), torch.bfloat16, DEV)
    dW2 = [torch.full_like(t, float("nan")) for t in b.dW]
    moe.moe_ffn_backward(shape, b.d_buf, b.d_plan, *b.wts, b.dy_in, dbuf2, *dW2, b.ws, gu=gu)
    torch.cuda.synchronize()
    wh = [host(t).astype(np.float64) for t in b.wts]
    dbuf_ref, dwg, dwu, dwd = oracle.expert_ffn_backward(b.o["buf"], _f64(b.dy_in), b.pl, *wh)
    assert_tol(host(dbuf2), dbuf_ref, moe.MOE_BF16, "dbuf (saved g|u)")
    for got, ref, nm in zip(dW2, (dwg, dwu, dwd), ("dW_gate", "dW_up", "dW_down")):
        assert_tol(host(got), ref, moe.MOE_BF16, nm + " (saved g|u)")
    assert_tol(host(dbuf2), host(b.dbuf).astype(np.float64), moe.MOE_BF16, "saved vs recomputed")


@pytest.mark.parametrize("case", [
    ("skewed_4ranks", 400, 128, 8, 2, 256, 4, 1.5),
    ("fine_grained", 512, 128, 32, 4, 128, 8, 1.0),
], ids=lambda c: c[0])
def test_backward_replica_reduction(case):
    """moe_ffn_backward_replicas: every filled replica slot holds its replica
    piece's weight gradient (against the oracle on that piece's rows), slots
    without a replica are not written, and the reduced gradients match the
    oracle and moe_ffn_backward's (fp32 bar: only the summation grouping
    differs)."""
    name, T, H, E, k, F, R, sb = case
    _say(f"[case] backward replica reduction {name}")
    shape = moe.Shape(T, H, E, k, F, R, E // R, moe.MOE_BF16)
    lg = synth.router_logits(T, E, 57)
    bias = synth.zipf_bias(E, sb, 57).astype(np.float32)
    b = Backward(shape, lg, bias, 58)
    n = E // R
    rgrad = torch.full((moe.moe_replica_grad_bytes(shape) // 4,), float("nan"), dtype=torch.float32,
                       device=DEV)
    dW2 = [torch.full_like(t, float("nan")) for t in b.dW]
    dbuf2 = alloc((shape.N, H), torch.bfloat16, DEV)
    moe.moe_ffn_backward_replicas(shape, b.d_buf, b.d_plan, *b.wts, b.dy_in, dbuf2, *dW2, rgrad,
                                  b.ws)
    torch.cuda.synchronize()
    wh = [host(t).astype(np.float64) for t in b.wts]
    rg, ru, rd, slots = oracle.replica_backward(b.o["buf"], _f64(b.dy_in), b.pl, *wh)
    assert len(slots) > 0
    rv = host(rgrad).reshape(R, n, 3, F * H)
    for r in range(R):
        for j in range(n):
            if (r, j) in slots:
                g, u, d = slots[(r, j)]
                for q, ref, nm in ((0, g, "gate"), (1, u, "up"), (2, d, "down")):
                    assert_tol(rv[r, j, q], ref.ravel(), moe.MOE_BF16, f"slot ({r},{j}) {nm}")
            else:
                assert np.isnan(rv[r, j]).all()               # not written
    for got, ref, ref2, nm in zip(dW2, (rg, ru, rd), b.dW, ("dW_gate", "dW_up", "dW_down")):
        assert_tol(host(got), ref, moe.MOE_BF16, nm + " (replica reduction)")
        assert_tol(host(got), host(ref2).astype(np.float64), moe.MOE_F32, nm + " vs expert sums")
    assert torch.equal(dbuf2.view(torch.int16), b.dbuf.view(torch.int16))
