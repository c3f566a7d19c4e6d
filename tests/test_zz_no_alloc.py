"""The allocation-free count (moe_count_noalloc) against moe_count through
the C ABI: bit-exact counts, offsets, stable indices, rank loads and error
word on consecutive calls that share the library's fixed device scratch --
a large batch, then a smaller one (both on the multi-launch path that uses
the scratch), then one small enough for the one-workgroup path, then a
batch with bad ids."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import expert_load_balance_amd as moe  # noqa: E402
from expert_load_balance_amd.layer import alloc  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ids(T, E, k, seed, s_bias):
    lg = synth.router_logits(T, E, seed)
    bias = synth.zipf_bias(E, s_bias, seed)
    shape = moe.Shape(T, 64, E, k, 64, 16 if E % 16 == 0 else 1, 1, moe.MOE_BF16)
    ids = alloc((T, k), torch.int32, DEV)
    w = alloc((T, k), torch.float32, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_route(shape, torch.from_numpy(lg).to(DEV), torch.from_numpy(bias).to(DEV), ids, w, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return shape, ids


def _count(shape, ids, fn):
    i32 = torch.int32
    out = dict(counts=alloc((shape.E,), i32, DEV), offsets=alloc((shape.E + 1,), i32, DEV),
               eidx=alloc((shape.N,), i32, DEV), rank_load=alloc((shape.R,), i32, DEV),
               err=torch.zeros(1, dtype=i32, device=DEV))
    for t in ("counts", "offsets", "eidx", "rank_load"):
        out[t].fill_(-9)
    if fn == "ws":
        ws = torch.empty(max(moe.moe_workspace_bytes(shape), 256), dtype=torch.uint8, device=DEV)
        moe.moe_count(shape, ids, out["counts"], out["offsets"], out["eidx"], out["rank_load"],
                      out["err"], ws)
    else:
        moe.moe_count_noalloc(shape, ids, out["counts"], out["offsets"], out["eidx"],
                              out["rank_load"], out["err"])
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}


def test_count_noalloc_matches_count_on_consecutive_calls():
    cases = [(8192, 256, 8, 71, 0.6),    # 65536 assignments: 64 counting workgroups
             (3000, 128, 8, 72, 0.2),    # 24000: fewer workgroups, stale tables beyond them
             (700, 64, 4, 73, 0.9)]      # 2800: the one-workgroup path
    for T, E, k, seed, sb in cases:
        print(f"[case] count_noalloc T={T} E={E} k={k}", flush=True)
        shape, ids = _ids(T, E, k, seed, sb)
        a = _count(shape, ids, "noalloc")
        b = _count(shape, ids, "ws")
        for name in ("counts", "offsets", "eidx", "rank_load", "err"):
            np.testing.assert_array_equal(a[name], b[name], err_msg=f"{name} T={T} E={E}")
        ref = oracle.count(ids.cpu().numpy(), E, shape.R)
        np.testing.assert_array_equal(a["eidx"], ref["eidx"])
        np.testing.assert_array_equal(a["counts"], ref["counts"])


def test_count_noalloc_flags_bad_ids_like_count():
    T, E, k = 5000, 64, 4                # 20000 assignments: the scratch path
    shape = moe.Shape(T, 64, E, k, 64, 16, 1, moe.MOE_BF16)
    base = ((np.arange(T)[:, None] * 3 + np.arange(k)[None, :]) % E).astype(np.int32)
    base[17, 2] = E + 3                  # out of range
    base[4001, 3] = base[4001, 0]        # repeated within a token
    ids = torch.from_numpy(base).to(DEV)
    a = _count(shape, ids, "noalloc")
    b = _count(shape, ids, "ws")
    for name in ("counts", "offsets", "eidx", "rank_load", "err"):
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)
    assert a["err"][0] & moe.ERR_RANGE and a["err"][0] & moe.ERR_REPEAT
