"""The C ABI without a GPU: the library loads, exports every entry point
include/moe.h declares, and rejects bad arguments on the host before any
launch (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import expert_load_balance_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.lib_path()):
        pytest.fail("libmoe.so is not built: run `python -m expert_load_balance_amd.build`")
    return moe.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared()
    assert len(names) == 40
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(moe.EXPORTED_SYMBOLS) == names


def test_shape_validation(lib):
    good = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_F32)
    assert moe.moe_check_shape(good) == 0
    bad = [dict(E=0), dict(E=257), dict(k=0), dict(k=9), dict(R=3), dict(R=0), dict(S=-1),
           dict(T=-1), dict(H=0), dict(dtype=7), dict(E=256, k=65, R=4)]
    for kw in bad:
        assert moe.moe_check_shape(good.replace(**kw)) == 1, kw
    assert moe.moe_check_shape(good.replace(H=62)) == 2          # fp32 rows are 16-byte vectors
    assert moe.moe_check_shape(good.replace(dtype=moe.MOE_BF16, F=96)) == 2
    assert moe.moe_check_shape(good.replace(T=1 << 28, k=8)) == 1  # N >= 2^31
    assert moe.moe_check_shape(good.replace(T=0)) == 0
    # bf16 GEMM copy offsets are 32-bit: buffer (N x H) and one expert's weights (F x H)
    bf = good.replace(dtype=moe.MOE_BF16, H=8192, F=1024, E=8, R=4, k=8)
    assert moe.moe_check_shape(bf.replace(T=32767)) == 0           # N*H*2 just below 2^32
    assert moe.moe_check_shape(bf.replace(T=32768)) == 2           # N*H*2 == 2^32
    assert moe.moe_check_shape(bf.replace(T=16, F=262144)) == 2     # F*H*2 >= 2^32
    # and one 256-row tile of h (256 x F): 512 F below 2^32 - 128
    narrow = bf.replace(T=16, H=64)
    assert moe.moe_check_shape(narrow.replace(F=(1 << 23) - 64)) == 0
    assert moe.moe_check_shape(narrow.replace(F=1 << 23)) == 2


def test_probe_rejects_bad_arguments(lib):
    """The calibration probe rejects its arguments on the host (no launch)."""
    f = lib.moe_probe_mfma
    f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    f.restype = ctypes.c_int
    p = ctypes.c_void_p(0x1000)
    assert f(0, 1, p, 256, None) == 1            # no workgroups
    assert f(1, 0, p, 256, None) == 1            # no iterations
    assert f(1, 1, None, 256, None) == 1         # no sink
    assert f(2, 1, p, 511, None) == 1            # sink shorter than 2 x 256
    g = lib.moe_probe_copy
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    g.restype = ctypes.c_int
    q = ctypes.c_void_p(0x2000)
    assert g(None, q, 64, 1, None) == 1          # no source
    assert g(p, q, 0, 1, None) == 1              # nothing to copy
    assert g(p, q, 40, 1, None) == 1             # not whole 16-byte vectors
    assert g(p, ctypes.c_void_p(0x2008), 64, 1, None) == 1  # misaligned
    assert g(p, q, 64, 0, None) == 1             # no workgroups
    h = lib.moe_probe_read
    h.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    h.restype = ctypes.c_int
    assert h(None, 64, 1, q, 256, None) == 1      # no source
    assert h(p, 0, 1, q, 256, None) == 1          # nothing to read
    assert h(p, 40, 1, q, 256, None) == 1         # not whole 16-byte vectors
    assert h(ctypes.c_void_p(0x1008), 64, 1, q, 256, None) == 1  # misaligned
    assert h(p, 64, 0, q, 256, None) == 1         # no workgroups
    assert h(p, 64, 2, q, 511, None) == 1         # sink shorter than 2 x 256
    assert h(p, 64, 1, None, 256, None) == 1      # no sink
    assert h(p, 1 << 31, 1, q, 256, None) == 1    # one chunk of 2 GiB


def test_plan_layout_and_workspace(lib):
    s = moe.Shape(4096, 2048, 128, 8, 768, 16, 8, moe.MOE_BF16)
    L = moe.moe_plan_layout(s)
    R, E, n = 16, 128, 8
    assert L["quota"] == 0 and L["win_off"] == R and L["seg_num"] == 2 * R + 1
    assert L["total"] == R + (R + 1) + R + 3 * R * 2 * n + R + R * n + R + E + 3 * E * R
    ws = moe.moe_workspace_bytes(s)
    assert ws >= 4096 * 8 * 768 * 2              # holds h [N][F] in bf16
    assert moe.moe_workspace_bytes(s.replace(R=3)) == 0


def test_null_and_bad_shape_rejected_before_launch(lib):
    s = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_F32)
    V = ctypes.c_void_p
    p = V(16)  # never dereferenced: validation fails first
    assert lib.moe_route(ctypes.byref(s), None, None, p, p, p, None) == 1
    assert lib.moe_route(ctypes.byref(s.replace(R=3)), p, None, p, p, p, None) == 1
    assert lib.moe_count(ctypes.byref(s), p, p, p, p, p, p, p, 1, None) == 1  # workspace too small
    assert lib.moe_plan(ctypes.byref(s), None, p, None) == 1
    ws_ok = moe.moe_workspace_bytes(s)
    assert lib.moe_count_plan(ctypes.byref(s), p, p, p, p, p, p, p, 1, p, None) == 1  # short ws
    assert lib.moe_count_plan(ctypes.byref(s), p, p, p, p, p, p, p, ws_ok, None, None) == 1  # no plan
    assert lib.moe_count_plan(ctypes.byref(s.replace(R=3)), p, p, p, p, p, p, p, ws_ok, p,
                              None) == 1
    assert lib.moe_permute(ctypes.byref(s), p, p, p, p, None, p, p, None) == 1
    assert lib.moe_grouped_gemm(ctypes.byref(s), p, p, p, p, p, p, p, 1, None) == 1
    assert lib.moe_combine(ctypes.byref(s), p, p, None, None, p, None) == 1
    st = moe.StatsT()
    assert lib.moe_stats(ctypes.byref(s), p, p, p, None, None, None, None, 0.0, p, 1 << 20,
                         ctypes.byref(st), None, None) == 1                 # factor must be > 0
    assert moe.moe_status_str(4).startswith("device error word")
    # the allocation-free count: NULLs, and a shape whose count tables exceed
    # its fixed 8 MiB scratch (N = 2^23 assignments over 256 experts)
    assert lib.moe_count_noalloc(ctypes.byref(s), None, p, p, p, p, p, None) == 1
    big = moe.Shape(1 << 20, 64, 256, 8, 64, 32, 8, moe.MOE_BF16)
    assert lib.moe_count_noalloc(ctypes.byref(big), p, p, p, p, p, p, None) == 1


def test_plan_bytes_and_bind_follow_the_layout(lib):
    # the named tables of moe_plan_bind sit at the layout's offsets of one
    # block of moe_plan_bytes (host arithmetic only; the block is not touched)
    for shp in [(16, 64, 8, 2, 128, 4, 2), (300, 64, 36, 5, 64, 12, 2), (8192, 7168, 256, 8, 2048, 32, 8)]:
        s = moe.Shape(*shp, moe.MOE_BF16)
        L = moe.moe_plan_layout(s)
        assert moe.moe_plan_bytes(s) == 4 * L["total"]
        base = 1 << 20
        t = moe.moe_plan_bind(s, base)
        for name in moe.PLAN_T_FIELDS:
            assert t[name] == base + 4 * L[name], name
    bad = moe.Shape(16, 64, 8, 2, 128, 3, 2, moe.MOE_BF16)     # R does not divide E
    assert moe.moe_plan_bytes(bad) == 0
    out = moe.PlanT()
    assert lib.moe_plan_bind(ctypes.byref(bad), ctypes.c_void_p(1 << 20), ctypes.byref(out)) == 1
    good = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_BF16)
    assert lib.moe_plan_bind(ctypes.byref(good), None, ctypes.byref(out)) == 1
    assert lib.moe_plan_bind(ctypes.byref(good), ctypes.c_void_p(1 << 20), None) == 1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "_LIB_PATH", "/nonexistent/libmoe.so")
    with pytest.raises(RuntimeError):
        moe.load()


def test_capacity_rows_and_rejections(lib):
    s = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_F32)
    # the hotspot fixture's capacity: ceil(32 / 8 * 1.25) = 5
    assert moe.moe_capacity_rows(s, 1.25) == 5
    assert moe.moe_capacity_rows(s, 1.0) == 4
    assert moe.moe_capacity_rows(s, 0.0) == -1
    assert moe.moe_capacity_rows(s, float("nan")) == -1
    assert moe.moe_capacity_rows(s.replace(R=3), 1.25) == -1
    p = ctypes.c_void_p(1)
    # cap < 1 and NULL buffers are rejected before any launch
    assert lib.moe_capacity_dispatch(ctypes.byref(s), 0, p, p, p, p, p, p, None) == 1
    assert lib.moe_capacity_dispatch(ctypes.byref(s), 5, None, p, p, p, p, p, None) == 1
    assert lib.moe_capacity_plan(ctypes.byref(s), 0, p, None) == 1
    assert lib.moe_capacity_combine(ctypes.byref(s), 5, None, p, p, None, p, None) == 1
    assert lib.moe_repack(ctypes.byref(s), None, p, None) == 1
    assert lib.moe_repack(ctypes.byref(s.replace(E=0)), p, p, None) == 1


def test_router_workspace_and_rejections(lib):
    """The router's K-split needs parts * T * E * 4 bytes of partial logits
    (at most 16 parts); none for fp32 or when the token tiles alone fill the
    GPU. Too small a workspace and too wide a W_r are rejected before launch."""
    bf = moe.Shape(2048, 4096, 8, 2, 64, 1, 0, moe.MOE_BF16)
    for T, H, E in [(2048, 4096, 8), (64, 4096, 128), (4096, 2048, 128), (8192, 7168, 256),
                    (1, 64, 8), (100, 256, 64)]:
        s = bf.replace(T=T, H=H, E=E, k=2)
        b = moe.moe_router_workspace_bytes(s)
        assert b % (T * E * 4) == 0 and b // (T * E * 4) in (0,) + tuple(range(2, 17)), (T, H, E)
    assert moe.moe_router_workspace_bytes(bf.replace(T=64)) > 0            # 2 tiles: split K
    assert moe.moe_router_workspace_bytes(bf.replace(T=1 << 16)) == 0      # 2048 tiles
    assert moe.moe_router_workspace_bytes(bf.replace(H=128)) == 0          # 2 stages: no split
    assert moe.moe_router_workspace_bytes(bf.replace(dtype=moe.MOE_F32)) == 0
    assert moe.moe_router_workspace_bytes(bf.replace(R=3)) == 0
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    s = bf.replace(T=64)
    need = moe.moe_router_workspace_bytes(s)
    assert lib.moe_router(ctypes.byref(s), p, p, None, p, p, p, p, p, need - 1, None) == 1
    assert lib.moe_router(ctypes.byref(s), p, p, None, p, p, p, p, None, need, None) == 1
    assert lib.moe_router(ctypes.byref(s), p, p, None, p, p, p, None, p, need, None) == 1
    wide = bf.replace(T=1, k=1, E=256, H=1 << 23, F=64)                  # E*H*2 == 2^32
    assert moe.moe_check_shape(wide) == 0
    assert lib.moe_router(ctypes.byref(wide), p, p, None, p, p, p, p, p, 1 << 40, None) == 2


def test_pool_bytes_and_slot_rejections(lib):
    s = moe.Shape(16, 64, 8, 2, 128, 4, 2, moe.MOE_F32)          # n = 2
    assert moe.moe_pool_bytes(s) == 4 * 2 * 3 * 128 * 64 * 4
    assert moe.moe_pool_bytes(s.replace(S=5)) == moe.moe_pool_bytes(s)   # at most n slots
    assert moe.moe_pool_bytes(s.replace(S=1)) == 4 * 1 * 3 * 128 * 64 * 4
    assert moe.moe_pool_bytes(s.replace(S=0)) == 0
    assert moe.moe_pool_bytes(s.replace(dtype=moe.MOE_BF16)) == 4 * 2 * 3 * 128 * 64 * 2
    assert moe.moe_pool_bytes(s.replace(R=3)) == 0
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    need = moe.moe_pool_bytes(s)
    assert lib.moe_prefetch_replicas(ctypes.byref(s), p, p, p, p, p, need - 1, None) == 1
    assert lib.moe_prefetch_replicas(ctypes.byref(s), None, p, p, p, p, need, None) == 1
    assert lib.moe_prefetch_replicas(ctypes.byref(s), p, p, p, p, None, need, None) == 1
    assert lib.moe_grouped_gemm_slots(ctypes.byref(s), p, p, p, p, p, p, need, p, p, 1,
                                      None) == 1                       # workspace too small
    assert lib.moe_grouped_gemm_slots(ctypes.byref(s), p, p, p, p, p, p, need - 1, p, p,
                                      1 << 30, None) == 1              # pool too small


def test_backward_workspace_and_rejections(lib):
    bf = moe.Shape(2048, 4096, 8, 2, 14336, 8, 1, moe.MOE_BF16)
    N, H, F = 4096, 4096, 14336
    b = moe.moe_backward_workspace_bytes(bf)
    assert b >= N * (2 * H + 5 * F) * 2                      # x, dy, g|u, dg|du, h
    assert moe.moe_backward_workspace_bytes(bf.replace(dtype=moe.MOE_F32)) >= N * (2 * H + 5 * F) * 4
    assert moe.moe_backward_workspace_bytes(bf.replace(R=3)) == 0
    s = moe.Shape(64, 128, 8, 2, 128, 4, 1, moe.MOE_BF16)
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    need = moe.moe_backward_workspace_bytes(s)
    assert lib.moe_ffn_backward(ctypes.byref(s), p, p, p, p, p, None, p, p, p, p, p, p, need - 1,
                                None) == 1                    # workspace too small
    assert lib.moe_ffn_backward(ctypes.byref(s), p, None, p, p, p, None, p, p, p, p, p, p, 1 << 30,
                                None) == 1                    # no plan
    assert lib.moe_grouped_gemm_train(ctypes.byref(s), p, p, p, p, p, p, None, p, 1 << 30,
                                      None) == 1              # bf16 needs the g | u buffer
    assert lib.moe_combine_backward(ctypes.byref(s), p, p, p, p, None, p, None) == 1
    assert lib.moe_permute_backward(ctypes.byref(s), None, p, p, None) == 1
    assert lib.moe_route_backward(ctypes.byref(s), p, p, None, p, None) == 1


def test_replica_grad_bytes_and_rejections(lib):
    s = moe.Shape(64, 128, 8, 2, 128, 4, 1, moe.MOE_BF16)       # n = 2
    assert moe.moe_replica_grad_bytes(s) == 4 * 2 * 3 * 128 * 128 * 4
    assert moe.moe_replica_grad_bytes(s.replace(R=3)) == 0
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    need = moe.moe_replica_grad_bytes(s)
    big = 1 << 40
    assert lib.moe_ffn_backward_replicas(ctypes.byref(s), p, p, p, p, p, None, p, p, p, p, p, p,
                                         need - 1, p, big, None) == 1      # slots too small
    assert lib.moe_ffn_backward_replicas(ctypes.byref(s.replace(dtype=moe.MOE_F32)), p, p, p, p,
                                         p, None, p, p, p, p, p, p, need, p, big, None) == 2
