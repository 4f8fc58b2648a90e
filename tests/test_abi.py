"""The C ABI library: it loads, exports every symbol include/moe.h declares, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from speculative_verify_moe_amd import _lib
    return _lib


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("moe_route_topk", "moe_align", "moe_experts_forward", "moe_layer_forward"):
        assert required in names
    assert len(names) >= 11


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(lib.EXPORTS), "binding and header disagree"


def test_capacity_arithmetic(lib):
    f = lib.moe_align_capacity
    assert f(3, 2, 4, 16) == 80          # roundup(6 + 4*15, 16)
    assert f(8, 8, 256, 16) == 64 + 64 * 15
    assert f(4096, 8, 256, 64) == -(-(32768 + 256 * 63) // 64) * 64
    assert f(0, 8, 256, 16) == 0
    assert f(1, 1, 1, 8) == 0          # BM not allowed
    assert f(-1, 1, 1, 16) == 0
    assert lib.moe_align_workspace_size(8, 8, 256) == 0          # one-block path
    assert lib.moe_align_workspace_size(4096, 8, 256) == 128 * 256 * 4


def _c(lib, name):
    return getattr(lib._lib, name)


def test_route_topk_validation(lib):
    f = _c(lib, "moe_route_topk")
    P = ctypes.c_void_p
    assert f(None, 0, 16, 2, 1, None, None, None) == lib.MOE_OK                  # T == 0: nothing to do
    assert f(None, -1, 16, 2, 1, None, None, None) == lib.MOE_ERR_INVALID_ARG
    assert f(P(16), 4, 16, 17, 1, P(16), P(16), None) == lib.MOE_ERR_INVALID_ARG  # k > E
    assert "top_k" in lib.moe_last_error()
    assert f(P(16), 4, 2000, 2, 1, P(16), P(16), None) == lib.MOE_ERR_INVALID_ARG  # E > 1024
    assert f(P(16), 4, 64, 33, 1, P(16), P(16), None) == lib.MOE_ERR_INVALID_ARG   # k > 32
    assert f(None, 4, 16, 2, 1, P(16), P(16), None) == lib.MOE_ERR_INVALID_ARG
    assert f(P(18), 4, 16, 2, 1, P(16), P(16), None) == lib.MOE_ERR_MISALIGNED


def test_align_validation(lib):
    f = _c(lib, "moe_align")
    P = ctypes.c_void_p
    good = [P(256)] * 5
    assert f(P(256), 8, 8, 256, 8, 1024, *good, None, 0, None) == lib.MOE_ERR_INVALID_ARG      # BM
    assert f(P(256), 8, 8, 256, 16, 1008, *good, None, 0, None) == lib.MOE_ERR_WORKSPACE       # cap too small
    assert "moe_align_capacity" in lib.moe_last_error()
    assert f(P(256), 8, 8, 256, 16, 1032, *good, None, 0, None) == lib.MOE_ERR_INVALID_ARG     # cap % BM
    assert f(P(256), 8, 8, 256, 16, 1024, None, *good[1:], None, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert f(P(256), 4096, 8, 256, 64, 48896, *good, None, 0, None) == lib.MOE_ERR_WORKSPACE  # ws needed


def _fake_layer(lib, T_shared=True, wtype=0, E=256, k=8, H=2048, I=512):
    P = ctypes.c_void_p
    sb = ctypes.c_void_p(4096) if wtype in (1, 2) else None  # fp8 row scales
    mb = ctypes.c_void_p(4097) if wtype == 3 else None       # MXFP4 block-scale bytes (any alignment)
    routed = lib._Bank(wtype, E, H, I, P(4096), P(4096), sb, sb, mb, mb)
    shared = lib._Bank(wtype, 1 if T_shared else 0, H, I, P(4096), P(4096), sb, sb, mb, mb)
    return lib._Layer(H, E, k, 1, P(4096), None, routed, shared, P(4096) if T_shared else None)


def test_layer_validation(lib):
    f = _c(lib, "moe_layer_forward")
    P = ctypes.c_void_p
    L = _fake_layer(lib)
    assert f(P(4096), 0, ctypes.byref(L), P(4096), None, None, None, None, 0, None) == lib.MOE_OK
    assert f(P(4096), -2, ctypes.byref(L), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert f(P(4096), 8, None, P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert f(P(4100), 8, ctypes.byref(L), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_MISALIGNED
    assert f(P(4096), 8, ctypes.byref(L), P(4096), None, None, None, P(4096), 10, None) == lib.MOE_ERR_WORKSPACE
    assert "moe_layer_workspace_size" in lib.moe_last_error()
    bad = _fake_layer(lib, H=2000)
    assert f(P(4096), 8, ctypes.byref(bad), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    bad = _fake_layer(lib, I=500)
    assert f(P(4096), 8, ctypes.byref(bad), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    nos = _fake_layer(lib)
    nos.shared_gate_w = None
    assert f(P(4096), 8, ctypes.byref(nos), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    fp8 = _fake_layer(lib, wtype=1)
    # fp8 weights are accepted on the prefill path too: the call gets as far as the workspace
    assert f(P(4096), 4096, ctypes.byref(fp8), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_WORKSPACE
    fp8.routed.s_down = None
    assert f(P(4096), 8, ctypes.byref(fp8), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    mx = _fake_layer(lib, wtype=3)
    # MXFP4 scale bytes travel in their own fields, with no alignment asked of them
    assert f(P(4096), 8, ctypes.byref(mx), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_WORKSPACE
    assert f(P(4096), 4096, ctypes.byref(mx), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_UNSUPPORTED
    mx.routed.mx_down = None
    assert f(P(4096), 8, ctypes.byref(mx), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert "mx_gate_up and mx_down" in lib.moe_last_error()
    mx = _fake_layer(lib, wtype=3)
    mx.routed.s_gate_up = ctypes.c_void_p(4098)  # fp8 row-scale fields are ignored for MXFP4
    assert f(P(4096), 8, ctypes.byref(mx), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_WORKSPACE
    fp8 = _fake_layer(lib, wtype=1)
    fp8.routed.mx_gate_up = None  # and the MXFP4 fields for fp8
    fp8.routed.s_gate_up = ctypes.c_void_p(4098)
    assert f(P(4096), 8, ctypes.byref(fp8), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_MISALIGNED
    wt = _fake_layer(lib)
    wt.routed.wtype = 7
    assert f(P(4096), 8, ctypes.byref(wt), P(4096), None, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG


def test_workspace_sizes_and_plans(lib):
    L = _fake_layer(lib)
    wsz = _c(lib, "moe_layer_workspace_size")
    plan = _c(lib, "moe_describe_plan")
    w8 = wsz(8, ctypes.byref(L))
    w4096 = wsz(4096, ctypes.byref(L))
    assert w8 > 8 * 8 * 512 * 2 and w4096 > 48896 * 512 * 2 + 32768 * 2048 * 2
    assert wsz(0, ctypes.byref(L)) == 0
    assert b"path=decode" in plan(8, ctypes.byref(L))
    assert b"path=prefill" in plan(4096, ctypes.byref(L))
    assert b"path=decode" in plan(64, ctypes.byref(L))
    assert b"path=prefill" in plan(65, ctypes.byref(L))
    # prefill with a shared expert: its two GEMMs are stages 0 and 1, on the second stream;
    # without one, or with fp8 activations, the routed and shared segments share one launch
    import bench
    p = plan(4096, ctypes.byref(L)).decode()
    assert bench.plan_stages(p) == ["shared_gate_up_mfma", "shared_down_mfma", "router_gemm_mfma", "topk", "align",
                                    "gemm_gate_up_mfma", "gemm_down_mfma", "combine"]
    assert "second stream" in p
    nos = _fake_layer(lib, T_shared=False)
    p = plan(4096, ctypes.byref(nos)).decode()
    assert bench.plan_stages(p) == ["router_gemm_mfma", "topk", "align", "gemm_gate_up_mfma", "gemm_down_mfma", "combine"]
    a8 = _fake_layer(lib, wtype=2)
    p = plan(4096, ctypes.byref(a8)).decode()
    assert bench.plan_stages(p)[0] == "router_gemm_mfma" and "second stream" not in p
    assert bench.plan_stages(plan(8, ctypes.byref(L)).decode()) in (
        ["moe_decode_fused"], ["router_rows", "topk_align_small", "gemv_gate_up", "gemv_down_combine"])
    ew = _c(lib, "moe_experts_workspace_size")
    tl = -(-(1 + 256 + 257 + 64) * 4 // 256) * 256           # compact touched-expert list
    assert ew(8, 8, ctypes.byref(L.routed), 16) == 8 * 8 * 512 * 2 + tl


def test_status_word_sits_in_the_synchronisation_words(lib):
    """The status word lies inside the words every plan keeps at offset 0, below the smallest
    workspace of any call."""
    off = lib._lib.moe_workspace_status_offset()
    assert off % 4 == 0 and 0 < off < 16384
    L = _fake_layer(lib, E=16, k=2, H=256, I=128)
    wsz = _c(lib, "moe_layer_workspace_size")
    for T in (1, 8, 64, 65, 4096):
        assert wsz(T, ctypes.byref(L)) >= off + 4


def test_stage_events_hook_bounds(lib):
    f = _c(lib, "moe_set_stage_events")
    arr = (ctypes.c_void_p * 65)()
    assert f(arr, 65) == lib.MOE_ERR_INVALID_ARG
    assert f(None, 0) == lib.MOE_OK


def test_stream_read_probe_rejects_bad_arguments(lib):
    """The streaming-read measurement aid validates before it touches a device."""
    f = _c(lib, "moe_measure_stream_read")
    buf = ctypes.c_void_p(1 << 20)    # never dereferenced: every call below fails validation
    sink = ctypes.c_void_p(1 << 21)
    assert f(None, 1024, 256, 8, sink, None) == lib.MOE_ERR_INVALID_ARG
    assert f(buf, 0, 256, 8, sink, None) == lib.MOE_ERR_INVALID_ARG
    assert f(buf, 1000, 256, 8, sink, None) == lib.MOE_ERR_INVALID_ARG
    assert f(ctypes.c_void_p((1 << 20) + 8), 1024, 256, 8, sink, None) == lib.MOE_ERR_MISALIGNED
    assert f(buf, 1024, 0, 8, sink, None) == lib.MOE_ERR_INVALID_ARG
    assert f(buf, 1024, 256, 6, sink, None) == lib.MOE_ERR_INVALID_ARG
    assert "depth" in lib.moe_last_error()
