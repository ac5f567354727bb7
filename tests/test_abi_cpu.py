"""The C ABI library loads and exports every symbol include/moe_verify.h
declares; host-side argument validation returns the documented codes before
anything reaches the GPU (CPU only, no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

import moe_speculative_decoding_router_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_verify.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libmoeverify.so is not built; run __graft_entry__.build()")
    return m.lib()


def test_exports_every_declared_symbol(lib):  # noqa: D103
    names = declared_functions()
    assert set(names) == set(m.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def layer(**kw):
    base = dict(H=512, I=256, E=32, k=4, wdtype=m.MOE_BF16, Wr=16, W_gu=16, W_d=16)
    base.update(kw)
    L = m._Layer()
    for k, v in base.items():
        setattr(L, k, v)
    return L


def ws_bytes(lib, L, T, bias=None):
    return lib.moe_verify_workspace_bytes(ctypes.byref(L), T, ctypes.byref(bias) if bias else None)


def test_workspace_bytes_and_shape_validation(lib):
    assert ws_bytes(lib, layer(), 5) > 0
    assert ws_bytes(lib, layer(), 64) > ws_bytes(lib, layer(), 5)
    for bad in (dict(k=0), dict(k=33, E=64), dict(k=40, E=32), dict(E=513), dict(H=0), dict(wdtype=7),
                dict(H=500), dict(H=544), dict(I=250), dict(wdtype=m.MOE_FP8_E4M3, H=512, I=192)):
        assert ws_bytes(lib, layer(**bad), 5) == 0, bad
    assert ws_bytes(lib, layer(), 0) == 0 and ws_bytes(lib, layer(), 65) == 0
    b = m._Bias(3, 0.5, 16)                       # cap < k
    assert ws_bytes(lib, layer(), 5, b) == 0 and b"cap" in lib.moe_last_error()
    b = m._Bias(8, 1.0, 16)                       # alpha outside [0, 1)
    assert ws_bytes(lib, layer(), 5, b) == 0 and b"alpha" in lib.moe_last_error()
    assert ws_bytes(lib, layer(), 5, m._Bias(8, 0.5, 16)) > 0


def test_verify_layer_rejects_before_launch(lib):
    L = layer()
    aux = m._Aux()
    rc = lib.moe_verify_layer(ctypes.byref(L), None, 5, None, 16, ctypes.byref(aux), 256, 1 << 30, None)
    assert rc == -1 and b"x and y" in lib.moe_last_error()
    need = ws_bytes(lib, L, 5)
    rc = lib.moe_verify_layer(ctypes.byref(L), 16, 5, None, 16, ctypes.byref(aux), 256, need - 1, None)
    assert rc == -3 and b"workspace" in lib.moe_last_error()
    rc = lib.moe_verify_layer(ctypes.byref(L), 16, 5, None, 16, ctypes.byref(aux), 255, need, None)
    assert rc == -1 and b"aligned" in lib.moe_last_error()
    Lf = layer(wdtype=m.MOE_FP8_E4M3, s_gu=None, s_d=None)
    rc = lib.moe_verify_layer(ctypes.byref(Lf), 16, 5, None, 16, ctypes.byref(aux), 256, 1 << 30, None)
    assert rc == -1 and b"s_gu" in lib.moe_last_error()
    Lx = layer(Wsh_gu=16)
    rc = lib.moe_verify_layer(ctypes.byref(Lx), 16, 5, None, 16, ctypes.byref(aux), 256, 1 << 30, None)
    assert rc == -1 and b"shared" in lib.moe_last_error()
    rc = lib.moe_verify_layer(ctypes.byref(layer(H=4004)), 16, 5, None, 16, ctypes.byref(aux), 256, 1 << 30, None)
    assert rc == -2


def test_union_stats_and_select_validation(lib):
    assert lib.union_stats(None, 1, 5, 8, 128, 16, 16, None) == -1
    assert lib.union_stats(16, 1, 0, 8, 128, 16, 16, None) == -1
    assert lib.union_stats(16, 1, 5, 8, 70000, 16, 16, None) == -1
    assert lib.union_stats(16, 0, 5, 8, 128, 16, 16, None) == 0          # nothing to do
    par = np.array([-1, -1, 0, 0, 1, 1], dtype=np.int32)
    bad = np.array([-1, 2, 0, 0, 1, 1], dtype=np.int32)                   # parent after child
    assert lib.select_drafts(bad.ctypes.data, 6, 16, 16, 4, 4, 1e-6, 1, 16, None) == -1
    assert b"BFS" in lib.moe_last_error()
    assert lib.select_drafts(par.ctypes.data, 6, 16, 16, 4, 7, 1e-6, 1, 16, None) == -1   # gamma > N
    assert lib.select_drafts(par.ctypes.data, 6, 16, 16, 4, 4, 0.0, 1, 16, None) == -1    # eps <= 0
    # a tree larger than the LDS stage is accepted (read from global memory);
    # nt = 0 keeps the check host-only
    assert lib.select_drafts(par.ctypes.data, 6, 16, 16, 4000, 4, 1e-6, 0, 16, None) == 0
    assert lib.select_drafts(par.ctypes.data, 6, 16, 16, 4097, 4, 1e-6, 0, 16, None) == -1  # W > 4096
    assert lib.select_drafts(par.ctypes.data, 6, 16, 16, 4, 0, 1e-6, 1, 16, None) == 0    # gamma 0
    assert lib.select_drafts(par.ctypes.data, 6, 16, 16, 4, 4, 1e-6, 0, 16, None) == 0    # no trees


def test_expand_validation(lib):
    par = np.array([-1, -1, 0, 0, 1, 1], dtype=np.int32)
    bad = np.array([-1, 2, 0, 0, 1, 1], dtype=np.int32)
    ok = lambda *a: lib.expand_drafts(*a)  # noqa: E731
    assert ok(None, 6, 16, 16, 4, 1.0, 1.0, None, 1, 16, 16, None) == -1               # parent NULL
    assert ok(bad.ctypes.data, 6, 16, 16, 4, 1.0, 1.0, None, 1, 16, 16, None) == -1    # BFS order
    assert b"BFS" in lib.moe_last_error()
    assert ok(par.ctypes.data, 6, 16, 16, 4, -1.0, 1.0, None, 1, 16, 16, None) == -1   # t_ar < 0
    assert ok(par.ctypes.data, 6, 16, 16, 4, 1.0, float("inf"), None, 1, 16, 16, None) == -1
    assert ok(par.ctypes.data, 6, 16, 16, 4000, 1.0, 1.0, None, 0, 16, 16, None) == 0   # beyond LDS: accepted
    assert ok(par.ctypes.data, 6, 16, 16, 4097, 1.0, 1.0, None, 0, 16, 16, None) == -1  # W > 4096
    assert ok(par.ctypes.data, 6, None, 16, 4, 1.0, 1.0, None, 1, 16, 16, None) == -1   # P NULL
    assert ok(par.ctypes.data, 6, None, None, 4, 1.0, 1.0, None, 0, None, None, None) == 0  # no trees
    big = np.full(1025, -1, dtype=np.int32)
    assert ok(big.ctypes.data, 1025, 16, 16, 1, 1.0, 1.0, None, 1, 16, 16, None) == -1  # N > 1024


def test_expert_bytes_matches_page_figures():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "page_figures.json")) as f:
        g = json.load(f)
    ds = g["deepseek_fp8_expert"]
    b = m.expert_bytes(ds["H"], ds["I"], "fp8")
    assert abs(b / 1e6 - ds["approx_MB"]) < 0.5          # "44 MB" per DeepSeek FP8 expert
    q = g["table2_qwen_delta"]
    delta_gb = q["experts_delta"] * q["n_layers"] * m.expert_bytes(q["H"], q["I"], "bf16") / 1e9
    assert abs(delta_gb - q["page_delta_GB"]) / q["page_delta_GB"] < q["rel_tol"]


def test_ragged_validation(lib):
    off = np.array([0, 2, 5], dtype=np.int32)
    assert lib.union_stats_segments(16, 1, 5, 4, 128, None, 2, 16, 16, None) == -1          # offsets NULL
    assert lib.union_stats_segments(16, 1, 6, 4, 128, off.ctypes.data, 2, 16, 16, None) == -1  # end != T
    bad = np.array([0, 3, 2, 5], dtype=np.int32)
    assert lib.union_stats_segments(16, 1, 5, 4, 128, bad.ctypes.data, 3, 16, 16, None) == -1  # decreasing
    assert lib.union_stats_segments(16, 0, 5, 4, 128, off.ctypes.data, 2, 16, 16, None) == 0   # nothing to do
    assert lib.gate_depths(16, 16, 0, 4, 8, 1.0, 1.0, 16, None) == -1       # S = 0
    assert lib.gate_depths(16, 16, 65, 4, 8, 1.0, 1.0, 16, None) == -1      # S > 64
    assert lib.gate_depths(16, 16, 4, 65, 8, 1.0, 1.0, 16, None) == -1      # Dmax > 64
    assert lib.gate_depths(16, 16, 4, 4, 1025, 1.0, 1.0, 16, None) == -1    # W > 1024
    assert lib.gate_depths(16, 16, 4, 4, 8, 0.0, 1.0, 16, None) == -1       # t_base <= 0
    assert lib.gate_depths(None, 16, 4, 4, 8, 1.0, 1.0, 16, None) == -1     # NULL


def test_stream_read_validation(lib):
    """moe_stream_read rejects bad arguments before any device work."""
    import ctypes
    buf = (ctypes.c_uint8 * 64)()
    out = (ctypes.c_uint32 * 1)()
    addr = (ctypes.addressof(buf) + 15) & ~15
    assert lib.moe_stream_read(None, 16, ctypes.addressof(out), None) == -1
    assert lib.moe_stream_read(addr, 16, None, None) == -1
    assert lib.moe_stream_read(addr, 0, ctypes.addressof(out), None) == -1
    assert lib.moe_stream_read(addr, 24, ctypes.addressof(out), None) == -1
    assert lib.moe_stream_read(addr + 4, 16, ctypes.addressof(out), None) == -1


def test_noalloc_rejects_calls_beyond_its_array(lib):
    # 513 slots x 4096 x 64 columns of hidden activations alone exceed the
    # 32 MiB array: refused before anything touches a device
    L = layer(H=512, I=4096, E=512, k=32)
    assert ws_bytes(lib, L, 64) > (32 << 20)
    rc = lib.moe_verify_layer_noalloc(ctypes.byref(L), 16, 64, None, 16, None, None)
    assert rc == -3 and b"no-allocation" in lib.moe_last_error()
    # invalid arguments keep their own codes
    assert lib.moe_verify_layer_noalloc(ctypes.byref(layer(k=0)), 16, 5, None, 16, None, None) == -1
    assert lib.moe_verify_layer_noalloc(None, 16, 5, None, 16, None, None) == -1
