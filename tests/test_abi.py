"""CPU tests of the C ABI: the library loads, exports every symbol the header declares, and validates
arguments on the host (returning its status codes) before anything is enqueued.

Calls that pass made-up device addresses are only run where no GPU is visible, so a validation bug could
never turn into a launch on real hardware.
"""
import ctypes
import os
import re

import pytest
import torch

import looped_linear_attention_amd as gl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdnloop.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="uses fake device addresses; CPU-only check")


@pytest.fixture(scope="module")
def lib():
    return gl.load()


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


def test_header_and_exports_agree(lib):
    declared = _header_functions()
    assert declared == sorted(gl.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_exported_symbols_in_dynamic_table():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", gl.lib_path()], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in gl.EXPORTED:
        assert name in syms, name


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = gl.gdn_status_string(code)
        assert s.startswith("GDN_")
    assert "unknown" in gl.gdn_status_string(-99)
    assert "gfx950" in gl.gdn_version()


def _ws_status(desc, op=gl.GDN_OP_LOOP_PREFILL):
    n = ctypes.c_size_t()
    return gl.load().gdn_workspace_bytes(ctypes.byref(desc), op, ctypes.byref(n)), n.value


@pytest.mark.parametrize("field,value,code", [
    ("chunk", 32, -3), ("dk", 96, -3), ("dv", 64, -3), ("d", 1000, -2), ("B", 0, -2), ("L", 0, -2),
    ("T", 0, -2), ("H", 0, -2), ("act", 7, -3), ("alpha_lo", 1.01, -2), ("alpha_lo", -0.1, -2),
    ("norm_eps", 0.0, -2), ("norm_eps", float("nan"), -2),
])
def test_descriptor_validation(field, value, code):
    desc = gl.make_desc(1, 128, 16, 128, 128)
    setattr(desc, field, value)
    st, _ = _ws_status(desc)
    assert st == code, gl.gdn_last_error()


@pytest.mark.parametrize("alpha_lo", [0.0, 0.9, 1.0])
def test_alpha_lo_range_accepted(alpha_lo):
    """alpha_lo = 1 is the delta rule without decay (alpha = 1 for every token)."""
    desc = gl.make_desc(1, 128, 16, 128, 128, alpha_lo=alpha_lo)
    assert _ws_status(desc)[0] == 0, gl.gdn_last_error()


def test_too_many_heads():
    desc = gl.make_desc(1, 64, 65, 64, 64)
    assert _ws_status(desc)[0] == -3


def test_decode_needs_single_token():
    desc = gl.make_desc(4, 2, 2, 128, 128)
    assert _ws_status(desc, gl.GDN_OP_LOOP_DECODE)[0] == -2
    assert _ws_status(desc, gl.GDN_OP_SCAN_DECODE)[0] == -2
    assert _ws_status(desc, 99)[0] == -3


def test_workspace_sizes():
    """Prefill workspace: bf16 q/k/v, fp32 gates, per-chunk W [D x 64], M [64 x 64], gamma [64], the chunk-start
    state [D x D] and E [64 x D] (both as bf16 hi/lo pairs, 4 bytes per element), and the bf16 GEMM operand
    for loops 2..T; every region rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256
    B, L, H, D, T = 2, 130, 3, 128, 4
    desc = gl.make_desc(B, L, H, D, D, T=T)
    st, n = _ws_status(desc)
    assert st == 0
    tok, Nc = B * L, (L + 63) // 64
    chunks = up(B * H * Nc * D * 64 * 4) + up(B * H * Nc * 64 * 64 * 4) + up(B * H * Nc * 64 * 4)
    exp = 3 * up(tok * H * D * 2) + 2 * up(tok * H * 4) + up(tok * H * D * 2) + chunks
    assert n == exp
    st, n = _ws_status(desc, gl.GDN_OP_SCAN_PREFILL)
    assert st == 0 and n == chunks
    # bf16 loop prefill of >= 1024 tokens with 2H <= 32: the projection GEMM leaves ceil(d / 128) fp32 partial
    # gate pre-activations [P][2H][tokens] in the workspace
    B, L, H, D = 1, 1100, 3, 64
    desc = gl.make_desc(B, L, H, D, D, T=T)
    tok, Nc, P = B * L, (L + 63) // 64, (H * D + 127) // 128
    chunks = up(B * H * Nc * D * 64 * 4) + up(B * H * Nc * 64 * 64 * 4) + up(B * H * Nc * 64 * 4)
    exp = 3 * up(tok * H * D * 2) + 2 * up(tok * H * 4) + up(tok * H * D * 2) + up(P * 2 * H * tok * 4) + chunks
    assert _ws_status(desc) == (0, exp)
    # ... but not for 2H > 32, nor for the fp32 path
    for H, act, eb in [(17, gl.GDN_BF16, 2), (3, gl.GDN_F32, 4)]:
        desc = gl.make_desc(B, L, H, D, D, T=T, act=act)
        chunks = up(B * H * Nc * D * 64 * 4) + up(B * H * Nc * 64 * 64 * 4) + up(B * H * Nc * 64 * 4)
        exp = 3 * up(tok * H * D * eb) + 2 * up(tok * H * 4) + (up(tok * H * D * 2) if eb == 2 else 0) + chunks
        assert _ws_status(desc) == (0, exp)
    st, n = _ws_status(gl.make_desc(64, 1, 16, 128, 128), gl.GDN_OP_SCAN_DECODE)
    assert st == 0 and n == 0


def test_packed_weight_bytes():
    n = ctypes.c_size_t()
    for H, D, act, rows in [(16, 128, gl.GDN_BF16, 16 * 384 + 128), (1, 64, gl.GDN_F32, 256 + 128),
                            (3, 64, gl.GDN_BF16, 640 + 128)]:
        desc = gl.make_desc(1, 8, H, D, D, act=act)
        assert gl.load().gdn_weights_packed_bytes(ctypes.byref(desc), ctypes.byref(n)) == 0
        assert n.value == rows * H * D * (4 if act == gl.GDN_F32 else 2)


def test_null_pointers_rejected_before_launch(lib):
    desc = gl.make_desc(1, 64, 2, 128, 128)
    P = ctypes.c_void_p
    st = lib.gdn_scan_prefill(ctypes.byref(desc), None, None, None, None, None, None, None, None, None, 0, None)
    assert st == -1 and "q" in gl.gdn_last_error()
    st = lib.gdn_loop_prefill(None, None, None, None, None, None, None, None, 0, None)
    assert st == -1
    st = lib.gdn_scan_decode(ctypes.byref(gl.make_desc(1, 1, 2, 128, 128)), None, None, None, None, None,
                             None, None, None)
    assert st == -1


@no_gpu
def test_alignment_and_workspace_rejected_before_launch(lib):
    desc = gl.make_desc(1, 64, 2, 128, 128)
    good = ctypes.c_void_p(0x100000)
    bad = ctypes.c_void_p(0x100004)
    args = [good] * 5
    st = lib.gdn_scan_prefill(ctypes.byref(desc), bad, *args[1:], None, good, None, good, 16, None)
    assert st == -6
    st = lib.gdn_scan_prefill(ctypes.byref(desc), *args, None, good, None, good, 16, None)
    assert st == -4 and "workspace" in gl.gdn_last_error()
    st = lib.gdn_scan_prefill(ctypes.byref(desc), *args, good, good, good, None, 1 << 30, None)
    assert st == -2  # s_final aliases s_init
    st = lib.gdn_loop_prefill(ctypes.byref(desc), good, good, good, good, None, None, None, 0, None)
    assert st == -2  # h_out aliases h0


def test_binding_checks_tensor_sizes_on_host():
    """The Python binding refuses host tensors and wrong element counts before calling the library."""
    desc = gl.make_desc(1, 64, 2, 128, 128)
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(gl.GdnError):
        gl.gdn_scan_prefill(desc, q, q, q, torch.zeros(1, 64, 2), torch.zeros(1, 64, 2), None,
                            torch.zeros(1, 64, 2, 128), None, None)


def test_timer_validation(lib):
    h = ctypes.c_void_p()
    assert lib.gdn_timer_create(9, 4, ctypes.byref(h)) == -2
    assert lib.gdn_timer_create(0, 0, ctypes.byref(h)) == -2
    assert lib.gdn_timer_create(0, 4, None) == -1
    assert lib.gdn_timer_attach(None) == -1
    assert lib.gdn_timer_detach() == 0
    assert lib.gdn_timer_destroy(None) == 0
    n, ms = ctypes.c_int(), ctypes.c_double()
    assert lib.gdn_timer_read(None, ctypes.byref(n), ctypes.byref(ms)) == -1
    assert lib.gdn_timer_set_stride(None, 2) == -1


@no_gpu
def test_timer_without_device_reports_hip_error():
    with pytest.raises(gl.GdnError, match="GDN_ERR_HIP"):
        gl.gdn_timer_create(gl.GDN_STAGE_PROJECT, 4)


@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "8"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """bench.py measures one GPU: a request for more exits with status 2 and says so, before it touches a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
