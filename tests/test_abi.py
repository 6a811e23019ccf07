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
    """Prefill workspace: bf16 q/k/v, fp32 gates, the bf16 GEMM operand for loops 2..T, the projection's
    partial gate pre-activations where it forms them, and per chunk W [D x 64], M [64 x 64] (each as bf16
    hi and lo planes, 4 bytes per element) and gamma [64]; every region rounded up to 256 bytes."""
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
    # backward: the chunk matrices plus the chunk-start states and the state gradients at chunk ends
    B, L, H, D = 2, 130, 3, 128
    Nc = (L + 63) // 64
    chunks = up(B * H * Nc * D * 64 * 4) + up(B * H * Nc * 64 * 64 * 4) + up(B * H * Nc * 64 * 4)
    # fp32 T, P, A, M^T; fp64 log-cumsum; gamma, c; the reverse carry's W^T (hi, lo), K^T, Q^T (hi, lo) bf16 planes
    # [D][64] and M^T dO [64][D] fp32
    mats = B * H * Nc * (4 * 64 * 64 * 4 + 64 * 8 + 2 * 64 * 4 + 6 * D * 64 * 2 + 64 * D * 4)
    assert _ws_status(gl.make_desc(B, L, H, D, D), gl.GDN_OP_SCAN_BACKWARD) == (
        0, chunks + 2 * up(B * H * Nc * D * D * 4) + up(mats))
    st, _ = _ws_status(gl.make_desc(B, L, H, D, D, act=gl.GDN_F32), gl.GDN_OP_SCAN_BACKWARD)
    assert st == -3   # fp32 inputs with 128-wide heads
    # loop backward: the loop prefill's regions (q, k, v, alpha, beta, the bf16 operand; gate partials from 1024
    # tokens), the scan backward's, then the raw projections (and for bf16 their gradient as bf16 hi/lo planes)
    # [M][P] and their transpose [P][Mp] (Mp = M rounded up to 64), x^T [d][Mp] and W^T [d][P] in the activation
    # dtype, the scan gradients, two dh buffers, the weight-gradient accumulators [d][P] (bf16: one per k-range
    # split of x^T dY), the split-k partials of dY W (bf16, when split) and the rho partials (32-row blocks).
    # A product with `tiles` 384 x 256 tiles splits its k range s ways, s in 1..smax minimising
    # ceil(tiles s / 256) / s + cost (s - 1).
    def split(tiles, smax, cost):
        best, bc = 1, 1e30
        for sp in range(1, smax + 1):
            c = -(-tiles * sp // 256) / sp + cost * (sp - 1)
            if c < bc - 1e-9:
                best, bc = sp, c
        return best

    for act, eb in [(gl.GDN_BF16, 2), (gl.GDN_F32, 4)]:
        B, L, H, D = 2, 130, 3, (128 if act == gl.GDN_BF16 else 64)
        d, tok, Nc = H * D, B * L, (L + 63) // 64
        P = (H * 3 * D + 127) // 128 * 128 + 128
        Mp = (tok + 63) // 64 * 64
        chunks = up(B * H * Nc * D * 64 * 4) + up(B * H * Nc * 64 * 64 * 4) + up(B * H * Nc * 64 * 4)
        mats = B * H * Nc * (4 * 64 * 64 * 4 + 64 * 8 + 2 * 64 * 4 + 6 * D * 64 * 2 + 64 * D * 4)
        xb = up(tok * d * 2) if act == gl.GDN_BF16 else 0   # the bf16 loop operand
        exp = (3 * up(tok * H * D * eb) + 2 * up(tok * H * 4) + xb + chunks + 2 * up(B * H * Nc * D * D * 4) + up(mats)
               + up(tok * P * 4) + (up(tok * P * 4) if act == gl.GDN_BF16 else 0) + up(P * Mp * 4) + up(d * Mp * eb) + up(d * P * eb) + 3 * up(tok * H * D * 4)
               + 2 * up(tok * H * 4) + 2 * up(tok * d * 4))
        bf = act == gl.GDN_BF16
        dws = split(-(-d // 384) * -(-P // 256), 3, 0.05) if bf else 1
        dxs = split(-(-tok // 384) * -(-d // 256), 4, 0.025)
        assert dxs == 4 and dws == (3 if bf else 1)   # the small shape splits both products
        exp += up(d * P * 4 * dws) + (up(dxs * tok * d * 4) if bf and dxs > 1 else 0) + up(((tok + 31) // 32) * d * 4)
        assert _ws_status(gl.make_desc(B, L, H, D, D, act=act), gl.GDN_OP_LOOP_BACKWARD) == (0, exp)
    st, _ = _ws_status(gl.make_desc(B, L, H, 128, 128, act=gl.GDN_F32), gl.GDN_OP_LOOP_BACKWARD)
    assert st == -3


@pytest.mark.parametrize("op", [gl.GDN_OP_LOOP_PREFILL, gl.GDN_OP_LOOP_DECODE])
def test_workspace_regions(op):
    """The documented regions (q, k, v, alpha, beta) lie in order at the start of the looped calls' workspace,
    256-byte aligned, sized [B*L, H, D] in the activation dtype and [B*L, H] fp32, inside the workspace."""
    up = lambda x: (x + 255) // 256 * 256
    for B, L, H, D, act, eb in [(2, 130, 3, 128, gl.GDN_BF16, 2), (1, 1100, 16, 128, gl.GDN_BF16, 2),
                                (3, 77, 1, 64, gl.GDN_F32, 4)]:
        if op == gl.GDN_OP_LOOP_DECODE:
            L = 1
        desc = gl.make_desc(B, L, H, D, D, T=4, act=act)
        total = gl.gdn_workspace_bytes(desc, op)
        tok = B * L
        expect = [(0, tok * H * D * eb), (up(tok * H * D * eb), tok * H * D * eb),
                  (2 * up(tok * H * D * eb), tok * H * D * eb), (3 * up(tok * H * D * eb), tok * H * 4),
                  (3 * up(tok * H * D * eb) + up(tok * H * 4), tok * H * 4)]
        for reg, (off, n) in zip((gl.GDN_WS_Q, gl.GDN_WS_K, gl.GDN_WS_V, gl.GDN_WS_ALPHA, gl.GDN_WS_BETA), expect):
            assert gl.gdn_workspace_region(desc, op, reg) == (off, n)
            assert off + n <= total
    desc = gl.make_desc(1, 64 if op == gl.GDN_OP_LOOP_PREFILL else 1, 2, 128, 128)
    n, o = ctypes.c_size_t(), ctypes.c_size_t()
    lib = gl.load()
    assert lib.gdn_workspace_region(ctypes.byref(desc), op, 5, ctypes.byref(o), ctypes.byref(n)) == -3
    assert lib.gdn_workspace_region(ctypes.byref(desc), gl.GDN_OP_SCAN_PREFILL, 0, ctypes.byref(o),
                                    ctypes.byref(n)) == -3
    assert lib.gdn_workspace_region(ctypes.byref(desc), op, 0, None, ctypes.byref(n)) in (-1, -2)


def test_grid_limits_rejected_before_launch():
    """Shapes whose launch grids or 32-bit token counts would not hold are refused on the host: more than
    65535 sequences in a prefill call, or B*L of 2^31 tokens or more."""
    for op in (gl.GDN_OP_LOOP_PREFILL, gl.GDN_OP_SCAN_PREFILL):
        st, _ = _ws_status(gl.make_desc(65536, 1, 1, 64, 64), op)
        assert st == -2 and "65535" in gl.gdn_last_error()
        assert _ws_status(gl.make_desc(65535, 2, 1, 64, 64), op)[0] == 0
    st, _ = _ws_status(gl.make_desc(4, 1 << 29, 1, 64, 64))
    assert st == -2 and "2^31" in gl.gdn_last_error()
    # decode calls run one workgroup per (sequence, head): many sequences are fine
    assert _ws_status(gl.make_desc(100000, 1, 1, 64, 64), gl.GDN_OP_SCAN_DECODE)[0] == 0


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
    # loop backward: h_loops required for T > 1, dh0 may not alias dh, then the workspace size
    o = [ctypes.c_void_p(0x100000 + 0x1000 * i) for i in range(12)]
    st = lib.gdn_loop_backward(ctypes.byref(desc), o[0], o[1], o[2], None, o[3], o[4], *o[5:11], good, 1 << 40, None)
    assert st == -1 and "h_loops" in gl.gdn_last_error()
    st = lib.gdn_loop_backward(ctypes.byref(desc), o[0], o[1], o[2], o[11], o[3], o[3], *o[5:11], good, 1 << 40, None)
    assert st == -2 and "alias" in gl.gdn_last_error()
    st = lib.gdn_loop_backward(ctypes.byref(desc), o[0], o[1], o[2], o[11], o[3], o[4], *o[5:11], good, 16, None)
    assert st == -4 and "workspace" in gl.gdn_last_error()
    st = lib.gdn_loop_backward(ctypes.byref(gl.make_desc(1, 64, 2, 128, 128, act=gl.GDN_F32)), o[0], o[1], o[2],
                               o[11], o[3], o[4], *o[5:11], good, 1 << 40, None)
    assert st == -3


def test_binding_checks_tensor_sizes_on_host():
    """The Python binding refuses host tensors and wrong element counts before calling the library."""
    desc = gl.make_desc(1, 64, 2, 128, 128)
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(gl.GdnError):
        gl.gdn_scan_prefill(desc, q, q, q, torch.zeros(1, 64, 2), torch.zeros(1, 64, 2), None,
                            torch.zeros(1, 64, 2, 128), None, None)


def test_timer_validation(lib):
    h = ctypes.c_void_p()
    assert lib.gdn_timer_create(12, 4, ctypes.byref(h)) == -2
    assert lib.gdn_timer_create(4, 4, ctypes.byref(h)) == -2   # not a stage
    assert lib.gdn_timer_create(8, 4, ctypes.byref(h)) == -2   # not a stage
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


def test_block_sizes_and_rejections(lib):
    """Packed block bytes: the mixer's packed weights, Wg^T, Wo^T, W13, W2^T in the activation dtype and the two
    fp32 norm weights, each region rounded up to 256 bytes; ffn must be a positive multiple of 64."""
    up = lambda x: (x + 255) // 256 * 256
    for act, eb in [(gl.GDN_BF16, 2), (gl.GDN_F32, 4)]:
        H, D = 4, 64
        d = H * D
        desc = gl.make_desc(1, 8, H, D, D, act=act)
        P = (H * 3 * D + 127) // 128 * 128 + 128
        F = 704
        exp = up(P * d * eb) + 2 * up(d * d * eb) + up(2 * F * d * eb) + up(d * F * eb) + 2 * up(d * 4)
        n = ctypes.c_size_t()
        assert lib.gdn_block_packed_bytes(ctypes.byref(desc), F, ctypes.byref(n)) == 0 and n.value == exp
        assert lib.gdn_block_packed_bytes(ctypes.byref(desc), 100, ctypes.byref(n)) == -2
        assert lib.gdn_block_workspace_bytes(ctypes.byref(desc), 0, ctypes.byref(n)) == -2
    desc = gl.make_desc(1, 64, 2, 128, 128)
    good = ctypes.c_void_p(0x100000)
    assert lib.gdn_block_forward(ctypes.byref(desc), 256, good, good, good, good, 1 << 40, None) == -2   # aliasing
    assert lib.gdn_block_loop_prefill(ctypes.byref(desc), 256, 0, good, good, good, ctypes.c_void_p(0x200000),
                                      good, 1 << 40, None) == -2   # no layers
    st = lib.gdn_block_forward(ctypes.byref(desc), 256, good, good, ctypes.c_void_p(0x200000), good, 16, None)
    assert st == -4 and "workspace" in gl.gdn_last_error()


def test_loop_prefill_pieces_setting():
    """The process-wide piece setting of gdn_loop_prefill: -1 loop by loop, 0 automatic (two pieces per sequence
    where L >= 16384 and the whole call's 16-column carry would fill at most half of the 256 CUs), > 0 pieces of
    that many tokens rounded up to a multiple of 256 and at least 1024; a single piece of a single sequence runs
    loop by loop; shapes the pieces do not apply to (fp32, T = 1, 2H > 32, sequences too short) always run loop
    by loop."""
    pieces = lambda *a, **k: gl.gdn_loop_prefill_pieces(gl.make_desc(*a, **k))
    lib = gl.load()
    assert lib.gdn_loop_prefill_set_pieces(-2) == -2
    try:
        gl.gdn_loop_prefill_set_pieces(0)
        assert pieces(1, 32768, 16, 128, 128) == 16384    # 128 carry workgroups: two pieces
        assert pieces(1, 16384, 16, 128, 128) == 8192
        assert pieces(1, 20000, 16, 128, 128) == 10240    # half, rounded up to 256
        assert pieces(1, 16383, 16, 128, 128) == 0        # shorter than 16384
        assert pieces(1, 4096, 16, 128, 128) == 0
        assert pieces(4, 32768, 16, 128, 128) == 0        # 512 carry workgroups: loop by loop
        assert pieces(1, 32768, 16, 128, 128, T=1) == 0
        assert pieces(1, 32768, 16, 128, 128, act=gl.GDN_F32) == 0
        assert pieces(1, 32768, 17, 128, 128) == 0        # 2H > 32: gates not from the GEMM's partials
        assert pieces(1, 2048, 16, 128, 128) == 0         # one piece
        gl.gdn_loop_prefill_set_pieces(1000)
        assert pieces(1, 4096, 16, 128, 128) == 1024
        assert pieces(4, 8192, 16, 128, 128) == 1024
        assert pieces(2, 1100, 16, 128, 128) == 1024      # one piece per sequence (the 76 left join it)
        assert pieces(1, 1100, 16, 128, 128) == 0
        gl.gdn_loop_prefill_set_pieces(5000)
        assert pieces(1, 4096, 16, 128, 128) == 0         # longer than the sequence
        assert pieces(3, 4096, 16, 128, 128) == 4096
        gl.gdn_loop_prefill_set_pieces(-1)
        assert pieces(1, 32768, 16, 128, 128) == 0
    finally:
        gl.gdn_loop_prefill_set_pieces(0)


def test_loop_prefill_pieces_workspace():
    """Shapes the pieces apply to add one state per (loop, sequence, head) [T][B][H][dk][dv] fp32 at the end of
    the loop prefill's workspace, whatever the setting; the halting call's workspace does not have it."""
    up = lambda x: (x + 255) // 256 * 256
    for B, L in [(1, 2048), (2, 1024), (1, 4096)]:
        H, D, T = 16, 128, 4
        tok, Nc, P = B * L, (L + 63) // 64, (H * D + 127) // 128
        chunks = up(B * H * Nc * D * 64 * 4) + up(B * H * Nc * 64 * 64 * 4) + up(B * H * Nc * 64 * 4)
        base = 3 * up(tok * H * D * 2) + 2 * up(tok * H * 4) + up(tok * H * D * 2) + up(P * 2 * H * tok * 4) + chunks
        desc = gl.make_desc(B, L, H, D, D, T=T)
        assert _ws_status(desc) == (0, base + up(T * B * H * D * D * 4))
        act = base + 3 * up(tok * 4) + up(4)
        assert _ws_status(desc, gl.GDN_OP_LOOP_PREFILL_ACT) == (0, act)
    # one sequence of fewer than 2048 tokens: no pieces, no state buffer
    B, L, H, D, T = 1, 2047, 16, 128, 4
    tok, Nc, P = B * L, (L + 63) // 64, (H * D + 127) // 128
    chunks = up(B * H * Nc * D * 64 * 4) + up(B * H * Nc * 64 * 64 * 4) + up(B * H * Nc * 64 * 4)
    base = 3 * up(tok * H * D * 2) + 2 * up(tok * H * 4) + up(tok * H * D * 2) + up(P * 2 * H * tok * 4) + chunks
    assert _ws_status(gl.make_desc(B, L, H, D, D, T=T)) == (0, base)


def test_decode_workspace_split_projection():
    """A bf16 loop decode of at most 64 sequences splits its projection over S channel ranges (S = 4, 2 or 1:
    the largest that divides the 64-channel blocks) and keeps the fp32 partial products [S][N][packed rows] at
    the end of its workspace; fp32 workloads and more than 64 sequences do not."""
    up = lambda x: (x + 255) // 256 * 256

    def base(N, H, D, eb):
        return 3 * up(N * H * D * eb) + 2 * up(N * H * 4) + (up(N * H * D * 2) if eb == 2 else 0)

    for N, H, D, S in [(64, 16, 128, 4), (1, 1, 128, 2), (7, 20, 64, 4), (3, 3, 64, 1)]:
        P = (H * 3 * D + 127) // 128 * 128 + 128
        exp = base(N, H, D, 2) + (up(S * N * P * 4) if S > 1 else 0)
        assert _ws_status(gl.make_desc(N, 1, H, D, D), gl.GDN_OP_LOOP_DECODE) == (0, exp)
    assert _ws_status(gl.make_desc(65, 1, 16, 128, 128), gl.GDN_OP_LOOP_DECODE) == (0, base(65, 16, 128, 2))
    assert _ws_status(gl.make_desc(8, 1, 2, 64, 64, act=gl.GDN_F32), gl.GDN_OP_LOOP_DECODE) == (0, base(8, 2, 64, 4))
    # the no-allocation decode still takes 64 sequences of width 2048
    assert _ws_status(gl.make_desc(64, 1, 16, 128, 128), gl.GDN_OP_LOOP_DECODE)[1] <= 8 << 20   # its 8 MiB scratch


def test_new_workspace_minimums_rejected_before_launch(lib):
    """On the host, before anything is enqueued: a loop decode workspace one byte short of the size without the
    projection-partials region (the size at which the projection runs unsplit) is refused, as is a pipelined-shape
    loop prefill workspace one byte short of the size with the pieces' state region."""
    up = lambda n: (n + 255) // 256 * 256
    o = [ctypes.c_void_p(0x100000 + 0x1000 * i) for i in range(8)]
    desc = gl.make_desc(64, 1, 16, 128, 128)
    full = _ws_status(desc, gl.GDN_OP_LOOP_DECODE)[1]
    unsplit = full - up(4 * 64 * (16 * 3 * 128 + 128) * 4)
    st = lib.gdn_loop_decode(ctypes.byref(desc), o[0], o[1], o[2], o[3], o[4], o[5], unsplit - 1, None)
    assert st == -4 and f"{unsplit} bytes" in gl.gdn_last_error()
    desc = gl.make_desc(1, 32768, 16, 128, 128)
    full = _ws_status(desc)[1]
    st = lib.gdn_loop_prefill(ctypes.byref(desc), o[0], o[1], o[2], o[3], None, None, o[5], full - 1, None)
    assert st == -4 and f"{full} bytes" in gl.gdn_last_error()
