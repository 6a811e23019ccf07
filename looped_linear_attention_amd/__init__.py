"""Python binding of libgdnloop: the looped gated-delta-rule (GDN) mixer on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgdnloop.so`` (built by ``looped_linear_attention_amd.build``).
PyTorch supplies device memory and the stream.  Functions carry the names of
the C entry points declared in ``include/gdnloop.h`` and take torch tensors in
place of pointers; each tensor's dtype, device, contiguity and element count
are checked against the descriptor on the host before the call, so a
mismatched buffer raises instead of reaching a kernel.

The library fails loudly: importing works without a GPU, but any entry point
raises ``GdnError`` if the shared library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "GDN_F32", "GDN_BF16", "GDN_OP_LOOP_PREFILL", "GDN_OP_LOOP_DECODE", "GDN_OP_SCAN_PREFILL", "GDN_OP_SCAN_DECODE",
    "GDN_OP_PROJECT", "GDN_OP_SCAN_BACKWARD", "GDN_OP_LOOP_PREFILL_ACT", "GDN_OP_LOOP_BACKWARD",
    "GDN_STAGE_PROJECT", "GDN_STAGE_SCAN_PREP", "GDN_STAGE_SCAN_CARRY", "GDN_STAGE_DECODE", "GDN_STAGE_GATES",
    "GDN_STAGE_BWD_CARRY", "GDN_STAGE_BWD_CHUNK", "GDN_STAGE_BWD_GEMM", "GDN_STAGE_BWD_OPS",
    "GDN_STAGE_BLOCK_GEMM", "GDN_WS_Q", "GDN_WS_K", "GDN_WS_V", "GDN_WS_ALPHA", "GDN_WS_BETA", "GDN_BWS_X1",
    "GDN_BWS_O", "GDN_BWS_Z", "GDN_BWS_H1", "GDN_BWS_X2", "GDN_BWS_U", "GdnError", "gdn_desc", "make_desc",
    "lib_path", "load", "EXPORTED", "workspace", "workspace_view", "block_workspace", "block_workspace_view",
    "gdn_weights_packed_bytes", "gdn_weights_pack", "gdn_workspace_bytes", "gdn_workspace_region", "gdn_project",
    "gdn_scan_prefill", "gdn_scan_backward", "gdn_scan_decode", "gdn_loop_prefill", "gdn_loop_prefill_act",
    "gdn_loop_prefill_set_pieces", "gdn_loop_prefill_pieces",
    "gdn_loop_decode", "gdn_loop_decode_noalloc", "gdn_loop_backward", "gdn_block_packed_bytes", "gdn_block_pack",
    "gdn_block_workspace_bytes", "gdn_block_workspace_region", "gdn_block_forward", "gdn_block_loop_prefill",
    "gdn_status_string", "gdn_last_error", "gdn_version", "gdn_timer_create", "gdn_timer_set_stride",
    "gdn_timer_attach", "gdn_timer_detach", "gdn_timer_reset", "gdn_timer_read", "gdn_timer_destroy",
]

GDN_F32, GDN_BF16 = 0, 1
(GDN_OP_LOOP_PREFILL, GDN_OP_LOOP_DECODE, GDN_OP_SCAN_PREFILL, GDN_OP_SCAN_DECODE, GDN_OP_PROJECT, GDN_OP_SCAN_BACKWARD,
 GDN_OP_LOOP_PREFILL_ACT, GDN_OP_LOOP_BACKWARD) = range(8)
GDN_STAGE_PROJECT, GDN_STAGE_SCAN_PREP, GDN_STAGE_SCAN_CARRY, GDN_STAGE_DECODE, GDN_STAGE_GATES = 0, 1, 2, 3, 5
GDN_STAGE_BWD_CARRY, GDN_STAGE_BWD_CHUNK, GDN_STAGE_BWD_GEMM, GDN_STAGE_BWD_OPS = 6, 7, 9, 10
GDN_STAGE_BLOCK_GEMM = 11
GDN_WS_Q, GDN_WS_K, GDN_WS_V, GDN_WS_ALPHA, GDN_WS_BETA = range(5)
GDN_BWS_X1, GDN_BWS_O, GDN_BWS_Z, GDN_BWS_H1, GDN_BWS_X2, GDN_BWS_U = range(16, 22)

# Every symbol the header declares (checked by the CPU test suite).
EXPORTED = [
    "gdn_weights_packed_bytes", "gdn_weights_pack", "gdn_workspace_bytes", "gdn_workspace_region", "gdn_project",
    "gdn_scan_prefill", "gdn_scan_backward", "gdn_scan_decode", "gdn_loop_prefill", "gdn_loop_prefill_act",
    "gdn_loop_prefill_set_pieces", "gdn_loop_prefill_pieces",
    "gdn_loop_decode", "gdn_loop_decode_noalloc", "gdn_loop_backward", "gdn_block_packed_bytes", "gdn_block_pack",
    "gdn_block_workspace_bytes", "gdn_block_workspace_region", "gdn_block_forward", "gdn_block_loop_prefill",
    "gdn_status_string", "gdn_last_error", "gdn_version", "gdn_timer_create", "gdn_timer_set_stride",
    "gdn_timer_attach", "gdn_timer_detach", "gdn_timer_reset", "gdn_timer_read", "gdn_timer_destroy",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdnloop.so")
_lib = None


class GdnError(RuntimeError):
    pass


class gdn_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("T", ctypes.c_int32), ("chunk", ctypes.c_int32), ("act", ctypes.c_int32),
                ("alpha_lo", ctypes.c_float), ("norm_eps", ctypes.c_float)]

    @property
    def act_dtype(self) -> torch.dtype:
        return torch.float32 if self.act == GDN_F32 else torch.bfloat16


def make_desc(B: int, L: int, H: int, dk: int, dv: int, T: int = 4, act=GDN_BF16,
              alpha_lo: float = 0.0, norm_eps: float = 1e-6, chunk: int = 64) -> gdn_desc:
    if isinstance(act, str):
        act = GDN_F32 if act == "f32" else GDN_BF16
    return gdn_desc(B, L, H, dk, dv, H * dv, T, chunk, act, alpha_lo, norm_eps)


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdnloop.so (raises GdnError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise GdnError(f"{_LIB_PATH} is missing: run `python -m looped_linear_attention_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, D, S, I = ctypes.c_void_p, ctypes.POINTER(gdn_desc), ctypes.c_size_t, ctypes.c_int
    sig = {
        "gdn_weights_packed_bytes": [D, ctypes.POINTER(S)],
        "gdn_weights_pack": [D, P, P, P, P, P, P, P],
        "gdn_workspace_bytes": [D, I, ctypes.POINTER(S)],
        "gdn_workspace_region": [D, I, I, ctypes.POINTER(S), ctypes.POINTER(S)],
        "gdn_project": [D, P, P, P, P, P, P, P, P],
        "gdn_scan_prefill": [D, P, P, P, P, P, P, P, P, P, S, P],
        "gdn_scan_decode": [D, P, P, P, P, P, P, P, P],
        "gdn_scan_backward": [D] + [P] * 15 + [S, P],
        "gdn_loop_prefill": [D, P, P, P, P, P, P, P, S, P],
        "gdn_loop_decode": [D, P, P, P, P, P, P, S, P],
        "gdn_loop_prefill_act": [D, P, P, P, P, ctypes.c_float, ctypes.c_float, P, P, P, P, S, P],
        "gdn_loop_prefill_set_pieces": [I],
        "gdn_loop_prefill_pieces": [D, ctypes.POINTER(I)],
        "gdn_loop_decode_noalloc": [D, P, P, P, P, P, P],
        "gdn_loop_backward": [D] + [P] * 13 + [S, P],
        "gdn_block_packed_bytes": [D, I, ctypes.POINTER(S)],
        "gdn_block_pack": [D, I] + [P] * 14,
        "gdn_block_workspace_bytes": [D, I, ctypes.POINTER(S)],
        "gdn_block_workspace_region": [D, I, I, ctypes.POINTER(S), ctypes.POINTER(S)],
        "gdn_block_forward": [D, I, P, P, P, P, S, P],
        "gdn_block_loop_prefill": [D, I, I, P, P, P, P, P, S, P],
        "gdn_timer_create": [I, I, ctypes.POINTER(P)],
        "gdn_timer_set_stride": [P, I],
        "gdn_timer_attach": [P],
        "gdn_timer_detach": [],
        "gdn_timer_reset": [P],
        "gdn_timer_read": [P, ctypes.POINTER(I), ctypes.POINTER(ctypes.c_double)],
        "gdn_timer_destroy": [P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load()
        raise GdnError(f"{lib.gdn_status_string(status).decode()} -- {lib.gdn_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype], numel: int,
         optional: bool = False):
    if t is None:
        if optional:
            return None
        raise GdnError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise GdnError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise GdnError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise GdnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GdnError(f"{name} must be {dtype} (got {t.dtype})")
    if t.numel() != numel:
        raise GdnError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise GdnError("ws must be a contiguous device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def gdn_status_string(status: int) -> str:
    return load().gdn_status_string(status).decode()


def gdn_last_error() -> str:
    return load().gdn_last_error().decode()


def gdn_version() -> str:
    return load().gdn_version().decode()


def gdn_weights_packed_bytes(desc: gdn_desc) -> int:
    n = ctypes.c_size_t()
    _check(load().gdn_weights_packed_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def gdn_workspace_bytes(desc: gdn_desc, op: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gdn_workspace_bytes(ctypes.byref(desc), op, ctypes.byref(n)))
    return n.value


def workspace(desc: gdn_desc, op: int, device="cuda") -> torch.Tensor:
    """Allocate the device workspace `op` needs (torch owns the memory)."""
    return torch.empty(max(gdn_workspace_bytes(desc, op), 256), dtype=torch.uint8, device=device)


def gdn_workspace_region(desc: gdn_desc, op: int, region: int):
    """(byte offset, bytes) of a documented region of a looped call's workspace."""
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().gdn_workspace_region(ctypes.byref(desc), op, region, ctypes.byref(off), ctypes.byref(n)))
    return off.value, n.value


def workspace_view(ws: torch.Tensor, desc: gdn_desc, op: int, region: int) -> torch.Tensor:
    """A typed view of a workspace region: q/k/v as [B*L, H, D] in the activation dtype, the gates as
    [B*L, H] fp32 (the view shares the workspace's memory)."""
    off, n = gdn_workspace_region(desc, op, region)
    if ws.numel() * ws.element_size() < off + n:
        raise GdnError("workspace is smaller than the region")
    raw = ws.view(torch.uint8)[off:off + n]
    tokens = desc.B * desc.L
    if region in (GDN_WS_ALPHA, GDN_WS_BETA):
        return raw.view(torch.float32).view(tokens, desc.H)
    return raw.view(desc.act_dtype).view(tokens, desc.H, desc.dk)


def gdn_block_packed_bytes(desc: gdn_desc, ffn: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gdn_block_packed_bytes(ctypes.byref(desc), ffn, ctypes.byref(n)))
    return n.value


def gdn_block_workspace_bytes(desc: gdn_desc, ffn: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gdn_block_workspace_bytes(ctypes.byref(desc), ffn, ctypes.byref(n)))
    return n.value


def block_workspace(desc: gdn_desc, ffn: int, device="cuda") -> torch.Tensor:
    """Allocate the device workspace of the LT2 block calls (torch owns the memory)."""
    return torch.empty(max(gdn_block_workspace_bytes(desc, ffn), 256), dtype=torch.uint8, device=device)


def gdn_block_workspace_region(desc: gdn_desc, ffn: int, region: int):
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().gdn_block_workspace_region(ctypes.byref(desc), ffn, region, ctypes.byref(off), ctypes.byref(n)))
    return off.value, n.value


def block_workspace_view(ws: torch.Tensor, desc: gdn_desc, ffn: int, region: int) -> torch.Tensor:
    """A typed view of a block workspace region ([B*L, width] in its dtype; q/k/v [B*L, H, D])."""
    off, n = gdn_block_workspace_region(desc, ffn, region)
    if ws.numel() * ws.element_size() < off + n:
        raise GdnError("workspace is smaller than the region")
    raw = ws.view(torch.uint8)[off:off + n]
    tokens = desc.B * desc.L
    if region in (GDN_WS_ALPHA, GDN_WS_BETA):
        return raw.view(torch.float32).view(tokens, desc.H)
    if region in (GDN_WS_Q, GDN_WS_K, GDN_WS_V):
        return raw.view(desc.act_dtype).view(tokens, desc.H, desc.dk)
    dt = torch.float32 if region in (GDN_BWS_O, GDN_BWS_H1) else desc.act_dtype
    return raw.view(dt).view(tokens, -1)


def gdn_block_pack(desc, ffn, g1, Wq, Wk, Wv, wa, wb, Wg, Wo, g2, W1, W3, W2, Wblock, stream=None):
    a, d, H, dk, dv, f = desc.act_dtype, desc.d, desc.H, desc.dk, desc.dv, torch.float32
    n = gdn_block_packed_bytes(desc, ffn)
    if Wblock.numel() * Wblock.element_size() != n or Wblock.device.type != "cuda":
        raise GdnError(f"Wblock must be a device buffer of {n} bytes")
    _check(load().gdn_block_pack(
        ctypes.byref(desc), ffn, _ptr(g1, "g1", f, d), _ptr(Wq, "Wq", a, d * H * dk), _ptr(Wk, "Wk", a, d * H * dk),
        _ptr(Wv, "Wv", a, d * H * dv), _ptr(wa, "wa", a, d * H), _ptr(wb, "wb", a, d * H),
        _ptr(Wg, "Wg", a, d * H * dv), _ptr(Wo, "Wo", a, H * dv * d), _ptr(g2, "g2", f, d),
        _ptr(W1, "W1", a, d * ffn), _ptr(W3, "W3", a, d * ffn), _ptr(W2, "W2", a, ffn * d),
        ctypes.c_void_p(Wblock.data_ptr()), _stream(stream)))


def gdn_block_forward(desc, ffn, h, Wblock, out, ws, stream=None):
    BL, d = desc.B * desc.L, desc.d
    wp, wn = _ws(ws)
    _check(load().gdn_block_forward(
        ctypes.byref(desc), ffn, _ptr(h, "h", torch.float32, BL * d), ctypes.c_void_p(Wblock.data_ptr()),
        _ptr(out, "out", torch.float32, BL * d), wp, wn, _stream(stream)))


def gdn_block_loop_prefill(desc, ffn, layers, h0, Wblocks, rho, h_out, ws, stream=None):
    BL, d, T = desc.B * desc.L, desc.d, desc.T
    n = gdn_block_packed_bytes(desc, ffn) * layers
    if Wblocks.numel() * Wblocks.element_size() != n or Wblocks.device.type != "cuda":
        raise GdnError(f"Wblocks must be a device buffer of {n} bytes ({layers} packed blocks)")
    wp, wn = _ws(ws)
    _check(load().gdn_block_loop_prefill(
        ctypes.byref(desc), ffn, layers, _ptr(h0, "h0", desc.act_dtype, BL * d), ctypes.c_void_p(Wblocks.data_ptr()),
        _ptr(rho, "rho", torch.float32, T * d), _ptr(h_out, "h_out", torch.float32, BL * d), wp, wn,
        _stream(stream)))


def gdn_weights_pack(desc, Wq, Wk, Wv, wa, wb, Wpack, stream=None):
    a, d, H, dk, dv = desc.act_dtype, desc.d, desc.H, desc.dk, desc.dv
    pb = gdn_weights_packed_bytes(desc)
    _check(load().gdn_weights_pack(
        ctypes.byref(desc), _ptr(Wq, "Wq", a, d * H * dk), _ptr(Wk, "Wk", a, d * H * dk),
        _ptr(Wv, "Wv", a, d * H * dv), _ptr(wa, "wa", a, d * H), _ptr(wb, "wb", a, d * H),
        _ptr(Wpack, "Wpack", a, pb // (4 if desc.act == GDN_F32 else 2)), _stream(stream)))


def gdn_project(desc, x, Wpack, q, k, v, alpha, beta, stream=None):
    a, M, H, D = desc.act_dtype, desc.B * desc.L, desc.H, desc.dk
    pb = gdn_weights_packed_bytes(desc)
    _check(load().gdn_project(
        ctypes.byref(desc), _ptr(x, "x", a, M * desc.d),
        _ptr(Wpack, "Wpack", a, pb // (4 if desc.act == GDN_F32 else 2)),
        _ptr(q, "q", a, M * H * D), _ptr(k, "k", a, M * H * D), _ptr(v, "v", a, M * H * D),
        _ptr(alpha, "alpha", torch.float32, M * H), _ptr(beta, "beta", torch.float32, M * H),
        _stream(stream)))


def gdn_scan_prefill(desc, q, k, v, alpha, beta, s_init, o, s_final, ws, stream=None):
    a, BL, H, D = desc.act_dtype, desc.B * desc.L, desc.H, desc.dk
    st = desc.B * H * D * D
    wp, wn = _ws(ws)
    _check(load().gdn_scan_prefill(
        ctypes.byref(desc), _ptr(q, "q", a, BL * H * D), _ptr(k, "k", a, BL * H * D),
        _ptr(v, "v", a, BL * H * D), _ptr(alpha, "alpha", torch.float32, BL * H),
        _ptr(beta, "beta", torch.float32, BL * H),
        _ptr(s_init, "s_init", torch.float32, st, optional=True),
        _ptr(o, "o", torch.float32, BL * H * D),
        _ptr(s_final, "s_final", torch.float32, st, optional=True), wp, wn, _stream(stream)))


def gdn_scan_backward(desc, q, k, v, alpha, beta, s_init, d_o, d_sfinal, dq, dk, dv, dalpha, dbeta, ds_init, ws,
                      stream=None):
    a, BL, H, D = desc.act_dtype, desc.B * desc.L, desc.H, desc.dk
    st = desc.B * H * D * D
    f = torch.float32
    wp, wn = _ws(ws)
    _check(load().gdn_scan_backward(
        ctypes.byref(desc), _ptr(q, "q", a, BL * H * D), _ptr(k, "k", a, BL * H * D),
        _ptr(v, "v", a, BL * H * D), _ptr(alpha, "alpha", f, BL * H), _ptr(beta, "beta", f, BL * H),
        _ptr(s_init, "s_init", f, st, optional=True), _ptr(d_o, "d_o", f, BL * H * D),
        _ptr(d_sfinal, "d_sfinal", f, st, optional=True), _ptr(dq, "dq", f, BL * H * D),
        _ptr(dk, "dk", f, BL * H * D), _ptr(dv, "dv", f, BL * H * D), _ptr(dalpha, "dalpha", f, BL * H),
        _ptr(dbeta, "dbeta", f, BL * H), _ptr(ds_init, "ds_init", f, st, optional=True), wp, wn, _stream(stream)))


def gdn_loop_backward(desc, h0, Wpack, rho, h_loops, dh, dh0, dWq, dWk, dWv, dwa, dwb, drho, ws, stream=None):
    a, BL, d, T, H = desc.act_dtype, desc.B * desc.L, desc.d, desc.T, desc.H
    pb = gdn_weights_packed_bytes(desc)
    f = torch.float32
    wp, wn = _ws(ws)
    _check(load().gdn_loop_backward(
        ctypes.byref(desc), _ptr(h0, "h0", a, BL * d),
        _ptr(Wpack, "Wpack", a, pb // (4 if desc.act == GDN_F32 else 2)), _ptr(rho, "rho", f, T * d),
        _ptr(h_loops, "h_loops", f, T * BL * d, optional=T == 1), _ptr(dh, "dh", f, BL * d),
        _ptr(dh0, "dh0", f, BL * d), _ptr(dWq, "dWq", f, d * H * desc.dk), _ptr(dWk, "dWk", f, d * H * desc.dk),
        _ptr(dWv, "dWv", f, d * H * desc.dv), _ptr(dwa, "dwa", f, d * H), _ptr(dwb, "dwb", f, d * H),
        _ptr(drho, "drho", f, T * d), wp, wn, _stream(stream)))


def gdn_scan_decode(desc, q, k, v, alpha, beta, states, o, stream=None):
    a, N, H, D = desc.act_dtype, desc.B, desc.H, desc.dk
    _check(load().gdn_scan_decode(
        ctypes.byref(desc), _ptr(q, "q", a, N * H * D), _ptr(k, "k", a, N * H * D),
        _ptr(v, "v", a, N * H * D), _ptr(alpha, "alpha", torch.float32, N * H),
        _ptr(beta, "beta", torch.float32, N * H),
        _ptr(states, "states", torch.float32, N * H * D * D),
        _ptr(o, "o", torch.float32, N * H * D), _stream(stream)))


def gdn_loop_prefill(desc, h0, Wpack, rho, h_out, states_out, h_loops, ws, stream=None):
    a, BL, d, T = desc.act_dtype, desc.B * desc.L, desc.d, desc.T
    pb = gdn_weights_packed_bytes(desc)
    wp, wn = _ws(ws)
    _check(load().gdn_loop_prefill(
        ctypes.byref(desc), _ptr(h0, "h0", a, BL * d),
        _ptr(Wpack, "Wpack", a, pb // (4 if desc.act == GDN_F32 else 2)),
        _ptr(rho, "rho", torch.float32, T * d), _ptr(h_out, "h_out", torch.float32, BL * d),
        _ptr(states_out, "states_out", torch.float32, T * desc.B * desc.H * desc.dk * desc.dv,
             optional=True),
        _ptr(h_loops, "h_loops", torch.float32, T * BL * d, optional=True), wp, wn,
        _stream(stream)))


def gdn_loop_prefill_set_pieces(tokens: int) -> None:
    """-1: loops one after another; 0: automatic; > 0: pieces of about that many tokens (process-wide)."""
    _check(load().gdn_loop_prefill_set_pieces(int(tokens)))


def gdn_loop_prefill_pieces(desc) -> int:
    """Tokens per piece that gdn_loop_prefill would use for desc now (0: loop by loop)."""
    n = ctypes.c_int()
    _check(load().gdn_loop_prefill_pieces(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def gdn_loop_prefill_act(desc, h0, Wpack, rho, w_halt, b_halt, eps, h_out, halt_loop, ponder, ws, stream=None):
    a, BL, d, T = desc.act_dtype, desc.B * desc.L, desc.d, desc.T
    pb = gdn_weights_packed_bytes(desc)
    wp, wn = _ws(ws)
    _check(load().gdn_loop_prefill_act(
        ctypes.byref(desc), _ptr(h0, "h0", a, BL * d),
        _ptr(Wpack, "Wpack", a, pb // (4 if desc.act == GDN_F32 else 2)),
        _ptr(rho, "rho", torch.float32, T * d), _ptr(w_halt, "w_halt", torch.float32, d), float(b_halt), float(eps),
        _ptr(h_out, "h_out", torch.float32, BL * d), _ptr(halt_loop, "halt_loop", torch.int32, BL, optional=True),
        _ptr(ponder, "ponder", torch.float32, BL, optional=True), wp, wn, _stream(stream)))


def gdn_loop_decode(desc, h_t, Wpack, rho, states, h_out, ws, stream=None):
    a, N, d, T = desc.act_dtype, desc.B, desc.d, desc.T
    pb = gdn_weights_packed_bytes(desc)
    wp, wn = _ws(ws)
    _check(load().gdn_loop_decode(
        ctypes.byref(desc), _ptr(h_t, "h_t", a, N * d),
        _ptr(Wpack, "Wpack", a, pb // (4 if desc.act == GDN_F32 else 2)),
        _ptr(rho, "rho", torch.float32, T * d),
        _ptr(states, "states", torch.float32, T * N * desc.H * desc.dk * desc.dv),
        _ptr(h_out, "h_out", torch.float32, N * d), wp, wn, _stream(stream)))


def gdn_loop_decode_noalloc(desc, h_t, Wpack, rho, states, h_out, stream=None):
    """gdn_loop_decode on the library's own device scratch (no workspace argument, nothing allocated)."""
    a, N, d, T = desc.act_dtype, desc.B, desc.d, desc.T
    pb = gdn_weights_packed_bytes(desc)
    _check(load().gdn_loop_decode_noalloc(
        ctypes.byref(desc), _ptr(h_t, "h_t", a, N * d),
        _ptr(Wpack, "Wpack", a, pb // (4 if desc.act == GDN_F32 else 2)),
        _ptr(rho, "rho", torch.float32, T * d),
        _ptr(states, "states", torch.float32, T * N * desc.H * desc.dk * desc.dv),
        _ptr(h_out, "h_out", torch.float32, N * d), _stream(stream)))


# ---- timers ------------------------------------------------------------------
def gdn_timer_create(stage: int, capacity: int) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().gdn_timer_create(stage, capacity, ctypes.byref(h)))
    return h


def gdn_timer_set_stride(timer, stride: int) -> None:
    _check(load().gdn_timer_set_stride(timer, stride))


def gdn_timer_attach(timer) -> None:
    _check(load().gdn_timer_attach(timer))


def gdn_timer_detach() -> None:
    _check(load().gdn_timer_detach())


def gdn_timer_reset(timer) -> None:
    _check(load().gdn_timer_reset(timer))


def gdn_timer_read(timer):
    n, ms = ctypes.c_int(), ctypes.c_double()
    _check(load().gdn_timer_read(timer, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def gdn_timer_destroy(timer) -> None:
    _check(load().gdn_timer_destroy(timer))
