"""Gated delta-rule recurrence (Gated DeltaNet / Kimi Delta Attention) on MI355X.

Thin Python binding of ``libgdr.so`` (C ABI in ``include/gdr.h``).  This module
only marshals arguments: it checks tensor placement, takes the current HIP
stream from torch and calls the library; every step of the computation runs
in the library's gfx950 kernels.  There is no fallback: if the library is
missing, the calls raise.

    o, S = gdr_prefill_chunked(q, k, v, beta, log_alpha, initial_state=S0, cu_seqlens=cu)
    o    = gdr_decode_step(q, k, v, beta, log_alpha, state)   # state updated in place
    o    = gdr_decode_tokens(q, k, v, beta, log_alpha, pool, num_commit=c, state_slots=s)
    g    = gdr_prefill_backward(q, k, v, beta, log_alpha, d_out, initial_state=S0, d_final_state=dS)

Value heads may share query-key heads: q and k carry Hk heads, v, the gates,
the states and the outputs H (a multiple of Hk); value head h reads q/k head
h // (H // Hk).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["gdr_prefill_chunked", "gdr_prefill_chunked_static", "gdr_decode_step", "gdr_decode_step_prologue", "gdr_decode_tokens", "gdr_layer_prologue",
           "gdr_prefill_backward", "gdr_prefill_backward_workspace_bytes", "prefill_chunked", "decode_step", "decode_tokens", "layer_prologue",
           "prefill_backward",
           "gdr_state_bytes", "GdrError", "load_library", "library_path"]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libgdr.so")

GDR_SUCCESS, GDR_ERROR_INVALID_VALUE, GDR_ERROR_NOT_SUPPORTED = 0, 1, 2
GDR_ERROR_INSUFFICIENT_WORKSPACE, GDR_ERROR_LAUNCH_FAILED = 3, 4
GDR_F32, GDR_BF16 = 0, 1
GDR_GATE_HEAD, GDR_GATE_CHANNEL = 0, 1
GDR_PROLOGUE_SILU, GDR_PROLOGUE_QK_NORM = 1, 2


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gdr status {status}: {message}")
        self.status = status


class PrefillShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("num_qk_heads", ctypes.c_int32)]

ABI_VERSION = 6


_lib = None


def load_library():
    """Load libgdr.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with `python -m gated_delta_rule_73_amd.build`")
        lib = ctypes.CDLL(library_path)
        p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.gdr_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillShape), i32, i32, i32, i32]
        lib.gdr_prefill_workspace_bytes.restype = sz
        lib.gdr_prefill_chunked.argtypes = [ctypes.POINTER(PrefillShape), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, p, p, p, p, p, p, p, i32, i32, ctypes.c_float, p, p, p,
                                            sz, p]
        lib.gdr_prefill_chunked.restype = ctypes.c_int
        lib.gdr_prefill_chunked_static.argtypes = [ctypes.POINTER(PrefillShape), ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int, p, p, p, p, p, p, p, i32, i32,
                                                   ctypes.c_float, p, p, p]
        lib.gdr_prefill_chunked_static.restype = ctypes.c_int
        lib.gdr_decode_step.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, p, p, p, p, p, p, ctypes.c_float, p, p]
        lib.gdr_decode_step.restype = ctypes.c_int
        lib.gdr_decode_tokens.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, p, p, p, p, p, p, p, p, p, i32, ctypes.c_float, p, p]
        lib.gdr_decode_tokens.restype = ctypes.c_int
        lib.gdr_layer_prologue.argtypes = [ctypes.POINTER(PrefillShape), ctypes.c_int, ctypes.c_int, p, p, p, p, p, i32,
                                           p, p, p, p, p, p, p, p]
        lib.gdr_layer_prologue.restype = ctypes.c_int
        lib.gdr_decode_step_prologue.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 p, p, p, p, i32, p, p, p, ctypes.c_float, p, p]
        lib.gdr_decode_step_prologue.restype = ctypes.c_int
        lib.gdr_prefill_backward_workspace_bytes.argtypes = [ctypes.POINTER(PrefillShape), ctypes.c_int, i32]
        lib.gdr_prefill_backward_workspace_bytes.restype = sz
        lib.gdr_prefill_backward_segment_workspace_bytes.argtypes = [ctypes.POINTER(PrefillShape), ctypes.c_int, i32]
        lib.gdr_prefill_backward_segment_workspace_bytes.restype = sz
        lib.gdr_prefill_backward.argtypes = [ctypes.POINTER(PrefillShape), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             p, p, p, p, p, p, p, ctypes.c_float, p, p, p, p, p, p, p, p, p, sz, p]
        lib.gdr_prefill_backward.restype = ctypes.c_int
        lib.gdr_state_bytes.argtypes = [ctypes.c_int64] * 4
        lib.gdr_state_bytes.restype = ctypes.c_uint64
        lib.gdr_status_string.argtypes = [ctypes.c_int]
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_last_error.restype = ctypes.c_char_p
        lib.gdr_abi_version.restype = ctypes.c_int
        if lib.gdr_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{library_path} has ABI {lib.gdr_abi_version()}, this binding needs {ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


def _check(status: int):
    if status != GDR_SUCCESS:
        raise GdrError(status, load_library().gdr_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def gdr_state_bytes(num_seqs: int, num_heads: int, head_dim_k: int, head_dim_v: int) -> int:
    return int(load_library().gdr_state_bytes(num_seqs, num_heads, head_dim_k, head_dim_v))


def gdr_prefill_chunked(q, k, v, beta, log_alpha, *, initial_state=None, cu_seqlens=None, chunk_size: int = 0,
                        dv_slice: int = 0, scale: float = 1.0, out=None, out_dtype=torch.float32,
                        final_state=None, output_final_state: bool = True, workspace=None):
    """Chunked prefill.  q, k [B, T, Hk, dk]; v [B, T, H, dv] (bf16 or fp32; Hk divides H);
    beta [B, T, H]; log_alpha [B, T, H] (per-head decay) or [B, T, H, dk]
    (per-key-channel decay), both fp32 or both bf16; initial_state [N, H, dv, dk] fp32 or None;
    cu_seqlens int32 [N+1] (packed, B == 1) or None.
    out_dtype (fp32 or bf16) applies when ``out`` is not given.
    workspace: uint8 device tensor, or None to allocate the size
    ``gdr_prefill_workspace_bytes`` reports (a smaller one makes a dense batch
    run in segments).
    Returns (out [B, T, H, dv], final_state [N, H, dv, dk] or None)."""
    lib = load_library()
    dev = q.device
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or beta.shape != (B, T, H):
        raise ValueError("shapes: q, k [B, T, Hk, dk], v [B, T, H, dv], beta [B, T, H]")
    if log_alpha.dim() == 3:
        gate = GDR_GATE_HEAD
    elif log_alpha.dim() == 4:
        gate = GDR_GATE_CHANNEL
    else:
        raise ValueError("log_alpha must be [B, T, H] or [B, T, H, dk]")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, q.dtype, dev)
    _need(beta, "beta", None, dev)
    _need(log_alpha, "log_alpha", beta.dtype, dev)
    _need(initial_state, "initial_state", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    if out is None:
        out = torch.empty(B, T, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", None, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty(N, H, dv, dk, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev)
    shape = PrefillShape(B, T, H, dk, dv, N, Hk)
    ws_bytes = lib.gdr_prefill_workspace_bytes(ctypes.byref(shape), gate, _dtype_code(q), int(chunk_size),
                                               int(cu_seqlens is not None))
    if workspace is None:
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    else:
        _need(workspace, "workspace", torch.uint8, dev)
        ws, ws_bytes = workspace, workspace.numel()
    _check(lib.gdr_prefill_chunked(
        ctypes.byref(shape), gate, _dtype_code(q), _dtype_code(beta), _dtype_code(out), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
        _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size), int(dv_slice), float(scale), _ptr(out),
        _ptr(final_state), _ptr(ws), int(ws_bytes), _stream(dev)))
    return out, final_state


def gdr_prefill_chunked_static(q, k, v, beta, log_alpha, *, initial_state=None, cu_seqlens=None,
                               chunk_size: int = 0, dv_slice: int = 0, scale: float = 1.0, out=None,
                               out_dtype=torch.float32, final_state=None, output_final_state: bool = True):
    """:func:`gdr_prefill_chunked` on the library's fixed per-device scratch
    (no workspace argument, no device allocation inside the call).  Calls that
    overlap on one GPU share that scratch and race.  Raises GdrError
    (insufficient workspace) when the problem does not fit the scratch."""
    lib = load_library()
    dev = q.device
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or beta.shape != (B, T, H):
        raise ValueError("shapes: q, k [B, T, Hk, dk], v [B, T, H, dv], beta [B, T, H]")
    if log_alpha.dim() not in (3, 4):
        raise ValueError("log_alpha must be [B, T, H] or [B, T, H, dk]")
    gate = GDR_GATE_HEAD if log_alpha.dim() == 3 else GDR_GATE_CHANNEL
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, q.dtype, dev)
    _need(beta, "beta", None, dev)
    _need(log_alpha, "log_alpha", beta.dtype, dev)
    _need(initial_state, "initial_state", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    if out is None:
        out = torch.empty(B, T, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", None, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty(N, H, dv, dk, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev)
    shape = PrefillShape(B, T, H, dk, dv, N, Hk)
    _check(lib.gdr_prefill_chunked_static(
        ctypes.byref(shape), gate, _dtype_code(q), _dtype_code(beta), _dtype_code(out), _ptr(q), _ptr(k), _ptr(v),
        _ptr(beta), _ptr(log_alpha), _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size), int(dv_slice),
        float(scale), _ptr(out), _ptr(final_state), _stream(dev)))
    return out, final_state


def gdr_prefill_backward_workspace_bytes(q, v, log_alpha, *, cu_seqlens=None, segment_chunks: int = 0) -> int:
    """Workspace bytes :func:`gdr_prefill_backward` needs for these shapes: one
    pass (segment_chunks 0), or a dense batch in time segments of
    segment_chunks >= 16 chunks (0 if that is not possible)."""
    lib = load_library()
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    gate = GDR_GATE_HEAD if log_alpha.dim() == 3 else GDR_GATE_CHANNEL
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    shape = PrefillShape(B, T, H, dk, dv, N, Hk)
    if segment_chunks:
        if cu_seqlens is not None:
            return 0
        return int(lib.gdr_prefill_backward_segment_workspace_bytes(ctypes.byref(shape), gate, int(segment_chunks)))
    return int(lib.gdr_prefill_backward_workspace_bytes(ctypes.byref(shape), gate, int(cu_seqlens is not None)))


def gdr_prefill_backward(q, k, v, beta, log_alpha, d_out, *, initial_state=None, d_final_state=None,
                         cu_seqlens=None, scale: float = 1.0, output_d_initial_state: bool = True,
                         workspace=None):
    """Gradients through :func:`gdr_prefill_chunked` (same q, k, v, beta,
    log_alpha, initial_state, cu_seqlens and scale, grouped q/k heads and
    bf16 gates included).  d_out [B, T, H, dv] fp32; d_final_state
    [N, H, dv, dk] fp32 or None (zeros).  workspace: uint8 device tensor, or
    None to allocate the one-pass size; a dense batch also runs in a smaller
    one, in time segments (see :func:`gdr_prefill_backward_workspace_bytes`).
    Returns a dict of fp32 tensors: dq, dk (q's shape), dv (v's), dbeta,
    dlog_alpha (log_alpha's shape) and d_initial_state [N, H, dv, dk] (None
    when not requested)."""
    lib = load_library()
    dev = q.device
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or beta.shape != (B, T, H):
        raise ValueError("shapes: q, k [B, T, Hk, dk], v [B, T, H, dv], beta [B, T, H]")
    if log_alpha.dim() == 3:
        gate = GDR_GATE_HEAD
    elif log_alpha.dim() == 4:
        gate = GDR_GATE_CHANNEL
    else:
        raise ValueError("log_alpha must be [B, T, H] or [B, T, H, dk]")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, q.dtype, dev)
    _need(beta, "beta", None, dev)
    _need(log_alpha, "log_alpha", beta.dtype, dev)
    _need(initial_state, "initial_state", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(d_out, "d_out", torch.float32, dev)
    _need(d_final_state, "d_final_state", torch.float32, dev)
    if d_out.shape != v.shape:
        raise ValueError("d_out must have v's shape")
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(q.shape, **f32), "dv": torch.empty(v.shape, **f32),
         "dbeta": torch.empty(beta.shape, **f32), "dlog_alpha": torch.empty(log_alpha.shape, **f32),
         "d_initial_state": torch.empty(N, H, dv, dk, **f32) if output_d_initial_state else None}
    shape = PrefillShape(B, T, H, dk, dv, N, Hk)
    ws_bytes = lib.gdr_prefill_backward_workspace_bytes(ctypes.byref(shape), gate, int(cu_seqlens is not None))
    if workspace is None:
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    else:
        _need(workspace, "workspace", torch.uint8, dev)
        ws, ws_bytes = workspace, workspace.numel()
    _check(lib.gdr_prefill_backward(
        ctypes.byref(shape), gate, _dtype_code(q), _dtype_code(beta), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
        _ptr(log_alpha),
        _ptr(initial_state), _ptr(cu_seqlens), float(scale), _ptr(d_out), _ptr(d_final_state), _ptr(g["dq"]),
        _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dbeta"]), _ptr(g["dlog_alpha"]), _ptr(g["d_initial_state"]),
        _ptr(ws), int(ws_bytes), _stream(dev)))
    return g


def gdr_decode_step(q, k, v, beta, log_alpha, state, *, scale: float = 1.0, out=None, out_dtype=torch.float32):
    """Decode step, one token per sequence: q, k [N, Hk, dk]; v [N, H, dv];
    beta [N, H]; log_alpha [N, H] or [N, H, dk] (gates fp32 or both bf16); state [N, H, dv, dk] fp32
    (updated in place).  Returns out [N, H, dv]."""
    lib = load_library()
    dev = q.device
    N, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N or beta.shape != (N, H):
        raise ValueError("shapes: q, k [N, Hk, dk], v [N, H, dv], beta [N, H]")
    gate = GDR_GATE_HEAD if log_alpha.dim() == 2 else GDR_GATE_CHANNEL
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, q.dtype, dev)
    _need(beta, "beta", None, dev)
    _need(log_alpha, "log_alpha", beta.dtype, dev)
    _need(state, "state", torch.float32, dev)
    if out is None:
        out = torch.empty(N, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", None, dev)
    _check(lib.gdr_decode_step(N, H, Hk, dk, dv, gate, _dtype_code(q), _dtype_code(beta), _dtype_code(out), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                               _ptr(log_alpha), _ptr(state), float(scale), _ptr(out), _stream(dev)))
    return out


def gdr_decode_tokens(q, k, v, beta, log_alpha, state_pool, *, num_tokens=None, num_commit=None,
                      state_slots=None, scale: float = 1.0, out=None, out_dtype=torch.float32):
    """Up to K tokens per sequence from a pool of states: q, k [N, K, Hk, dk];
    v [N, K, H, dv]; beta [N, K, H]; log_alpha [N, K, H] or [N, K, H, dk];
    state_pool [P, H, dv, dk] fp32; num_tokens, num_commit, state_slots int32
    [N] device tensors or None (K tokens, all committed, slot n).  Runs each
    sequence's tokens from its slot, writes out [N, K, H, dv] for its tokens
    and keeps in the slot the state after its first num_commit tokens (0: the
    slot is left as it was).  Returns out."""
    lib = load_library()
    dev = q.device
    N, K, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (N, K) or beta.shape != (N, K, H):
        raise ValueError("shapes: q, k [N, K, Hk, dk], v [N, K, H, dv], beta [N, K, H]")
    gate = GDR_GATE_HEAD if log_alpha.dim() == 3 else GDR_GATE_CHANNEL
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, q.dtype, dev)
    _need(beta, "beta", None, dev)
    _need(log_alpha, "log_alpha", beta.dtype, dev)
    _need(state_pool, "state_pool", torch.float32, dev)
    for t, nm in ((num_tokens, "num_tokens"), (num_commit, "num_commit"), (state_slots, "state_slots")):
        _need(t, nm, torch.int32, dev)
        if t is not None and t.shape != (N,):
            raise ValueError(f"{nm} must have shape [{N}]")
    if state_pool.dim() != 4 or state_pool.shape[1:] != (H, dv, dk):
        raise ValueError(f"state_pool must be [P, {H}, {dv}, {dk}]")
    if out is None:
        out = torch.empty(N, K, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", None, dev)
    _check(lib.gdr_decode_tokens(N, K, H, Hk, dk, dv, gate, _dtype_code(q), _dtype_code(beta), _dtype_code(out), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(num_tokens), _ptr(num_commit),
                                 _ptr(state_slots), _ptr(state_pool), int(state_pool.shape[0]), float(scale),
                                 _ptr(out), _stream(dev)))
    return out


def gdr_layer_prologue(x, conv_weight, a_logit, b_logit, *, num_qk_heads: int, head_dim_k: int, head_dim_v: int,
                       conv_state=None, update_conv_state: bool = True, cu_seqlens=None, silu: bool = False,
                       qk_norm: bool = True):
    """Short causal convolution (width 4) of the projected channels, optional
    SiLU, per-head L2 norm of q and k, and the gate activations, in one pass.
    x [B, T, C] (bf16 or fp32) with C = 2 Hk dk + H dv channels (q, k, v);
    conv_weight [C, 4] fp32 (tap j multiplies x_{t-3+j}); a_logit [B, T, H] or
    [B, T, H, dk] and b_logit [B, T, H] fp32; conv_state [N, 3, C] (x's dtype)
    or None (zeros), updated in place to each sequence's last three inputs
    when update_conv_state.  Returns (q, k [B, T, Hk, dk], v [B, T, H, dv],
    beta = sigmoid(b), log_alpha = -softplus(a))."""
    lib = load_library()
    dev = x.device
    B, T, C = x.shape
    H = b_logit.shape[-1]
    Hk, dk, dv = num_qk_heads, head_dim_k, head_dim_v
    if C != 2 * Hk * dk + H * dv or b_logit.shape != (B, T, H):
        raise ValueError(f"x must be [B, T, 2*Hk*dk + H*dv] = [{B}, {T}, {2 * Hk * dk + H * dv}], b_logit [B, T, H]")
    gate = GDR_GATE_HEAD if a_logit.dim() == 3 else GDR_GATE_CHANNEL
    _need(x, "x", None, dev)
    _need(conv_weight, "conv_weight", torch.float32, dev)
    _need(a_logit, "a_logit", torch.float32, dev)
    _need(b_logit, "b_logit", torch.float32, dev)
    _need(conv_state, "conv_state", x.dtype, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    if conv_state is not None and conv_state.shape != (N, 3, C):
        raise ValueError(f"conv_state must be [{N}, 3, {C}]")
    q = torch.empty(B, T, Hk, dk, dtype=x.dtype, device=dev)
    k = torch.empty_like(q)
    v = torch.empty(B, T, H, dv, dtype=x.dtype, device=dev)
    beta = torch.empty(B, T, H, dtype=torch.float32, device=dev)
    log_alpha = torch.empty_like(a_logit)
    shape = PrefillShape(B, T, H, dk, dv, N, Hk)
    flags = (GDR_PROLOGUE_SILU if silu else 0) | (GDR_PROLOGUE_QK_NORM if qk_norm else 0)
    _check(lib.gdr_layer_prologue(ctypes.byref(shape), gate, _dtype_code(x), _ptr(x), _ptr(conv_weight),
                                  _ptr(conv_state), _ptr(conv_state) if update_conv_state else None, _ptr(cu_seqlens),
                                  flags, _ptr(a_logit), _ptr(b_logit), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                  _ptr(log_alpha), _stream(dev)))
    return q, k, v, beta, log_alpha


def gdr_decode_step_prologue(x, conv_weight, a_logit, b_logit, state, *, num_qk_heads: int, head_dim_k: int,
                             head_dim_v: int, conv_state=None, update_conv_state: bool = True, silu: bool = False,
                             qk_norm: bool = True, scale: float = 1.0, out=None, out_dtype=torch.float32):
    """One decode step from the token's projected channels: the layer prologue
    (as :func:`gdr_layer_prologue` with T = 1) fused with the state update (as
    :func:`gdr_decode_step`).  x [N, C] (bf16 or fp32), C = 2 Hk dk + H dv;
    conv_weight [C, 4] fp32; a_logit [N, H] or [N, H, dk] and b_logit [N, H]
    fp32; state [N, H, dv, dk] fp32, updated in place; conv_state [N, 3, C]
    (x's dtype) or None (zeros), advanced in place when update_conv_state.
    Returns out [N, H, dv]."""
    lib = load_library()
    dev = x.device
    N, C = x.shape
    H = b_logit.shape[-1]
    Hk, dk, dv = num_qk_heads, head_dim_k, head_dim_v
    if C != 2 * Hk * dk + H * dv or b_logit.shape != (N, H) or state.shape != (N, H, dv, dk):
        raise ValueError(f"x must be [N, 2*Hk*dk + H*dv] = [{N}, {2 * Hk * dk + H * dv}], b_logit [N, H], "
                         f"state [N, H, dv, dk]")
    gate = GDR_GATE_HEAD if a_logit.dim() == 2 else GDR_GATE_CHANNEL
    _need(x, "x", None, dev)
    _need(conv_weight, "conv_weight", torch.float32, dev)
    _need(a_logit, "a_logit", torch.float32, dev)
    _need(b_logit, "b_logit", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    _need(conv_state, "conv_state", x.dtype, dev)
    if conv_state is not None and conv_state.shape != (N, 3, C):
        raise ValueError(f"conv_state must be [{N}, 3, {C}]")
    if out is None:
        out = torch.empty(N, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", None, dev)
    flags = (GDR_PROLOGUE_SILU if silu else 0) | (GDR_PROLOGUE_QK_NORM if qk_norm else 0)
    _check(lib.gdr_decode_step_prologue(N, H, Hk, dk, dv, gate, _dtype_code(x), _dtype_code(out), _ptr(x),
                                        _ptr(conv_weight), _ptr(conv_state),
                                        _ptr(conv_state) if update_conv_state else None, flags, _ptr(a_logit),
                                        _ptr(b_logit), _ptr(state), float(scale), _ptr(out), _stream(dev)))
    return out


prefill_chunked = gdr_prefill_chunked
decode_step = gdr_decode_step
decode_tokens = gdr_decode_tokens
layer_prologue = gdr_layer_prologue
prefill_backward = gdr_prefill_backward
