"""gdr_prefill_chunked_static (the library's fixed per-device scratch in place
of a caller workspace) against gdr_prefill_chunked on the same inputs, over
consecutive calls that reuse the scratch (the second smaller than the first),
and its rejection of a problem larger than the scratch."""
import ctypes

import pytest
import torch

import gated_delta_rule_73_amd as gdr
from parity import TOL, assert_close, gpu_available, say
from workloads import Workload, prefill_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]
DEV = "cuda"
SCRATCH = 64 << 20


def _inputs(name, dk, dv, H, T, gate, B=1, lengths=None, seed=0):
    w = Workload(name, "prefill", heads=H, dk=dk, dv=dv, qkv_dtype=torch.bfloat16, gate=gate, batch=B, seqlen=T,
                 init_state=True, seed=seed)
    return prefill_inputs(w, DEV, lengths=lengths)


def _args(inp):
    return (inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"])


def _static_raw(inp, chunk=0):
    """The static entry point called through the C-ABI with preallocated
    outputs; the device allocator must not move."""
    lib = gdr.load_library()
    q, v = inp["q"], inp["v"]
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    cu = inp["cu_seqlens"]
    N = cu.numel() - 1 if cu is not None else B
    out = torch.empty(B, T, H, dv, dtype=torch.float32, device=DEV)
    fin = torch.empty(N, H, dv, dk, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    gate = gdr.GDR_GATE_CHANNEL if inp["log_alpha"].dim() == 4 else gdr.GDR_GATE_HEAD
    shape = gdr.PrefillShape(B, T, H, dk, dv, N, Hk)
    p = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    st = lib.gdr_prefill_chunked_static(
        ctypes.byref(shape), gate, gdr.GDR_BF16, gdr.GDR_F32, gdr.GDR_F32, p(q), p(inp["k"]), p(v), p(inp["beta"]),
        p(inp["log_alpha"]), p(inp["initial_state"]), p(cu), int(chunk), 0, 1.0, p(out), p(fin),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == gdr.GDR_SUCCESS, lib.gdr_last_error().decode()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return out, fin


def _compare(label, inp, chunk=0):
    say(f"static scratch: {label}")
    out_s, fin_s = _static_raw(inp, chunk)
    out_r, fin_r = gdr.gdr_prefill_chunked(*_args(inp), initial_state=inp["initial_state"],
                                           cu_seqlens=inp["cu_seqlens"], chunk_size=chunk)
    torch.cuda.synchronize()
    assert_close("out vs gdr_prefill_chunked", out_s, out_r, TOL[torch.bfloat16])
    assert_close("final_state vs gdr_prefill_chunked", fin_s, fin_r, TOL[torch.bfloat16])
    return out_s, fin_s


def test_static_scratch_consecutive_calls():
    # 1: a dense KDA batch whose one-pass records (about 120 MiB) exceed the
    # scratch, so it runs in segments; with a caller workspace of the same
    # size the existing entry point takes the same schedule, bit for bit
    big = _inputs("kda_dense", 128, 128, 8, 8192, "channel", B=2, seed=11)
    out_s, fin_s = _compare("KDA B=2 T=8192 H=8 d=128 (segmented)", big)
    ws = torch.empty(SCRATCH, dtype=torch.uint8, device=DEV)
    out_w, fin_w = gdr.gdr_prefill_chunked(*_args(big), initial_state=big["initial_state"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_w) and torch.equal(fin_s, fin_w)
    del big, ws, out_w, fin_w
    # 2: smaller, packed GDN (one pass over every chunk fits)
    small = _inputs("gdn_packed", 64, 64, 4, 700, "head", lengths=[300, 17, 383], seed=12)
    _compare("packed GDN 3 sequences, 700 tokens, H=4 d=64", small)
    # 3: smaller still, 64-token chunks at d_k = 64
    tiny = _inputs("gdn_c64", 64, 64, 2, 200, "head", seed=13)
    _compare("GDN T=200 H=2 d=64, chunk 64", tiny, chunk=64)
    # 4: 64-token chunks at d_k = 128 (the two kernels), records past the
    # scratch, so in segments
    wide = _inputs("kda_wide", 128, 128, 8, 8192, "channel", B=2, seed=14)
    _compare("KDA B=2 T=8192 H=8 d=128, chunk 64 (segmented)", wide, chunk=64)


def test_static_scratch_rejects_larger_problem():
    """A packed batch always needs its one-pass workspace: 64K tokens x 16
    heads of d=128 records is far past 64 MiB.  Rejected before anything is
    enqueued (the pointers are never dereferenced)."""
    lib = gdr.load_library()
    cu = torch.tensor([0, 30000, 65536], dtype=torch.int32, device=DEV)
    bufs = [torch.empty(256, dtype=torch.float32, device=DEV) for _ in range(7)]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    shape = gdr.PrefillShape(1, 65536, 16, 128, 128, 2, 16)
    st = lib.gdr_prefill_chunked_static(
        ctypes.byref(shape), gdr.GDR_GATE_HEAD, gdr.GDR_BF16, gdr.GDR_F32, gdr.GDR_F32, p(bufs[0]), p(bufs[1]),
        p(bufs[2]), p(bufs[3]), p(bufs[4]), None, p(cu), 0, 0, 1.0, p(bufs[5]), p(bufs[6]),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    msg = lib.gdr_last_error().decode()
    say(f"  rejected: status {st}: {msg}")
    assert st == gdr.GDR_ERROR_INSUFFICIENT_WORKSPACE
    assert "static scratch" in msg
