"""Backward of the chunked prefill on the GPU vs the fp64 oracle's gradients.

Every gradient (dq, dk, dv, dbeta, dlog_alpha, d_initial_state) is compared
element by element with the oracle on the same seeded inputs and loss
gradients.  The GPU computes in fp32 from the stored bf16/fp32 values the
oracle also sees, so the bar is fp32 arithmetic: max |gpu - oracle| <=
TOL_BWD * RMS(oracle) per tensor.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_73_amd as gdr
import oracle
from parity import assert_close, gpu_available, say, to_np
from workloads import WORKLOADS, Workload, backward_cotangents, prefill_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]
DEV = "cuda"
TOL_BWD = 1e-3
NAMES = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "d_initial_state")


def _gpu(inp, cot, *, scale=1.0, with_final=True, with_init=True):
    g = gdr.gdr_prefill_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], cot["d_out"],
                                 initial_state=inp["initial_state"],
                                 d_final_state=cot["d_final_state"] if with_final else None,
                                 cu_seqlens=inp["cu_seqlens"], scale=scale, output_d_initial_state=with_init)
    torch.cuda.synchronize()
    return g


def _oracle(inp, cot, *, scale=1.0, with_final=True, sl=None):
    cu = inp["cu_seqlens"]
    return oracle.recurrence_backward(
        inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], cot["d_out"],
        initial_state=inp["initial_state"], d_final_state=cot["d_final_state"] if with_final else None,
        seq_bounds=None if cu is None else cu.cpu().numpy(), scale=scale)


def _check(inp, cot, label, tol=TOL_BWD, **kw):
    say(f"backward {label} {kw}")
    got = _gpu(inp, cot, **kw)
    ref = _oracle(inp, cot, scale=kw.get("scale", 1.0), with_final=kw.get("with_final", True))
    worst = 0.0
    for name in NAMES:
        if got[name] is None:
            continue
        worst = max(worst, assert_close(name, got[name], ref[name], tol))
    return got, worst


def _small(dk, dv, H, T, gate, dtype, init, seed, B=1, lengths=None):
    w = Workload("small", "backward", heads=H, dk=dk, dv=dv, qkv_dtype=dtype, gate=gate, batch=B, seqlen=T,
                 init_state=init, seed=seed)
    inp = prefill_inputs(w, DEV, lengths=lengths)
    return inp, backward_cotangents(inp, seed, DEV)


CASES = [
    # dk, dv, H, T, gate, init, B
    (32, 32, 2, 100, "head", False, 1),
    (32, 32, 2, 31, "channel", True, 1),      # one ragged chunk
    (64, 96, 2, 70, "channel", True, 1),      # value rows in two-wave slices
    (64, 64, 2, 97, "channel", True, 1),
    (64, 128, 1, 32, "head", True, 2),        # exactly one chunk per sequence
    (128, 64, 3, 77, "head", True, 1),
    (128, 128, 2, 130, "channel", True, 2),
    (128, 128, 2, 200, "head", False, 1),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"dk{c[0]}-dv{c[1]}-H{c[2]}-T{c[3]}-{c[4]}-s0{int(c[5])}-B{c[6]}")
def test_backward_shapes(case, dtype):
    dk, dv, H, T, gate, init, B = case
    inp, cot = _small(dk, dv, H, T, gate, dtype, init, seed=dk + dv + T, B=B)
    _check(inp, cot, f"{case} {dtype}")


# Enough (sequence, head) units that the state scans take four waves (64 value
# rows) per workgroup on a 256-CU device, at the small key widths the large
# workloads do not reach.
# (With a per-head decay the four-wave scans stage raw q and k, scaled per row,
# so those cases also run with fp32 q/k/v.)
FOUR_WAVE_CASES = [
    # dk, dv, H, T, gate, B, dtype
    (32, 64, 72, 70, "channel", 1, torch.bfloat16),
    (64, 128, 40, 45, "head", 2, torch.bfloat16),
    (32, 128, 36, 33, "head", 2, torch.bfloat16),
    (64, 128, 40, 45, "head", 2, torch.float32),
    (128, 64, 80, 37, "head", 1, torch.float32),
]


@pytest.mark.parametrize("case", FOUR_WAVE_CASES,
                         ids=lambda c: f"dk{c[0]}-dv{c[1]}-H{c[2]}-T{c[3]}-{c[4]}-B{c[5]}-{str(c[6])[6:]}")
def test_backward_four_wave_scan_small_keys(case):
    dk, dv, H, T, gate, B, dtype = case
    inp, cot = _small(dk, dv, H, T, gate, dtype, True, seed=3 * dk + T, B=B)
    _check(inp, cot, f"four-wave scan {case}")


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_backward_packed_with_empty_and_one_token_sequences(gate):
    """Packed sequences of 37, 0, 100, 1 and 64 tokens: ragged chunks, an empty
    sequence (its initial-state gradient is its final-state gradient) and a
    single token."""
    inp, cot = _small(128, 128, 2, 0, gate, torch.bfloat16, True, seed=21, lengths=[37, 0, 100, 1, 64])
    got, _ = _check(inp, cot, f"packed {gate}")
    torch.testing.assert_close(got["d_initial_state"][1], cot["d_final_state"][1], rtol=0, atol=0)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_backward_packed_four_wave_scan(gate):
    """The same kind of packed batch with enough heads for four-wave scans
    (with a per-head decay, the raw q/k staging) at d_v = 64."""
    inp, cot = _small(64, 64, 40, 0, gate, torch.bfloat16, True, seed=23, lengths=[37, 0, 70, 1, 33])
    got, _ = _check(inp, cot, f"packed four-wave {gate}")
    torch.testing.assert_close(got["d_initial_state"][1], cot["d_final_state"][1], rtol=0, atol=0)


def test_backward_without_final_gradient_or_initial_state():
    """No final-state gradient (zeros), no initial state (zeros), no
    initial-state gradient requested, a query scale."""
    inp, cot = _small(128, 128, 2, 150, "channel", torch.bfloat16, False, seed=22)
    _check(inp, cot, "no dS_final", scale=0.125, with_final=False, with_init=False)


def test_backward_strong_decay():
    """Per-channel log decay three times the workload's (a 32-token chunk then
    spans up to ~ 100 nats of decay per channel), exercising the shifted
    Gram operands."""
    inp, cot = _small(128, 128, 2, 96, "channel", torch.bfloat16, True, seed=23)
    inp["log_alpha"] = (3.0 * inp["log_alpha"]).contiguous()
    _check(inp, cot, "strong decay")


def test_backward_is_deterministic():
    inp, cot = _small(128, 128, 4, 300, "channel", torch.bfloat16, True, seed=24)
    a = _gpu(inp, cot)
    b = _gpu(inp, cot)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_backward_grouped_heads(gate):
    """2 q/k heads shared by 6 value heads: each q/k head's gradient is the sum
    over its group (the oracle's adjoint of the repetition)."""
    w = Workload("small", "backward", heads=6, qk_heads=2, dk=64, dv=64, qkv_dtype=torch.bfloat16, gate=gate,
                 batch=1, seqlen=77, init_state=True, seed=25)
    inp = prefill_inputs(w, DEV)
    cot = backward_cotangents(inp, 25, DEV)
    assert inp["q"].shape[2] == 2 and inp["v"].shape[2] == 6
    _check(inp, cot, f"grouped {gate}")


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_backward_grouped_packed(gate):
    """Grouped heads (4 q/k heads, 16 value heads, d = 128) over packed sequences."""
    w = Workload("small", "backward", heads=16, qk_heads=4, dk=128, dv=128, qkv_dtype=torch.bfloat16, gate=gate,
                 batch=1, seqlen=0, init_state=True, seed=26)
    inp = prefill_inputs(w, DEV, lengths=[45, 130, 3])
    cot = backward_cotangents(inp, 26, DEV)
    _check(inp, cot, f"grouped packed {gate}")


def test_gdn_backward_8k_workload():
    """B=1, T=8192, H=16, d=128, bf16, per-head decay, S0 ~ N(0, 0.02^2):
    every gradient of every head against the oracle."""
    w = WORKLOADS["gdn_backward_8k"]
    inp = prefill_inputs(w, DEV)
    cot = backward_cotangents(inp, w.seed, DEV)
    _check(inp, cot, "gdn_backward_8k")


@pytest.mark.slow
def test_kda_backward_32k_workload():
    """B=2, T=32768, H=32, d=128, bf16, per-channel decay, S0: every element of
    every gradient against the oracle (all host cores)."""
    w = WORKLOADS["kda_backward_32k"]
    inp = prefill_inputs(w, DEV)
    cot = backward_cotangents(inp, w.seed, DEV)
    _check(inp, cot, "kda_backward_32k (whole tensors)")


@pytest.mark.slow
def test_gdn_gva_backward_32k_workload():
    """The pages' Gated DeltaNet shape: T=32768, 16 q/k heads shared by 48
    value heads, d=128, bf16, S0: every element of every gradient against the
    oracle (dq and dk sum over the three value heads of each group)."""
    w = WORKLOADS["gdn_gva_backward_32k"]
    inp = prefill_inputs(w, DEV)
    cot = backward_cotangents(inp, w.seed, DEV)
    _check(inp, cot, "gdn_gva_backward_32k (whole tensors)")


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_backward_bf16_gates(gate):
    """beta and log alpha stored in bf16 (the forward's bf16-gate variant); the
    oracle reads the same bf16 values exactly; the gate gradients are fp32."""
    w = Workload("small", "backward", heads=2, dk=128, dv=128, qkv_dtype=torch.bfloat16, gate=gate, batch=1,
                 seqlen=100, init_state=True, seed=27)
    inp = prefill_inputs(w, DEV, gate_dtype=torch.bfloat16)
    cot = backward_cotangents(inp, 27, DEV)
    got, _ = _check(inp, cot, f"bf16 gates {gate}")
    assert got["dbeta"].dtype == torch.float32 and got["dlog_alpha"].dtype == torch.float32


def test_backward_empty_dense_batch_passes_the_state_gradient_through():
    """T = 0: no tokens, so the initial-state gradient is the final-state one."""
    inp, cot = _small(64, 64, 2, 0, "channel", torch.bfloat16, True, seed=28, B=2)
    g = _gpu(inp, cot)
    assert torch.equal(g["d_initial_state"], cot["d_final_state"])


SEGMENT_CASES = [
    # dk, dv, H, T, gate, B, segment chunks
    (128, 128, 2, 32 * 40 + 5, "channel", 2, 16),   # 41 chunks: segments of 16, 16, 9 (ragged last chunk)
    (64, 64, 3, 32 * 33, "head", 1, 16),            # 33 chunks: 16, 16, 1
    (128, 64, 2, 32 * 20 - 7, "head", 2, 16),       # 20 chunks: 16, 4
    (32, 32, 2, 32 * 50, "channel", 1, 24),         # 50 chunks: 24, 24, 2
]


@pytest.mark.parametrize("case", SEGMENT_CASES,
                         ids=lambda c: f"dk{c[0]}-dv{c[1]}-H{c[2]}-T{c[3]}-{c[4]}-B{c[5]}-S{c[6]}")
def test_backward_in_time_segments(case):
    """A workspace holding one segment's records and states (dense batch):
    the call runs in time segments, rebuilding each segment's records and
    forward states from the state entering it and carrying the state
    gradient from segment to segment.  Every gradient equals the one-pass
    call's bit for bit, and stays within the bound against the oracle."""
    dk, dv, H, T, gate, B, S = case
    inp, cot = _small(dk, dv, H, T, gate, torch.bfloat16, True, seed=dk + T + S, B=B)
    one = _gpu(inp, cot)
    nbytes = gdr.gdr_prefill_backward_workspace_bytes(inp["q"], inp["v"], inp["log_alpha"], segment_chunks=S)
    full = gdr.gdr_prefill_backward_workspace_bytes(inp["q"], inp["v"], inp["log_alpha"])
    assert 0 < nbytes < full
    say(f"backward in segments {case}: workspace {nbytes} of {full} bytes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    seg = gdr.gdr_prefill_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], cot["d_out"],
                                   initial_state=inp["initial_state"], d_final_state=cot["d_final_state"],
                                   workspace=ws)
    torch.cuda.synchronize()
    for name in NAMES:
        assert torch.equal(seg[name], one[name]), name
    ref = _oracle(inp, cot)
    for name in NAMES:
        assert_close(name, seg[name], ref[name], TOL_BWD)


def test_backward_in_time_segments_without_state_gradients():
    """Segments with no final-state gradient and no initial-state gradient
    requested: the carried gradient starts from zeros, and nothing is written
    for the first segment's incoming state."""
    inp, cot = _small(64, 64, 2, 32 * 36, "channel", torch.bfloat16, False, seed=31)
    one = _gpu(inp, cot, with_final=False, with_init=False)
    nbytes = gdr.gdr_prefill_backward_workspace_bytes(inp["q"], inp["v"], inp["log_alpha"], segment_chunks=16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    seg = gdr.gdr_prefill_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], cot["d_out"],
                                   initial_state=None, d_final_state=None, output_d_initial_state=False, workspace=ws)
    torch.cuda.synchronize()
    for name in NAMES[:-1]:
        assert torch.equal(seg[name], one[name]), name
    assert seg["d_initial_state"] is None


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_backward_in_time_segments_grouped_heads_bf16_gates(gate):
    """Time segments with 2 q/k heads shared by 6 value heads and bf16 gates:
    each value head's dq and dk stay whole-length in the workspace and are
    summed over each group once, after the last segment."""
    w = Workload("small", "backward", heads=6, qk_heads=2, dk=64, dv=64, qkv_dtype=torch.bfloat16, gate=gate,
                 batch=2, seqlen=32 * 35 + 9, init_state=True, seed=33)
    inp = prefill_inputs(w, DEV, gate_dtype=torch.bfloat16)
    cot = backward_cotangents(inp, 33, DEV)
    one = _gpu(inp, cot)
    nbytes = gdr.gdr_prefill_backward_workspace_bytes(inp["q"], inp["v"], inp["log_alpha"], segment_chunks=16)
    assert 0 < nbytes < gdr.gdr_prefill_backward_workspace_bytes(inp["q"], inp["v"], inp["log_alpha"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    seg = gdr.gdr_prefill_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], cot["d_out"],
                                   initial_state=inp["initial_state"], d_final_state=cot["d_final_state"],
                                   workspace=ws)
    torch.cuda.synchronize()
    for name in NAMES:
        assert torch.equal(seg[name], one[name]), name
    ref = _oracle(inp, cot)
    for name in NAMES:
        assert_close(name, seg[name], ref[name], TOL_BWD)
