"""Decode step on the GPU vs the fp64 oracle (the recurrence with T = 1)."""
import pytest
import torch

import gated_delta_rule_73_amd as gdr
import oracle
from parity import TOL, assert_close, assert_close_rounded, gpu_available, say
from workloads import WORKLOADS, decode_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]
DEV = "cuda"


def _run_and_check(inp, dtype, label):
    say(f"decode {label}")
    state_ref = inp["state"].clone()
    out = gdr.gdr_decode_step(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["state"])
    torch.cuda.synchronize()
    ref_o, ref_s = oracle.decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], state_ref)
    assert_close("out", out, ref_o, TOL[dtype])
    assert_close("state", inp["state"], ref_s, TOL[dtype])


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_decode_full_workload(gate):
    """256 sequences x 32 heads, 128 x 128 fp32 states, bf16 q/k/v."""
    w = WORKLOADS["decode_256x32"]
    _run_and_check(decode_inputs(w, DEV, gate=gate), torch.bfloat16, f"256x32x128 {gate}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 20), (64, 64), (128, 4), (128, 200)])
def test_decode_small_shapes(dtype, gate, dk, dv):
    w = WORKLOADS["decode_256x32"]
    inp = decode_inputs(w, DEV, gate=gate, num_seqs=5, heads=3, dk=dk, dv=dv, seed=100 + dk + dv, qkv_dtype=dtype)
    _run_and_check(inp, dtype, f"N=5 H=3 dk={dk} dv={dv} {gate} {dtype}")


def test_decode_deterministic_and_scale():
    w = WORKLOADS["decode_256x32"]
    inp = decode_inputs(w, DEV, gate="channel", num_seqs=64, heads=8, seed=7)
    s1, s2 = inp["state"].clone(), inp["state"].clone()
    o1 = gdr.gdr_decode_step(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], s1)
    o2 = gdr.gdr_decode_step(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], s2, scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal((o1.float() * 0.5).to(o1.dtype), o2)  # halving is exact in bf16


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_decode_bf16_output(gate):
    """bf16 outputs: the oracle's value up to one bf16 rounding."""
    w = WORKLOADS["decode_256x32"]
    inp = decode_inputs(w, DEV, gate=gate, num_seqs=64, heads=32, seed=9)
    state_ref = inp["state"].clone()
    out = gdr.gdr_decode_step(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["state"],
                              out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref_o, ref_s = oracle.decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], state_ref)
    assert out.dtype == torch.bfloat16
    assert_close_rounded("out (bf16)", out, ref_o, TOL[torch.bfloat16])
    assert_close("state", inp["state"], ref_s, TOL[torch.bfloat16])


def test_decode_poisoned_output_fully_written():
    w = WORKLOADS["decode_256x32"]
    inp = decode_inputs(w, DEV, gate="head", num_seqs=9, heads=5, seed=8)
    out = torch.full((9, 5, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    gdr.gdr_decode_step(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["state"], out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_decode_steps_match_oracle_prefill():
    """k decode steps from a state = the oracle's prefill of those k tokens."""
    w = WORKLOADS["decode_256x32"]
    steps = [decode_inputs(w, DEV, gate="channel", num_seqs=4, heads=2, seed=200 + i) for i in range(6)]
    state = steps[0]["state"].clone()
    s0 = state.clone()
    outs = []
    for st in steps:
        outs.append(gdr.gdr_decode_step(st["q"], st["k"], st["v"], st["beta"], st["log_alpha"], state))
    torch.cuda.synchronize()
    cat = lambda key: torch.stack([s[key] for s in steps], dim=1)
    ref_o, ref_s = oracle.recurrence(cat("q"), cat("k"), cat("v"), cat("beta"), cat("log_alpha"), initial_state=s0)
    assert_close("out", torch.stack(outs, dim=1), ref_o, TOL[torch.bfloat16])
    assert_close("state", state, ref_s, TOL[torch.bfloat16])
