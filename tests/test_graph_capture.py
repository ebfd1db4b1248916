"""The library's calls inside a captured HIP graph: they allocate nothing and
never synchronise, so a serving loop can capture a decode step and replay
it.  Each replay is checked against the same calls run eagerly, with eager
work and synchronisations between the replays."""
import pytest
import torch

import gated_delta_rule_73_amd as gdr
from parity import gpu_available, say
from workloads import WORKLOADS, Workload, backward_cotangents, decode_inputs, decode_tokens_inputs, prefill_inputs, \
    prologue_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]
DEV = "cuda"


def test_decode_calls_replay_in_a_graph():
    d = decode_inputs(WORKLOADS["decode_256x32"], DEV, gate="channel", num_seqs=32, heads=8, seed=500)
    m = decode_tokens_inputs(WORKLOADS["mtp_decode_256x48"], DEV, num_seqs=16, slots=24, seed=501)
    pi = prologue_inputs(WORKLOADS["prologue_gdn_32k"], DEV, seqlen=1, batch=16, heads=6, qk_heads=2, seed=502)
    state0, pool0, conv0 = d["state"].clone(), m["state_pool"].clone(), pi["conv_state"].clone()
    o1 = torch.empty(32, 8, 128, device=DEV)
    o2 = torch.empty(16, 4, 48, 128, device=DEV)

    def step():
        gdr.gdr_decode_step(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["state"], out=o1)
        gdr.gdr_decode_tokens(m["q"], m["k"], m["v"], m["beta"], m["log_alpha"], m["state_pool"], out=o2,
                              num_commit=m["num_commit"], state_slots=m["state_slots"])
        return gdr.gdr_layer_prologue(pi["x"], pi["conv_weight"], pi["a_logit"], pi["b_logit"],
                                      num_qk_heads=2, head_dim_k=128, head_dim_v=128, conv_state=pi["conv_state"])

    # eager reference: three steps from the saved states
    ref = []
    for _ in range(3):
        q, *_ = step()
        torch.cuda.synchronize()
        ref.append((o1.clone(), o2.clone(), q.clone(), d["state"].clone(), m["state_pool"].clone(),
                    pi["conv_state"].clone()))
    # capture one step (from a side stream, as torch requires), then replay from the same start
    d["state"].copy_(state0)
    m["state_pool"].copy_(pool0)
    pi["conv_state"].copy_(conv0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        saved = (d["state"].clone(), m["state_pool"].clone(), pi["conv_state"].clone())
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            qg, *_ = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # capture does not run the work; put the states back to the start anyway
    d["state"].copy_(saved[0])
    m["state_pool"].copy_(saved[1])
    pi["conv_state"].copy_(saved[2])
    torch.cuda.synchronize()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device=DEV).sum().item()      # eager work between replays
        got = (o1, o2, qg, d["state"], m["state_pool"], pi["conv_state"])
        for name, a, b in zip(("decode out", "multi-token out", "prologue q", "state", "pool", "conv state"),
                              got, ref[i]):
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager run"
        say(f"replay {i}: identical to the eager step")


def test_training_step_forward_and_backward_replay_in_a_graph():
    """A prefill and its backward captured together (their outputs and
    workspaces come from the graph's own pool) replay identically to the
    eager calls, with eager calls and synchronisations between the replays."""
    w = Workload("small", "backward", heads=4, dk=128, dv=128, qkv_dtype=torch.bfloat16, gate="channel", batch=2,
                 seqlen=100, init_state=True, seed=503)
    inp = prefill_inputs(w, DEV)
    cot = backward_cotangents(inp, 503, DEV)

    def step():
        out, fin = gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                           initial_state=inp["initial_state"])
        g = gdr.gdr_prefill_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], cot["d_out"],
                                     initial_state=inp["initial_state"], d_final_state=cot["d_final_state"])
        return [out, fin] + [g[n] for n in ("dq", "dk", "dv", "dbeta", "dlog_alpha", "d_initial_state")]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(gr, stream=s):
            captured = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(3):
        for t in captured:
            t.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        step()                                   # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(captured, eager):
            assert torch.equal(a, b), f"replay {i}"
        say(f"  replay {i}: forward and backward identical to the eager calls")
