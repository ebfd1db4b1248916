"""Chunked prefill on the GPU vs the fp64 oracle (sequential recurrence)."""
import pytest
import torch

import gated_delta_rule_73_amd as gdr
import oracle
from parity import TOL, assert_close, assert_close_rounded, gpu_available, say, to_np
from workloads import WORKLOADS, Workload, packed_lengths, prefill_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]
DEV = "cuda"


def _gpu(inp, **kw):
    out, fin = gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                       initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return out, fin


def _oracle(inp):
    cu = inp["cu_seqlens"]
    return oracle.recurrence(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                             initial_state=inp["initial_state"],
                             seq_bounds=None if cu is None else cu.cpu().numpy())


def _check_all(inp, label, **kw):
    say(f"prefill {label} {kw}")
    out, fin = _gpu(inp, **kw)
    ref_o, ref_s = _oracle(inp)
    tol = TOL[inp["q"].dtype]
    assert_close("out", out, ref_o, tol)
    assert_close("final_state", fin, ref_s, tol)
    return out, fin


def _small(dk, dv, H, T, gate, dtype, init, seed, B=1, lengths=None, Hk=0):
    w = Workload("small", "prefill", heads=H, dk=dk, dv=dv, qkv_dtype=dtype, gate=gate, batch=B, seqlen=T,
                 init_state=init, seed=seed, qk_heads=Hk)
    return prefill_inputs(w, DEV, lengths=lengths)


# ------------------------------------------------------------ workloads ----
def test_tiny_gdn_workload():
    """B=1, H=2, T=64, d=16, fp32, chunk 16, zero initial state."""
    w = WORKLOADS["tiny_gdn"]
    _check_all(prefill_inputs(w, DEV), "tiny_gdn", chunk_size=w.chunk)


def test_gdn_prefill_8k_workload():
    """B=1, H=16, T=8192, d=128, bf16 q/k/v, per-head decay, chunk size 64 as
    the workload states."""
    w = WORKLOADS["gdn_prefill_8k"]
    _check_all(prefill_inputs(w, DEV), "gdn_prefill_8k", chunk_size=64)


@pytest.mark.slow
def test_kda_prefill_32k_workload():
    """B=2, H=32, T=32768, d=128, bf16, per-channel decay, S0 ~ N(0, 0.02^2):
    every element of out and final_state against the oracle (all host cores)."""
    w = WORKLOADS["kda_prefill_32k"]
    _check_all(prefill_inputs(w, DEV), "kda_prefill_32k (whole tensors)")


@pytest.mark.slow
def test_kda_prefill_32k_workload_chunk64():
    """The same workload with 64-token chunks (the two-kernel path's
    four-block inverse and split chain slots over 512 chunks per sequence):
    whole tensors against the oracle."""
    w = WORKLOADS["kda_prefill_32k"]
    _check_all(prefill_inputs(w, DEV), "kda_prefill_32k, chunk 64 (whole tensors)", chunk_size=64)


@pytest.mark.slow
def test_packed_gdn_256k_workload_chunk64():
    """Packed sequences of ragged lengths with 64-token chunks."""
    w = WORKLOADS["packed_gdn_256k"]
    _check_all(prefill_inputs(w, DEV), "packed_gdn_256k, chunk 64 (whole tensors)", chunk_size=64)


@pytest.mark.slow
def test_packed_gdn_256k_workload():
    """262144 tokens as 8 packed sequences (4096..61440 each), H=16, d=128."""
    w = WORKLOADS["packed_gdn_256k"]
    _check_all(prefill_inputs(w, DEV), "packed_gdn_256k (whole tensors)")


@pytest.mark.slow
def test_gdn_gva_prefill_32k_workload():
    """B=1, T=32768, 16 query-key heads shared by 48 value heads, d=128,
    bf16, per-head decay, S0 ~ N(0, 0.02^2): every element of out and
    final_state against the oracle."""
    w = WORKLOADS["gdn_gva_prefill_32k"]
    _check_all(prefill_inputs(w, DEV), "gdn_gva_prefill_32k (whole tensors)")


# -------------------------------------------------------- shape sweeps ----
BF16_CASES = [
    # dk, dv, H, T, gate, init, chunk, dv_slice
    (128, 128, 2, 1, "head", False, 32, 32),
    (128, 128, 2, 31, "channel", True, 32, 32),
    (128, 128, 1, 32, "head", True, 32, 16),
    (128, 128, 3, 33, "channel", False, 32, 16),
    (128, 128, 2, 197, "head", True, 32, 32),
    (128, 128, 2, 197, "channel", True, 32, 16),
    (128, 64, 1, 300, "channel", True, 32, 32),
    (64, 64, 3, 130, "head", True, 32, 32),
    (64, 32, 2, 129, "channel", True, 32, 16),
    (32, 32, 1, 95, "head", False, 32, 32),
    (32, 48, 2, 100, "channel", True, 32, 16),
    (32, 48, 2, 100, "head", True, 32, 16),
    (128, 128, 2, 197, "channel", True, 32, 64),
    (128, 128, 3, 95, "head", False, 32, 64),
    (128, 64, 2, 130, "channel", True, 32, 64),
]


@pytest.mark.parametrize("dk,dv,H,T,gate,init,chunk,dvs", BF16_CASES)
def test_prefill_bf16_shapes(dk, dv, H, T, gate, init, chunk, dvs):
    inp = _small(dk, dv, H, T, gate, torch.bfloat16, init, seed=dk + dv + T + H)
    _check_all(inp, f"bf16 dk={dk} dv={dv} H={H} T={T} {gate} init={init}", chunk_size=chunk, dv_slice=dvs)


# 64-token chunks: the same two kernels with the UT inverse over four 16-token
# blocks and the chain's split record slots
CHUNK64_CASES = [
    # dk, dv, H, T, gate, init, dv_slice (0: automatic)
    (128, 128, 2, 1, "head", False, 0),
    (128, 128, 2, 63, "channel", True, 32),
    (128, 128, 1, 64, "head", True, 16),
    (128, 128, 3, 65, "channel", False, 16),
    (128, 128, 2, 200, "head", True, 32),
    (128, 128, 2, 513, "channel", True, 0),
    (128, 64, 1, 300, "channel", True, 32),
    (128, 16, 2, 129, "head", True, 16),
    (64, 64, 3, 130, "head", True, 32),
    (64, 32, 2, 129, "channel", True, 16),
    (64, 48, 2, 191, "channel", True, 16),
    (32, 32, 1, 95, "head", False, 32),
    (32, 48, 2, 100, "channel", True, 16),
    (32, 128, 2, 257, "head", True, 0),
]


@pytest.mark.parametrize("dk,dv,H,T,gate,init,dvs", CHUNK64_CASES)
def test_prefill_chunk64_shapes(dk, dv, H, T, gate, init, dvs):
    inp = _small(dk, dv, H, T, gate, torch.bfloat16, init, seed=3 * dk + dv + T + H)
    _check_all(inp, f"chunk 64 dk={dk} dv={dv} H={H} T={T} {gate} init={init} dvs={dvs}", chunk_size=64, dv_slice=dvs)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_chunk64_more_units_than_workgroups(gate):
    """300 heads of 32 value channels at 64-token chunks: more chain
    workgroups than the device holds at once, so they run in several rounds."""
    inp = _small(64, 32, 300, 70, gate, torch.bfloat16, True, seed=301)
    _check_all(inp, f"chunk 64, 300 heads {gate}", chunk_size=64)


def test_prefill_chunk64_workspace_reuse_and_scale():
    """Two different calls through one caller workspace, then a readout scale:
    o(s) = s o(1)."""
    a = _small(128, 128, 4, 333, "channel", torch.bfloat16, True, seed=311)
    b = _small(128, 128, 4, 97, "head", torch.bfloat16, False, seed=312)
    ws = torch.empty(32 << 20, dtype=torch.uint8, device=DEV)      # more than either call needs
    for inp, label in ((a, "first"), (b, "second"), (a, "first again")):
        _check_all(inp, f"workspace reuse: {label}", chunk_size=64, workspace=ws)
    ref_o, ref_s = _oracle(a)
    o, s = _gpu(a, chunk_size=64, scale=0.37)
    assert_close("out (scale 0.37)", o, 0.37 * ref_o, TOL[torch.bfloat16])
    assert_close("final_state (scale only reads out)", s, ref_s, TOL[torch.bfloat16])


F32_CASES = [
    (16, 16, 2, 1, "head", False, 16),
    (16, 16, 2, 17, "channel", True, 16),
    (32, 16, 1, 15, "head", True, 16),
    (32, 32, 2, 70, "channel", True, 32),
    (64, 48, 1, 33, "head", True, 32),
    (128, 64, 2, 100, "channel", True, 16),
    (128, 32, 1, 16, "head", False, 16),
    (128, 32, 1, 77, "head", True, 32),
    (64, 16, 2, 64, "channel", True, 32),
]


@pytest.mark.parametrize("dk,dv,H,T,gate,init,chunk", F32_CASES)
def test_prefill_f32_shapes(dk, dv, H, T, gate, init, chunk):
    inp = _small(dk, dv, H, T, gate, torch.float32, init, seed=7 * dk + T)
    _check_all(inp, f"fp32 dk={dk} dv={dv} H={H} T={T} {gate}", chunk_size=chunk)


GROUPED_CASES = [
    # dk, dv, H, Hk, T, gate, dtype
    (128, 128, 6, 2, 197, "head", torch.bfloat16),
    (128, 128, 6, 2, 130, "channel", torch.bfloat16),
    (64, 64, 3, 1, 100, "head", torch.bfloat16),
    (128, 64, 8, 4, 64, "channel", torch.bfloat16),
    (32, 32, 4, 2, 70, "channel", torch.float32),
    (64, 48, 6, 3, 45, "head", torch.float32),
]


@pytest.mark.parametrize("dk,dv,H,Hk,T,gate,dtype", GROUPED_CASES)
def test_prefill_grouped_value_heads(dk, dv, H, Hk, T, gate, dtype):
    """Hk query-key heads shared by groups of H / Hk consecutive value heads."""
    inp = _small(dk, dv, H, T, gate, dtype, True, seed=dk + H + T, Hk=Hk)
    assert inp["q"].shape[2] == Hk and inp["v"].shape[2] == H
    _check_all(inp, f"grouped H={H} Hk={Hk} dk={dk} dv={dv} T={T} {gate} {dtype}")


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_bf16_gates(gate):
    """beta and log alpha stored in bf16 (the oracle reads the same bf16 values)."""
    w = Workload("small", "prefill", heads=4, qk_heads=2, dk=128, dv=128, qkv_dtype=torch.bfloat16, gate=gate,
                 batch=2, seqlen=197, init_state=True, seed=81)
    inp = prefill_inputs(w, DEV, gate_dtype=torch.bfloat16)
    assert inp["beta"].dtype == inp["log_alpha"].dtype == torch.bfloat16
    _check_all(inp, f"bf16 gates {gate}")
    w1 = Workload("small", "prefill", heads=2, dk=64, dv=64, qkv_dtype=torch.bfloat16, gate=gate, batch=2,
                  seqlen=100, init_state=True, seed=82)
    _check_all(prefill_inputs(w1, DEV, gate_dtype=torch.bfloat16), f"bf16 gates ungrouped {gate}")


@pytest.mark.parametrize("chunk", [0, 64])
def test_prefill_grouped_packed(chunk):
    lens = [33, 0, 100, 7]
    inp = _small(128, 128, 4, 0, "channel", torch.bfloat16, True, seed=71, lengths=lens, Hk=2)
    _check_all(inp, f"grouped packed {lens}", chunk_size=chunk)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_chunk64_grouped_bf16_gates_packed(gate):
    """64-token chunks with value heads sharing q/k heads, bf16 gates, and a
    packed batch holding empty, one-token and ragged sequences."""
    w = Workload("small", "prefill", heads=6, qk_heads=2, dk=64, dv=64, qkv_dtype=torch.bfloat16, gate=gate,
                 batch=1, seqlen=0, init_state=True, seed=83)
    lens = [130, 0, 1, 64, 65, 0, 257]
    inp = prefill_inputs(w, DEV, gate_dtype=torch.bfloat16, lengths=lens)
    _, fin = _check_all(inp, f"chunk 64, grouped, bf16 gates, packed {lens} {gate}", chunk_size=64)
    assert torch.equal(fin[1], inp["initial_state"][1]) and torch.equal(fin[5], inp["initial_state"][5])


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_dense_batch(gate):
    inp = _small(128, 128, 3, 150, gate, torch.bfloat16, True, seed=31, B=3)
    _check_all(inp, f"dense B=3 {gate}")


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_packed_with_empty_and_ragged(gate):
    lens = [70, 0, 1, 129, 64, 0, 200]
    inp = _small(128, 64, 2, 0, gate, torch.bfloat16, True, seed=41, lengths=lens)
    _, fin = _check_all(inp, f"packed {lens} {gate}")
    assert torch.equal(fin[1], inp["initial_state"][1]) and torch.equal(fin[5], inp["initial_state"][5])


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_segments(gate):
    """A workspace smaller than the one-pass size: the dense batch runs in
    segments (here 64 chunks, the last one partial) with the state carried
    between them; outputs and states match the one-pass run bit for bit."""
    T = 64 * 32 * 2 + 77                                   # 131 chunks -> segments 64, 64, 3
    inp = _small(64, 64, 2, T, gate, torch.bfloat16, True, seed=61, B=2)
    out, fin = _check_all(inp, f"one pass {gate}", chunk_size=32)
    rec = -(-((64 * 4 if gate == "channel" else 16) + (3 * 32 * 64 + 2 * 32 * 32) * 2) // 256) * 256
    ws_bytes = 2 * 64 * 2 * rec + 2 * 2 * 64 * 64 * 4   # records of one 64-chunk segment + carried state
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    say("segments of 64 chunks; then in place; then without the final state")
    o1, f1 = _gpu(inp, workspace=ws, chunk_size=32)
    state = inp["initial_state"].clone()
    o2, _ = gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                    initial_state=state, final_state=state, workspace=ws, chunk_size=32)
    o3, f3 = gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                     initial_state=inp["initial_state"], output_final_state=False, workspace=ws,
                                     chunk_size=32)
    torch.cuda.synchronize()
    assert f3 is None
    for o in (o1, o2, o3):
        assert torch.equal(o, out)
    assert torch.equal(f1, fin) and torch.equal(state, fin)
    with pytest.raises(gdr.GdrError, match="workspace"):
        gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                workspace=ws[: 2 * 15 * 2 * rec], chunk_size=32)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_segments_chunk64(gate):
    """The same at 64-token chunks (d_k = 128, the two-kernel path): 130
    chunks in segments of 64, 64 and 2 match the one-pass run bit for bit."""
    T = 64 * 64 * 2 + 77
    inp = _small(128, 128, 2, T, gate, torch.bfloat16, True, seed=67, B=2)
    out, fin = _check_all(inp, f"one pass, chunk 64, {gate}", chunk_size=64)
    rec = -(-((128 * 4 if gate == "channel" else 16) + (3 * 64 * 128 + 2 * 64 * 64) * 2) // 256) * 256
    ws = torch.empty(2 * 64 * 2 * rec + 2 * 2 * 128 * 128 * 4, dtype=torch.uint8, device=DEV)
    say("segments of 64 chunks of 64 tokens")
    o1, f1 = _gpu(inp, workspace=ws, chunk_size=64)
    assert torch.equal(o1, out) and torch.equal(f1, fin)


# ------------------------------------------------------- GPU properties ----
def test_prefill_deterministic():
    inp = _small(128, 128, 2, 333, "channel", torch.bfloat16, True, seed=51)
    o1, s1 = _gpu(inp)
    o2, s2 = _gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_slice_invariance(gate):
    inp = _small(128, 128, 2, 256, gate, torch.bfloat16, True, seed=52)
    ref_o, ref_s = _oracle(inp)
    for dvs in (16, 32):
        say(f"dv_slice {dvs}")
        o, s = _gpu(inp, dv_slice=dvs)
        assert_close("out", o, ref_o, TOL[torch.bfloat16])
        assert_close("final_state", s, ref_s, TOL[torch.bfloat16])


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_chunk_invariance_fp32(gate):
    inp = _small(64, 32, 2, 150, gate, torch.float32, True, seed=56)
    ref_o, ref_s = _oracle(inp)
    for chunk in (16, 32):
        say(f"chunk {chunk}")
        o, s = _gpu(inp, chunk_size=chunk)
        assert_close("out", o, ref_o, TOL[torch.float32])
        assert_close("final_state", s, ref_s, TOL[torch.float32])


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_chunk_invariance_bf16(gate):
    """32- and 64-token chunks compute the same function: each within the bf16
    bound of the oracle, and within that bound of each other."""
    inp = _small(128, 128, 3, 333, gate, torch.bfloat16, True, seed=57)
    ref_o, ref_s = _oracle(inp)
    got = {}
    for chunk in (32, 64):
        say(f"chunk {chunk}")
        got[chunk] = _gpu(inp, chunk_size=chunk)
        assert_close("out", got[chunk][0], ref_o, TOL[torch.bfloat16])
        assert_close("final_state", got[chunk][1], ref_s, TOL[torch.bfloat16])
    assert_close("out, chunk 64 vs 32", got[64][0], to_np(got[32][0]), TOL[torch.bfloat16])


def test_prefill_in_place_state_and_poisoned_output():
    inp = _small(128, 128, 2, 100, "head", torch.bfloat16, True, seed=53)
    ref_o, ref_s = _oracle(inp)
    state = inp["initial_state"].clone()
    out = torch.full(inp["v"].shape, float("nan"), dtype=torch.float32, device=DEV)
    gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], initial_state=state,
                            out=out, final_state=state)
    torch.cuda.synchronize()
    assert_close("out", out, ref_o, TOL[torch.bfloat16])
    assert_close("final_state (in place)", state, ref_s, TOL[torch.bfloat16])


@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("chunk", [0, 64])
def test_prefill_bf16_output(gate, chunk):
    inp = _small(128, 128, 2, 190, gate, torch.bfloat16, True, seed=55)
    ref_o, ref_s = _oracle(inp)
    out, fin = _gpu(inp, out_dtype=torch.bfloat16, chunk_size=chunk)
    assert out.dtype == torch.bfloat16
    assert_close_rounded("out (bf16)", out, ref_o, TOL[torch.bfloat16])
    assert_close("final_state", fin, ref_s, TOL[torch.bfloat16])


def test_prefill_continuation_then_decode():
    """prefill(x[:T1]) -> prefill(x[T1:T2], S) -> decode steps: every piece
    matches the oracle's single pass over the whole sequence (the prefill's
    final state is the decode step's input, unchanged in layout)."""
    T, T1, T2 = 200, 77, 190
    inp = _small(128, 128, 2, T, "channel", torch.bfloat16, True, seed=54)
    ref_o, ref_s = _oracle(inp)
    part = lambda a, b: {**{k_: inp[k_][:, a:b].contiguous() for k_ in ("q", "k", "v", "beta", "log_alpha")},
                         "cu_seqlens": None}
    o1, s1 = _gpu({**part(0, T1), "initial_state": inp["initial_state"]})
    o2, s2 = _gpu({**part(T1, T2), "initial_state": s1})
    outs = [o1, o2]
    state = s2
    for t in range(T2, T):
        o = gdr.gdr_decode_step(inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(), inp["v"][:, t].contiguous(),
                                inp["beta"][:, t].contiguous(), inp["log_alpha"][:, t].contiguous(), state)
        outs.append(o[:, None])
    torch.cuda.synchronize()
    assert_close("out", torch.cat(outs, dim=1), ref_o, TOL[torch.bfloat16])
    assert_close("final_state", state, ref_s, TOL[torch.bfloat16])


# ------------------------------------------------------------ edge cases ----
@pytest.mark.parametrize("dk,dv,gate,Hk", [(128, 256, "channel", 0), (128, 256, "head", 2), (32, 256, "head", 0),
                                           (64, 208, "channel", 0)])
def test_prefill_largest_value_dims(dk, dv, gate, Hk):
    """head_dim_v up to its limit (256: eight 32-channel slices)."""
    inp = _small(dk, dv, 4, 150, gate, torch.bfloat16, True, seed=90 + dv, Hk=Hk)
    _check_all(inp, f"dk={dk} dv={dv} {gate} Hk={Hk}")


def test_prefill_empty_dense_batch_keeps_the_state():
    """T = 0: no outputs, and the final state is the initial state exactly."""
    inp = _small(128, 128, 3, 0, "channel", torch.bfloat16, True, seed=95, B=2)
    out, fin = _gpu(inp)
    assert out.numel() == 0
    assert torch.equal(fin, inp["initial_state"])


def test_prefill_one_chunk_ragged():
    for T in (5, 31, 32, 33):
        inp = _small(128, 128, 2, T, "channel", torch.bfloat16, True, seed=96 + T)
        _check_all(inp, f"T={T}")


@pytest.mark.slow
def test_prefill_long_single_sequence():
    """One sequence of 65536 tokens (2048 chunks on one chain), 4 heads."""
    w = Workload("long", "prefill", heads=4, dk=128, dv=128, qkv_dtype=torch.bfloat16, gate="channel", batch=1,
                 seqlen=65536, init_state=True, seed=97)
    _check_all(prefill_inputs(w, DEV), "long single sequence (whole tensors)")


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("edge", ["low", "high"])
def test_prefill_bf16_operand_range_edges(edge, gate, chunk):
    """The bf16 prefill carries v and the state into its products as fp16.
    At both documented edges of their range it still meets the bound: v and
    S0 scaled down by 1e-4 (RMS of v 1e-4: fp16 subnormals begin at 6.1e-5),
    and scaled up until the largest |v| is 60000 (fp16's largest finite value
    is 65504; the state stays below it here)."""
    inp = _small(128, 128, 2, 1024, gate, torch.bfloat16, True, seed=300 + chunk + (gate == "head"))
    if edge == "low":
        s = 1e-4
    else:
        s = 60000.0 / float(inp["v"].float().abs().max())
    inp["v"] = (inp["v"].float() * s).to(torch.bfloat16)
    inp["initial_state"] = inp["initial_state"] * s
    say(f"  v scaled by {s:.4g}: max|v| = {float(inp['v'].float().abs().max()):.4g}")
    _check_all(inp, f"operand range {edge} {gate}", chunk_size=chunk)
