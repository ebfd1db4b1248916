"""Seeded synthetic inputs for the gated delta-rule recurrence.

This module only draws random numbers; it holds none of the recurrence's
arithmetic.  Both the oracle-side tests and the GPU path take their inputs
from here, so the two see bit-identical stored values.

The pages publish no dataset for this layer, so every input is synthetic with
the shapes the pages' models use (head dimension 128: page "How the New Flash
Models Work: Inside GLM-5.3-Flash and Qwen3.8-Flash-Next", section "The two
stacks, layer by layer"; page "Qwen3.8-Flash-Next and GLM-5.3-Flash share a
3:1 long-context pattern", sections "Gated DeltaNet carries most of the
sequence" and "Kimi Delta Attention extends recurrent memory control").

Recipe (per workload, one seed):
  q, k ~ N(0, 1), L2-normalised over the key dimension per (token, head),
  v ~ N(0, 1), beta = sigmoid(N(0, 1)), log_alpha = -softplus(N(0, 1))
  (one value per (token, head) for per-head decay, one per key channel for
  per-channel decay), initial state ~ N(0, 0.02^2) where asked for.
  Draw order: q, k, v, beta logits, alpha logits, initial state.
  Grouped value heads: q and k are drawn with the query-key head count, v,
  the gates and the states with the value head count.
  Multi-token decode adds, after the states: the slot of each sequence (a
  random choice of distinct slots of the pool), the accepted count of each
  sequence's previous draft (uniform in [0, K - 1]: the tokens its call
  replays and commits) -- so every call reads every state and writes those
  with at least one accepted token.
  The backward adds the loss's gradients with respect to the outputs and the
  final states, d_out ~ N(0, 1) and d_final_state ~ N(0, 1), from a generator
  seeded with the workload's seed + 1000003, so the forward inputs are the
  prefill workload's own.
  Draws are fp32 from torch's seeded generator on the target device; q/k/v are
  then rounded to the storage dtype (bf16 round-to-nearest-even), states stay
  fp32, and gates stay fp32 unless a bf16 gate variant is asked for (then beta
  and log alpha are rounded to bf16 after their fp32 draw).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill", "decode", "prologue" or "backward"
    heads: int
    dk: int
    dv: int
    qkv_dtype: torch.dtype
    gate: str = "head"        # "head" (Gated DeltaNet) or "channel" (Kimi Delta Attention)
    batch: int = 1            # prefill: dense batch; decode: number of sequences
    seqlen: int = 0           # prefill: tokens per sequence (dense) or total (packed)
    chunk: int = 64
    init_state: bool = False
    packed: dict = field(default_factory=dict)   # {"num_seqs", "min_len", "max_len"}
    seed: int = 0
    qk_heads: int = 0         # query-key heads shared by the value heads (0: = heads)
    tokens: int = 1           # decode: tokens per sequence per call
    slots: int = 0            # multi-token decode: state pool slots (0: one per sequence)


WORKLOADS = {
    "tiny_gdn": Workload("tiny_gdn", "prefill", heads=2, dk=16, dv=16, qkv_dtype=torch.float32,
                         gate="head", batch=1, seqlen=64, chunk=16, init_state=False, seed=0),
    "gdn_prefill_8k": Workload("gdn_prefill_8k", "prefill", heads=16, dk=128, dv=128,
                               qkv_dtype=torch.bfloat16, gate="head", batch=1, seqlen=8192,
                               chunk=64, init_state=False, seed=1),
    "kda_prefill_32k": Workload("kda_prefill_32k", "prefill", heads=32, dk=128, dv=128,
                                qkv_dtype=torch.bfloat16, gate="channel", batch=2, seqlen=32768,
                                chunk=64, init_state=True, seed=2),
    "decode_256x32": Workload("decode_256x32", "decode", heads=32, dk=128, dv=128,
                              qkv_dtype=torch.bfloat16, gate="both", batch=256, init_state=True,
                              seed=3),
    "packed_gdn_256k": Workload("packed_gdn_256k", "prefill", heads=16, dk=128, dv=128,
                                qkv_dtype=torch.bfloat16, gate="head", batch=1, seqlen=262144,
                                chunk=64, init_state=True,
                                packed={"num_seqs": 8, "min_len": 4096, "max_len": 61440}, seed=4),
    # the Gated DeltaNet layer shape of the pages' Qwen model: 16 query-key
    # heads shared by 48 value heads of dimension 128
    "gdn_gva_prefill_32k": Workload("gdn_gva_prefill_32k", "prefill", heads=48, qk_heads=16, dk=128, dv=128,
                                    qkv_dtype=torch.bfloat16, gate="head", batch=1, seqlen=32768,
                                    init_state=True, seed=5),
    # speculative decode with that shape: 4 drafted tokens per sequence, the
    # previous draft's accepted tokens replayed and committed in the same call
    "mtp_decode_256x48": Workload("mtp_decode_256x48", "decode", heads=48, qk_heads=16, dk=128, dv=128,
                                  qkv_dtype=torch.bfloat16, gate="head", batch=256, tokens=4, slots=512, seed=6),
    # the backward (training) pass on the two prefill shapes, with an initial
    # state so its gradient is exercised
    "gdn_backward_8k": Workload("gdn_backward_8k", "backward", heads=16, dk=128, dv=128,
                                qkv_dtype=torch.bfloat16, gate="head", batch=1, seqlen=8192,
                                init_state=True, seed=8),
    "kda_backward_32k": Workload("kda_backward_32k", "backward", heads=32, dk=128, dv=128,
                                 qkv_dtype=torch.bfloat16, gate="channel", batch=2, seqlen=32768,
                                 init_state=True, seed=9),
    "gdn_gva_backward_32k": Workload("gdn_gva_backward_32k", "backward", heads=48, qk_heads=16, dk=128, dv=128,
                                     qkv_dtype=torch.bfloat16, gate="head", batch=1, seqlen=32768,
                                     init_state=True, seed=10),
    # the layer prologue on that shape: the 10240 projected q/k/v channels of
    # 32768 tokens, with a convolution state
    "prologue_gdn_32k": Workload("prologue_gdn_32k", "prologue", heads=48, qk_heads=16, dk=128, dv=128,
                                 qkv_dtype=torch.bfloat16, gate="head", batch=1, seqlen=32768, init_state=True,
                                 seed=7),
    # one decode step of that layer fed from its projected channels: the
    # prologue (convolution with its state, q/k norm, gates) fused with the
    # state update, 256 sequences
    "decode_prologue_256x48": Workload("decode_prologue_256x48", "decode", heads=48, qk_heads=16, dk=128, dv=128,
                                       qkv_dtype=torch.bfloat16, gate="head", batch=256, init_state=True, seed=11),
}


def packed_lengths(total: int, num_seqs: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Lengths uniform in [lo, hi] summing to ``total``: draw the first
    num_seqs-1 uniformly, give the rest to the last one, and redraw until the
    last one also lies in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for _ in range(100000):
        head = rng.integers(lo, hi + 1, size=num_seqs - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]]).astype(np.int64)
    raise RuntimeError("length sampler did not converge")


def _unit_norm(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(w: Workload, device="cpu", *, seqlen: int | None = None, batch: int | None = None,
                   heads: int | None = None, lengths=None, gate: str | None = None, seed: int | None = None,
                   init_state: bool | None = None, gate_dtype=torch.float32):
    """Inputs of a prefill workload (optionally resized for tests).

    Returns a dict with q, k, v [B, T, H, d], beta [B, T, H], log_alpha
    [B, T, H] or [B, T, H, dk], initial_state [N, H, dv, dk] or None and
    cu_seqlens (int32 [N+1], packed workloads only).
    """
    B = w.batch if batch is None else batch
    T = w.seqlen if seqlen is None else seqlen
    H = w.heads if heads is None else heads
    Hk = (w.qk_heads or w.heads) if heads is None else H // (w.heads // (w.qk_heads or w.heads))
    gate = w.gate if gate is None else gate
    seed = w.seed if seed is None else seed
    init_state = w.init_state if init_state is None else init_state
    dk, dv = w.dk, w.dv
    cu = None
    if lengths is not None or w.packed:
        if lengths is None:
            p = w.packed
            lengths = packed_lengths(T, p["num_seqs"], p["min_len"], p["max_len"], seed)
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        B = 1
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=device)
        N = len(lengths)
    else:
        N = B
    g = _gen(device, seed)
    f32 = torch.float32
    q = _unit_norm(torch.randn(B, T, Hk, dk, generator=g, device=device, dtype=f32)).to(w.qkv_dtype)
    k = _unit_norm(torch.randn(B, T, Hk, dk, generator=g, device=device, dtype=f32)).to(w.qkv_dtype)
    v = torch.randn(B, T, H, dv, generator=g, device=device, dtype=f32).to(w.qkv_dtype)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=g, device=device, dtype=f32))
    ashape = (B, T, H) if gate == "head" else (B, T, H, dk)
    log_alpha = -torch.nn.functional.softplus(torch.randn(*ashape, generator=g, device=device, dtype=f32))
    s0 = None
    if init_state:
        s0 = 0.02 * torch.randn(N, H, dv, dk, generator=g, device=device, dtype=f32)
    return {"q": q, "k": k, "v": v, "beta": beta.to(gate_dtype), "log_alpha": log_alpha.to(gate_dtype),
            "initial_state": s0, "cu_seqlens": cu}


def backward_cotangents(inp, seed: int, device="cpu"):
    """Gradients of a synthetic loss with respect to the prefill's outputs
    and final states: d_out ~ N(0, 1) with v's shape and d_final_state ~
    N(0, 1) [N, H, dv, dk], fp32 (generator seed: seed + 1000003)."""
    B, T, H, dv = inp["v"].shape
    dk = inp["k"].shape[-1]
    cu = inp["cu_seqlens"]
    N = B if cu is None else cu.numel() - 1
    g = _gen(device, seed + 1000003)
    d_out = torch.randn(B, T, H, dv, generator=g, device=device, dtype=torch.float32)
    d_final = torch.randn(N, H, dv, dk, generator=g, device=device, dtype=torch.float32)
    return {"d_out": d_out, "d_final_state": d_final}


def decode_inputs(w: Workload, device="cpu", *, gate: str = "head", num_seqs: int | None = None,
                  heads: int | None = None, dk: int | None = None, dv: int | None = None,
                  seed: int | None = None, qkv_dtype=None, qk_heads: int | None = None, gate_dtype=torch.float32):
    """One token per sequence: q, k [N, Hk, dk], v [N, H, dv], beta [N, H],
    log_alpha [N, H] or [N, H, dk], state [N, H, dv, dk] (fp32)."""
    N = w.batch if num_seqs is None else num_seqs
    H = w.heads if heads is None else heads
    Hk = qk_heads or (w.qk_heads if heads is None and w.qk_heads else H)
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    dt = w.qkv_dtype if qkv_dtype is None else qkv_dtype
    g = _gen(device, w.seed if seed is None else seed)
    f32 = torch.float32
    q = _unit_norm(torch.randn(N, Hk, dk, generator=g, device=device, dtype=f32)).to(dt)
    k = _unit_norm(torch.randn(N, Hk, dk, generator=g, device=device, dtype=f32)).to(dt)
    v = torch.randn(N, H, dv, generator=g, device=device, dtype=f32).to(dt)
    beta = torch.sigmoid(torch.randn(N, H, generator=g, device=device, dtype=f32))
    ashape = (N, H) if gate == "head" else (N, H, dk)
    log_alpha = -torch.nn.functional.softplus(torch.randn(*ashape, generator=g, device=device, dtype=f32))
    state = 0.02 * torch.randn(N, H, dv, dk, generator=g, device=device, dtype=f32)
    return {"q": q, "k": k, "v": v, "beta": beta.to(gate_dtype), "log_alpha": log_alpha.to(gate_dtype),
            "state": state}


def decode_tokens_inputs(w: Workload, device="cpu", *, gate: str | None = None, num_seqs: int | None = None,
                         heads: int | None = None, qk_heads: int | None = None, tokens: int | None = None,
                         slots: int | None = None, dk: int | None = None, dv: int | None = None,
                         seed: int | None = None, qkv_dtype=None, gate_dtype=torch.float32):
    """Several tokens per sequence from a pool of states: q, k [N, K, Hk, dk],
    v [N, K, H, dv], beta [N, K, H], log_alpha [N, K, H] or [N, K, H, dk],
    state_pool [P, H, dv, dk] (fp32), state_slots [N] (distinct slots, int32),
    num_commit [N] (int32, uniform in [0, K - 1]); num_tokens is left to the
    caller (None: all K)."""
    N = w.batch if num_seqs is None else num_seqs
    H = w.heads if heads is None else heads
    Hk = qk_heads or (w.qk_heads if heads is None and w.qk_heads else H)
    K = w.tokens if tokens is None else tokens
    P = (w.slots or N) if slots is None else slots
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    gate = w.gate if gate is None else gate
    dt = w.qkv_dtype if qkv_dtype is None else qkv_dtype
    g = _gen(device, w.seed if seed is None else seed)
    f32 = torch.float32
    q = _unit_norm(torch.randn(N, K, Hk, dk, generator=g, device=device, dtype=f32)).to(dt)
    k = _unit_norm(torch.randn(N, K, Hk, dk, generator=g, device=device, dtype=f32)).to(dt)
    v = torch.randn(N, K, H, dv, generator=g, device=device, dtype=f32).to(dt)
    beta = torch.sigmoid(torch.randn(N, K, H, generator=g, device=device, dtype=f32))
    ashape = (N, K, H) if gate == "head" else (N, K, H, dk)
    log_alpha = -torch.nn.functional.softplus(torch.randn(*ashape, generator=g, device=device, dtype=f32))
    pool = 0.02 * torch.randn(P, H, dv, dk, generator=g, device=device, dtype=f32)
    slots_ = torch.randperm(P, generator=g, device=device)[:N].to(torch.int32)
    commit = torch.randint(0, K, (N,), generator=g, device=device, dtype=torch.int32)
    return {"q": q, "k": k, "v": v, "beta": beta.to(gate_dtype), "log_alpha": log_alpha.to(gate_dtype),
            "state_pool": pool, "state_slots": slots_, "num_commit": commit}


def prologue_inputs(w: Workload, device="cpu", *, seqlen: int | None = None, batch: int | None = None,
                    heads: int | None = None, qk_heads: int | None = None, dk: int | None = None,
                    dv: int | None = None, lengths=None, gate: str | None = None, seed: int | None = None,
                    init_state: bool | None = None, x_dtype=None):
    """Inputs of the layer prologue: x [B, T, C] (C = 2 Hk dk + H dv) ~ N(0, 1)
    in x_dtype, convolution taps [C, 4] ~ N(0, 0.5^2) (fp32), gate logits
    a [B, T, H(, dk)] and b [B, T, H] ~ N(0, 1) (fp32), a convolution state
    [N, 3, C] ~ N(0, 1) when asked for, cu_seqlens for packed lengths.
    Draw order: x, taps, a, b, state."""
    B = w.batch if batch is None else batch
    T = w.seqlen if seqlen is None else seqlen
    H = w.heads if heads is None else heads
    if qk_heads:
        Hk = qk_heads
    else:
        Hk = (w.qk_heads or w.heads) if heads is None else H
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    gate = w.gate if gate is None else gate
    dt = w.qkv_dtype if x_dtype is None else x_dtype
    init_state = w.init_state if init_state is None else init_state
    cu = None
    N = B
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        T, B, N = int(lengths.sum()), 1, len(lengths)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=device)
    C = 2 * Hk * dk + H * dv
    g = _gen(device, w.seed if seed is None else seed)
    f32 = torch.float32
    x = torch.randn(B, T, C, generator=g, device=device, dtype=f32).to(dt)
    wt = 0.5 * torch.randn(C, 4, generator=g, device=device, dtype=f32)
    ashape = (B, T, H) if gate == "head" else (B, T, H, dk)
    a = torch.randn(*ashape, generator=g, device=device, dtype=f32)
    b = torch.randn(B, T, H, generator=g, device=device, dtype=f32)
    st = torch.randn(N, 3, C, generator=g, device=device, dtype=f32).to(dt) if init_state else None
    return {"x": x, "conv_weight": wt, "a_logit": a, "b_logit": b, "conv_state": st, "cu_seqlens": cu,
            "num_qk_heads": Hk, "head_dim_k": dk, "head_dim_v": dv}


def decode_prologue_inputs(w: Workload, device="cpu", *, num_seqs: int | None = None, steps: int = 1,
                           heads: int | None = None, qk_heads: int | None = None, dk: int | None = None,
                           dv: int | None = None, gate: str | None = None, seed: int | None = None,
                           init_conv_state: bool = True, x_dtype=None):
    """Decode steps fed from projected channels: the prologue inputs of
    ``steps`` tokens per sequence (x [N, steps, C], taps, gate logits and a
    convolution state, drawn as by prologue_inputs) and a recurrent state
    [N, H, dv, dk] ~ N(0, 0.02^2) drawn after them."""
    N = w.batch if num_seqs is None else num_seqs
    H = w.heads if heads is None else heads
    Hk = qk_heads or (w.qk_heads if heads is None and w.qk_heads else H)
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    s = w.seed if seed is None else seed
    p = prologue_inputs(w, device, seqlen=steps, batch=N, heads=H, qk_heads=Hk, dk=dk, dv=dv, gate=gate, seed=s,
                        init_state=init_conv_state, x_dtype=x_dtype)
    g = _gen(device, s + 7919)
    p["state"] = 0.02 * torch.randn(N, H, dv, dk, generator=g, device=device, dtype=torch.float32)
    return p
