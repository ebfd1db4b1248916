"""Benchmark of the gated delta-rule hot path on one MI355X.

One step = one chunked prefill of the Kimi-Delta-Attention workload
(B=2, T=32768, H=32, d=128, bf16 q/k/v, fp32 gates and state) followed by one
decode step of 256 sequences x 32 heads (128x128 fp32 states, in place) with
per-head decay and one with per-channel decay.  Prints one JSON line.

Further workloads are timed in their own loops and reported beside the step
(not part of `value`):
- the per-head-decay prefill at T=8192, cache-warm and with a 512 MiB write
  between calls (its ~170 MB working set otherwise stays in the 256 MB
  last-level cache);
- the packed batch of 8 sequences (262144 tokens);
- the grouped-head Gated DeltaNet prefill (16 query-key heads shared by 48
  value heads, T=32768);
- the speculative multi-token decode over a pool of state slots (256
  sequences x 48 value heads, 4 tokens each, a per-sequence committed prefix);
- the layer prologue on the grouped shape (T=32768, 10240 channels);
- one decode step of that layer fed from its projected channels, the fused
  call (prologue and state update in one kernel) beside the two calls it
  replaces.
Two measured ceilings of the same GPU are reported with them: a large bf16
GEMM (the library GEMM, for the MFMA side) and a 512 MiB read-modify-write
(for the HBM side).

value = prefill throughput (B*T tokens, all heads) in Mtok/s.  Times come from
HIP events on the stream the kernels are launched on, over the timed steps.
One prefill call is two kernels (the per-chunk record kernel and the chain
kernel).  The roofline object reports the call against the bf16 MFMA roof:
the algorithmic flops of the chunked form's dense products at the chunk size
used (stated as "chunk"), divided by the call's time.  HBM is reported beside
it on the call's algorithmic bytes, counting bf16 outputs (and the fp32
outputs the headline writes), with the measured HBM traffic of both kernels.
cpu_baseline times the fp64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA
PROFILE_PMC = os.path.join(ROOT, "profiles", "prefill_kda_32k_traffic.json")
# the sources that define the headline prefill's two kernels and their launch
KERNEL_SOURCES = ["prefill_impl.h", "prefill_shapes.h", "prefill_bf16_kda.hip", "prefill.hip", "common.h"]


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (a comment edit does not
    change the kernels the counters describe)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_73_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def prefill_alg_bytes(B, T, H, dk, dv, kda, out_bytes, init_state=True, final_state=True, Hk=None, gate_bytes=4):
    tok = B * T * H
    b = B * T * (H if Hk is None else Hk) * 2 * dk * 2   # q, k (bf16; shared by value-head groups)
    b += tok * dv * 2                            # v (bf16)
    b += tok * gate_bytes                        # beta
    b += tok * (dk if kda else 1) * gate_bytes   # log alpha
    b += tok * dv * out_bytes                    # out
    b += (int(init_state) + int(final_state)) * B * H * dv * dk * 4
    return b


def prefill_alg_flops(B, T, H, dk, dv, C):
    # dense chunk products of the chunked form, full C x C tiles
    return B * T * H * (4 * C * (dk + dv) + 6 * dk * dv)


def backward_alg_bytes(B, T, H, dk, dv, kda, N, qkv_bytes=2, init_state=True, Hk=None):
    """Bytes the backward must move once: q, k, v, beta, log alpha and d_out
    in; dq, dk, dv, dbeta, dlog alpha out (fp32); the initial state and the
    final-state gradient in, the initial-state gradient out.  q, k and their
    gradients come once per q/k head (Hk of them)."""
    Hk = H if Hk is None else Hk
    gate = 4 * dk if kda else 4
    per_v = qkv_bytes * dv + 4 + gate + 4 * dv + 4 * dv + 4 + gate   # v, gates, d_out; dv, dbeta, dlog alpha
    per_qk = (qkv_bytes + 4) * 2 * dk                                 # q, k; dq, dk
    states = N * H * dv * dk * 4 * (3 if init_state else 2)
    return B * T * (H * per_v + Hk * per_qk) + states


def backward_alg_flops(B, T, H, dk, dv, C=32):
    """Flops of the chunked backward's dense products per token-head (full
    C x C tiles): the chunk records (A, M, W), the forward state pass
    (T diag(b) V, W S^T, U^T K_end), the backward state pass (M^T dO,
    K_end dS^T, dU^T W, dO^T Q e^g) and the chunk gradients (five C dk dv,
    five C^2 dv, five C^2 dk products and the two C^3 of the inverse's
    adjoint), divided by C."""
    per = 2 * 3 * C * dk
    per += 2 * (C * dv + 2 * dk * dv)
    per += 2 * (C * dv + 3 * dk * dv)
    per += 2 * (5 * dk * dv + 5 * C * dv + 5 * C * dk + 2 * C * C)
    return B * T * H * per


def decode_alg_bytes(N, H, dk, dv, kda, out_bytes):
    u = N * H
    return u * (2 * dv * dk * 4 + (2 * dk + dv) * 2 + 4 + (dk if kda else 1) * 4 + dv * out_bytes)


def decode_tokens_alg_bytes(N, K, H, Hk, dk, dv, kda, out_bytes, n_written):
    """Every sequence's state read once, the states of the n_written
    sequences that commit tokens written once, the K tokens' inputs read and
    their outputs written once."""
    st = H * dv * dk * 4
    tok = N * K
    return (N + n_written) * st + tok * (Hk * 2 * dk * 2 + H * dv * 2 + H * 4 + H * (dk if kda else 1) * 4
                                         + H * dv * out_bytes)


def time_calls(fn, steps, between=None):
    """Seconds per call of fn over `steps` calls, from HIP events on the
    current stream (the stream the binding launches on) recorded around each
    call: (mean, median, min).  `between`, if given, runs between calls,
    outside the timed intervals."""
    import statistics

    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        if between is not None:
            between()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) / 1e3 for a, b in ev]
    return sum(t) / len(t), statistics.median(t), min(t)


def time_back_to_back(fn, steps):
    """Mean seconds per call of fn over `steps` calls issued back to back
    between one pair of HIP events on the current stream: no event sits
    between two calls, so the figure carries no per-call event cost."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / steps


def time_per_launch(fn, steps):
    """Mean seconds per call of fn over `steps` back-to-back calls."""
    return time_calls(fn, steps)[0]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, H, target_s):
    """fp64 oracle over the first tokens of every (sequence, head) unit of the
    prefill workload, timed on the host cores.  The token count grows from a
    short probe until one run takes at least target_s/4 (or covers the whole
    sequence); that run is repeated until target_s of wall time has passed."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    B, T = inp["q"].shape[:2]
    threads = min(cores, B * H)
    s0 = inp["initial_state"].cpu()
    host = {k: inp[k].cpu() for k in ("q", "k", "v", "beta", "log_alpha")}

    def run(n):
        sub = {k: host[k][:, :n].contiguous() for k in host}
        t0 = time.perf_counter()
        oracle.recurrence(sub["q"], sub["k"], sub["v"], sub["beta"], sub["log_alpha"], initial_state=s0,
                          num_threads=threads)
        return time.perf_counter() - t0

    n = 128
    dt = run(n)
    while dt < target_s / 4 and n < T:
        n = int(min(T, max(2 * n, n * (target_s / 3) / max(dt, 1e-3))))
        dt = run(n)
    reps, total = 1, dt
    while total < target_s:
        total += run(n)
        reps += 1
    tokens = B * n * reps  # every head of these tokens
    return {"value": tokens / total / 1e6, "unit": "Mtok/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"first {n} of {T} tokens of all {B}x{H} (sequence, head) units of the prefill "
                      f"workload, fp64, {reps} run(s), {total:.1f} s wall"}


def prologue_alg_bytes(tokens, C, H, NA, N, x_bytes):
    """x read and q/k/v written once, the taps, the gate logits read and the
    gates written once, the convolution state read and written once."""
    return (2 * tokens * C * x_bytes + C * 16 + 2 * tokens * H * 4 + 2 * tokens * H * NA * 4
            + 2 * N * 3 * C * x_bytes)


def extra_workloads(args, gdr, torch, dev, WORKLOADS, prefill_inputs, decode_tokens_inputs):
    """The grouped-head prefill and the multi-token decode, each timed in its
    own loop of args.steps calls after args.warmup untimed ones."""
    res = {}

    def prefill_entry(w, inp, label, flush=None, out_dtype=torch.float32, chunk=0):
        B, T, Hk, dk = inp["q"].shape
        H, dv = inp["v"].shape[2:]
        po = torch.empty(B, T, H, dv, dtype=out_dtype, device=dev)
        N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
        pf = torch.empty(N, H, dv, dk, dtype=torch.float32, device=dev)
        f = lambda: gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                            initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"],
                                            out=po, final_state=pf, chunk_size=chunk)
        for _ in range(args.warmup):
            f()
        mean, med, mn = time_calls(f, args.steps, between=flush)
        kda = inp["log_alpha"].dim() == 4
        by = prefill_alg_bytes(B, T, H, dk, dv, kda, po.element_size(), inp["initial_state"] is not None, True,
                               Hk=Hk, gate_bytes=inp["beta"].element_size())
        if inp["cu_seqlens"] is not None:   # one initial and one final state per sequence, not per row
            by += (N - B) * 2 * H * dv * dk * 4
        fl = prefill_alg_flops(B, T, H, dk, dv, chunk or 32)
        return {"workload": label, "us_per_launch": round(mean * 1e6, 2), "us_median": round(med * 1e6, 2),
                "us_min": round(mn * 1e6, 2), "Mtok_s": round(B * T / mean / 1e6, 3), "alg_bytes": by,
                "hbm_GBps": round(by / mean / 1e9, 1), "frac_of_hbm_peak": round(by / mean / 1e9 / HBM_PEAK_GBS, 4),
                "alg_flops": fl, "mfma_frac": round(fl / mean / (BF16_MFMA_PEAK_TFLOPS * 1e12), 4)}

    w2 = WORKLOADS["kda_prefill_32k"]
    print(f"[bench] {w2.name} with bf16 outputs", file=sys.stderr, flush=True)
    g2 = prefill_inputs(w2, dev)
    res["kda_prefill_32k_bf16_out"] = prefill_entry(
        w2, g2, f"{w2.name} writing its outputs in bf16 (rounded to nearest even) instead of fp32: B=2, T=32768, "
                "H=32, d=128, bf16 q/k/v, per-channel decay, S0 given; not parity-equal to the fp32-output line: "
                "its parity test allows the output rounding on top of the bound (tol x RMS + 2^-8 |ref|), since "
                "rounding alone exceeds 2e-2 x RMS on the largest outputs", out_dtype=torch.bfloat16)
    del g2
    print(f"[bench] {w2.name} at chunk size 64", file=sys.stderr, flush=True)
    g2 = prefill_inputs(w2, dev)
    res["kda_prefill_32k_chunk64"] = prefill_entry(
        w2, g2, f"{w2.name} with 64-token chunks (the automatic chunk is 32): B=2, T=32768, H=32, d=128, bf16 "
                "q/k/v, per-channel decay, S0 given, fp32 out; mfma_frac counts the dense products at C = 64",
        chunk=64)
    del g2
    print(f"[bench] {w2.name} with bf16 gates", file=sys.stderr, flush=True)
    g2 = prefill_inputs(w2, dev, gate_dtype=torch.bfloat16)
    res["kda_prefill_32k_bf16_gates"] = prefill_entry(
        w2, g2, f"{w2.name} with beta and log alpha stored in bf16 (rounded from the same fp32 draws): B=2, "
                "T=32768, H=32, d=128, bf16 q/k/v, per-channel decay, S0 given, fp32 out")
    del g2

    w1 = WORKLOADS["gdn_prefill_8k"]
    print(f"[bench] {w1.name}", file=sys.stderr, flush=True)
    g1 = prefill_inputs(w1, dev)
    lbl = f"{w1.name}: B=1, T=8192, H=16, d=128, bf16 q/k/v, per-head decay, zero initial state, fp32 out"
    flush_buf = torch.empty(1 << 27, dtype=torch.float32, device=dev)     # 512 MiB
    res["gdn_prefill_8k"] = {"cache_warm": prefill_entry(w1, g1, lbl),
                             "after_512MiB_write": prefill_entry(w1, g1, lbl, flush=lambda: flush_buf.fill_(1.0)),
                             # its stated chunk size (the two kernels at 64-token chunks)
                             "chunk_64": prefill_entry(w1, g1, lbl + "; chunk size 64", chunk=64)}
    del g1

    w4 = WORKLOADS["packed_gdn_256k"]
    print(f"[bench] {w4.name}", file=sys.stderr, flush=True)
    g4 = prefill_inputs(w4, dev)
    lens = (g4["cu_seqlens"][1:] - g4["cu_seqlens"][:-1]).tolist()
    res["packed_gdn_256k"] = prefill_entry(w4, g4, f"{w4.name}: 8 packed sequences of {lens} tokens (262144), "
                                                   "H=16, d=128, bf16 q/k/v, per-head decay, S0 given, fp32 out")
    del g4

    print("[bench] measured ceilings", file=sys.stderr, flush=True)
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    mean, med, mn = time_calls(lambda: torch.matmul(a, b, out=c), 10)
    gemm_tflops = 2 * n ** 3 / med / 1e12
    del a, b, c
    for _ in range(3):
        flush_buf.add_(1.0)
    mean, med, mn = time_calls(lambda: flush_buf.add_(1.0), 10)
    rmw_gbs = 2 * flush_buf.numel() * 4 / med / 1e9
    del flush_buf
    res["measured_ceilings"] = {
        "bf16_gemm_8192_TFLOPs": round(gemm_tflops, 1), "bf16_gemm_frac_of_peak": round(gemm_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "rmw_512MiB_GBps": round(rmw_gbs, 1), "rmw_frac_of_peak": round(rmw_gbs / HBM_PEAK_GBS, 4),
        "note": "library bf16 GEMM (torch.matmul, 8192^3) and an in-place add over 512 MiB of fp32, median of 10"}

    wg = WORKLOADS["gdn_gva_prefill_32k"]
    print(f"[bench] {wg.name}", file=sys.stderr, flush=True)
    g = prefill_inputs(wg, dev)
    B, T, Hk, dk = g["q"].shape
    H, dv = g["v"].shape[2:]
    gout = torch.empty(B, T, H, dv, dtype=torch.float32, device=dev)
    gfin = torch.empty_like(g["initial_state"])
    f = lambda: gdr.gdr_prefill_chunked(g["q"], g["k"], g["v"], g["beta"], g["log_alpha"],
                                        initial_state=g["initial_state"], out=gout, final_state=gfin)
    for _ in range(args.warmup):
        f()
    t, med, mn = time_calls(f, args.steps)
    by = prefill_alg_bytes(B, T, H, dk, dv, False, 4, Hk=Hk)
    res["grouped_prefill"] = {
        "workload": f"{wg.name}: B={B}, T={T}, {Hk} q/k heads shared by {H} value heads, d={dk}, bf16 q/k/v, "
                    "per-head decay, S0 given, fp32 out",
        "us_per_launch": round(t * 1e6, 2), "us_median": round(med * 1e6, 2), "us_min": round(mn * 1e6, 2),
        "Mtok_s": round(B * T / t / 1e6, 3), "alg_bytes": by,
        "hbm_GBps": round(by / t / 1e9, 1), "frac_of_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(prefill_alg_flops(B, T, H, dk, dv, 32) / t / (BF16_MFMA_PEAK_TFLOPS * 1e12), 4)}
    del g, gout, gfin

    from workloads import prologue_inputs

    wpl = WORKLOADS["prologue_gdn_32k"]
    print(f"[bench] {wpl.name}", file=sys.stderr, flush=True)
    pi = prologue_inputs(wpl, dev)
    B, T, C = pi["x"].shape
    H = pi["b_logit"].shape[-1]
    f = lambda: gdr.gdr_layer_prologue(pi["x"], pi["conv_weight"], pi["a_logit"], pi["b_logit"],
                                       num_qk_heads=pi["num_qk_heads"], head_dim_k=pi["head_dim_k"],
                                       head_dim_v=pi["head_dim_v"], conv_state=pi["conv_state"])
    for _ in range(args.warmup):
        f()
    t, med, mn = time_calls(f, args.steps)
    by = prologue_alg_bytes(B * T, C, H, 1, B, 2)
    res["layer_prologue"] = {
        "workload": f"{wpl.name}: B={B}, T={T}, {C} projected channels ({pi['num_qk_heads']} q/k heads and {H} value "
                    "heads of 128), bf16, width-4 convolution with its state, q/k L2 norm, per-head gates",
        "us_per_call": round(t * 1e6, 2), "us_median": round(med * 1e6, 2), "us_min": round(mn * 1e6, 2),
        "Mtok_s": round(B * T / t / 1e6, 3), "alg_bytes": by, "GBps": round(by / t / 1e9, 1),
        "frac_of_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    del pi

    wm = WORKLOADS["mtp_decode_256x48"]
    print(f"[bench] {wm.name}", file=sys.stderr, flush=True)
    m = decode_tokens_inputs(wm, dev)
    N, K, Hk, dk = m["q"].shape
    H, dv = m["v"].shape[2:]
    mout = torch.empty(N, K, H, dv, dtype=torch.float32, device=dev)
    f = lambda: gdr.gdr_decode_tokens(m["q"], m["k"], m["v"], m["beta"], m["log_alpha"], m["state_pool"],
                                      num_commit=m["num_commit"], state_slots=m["state_slots"], out=mout)
    for _ in range(args.warmup):
        f()
    t, med, mn = time_calls(f, args.steps)
    tb = time_back_to_back(f, args.steps)
    n_written = int((m["num_commit"] > 0).sum())
    by = decode_tokens_alg_bytes(N, K, H, Hk, dk, dv, False, 4, n_written)
    res["multi_token_decode"] = {
        "workload": f"{wm.name}: {N} sequences x {H} value heads ({Hk} q/k heads), d={dk}, {K} tokens each, "
                    f"states in a pool of {wm.slots} slots, committed prefix uniform in [0, {K - 1}] "
                    f"({n_written} of {N} sequences write their state), per-head decay, fp32 out",
        "us_per_call": round(t * 1e6, 2), "us_median": round(med * 1e6, 2), "us_min": round(mn * 1e6, 2),
        "Mtok_s": round(N * K / t / 1e6, 4), "alg_bytes": by,
        "GBps": round(by / t / 1e9, 1), "frac_of_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
        # the per-call figures carry one event pair per call, which costs this
        # call about 12 us of device time; calls issued back to back do not
        "us_back_to_back": round(tb * 1e6, 2),
        "frac_of_hbm_peak_back_to_back": round(by / tb / 1e9 / HBM_PEAK_GBS, 4)}
    del m, mout

    from workloads import backward_cotangents

    res["prefill_backward"] = {}
    for name in ("kda_backward_32k", "gdn_backward_8k", "gdn_gva_backward_32k"):
        wb = WORKLOADS[name]
        print(f"[bench] {wb.name}", file=sys.stderr, flush=True)
        bi = prefill_inputs(wb, dev)
        bc = backward_cotangents(bi, wb.seed, dev)
        B, T, Hk, dk = bi["q"].shape
        H, dv = bi["v"].shape[2:]
        kda = bi["log_alpha"].dim() == 4
        f = lambda: gdr.gdr_prefill_backward(bi["q"], bi["k"], bi["v"], bi["beta"], bi["log_alpha"], bc["d_out"],
                                             initial_state=bi["initial_state"], d_final_state=bc["d_final_state"])
        for _ in range(args.warmup):
            f()
        steps = max(1, min(args.steps, 5)) if T * B >= 32768 else args.steps
        t, med, mn = time_calls(f, steps)
        by = backward_alg_bytes(B, T, H, dk, dv, kda, B, Hk=Hk)
        fl = backward_alg_flops(B, T, H, dk, dv)
        res["prefill_backward"][name] = {
            "workload": f"{name}: gradients of q, k, v, beta, log alpha and the initial state through the chunked "
                        f"prefill, B={B}, T={T}, H={H}" + (f" value heads sharing {Hk} q/k heads" if Hk != H else "")
                        + f", d={dk}, bf16 q/k/v, fp32 gates, d_out and d_final_state ~ N(0, 1), "
                        f"{'per-channel' if kda else 'per-head'} decay, S0 given; fp32 accumulation, the large "
                        f"products as split bf16 (hi/lo operands, three bf16 MFMAs each), the C x C ones in fp32",
            "calls": steps, "us_per_call": round(t * 1e6, 1), "us_median": round(med * 1e6, 1),
            "us_min": round(mn * 1e6, 1), "Mtok_s": round(B * T / t / 1e6, 3), "alg_bytes": by,
            "GBps": round(by / t / 1e9, 1), "frac_of_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
            "alg_flops": fl, "TFLOPs": round(fl / t / 1e12, 2),
            "frac_of_fp32_mfma_peak": round(fl / t / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            # a split-bf16 product issues three bf16 MFMAs: its dense roof is a third of bf16's
            "frac_of_split_bf16_peak": round(fl / t / 1e12 / (BF16_MFMA_PEAK_TFLOPS / 3), 4)}
        del bi, bc
        torch.cuda.empty_cache()

    # the KDA 32K backward inside a 4 GB workspace: time segments (the library
    # takes the fewest equal segments that fit, as found here)
    wb = WORKLOADS["kda_backward_32k"]
    print(f"[bench] {wb.name} in a 4 GB workspace", file=sys.stderr, flush=True)
    bi = prefill_inputs(wb, dev)
    bc = backward_cotangents(bi, wb.seed, dev)
    B, T, Hk, dk = bi["q"].shape
    H, dv = bi["v"].shape[2:]
    cap = 4_000_000_000
    ws_of = lambda s: gdr.gdr_prefill_backward_workspace_bytes(bi["q"], bi["v"], bi["log_alpha"], segment_chunks=s)
    nct = -(-T // 32)
    S = next(max(16, -(-nct // ns)) for ns in range(2, nct + 1) if 0 < ws_of(max(16, -(-nct // ns))) <= cap)
    ws = torch.empty(ws_of(S), dtype=torch.uint8, device=dev)
    f = lambda: gdr.gdr_prefill_backward(bi["q"], bi["k"], bi["v"], bi["beta"], bi["log_alpha"], bc["d_out"],
                                         initial_state=bi["initial_state"], d_final_state=bc["d_final_state"],
                                         workspace=ws)
    for _ in range(max(1, min(args.warmup, 2))):
        f()
    steps = max(1, min(args.steps, 5))
    t, med, mn = time_calls(f, steps)
    res["prefill_backward"]["kda_backward_32k_in_4GB"] = {
        "workload": f"kda_backward_32k with a workspace of at most {cap} bytes: segments of {S} chunks "
                    f"({-(-nct // S)} segments; the one-pass workspace is "
                    f"{gdr.gdr_prefill_backward_workspace_bytes(bi['q'], bi['v'], bi['log_alpha'])} bytes); "
                    "gradients equal to the one-pass call's bit for bit",
        "workspace_bytes": ws.numel(), "segment_chunks": S, "calls": steps, "us_per_call": round(t * 1e6, 1),
        "us_median": round(med * 1e6, 1), "us_min": round(mn * 1e6, 1), "Mtok_s": round(B * T / t / 1e6, 3)}
    del bi, bc, ws
    torch.cuda.empty_cache()

    # one decode step fed from the layer's projected channels: the fused call
    # against the two calls it replaces (layer prologue, then decode step)
    from workloads import decode_prologue_inputs
    wdp = WORKLOADS["decode_prologue_256x48"]
    print(f"[bench] {wdp.name}", file=sys.stderr, flush=True)
    dp = decode_prologue_inputs(wdp, dev)
    N, H, Hk, dk, dv = wdp.batch, wdp.heads, wdp.qk_heads, wdp.dk, wdp.dv
    x1, a1, b1 = dp["x"][:, 0].contiguous(), dp["a_logit"][:, 0].contiguous(), dp["b_logit"][:, 0].contiguous()
    x3, a3, b3 = dp["x"], dp["a_logit"], dp["b_logit"]
    dout = torch.empty(N, H, dv, dtype=torch.float32, device=dev)
    kw = dict(num_qk_heads=Hk, head_dim_k=dk, head_dim_v=dv, conv_state=dp["conv_state"])
    fused = lambda: gdr.gdr_decode_step_prologue(x1, dp["conv_weight"], a1, b1, dp["state"], out=dout, **kw)

    def unfused():
        q, k, v, beta, la = gdr.gdr_layer_prologue(x3, dp["conv_weight"], a3, b3, **kw)
        gdr.gdr_decode_step(q[:, 0], k[:, 0], v[:, 0], beta[:, 0], la[:, 0], dp["state"], out=dout)

    res["decode_with_prologue"] = {
        "workload": f"{wdp.name}: one token for each of {N} sequences x {H} value heads ({Hk} q/k heads), d={dk}, "
                    f"from bf16 projected channels ({2 * Hk * dk + H * dv} per token) with a convolution state: "
                    f"width-4 convolution, q/k L2 norm, per-head gates, then the state update; fp32 out"}
    C = 2 * Hk * dk + H * dv
    common = N * H * dv * dk * 4 * 2 + N * C * 2 + N * 3 * C * 2 * 2 + C * 16 + N * H * 4 * 2 + N * H * dv * 4
    qkv_rt = 2 * (N * (2 * Hk * dk + H * dv) * 2 + N * H * 4 * 2)   # q, k, v (bf16) and gates written, read back
    for name, f, by in (("fused", fused, common), ("unfused", unfused, common + qkv_rt)):
        for _ in range(args.warmup):
            f()
        t, med, mn = time_calls(f, args.steps)
        res["decode_with_prologue"][name] = {
            "us_per_call": round(t * 1e6, 2), "us_median": round(med * 1e6, 2), "us_min": round(mn * 1e6, 2),
            "alg_bytes": by, "GBps": round(by / t / 1e9, 1), "frac_of_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    res["decode_with_prologue"]["bytes_saved_per_call"] = qkv_rt
    del dp, dout
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--dv-slice", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the oracle sample")
    ap.add_argument("--copy-reference", action="store_true",
                    help="also run one 1 GiB device copy (a known-size kernel for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_73_amd as gdr
    from workloads import WORKLOADS, decode_inputs, decode_tokens_inputs, prefill_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wp = WORKLOADS["kda_prefill_32k"]
    wd = WORKLOADS["decode_256x32"]
    print(f"[bench] generating inputs ({wp.name}, {wd.name})", file=sys.stderr, flush=True)
    inp = prefill_inputs(wp, dev)
    dec = {g: decode_inputs(wd, dev, gate=g) for g in ("head", "channel")}
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    out = torch.empty(B, T, H, dv, dtype=torch.float32, device=dev)
    fin = torch.empty_like(inp["initial_state"])
    dout = {g: torch.empty(wd.batch, wd.heads, wd.dv, dtype=torch.float32, device=dev) for g in dec}

    def prefill():
        gdr.gdr_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                                initial_state=inp["initial_state"], chunk_size=args.chunk,
                                dv_slice=args.dv_slice, out=out, final_state=fin)

    def decode(g):
        d = dec[g]
        gdr.gdr_decode_step(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["state"], out=dout[g])

    if args.copy_reference:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        prefill()
        decode("head")
        decode("channel")
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)

    # K steps of the whole path, timed as K prefills back to back, then K
    # decode steps (per-head decay, then per-channel decay) back to back, so
    # that each kernel's time is its own steady state (a decode right after a
    # prefill would also pay for writing back the prefill's dirty cache lines).
    K = args.steps
    ev_p = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev_d = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev_p[0].record()
    for s_ in range(K):
        prefill()
        ev_p[s_ + 1].record()
    ev_d[0].record()
    for s_ in range(K):
        decode("head")
        ev_d[2 * s_ + 1].record()
        decode("channel")
        ev_d[2 * s_ + 2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    import statistics

    i_pre = [ev_p[i].elapsed_time(ev_p[i + 1]) / 1e3 for i in range(K)]       # s per launch
    i_dg = [ev_d[2 * i].elapsed_time(ev_d[2 * i + 1]) / 1e3 for i in range(K)]
    i_dk = [ev_d[2 * i + 1].elapsed_time(ev_d[2 * i + 2]) / 1e3 for i in range(K)]
    t_pre, t_dg, t_dk = (sum(x) / K for x in (i_pre, i_dg, i_dk))
    spread = lambda x: {"us_median": round(statistics.median(x) * 1e6, 2), "us_min": round(min(x) * 1e6, 2)}

    chunk = args.chunk or 32
    tokens = B * T
    pre_bytes = prefill_alg_bytes(B, T, H, dk, dv, True, 4)
    pre_bytes_bf16o = prefill_alg_bytes(B, T, H, dk, dv, True, 2)
    pre_flops = prefill_alg_flops(B, T, H, dk, dv, chunk)
    pre_tflops = pre_flops / t_pre / 1e12
    dg_bytes = decode_alg_bytes(wd.batch, wd.heads, wd.dk, wd.dv, False, 4)
    dk_bytes = decode_alg_bytes(wd.batch, wd.heads, wd.dk, wd.dv, True, 4)
    pre_gbs = pre_bytes / t_pre / 1e9

    traffic = None
    if os.path.exists(PROFILE_PMC):
        rec = json.load(open(PROFILE_PMC))
        if rec.get("kernel_source_hash") == kernel_source_hash() and rec.get("chunk") == chunk:
            traffic = rec.get("hbm_bytes_per_launch")

    result = {
        "metric": "delta-rule prefill Mtok/s at T=32K (MFMA %) + decode step HBM GB/s (% peak)",
        "value": round(tokens / t_pre / 1e6, 3),
        "unit": "Mtok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "kda_prefill_32k + decode_256x32 (per-head and per-channel decay)",
            "prefill": {"batch": B, "seq_len": T, "heads": H, "d_k": dk, "d_v": dv, "gate": "per-channel",
                        "chunk": chunk, "dv_slice": args.dv_slice or "auto", "initial_state": True,
                        "out_dtype": "fp32"},
            "decode": {"num_seqs": wd.batch, "heads": wd.heads, "d_k": wd.dk, "d_v": wd.dv,
                       "state": "fp32 in place", "out_dtype": "fp32"},
            "precision": "bf16 q/k/v, fp32 gates and states; fp16/bf16 MFMA operands (hi/lo split on the "
                         "value-carrying ones), fp32 accumulation",
        },
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": f"prep_kernel<128,{chunk},KDA,bf16> + chain_kernel<128,32,{chunk},KDA,bf16> "
                               "(one prefill call)",
                     "chunk": chunk, "alg_flops_per_launch": pre_flops,
                     "alg_flops_per_token_head": pre_flops // (B * T * H), "avg_launch_us": round(t_pre * 1e6, 2),
                     "hbm_beside": {
                         "peak_GBps": HBM_PEAK_GBS,
                         "bf16_out": {"alg_bytes_per_launch": pre_bytes_bf16o,
                                      "GBps": round(pre_bytes_bf16o / t_pre / 1e9, 1),
                                      "frac": round(pre_bytes_bf16o / t_pre / 1e9 / HBM_PEAK_GBS, 4)},
                         "fp32_out": {"alg_bytes_per_launch": pre_bytes, "GBps": round(pre_gbs, 1),
                                      "frac": round(pre_gbs / HBM_PEAK_GBS, 4)}}},
        "prefill": {"us_per_launch": round(t_pre * 1e6, 2), **spread(i_pre), "Mtok_s": round(tokens / t_pre / 1e6, 3),
                    "mfma_frac": round(pre_flops / t_pre / (BF16_MFMA_PEAK_TFLOPS * 1e12), 4),
                    "alg_flops": pre_flops, "hbm_GBps": round(pre_gbs, 1)},
        "decode": {
            "per_head_decay": {"us_per_step": round(t_dg * 1e6, 2), **spread(i_dg), "GBps": round(dg_bytes / t_dg / 1e9, 1),
                               "frac_of_hbm_peak": round(dg_bytes / t_dg / 1e9 / HBM_PEAK_GBS, 4),
                               "Mtok_s": round(wd.batch / t_dg / 1e6, 4), "alg_bytes": dg_bytes},
            "per_channel_decay": {"us_per_step": round(t_dk * 1e6, 2), **spread(i_dk), "GBps": round(dk_bytes / t_dk / 1e9, 1),
                                  "frac_of_hbm_peak": round(dk_bytes / t_dk / 1e9 / HBM_PEAK_GBS, 4),
                                  "Mtok_s": round(wd.batch / t_dk / 1e6, 4), "alg_bytes": dk_bytes},
        },
        "cpu_baseline": None,
    }
    result.update(extra_workloads(args, gdr, torch, dev, WORKLOADS, prefill_inputs, decode_tokens_inputs))
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, H, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
