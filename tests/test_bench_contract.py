"""bench.py's command-line contract, checked without a GPU: it measures one
GPU only and says so when asked for more; its algorithmic byte counts follow
the stated formulas."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_algorithmic_bytes():
    # KDA 32K headline: q, k, v bf16; beta and per-channel log alpha fp32; fp32 out; S0 and S_final
    tok = 2 * 32768 * 32
    expect = tok * (3 * 128 * 2 + 4 + 128 * 4 + 128 * 4) + 2 * 2 * 32 * 128 * 128 * 4
    assert bench.prefill_alg_bytes(2, 32768, 32, 128, 128, True, 4) == expect == 3774873600
    # grouped heads read q/k once per q/k head
    g = bench.prefill_alg_bytes(1, 100, 48, 128, 128, False, 4, Hk=16)
    assert g == 100 * 16 * 2 * 128 * 2 + 100 * 48 * (128 * 2 + 4 + 4 + 128 * 4) + 2 * 48 * 128 * 128 * 4
    # decode: state read and written, token inputs, fp32 out
    assert bench.decode_alg_bytes(256, 32, 128, 128, False, 4) == 256 * 32 * (2 * 128 * 128 * 4 + 384 * 2 + 8 + 512)
    # multi-token decode: every state read, n_written written
    assert bench.decode_tokens_alg_bytes(2, 3, 4, 2, 16, 16, True, 4, 1) == \
        3 * 4 * 16 * 16 * 4 + 6 * (2 * 2 * 16 * 2 + 4 * (16 * 2 + 4 + 16 * 4 + 16 * 4))


def test_prefill_roofline_accounting():
    """The prefill's MFMA roof uses the chunked form's dense flops per
    token-head at the stated chunk (4 C (dk + dv) + 6 dk dv); HBM beside it
    counts bf16 outputs (2 bytes less per output element than fp32)."""
    tok = 2 * 32768 * 32
    assert bench.prefill_alg_flops(2, 32768, 32, 128, 128, 32) == tok * 131072
    assert bench.prefill_alg_flops(2, 32768, 32, 128, 128, 64) == tok * 163840
    assert bench.prefill_alg_bytes(2, 32768, 32, 128, 128, True, 2) == 3238002688
