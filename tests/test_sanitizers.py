"""Host AddressSanitizer + UndefinedBehaviorSanitizer run (CPU only).

The oracle and the host code of the HIP library (argument validation,
workspace sizing and layout, the C-ABI entry points up to the launch) are
rebuilt with both sanitizers; the oracle's pins and the host C-ABI tests then
run against those builds in a child process with the clang ASan runtime
preloaded (it carries the UBSan handlers too).  Any report aborts the child.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_sanitizers(tmp_path):
    runtime = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtime:
        pytest.skip("no clang ASan runtime in this image")
    from gated_delta_rule_73_amd import build as gbuild
    import oracle

    lib = gbuild.build(sanitize=True)
    orc = oracle.build_sanitized(str(tmp_path / "libgdr_oracle_sanitized.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime[-1],
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               GDR_SANITIZED_LIBRARY=lib, GDR_SANITIZED_ORACLE=orc,
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests"), env.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "sanitize_paths", "-m", "not gpu",
                        "tests/test_abi_host.py", "tests/test_oracle.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    print(tail)
    assert r.returncode == 0, tail
    assert "passed" in r.stdout
    loaded = [ln for ln in r.stdout.splitlines() if ln.startswith("sanitized libraries loaded:")]
    assert loaded and lib in loaded[-1] and orc in loaded[-1], loaded
