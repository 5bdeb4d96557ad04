"""The C ABI's host logic under AddressSanitizer, UndefinedBehaviorSanitizer and
LeakSanitizer (tests/abi_sanitize): the ledger, rope-width resolution and every
check that fails before device work, without a GPU; and, on the GPU, allocation
failure injected at every device allocation of eagle3_load and eagle3_trunk_load
(EAGLE3_E_OOM, no handle, nothing left allocated)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
EXE = os.path.join(ROOT, "eagle_draft_head_amd", "_asan", "abi_check")
SUPP = os.path.join(HERE, "abi_sanitize", "lsan.supp")


def _run(mode):
    if not os.path.exists(EXE):
        import sys
        sys.path.insert(0, os.path.join(HERE, "abi_sanitize"))
        from sanitized_build import build
        build()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["LSAN_OPTIONS"] = f"suppressions={SUPP}:print_suppressions=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([EXE, mode], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-3000:])
    print(r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-2000:]
    assert f"abi_check {mode}: 0 failed checks" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    return r.stdout


def test_abi_host_paths_under_sanitizers():
    _run("host")


@pytest.mark.gpu
def test_allocation_failures_release_everything():
    out = _run("device")
    assert "eagle3_load (bf16 batched):" in out and "eagle3_load (int4):" in out
    assert "eagle3_trunk_load:" in out
