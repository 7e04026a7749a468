"""The engine's host code (configuration checks, workspace layout, pack
validation, model creation's refusals, the per-kernel entry points' shape
checks) under AddressSanitizer and UndefinedBehaviorSanitizer, CPU tier:
tests/host_sanitizer_driver.cpp drives a build of the library whose host
code carries both sanitizers (`build.py --host-sanitize`); any memory error,
leak or undefined behaviour they see ends the driver with an error."""
import os
import subprocess

from conftest import gpu_available


def test_host_paths_under_address_and_undefined_behaviour_sanitizers():
    from transformer_text_embedding_amd import build as bb
    if not os.path.exists(bb.SANITIZE_DRIVER):
        bb.build_host_sanitized()
    env = dict(os.environ)
    # leaks are checked where no device runtime is initialised behind the
    # library's back (the HIP runtime keeps allocations until exit)
    env["ASAN_OPTIONS"] = f"detect_leaks={0 if gpu_available() else 1}:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.pop("TTE_DEBUG", None)
    r = subprocess.run([bb.SANITIZE_DRIVER], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks done, 0 failed" in out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
