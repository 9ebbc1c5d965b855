"""The C ABI's validation and error paths under AddressSanitizer (leak
detection on) and UndefinedBehaviorSanitizer, on the CPU: the library is
built with both sanitizers on its host code (the device code is built as
usual) and tests/abi_driver.c walks every entry point's argument checks,
workspace queries and the timing calls.  No GPU is needed (valid argument
sets stop at the device check)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def _device_visible() -> bool:
    try:
        import torch
    except ImportError:
        return True   # cannot tell: treat as visible
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
@pytest.mark.timeout(600)
def test_abi_paths_under_asan_and_ubsan(tmp_path):
    # the driver's valid argument sets carry fake device pointers: they must
    # stop at the device check, so this runs only where no device is visible
    if _device_visible():
        pytest.skip("a device is visible: the driver's fake-pointer calls are not made")
    lib = tmp_path / "liblact_san.so"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "test_layers_amd", "csrc"),
                        os.path.join(ROOT, "test_layers_amd", "csrc", "lact.hip"), "-o", str(lib)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_driver"
    r = subprocess.run([CLANG, "-std=c11", "-g", "-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_driver.c"),
                        "-L", str(tmp_path), "-llact_san", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    assert "0 failures" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
