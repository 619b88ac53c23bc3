"""AddressSanitizer + UndefinedBehaviorSanitizer over the library's host code (CPU only).

The HIP sources are compiled for the host alone (no device code object) with ASan and UBSan, and a
driver (tests/sanitize/driver.cpp) runs every validation, workspace-layout and buffer-check path
through them: a table of edge cases and a seeded fuzz of 20000 descriptors, valid and invalid.
Nothing is launched: without a GPU every valid call stops at the device-buffer check.  Any
sanitizer report, or an unknown status, fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_chunk_amd", "csrc")
SOURCES = ["errors.hip", "profile.hip", "ttt_layer.hip", "ttt_backward.hip", "ttt_full_bwd.hip", "linattn.hip",
           "swa.hip"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    # sanitizers on the host side only (-Xarch_host): the device code is built as usual for gfx950
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
              "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    # the sources compile in parallel
    procs = [subprocess.Popen([hipcc, *common, *san, "-fPIC", "-c", os.path.join(CSRC, s), "-o",
                               str(tmp_path / (s + ".o"))], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
             for s in SOURCES]
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-4000:]
    lib = tmp_path / "libttt_san.so"
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *san,
                        *[str(tmp_path / (s + ".o")) for s in SOURCES], "-o", str(lib)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = tmp_path / "driver"
    r = subprocess.run([hipcc, *common, *san, "-x", "c++", os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
                        "-L", str(tmp_path), "-lttt_san", "-Wl,-rpath," + str(tmp_path), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    # leaks inside the HIP runtime are not this library's; every other ASan / UBSan report is fatal
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert "all calls returned known statuses" in out
