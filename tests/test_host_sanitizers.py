"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.hip's host side (argument validation, size queries, the cost-table
interpolation) is compiled host-only with both sanitizers and linked into
tests/sanitize/host_validation.cpp, which drives every entry point of
include/q4g64.h with invalid arguments (extreme integers, NULL and misaligned
pointers, NaN and infinite floats, window and struct arrays of exactly the
documented length) and checks every status code and size. No device code is
built, and no call reaches a launch; the run needs no GPU. Any signed
overflow, out-of-bounds read or leak ends the run with a sanitizer report.
"""

import hashlib
import os
import pathlib
import shutil
import subprocess
import tempfile

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
CSRC = ROOT / "bit_weight_only_q4g64_amd" / "csrc"
DRIVER = ROOT / "tests" / "sanitize" / "host_validation.cpp"
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _sources():
    return sorted(CSRC.glob("*.h")) + sorted(CSRC.glob("*.hip")) + [ROOT / "include" / "q4g64.h", DRIVER]


def _build(out: pathlib.Path) -> pathlib.Path:
    exe = out / "host_validation"
    if exe.exists():
        return exe
    tmp = pathlib.Path(tempfile.mkdtemp(prefix="build_", dir=out))
    empty = tmp / "empty.hipfb"  # no device code object: nothing can be launched
    empty.write_bytes(b"")
    obj = tmp / "api_host.o"
    compile_api = [
        HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
        "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(empty),
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", str(ROOT / "include"), "-c", str(CSRC / "api.hip"), "-o", str(obj),
    ]
    r = subprocess.run(compile_api, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    link = [CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1", "-std=c++17",
            "-I", str(ROOT / "include"), str(DRIVER), str(obj),
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(tmp / "host_validation")]
    r = subprocess.run(link, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    os.replace(tmp / "host_validation", exe)
    shutil.rmtree(tmp, ignore_errors=True)
    return exe


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm compilers")
def test_host_validation_is_clean_under_sanitizers():
    h = hashlib.sha256()
    for p in _sources():
        h.update(p.name.encode())
        h.update(p.read_bytes())
    out = pathlib.Path(tempfile.gettempdir()) / f"q4g64_host_sanitize_{h.hexdigest()[:16]}"
    out.mkdir(exist_ok=True)
    exe = _build(out)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    # the fake device addresses are never touched; no GPU may be needed or used
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-6000:]
    assert "runtime error" not in log and "Sanitizer" not in log, log[-6000:]
    assert log.strip().splitlines()[-1].endswith(", 0 failed"), log[-2000:]
