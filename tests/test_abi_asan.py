"""Host code of the runtime under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU): kva_runtime.hip is compiled with the sanitizers on its
host half (device code as usual), linked with the other kernels' objects
into tests/asan/abi_host_asan.cpp, and run.  The driver exercises every
host-only path: config validation, the head plan, the weight packing into
each device layout (ragged row counts, short buffers, an overflowing q8_0
scale), the fp16 conversion, status strings and NULL handling.  Any heap or
stack overflow, use after free, leak or undefined behaviour aborts it."""
import os
import shutil
import subprocess

import pytest

from learned_kv_approximation_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.slow
def test_runtime_host_code_under_sanitizers(tmp_path):
    try:
        _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not available")
    objs, procs = [], []
    for src in _build.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        cmd = _build.compile_command(src, obj)
        if src == "kva_runtime.hip":
            cmd = cmd[:1] + SAN_HOST + cmd[1:]
        objs.append(obj)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for cmd, p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, " ".join(cmd) + "\n" + err[-3000:]
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "abi_host_asan")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    r = subprocess.run([CLANG, "-std=c++17", "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "asan", "abi_host_asan.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(shutil.which("hipcc") or
                                                                             "/opt/rocm/bin/hipcc"))), "lib")
    r = subprocess.run([CLANG, *san, drv, *objs, f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi host checks ok" in r.stdout
