"""Host-side checks of the C-ABI library under AddressSanitizer and UBSan (CPU;
no kernel is launched): the workspace layout, the tile-list bounds against
adversarial per-expert loads, and every entry point's argument validation
(tests/host/check_host.cpp).  The check program includes the library's API source
compiled with host-only sanitizers and links the library's kernel objects."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_checks_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not found")
    from mixture_experts_amd import build as B
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "moe_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build(verbose=False)
    check_o, exe = str(tmp_path / "check_host.o"), str(tmp_path / "check_host")
    compile_cmd = [hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fno-gpu-rdc",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-I", os.path.join(ROOT, "include"), "-I", B.CSRC,
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined",
                   "-c", os.path.join(ROOT, "tests", "host", "check_host.cpp"), "-o", check_o]
    r = subprocess.run(compile_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    link_cmd = [clang, "-fsanitize=address,undefined", check_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-3000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "host checks: 0 failures" in r.stdout
