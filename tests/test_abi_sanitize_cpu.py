"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

qsa_api.cpp (argument validation, workspace carving, launch set-up) is compiled for
the host alone with both sanitizers and linked, with the library's kernel objects,
into the driver tests/abi_sanitize_main.cpp.  The driver calls every entry point
with one defect at a time and checks each documented status; without a GPU its
well-formed calls reach the launch code and must report QSA_E_HIP.  Any sanitizer
report fails the test.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_c4_amd", "csrc")
OBJ = os.path.join(ROOT, "_build")
KERNEL_OBJS = ["qsa_build.o", "qsa_index.o", "qsa_topk.o", "qsa_prefill.o", "qsa_attn.o"]
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not all(os.path.exists(os.path.join(OBJ, o)) for o in KERNEL_OBJS):
        from block_sparse_attention_c4_amd import build
        build.build()
    flags = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-Wno-c++20-extensions", *SAN]
    api = str(tmp_path / "api.o")
    main = str(tmp_path / "main.o")
    exe = str(tmp_path / "abi_sanitize")
    _run([CLANG, *flags, "-c", os.path.join(CSRC, "qsa_api.cpp"), "-o", api])
    _run([CLANG, *flags, "-c", os.path.join(ROOT, "tests", "abi_sanitize_main.cpp"), "-o", main])
    _run([CLANG, *SAN, "-o", exe, main, api, *[os.path.join(OBJ, o) for o in KERNEL_OBJS],
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit; leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0 and "PASSED" in r.stdout, out

