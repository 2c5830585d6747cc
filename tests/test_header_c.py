"""include/attn.h used from C and from C++ (CPU only).

tests/c_abi/header_use.c is built against the header alone, with gcc as C99
and with g++ as C++11, both under -Wall -Wextra -Werror -pedantic, and
linked to the built libattn.so; then once more each way with HIP's runtime API
header included first, which declares the same stream type.  The program assigns every entry point to a
function pointer of its documented type (so a changed prototype fails to
build), checks the enum values, the status names and the workspace queries,
and calls each compute entry point with null tensors, which every one must
refuse with ATTN_ERR_INVALID_ARG before any HIP call."""
import os
import re
import shutil
import subprocess

import pytest

import exact_scaled_dot_sdpa_amd as E

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "header_use.c")
INC = os.path.join(ROOT, "include")

HIP_API = "/opt/rocm/include/hip/hip_runtime_api.h"
# the same program with HIP's runtime API header included before attn.h
# (-include), as a program that also calls HIP itself would; HIP's headers are
# system headers here, so only attn.h's own warnings count
WITH_HIP = ["-isystem", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-include", "hip/hip_runtime_api.h"]

COMPILERS = [("gcc", ["-std=c99", "-x", "c"]), ("g++", ["-std=c++11", "-x", "c++"]),
             ("gcc", ["-std=c99", *WITH_HIP, "-x", "c"]), ("g++", ["-std=c++11", *WITH_HIP, "-x", "c++"])]


@pytest.mark.parametrize("cc,lang", COMPILERS, ids=["c99", "c++11", "c99-after-hip", "c++11-after-hip"])
def test_header_builds_links_and_runs(tmp_path, cc, lang):
    if shutil.which(cc) is None:
        pytest.skip("needs %s" % cc)
    if "-include" in lang and not os.path.exists(HIP_API):
        pytest.skip("needs %s" % HIP_API)
    libdir = os.path.dirname(E.lib_path())
    exe = str(tmp_path / "header_use")
    cmd = [cc, *lang, "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INC, SRC, "-x", "none", "-L", libdir,
           "-lattn", "-Wl,-rpath," + libdir, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_readme_c_example_compiles(tmp_path):
    """The C example in README.md compiles as C99 against include/attn.h and
    HIP's runtime API header (compile only: it needs a GPU to run)."""
    if shutil.which("gcc") is None or not os.path.exists(HIP_API):
        pytest.skip("needs gcc and %s" % HIP_API)
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```c\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1, "README.md should hold exactly one C example"
    src = tmp_path / "readme_example.c"
    src.write_text(blocks[0])
    b = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-isystem", "/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", "-I", INC, "-c", str(src), "-o", str(tmp_path / "ex.o")],
                       capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
