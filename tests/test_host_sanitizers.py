"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

  * The fp64 oracle (oracle/oracle.c), rebuilt with the sanitizers, runs every
    pin of tests/oracle_pins.py.
  * The C-ABI layer (csrc/attn_api.hip: validation, workspace sizing,
    dispatch), built host-only with g++ against launch stubs
    (tests/host_sanitize/launch_stubs.cpp), runs every case table of
    tests/test_abi_host.py plus one valid call of each entry point.

Each run happens in a child process that preloads gcc's ASan runtime.  Two
planted mistakes, each in a copy of the source, check that the set-up catches
what it should: an out-of-bounds read in the oracle, and a 32-bit overflow in
the ABI layer's size arithmetic."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
API = os.path.join(ROOT, "exact_scaled_dot_sdpa_amd", "csrc", "attn_api.hip")
STUBS = os.path.join(ROOT, "tests", "host_sanitize", "launch_stubs.cpp")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _asan_runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not out or not os.path.exists(out):
        pytest.skip("gcc's libasan.so is not installed")
    return out


def _run(script, *args):
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([sys.executable, "-c", script, *args], capture_output=True, text=True, env=env,
                          cwd=ROOT, timeout=600)


def _build_oracle(src, out):
    subprocess.run(["gcc", "-std=c99", "-fopenmp", "-fPIC", "-shared", *SAN, "-o", out, src, "-lm"], check=True)


def _build_api(src, out):
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__=1", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.dirname(API), "-fPIC", "-shared", *SAN,
                    "-o", out, "-x", "c++", src, "-x", "c++", STUBS], check=True)


PINS = """
import sys
sys.path[:0] = [%r, %r]
import oracle
import oracle_pins as P
orc = oracle.Oracle(sys.argv[1])
for pin in P.ALL_PINS:
    pin(orc)
print("pins ok", len(P.ALL_PINS), flush=True)
""" % (ROOT, os.path.join(ROOT, "tests"))

TABLES = """
import ctypes, sys
sys.path[:0] = [%r, %r]
from exact_scaled_dot_sdpa_amd import _binding
import test_abi_host as T
L = _binding.bind_signatures(ctypes.CDLL(sys.argv[1]))
n = 0
for helper, cases in T.ALL_TABLES:
    for kw, status in cases:
        got = helper(L=L, **kw)
        assert got == status, (helper.__name__, kw, got, status)
        n += 1
    assert helper(L=L) == 0, helper.__name__   # the defaults are a valid call: reaches the (stubbed) launch
for args in [(16, 32, 8, 4096, 128), (1, 1, 1, 1, 64), (1, 3, 2, 100, 64)]:
    L.attn_decode_workspace_bytes(*args)
    L.attn_decode_split_workspace_bytes(*args, 100)
L.attn_bwd_workspace_bytes(2, 8, 100)
for st in range(-1, 6):
    L.attn_status_str(st)
print("tables ok", n, flush=True)
""" % (ROOT, os.path.join(ROOT, "tests"))


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _build_oracle(ORACLE_C, lib)
    r = _run(PINS, lib)
    assert r.returncode == 0 and "pins ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


def test_planted_oracle_overflow_is_caught(tmp_path):
    """A copy of the oracle whose row-max loop reads one score past the end
    of its scratch row must fail under the sanitizers."""
    src = open(ORACLE_C).read()
    old = "for (j = 1; j < nvis; ++j)\n        if (s[j] > m)"
    assert src.count(old) == 1
    bad = tmp_path / "oracle_bad.c"
    bad.write_text(src.replace(old, "for (j = 1; j <= nvis; ++j)\n        if (s[j] > m)"))
    lib = str(tmp_path / "liboracle_bad.so")
    _build_oracle(str(bad), lib)
    r = _run(PINS, lib)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]


def test_abi_layer_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libattn_host_san.so")
    _build_api(API, lib)
    r = _run(TABLES, lib)
    assert r.returncode == 0 and "tables ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


def test_planted_abi_overflow_is_caught(tmp_path):
    """A copy of the ABI layer that multiplies the decode cache rows in 32-bit
    int (B * Hkv * max_seq_len) must fail on the case table's 2^32-row call."""
    src = open(API).read()
    old = "(long long)B * Hkv * Lmax"
    assert src.count(old) == 1
    bad = tmp_path / "attn_api_bad.hip"
    bad.write_text(src.replace(old, "(long long)(B * Hkv * Lmax)"))
    lib = str(tmp_path / "libattn_host_bad.so")
    _build_api(str(bad), lib)
    r = _run(TABLES, lib)
    assert r.returncode != 0 and "runtime error" in r.stderr, r.stderr[-2000:]
