"""Host-side checks of libattn.so (CPU only): the library loads, exports every
entry point include/attn.h declares, and rejects invalid arguments before any
HIP runtime call.  No call made here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import exact_scaled_dot_sdpa_amd as E

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

P = 1 << 20  # a 16-byte aligned fake device address; never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names == sorted(["attn_fwd", "attn_decode", "attn_decode_paged", "attn_decode_workspace_bytes",
                            "attn_bwd", "attn_bwd_workspace_bytes", "attn_fwd_fp8", "attn_status_str"])
    lib = ctypes.CDLL(E.lib_path())
    for n in names:
        assert hasattr(lib, n), "libattn.so does not export %s" % n


def test_status_strings():
    assert E.attn_status_str(0) == "ATTN_OK"
    assert E.attn_status_str(1) == "ATTN_ERR_INVALID_ARG"
    assert E.attn_status_str(2) == "ATTN_ERR_UNSUPPORTED"
    assert E.attn_status_str(3) == "ATTN_ERR_WORKSPACE"
    assert E.attn_status_str(4) == "ATTN_ERR_LAUNCH"
    assert E.attn_status_str(99) == "ATTN_ERR_UNKNOWN"


def fwd(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, scale=0.125, causal=0, dtype=1):
    return E.lib().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=3, Hkv=2), E.ATTN_ERR_INVALID_ARG),        # Hq % Hkv != 0
    (dict(Hq=0), E.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=0), E.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(Nq=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(Nk=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(d=96), E.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), E.ATTN_ERR_UNSUPPORTED),
    (dict(causal=1, Nq=9, Nk=8), E.ATTN_ERR_INVALID_ARG),  # causal needs Nq <= Nk
    (dict(scale=float("nan")), E.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), E.ATTN_ERR_INVALID_ARG),
    (dict(dtype=7), E.ATTN_ERR_INVALID_ARG),
    (dict(q=None), E.ATTN_ERR_INVALID_ARG),
    (dict(o=None), E.ATTN_ERR_INVALID_ARG),
    (dict(k=None), E.ATTN_ERR_INVALID_ARG),
    (dict(q=P + 2), E.ATTN_ERR_INVALID_ARG),            # misaligned
    (dict(v=P + 8), E.ATTN_ERR_INVALID_ARG),
    (dict(lse=P + 2), E.ATTN_ERR_INVALID_ARG),
    (dict(B=0), E.ATTN_OK),                              # empty: no-op
    (dict(Nq=0), E.ATTN_OK),
    (dict(Nq=0, Nk=0, causal=1), E.ATTN_OK),
])
def test_fwd_validation(kw, status):
    assert fwd(**kw) == status


def dec(q=P, kc=P, vc=P, sl=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Lmax=512, d=128, scale=0.09, kps=0, dtype=1,
        ws=P, ws_bytes=1 << 30):
    return E.lib().attn_decode(q, kc, vc, sl, o, lse, B, Hq, Hkv, Lmax, d, scale, kps, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), E.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(Lmax=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), E.ATTN_ERR_INVALID_ARG),
    (dict(kps=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(dtype=0), E.ATTN_ERR_UNSUPPORTED),            # fp32 decode not implemented
    (dict(d=96), E.ATTN_ERR_UNSUPPORTED),
    (dict(sl=None), E.ATTN_ERR_INVALID_ARG),
    (dict(sl=P + 2), E.ATTN_ERR_INVALID_ARG),
    (dict(q=None), E.ATTN_ERR_INVALID_ARG),
    (dict(kc=P + 4), E.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), E.ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=1024), E.ATTN_ERR_WORKSPACE),
    (dict(ws=P + 4), E.ATTN_ERR_WORKSPACE),
    (dict(B=0), E.ATTN_OK),
])
def test_decode_validation(kw, status):
    assert dec(**kw) == status


def _ws_bytes(B, Hq, Hkv, Lmax, d, kps):
    """The workspace size the header documents: slots of min(G, 16) heads,
    one per (sequence, K/V head, block of 16 query heads) plus one per split
    workgroup beyond the first; fp32 outputs, then (256-byte aligned) fp32
    LSEs."""
    G = Hq // Hkv
    nhb = -(-G // 16)
    gb = min(G, 16)
    if kps > 0:
        n_wg = min(max(-(-(B * Hkv * nhb * Lmax) // kps), 1), 2048)
    else:
        n_wg = 2048
    rows = (B * Hkv * nhb + n_wg - 1) * gb
    return -(-(rows * d * 4) // 256) * 256 + rows * 4


def test_decode_workspace_bytes():
    f = E.attn_decode_workspace_bytes
    for args in [(16, 32, 8, 4096, 128, 0), (16, 32, 8, 4096, 128, 1024), (1, 1, 1, 0, 64, 0),
                 (3, 6, 2, 100, 64, 0), (2, 64, 2, 777, 128, 100), (2, 40, 2, 300, 64, 7)]:
        assert f(*args) == _ws_bytes(*args), args
    # 16 x 8 segments + 512 workgroups of 1024 keys - 1, four heads each
    assert f(16, 32, 8, 4096, 128, 1024) == 639 * 4 * 128 * 4 + 639 * 4 * 4
    assert f(1, 3, 2, 100, 64) == 0                  # invalid sizes
    assert f(1, 2, 1, 100, 96) == 0
    assert f(1, 2, 1, 100, 64, -1) == 0
    # exactly the workspace that size reports is accepted, one byte less is not
    need = f(2, 8, 2, 512, 128)
    assert dec(ws_bytes=need - 1) == E.ATTN_ERR_WORKSPACE


def pdec(q=P, kp=P, vp=P, bt=P, sl=P, o=P, lse=P, B=2, Hq=8, Hkv=2, nb=16, bs=32, mb=8, d=128, scale=0.09, kps=0,
         dtype=1, ws=P, ws_bytes=1 << 30):
    return E.lib().attn_decode_paged(q, kp, vp, bt, sl, o, lse, B, Hq, Hkv, nb, bs, mb, d, scale, kps, dtype, ws,
                                     ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(nb=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(bs=0), E.ATTN_ERR_INVALID_ARG),
    (dict(mb=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(bt=None), E.ATTN_ERR_INVALID_ARG),
    (dict(bt=P + 2), E.ATTN_ERR_INVALID_ARG),
    (dict(mb=1 << 20, bs=1 << 12), E.ATTN_ERR_UNSUPPORTED),     # max_blocks * block_size >= 2^31
    (dict(nb=1 << 20, bs=1 << 10), E.ATTN_ERR_UNSUPPORTED),     # pool rows >= 2^31
    (dict(Hq=6, Hkv=4), E.ATTN_ERR_INVALID_ARG),
    (dict(dtype=0), E.ATTN_ERR_UNSUPPORTED),
    (dict(d=96), E.ATTN_ERR_UNSUPPORTED),
    (dict(kp=None), E.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), E.ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=1024), E.ATTN_ERR_WORKSPACE),
    (dict(B=0), E.ATTN_OK),
])
def test_decode_paged_validation(kw, status):
    assert pdec(**kw) == status


def test_decode_paged_workspace_is_the_contiguous_one():
    """Sized like attn_decode with max_seq_len = max_blocks * block_size: one
    byte less is refused (a sufficient size would launch, so it is not tried
    here)."""
    need = E.attn_decode_workspace_bytes(2, 8, 2, 8 * 32, 128)
    assert pdec(ws_bytes=need - 1) == E.ATTN_ERR_WORKSPACE


def bwd(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=128, scale=0.09,
        causal=0, dtype=1, ws=P, ws_bytes=1 << 30):
    return E.lib().attn_bwd(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, ws,
                            ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=3, Hkv=2), E.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=0), E.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(Nq=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(causal=1, Nq=65), E.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), E.ATTN_ERR_INVALID_ARG),
    (dict(dtype=5), E.ATTN_ERR_INVALID_ARG),
    (dict(dtype=0), E.ATTN_ERR_UNSUPPORTED),             # fp32 backward not implemented
    (dict(d=32), E.ATTN_ERR_UNSUPPORTED),
    (dict(lse=None), E.ATTN_ERR_INVALID_ARG),
    (dict(do=None), E.ATTN_ERR_INVALID_ARG),
    (dict(dq=None), E.ATTN_ERR_INVALID_ARG),
    (dict(dv=None), E.ATTN_ERR_INVALID_ARG),
    (dict(k=None), E.ATTN_ERR_INVALID_ARG),
    (dict(o=P + 8), E.ATTN_ERR_INVALID_ARG),             # misaligned
    (dict(dk=P + 2), E.ATTN_ERR_INVALID_ARG),
    (dict(lse=P + 2), E.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), E.ATTN_ERR_WORKSPACE),
    (dict(ws=P + 4), E.ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=1 * 4 * 64 * 8 - 1), E.ATTN_ERR_WORKSPACE),
    (dict(Nq=1 << 16, Nk=1 << 16, Hq=1 << 15, Hkv=1 << 15), E.ATTN_ERR_UNSUPPORTED),  # rows >= 2^31
    (dict(B=0), E.ATTN_OK),
    (dict(Nq=0, Nk=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None, ws=None),
     E.ATTN_OK),
])
def test_bwd_validation(kw, status):
    assert bwd(**kw) == status


def test_bwd_workspace_bytes():
    assert E.attn_bwd_workspace_bytes(2, 8, 100) == 2 * 8 * 100 * 8
    assert E.attn_bwd_workspace_bytes(0, 8, 100) == 0
    assert E.attn_bwd_workspace_bytes(1, 0, 100) == 0
    assert E.attn_bwd_workspace_bytes(1, 4, -1) == 0


def fwd8(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128, scale=0.09, v_scale=1.0, causal=0):
    return E.lib().attn_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, v_scale, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=3, Hkv=2), E.ATTN_ERR_INVALID_ARG),
    (dict(Nk=-1), E.ATTN_ERR_INVALID_ARG),
    (dict(causal=1, Nq=9), E.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), E.ATTN_ERR_INVALID_ARG),
    (dict(v_scale=float("nan")), E.ATTN_ERR_INVALID_ARG),
    (dict(d=80), E.ATTN_ERR_UNSUPPORTED),
    (dict(q=None), E.ATTN_ERR_INVALID_ARG),
    (dict(v=None), E.ATTN_ERR_INVALID_ARG),
    (dict(k=P + 8), E.ATTN_ERR_INVALID_ARG),
    (dict(lse=P + 1), E.ATTN_ERR_INVALID_ARG),
    (dict(B=0), E.ATTN_OK),
    (dict(Nq=0), E.ATTN_OK),
])
def test_fwd_fp8_validation(kw, status):
    assert fwd8(**kw) == status
