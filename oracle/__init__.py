"""fp64 CPU oracle for exact scaled dot-product attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and this package imports
nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module only marshals numpy arrays into it.  What it computes, and which page
passage each step follows, is documented at the top of ``oracle.c``:

    s_ij = scale * q_i . k_j ;  a_ij = softmax_j(s_ij) over visible j ;
    o_i = sum_j a_ij v_j ;      lse_i = ln sum_j exp(s_ij)

with bottom-right causal alignment and contiguous GQA groups, and the
gradients dq, dk, dv of that definition for an upstream gradient do of o.

Every function takes float64 arrays.  Inputs that the GPU sees as bf16 or fp32
must be widened to float64 from exactly the stored values before the call.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def _bind(path):
    lib = ctypes.CDLL(path)
    c_int, c_long, c_double = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.oracle_attn.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp] + [c_int] * 6 + [c_double, c_int, c_int]
    lib.oracle_attn.restype = c_int
    lib.oracle_attn_rows.argtypes = [_dp, _dp, _dp, _ip, c_long, _dp, _dp] + [c_int] * 6 + [c_double, c_int, c_int]
    lib.oracle_attn_rows.restype = c_int
    lib.oracle_blockwise.argtypes = [_dp, _dp, _dp, _dp, _dp] + [c_int] * 6 + [c_double, c_int, c_int, c_int]
    lib.oracle_blockwise.restype = c_int
    lib.oracle_decode.argtypes = [_dp, _dp, _dp, _ip, _dp, _dp] + [c_int] * 5 + [c_double, c_int]
    lib.oracle_decode_paged.argtypes = [_dp, _dp, _dp, _ip, _ip, _dp, _dp] + [c_int] * 7 + [c_double, c_int]
    lib.oracle_decode.restype = c_int
    lib.oracle_decode_paged.restype = c_int
    lib.oracle_attn_bwd.argtypes = [_dp] * 7 + [c_int] * 6 + [c_double, c_int, c_int]
    lib.oracle_attn_bwd.restype = c_int
    lib.oracle_attn_bwd_rows.argtypes = ([_dp] * 4 + [_ip, c_long, _ip, c_long] + [_dp] * 3 + [c_int] * 6 +
                                         [c_double, c_int, c_int])
    lib.oracle_attn_bwd_rows.restype = c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = c_int
    return lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B,H,N,d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if k.shape != v.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (q.shape, k.shape, v.shape))
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Nq, Nk, d


class Oracle:
    """The oracle bound to one compiled library (the default one, or a copy
    compiled elsewhere, e.g. a deliberately broken copy in a test)."""

    def __init__(self, lib_path):
        self.path = lib_path
        self.lib = _bind(lib_path)

    def max_threads(self) -> int:
        return self.lib.oracle_max_threads()

    def attn(self, q, k, v, scale, causal=False, weights=False, nthreads=0):
        """Direct definition.  Returns (o [B,Hq,Nq,d], lse [B,Hq,Nq]) and, with
        weights=True, also the weight matrix a [B,Hq,Nq,Nk] (0 where masked)."""
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
        q, qp = _f64(q)
        k, kp = _f64(k)
        v, vp = _f64(v)
        o = np.zeros((B, Hq, Nq, d))
        lse = np.zeros((B, Hq, Nq))
        w = np.zeros((B, Hq, Nq, Nk)) if weights else None
        rc = self.lib.oracle_attn(qp, kp, vp, o.ctypes.data_as(_dp), lse.ctypes.data_as(_dp),
                                  w.ctypes.data_as(_dp) if weights else None,
                                  B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                  int(nthreads))
        if rc:
            raise RuntimeError("oracle_attn failed")
        return (o, lse, w) if weights else (o, lse)

    def attn_rows(self, q, k, v, scale, causal, rows, nthreads=0):
        """Direct definition for selected rows only.  rows: int array [n,3] of
        (b, h, i).  Returns (o [n,d], lse [n])."""
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
        q, qp = _f64(q)
        k, kp = _f64(k)
        v, vp = _f64(v)
        rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
        n = rows.shape[0]
        o = np.zeros((n, d))
        lse = np.zeros((n,))
        rc = self.lib.oracle_attn_rows(qp, kp, vp, rows.ctypes.data_as(_ip), n,
                                       o.ctypes.data_as(_dp), lse.ctypes.data_as(_dp),
                                       B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                       int(nthreads))
        if rc:
            raise RuntimeError("oracle_attn_rows failed")
        return o, lse

    def blockwise(self, q, k, v, scale, causal, beta, nthreads=0):
        """The blockwise (m, l, u) recurrence with key blocks of size beta."""
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
        q, qp = _f64(q)
        k, kp = _f64(k)
        v, vp = _f64(v)
        o = np.zeros((B, Hq, Nq, d))
        lse = np.zeros((B, Hq, Nq))
        rc = self.lib.oracle_blockwise(qp, kp, vp, o.ctypes.data_as(_dp), lse.ctypes.data_as(_dp),
                                       B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                       int(beta), int(nthreads))
        if rc:
            raise RuntimeError("oracle_blockwise failed")
        return o, lse

    def attn_bwd(self, q, k, v, do, scale, causal=False, nthreads=0):
        """Gradients of the direct definition for the upstream gradient do
        [B,Hq,Nq,d] of o.  Returns (dq [B,Hq,Nq,d], dk [B,Hkv,Nk,d],
        dv [B,Hkv,Nk,d])."""
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
        if tuple(do.shape) != (B, Hq, Nq, d):
            raise ValueError("do must have q's shape")
        q, qp = _f64(q)
        k, kp = _f64(k)
        v, vp = _f64(v)
        do, dop = _f64(do)
        dq = np.zeros((B, Hq, Nq, d))
        dk = np.zeros((B, Hkv, Nk, d))
        dv = np.zeros((B, Hkv, Nk, d))
        rc = self.lib.oracle_attn_bwd(qp, kp, vp, dop, dq.ctypes.data_as(_dp), dk.ctypes.data_as(_dp),
                                      dv.ctypes.data_as(_dp), B, Hq, Hkv, Nq, Nk, d, float(scale),
                                      int(bool(causal)), int(nthreads))
        if rc:
            raise RuntimeError("oracle_attn_bwd failed")
        return dq, dk, dv

    def attn_bwd_rows(self, q, k, v, do, scale, causal, qrows, krows, nthreads=0):
        """Selected gradient rows: dq at qrows (int [n,3] of b, h, i) and dk, dv
        at krows (int [m,3] of b, hk, j).  Returns (dq [n,d], dk [m,d], dv [m,d])."""
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
        if tuple(do.shape) != (B, Hq, Nq, d):
            raise ValueError("do must have q's shape")
        q, qp = _f64(q)
        k, kp = _f64(k)
        v, vp = _f64(v)
        do, dop = _f64(do)
        qr = np.ascontiguousarray(qrows, dtype=np.int32).reshape(-1, 3)
        kr = np.ascontiguousarray(krows, dtype=np.int32).reshape(-1, 3)
        dq = np.zeros((qr.shape[0], d))
        dk = np.zeros((kr.shape[0], d))
        dv = np.zeros((kr.shape[0], d))
        rc = self.lib.oracle_attn_bwd_rows(qp, kp, vp, dop, qr.ctypes.data_as(_ip), qr.shape[0],
                                           kr.ctypes.data_as(_ip), kr.shape[0], dq.ctypes.data_as(_dp),
                                           dk.ctypes.data_as(_dp), dv.ctypes.data_as(_dp), B, Hq, Hkv, Nq, Nk,
                                           d, float(scale), int(bool(causal)), int(nthreads))
        if rc:
            raise RuntimeError("oracle_attn_bwd_rows failed")
        return dq, dk, dv

    def decode(self, q, k_cache, v_cache, seq_lens, scale, nthreads=0):
        """One-token decode.  q [B,Hq,d], caches [B,Hkv,Lmax,d], seq_lens [B].
        Returns (o [B,Hq,d], lse [B,Hq])."""
        if q.ndim != 3 or k_cache.ndim != 4 or k_cache.shape != v_cache.shape:
            raise ValueError("decode shapes: q [B,Hq,d], caches [B,Hkv,Lmax,d]")
        B, Hq, d = q.shape
        Bk, Hkv, Lmax, dk = k_cache.shape
        if Bk != B or dk != d or Hq % Hkv:
            raise ValueError("decode shape mismatch")
        q, qp = _f64(q)
        kc, kp = _f64(k_cache)
        vc, vp = _f64(v_cache)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seq_lens must be [B]")
        o = np.zeros((B, Hq, d))
        lse = np.zeros((B, Hq))
        rc = self.lib.oracle_decode(qp, kp, vp, sl.ctypes.data_as(_ip), o.ctypes.data_as(_dp),
                                    lse.ctypes.data_as(_dp), B, Hq, Hkv, Lmax, d, float(scale),
                                    int(nthreads))
        if rc:
            raise RuntimeError("oracle_decode failed")
        return o, lse

    def decode_paged(self, q, k_pages, v_pages, block_table, seq_lens, scale, nthreads=0):
        """One-token decode against a paged cache.  q [B,Hq,d], pages
        [num_blocks,Hkv,block_size,d], block_table int32 [B,max_blocks],
        seq_lens [B].  Returns (o [B,Hq,d], lse [B,Hq])."""
        if q.ndim != 3 or k_pages.ndim != 4 or k_pages.shape != v_pages.shape:
            raise ValueError("paged decode shapes: q [B,Hq,d], pages [num_blocks,Hkv,block_size,d]")
        B, Hq, d = q.shape
        nb, Hkv, bs, dk = k_pages.shape
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if dk != d or Hq % Hkv or bt.ndim != 2 or bt.shape[0] != B:
            raise ValueError("paged decode shape mismatch")
        q, qp = _f64(q)
        kpg, kpp = _f64(k_pages)
        vpg, vpp = _f64(v_pages)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seq_lens must be [B]")
        o = np.zeros((B, Hq, d))
        lse = np.zeros((B, Hq))
        rc = self.lib.oracle_decode_paged(qp, kpp, vpp, bt.ctypes.data_as(_ip), sl.ctypes.data_as(_ip),
                                          o.ctypes.data_as(_dp), lse.ctypes.data_as(_dp), B, Hq, Hkv, nb, bs,
                                          bt.shape[1], d, float(scale), int(nthreads))
        if rc:
            raise RuntimeError("oracle_decode_paged failed")
        return o, lse


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c next to this file (built on first use)."""
    global _default
    if _default is None:
        src = os.path.join(_HERE, "oracle.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
            from . import build as _build

            _build.build()
        _default = Oracle(_LIB_PATH)
    return _default


def max_threads() -> int:
    return default().max_threads()


def attn(*a, **kw):
    return default().attn(*a, **kw)


def attn_rows(*a, **kw):
    return default().attn_rows(*a, **kw)


def blockwise(*a, **kw):
    return default().blockwise(*a, **kw)


def decode(*a, **kw):
    return default().decode(*a, **kw)


def decode_paged(*a, **kw):
    return default().decode_paged(*a, **kw)


def attn_bwd(*a, **kw):
    return default().attn_bwd(*a, **kw)


def attn_bwd_rows(*a, **kw):
    return default().attn_bwd_rows(*a, **kw)
