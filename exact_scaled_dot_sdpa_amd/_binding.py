"""ctypes binding of libattn.so.  Argument marshalling only."""
import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_LAUNCH = 0, 1, 2, 3, 4

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s failed: %s (%d)" % (what, attn_status_str(status), status))
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            "libattn.so is not built (expected at %s); run `python -m exact_scaled_dot_sdpa_amd.build`"
            % _LIB_PATH)
    L = bind_signatures(ctypes.CDLL(_LIB_PATH))
    _lib = L
    return L


def bind_signatures(L):
    """Set the argument and result types of every entry point of include/attn.h
    on the ctypes library L; returns L."""
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd.restype = i
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode_split_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_decode_split_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_decode.restype = i
    L.attn_decode_split.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.attn_decode_split.restype = i
    L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_decode_noalloc.restype = i
    L.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.attn_decode_paged.restype = i
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, i, vp]
    L.attn_fwd_fp8.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [vp] * 9 + [i] * 6 + [f, i, i, vp, sz, vp]
    L.attn_bwd.restype = i
    L.attn_status_str.argtypes = [i]
    L.attn_status_str.restype = ctypes.c_char_p
    return L


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _check_dev(name, t, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _stream_handle(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def attn_fwd(q, k, v, scale=None, causal=False, o=None, lse=None, return_lse=True, stream=None):
    """O = softmax(scale * Q K^T [+ causal mask]) V for q [B,Hq,Nq,d],
    k/v [B,Hkv,Nk,d] (device tensors, bf16 or fp32, contiguous).
    Returns (o, lse) (lse fp32 [B,Hq,Nq]) or o when return_lse is False."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] expected")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("batch or head-dim mismatch: q %s k %s" % (tuple(q.shape), tuple(k.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _check_dev("o", o, q.dtype)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq, Nq):
            raise ValueError("lse must be [B,Hq,Nq]")
    st = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        lse.data_ptr() if lse is not None else None,
                        B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _dtype_code(q),
                        _stream_handle(q, stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return (o, lse) if return_lse else o


def attn_fwd_fp8(q, k, v, scale=None, v_scale=1.0, causal=False, o=None, lse=None, return_lse=True, stream=None):
    """attn_fwd for q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] in torch.float8_e4m3fn:
    O = v_scale * softmax(scale * Q K^T [+ causal mask]) V in bf16.  Returns
    (o, lse) or o."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.float8_e4m3fn)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] expected")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("batch or head-dim mismatch: q %s k %s" % (tuple(q.shape), tuple(k.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check_dev("o", o, torch.bfloat16)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq, Nq):
            raise ValueError("lse must be [B,Hq,Nq]")
    st = lib().attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Nq, Nk, d, float(scale),
                            float(v_scale), int(bool(causal)), _stream_handle(q, stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8")
    return (o, lse) if return_lse else o


def attn_bwd_workspace_bytes(B, Hq, Nq) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Nq))


def attn_bwd(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """Gradients (dq, dk, dv) of attn_fwd for the upstream gradient dout of o.
    q, o, dout [B,Hq,Nq,d] and k, v [B,Hkv,Nk,d] bf16, lse fp32 [B,Hq,Nq]
    (attn_fwd's outputs for the same q, k, v, scale, causal)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_dev(name, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q/o/dout [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] expected")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if Bk != B or dk_ != d or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("attn_bwd shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_dev(name, t, q.dtype)
        if t.shape != ref.shape:
            raise ValueError("%s must have %s's shape" % (name, "q" if ref is q else "k"))
    need = attn_bwd_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                        int(bool(causal)), _dtype_code(q), workspace.data_ptr(), ws_bytes,
                        _stream_handle(q, stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def attn_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, d) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, d))


def attn_decode_split_workspace_bytes(B, Hq, Hkv, max_seq_len, d, keys_per_split) -> int:
    return int(lib().attn_decode_split_workspace_bytes(B, Hq, Hkv, max_seq_len, d, keys_per_split))


def _decode_outputs(q, o, lse, return_lse):
    """Caller-supplied or new o [B,Hq,d] (q's dtype) and lse fp32 [B,Hq]."""
    torch = _torch()
    B, Hq, _ = q.shape
    if o is None:
        o = torch.empty_like(q)
    _check_dev("o", o, q.dtype)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape %s, got %s" % (tuple(q.shape), tuple(o.shape)))
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B,Hq] = %s, got %s" % ((B, Hq), tuple(lse.shape)))
    return o, lse


def _workspace(workspace, need, device):
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _check_dev("workspace", workspace)
    return workspace, workspace.numel() * workspace.element_size()


def _decode_shapes(q, k_cache, v_cache, seq_lens):
    torch = _torch()
    _check_dev("q", q)
    _check_dev("k_cache", k_cache, q.dtype)
    _check_dev("v_cache", v_cache, q.dtype)
    _check_dev("seq_lens", seq_lens, torch.int32)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [B,Hq,d], caches [B,Hkv,Lmax,d] expected")
    B, Hq, d = q.shape
    Bk, Hkv, Lmax, dk = k_cache.shape
    if Bk != B or dk != d or tuple(seq_lens.shape) != (B,):
        raise ValueError("decode shape mismatch")
    return B, Hq, Hkv, Lmax, d


def attn_decode(q, k_cache, v_cache, seq_lens, scale=None, o=None, lse=None, workspace=None, return_lse=True,
                stream=None):
    """One decode step: q [B,Hq,d] against caches [B,Hkv,Lmax,d] (bf16) with
    seq_lens int32 [B] on the device.  Returns (o, lse) or o."""
    B, Hq, Hkv, Lmax, d = _decode_shapes(q, k_cache, v_cache, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _decode_outputs(q, o, lse, return_lse)
    workspace, ws_bytes = _workspace(workspace, attn_decode_workspace_bytes(B, Hq, Hkv, Lmax, d), q.device)
    st = lib().attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                           o.data_ptr(), lse.data_ptr() if lse is not None else None,
                           B, Hq, Hkv, Lmax, d, float(scale), _dtype_code(q),
                           workspace.data_ptr(), ws_bytes, _stream_handle(q, stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode")
    return (o, lse) if return_lse else o


def attn_decode_noalloc(q, k_cache, v_cache, seq_lens, o, lse=None, scale=None, stream=None):
    """attn_decode with no workspace: the partial results go to the library's
    own device array (ATTN_DECODE_NOALLOC_MAX_BYTES), so the call allocates
    nothing.  o [B,Hq,d] and lse [B,Hq] (or None) are the caller's.  Calls
    that overlap in time on one device share that array and race."""
    B, Hq, Hkv, Lmax, d = _decode_shapes(q, k_cache, v_cache, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_dev("o", o, q.dtype)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape %s, got %s" % (tuple(q.shape), tuple(o.shape)))
    if lse is not None:
        _check_dev("lse", lse, _torch().float32)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B,Hq] = %s, got %s" % ((B, Hq), tuple(lse.shape)))
    st = lib().attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                   o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                   B, Hq, Hkv, Lmax, d, float(scale), _dtype_code(q), _stream_handle(q, stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_noalloc")
    return o, lse


def attn_decode_split(q, k_cache, v_cache, seq_lens, keys_per_split, scale=None, o=None, lse=None, workspace=None,
                      return_lse=True, stream=None):
    """attn_decode with an explicit split: ranges of about keys_per_split keys
    of the max_seq_len-sized cache (0: the default split)."""
    B, Hq, Hkv, Lmax, d = _decode_shapes(q, k_cache, v_cache, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _decode_outputs(q, o, lse, return_lse)
    need = attn_decode_split_workspace_bytes(B, Hq, Hkv, Lmax, d, keys_per_split)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    st = lib().attn_decode_split(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                 o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                 B, Hq, Hkv, Lmax, d, float(scale), int(keys_per_split), _dtype_code(q),
                                 workspace.data_ptr(), ws_bytes, _stream_handle(q, stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_split")
    return (o, lse) if return_lse else o


def attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale=None, o=None, lse=None, workspace=None,
                      keys_per_split=0, return_lse=True, stream=None):
    """One decode step against a paged cache: q [B,Hq,d], pools k_pages /
    v_pages [num_blocks,Hkv,block_size,d] (bf16), block_table int32
    [B,max_blocks_per_seq] and seq_lens int32 [B] on the device.  Returns
    (o, lse) or o."""
    torch = _torch()
    _check_dev("q", q)
    _check_dev("k_pages", k_pages, q.dtype)
    _check_dev("v_pages", v_pages, q.dtype)
    _check_dev("block_table", block_table, torch.int32)
    _check_dev("seq_lens", seq_lens, torch.int32)
    if q.dim() != 3 or k_pages.dim() != 4 or k_pages.shape != v_pages.shape or block_table.dim() != 2:
        raise ValueError("q [B,Hq,d], pools [num_blocks,Hkv,block_size,d], block_table [B,max_blocks] expected")
    B, Hq, d = q.shape
    nb, Hkv, bs, dk = k_pages.shape
    if dk != d or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("paged decode shape mismatch")
    mb = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _decode_outputs(q, o, lse, return_lse)
    need = attn_decode_split_workspace_bytes(B, Hq, Hkv, mb * bs, d, keys_per_split)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    st = lib().attn_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                 seq_lens.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                 B, Hq, Hkv, nb, bs, mb, d, float(scale), int(keys_per_split), _dtype_code(q),
                                 workspace.data_ptr(), ws_bytes, _stream_handle(q, stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged")
    return (o, lse) if return_lse else o
