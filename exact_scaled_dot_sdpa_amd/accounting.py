"""FLOP and byte accounting for the roofline figures.

Counting rules (algorithmic work only, never the work a kernel avoids or wastes):
  * FLOPs are matrix FLOPs: 2*d for q.k plus 2*d for p*v per VISIBLE (query,
    key) pair; exp, max and sum are not counted.  A causal square head has
    N(N+1)/2 visible pairs.
  * Bytes are the compulsory device-memory bytes: read q, k, v once, write o
    and lse once; for decode, read only the valid cache rows.

Byte formulas from the pages (cited by title and section):
  * "从注意力到 IO 感知执行" (auturnal.com review), sec. 4 and sec. 6: one
    head's fp32 score matrix takes n^2 * 4 bytes, i.e. 1, 4, 16 and 64 MiB at
    n = 512, 1024, 2048, 4096; sec. 9 / eq. (3): a KV cache takes
    2 * L * n * h_kv * d_h * b bytes.
  * pwwt.cn engineering blog, sec. 2.1 (64 MB for one fp32 head at n=4096),
    sec. 3.2 (LLaMA-7B: 32 MB per layer at n=2048 in FP16) and sec. 7.3
    (32 layers at n=8192: about 4 GB).
"""
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def visible_pairs(Nq: int, Nk: int, causal: bool) -> int:
    """Number of (query, key) pairs that survive the mask for one head
    (bottom-right causal alignment: row i sees keys 0 .. i + Nk - Nq)."""
    if not causal:
        return Nq * Nk
    off = Nk - Nq
    return sum(max(0, min(Nk, i + off + 1)) for i in range(Nq))


def prefill_flops(B, Hq, Nq, Nk, d, causal) -> int:
    return 4 * d * B * Hq * visible_pairs(Nq, Nk, causal)


def bwd_flops(B, Hq, Nq, Nk, d, causal) -> int:
    """Backward-pass matrix FLOPs: five products per visible pair (the
    recomputed scores, dP, dV, dK, dQ), 2*d each, i.e. 2.5x the forward."""
    return 10 * d * B * Hq * visible_pairs(Nq, Nk, causal)


def prefill_bytes(B, Hq, Hkv, Nq, Nk, d, dtype, with_lse=True) -> int:
    """Read q, k, v once and write o (and lse); fp8 inputs give a bf16 o."""
    e = ELEM_BYTES[dtype]
    eo = 2 if dtype == "fp8" else e
    b = e * (B * Hq * Nq * d + 2 * B * Hkv * Nk * d) + eo * B * Hq * Nq * d
    if with_lse:
        b += 4 * B * Hq * Nq
    return b


def decode_flops(seq_lens, Hq, d) -> int:
    return 4 * d * Hq * int(sum(int(x) for x in seq_lens))


def decode_bytes(seq_lens, Hq, Hkv, d, dtype, with_lse=True) -> int:
    """Valid cache rows of K and V, plus q and o, lse and the seq_lens vector."""
    e = ELEM_BYTES[dtype]
    B = len(seq_lens)
    L = int(sum(int(x) for x in seq_lens))
    b = 2 * L * Hkv * d * e + 2 * B * Hq * d * e + 4 * B
    if with_lse:
        b += 4 * B * Hq
    return b


def score_matrix_bytes(n: int, elem_bytes: int = 4, heads: int = 1) -> int:
    """Bytes of an explicit n x n score matrix per head (what the fused
    kernel never writes)."""
    return n * n * elem_bytes * heads


def kv_cache_bytes(layers: int, n: int, h_kv: int, d_h: int, elem_bytes: int,
                   batch: int = 1) -> int:
    """M_KV = 2 * L * n * h_kv * d_h * b, times the batch."""
    return 2 * layers * n * h_kv * d_h * elem_bytes * batch
