"""Seeded synthetic inputs and the workload table.

This module holds no attention arithmetic.  It only draws iid N(0, 1) values
from a seeded CPU ``torch.Generator`` (in fp32, then rounded to nearest even to
the workload's element type: fp32, bf16 or fp8 e4m3) and describes the workload shapes.  The HIP path
and the oracle consume the very same rounded values.

Draw order is fixed: q, k, v for prefill (then do for the backward pass);
seq_lens, q, k_cache, v_cache for decode; seq_lens, q, k_pages, v_pages, block order for paged decode.
seq_lens are uniform integers in [lo, hi] inclusive.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


@dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str
    causal: bool
    seed: int
    note: str = ""
    Nk: int = 0  # key/value length; 0 = N (self-attention)

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    @property
    def Nq(self) -> int:
        return self.N

    @property
    def Nkv(self) -> int:
        return self.Nk if self.Nk > 0 else self.N


@dataclass(frozen=True)
class Decode:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lmax: int
    d: int
    dtype: str
    lo: int
    hi: int
    seed: int
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


# The workloads.  Seeds are 1000 + the workload's position in this list.
WORKLOADS = {
    "C1": Prefill("C1", 1, 1, 1, 128, 64, "f32", False, 1000,
                  "single head, fp32, with the invariant probes"),
    "C2a": Prefill("C2a", 4, 12, 12, 1024, 64, "bf16", False, 1001,
                   "GPT-2-small-shaped MHA prefill, non-causal"),
    "C2b": Prefill("C2b", 4, 12, 12, 1024, 64, "bf16", True, 1001,
                   "GPT-2-small-shaped MHA prefill, causal"),
    "C3a": Prefill("C3a", 1, 12, 12, 2048, 64, "bf16", True, 1002,
                   "12-head d_model=768 layer at N=2048"),
    "C3a'": Prefill("C3a'", 1, 32, 32, 2048, 128, "bf16", True, 1002,
                    "32 heads of 128 at N=2048 (literal reading of the config)"),
    "C3b": Prefill("C3b", 1, 32, 32, 4096, 128, "bf16", True, 1002,
                   "LLaMA-7B-shaped layer at N=4096"),
    "C4": Prefill("C4", 1, 64, 8, 8192, 128, "bf16", True, 1003,
                  "GQA prefill, 64 query heads over 8 KV heads, one 70B-class layer"),
    "C5": Decode("C5", 16, 32, 8, 4096, 128, "bf16", 512, 4096, 1004,
                 "KV-cache decode, 16 sequences, 32 Q heads over 8 KV heads"),
    "X1": Prefill("X1", 1, 64, 8, 2048, 128, "bf16", True, 1005,
                  "chunked prefill: a 2048-token chunk attending causally (bottom-right) to 8192 "
                  "cached tokens plus itself, on the GQA layer's heads", Nk=10240),
    "X2": Prefill("X2", 4, 16, 16, 2048, 128, "bf16", False, 1006,
                  "cross-attention: 2048 decoder queries over 4096 encoder keys, non-causal", Nk=4096),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(shape, dtype: str, g: torch.Generator) -> torch.Tensor:
    """iid N(0,1) drawn in fp32, rounded to nearest even to ``dtype``."""
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x.to(DTYPES[dtype])


def prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed):
    """q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] on the CPU, in ``dtype``."""
    g = _gen(seed)
    q = randn((B, Hq, Nq, d), dtype, g)
    k = randn((B, Hkv, Nk, d), dtype, g)
    v = randn((B, Hkv, Nk, d), dtype, g)
    return q, k, v


def bwd_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed):
    """q, k, v as ``prefill_inputs`` with the same seed, then the upstream
    gradient do [B,Hq,Nq,d] (iid N(0, 1) like the rest)."""
    g = _gen(seed)
    q = randn((B, Hq, Nq, d), dtype, g)
    k = randn((B, Hkv, Nk, d), dtype, g)
    v = randn((B, Hkv, Nk, d), dtype, g)
    do = randn((B, Hq, Nq, d), dtype, g)
    return q, k, v, do


def decode_inputs(B, Hq, Hkv, Lmax, d, dtype, seed, lo=512, hi=4096,
                  seq_lens: Optional[torch.Tensor] = None):
    """(seq_lens int32 [B], q [B,Hq,d], k_cache/v_cache [B,Hkv,Lmax,d]) on the CPU."""
    g = _gen(seed)
    drawn = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)
    if seq_lens is None:
        seq_lens = drawn
    seq_lens = seq_lens.to(torch.int32).clamp(max=Lmax)
    q = randn((B, Hq, d), dtype, g)
    kc = randn((B, Hkv, Lmax, d), dtype, g)
    vc = randn((B, Hkv, Lmax, d), dtype, g)
    return seq_lens, q, kc, vc


def paged_decode_inputs(B, Hq, Hkv, d, block_size, max_blocks, dtype, seed, lo=512, hi=4096, spare_blocks=0):
    """A paged KV cache holding the same kind of data as ``decode_inputs``:
    (seq_lens int32 [B], q [B,Hq,d], k_pages/v_pages [num_blocks,Hkv,block_size,d],
    block_table int32 [B,max_blocks]) on the CPU.  The pool has exactly the
    blocks the sequences' lengths need plus ``spare_blocks`` unused ones, in
    a seeded random order; table entries past a sequence's last block point
    at pool block 0 (they are never read)."""
    g = _gen(seed)
    Lmax = max_blocks * block_size
    seq_lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).clamp(max=Lmax).to(torch.int32)
    nblk = [(int(L) + block_size - 1) // block_size for L in seq_lens]
    num_blocks = sum(nblk) + spare_blocks
    q = randn((B, Hq, d), dtype, g)
    kp = randn((num_blocks, Hkv, block_size, d), dtype, g)
    vp = randn((num_blocks, Hkv, block_size, d), dtype, g)
    order = torch.randperm(num_blocks, generator=g).to(torch.int32)
    table = torch.zeros((B, max_blocks), dtype=torch.int32)
    at = 0
    for b in range(B):
        table[b, :nblk[b]] = order[at:at + nblk[b]]
        at += nblk[b]
    return seq_lens, q, kp, vp, table


def workload_inputs(name: str, seed_offset: int = 0):
    """Inputs of a named workload (prefill: (q,k,v); decode: (seq_lens,q,kc,vc))."""
    w = WORKLOADS[name]
    if isinstance(w, Prefill):
        return prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, w.dtype, w.seed + seed_offset)
    return decode_inputs(w.B, w.Hq, w.Hkv, w.Lmax, w.d, w.dtype, w.seed + seed_offset, w.lo, w.hi)


def to_f64(t: torch.Tensor):
    """Widen exactly-stored values to a float64 numpy array (for the oracle)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
