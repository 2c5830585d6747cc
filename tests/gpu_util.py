"""Shared helpers of the GPU tests: run the HIP path through the binding and
compare with the fp64 oracle on the same rounded inputs."""
import sys

import numpy as np
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I

# max-abs tolerances against the fp64 oracle
TOL_O = {"f32": 1e-5, "bf16": 1.5e-2}
TOL_LSE = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.to("cuda").contiguous()


def gpu_fwd(q, k, v, scale, causal):
    """Run attn_fwd on CPU tensors; returns (o f64 numpy, lse f64 numpy)."""
    o, lse = E.attn_fwd(dev(q), dev(k), dev(v), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return I.to_f64(o), I.to_f64(lse)


def gpu_decode(seq_lens, q, kc, vc, scale, keys_per_split=0):
    o, lse = E.attn_decode(dev(q), dev(kc), dev(vc), dev(seq_lens.to(torch.int32)), scale=scale,
                           keys_per_split=keys_per_split)
    torch.cuda.synchronize()
    return I.to_f64(o), I.to_f64(lse)


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    if np.isnan(d).any():
        return float("nan")
    return float(d.max()) if d.size else 0.0


def assert_close(name, got, ref, tol):
    e = max_err(got, ref)
    say("  %-40s max-abs err %.3e (tol %.1e)" % (name, e, tol))
    assert e == e, "%s: NaN in the result" % name
    assert e <= tol, "%s: max-abs err %.3e > %.1e" % (name, e, tol)
    return e


def sample_rows(B, H, N, n_random, seed, extra_i=()):
    """(b, h, i) triples: every head's first and last rows, tile edges, plus
    n_random uniform picks."""
    rng = np.random.default_rng(seed)
    rows = set()
    edge_i = {0, 1, 2, N - 1, N - 2, min(N - 1, 127), min(N - 1, 128), N // 2} | set(extra_i)
    for b in range(B):
        for h in range(H):
            for i in (0, N - 1):
                rows.add((b, h, i))
    for b in range(B):
        for i in edge_i:
            if 0 <= i < N:
                rows.add((b, int(rng.integers(H)), i))
    for _ in range(n_random):
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))))
    return np.array(sorted(rows), dtype=np.int32)
