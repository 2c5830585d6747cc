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


def narrow_form_copies(Nq):
    """Copies of one head that give the forward a grid of at least two
    128-row workgroups per CU.  A causal grid of fewer than one per CU runs
    the key-split form, which adds its sums in another order; copies of a
    head in this many heads run the 4-wave 128-row form, whose row
    arithmetic the wider forms share."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return -(-2 * cus // -(-Nq // 128))


def one_head(t, b, h, copies):
    """Head h of batch entry b as a [1, copies, N, d] tensor."""
    return t[b:b + 1, h:h + 1].repeat(1, copies, 1, 1)


def gpu_decode(seq_lens, q, kc, vc, scale, keys_per_split=0):
    """attn_decode (default split), or attn_decode_split for keys_per_split > 0."""
    if keys_per_split:
        o, lse = E.attn_decode_split(dev(q), dev(kc), dev(vc), dev(seq_lens.to(torch.int32)), keys_per_split,
                                     scale=scale)
    else:
        o, lse = E.attn_decode(dev(q), dev(kc), dev(vc), dev(seq_lens.to(torch.int32)), scale=scale)
    torch.cuda.synchronize()
    return I.to_f64(o), I.to_f64(lse)


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):  # inf - inf of equal infinities is masked out here
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


def assert_rel_per_group(name, got, ref, group_axes, rel=2.0 ** -6):
    """Per group of outputs (the leading `group_axes` axes index a group:
    a sequence, or a (batch, head) pair), max |got - ref| <= rel * max |ref|
    of that group.  Over many keys softmax(QK^T)V shrinks towards 0 (about
    sqrt(e / L) for L keys of N(0,1) values), so the absolute bf16 bound
    alone would pass even an all-zero output; 2^-6 leaves room for the
    output's bf16 rounding (2^-9 relative) plus the weights' (2^-9 relative
    each, averaged over the keys) several times over."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lead = got.shape[:group_axes]
    g = got.reshape(int(np.prod(lead)), -1)
    r = ref.reshape(int(np.prod(lead)), -1)
    err = np.abs(g - r).max(axis=1)
    top = np.abs(r).max(axis=1)
    ratio = float((err / np.maximum(top, 1e-300)).max())
    say("  %-40s max err / max|ref| per group %.3e (bound %.3e)" % (name, ratio, rel))
    assert np.all(err <= rel * top), "%s: relative error %.3e > %.3e" % (name, ratio, rel)


def grad_floors(orc, q, k, v, do, scale, causal):
    """Absolute error floors for the gradient checks, which are otherwise
    relative to each reference tensor's largest entry.  ds = p (dp - D)
    cancels: where a row sees a single key it is exactly 0 by definition (o is
    that key's v), while the kernels form dp on the MFMA and D = do . o in
    another summation order, so ds is fp32 rounding noise of at most
    eps = d 2^-22 max|do| max|v| per entry (16 d unit roundoffs of the
    products' scale), and a reference that is 0 everywhere (every row sees one
    key) leaves the relative bound no room for it.  That noise reaches
      dq_i = scale sum_j ds_ij k_j  weighted by p_ij, which sums to 1 over j:
             floor |scale| max|k| eps;
      dk_j = scale sum_i ds_ij q_i  weighted by the column sums of P (over the
             query rows and the heads that share key j): floor |scale| max|q|
             eps max_j sum_i p_ij, the column sums read off the oracle's dv
             for do = 1;
      dv   has no such cancellation: floor 0."""
    q64, k64, v64, do64 = (I.to_f64(t) for t in (q, k, v, do))
    if q64.size == 0 or k64.size == 0:
        return {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    eps = q64.shape[3] * 2.0 ** -22 * np.abs(do64).max() * np.abs(v64).max()
    col = orc.attn_bwd(q64, k64, v64, np.ones_like(do64), scale, causal)[2]
    return {"dq": abs(scale) * np.abs(k64).max() * eps,
            "dk": abs(scale) * np.abs(q64).max() * eps * float(np.abs(col).max()),
            "dv": 0.0}


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
