"""Parity of attn_bwd on fp32 inputs (the fp32 backward kernels) with the
fp64 oracle's gradients.

The HIP fp32 forward produces o and lse, the HIP fp32 backward the
gradients; the oracle computes the gradients of the definition from q, k, v
and do alone.

Tolerance (fp32).  Every product and sum is fp32: a dot product of d terms
or a sum over up to a few thousand rows carries a relative rounding error of
order sqrt(n) * 2^-24 of its terms' magnitudes (about 1e-6 here), and the
recomputed weights p inherit the forward's lse error (also about 1e-6
relative).  The cancellation in ds = p (dp - D) turns an absolute error of
that size in dp and D into one of p * 1e-6.  The test bounds max |g - ref| by
3e-5 * max |ref| + 2e-6 per tensor: about 30 times the expected error, and
more than 500 times tighter than the bf16 backward's bound, so a wrong
scale, mask, group sum or D term fails it.
"""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

TOL_REL = 3e-5
TOL_ABS = 2e-6


def gpu_fwd_bwd(q, k, v, do, scale, causal):
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = E.attn_fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = E.attn_bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float32
    return I.to_f64(dq), I.to_f64(dk), I.to_f64(dv)


def check(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), "%s: non-finite gradient" % name
    m = float(np.abs(ref).max())
    e = float(np.abs(got - ref).max())
    say("  %-30s max err %.3e (max|ref| %.3e, bound %.3e)" % (name, e, m, TOL_REL * m + TOL_ABS))
    assert e <= TOL_REL * m + TOL_ABS, "%s: max err %.3e > %.1e * %.3e + %.1e" % (name, e, TOL_REL, m, TOL_ABS)


CASES = [
    # d, B, Hq, Hkv, Nq, Nk, causal, scale
    (64, 1, 2, 1, 50, 50, False, None),
    (64, 2, 4, 2, 130, 130, True, None),
    (128, 1, 3, 3, 100, 161, True, None),   # chunked causal: Nq < Nk, bottom-right
    (128, 1, 8, 2, 200, 200, True, None),   # GQA, group of 4
    (128, 2, 2, 1, 64, 300, False, None),   # cross-attention
    (64, 1, 4, 1, 1, 77, True, None),       # one query row
    (128, 1, 2, 2, 90, 90, False, -0.1),    # negative scale
    (64, 1, 2, 1, 40, 70, False, 0.0),      # zero scale: uniform weights
    (128, 1, 16, 1, 33, 33, True, None),    # group of 16
]


@pytest.mark.parametrize("d,B,Hq,Hkv,Nq,Nk,causal,scale", CASES)
def test_bwd_f32_matches_oracle(orc, d, B, Hq, Hkv, Nq, Nk, causal, scale):
    scale = 1 / np.sqrt(d) if scale is None else scale
    q, k, v, do = I.bwd_inputs(B, Hq, Hkv, Nq, Nk, d, "f32", seed=3000 + Nq + Nk + Hq)
    say("[bwd f32] d=%d B=%d Hq=%d Hkv=%d Nq=%d Nk=%d causal=%s scale=%g" % (d, B, Hq, Hkv, Nq, Nk, causal, scale))
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, causal)
    rq, rk, rv = orc.attn_bwd(I.to_f64(q), I.to_f64(k), I.to_f64(v), I.to_f64(do), scale, causal)
    check("dq", dq, rq)
    check("dk", dk, rk)
    check("dv", dv, rv)


def test_bwd_f32_single_key_gives_zero_dq_dk(orc):
    """With one visible key per row the weights are exactly 1, so dq and dk
    vanish (ds = p (dp - D) with dp = D) and dv is the sum of do over the
    rows; the kernels leave only fp32 rounding noise in dq and dk."""
    q, k, v, do = I.bwd_inputs(1, 2, 1, 17, 1, 64, "f32", seed=3100)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, 0.125, False)
    assert np.abs(dq).max() < 1e-5 and np.abs(dk).max() < 1e-5
    ref_dv = I.to_f64(do).sum(axis=(1, 2))  # [B, d]: every row's weight on key 0 is 1
    check("dv (single key)", dv[:, 0, 0, :], ref_dv)


def test_bwd_f32_run_twice_bitwise():
    q, k, v, do = (dev(t) for t in I.bwd_inputs(1, 4, 2, 150, 150, 128, "f32", seed=3200))
    o, lse = E.attn_fwd(q, k, v, scale=0.09, causal=True)
    a = E.attn_bwd(q, k, v, o, do, lse, scale=0.09, causal=True)
    b = E.attn_bwd(q, k, v, o, do, lse, scale=0.09, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
