"""Parity of attn_bwd (the HIP backward kernels) with the fp64 oracle.

The HIP forward produces o and lse, the HIP backward the gradients; the
oracle computes the gradients of the definition from q, k, v and do alone.

Tolerance (bf16).  Each gradient goes through at most three roundings to
bf16 on the way -- o (read back for D_i = do_i . o_i), the weights p or ds as
MFMA operands, and the output -- each at most 2^-9 relative, with fp32
accumulation in between.  Compared with the largest magnitude of the
gradient tensor this stays below 3 * 2^-9 = 5.9e-3 per contribution; sums of
such errors over rows grow more slowly than the sums themselves.  The test
bounds max |g - ref| by 2e-2 * max |ref| per tensor (about five bf16 ulps of
the largest entry) and the RMS error by 6e-3 * RMS(ref), each plus an absolute
floor for dq and dk at the fp32 rounding scale of the cancellation in
ds = p (dp - D) (gpu_util.grad_floors): with a single key in every row, dq and
dk are exactly zero and the kernels return rounding noise.
"""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import dev, grad_floors, narrow_form_copies, one_head, say

pytestmark = pytest.mark.gpu

TOL_MAX = 2e-2
TOL_RMS = 6e-3


def gpu_fwd_bwd(q, k, v, do, scale, causal):
    """HIP forward then HIP backward on CPU tensors; returns f64 numpy (dq, dk, dv)."""
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = E.attn_fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = E.attn_bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return I.to_f64(dq), I.to_f64(dk), I.to_f64(dv)


def check_grad(name, got, ref, floor=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "%s: non-finite gradient" % name
    if ref.size == 0:
        return
    scale_max = float(np.abs(ref).max())
    scale_rms = float(np.sqrt(np.mean(ref ** 2)))
    e_max = float(np.abs(got - ref).max())
    e_rms = float(np.sqrt(np.mean((got - ref) ** 2)))
    say("  %-34s max err %.3e = %.2e of max|ref| %.3e; rms err %.2e of rms" %
        (name, e_max, e_max / max(scale_max, 1e-300), scale_max, e_rms / max(scale_rms, 1e-300)))
    assert e_max <= TOL_MAX * scale_max + floor, "%s: max err %.3e > %.1e * %.3e + %.1e" % (
        name, e_max, TOL_MAX, scale_max, floor)
    assert e_rms <= TOL_RMS * scale_rms + floor, "%s: rms err %.3e > %.1e * %.3e + %.1e" % (
        name, e_rms, TOL_RMS, scale_rms, floor)


CASES = [
    # d, B, Hq, Hkv, Nq, Nk, causal
    (128, 2, 4, 2, 200, 200, True),
    (128, 2, 4, 2, 200, 200, False),
    (64, 1, 3, 1, 77, 300, False),     # cross-attention, rectangular
    (128, 1, 2, 2, 100, 333, True),    # chunked prefill (bottom-right)
    (64, 3, 2, 2, 1, 1, True),
    (128, 1, 8, 1, 65, 129, True),     # MQA
    (64, 1, 16, 2, 129, 63, False),    # Nk below one tile
    (128, 1, 1, 1, 1000, 1000, True),
    (128, 2, 16, 4, 520, 700, True),   # GQA chunked, ragged tails on both sides
    (64, 2, 8, 8, 300, 257, False),
    (64, 1, 4, 1, 640, 640, True),
    (128, 3, 6, 6, 300, 400, True),    # one query head per K/V head: tiles heaviest first across batch and heads
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d%d_B%d_H%d-%d_Nq%d_Nk%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_bwd_parity(orc, case):
    d, B, Hq, Hkv, Nq, Nk, causal = case
    say("[bwd] %s" % (case,))
    q, k, v, do = I.bwd_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=31 + Nq + Nk + Hq)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, causal)
    rq, rk, rv = orc.attn_bwd(I.to_f64(q), I.to_f64(k), I.to_f64(v), I.to_f64(do), scale, causal)
    fl = grad_floors(orc, q, k, v, do, scale, causal)
    check_grad("dq", dq, rq, fl["dq"])
    check_grad("dk", dk, rk, fl["dk"])
    check_grad("dv", dv, rv, fl["dv"])


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.5])
def test_bwd_scales(orc, scale):
    """scale 0 (uniform weights: dq = dk = 0), a negative scale and a large one."""
    d, B, Hq, Hkv, Nq, Nk = 64, 1, 4, 2, 150, 150
    q, k, v, do = I.bwd_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=77)
    for causal in (False, True):
        say("[bwd] scale=%g causal=%s" % (scale, causal))
        dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, causal)
        rq, rk, rv = orc.attn_bwd(I.to_f64(q), I.to_f64(k), I.to_f64(v), I.to_f64(do), scale, causal)
        if scale == 0.0:
            assert np.all(dq == 0) and np.all(dk == 0), "scale 0: dq and dk must vanish"
        else:
            fl = grad_floors(orc, q, k, v, do, scale, causal)
            check_grad("dq", dq, rq, fl["dq"])
            check_grad("dk", dk, rk, fl["dk"])
        check_grad("dv", dv, rv)


def test_bwd_empty_sides_rejected():
    """Nq = 0 or Nk = 0 is an invalid size: refused before any launch."""
    for Nq, Nk in ((0, 70), (40, 0)):
        q, k, v, do = I.bwd_inputs(1, 2, 1, Nq, Nk, 128, "bf16", seed=5)
        say("[bwd] Nq = %d, Nk = %d" % (Nq, Nk))
        qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
        lse = torch.zeros(1, 2, Nq, dtype=torch.float32, device="cuda")
        with pytest.raises(E.AttnError) as ei:
            E.attn_bwd(qd, kd, vd, torch.zeros_like(qd), dod, lse)
        assert ei.value.status == E.ATTN_ERR_INVALID_ARG


def test_bwd_deterministic():
    """No atomics: two calls give identical bits."""
    q, k, v, do = I.bwd_inputs(1, 8, 2, 333, 333, 128, "bf16", seed=8)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = E.attn_fwd(qd, kd, vd, causal=True)
    a = E.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    b = E.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _sample_keys(B, Hkv, Nk, groups, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for (b, hk) in groups:
        for j in (0, 1, 31, 32, 63, 64, 127, 128, Nk // 2, Nk - 2, Nk - 1):
            if 0 <= j < Nk:
                rows.add((b, hk, j))
        for _ in range(n_random):
            rows.add((b, hk, int(rng.integers(Nk))))
    return np.array(sorted(rows), dtype=np.int32)


@pytest.mark.parametrize("name", ["C4", "X1", "C3b"])
def test_bwd_workload_sampled(orc, name):
    """Full-size workloads: dq on sampled query rows of every head, dk / dv on
    sampled key rows of one K/V head group (the oracle needs every row of a
    group's heads for a key row)."""
    w = I.WORKLOADS[name]
    q, k, v, do = I.bwd_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, w.dtype, seed=w.seed + 500)
    say("[bwd] %s full size q%s k%s" % (name, tuple(q.shape), tuple(k.shape)))
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, w.scale, w.causal)
    rng = np.random.default_rng(w.seed)
    qrows = np.array(sorted({(0, int(h), int(i)) for h, i in zip(rng.integers(w.Hq, size=96),
                                                                  rng.integers(w.Nq, size=96))}
                            | {(0, h, 0) for h in range(0, w.Hq, 7)} | {(0, h, w.Nq - 1) for h in range(0, w.Hq, 5)}),
                     dtype=np.int32)
    hk = w.Hkv // 2
    krows = _sample_keys(w.B, w.Hkv, w.Nkv, [(0, hk)], 24, w.seed + 1)
    rq, rk, rv = orc.attn_bwd_rows(I.to_f64(q), I.to_f64(k), I.to_f64(v), I.to_f64(do), w.scale, w.causal,
                                   qrows, krows)
    check_grad("%s dq (%d rows)" % (name, len(qrows)), dq[qrows[:, 0], qrows[:, 1], qrows[:, 2]], rq)
    check_grad("%s dk (%d rows)" % (name, len(krows)), dk[krows[:, 0], krows[:, 1], krows[:, 2]], rk)
    check_grad("%s dv (%d rows)" % (name, len(krows)), dv[krows[:, 0], krows[:, 1], krows[:, 2]], rv)


@pytest.mark.parametrize("Nq,Nk,Hq,Hkv", [(583, 601, 128, 16), (600, 650, 128, 32), (583, 601, 128, 8),
                                         (600, 650, 192, 16)])
def test_dq_workgroup_forms_agree(Nq, Nk, Hq, Hkv):
    """On causal layers with many query heads the dq kernel runs 8-wave
    workgroups over the same query positions of 8 heads (group of 8) or 4
    heads (group of 4) that share a K/V head; one head alone is too small a
    grid for that and runs 4-wave workgroups of 128 rows; groups of 16 and 12
    take two and three blocks of heads.  Each row's arithmetic is the same in
    both forms, so dq must agree bit for bit.  The single head is repeated as
    separate heads so that its forward (whose O and LSE the backward reads)
    also runs a form that shares the row arithmetic, not the key-split form
    of very small grids."""
    B, d = 2, 128
    q, k, v, do = I.bwd_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=91 + Nq)
    dq_all = gpu_fwd_bwd(q, k, v, do, 0.09, True)[0]
    G = Hq // Hkv
    R = narrow_form_copies(Nq)
    for b, h in [(0, 0), (1, 37), (1, Hq - 1)]:
        hk = h // G
        say("[bwd forms] b=%d h=%d" % (b, h))
        dq1 = gpu_fwd_bwd(one_head(q, b, h, R), one_head(k, b, hk, R), one_head(v, b, hk, R), one_head(do, b, h, R),
                          0.09, True)[0]
        assert np.array_equal(dq1[0, 0], dq_all[b, h]), (b, h)
