"""Parity on seeded random shapes: every entry point against the fp64 oracle
on shapes drawn from fixed seeds (batch, query heads and group size, lengths
on both sides of tile boundaries, head dim, causality, scale), to reach
combinations of sizes that the hand-picked cases in the other files do not.
Tolerances are those of the other parity tests."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, dev, gpu_decode, gpu_fwd, grad_floors, say

pytestmark = pytest.mark.gpu

# lengths around the 32-, 64- and 128-row tiles
LENGTHS = [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 191, 200, 257, 383, 511]


def _prefill_shapes(n, seed, max_len=511):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.integers(1, 4))
        Nk = int(rng.choice([x for x in LENGTHS if x <= max_len]))
        causal = bool(rng.integers(0, 2))
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.choice([x for x in LENGTHS if x <= max_len]))
        scale = float(rng.choice([1.0 / np.sqrt(d), 0.05, -0.08]))
        out.append((d, B, Hkv * G, Hkv, Nq, Nk, causal, round(scale, 6)))
    return out


def _ids(c):
    return "d%d_B%d_H%d-%d_Nq%d_Nk%d_%s_s%g" % (c[0], c[1], c[2], c[3], c[4], c[5], "c" if c[6] else "f", c[7])


@pytest.mark.parametrize("case", _prefill_shapes(20, 2024), ids=_ids)
def test_random_fwd_bf16(orc, case):
    d, B, Hq, Hkv, Nq, Nk, causal, scale = case
    say("[random fwd] %s" % (case,))
    q, k, v = I.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=5000 + Nq * 7 + Nk + Hq)
    o, lse = gpu_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), scale, causal)
    assert_close("O", o, o_ref, TOL_O["bf16"])
    assert_close("LSE", lse, lse_ref, TOL_LSE)


@pytest.mark.parametrize("case", _prefill_shapes(6, 2025, max_len=200), ids=_ids)
def test_random_fwd_f32(orc, case):
    d, B, Hq, Hkv, Nq, Nk, causal, scale = case
    say("[random fwd f32] %s" % (case,))
    q, k, v = I.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "f32", seed=5100 + Nq * 7 + Nk + Hq)
    o, lse = gpu_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), scale, causal)
    assert_close("O", o, o_ref, TOL_O["f32"])
    assert_close("LSE", lse, lse_ref, TOL_LSE)


@pytest.mark.parametrize("case", _prefill_shapes(10, 2026), ids=_ids)
def test_random_fwd_fp8(orc, case):
    d, B, Hq, Hkv, Nq, Nk, causal, scale = case
    say("[random fwd fp8] %s" % (case,))
    q, k, v = I.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "fp8", seed=5200 + Nq * 7 + Nk + Hq)
    o, lse = E.attn_fwd_fp8(dev(q), dev(k), dev(v), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), scale, causal)
    assert_close("O", I.to_f64(o), o_ref, TOL_O["bf16"])
    assert_close("LSE", I.to_f64(lse), lse_ref, TOL_LSE)


def _decode_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 4, 5, 8, 16, 20]))
        B = int(rng.integers(1, 20))
        Lmax = int(rng.choice([1, 64, 100, 640, 1500]))
        kps = int(rng.choice([0, 0, 1, 37, 256]))
        out.append((d, B, Hkv * G, Hkv, Lmax, kps))
    return out


@pytest.mark.parametrize("case", _decode_shapes(14, 2027),
                         ids=lambda c: "d%d_B%d_H%d-%d_L%d_kps%d" % c)
def test_random_decode(orc, case):
    d, B, Hq, Hkv, Lmax, kps = case
    say("[random decode] %s" % (case,))
    sl, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "bf16", seed=5300 + B * 13 + Lmax + Hq, lo=0, hi=Lmax)
    o, lse = gpu_decode(sl, q, kc, vc, 1.0 / np.sqrt(d), kps)
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), 1.0 / np.sqrt(d))
    assert_close("O", o, o_ref, TOL_O["bf16"])
    assert_close("LSE", lse, lse_ref, TOL_LSE)


@pytest.mark.parametrize("case", _decode_shapes(8, 2028),
                         ids=lambda c: "d%d_B%d_H%d-%d_L%d_kps%d" % c)
def test_random_decode_paged(orc, case):
    d, B, Hq, Hkv, Lmax, kps = case
    bs = int(np.random.default_rng(Lmax + B).choice([1, 8, 16, 32, 64, 100]))
    say("[random paged] %s bs=%d" % (case, bs))
    sl, q, kp, vp, bt = I.paged_decode_inputs(B, Hq, Hkv, d, bs, -(-Lmax // bs), "bf16", seed=5400 + B + Lmax,
                                              lo=0, hi=Lmax, spare_blocks=1)
    o, lse = E.attn_decode_paged(dev(q), dev(kp), dev(vp), dev(bt), dev(sl), scale=1.0 / np.sqrt(d),
                                 keys_per_split=kps)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(),
                                      1.0 / np.sqrt(d))
    assert_close("O", I.to_f64(o), o_ref, TOL_O["bf16"])
    assert_close("LSE", I.to_f64(lse), lse_ref, TOL_LSE)


@pytest.mark.parametrize("case", _decode_shapes(6, 2031), ids=lambda c: "d%d_B%d_H%d-%d_L%d_kps%d" % c)
def test_random_decode_f32(orc, case):
    d, B, Hq, Hkv, Lmax, kps = case
    say("[random decode f32] %s" % (case,))
    sl, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "f32", seed=5600 + B * 13 + Lmax + Hq, lo=0, hi=Lmax)
    o, lse = gpu_decode(sl, q, kc, vc, 1.0 / np.sqrt(d), kps)
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), 1.0 / np.sqrt(d))
    assert_close("O", o, o_ref, TOL_O["f32"])
    assert_close("LSE", lse, lse_ref, TOL_LSE)


@pytest.mark.parametrize("case", _decode_shapes(4, 2032), ids=lambda c: "d%d_B%d_H%d-%d_L%d_kps%d" % c)
def test_random_decode_paged_f32(orc, case):
    d, B, Hq, Hkv, Lmax, kps = case
    bs = int(np.random.default_rng(Lmax + B + 1).choice([1, 8, 16, 32, 64, 100]))
    say("[random paged f32] %s bs=%d" % (case, bs))
    sl, q, kp, vp, bt = I.paged_decode_inputs(B, Hq, Hkv, d, bs, -(-Lmax // bs), "f32", seed=5700 + B + Lmax,
                                              lo=0, hi=Lmax, spare_blocks=1)
    o, lse = E.attn_decode_paged(dev(q), dev(kp), dev(vp), dev(bt), dev(sl), scale=1.0 / np.sqrt(d),
                                 keys_per_split=kps)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(),
                                      1.0 / np.sqrt(d))
    assert_close("O", I.to_f64(o), o_ref, TOL_O["f32"])
    assert_close("LSE", I.to_f64(lse), lse_ref, TOL_LSE)


@pytest.mark.parametrize("case", _prefill_shapes(10, 2029, max_len=383), ids=_ids)
def test_random_bwd(orc, case):
    """Gradients against the oracle's, relative to each tensor's largest
    magnitude (the backward test's bound: 2e-2 of max|ref|, 6e-3 of RMS, plus
    the rounding floor of dq and dk where the reference is exactly zero)."""
    d, B, Hq, Hkv, Nq, Nk, causal, scale = case
    say("[random bwd] %s" % (case,))
    q, k, v, do = I.bwd_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=5500 + Nq * 7 + Nk + Hq)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = E.attn_fwd(qd, kd, vd, scale=scale, causal=causal)
    grads = E.attn_bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    refs = orc.attn_bwd(I.to_f64(q), I.to_f64(k), I.to_f64(v), I.to_f64(do), scale, causal)
    floors = grad_floors(orc, q, k, v, do, scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        floor = floors[name]
        g = I.to_f64(g)
        assert np.isfinite(g).all(), name
        top = float(np.abs(r).max())
        rms = float(np.sqrt(np.mean(r ** 2)))
        e_max = float(np.abs(g - r).max())
        e_rms = float(np.sqrt(np.mean((g - r) ** 2)))
        say("  %s max err %.2e of max|ref|, rms err %.2e of rms" % (name, e_max / max(top, 1e-300),
                                                                   e_rms / max(rms, 1e-300)))
        assert e_max <= 2e-2 * top + floor and e_rms <= 6e-3 * rms + floor, name


@pytest.mark.parametrize("case", _prefill_shapes(6, 2039, max_len=200), ids=_ids)
def test_random_bwd_f32(orc, case):
    """fp32 gradients against the oracle's, at the fp32 backward test's
    bound: max |g - ref| <= 3e-5 * max|ref| + 2e-6 per tensor."""
    d, B, Hq, Hkv, Nq, Nk, causal, scale = case
    say("[random bwd f32] %s" % (case,))
    q, k, v, do = I.bwd_inputs(B, Hq, Hkv, Nq, Nk, d, "f32", seed=5600 + Nq * 7 + Nk + Hq)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = E.attn_fwd(qd, kd, vd, scale=scale, causal=causal)
    grads = E.attn_bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    refs = orc.attn_bwd(I.to_f64(q), I.to_f64(k), I.to_f64(v), I.to_f64(do), scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        assert g.dtype == torch.float32, name
        g = I.to_f64(g)
        assert np.isfinite(g).all(), name
        top = float(np.abs(r).max())
        e_max = float(np.abs(g - r).max())
        say("  %s max err %.2e (max|ref| %.2e)" % (name, e_max, top))
        assert e_max <= 3e-5 * top + 2e-6, name
