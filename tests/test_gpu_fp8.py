"""Parity of attn_fwd_fp8 (fp8 e4m3 q, k, v; bf16 output) with the fp64 oracle.

The inputs are iid N(0, 1) rounded to e4m3; the oracle receives the same
stored values widened to fp64.  The kernel's weights are rounded to bf16, as
in the bf16 kernel, so the bf16 tolerances apply (O max-abs 1.5e-2, times
v_scale; LSE 1e-3).  Its scores come from the fp8 matrix instruction, whose
internal sums keep about 16 significant bits: an absolute score error of up
to ~2^-16 * sum_c |q_c k_c| before scaling (measured on gfx950), which stays
far below those tolerances for the scales tested here (|scale| <= 0.6)."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, dev, say

pytestmark = pytest.mark.gpu


def fp8_fwd(q, k, v, scale, causal, v_scale=1.0):
    o, lse = E.attn_fwd_fp8(dev(q), dev(k), dev(v), scale=scale, v_scale=v_scale, causal=causal)
    torch.cuda.synchronize()
    return I.to_f64(o), I.to_f64(lse)


CASES = [
    # d, B, Hq, Hkv, Nq, Nk, causal
    (128, 2, 4, 2, 200, 200, True),
    (128, 2, 4, 2, 200, 200, False),
    (64, 1, 3, 1, 77, 300, False),     # cross-attention
    (128, 1, 2, 2, 100, 333, True),    # chunked prefill (bottom-right)
    (64, 3, 2, 2, 1, 1, True),
    (128, 1, 8, 1, 65, 129, True),     # MQA
    (64, 1, 16, 2, 129, 63, False),    # Nk below one tile
    (128, 1, 1, 1, 1000, 1000, True),
    (128, 2, 64, 16, 1000, 1000, True),
    (64, 2, 128, 8, 700, 1100, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d%d_B%d_H%d-%d_Nq%d_Nk%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_fp8_parity(orc, case):
    d, B, Hq, Hkv, Nq, Nk, causal = case
    q, k, v = I.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "fp8", seed=41 + Nq + Nk)
    scale = 1.0 / np.sqrt(d)
    say("[fp8] %s" % (case,))
    o, lse = fp8_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), scale, causal)
    assert_close("fp8 O", o, o_ref, TOL_O["bf16"])
    assert_close("fp8 LSE", lse, lse_ref, TOL_LSE)


@pytest.mark.parametrize("scale,v_scale", [(-0.2, 1.0), (0.0, 1.0), (0.6, 1.0), (0.09, 0.37), (0.09, 3.0)])
def test_fp8_scales(orc, scale, v_scale):
    """Negative, zero and large score scales (dequantisation factors folded
    in), and the output factor v_scale."""
    q, k, v = I.prefill_inputs(1, 4, 2, 150, 150, 128, "fp8", seed=9)
    for causal in (False, True):
        say("[fp8] scale=%g v_scale=%g causal=%s" % (scale, v_scale, causal))
        o, lse = fp8_fwd(q, k, v, scale, causal, v_scale)
        o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), scale, causal)
        # a large scale makes rows peaky, so |O| reaches single value entries:
        # bound the bf16 output rounding relative to |O| as the bf16 stress test does
        bound = v_scale * (1e-2 + 2.0 ** -8 * np.abs(o_ref))
        excess = float((np.abs(o - v_scale * o_ref) - bound).max())
        say("  max |err| - bound = %.3e" % excess)
        assert excess <= 0
        assert_close("fp8 LSE", lse, lse_ref, TOL_LSE)


def test_fp8_matches_bf16_path():
    """Every e4m3 value is a bf16 value, so on the same values the two kernels
    differ only in how the score sums are rounded: fp32 in the bf16 kernel,
    about 16 bits inside the fp8 instruction.  With sum_c |q_c k_c| <= ~150
    here, the scaled scores differ by at most scale * 2^-16 * 150 = 2e-4,
    which bounds the LSE difference; O differs by at most two bf16 ulps of
    values below 2 (one rounding flip on either side), 1.6e-2."""
    q, k, v = I.prefill_inputs(1, 8, 2, 333, 333, 128, "fp8", seed=10)
    o8, l8 = E.attn_fwd_fp8(dev(q), dev(k), dev(v), causal=True)
    o16, l16 = E.attn_fwd(dev(q.to(torch.bfloat16)), dev(k.to(torch.bfloat16)), dev(v.to(torch.bfloat16)),
                          causal=True)
    torch.cuda.synchronize()
    d_o = float((o8.float() - o16.float()).abs().max())
    d_l = float((l8 - l16).abs().max())
    say("  fp8 vs bf16 kernel: max |dO| %.3e max |dLSE| %.3e" % (d_o, d_l))
    assert d_o <= 1.6e-2 and d_l <= 2e-4


def test_fp8_workload_full_size(orc):
    """The GQA prefill workload in fp8 at full size, every output element
    against the oracle on the same e4m3 values."""
    w = I.WORKLOADS["C4"]
    q, k, v = I.prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, "fp8", w.seed)
    say("[fp8] C4 full size")
    o, lse = E.attn_fwd_fp8(dev(q), dev(k), dev(v), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), w.scale, w.causal)
    assert_close("C4 fp8 O (all rows)", I.to_f64(o), o_ref, TOL_O["bf16"])
    assert_close("C4 fp8 LSE", I.to_f64(lse), lse_ref, TOL_LSE)


def test_fp8_empty_keys_rejected():
    q = torch.randn(1, 2, 5, 64).to(torch.float8_e4m3fn).cuda()
    k = torch.empty(1, 1, 0, 64, dtype=torch.float8_e4m3fn, device="cuda")
    with pytest.raises(E.AttnError) as ei:
        E.attn_fwd_fp8(q, k, k.clone(), causal=False)
    assert ei.value.status == E.ATTN_ERR_INVALID_ARG
