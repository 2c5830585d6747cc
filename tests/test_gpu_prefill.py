"""Parity of attn_fwd (the HIP prefill kernels) with the fp64 oracle."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, dev, gpu_fwd, max_err, narrow_form_copies, one_head, say

pytestmark = pytest.mark.gpu


def _full_parity(orc, q, k, v, scale, causal, dtype, label):
    say("[prefill] %s q%s k%s %s causal=%s" % (label, tuple(q.shape), tuple(k.shape), dtype, causal))
    o, lse = gpu_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), scale, causal)
    assert_close(label + " O", o, o_ref, TOL_O[dtype])
    assert_close(label + " LSE", lse, lse_ref, TOL_LSE)


@pytest.mark.parametrize("name,causal", [
    ("C1", False), ("C1", True), ("C2a", False), ("C2b", True), ("C3a", True),
])
def test_workload_full_parity(orc, name, causal):
    w = I.WORKLOADS[name]
    q, k, v = I.workload_inputs(name)
    _full_parity(orc, q, k, v, w.scale, causal, w.dtype, name)


@pytest.mark.parametrize("name", ["C3a'", "C3b", "C4", "X1", "X2"])
def test_workload_full_size_parity(orc, name):
    """Full-size workloads in the launch configuration the benchmark times,
    compared with the oracle on every output element (the oracle runs the
    definition over the whole tensor: about 10 s for the GQA layer on 16 host
    cores)."""
    w = I.WORKLOADS[name]
    q, k, v = I.workload_inputs(name)
    say("[prefill] %s full size q%s k%s causal=%s" % (name, tuple(q.shape), tuple(k.shape), w.causal))
    o, lse = gpu_fwd(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), w.scale, w.causal)
    assert_close(name + " O (all %d rows)" % (w.B * w.Hq * w.Nq), o, o_ref, TOL_O[w.dtype])
    assert_close(name + " LSE", lse, lse_ref, TOL_LSE)


RAGGED = [
    # dtype, d, B, Hq, Hkv, Nq, Nk, causal
    ("bf16", 128, 2, 4, 2, 200, 200, True),
    ("bf16", 128, 2, 4, 2, 200, 200, False),
    ("bf16", 64, 1, 3, 1, 77, 300, False),     # cross-attention, rectangular
    ("bf16", 128, 1, 2, 2, 100, 333, True),    # chunked prefill (bottom-right)
    ("bf16", 64, 3, 2, 2, 1, 1, True),
    ("bf16", 128, 1, 8, 1, 65, 129, True),     # MQA
    ("bf16", 64, 1, 16, 2, 129, 63, False),    # Nk < one tile
    ("bf16", 128, 1, 1, 1, 1000, 1000, True),
    # key-split form: fewer key tiles than key groups, odd tile counts
    ("bf16", 64, 1, 2, 1, 130, 130, True),
    ("bf16", 128, 1, 3, 3, 90, 200, True),
    ("bf16", 64, 2, 3, 1, 50, 700, True),      # chunked prefill
    ("bf16", 128, 1, 2, 1, 1, 500, True),      # one query row over 8 key tiles, both groups busy
    ("bf16", 64, 1, 2, 1, 40, 300, True),      # 5 key tiles over 4 groups: runs of 1, 1, 1, 2
    # causal, one query head per K/V head: tiles dispatched heaviest first across batch and heads
    ("bf16", 128, 3, 5, 5, 300, 300, True),    # key-split form
    ("bf16", 64, 2, 40, 40, 400, 400, True),   # 4-wave form
    # more work groups than the chip holds at once, ragged tails
    ("bf16", 128, 2, 64, 16, 1000, 1000, True),
    ("bf16", 64, 2, 128, 8, 700, 1100, True),    # chunked prefill
    ("bf16", 128, 1, 256, 32, 520, 300, False),  # cross-attention
    # causal chunks with enough 256-row work items: the 8-wave kernel
    ("bf16", 64, 2, 128, 16, 300, 1000, True),
    ("bf16", 128, 2, 128, 16, 300, 700, True),
    ("bf16", 64, 2, 128, 8, 300, 260, False),   # non-causal, Nk < Nq, 8 waves
    ("f32", 64, 2, 2, 1, 100, 100, True),
    ("f32", 128, 1, 4, 2, 70, 130, True),
    ("f32", 128, 1, 2, 1, 33, 17, False),
    # grids of at least 256 row tiles of 16: the four-rows-per-wave fp32 form
    ("f32", 64, 2, 8, 4, 250, 250, True),
    ("f32", 128, 1, 16, 2, 260, 300, True),    # chunked prefill
    ("f32", 128, 1, 16, 16, 256, 100, False),  # Nk < Nq, one partial key tile
    ("f32", 64, 1, 16, 4, 300, 200, False),    # Nq > Nk, ragged row and key tails
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "%s_d%d_B%d_H%d-%d_Nq%d_Nk%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "causal" if c[7] else "full"))
def test_ragged_parity(orc, case):
    dtype, d, B, Hq, Hkv, Nq, Nk, causal = case
    q, k, v = I.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed=7 + Nq + Nk)
    _full_parity(orc, q, k, v, 1.0 / np.sqrt(d), causal, dtype, "ragged")


def test_large_scores(orc):
    """scale = 1 makes scores of size ~10 (d = 128): the online rescaling is
    exercised and each row is dominated by a few keys, so |O| reaches the
    magnitude of single value entries (up to ~5).  A bf16 output near 4..8 has
    a half-ulp of 1.6e-2 by itself, so this stress test bounds the bf16 error
    element-wise by 1e-2 + 2^-8 |O_ref| (the output rounding plus the
    probability rounding) instead of a flat 1.5e-2."""
    q, k, v = I.prefill_inputs(1, 2, 1, 300, 300, 128, "bf16", seed=11)
    o, lse = gpu_fwd(q, k, v, 1.0, True)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), 1.0, True)
    bound = 1e-2 + 2.0 ** -8 * np.abs(o_ref)
    excess = float((np.abs(o - o_ref) - bound).max())
    say("  scale=1 bf16: max |err| - bound = %.3e, max |O_ref| = %.2f" % (excess, np.abs(o_ref).max()))
    assert excess <= 0
    assert_close("scale=1 bf16 LSE", lse, lse_ref, TOL_LSE)
    # fp32: the scores' own fp32 rounding (about 1e-7 relative on scores of
    # size ~25) is 8x larger than at scale 1/sqrt(64), so the bound is 8x the
    # 1e-5 of the fp32 workload.
    q, k, v = I.prefill_inputs(1, 2, 1, 100, 100, 64, "f32", seed=12)
    o, lse = gpu_fwd(q, k, v, 1.0, False)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), 1.0, False)
    assert_close("scale=1 fp32 O", o, o_ref, 8e-5)
    assert_close("scale=1 fp32 LSE", lse, lse_ref, TOL_LSE)


def test_empty_sizes_rejected():
    """Nk = 0, Nq = 0 and B = 0 are invalid sizes: refused before any launch,
    o left untouched."""
    q = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 1, 0, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 3.0)
    for args in ((q, k, k.clone()), (q[:, :, :0], k, k.clone()), (q[:0], k[:0], k[:0])):
        with pytest.raises(E.AttnError) as ei:
            E.attn_fwd(*args, causal=False, o=o if args[0] is q else None)
        assert ei.value.status == E.ATTN_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (o == 3.0).all().item()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_probes_through_kernel(orc, dtype):
    """The invariant probes, through the kernel: V = ones, identical keys,
    causal row 0, shift invariance."""
    B, H, N, d = 1, 2, 150, 64
    tol = TOL_O[dtype]
    q, k, v = I.prefill_inputs(B, H, H, N, N, d, dtype, seed=21)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        ones = torch.ones_like(v)
        o, _ = gpu_fwd(q, k, ones, scale, causal)
        assert_close("V=ones causal=%s" % causal, o, np.ones_like(o), 1e-6 if dtype == "f32" else 2 ** -8)
        kk = k[:, :, :1].expand(B, H, N, d).contiguous()
        o, lse = gpu_fwd(q, kk, v, scale, causal)
        o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(kk), I.to_f64(v), scale, causal)
        assert_close("identical keys causal=%s" % causal, o, o_ref, tol)
        assert_close("identical keys lse", lse, lse_ref, TOL_LSE)
    o, lse = gpu_fwd(q, k, v, scale, True)
    assert np.array_equal(o[:, :, 0], I.to_f64(v)[:, :, 0]), "causal row 0 must return v_0"
    s00 = scale * np.einsum("bhc,bhc->bh", I.to_f64(q)[:, :, 0], I.to_f64(k)[:, :, 0])
    assert_close("causal row 0 lse", lse[:, :, 0], s00, 1e-5)
    if dtype == "f32":
        # K' = K + 1 w^T shifts row i by scale * q_i . w
        w = torch.randn(d, generator=torch.Generator().manual_seed(5)) * 0.5
        o1, l1 = gpu_fwd(q, k, v, scale, False)
        o2, l2 = gpu_fwd(q, k + w, v, scale, False)
        assert_close("shift invariance O", o2, o1, 1e-5)
        shift = scale * (I.to_f64(q) @ I.to_f64(w))
        assert_close("shift invariance LSE", l2, l1 + shift, 1e-4)


@pytest.mark.parametrize("G", [2, 8])
def test_gqa_equals_repeated_mha(G):
    q, k, v = I.prefill_inputs(1, 2 * G, 2, 257, 257, 128, "bf16", seed=31)
    o1, l1 = gpu_fwd(q, k, v, 0.1, True)
    o2, l2 = gpu_fwd(q, k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1), 0.1, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal,Nq,Nk,Hq,Hkv", [(False, 300, 520, 128, 16), (True, 300, 700, 128, 16),
                                                (True, 583, 601, 128, 16), (True, 600, 650, 128, 32),
                                                (True, 583, 601, 128, 8), (True, 600, 650, 192, 16)])
def test_wide_and_narrow_workgroups_agree(causal, Nq, Nk, Hq, Hkv):
    """With many query heads the launch uses 8-wave workgroups: 256 rows of
    one head for non-causal and chunked-causal layers, and for causal layers
    with rows at very different depths the same 32 query positions of the 8
    heads that share a K/V head (group of 8), or 64 positions of 4 heads
    (group of 4); groups of 16 and 12 take two and three such blocks of
    heads.  Copies of one head as separate heads (MHA) are too few rows for
    any of them and use 128-row workgroups of 4 waves.  Each row's arithmetic
    is the same in every form, so the outputs must agree bit for bit."""
    B, d = 2, 128
    q, k, v = I.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=61 + Nq)
    o_all, l_all = gpu_fwd(q, k, v, 0.09, causal)
    G = Hq // Hkv
    R = narrow_form_copies(Nq)
    for b, h in [(0, 0), (1, 37), (1, Hq - 1)]:
        hk = h // G
        o1, l1 = gpu_fwd(one_head(q, b, h, R), one_head(k, b, hk, R), one_head(v, b, hk, R), 0.09, causal)
        assert np.array_equal(o1[0, 0], o_all[b, h]) and np.array_equal(l1[0, 0], l_all[b, h]), (b, h)
        assert np.array_equal(o1[0, R - 1], o1[0, 0]), (b, h)


@pytest.mark.parametrize("d,Nq,Nk,causal", [(64, 1000, 1000, True), (128, 1000, 1000, True),
                                            (64, 300, 900, True), (128, 257, 300, True)])
def test_key_split_form_close_to_4wave_form(orc, d, Nq, Nk, causal):
    """One causal head is a grid of fewer 128-row workgroups than CUs: its
    key range is split over the key groups of one workgroup and the partial
    states merged.  That changes only the order of the sums (and the points
    where the reference of each part is raised), so the result stays within
    the parity bound of the oracle and within a few bf16 units of the 4-wave
    form of the same rows."""
    q, k, v = I.prefill_inputs(1, 1, 1, Nq, Nk, d, "bf16", seed=71 + Nq + d)
    scale = 1.0 / np.sqrt(d)
    o1, l1 = gpu_fwd(q, k, v, scale, causal)
    R = narrow_form_copies(Nq)
    o4, l4 = gpu_fwd(one_head(q, 0, 0, R), one_head(k, 0, 0, R), one_head(v, 0, 0, R), scale, causal)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), scale, causal)
    assert_close("key-split O", o1, o_ref, TOL_O["bf16"])
    assert_close("key-split LSE", l1, lse_ref, TOL_LSE)
    # two bf16 units of the output's magnitude, plus the rounding of P
    excess = float((np.abs(o1[0, 0] - o4[0, 0]) - (2.0 ** -8 + 2.0 ** -6 * np.abs(o4[0, 0]))).max())
    say("  key-split vs 4-wave: max |diff| - bound = %.3e" % excess)
    assert excess <= 0
    assert_close("key-split vs 4-wave LSE", l1[0, 0], l4[0, 0], 1e-4)


def test_run_twice_bitwise():
    q, k, v = I.prefill_inputs(2, 8, 2, 513, 513, 128, "bf16", seed=41)
    a = gpu_fwd(q, k, v, 0.088, True)
    b = gpu_fwd(q, k, v, 0.088, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_lse_optional(orc):
    q, k, v = I.prefill_inputs(1, 2, 2, 64, 64, 64, "bf16", seed=51)
    o = E.attn_fwd(dev(q), dev(k), dev(v), causal=True, return_lse=False)
    torch.cuda.synchronize()
    o_ref, _ = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), 1 / 8.0, True)
    assert max_err(I.to_f64(o), o_ref) <= TOL_O["bf16"]
