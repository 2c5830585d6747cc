"""Parity of attn_decode / attn_decode_paged on fp32 caches with the fp64
oracle, at the fp32 tolerance (max-abs O <= 1e-5, LSE <= 1e-3).

The fp32 path shares the bf16 path's range walk, LDS ring and merge, with
fp32 products throughout (v_mfma_f32_16x16x4_f32, P kept in fp32).  The
cases mirror the bf16 ones: the decode workload's shape, every split from one
key per range to one range per segment, group sizes 1-32 at d = 64 and 128,
empty and clamped sequences, many short sequences, paged pools with odd
block sizes and NaN-poisoned unused blocks, negative and zero scales, and
the equivalence with the last row of a causal fp32 prefill."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, dev, gpu_decode, gpu_fwd, say

pytestmark = pytest.mark.gpu

TOL = TOL_O["f32"]


def _parity(orc, sl, q, kc, vc, scale, label, kps=0):
    say("[decode f32] %s q%s cache%s kps=%d L=%s" % (label, tuple(q.shape), tuple(kc.shape), kps, sl.tolist()[:8]))
    assert q.dtype == torch.float32
    o, lse = gpu_decode(sl, q, kc, vc, scale, kps)
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), scale)
    assert_close(label + " O", o, o_ref, TOL)
    assert_close(label + " LSE", lse, lse_ref, TOL_LSE)
    return o, lse


def _paged(sl, q, kp, vp, bt, scale, kps=0):
    o, lse = E.attn_decode_paged(dev(q), dev(kp), dev(vp), dev(bt), dev(sl.to(torch.int32)), scale=scale,
                                 keys_per_split=kps)
    torch.cuda.synchronize()
    return I.to_f64(o), I.to_f64(lse)


def _paged_parity(orc, sl, q, kp, vp, bt, scale, label, kps=0):
    say("[paged f32] %s q%s pool%s table%s kps=%d" % (label, tuple(q.shape), tuple(kp.shape), tuple(bt.shape), kps))
    o, lse = _paged(sl, q, kp, vp, bt, scale, kps)
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(), scale)
    assert_close(label + " O", o, o_ref, TOL)
    assert_close(label + " LSE", lse, lse_ref, TOL_LSE)
    return o, lse


def test_decode_workload_shape_f32(orc):
    """16 sequences, 32 query heads over 8 K/V heads, d = 128, lengths
    uniform in [512, 4096], in fp32 (default split)."""
    sl, q, kc, vc = I.decode_inputs(16, 32, 8, 4096, 128, "f32", seed=2101)
    _parity(orc, sl, q, kc, vc, 1 / np.sqrt(128), "16 x 32/8 heads, d=128")


@pytest.mark.parametrize("kps", [1, 33, 100, 1 << 20])
def test_split_count_invariance_f32(orc, kps):
    sl, q, kc, vc = I.decode_inputs(4, 32, 8, 2048, 128, "f32", seed=2102, lo=1, hi=2048)
    o_ref, l_ref = gpu_decode(sl, q, kc, vc, 0.088, 0)
    o, l = _parity(orc, sl, q, kc, vc, 0.088, "split", kps)
    assert_close("kps=%d vs default (O)" % kps, o, o_ref, TOL)
    assert_close("kps=%d vs default (LSE)" % kps, l, l_ref, 1e-5)


@pytest.mark.parametrize("G,d", [(1, 128), (3, 64), (4, 128), (4, 64), (8, 64), (16, 128), (24, 128), (32, 64)])
def test_group_sizes_f32(orc, G, d):
    Hkv = 2
    sl, q, kc, vc = I.decode_inputs(3, G * Hkv, Hkv, 700, d, "f32", seed=2110 + G, lo=1, hi=700)
    _parity(orc, sl, q, kc, vc, 1.0 / np.sqrt(d), "G=%d d=%d" % (G, d))


def test_edge_lengths_f32(orc):
    """seq_len 0 (O = 0, LSE = -inf), 1, a ragged tail, exactly one chunk
    boundary, and values beyond max_seq_len (clamped); default split and one
    key per range."""
    B, Hq, Hkv, Lmax, d = 6, 8, 2, 600, 64
    _, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "f32", seed=2120)
    sl = torch.tensor([0, 1, 257, 256, 600, 5000], dtype=torch.int32)
    for kps in (0, 1):
        o, lse = _parity(orc, sl, q, kc, vc, 0.125, "edge lengths", kps)
        assert (o[0] == 0).all() and np.isneginf(lse[0]).all()


def test_many_short_sequences_f32(orc):
    """150 sequences (three pages of 64) of 0..40 keys, some empty, in ranges
    of 7 keys: ranges cross many sequence boundaries."""
    B, Hq, Hkv, Lmax, d = 150, 8, 2, 48, 128
    _, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "f32", seed=2130)
    g = torch.Generator().manual_seed(2131)
    sl = torch.randint(0, 41, (B,), generator=g, dtype=torch.int32)
    sl[::7] = 0
    _parity(orc, sl, q, kc, vc, 0.088, "150 short sequences", 7)


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_negative_and_zero_scale_f32(orc, scale):
    """A negative scale flips every score (the kernel negates q exactly); a
    zero scale gives every visible key the same weight."""
    sl, q, kc, vc = I.decode_inputs(3, 8, 2, 300, 128, "f32", seed=2140, lo=1, hi=300)
    _parity(orc, sl, q, kc, vc, scale, "scale=%g" % scale)


def test_decode_matches_prefill_last_row_f32(orc):
    """attn_decode of a sequence equals the last row of causal fp32 attn_fwd
    over the same keys (bottom-right alignment)."""
    L, Hq, Hkv, d = 333, 8, 2, 64
    qp, k, v = I.prefill_inputs(1, Hq, Hkv, L, L, d, "f32", seed=2150)
    o_p, l_p = gpu_fwd(qp, k, v, 0.125, True)
    q = qp[:, :, L - 1, :].contiguous()
    sl = torch.tensor([L], dtype=torch.int32)
    o_d, l_d = gpu_decode(sl, q, k, v, 0.125)
    assert_close("decode vs prefill last row (O)", o_d, o_p[:, :, L - 1, :], 2 * TOL)
    assert_close("decode vs prefill last row (LSE)", l_d, l_p[:, :, L - 1], 1e-5)


@pytest.mark.parametrize("bs,G,d,kps", [(16, 4, 128, 0), (1, 8, 64, 0), (7, 4, 128, 100), (64, 16, 64, 1),
                                        (33, 24, 128, 0)])
def test_paged_f32(orc, bs, G, d, kps):
    Hkv = 2
    sl, q, kp, vp, bt = I.paged_decode_inputs(5, G * Hkv, Hkv, d, bs, -(-700 // bs), "f32", seed=2160 + bs + G,
                                              lo=0, hi=700, spare_blocks=2)
    _paged_parity(orc, sl, q, kp, vp, bt, 1 / np.sqrt(d), "bs=%d G=%d d=%d" % (bs, G, d), kps)


def test_paged_unused_blocks_never_read_f32(orc):
    """Every block that holds no valid row is poisoned with NaN: the results
    are bit-identical to the clean pool's."""
    sl, q, kp, vp, bt = I.paged_decode_inputs(6, 8, 2, 128, 32, 20, "f32", seed=2170, lo=100, hi=640, spare_blocks=5)
    o1, l1 = _paged_parity(orc, sl, q, kp, vp, bt, 0.088, "clean pool")
    used = set()
    for b in range(6):
        used.update(int(x) for x in bt[b, :(int(sl[b]) + 31) // 32].tolist())
    kpp, vpp = kp.clone(), vp.clone()
    for blk in range(kp.shape[0]):
        if blk not in used:
            kpp[blk] = float("nan")
            vpp[blk] = float("nan")
    o2, l2 = _paged(sl, q, kpp, vpp, bt, 0.088)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_noalloc_f32_matches_decode():
    """attn_decode_noalloc on fp32 caches reproduces attn_decode bit for bit."""
    sl, q, kc, vc = (dev(t) for t in I.decode_inputs(4, 32, 8, 1024, 128, "f32", seed=2180, lo=1, hi=1024))
    o_ref, l_ref = E.attn_decode(q, kc, vc, sl, scale=0.088)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((4, 32), float("nan"), dtype=torch.float32, device="cuda")
    E.attn_decode_noalloc(q, kc, vc, sl, o, lse, scale=0.088)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
