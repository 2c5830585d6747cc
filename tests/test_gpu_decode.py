"""Parity of attn_decode (the split-KV HIP kernels) with the fp64 oracle.

The split kernel cuts the keys of the whole batch (every sequence, K/V head
and block of 16 query heads laid end to end) into equal ranges, one per
workgroup; keys_per_split sets the range length (0: two ranges per compute
unit).  The cases below cover ranges shorter than a
chunk, ranges that span many short sequences, several pages of 64 sequences,
empty sequences and workgroups whose range is empty."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, dev, gpu_decode, gpu_fwd, say

pytestmark = pytest.mark.gpu


def _parity(orc, seq_lens, q, kc, vc, scale, label, kps=0):
    say("[decode] %s q%s cache%s kps=%d L=%s" % (label, tuple(q.shape), tuple(kc.shape), kps,
                                                 seq_lens.tolist()[:8]))
    o, lse = gpu_decode(seq_lens, q, kc, vc, scale, kps)
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), seq_lens.numpy(), scale)
    assert_close(label + " O", o, o_ref, TOL_O["bf16"])
    assert_close(label + " LSE", lse, lse_ref, TOL_LSE)
    return o, lse


def test_c5_full_parity(orc):
    """The KV-cache decode workload at full size (default split)."""
    w = I.WORKLOADS["C5"]
    sl, q, kc, vc = I.workload_inputs("C5")
    _parity(orc, sl, q, kc, vc, w.scale, "C5")


@pytest.mark.parametrize("kps", [1, 64, 100, 512, 4096, 1 << 20])
def test_split_count_invariance(orc, kps):
    sl, q, kc, vc = I.decode_inputs(4, 32, 8, 2048, 128, "bf16", seed=61, lo=1, hi=2048)
    o_ref, l_ref = gpu_decode(sl, q, kc, vc, 0.088, 0)
    o, l = _parity(orc, sl, q, kc, vc, 0.088, "split", kps)
    assert_close("kps=%d vs default (LSE)" % kps, l, l_ref, 1e-5)
    assert_close("kps=%d vs default (O)" % kps, o, o_ref, 2 ** -6)


@pytest.mark.parametrize("G,d", [(1, 128), (2, 64), (3, 128), (4, 64), (5, 64), (8, 128), (16, 128), (16, 64),
                                 (24, 128), (32, 64)])
def test_group_sizes(orc, G, d):
    Hkv = 2
    sl, q, kc, vc = I.decode_inputs(3, G * Hkv, Hkv, 700, d, "bf16", seed=70 + G, lo=1, hi=700)
    _parity(orc, sl, q, kc, vc, 1.0 / np.sqrt(d), "G=%d d=%d" % (G, d))


def test_edge_lengths(orc):
    """seq_len 0 (O = 0, LSE = -inf), 1, a ragged tail, exactly one split, and
    values beyond max_seq_len (clamped)."""
    B, Hq, Hkv, Lmax, d = 6, 8, 2, 600, 128
    _, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "bf16", seed=80)
    sl = torch.tensor([0, 1, 257, 256, 600, 5000], dtype=torch.int32)
    o, lse = gpu_decode(sl, q, kc, vc, 0.088)
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
    o_ref, l_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), 0.088)
    assert_close("edge lengths O", o, o_ref, TOL_O["bf16"])
    assert_close("edge lengths LSE", lse, l_ref, TOL_LSE)
    # one key per workgroup range: most of the 2048 workgroups get no key
    o, lse = gpu_decode(sl, q, kc, vc, 0.088, keys_per_split=1)
    assert_close("edge lengths O, 1-key ranges", o, o_ref, TOL_O["bf16"])
    assert_close("edge lengths LSE, 1-key ranges", lse, l_ref, TOL_LSE)


@pytest.mark.parametrize("kps", [0, 1, 33])
def test_many_short_sequences(orc, kps):
    """150 sequences (three pages of 64) of 0..40 keys, some empty: ranges
    cross many sequence boundaries and several workgroups get no keys."""
    B, Hq, Hkv, Lmax, d = 150, 8, 2, 48, 128
    _, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "bf16", seed=85)
    g = torch.Generator().manual_seed(86)
    sl = torch.randint(0, 41, (B,), generator=g, dtype=torch.int32)
    sl[::7] = 0
    o, lse = _parity(orc, sl, q, kc, vc, 0.088, "150 short sequences", kps)
    assert (o[sl.numpy() == 0] == 0).all() and np.isneginf(lse[sl.numpy() == 0]).all()


@pytest.mark.parametrize("B,hi,kps", [(65, 30, 0), (577, 24, 0), (1100, 16, 5), (3000, 8, 0), (2000, 12, 1)])
def test_large_batches(orc, B, hi, kps):
    """Batches past one page of 64 sequence lengths.  The split kernel loads
    the other pages eight at a time, for the batch total and again to find
    each range's first key, so 577 and more sequences span several groups of
    eight pages; empty sequences sit in every page, a whole page is empty,
    and so is the last sequence.  keys_per_split = 1 gives 2048 ranges of a
    few keys each."""
    Hq, Hkv, d = 8, 2, 64
    _, q, kc, vc = I.decode_inputs(B, Hq, Hkv, hi, d, "bf16", seed=90 + B)
    g = torch.Generator().manual_seed(91 + B)
    sl = torch.randint(0, hi + 1, (B,), generator=g, dtype=torch.int32)
    sl[::11] = 0
    sl[-1] = 0
    if B >= 192:
        sl[128:192] = 0
    o, lse = _parity(orc, sl, q, kc, vc, 0.125, "%d sequences" % B, kps)
    assert (o[sl.numpy() == 0] == 0).all() and np.isneginf(lse[sl.numpy() == 0]).all()


def test_large_batch_paged(orc):
    """A paged cache with 1500 sequences of up to 40 keys in blocks of 16."""
    sl, q, kp, vp, bt = I.paged_decode_inputs(1500, 8, 2, 64, 16, 3, "bf16", seed=95, lo=0, hi=40, spare_blocks=3)
    say("[paged] 1500 sequences, pool%s" % (tuple(kp.shape),))
    o, lse = E.attn_decode_paged(dev(q), dev(kp), dev(vp), dev(bt), dev(sl), scale=0.125)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(), 0.125)
    assert_close("1500-sequence paged O", I.to_f64(o), o_ref, TOL_O["bf16"])
    assert_close("1500-sequence paged LSE", I.to_f64(lse), lse_ref, TOL_LSE)


def test_empty_cache_rejected():
    """max_seq_len = 0 (and B = 0) are invalid sizes: the call is refused
    before any launch and leaves o untouched."""
    B, Hq, Hkv, d = 3, 8, 2, 64
    q = dev(torch.randn(B, Hq, d).to(torch.bfloat16))
    kc = torch.empty(B, Hkv, 0, d, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(E.AttnError) as ei:
        E.attn_decode(q, kc, kc.clone(), dev(torch.zeros(B, dtype=torch.int32)), o=o)
    assert ei.value.status == E.ATTN_ERR_INVALID_ARG
    with pytest.raises(E.AttnError) as ei:
        E.attn_decode(q[:0], kc[:0], kc[:0], dev(torch.zeros(0, dtype=torch.int32)))
    assert ei.value.status == E.ATTN_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (o == 7.0).all().item()


def test_nan_padding_never_read():
    """Cache rows at or beyond seq_len are poisoned with NaN; the result must
    equal the unpoisoned one bit for bit."""
    sl, q, kc, vc = I.decode_inputs(5, 16, 4, 1000, 128, "bf16", seed=90, lo=1, hi=999)
    o1, l1 = gpu_decode(sl, q, kc, vc, 0.088)
    kp, vp = kc.clone(), vc.clone()
    for b, L in enumerate(sl.tolist()):
        kp[b, :, L:] = float("nan")
        vp[b, :, L:] = float("nan")
    o2, l2 = gpu_decode(sl, q, kp, vp, 0.088)
    assert np.isfinite(o2).all()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_matches_prefill_last_row(orc):
    """A decode step equals the last row of causal prefill over the same rows."""
    L, Hq, Hkv, d = 777, 8, 2, 128
    g = torch.Generator().manual_seed(99)
    qf = torch.randn(1, Hq, L, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, Hkv, L, d, generator=g).to(torch.bfloat16)
    v = torch.randn(1, Hkv, L, d, generator=g).to(torch.bfloat16)
    op, lp = gpu_fwd(qf, k, v, 0.088, True)
    od, ld = gpu_decode(torch.tensor([L], dtype=torch.int32), qf[:, :, L - 1].contiguous(), k, v, 0.088)
    assert_close("decode vs prefill last row (LSE)", ld[0], lp[0, :, L - 1], 1e-5)
    assert_close("decode vs prefill last row (O)", od[0], op[0, :, L - 1], 2 * TOL_O["bf16"])
    o_ref, l_ref = orc.attn_rows(I.to_f64(qf), I.to_f64(k), I.to_f64(v), 0.088, True,
                                 np.array([[0, h, L - 1] for h in range(Hq)], dtype=np.int32))
    assert_close("decode vs oracle last row", od[0], o_ref, TOL_O["bf16"])


def test_run_twice_bitwise():
    sl, q, kc, vc = I.decode_inputs(8, 32, 8, 1024, 128, "bf16", seed=95, lo=1, hi=1024)
    a = gpu_decode(sl, q, kc, vc, 0.088)
    b = gpu_decode(sl, q, kc, vc, 0.088)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_workspace_reuse_and_explicit_buffer(orc):
    """One workspace filled with garbage serves calls of different sizes in
    turn; a buffer one word short is refused."""
    need = max(E.attn_decode_workspace_bytes(4, 32, 8, 512, 128), E.attn_decode_workspace_bytes(9, 16, 2, 300, 64))
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda")
    for args, seed in [((4, 32, 8, 512, 128), 97), ((9, 16, 2, 300, 64), 98), ((4, 32, 8, 512, 128), 99)]:
        B, Hq, Hkv, Lmax, d = args
        sl, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "bf16", seed=seed, lo=1, hi=Lmax)
        o, lse = E.attn_decode(dev(q), dev(kc), dev(vc), dev(sl), workspace=ws)
        torch.cuda.synchronize()
        o_ref, l_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), 1 / np.sqrt(d))
        assert_close("shared workspace O %s" % (args,), I.to_f64(o), o_ref, TOL_O["bf16"])
        assert_close("shared workspace LSE %s" % (args,), I.to_f64(lse), l_ref, TOL_LSE)
    small = E.attn_decode_workspace_bytes(4, 32, 8, 512, 128)
    with pytest.raises(E.AttnError):
        E.attn_decode(dev(q), dev(kc), dev(vc), dev(sl), workspace=ws[: small - 16])


# ---------------------------------------------------------------------------
# Paged KV cache (attn_decode_paged)
# ---------------------------------------------------------------------------
def gpu_decode_paged(sl, q, kp, vp, bt, scale, keys_per_split=0):
    o, lse = E.attn_decode_paged(dev(q), dev(kp), dev(vp), dev(bt), dev(sl.to(torch.int32)), scale=scale,
                                 keys_per_split=keys_per_split)
    torch.cuda.synchronize()
    return I.to_f64(o), I.to_f64(lse)


def _paged_parity(orc, sl, q, kp, vp, bt, scale, label, kps=0):
    say("[paged] %s q%s pool%s table%s kps=%d L=%s" % (label, tuple(q.shape), tuple(kp.shape), tuple(bt.shape), kps,
                                                       sl.tolist()[:8]))
    o, lse = gpu_decode_paged(sl, q, kp, vp, bt, scale, kps)
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(), scale)
    assert_close(label + " O", o, o_ref, TOL_O["bf16"])
    assert_close(label + " LSE", lse, lse_ref, TOL_LSE)
    return o, lse


@pytest.mark.parametrize("bs", [16, 64, 256])
def test_paged_kv_cache_workload(orc, bs):
    """The KV-cache decode workload's shape (16 sequences, 32 query heads over
    8 KV heads, d = 128, lengths uniform in [512, 4096]) in a shuffled pool."""
    sl, q, kp, vp, bt = I.paged_decode_inputs(16, 32, 8, 128, bs, 4096 // bs, "bf16", seed=1104, spare_blocks=3)
    _paged_parity(orc, sl, q, kp, vp, bt, 1 / np.sqrt(128), "C5 paged bs=%d" % bs)


@pytest.mark.parametrize("bs,G,d,kps", [(32, 4, 128, 0), (48, 2, 64, 0), (1, 8, 128, 0), (7, 4, 64, 100),
                                        (128, 16, 128, 1), (33, 24, 128, 0)])
def test_paged_block_sizes_and_groups(orc, bs, G, d, kps):
    Hkv = 2
    sl, q, kp, vp, bt = I.paged_decode_inputs(5, G * Hkv, Hkv, d, bs, -(-700 // bs), "bf16", seed=1200 + bs + G,
                                              lo=0, hi=700, spare_blocks=2)
    _paged_parity(orc, sl, q, kp, vp, bt, 1 / np.sqrt(d), "bs=%d G=%d d=%d" % (bs, G, d), kps)


def test_paged_equals_contiguous(orc):
    """The same rows paged (identity table) and contiguous give the same
    results within tolerance, and both match the oracle."""
    sl, q, kc, vc = I.decode_inputs(6, 16, 4, 1024, 128, "bf16", seed=1300, lo=1, hi=1024)
    bs = 64
    mb = 1024 // bs
    kp = kc.reshape(6, 4, mb, bs, 128).permute(0, 2, 1, 3, 4).reshape(6 * mb, 4, bs, 128).contiguous()
    vp = vc.reshape(6, 4, mb, bs, 128).permute(0, 2, 1, 3, 4).reshape(6 * mb, 4, bs, 128).contiguous()
    bt = torch.arange(6 * mb, dtype=torch.int32).reshape(6, mb)
    op, lp = gpu_decode_paged(sl, q, kp, vp, bt, 0.088)
    oc, lc = gpu_decode(sl, q, kc, vc, 0.088)
    assert_close("paged vs contiguous O", op, oc, TOL_O["bf16"])
    assert_close("paged vs contiguous LSE", lp, lc, 1e-5)
    o_ref, l_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), 0.088)
    assert_close("paged vs oracle O", op, o_ref, TOL_O["bf16"])


def test_paged_shared_prefix_unused_blocks_and_clamping(orc):
    """Sequences sharing prefix blocks; every block no valid row lives in is
    poisoned with NaN (never read: bitwise equal results); table entries out
    of range are clamped into the pool, as the oracle does."""
    sl, q, kp, vp, bt = I.paged_decode_inputs(6, 8, 2, 128, 32, 20, "bf16", seed=1400, lo=100, hi=640,
                                              spare_blocks=5)
    bt[1, :3] = bt[0, :3]
    bt[3, :2] = bt[0, :2]
    o1, l1 = _paged_parity(orc, sl, q, kp, vp, bt, 0.088, "shared prefix")
    used = set()
    for b in range(6):
        used.update(int(x) for x in bt[b, :(int(sl[b]) + 31) // 32].tolist())
    kpp, vpp = kp.clone(), vp.clone()
    for blk in range(kp.shape[0]):
        if blk not in used:
            kpp[blk] = float("nan")
            vpp[blk] = float("nan")
    o2, l2 = gpu_decode_paged(sl, q, kpp, vpp, bt, 0.088)
    assert np.isfinite(o2).all()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    bt2 = bt.clone()
    bt2[2, 0] = -5
    bt2[4, 1] = kp.shape[0] + 9
    _paged_parity(orc, sl, q, kp, vp, bt2, 0.088, "clamped entries")


def test_paged_empty_pool_rejected():
    """A pool of no blocks is an invalid size: refused before any launch."""
    q = dev(torch.randn(3, 8, 64).to(torch.bfloat16))
    kp = torch.empty(0, 2, 32, 64, dtype=torch.bfloat16, device="cuda")
    bt = dev(torch.zeros(3, 4, dtype=torch.int32))
    with pytest.raises(E.AttnError) as ei:
        E.attn_decode_paged(q, kp, kp.clone(), bt, dev(torch.tensor([5, 0, 100], dtype=torch.int32)))
    assert ei.value.status == E.ATTN_ERR_INVALID_ARG
