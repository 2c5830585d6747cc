"""Tensors past 2^32 elements: every kernel addresses rows with 64-bit
offsets.

Each case allocates device tensors of at least 2^32 elements (8 GiB of bf16
each) and checks, against the oracle, the heads or sequences that sit at the
far end, where an element offset no longer fits in 32 bits: a 32-bit product
anywhere in the address arithmetic would read or write the wrong rows there.

  * attn_fwd, attn_fwd_fp8 and attn_bwd on B=1024 batches of 128 heads of 256
    rows (d = 128): q, k and v each hold 2^32 elements.  The first and last
    batches hold seeded inputs, the rest zeros; both are compared with the
    oracle, every row.
  * attn_decode on a [2, 8, 2^21, 128] cache (2^32 elements): the rows of the
    last sequence start past 2^31 elements.  Rows at or past seq_lens are NaN.
  * attn_decode_paged on a pool of 65536 blocks of 64 rows (2^32 elements),
    the sequences' blocks at the top of the pool, every other block NaN.
  * The fp32 paths (forward and backward, decode, paged decode) the same way,
    at sizes (2.2e9 to 3.2e9 elements) that already put the checked rows past
    2^31 elements and 2^33 bytes.

The largest case needs about 80 GiB of device memory; each case is skipped on
a device with less free memory than it needs."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, grad_floors, say

pytestmark = pytest.mark.gpu

GiB = 1 << 30


def _need(gib):
    free, _ = torch.cuda.mem_get_info()
    if free < gib * GiB:
        pytest.skip("needs %d GiB of free device memory, %d GiB free" % (gib, free // GiB))


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


B, H, N, D = 1024, 128, 256, 128  # B*H*N*D = 2^32
SCALE = 1 / np.sqrt(D)


def _big_inputs(dtype, seed, with_do=False, nb=B):
    """Zero-filled [nb, H, N, D] device tensors whose first and last batches
    hold seeded inputs; also returns those CPU inputs, batch 0 then nb-1."""
    tdt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "f32": torch.float32}[dtype]
    n = 4 if with_do else 3
    big = []
    for _ in range(n):
        t = torch.empty((nb, H, N, D), dtype=torch.uint8 if dtype == "fp8" else tdt, device="cuda")
        t.zero_()
        big.append(t.view(tdt) if dtype == "fp8" else t)
    if with_do:
        small = I.bwd_inputs(2, H, H, N, N, D, dtype, seed)
    else:
        small = I.prefill_inputs(2, H, H, N, N, D, dtype, seed)
    for t, s in zip(big, small):
        t[0].copy_(s[0].to("cuda"))
        t[nb - 1].copy_(s[1].to("cuda"))
    assert big[0].numel() > 1 << 31
    return big, small


def _check_prefill(orc, o, lse, small, label, tol=TOL_O["bf16"]):
    nb = o.shape[0]
    o = o[[0, nb - 1]].cpu()
    lse = lse[[0, nb - 1]].cpu()
    q, k, v = (I.to_f64(t) for t in small[:3])
    o_ref, lse_ref = orc.attn(q, k, v, SCALE, True)
    assert_close(label + " O (first and last batch)", I.to_f64(o), o_ref, tol)
    assert_close(label + " LSE (first and last batch)", I.to_f64(lse), lse_ref, TOL_LSE)


def test_fwd_past_2_32_elements(orc):
    _need(40)
    (q, k, v), small = _big_inputs("bf16", 7200)
    say("[large] attn_fwd q%s (%d elements each)" % (tuple(q.shape), q.numel()))
    o, lse = E.attn_fwd(q, k, v, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    _check_prefill(orc, o, lse, small, "fwd")
    # the zero-filled batches: uniform weights over zero values
    assert torch.count_nonzero(o[1:B - 1]).item() == 0


def test_fwd_fp8_past_2_32_elements(orc):
    _need(24)
    (q, k, v), small = _big_inputs("fp8", 7201)
    say("[large] attn_fwd_fp8 q%s (%d elements each)" % (tuple(q.shape), q.numel()))
    o, lse = E.attn_fwd_fp8(q, k, v, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    _check_prefill(orc, o, lse, small, "fwd fp8")


def test_bwd_past_2_32_elements(orc):
    _need(80)
    (q, k, v, do), small = _big_inputs("bf16", 7202, with_do=True)
    say("[large] attn_bwd q%s (%d elements each)" % (tuple(q.shape), q.numel()))
    o, lse = E.attn_fwd(q, k, v, scale=SCALE, causal=True)
    grads = E.attn_bwd(q, k, v, o, do, lse, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    del o, lse
    qs, ks, vs, dos = small
    refs = orc.attn_bwd(I.to_f64(qs), I.to_f64(ks), I.to_f64(vs), I.to_f64(dos), SCALE, True)
    floors = grad_floors(orc, qs, ks, vs, dos, SCALE, True)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        g = I.to_f64(g[[0, B - 1]].cpu())
        assert np.isfinite(g).all(), name
        top = float(np.abs(r).max())
        rms = float(np.sqrt(np.mean(r ** 2)))
        e_max = float(np.abs(g - r).max())
        e_rms = float(np.sqrt(np.mean((g - r) ** 2)))
        say("  %s max err %.2e of max|ref|, rms err %.2e of rms" % (name, e_max / top, e_rms / rms))
        assert e_max <= 2e-2 * top + floors[name] and e_rms <= 6e-3 * rms + floors[name], name


def test_decode_past_2_32_elements(orc):
    _need(24)
    Bd, Hq, Hkv, Lmax = 2, 32, 8, 1 << 21
    sl, q, kc, vc = I.decode_inputs(Bd, Hq, Hkv, 1900, D, "bf16", seed=7203, lo=700, hi=1900)
    Lv = int(sl.max())
    big = []
    for c in (kc, vc):
        t = torch.full((Bd, Hkv, Lmax, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        for b in range(Bd):
            t[b, :, :int(sl[b])].copy_(c[b, :, :int(sl[b])].to("cuda"))
        big.append(t)
    assert big[0].numel() == 1 << 32
    say("[large] attn_decode cache%s, seq_lens %s" % (tuple(big[0].shape), sl.tolist()))
    o, lse = E.attn_decode(q.cuda(), big[0], big[1], sl.cuda(), scale=SCALE)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc[:, :, :Lv]), I.to_f64(vc[:, :, :Lv]), sl.numpy(), SCALE)
    assert_close("decode O", I.to_f64(o), o_ref, TOL_O["bf16"])
    assert_close("decode LSE", I.to_f64(lse), lse_ref, TOL_LSE)


def test_decode_paged_past_2_32_elements(orc):
    _need(24)
    Bd, Hq, Hkv, bs, nb = 3, 32, 8, 64, 1 << 16
    sl, q, kp, vp, bt = I.paged_decode_inputs(Bd, Hq, Hkv, D, bs, 40, "bf16", seed=7204, lo=100, hi=2560)
    top = nb - kp.shape[0]  # the used blocks go to the top of the pool
    big = []
    for p in (kp, vp):
        t = torch.full((nb, Hkv, bs, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        t[top:].copy_(p.to("cuda"))
        big.append(t)
    assert big[0].numel() == 1 << 32
    bt_big = bt + top
    say("[large] attn_decode_paged pool%s, blocks from %d, seq_lens %s" % (tuple(big[0].shape), top, sl.tolist()))
    o, lse = E.attn_decode_paged(q.cuda(), big[0], big[1], bt_big.cuda(), sl.cuda(), scale=SCALE)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(), SCALE)
    assert_close("paged decode O", I.to_f64(o), o_ref, TOL_O["bf16"])
    assert_close("paged decode LSE", I.to_f64(lse), lse_ref, TOL_LSE)


# fp32: 520 batches (2.2e9 elements, 8.7 GB per tensor) already put the last
# batch past 2^31 elements and its bytes past 2^33.
NB32 = 520


def test_fwd_bwd_f32_past_2_31_elements(orc):
    _need(80)
    (q, k, v, do), small = _big_inputs("f32", 7205, with_do=True, nb=NB32)
    say("[large] fp32 attn_fwd + attn_bwd q%s (%d elements each)" % (tuple(q.shape), q.numel()))
    o, lse = E.attn_fwd(q, k, v, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    _check_prefill(orc, o, lse, small, "fwd f32", TOL_O["f32"])
    grads = E.attn_bwd(q, k, v, o, do, lse, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    del o, lse
    qs, ks, vs, dos = small
    refs = orc.attn_bwd(I.to_f64(qs), I.to_f64(ks), I.to_f64(vs), I.to_f64(dos), SCALE, True)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        g = I.to_f64(g[[0, NB32 - 1]].cpu())
        top = float(np.abs(r).max())
        e_max = float(np.abs(g - r).max())
        say("  %s max err %.2e (max|ref| %.2e)" % (name, e_max, top))
        assert e_max <= 3e-5 * top + 2e-6, name


def test_decode_f32_past_2_31_elements(orc):
    _need(32)
    Bd, Hq, Hkv, Lmax = 2, 32, 8, 3 << 19  # 3.2e9 elements per cache
    sl, q, kc, vc = I.decode_inputs(Bd, Hq, Hkv, 1900, D, "f32", seed=7206, lo=700, hi=1900)
    Lv = int(sl.max())
    big = []
    for c in (kc, vc):
        t = torch.full((Bd, Hkv, Lmax, D), float("nan"), dtype=torch.float32, device="cuda")
        for b in range(Bd):
            t[b, :, :int(sl[b])].copy_(c[b, :, :int(sl[b])].to("cuda"))
        big.append(t)
    say("[large] fp32 attn_decode cache%s, seq_lens %s" % (tuple(big[0].shape), sl.tolist()))
    o, lse = E.attn_decode(q.cuda(), big[0], big[1], sl.cuda(), scale=SCALE)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc[:, :, :Lv]), I.to_f64(vc[:, :, :Lv]), sl.numpy(), SCALE)
    assert_close("decode f32 O", I.to_f64(o), o_ref, TOL_O["f32"])
    assert_close("decode f32 LSE", I.to_f64(lse), lse_ref, TOL_LSE)


def test_decode_paged_f32_past_2_31_elements(orc):
    _need(32)
    Bd, Hq, Hkv, bs, nb = 3, 32, 8, 64, 40000  # 2.6e9 elements per pool
    sl, q, kp, vp, bt = I.paged_decode_inputs(Bd, Hq, Hkv, D, bs, 40, "f32", seed=7207, lo=100, hi=2560)
    top = nb - kp.shape[0]
    big = []
    for p in (kp, vp):
        t = torch.full((nb, Hkv, bs, D), float("nan"), dtype=torch.float32, device="cuda")
        t[top:].copy_(p.to("cuda"))
        big.append(t)
    say("[large] fp32 attn_decode_paged pool%s, blocks from %d, seq_lens %s" % (tuple(big[0].shape), top,
                                                                               sl.tolist()))
    o, lse = E.attn_decode_paged(q.cuda(), big[0], big[1], (bt + top).cuda(), sl.cuda(), scale=SCALE)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(), SCALE)
    assert_close("paged decode f32 O", I.to_f64(o), o_ref, TOL_O["f32"])
    assert_close("paged decode f32 LSE", I.to_f64(lse), lse_ref, TOL_LSE)
