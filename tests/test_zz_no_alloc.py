"""attn_decode_noalloc (the decode call that allocates nothing) against
attn_decode on the same inputs, through the C ABI: two calls in a row, the
second with a smaller input, each bit-identical to attn_decode (same kernels,
same split) and within the bf16 tolerances of the fp64 oracle; sizes whose
partial results exceed the library's scratch array are refused."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, dev, say

pytestmark = pytest.mark.gpu


def _check(orc, B, Hq, Hkv, Lmax, d, seed):
    sl, q, kc, vc = I.decode_inputs(B, Hq, Hkv, Lmax, d, "bf16", seed=seed, lo=0, hi=Lmax)
    say("[noalloc] B%d Hq%d Hkv%d Lmax%d d%d L=%s" % (B, Hq, Hkv, Lmax, d, sl.tolist()[:8]))
    qd, kd, vd, sd = dev(q), dev(kc), dev(vc), dev(sl)
    scale = 1.0 / np.sqrt(d)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    E.attn_decode_noalloc(qd, kd, vd, sd, o, lse, scale=scale)
    o_ref, lse_ref = E.attn_decode(qd, kd, vd, sd, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "differs from attn_decode"
    oo, lo = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), scale)
    assert_close("noalloc O", I.to_f64(o), oo, TOL_O["bf16"])
    assert_close("noalloc LSE", I.to_f64(lse), lo, TOL_LSE)


def test_noalloc_matches_decode_twice(orc):
    """The decode workload's shape, then a smaller one: the second call
    reuses the array the first one left its partial results in."""
    _check(orc, 16, 32, 8, 4096, 128, seed=7001)
    _check(orc, 3, 8, 2, 700, 64, seed=7002)


def test_noalloc_refuses_oversize():
    B, Hq, Hkv, d = 2000, 128, 8, 128
    need = E.attn_decode_workspace_bytes(B, Hq, Hkv, 1, d)
    assert need > 32 << 20
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, Hkv, 1, d, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 5.0)
    with pytest.raises(E.AttnError) as ei:
        E.attn_decode_noalloc(q, kc, kc, torch.ones(B, dtype=torch.int32, device="cuda"), o)
    assert ei.value.status == E.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (o == 5.0).all().item()


def test_noalloc_under_graph_capture():
    """The use the entry point is for: a decode step captured in a HIP graph
    with no workspace to allocate, replayed several times.  Between the
    replays an eager call of another size reuses the same array and the
    stream is synchronised; every replay and every eager call reproduces
    attn_decode bit for bit."""
    sl, q, kc, vc = (dev(t) for t in I.decode_inputs(4, 32, 8, 1024, 128, "bf16", seed=7003, lo=1, hi=1024))
    s2, q2, k2, v2 = (dev(t) for t in I.decode_inputs(3, 8, 2, 700, 64, "bf16", seed=7004, lo=0, hi=700))
    o_ref, lse_ref = E.attn_decode(q, kc, vc, sl, scale=0.088)
    o2_ref, lse2_ref = E.attn_decode(q2, k2, v2, s2, scale=0.125)
    o = torch.empty_like(q)
    lse = torch.empty(4, 32, dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(q2)
    lse2 = torch.empty(3, 8, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        E.attn_decode_noalloc(q, kc, vc, sl, o, lse, scale=0.088)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.attn_decode_noalloc(q, kc, vc, sl, o, lse, scale=0.088)
    for rep in range(4):
        say("[noalloc graph] replay %d" % rep)
        o.zero_()
        lse.zero_()
        E.attn_decode_noalloc(q2, k2, v2, s2, o2, lse2, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(o2, o2_ref) and torch.equal(lse2, lse2_ref), "eager call %d" % rep
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "replay %d" % rep
