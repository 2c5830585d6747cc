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
