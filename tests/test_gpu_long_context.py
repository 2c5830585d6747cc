"""Long-context extremes against the fp64 oracle.

Decode: one sequence of 131072 keys per batch entry, so every split
workgroup falls inside the same few segments and the merge kernel folds about
a hundred partial results per segment; a second batch mixes that length with
a 3-key sequence and an empty one.  Prefill: a short ragged query chunk
attending to 65536 keys, causal with bottom-right alignment and non-causal,
compared on every output element.  Each case also bounds the error relative
to the largest output of each sequence (decode) or head (prefill): over this
many keys the outputs shrink to a few hundredths, where the absolute bf16
bound alone would not constrain them."""
import numpy as np
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import TOL_LSE, TOL_O, assert_close, assert_rel_per_group, dev, gpu_decode, say
from gpu_util import gpu_fwd as gpu_fwd_np

pytestmark = pytest.mark.gpu

LONG = 1 << 17


def test_decode_one_long_sequence(orc):
    sl, q, kc, vc = I.decode_inputs(1, 32, 8, LONG, 128, "bf16", seed=901, lo=LONG, hi=LONG)
    assert sl.tolist() == [LONG]
    say("[decode-long] q%s cache%s L=%d" % (tuple(q.shape), tuple(kc.shape), LONG))
    o, lse = gpu_decode(sl, q, kc, vc, 128 ** -0.5)
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), 128 ** -0.5)
    assert_close("L=2^17 O", o, o_ref, TOL_O["bf16"])
    assert_rel_per_group("L=2^17 O", o, o_ref, 1)
    assert_close("L=2^17 LSE", lse, lse_ref, TOL_LSE)


def test_decode_long_mixed_with_short_and_empty(orc):
    _, q, kc, vc = I.decode_inputs(3, 16, 4, LONG, 64, "bf16", seed=902)
    sl = torch.tensor([3, LONG, 0], dtype=torch.int32)
    say("[decode-long] q%s cache%s L=%s" % (tuple(q.shape), tuple(kc.shape), sl.tolist()))
    o, lse = gpu_decode(sl, q, kc, vc, 0.125)
    o_ref, lse_ref = orc.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), 0.125)
    assert_close("mixed O", o, o_ref, TOL_O["bf16"])
    assert_rel_per_group("mixed O (sequences 0, 1)", o[:2], o_ref[:2], 1)
    assert_close("mixed LSE", lse, lse_ref, TOL_LSE)
    assert (o[2] == 0).all() and np.isneginf(lse[2]).all(), "empty sequence: O = 0 and LSE = -inf"


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_short_chunk_over_long_keys(orc, causal):
    B, Hq, Hkv, Nq, Nk, d = 1, 8, 2, 300, 1 << 16, 128
    q, k, v = I.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=903 + causal)
    say("[prefill-long] q%s k%s causal=%s" % (tuple(q.shape), tuple(k.shape), causal))
    o, lse = gpu_fwd_np(q, k, v, d ** -0.5, causal)
    o_ref, lse_ref = orc.attn(I.to_f64(q), I.to_f64(k), I.to_f64(v), d ** -0.5, causal)
    assert_close("Nk=2^16 O", o, o_ref, TOL_O["bf16"])
    assert_rel_per_group("Nk=2^16 O", o, o_ref, 2)
    assert_close("Nk=2^16 LSE", lse, lse_ref, TOL_LSE)


def test_paged_decode_long_sequences(orc):
    """Paged cache at block size 16: each 100k+-key sequence spans over 6000
    pool blocks in shuffled order, so the wave's 64-entry page of the block
    table is reloaded about a hundred times per sequence."""
    bs = 16
    sl, q, kp, vp, bt = I.paged_decode_inputs(2, 16, 4, 128, bs, LONG // bs, "bf16", seed=905, lo=100000, hi=LONG,
                                              spare_blocks=5)
    say("[paged-long] q%s pool%s table%s L=%s" % (tuple(q.shape), tuple(kp.shape), tuple(bt.shape), sl.tolist()))
    o, lse = E.attn_decode_paged(dev(q), dev(kp), dev(vp), dev(bt), dev(sl), scale=128 ** -0.5)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode_paged(I.to_f64(q), I.to_f64(kp), I.to_f64(vp), bt.numpy(), sl.numpy(), 128 ** -0.5)
    assert_close("paged L>=1e5 O", I.to_f64(o), o_ref, TOL_O["bf16"])
    assert_rel_per_group("paged L>=1e5 O", I.to_f64(o), o_ref, 1)
    assert_close("paged L>=1e5 LSE", I.to_f64(lse), lse_ref, TOL_LSE)
