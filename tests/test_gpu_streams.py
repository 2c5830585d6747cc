"""Calls issued on several streams at once give the same bits as the same
calls issued one after another.

The library keeps no per-call state outside the caller's buffers (outputs and
workspaces), so calls that overlap in time on one device cannot interact.
Every entry point that takes a workspace, or none, runs here on four side
streams at the default priority, three rounds each, and every output is
compared bit for bit with a serial run on the current stream.
(attn_decode_noalloc is left out: its calls share the library's own device
array and, as its declaration says, race when they overlap.)"""
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _jobs():
    """(name, call) pairs; each call issues its work on the current stream
    and returns its output tensors."""
    jobs = []

    q, k, v = (dev(t) for t in I.prefill_inputs(2, 8, 2, 700, 700, 128, "bf16", seed=7100))
    jobs.append(("fwd bf16 causal", lambda: E.attn_fwd(q, k, v, scale=0.088, causal=True)))

    q2, k2, v2 = (dev(t) for t in I.prefill_inputs(1, 4, 4, 200, 450, 64, "bf16", seed=7101))
    jobs.append(("fwd bf16 rect", lambda: E.attn_fwd(q2, k2, v2, scale=0.125, causal=False)))

    q3, k3, v3 = (dev(t) for t in I.prefill_inputs(1, 2, 1, 150, 150, 64, "f32", seed=7102))
    jobs.append(("fwd f32", lambda: E.attn_fwd(q3, k3, v3, scale=0.125, causal=True)))

    q4, k4, v4 = (dev(t) for t in I.prefill_inputs(1, 8, 2, 333, 333, 128, "fp8", seed=7103))
    jobs.append(("fwd fp8", lambda: E.attn_fwd_fp8(q4, k4, v4, scale=0.088, causal=True)))

    sl, qd, kc, vc = (dev(t) for t in I.decode_inputs(8, 16, 4, 1500, 128, "bf16", seed=7104, lo=1, hi=1500))
    jobs.append(("decode", lambda: E.attn_decode(qd, kc, vc, sl, scale=0.088)))
    jobs.append(("decode split", lambda: E.attn_decode_split(qd, kc, vc, sl, keys_per_split=100, scale=0.088)))

    slp, qp, kp, vp, bt = (dev(t) for t in I.paged_decode_inputs(6, 16, 4, 128, 32, 40, "bf16", seed=7105,
                                                                lo=0, hi=1280, spare_blocks=3))
    jobs.append(("decode paged", lambda: E.attn_decode_paged(qp, kp, vp, bt, slp.to(torch.int32), scale=0.088)))

    qb, kb, vb, dob = (dev(t) for t in I.bwd_inputs(1, 4, 2, 300, 300, 128, "bf16", seed=7106))
    ob, lseb = E.attn_fwd(qb, kb, vb, scale=0.088, causal=True)
    jobs.append(("bwd bf16", lambda: E.attn_bwd(qb, kb, vb, ob, dob, lseb, scale=0.088, causal=True)))

    qf, kf, vf, dof = (dev(t) for t in I.bwd_inputs(1, 2, 1, 100, 100, 64, "f32", seed=7107))
    of, lsef = E.attn_fwd(qf, kf, vf, scale=0.125, causal=False)
    jobs.append(("bwd f32", lambda: E.attn_bwd(qf, kf, vf, of, dof, lsef, scale=0.125, causal=False)))
    torch.cuda.synchronize()
    return jobs


def _flat(out):
    return list(out) if isinstance(out, (tuple, list)) else [out]


def test_concurrent_streams_match_serial():
    jobs = _jobs()
    serial = {}
    for name, call in jobs:
        serial[name] = [t.clone() for t in _flat(call())]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in range(4)]
    results = []
    for rnd in range(3):
        for i, (name, call) in enumerate(jobs):
            s = streams[(i + rnd) % len(streams)]
            with torch.cuda.stream(s):
                results.append((name, rnd, _flat(call())))
    torch.cuda.synchronize()

    for name, rnd, outs in results:
        ref = serial[name]
        assert len(outs) == len(ref), name
        for j, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), "%s (round %d, output %d) differs from the serial call" % (name, rnd, j)
    say("[streams] %d concurrent calls on %d streams match the serial ones" % (len(results), len(streams)))
