"""The entry points under HIP graph capture.  A forward pass, a decode step
(contiguous and paged cache) and a backward pass captured in one graph (bf16,
and again fp32), replayed several times with other
eager work and synchronisations between the replays, reproduce the eager
results bit for bit on every replay.  (None of the launches records a memset;
every output is written by the kernels.)"""
import pytest
import torch

import exact_scaled_dot_sdpa_amd as E
from exact_scaled_dot_sdpa_amd import inputs as I
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dev = torch.device("cuda")
    B, Hq, Hkv, N, d = 1, 8, 2, 700, 128
    q, k, v, do = (t.to(dev) for t in I.bwd_inputs(B, Hq, Hkv, N, N, d, "bf16", seed=71))
    sl, qd, kc, vc = (t.to(dev) for t in I.decode_inputs(4, 32, 8, 1024, 128, "bf16", seed=72, lo=1, hi=1024))
    slp, qp, kp, vp, bt = (t.to(dev) for t in I.paged_decode_inputs(4, 32, 8, 128, 64, 16, "bf16", seed=73,
                                                                    lo=1, hi=1024))
    ws_d = torch.empty(E.attn_decode_workspace_bytes(4, 32, 8, 1024, 128), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(E.attn_bwd_workspace_bytes(B, Hq, N), dtype=torch.uint8, device=dev)

    ws_p = torch.empty_like(ws_d)

    def run(o, l, od, ld, op, lp, dq, dk, dv):
        E.attn_fwd(q, k, v, scale=0.09, causal=True, o=o, lse=l)
        E.attn_decode(qd, kc, vc, sl, scale=0.088, o=od, lse=ld, workspace=ws_d)
        E.attn_decode_paged(qp, kp, vp, bt, slp, scale=0.088, o=op, lse=lp, workspace=ws_p)
        E.attn_bwd(q, k, v, o, do, l, scale=0.09, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws_b)

    def outputs():
        return (torch.empty_like(q), torch.empty(B, Hq, N, device=dev), torch.empty_like(qd),
                torch.empty(4, 32, device=dev), torch.empty_like(qp), torch.empty(4, 32, device=dev),
                torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))

    ref = outputs()
    run(*ref)
    torch.cuda.synchronize()

    got = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        run(*got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*got)
    names = ["o", "lse", "o_dec", "lse_dec", "o_paged", "lse_paged", "dq", "dk", "dv"]
    for rep in range(4):
        for t in got:
            t.zero_()
        E.attn_fwd(q, k, v, scale=0.5, causal=False)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, got, ref):
            assert torch.equal(a, b), "replay %d: %s differs from the eager result" % (rep, name)
        say("  graph replay %d: all outputs bit-equal to eager" % rep)


def test_graph_replays_match_eager_f32():
    """The fp32 paths under capture: forward, decode (contiguous and paged)
    and backward on fp32 inputs, replayed with eager work in between, each
    replay bit-equal to the eager result."""
    dev = torch.device("cuda")
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 64
    q, k, v, do = (t.to(dev) for t in I.bwd_inputs(B, Hq, Hkv, N, N, d, "f32", seed=81))
    sl, qd, kc, vc = (t.to(dev) for t in I.decode_inputs(4, 16, 4, 700, 128, "f32", seed=82, lo=1, hi=700))
    slp, qp, kp, vp, bt = (t.to(dev) for t in I.paged_decode_inputs(3, 8, 2, 64, 32, 12, "f32", seed=83,
                                                                    lo=1, hi=384))
    ws_d = torch.empty(E.attn_decode_workspace_bytes(4, 16, 4, 700, 128), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(E.attn_decode_workspace_bytes(3, 8, 2, 384, 64), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(E.attn_bwd_workspace_bytes(B, Hq, N), dtype=torch.uint8, device=dev)

    def run(o, l, od, ld, op, lp, dq, dk, dv):
        E.attn_fwd(q, k, v, scale=0.12, causal=True, o=o, lse=l)
        E.attn_decode(qd, kc, vc, sl, scale=0.088, o=od, lse=ld, workspace=ws_d)
        E.attn_decode_paged(qp, kp, vp, bt, slp, scale=0.125, o=op, lse=lp, workspace=ws_p)
        E.attn_bwd(q, k, v, o, do, l, scale=0.12, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws_b)

    def outputs():
        return (torch.empty_like(q), torch.empty(B, Hq, N, device=dev), torch.empty_like(qd),
                torch.empty(4, 16, device=dev), torch.empty_like(qp), torch.empty(3, 8, device=dev),
                torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))

    ref = outputs()
    run(*ref)
    torch.cuda.synchronize()
    got = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        run(*got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*got)
    names = ["o", "lse", "o_dec", "lse_dec", "o_paged", "lse_paged", "dq", "dk", "dv"]
    for rep in range(3):
        for t in got:
            t.zero_()
        E.attn_fwd(q, k, v, scale=0.5, causal=False)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, got, ref):
            assert torch.equal(a, b), "replay %d: %s differs from the eager result" % (rep, name)
        say("  fp32 graph replay %d: all outputs bit-equal to eager" % rep)
