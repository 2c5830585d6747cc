#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-paged] [--no-graph] [--no-rect]
                    [--no-bwd] [--no-fp8] [--no-configs]

One step is one pass of the whole path over synthetic inputs already resident
in device memory:
  * prefill: attn_fwd on the GQA workload (B=1, 64 query heads over 8 KV heads,
    N=8192, d=128, bf16, causal), and
  * decode:  attn_decode on the KV-cache workload (16 sequences, 32 query heads
    over 8 KV heads, d=128, bf16 cache, lengths uniform in [512, 4096]); each
    step reads one of 4 distinct cache replicas (>= 600 MB together), so the
    cache is read from HBM rather than from the 256 MB last-level cache.

The JSON line reports the prefill throughput in TFLOP/s as `value` (algorithmic
FLOPs: 4*d per visible query/key pair), the decode bandwidth in GB/s (valid
cache rows plus q, o, lse) in `decode`, and for each kernel its roofline
fraction from its average duration measured with HIP events on the stream the
kernels run on (mean, with the median beside it).  The prefill roofline also
gives the engine clock that the committed SQ counter run observed over the
kernel (`sclk_ghz_counters`) and the same rate against the dense peak scaled
to that clock (`frac_at_sclk`); `frac` stays against the published peak.
`cpu_baseline` times the
fp64 oracle on a bounded sample of the prefill rows on the host cores, and
(`per_config`) on each smaller prefill workload in full, next to that
workload's GPU time; `parity` compares the timed prefill's outputs with the
oracle's on those sampled rows, `decode.parity` the timed decode's outputs on
every row, and each `per_config` entry that workload's GPU outputs on every
row (max-abs errors against the tolerances 1.5e-2 for bf16 O, 1e-5 for fp32
O, 1e-3 for LSE).  `startup` gives the library load and each kernel's first
(cold) call.  The other objects are measured before the main steps, each with
its own warm-up, so that the main loop starts on a chip whose clock has
settled under load (that takes some 50 ms, more than a few warm-up steps):
`decode_graph` times the decode workload on its own, eager and replayed from a
HIP graph, and `decode_paged` times it against a paged cache (block table over
a shuffled pool), replayed from a HIP graph as well (calls issued one by one
from Python add the binding's host work and the per-dispatch cost);
`chunked_prefill` (a 2048-token chunk over 8192 cached tokens,
causal bottom-right) and `cross_attention` (2048 queries over 4096 keys,
non-causal) time attn_fwd on the two rectangular workloads the same way;
`backward` times attn_bwd (all three kernels) on the prefill workload with the
forward's o and lse and a seeded upstream gradient, counting 2.5x the forward
FLOPs (five matrix products per visible pair); `fp8_prefill` times
attn_fwd_fp8 on the prefill workload's shape with e4m3 inputs (scores on the
fp8 MFMA, P V on the bf16 MFMA; its peak is the 3.33 PFLOP/s that half the
FLOPs at 5.0 and half at 2.5 PFLOP/s allow); `other_configs` times attn_fwd
on the smaller prefill shapes (C1 fp32, C2a/C2b GPT-2-small-sized, C3a/C3a'/C3b)
once each, replayed from a HIP graph, for context: they are parity cases and
too small to fill the chip.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (published)
PEAK_SCLK_GHZ = 2.4         # the engine clock the published MFMA peaks assume
METRIC = "attn fwd TFLOP/s & % bf16 MFMA peak (prefill); KV-cache GB/s & % HBM (decode)"
N_REPLICAS = 4


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the GPU clock settles within about 50 ms of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target seconds of oracle work (the small calibration sample runs slower per row, "
                         "so the sample lands at about two thirds of this)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--only", choices=["prefill", "decode", "bwd", "fp8"], default=None,
                    help="run one kernel only (for profiling runs)")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache decode measurement")
    ap.add_argument("--no-graph", action="store_true", help="skip the decode-alone and graph-replay measurement")
    ap.add_argument("--paged-block-size", type=int, default=64)
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 prefill measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the smaller prefill configs")
    ap.add_argument("--no-rect", action="store_true",
                    help="skip the chunked-prefill and cross-attention measurements")
    return ap.parse_args()


def _stored(name, kernel, field):
    """A per-kernel figure from a committed counter summary
    (profiles/<name>.json), or None when it is absent or was taken on other
    kernel sources."""
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from exact_scaled_dot_sdpa_amd.build import source_digest

    e = t.get("kernels", {}).get(kernel)
    if e is None or e.get("source_digest") != source_digest(kernel):
        return None
    return e.get(field)


def stored_traffic(kernel):
    """Per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE run), or None."""
    return _stored("traffic", kernel, "bytes_per_launch")


def stored_clock(kernel):
    """The engine clock (GHz) the SQ counter run observed over the kernel
    (SQ_CYCLES per shader engine over the dispatch duration), or None."""
    return _stored("counters", kernel, "clock_ghz")


def paged_decode_line(E, A, I, dev, block_size, reps=4, steps=20, warmup=50):
    """The decode workload's shape in a paged cache (shuffled pool of
    block_size-row blocks), timed on its own after the main loop."""
    import torch

    wd = I.WORKLOADS["C5"]
    sl, q, kp, vp, bt = I.paged_decode_inputs(wd.B, wd.Hq, wd.Hkv, wd.d, block_size, wd.Lmax // block_size,
                                              wd.dtype, seed=wd.seed, lo=wd.lo, hi=wd.hi)
    pools = [(kp.to(dev), vp.to(dev)) for _ in range(reps)]
    q, sl_d, bt = q.to(dev), sl.to(dev), bt.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = torch.empty(E.attn_decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.Lmax, wd.d), dtype=torch.uint8,
                     device=dev)

    def call(i):
        k_p, v_p = pools[i % reps]
        E.attn_decode_paged(q, k_p, v_p, bt, sl_d, scale=wd.scale, o=o, lse=lse, workspace=ws)

    eager = timed_ms(call, steps, warmup)
    ms = graph_ms(call, reps)
    by = A.decode_bytes(sl.tolist(), wd.Hq, wd.Hkv, wd.d, wd.dtype)
    return {"value": round(by / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "frac_hbm": round(by / (ms * 1e-3) / 1e9 /
            PEAK_HBM_GBS, 4), "avg_launch_ms": round(ms, 5), "eager_ms": round(eager, 5), "block_size": block_size,
            "sum_seq_len": int(sl.sum()), "bytes_per_launch": by,
            "note": "same shape and lengths as the decode workload, rows in a shuffled pool of blocks; avg_launch_ms "
                    "from a HIP graph of one call per pool replica replayed back to back (eager_ms: the same calls "
                    "issued one by one from Python, with the binding's host work and the per-dispatch cost on top)"}


def graph_ms(call, n, replays=20):
    """Average duration of call(0) .. call(n-1) captured in one HIP graph and
    replayed `replays` times back to back: the kernels' own time, with no
    host work between launches."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        for i in range(n):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            call(i)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (replays * n)


def decode_graph_line(E, A, I, dev, qd, sl, caches, od, lsed, ws, steps=40, warmup=20, replays=20):
    """The decode step on its own: eager back-to-back calls, and the same
    calls replayed from a HIP graph that holds one call per cache replica
    (the form a serving loop runs them in)."""
    wd = I.WORKLOADS["C5"]

    def call(i):
        kc, vc = caches[i % len(caches)]
        E.attn_decode(qd, kc, vc, sl, scale=wd.scale, o=od, lse=lsed, workspace=ws)

    eager = timed_ms(call, steps, warmup)
    graph = graph_ms(call, len(caches), replays)
    by = A.decode_bytes(sl.cpu().tolist(), wd.Hq, wd.Hkv, wd.d, wd.dtype)
    return {"value": round(by / (graph * 1e-3) / 1e9, 1), "unit": "GB/s",
            "frac_hbm": round(by / (graph * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "graph_call_ms": round(graph, 5),
            "eager_alone_ms": round(eager, 5),
            "eager_alone_gbs": round(by / (eager * 1e-3) / 1e9, 1),
            "note": "the decode workload on its own (not after a prefill): eager back-to-back calls, and the same "
                    "calls replayed from a HIP graph of one call per cache replica"}


def timed_ms(call, steps, warmup):
    """Average duration of call() over `steps` launches, from HIP events on the
    current stream, after `warmup` untimed ones."""
    import torch

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        call(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) / steps


def rect_prefill_line(E, A, I, dev, name, steps=20, warmup=50):
    """attn_fwd on a rectangular workload (Nq != Nk), timed on its own."""
    import torch

    w = I.WORKLOADS[name]
    q, k, v = (t.to(dev) for t in I.workload_inputs(name))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ms = timed_ms(lambda i: E.attn_fwd(q, k, v, scale=w.scale, causal=w.causal, o=o, lse=lse), steps, warmup)
    fl = A.prefill_flops(w.B, w.Hq, w.Nq, w.Nkv, w.d, w.causal)
    tf = fl / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(ms, 5), "flops_per_launch": fl,
            "shape": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nkv, "d": w.d,
                      "causal": w.causal}, "note": w.note}


def backward_line(E, A, I, dev, q, k, v, o, lse, w, steps=20, warmup=50):
    """attn_bwd on the prefill workload, timed on its own."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 500)
    do = I.randn(tuple(q.shape), w.dtype, g).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(E.attn_bwd_workspace_bytes(w.B, w.Hq, w.Nq), dtype=torch.uint8, device=dev)
    ms = timed_ms(lambda i: E.attn_bwd(q, k, v, o, do, lse, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dv,
                                       workspace=ws), steps, warmup)
    fl = A.bwd_flops(w.B, w.Hq, w.Nq, w.Nkv, w.d, w.causal)
    tf = fl / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(ms, 5), "flops_per_launch": fl,
            "kernels": "bwd_pre_kernel<128> + bwd_dq_kernel<128,true,8,8> + bwd_dkdv_kernel<128,true>",
            "note": "algorithmic FLOPs = 2.5x the forward's (S, dP, dV, dK, dQ products); the kernels "
                    "recompute S and dP once more for dQ"}


def fp8_prefill_line(E, A, I, dev, steps=20, warmup=50):
    """attn_fwd_fp8 on the prefill workload's shape (e4m3 q, k, v), timed on its own."""
    import torch

    w = I.WORKLOADS["C4"]
    q, k, v = (t.to(dev) for t in I.prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, "fp8", w.seed))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ms = timed_ms(lambda i: E.attn_fwd_fp8(q, k, v, scale=w.scale, causal=w.causal, o=o, lse=lse), steps, warmup)
    fl = A.prefill_flops(w.B, w.Hq, w.Nq, w.Nkv, w.d, w.causal)
    tf = fl / (ms * 1e-3) / 1e12
    peak = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
    return {"value": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / peak, 4), "peak": round(peak, 1),
            "avg_launch_ms": round(ms, 5), "flops_per_launch": fl,
            "bytes_per_launch": A.prefill_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, "fp8"),
            "kernel": "prefill_fp8_kernel<128,true>",
            "note": "e4m3 q, k, v (seeded N(0,1) rounded to e4m3); scores on the fp8 MFMA, P V on the bf16 MFMA "
                    "with V widened exactly; bf16 output"}


# the smaller prefill workloads, timed one by one (and, in the oracle's leg, run in full)
OTHER_CONFIGS = ("C1", "C2a", "C2b", "C3a", "C3a'", "C3b")


def other_configs_line(E, A, I, dev, steps=20, warmup=20):
    """attn_fwd on the smaller prefill shapes, each timed on its own: 10 calls
    captured in a HIP graph and replayed, so that neither the binding's host
    work nor the per-dispatch cost is timed with these short kernels; calls
    issued one by one from Python are kept as eager_us."""
    import torch

    out, outputs = {}, {}
    for name in OTHER_CONFIGS:
        w = I.WORKLOADS[name]
        causal = w.causal
        q, k, v = (t.to(dev) for t in I.workload_inputs(name))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        def call(i, q=q, k=k, v=v, o=o, lse=lse, w=w, causal=causal):
            E.attn_fwd(q, k, v, scale=w.scale, causal=causal, o=o, lse=lse)

        eager = timed_ms(call, steps, warmup)
        ms = graph_ms(call, 10, replays=10)
        fl = A.prefill_flops(w.B, w.Hq, w.Nq, w.Nkv, w.d, causal)
        by = A.prefill_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, w.dtype)
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"shape": "%s B%d H%d N%d d%d %s" % (w.dtype, w.B, w.Hq, w.Nq, w.d,
                                                         "causal" if causal else "full"),
                     "us": round(ms * 1e3, 2), "eager_us": round(eager * 1e3, 2), "tflops": round(tf, 2),
                     "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4) if w.dtype == "bf16" else None,
                     "gbs": round(by / (ms * 1e-3) / 1e9, 1)}
        torch.cuda.synchronize()
        outputs[name] = (o.cpu(), lse.cpu())
    return out, outputs


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


TOL_O = {"f32": 1e-5, "bf16": 1.5e-2}
TOL_LSE = 1e-3


def _max_abs(a, b):
    """max |a - b| with equal infinities counting as equal (NaN if any NaN)."""
    import numpy as np

    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(a - b))
    return float(d.max()) if d.size else 0.0


def cpu_baseline(q, k, v, w, target_s, per_config=(), gpu_out=None, gpu_config_out=None):
    """The oracle, as it stands, on a bounded sample of prefill rows.  With
    gpu_out = (o, lse) of the timed prefill, the same rows are compared with
    the oracle's (`parity`); gpu_config_out[name] = (o, lse) of each smaller
    workload is compared with its full oracle run."""
    import numpy as np

    import oracle
    from exact_scaled_dot_sdpa_amd import inputs as I

    nthreads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    qd, kd, vd = I.to_f64(q), I.to_f64(k), I.to_f64(v)
    rng = np.random.default_rng(12345)

    def sample(n):
        b = np.zeros(n, dtype=np.int32)
        h = rng.integers(0, w.Hq, n).astype(np.int32)
        i = rng.integers(0, w.N, n).astype(np.int32)
        return np.stack([b, h, i], axis=1)

    def flops(rows):
        # 4*d per visible pair; row i of a causal square head sees i+1 keys
        return float(4 * w.d * (rows[:, 2].astype(np.int64) + 1).sum())

    rows = sample(max(64, nthreads * 4))
    t0 = time.perf_counter()
    oracle.attn_rows(qd, kd, vd, w.scale, w.causal, rows, nthreads=nthreads)
    dt = time.perf_counter() - t0
    rate = flops(rows) / max(dt, 1e-6)
    n = int(min(max(64, rows.shape[0] * max(target_s, 0.5) / max(dt, 1e-6)), w.Hq * w.N))
    rows = sample(n)
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attn_rows(qd, kd, vd, w.scale, w.causal, rows, nthreads=nthreads)
    dt = time.perf_counter() - t0
    f = flops(rows)
    res = {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": nthreads,
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": "%d random (head, row) pairs of the GQA causal prefill workload (%.3g GFLOP of the "
                  "%.4g GFLOP total), fp64, %.1f s; calibration rate %.3g GFLOP/s"
                  % (n, f / 1e9, 4.0 * w.d * w.Hq * w.N * (w.N + 1) / 2 / 1e9, dt, rate / 1e9),
        "seconds": dt,
    }
    if gpu_out is not None:
        o_gpu, lse_gpu = gpu_out
        sel = (rows[:, 0], rows[:, 1], rows[:, 2])
        eo = _max_abs(I.to_f64(o_gpu[sel]), o_ref)
        el = _max_abs(I.to_f64(lse_gpu[sel]), lse_ref)
        res["parity"] = {"rows": int(n), "max_abs_o": eo, "max_abs_lse": el, "tol_o": TOL_O[w.dtype],
                         "tol_lse": TOL_LSE, "within_tol": bool(eo <= TOL_O[w.dtype] and el <= TOL_LSE),
                         "note": "the timed prefill's o and lse on the oracle's sampled rows"}
    if per_config:
        # the smaller prefill configs in full, for the oracle's wall time next
        # to the GPU's (a few seconds together)
        from exact_scaled_dot_sdpa_amd import accounting as A
        per = {}
        for name in per_config:
            c = I.WORKLOADS[name]
            cq, ck, cv = [I.to_f64(t) for t in I.workload_inputs(name)]
            t0 = time.perf_counter()
            co, cl = oracle.attn(cq, ck, cv, c.scale, c.causal, nthreads=nthreads)
            cdt = time.perf_counter() - t0
            cf = A.prefill_flops(c.B, c.Hq, c.Nq, c.Nkv, c.d, c.causal)
            per[name] = {"seconds": round(cdt, 4), "gflop": round(cf / 1e9, 3), "gflops": round(cf / cdt / 1e9, 1)}
            if gpu_config_out and name in gpu_config_out:
                go, gl = gpu_config_out[name]
                eo, el = _max_abs(I.to_f64(go), co), _max_abs(I.to_f64(gl), cl)
                per[name].update({"max_abs_o": eo, "max_abs_lse": el,
                                  "within_tol": bool(eo <= TOL_O[c.dtype] and el <= TOL_LSE)})
        res["per_config"] = per
    return res


def decode_parity(sl, q, kc, vc, o, lse, w):
    """The timed decode's o and lse against the oracle on the whole workload."""
    import oracle
    from exact_scaled_dot_sdpa_amd import inputs as I

    o_ref, lse_ref = oracle.decode(I.to_f64(q), I.to_f64(kc), I.to_f64(vc), sl.numpy(), w.scale)
    eo, el = _max_abs(I.to_f64(o), o_ref), _max_abs(I.to_f64(lse), lse_ref)
    return {"rows": int(o_ref.shape[0] * o_ref.shape[1]), "max_abs_o": eo, "max_abs_lse": el,
            "tol_o": TOL_O[w.dtype], "tol_lse": TOL_LSE,
            "within_tol": bool(eo <= TOL_O[w.dtype] and el <= TOL_LSE),
            "note": "the timed decode's o and lse (last step) against the oracle, every row"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(asked for --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_scaled_dot_sdpa_amd as E
    from exact_scaled_dot_sdpa_amd import accounting as A
    from exact_scaled_dot_sdpa_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # one-time costs, reported apart from the timed steps: loading the library,
    # and (below) the first call of each kernel, which also loads its code
    t0 = time.perf_counter()
    E.lib()
    startup = {"lib_load_ms": round((time.perf_counter() - t0) * 1e3, 3)}

    wp = I.WORKLOADS["C4"]
    wd = I.WORKLOADS["C5"]
    run_p = args.only in (None, "prefill")
    run_d = args.only in (None, "decode")
    run_b = args.only in (None, "bwd") and not args.no_bwd
    run_8 = args.only in (None, "fp8") and not args.no_fp8

    # ---- inputs, resident in HBM before timing --------------------------
    q_cpu, k_cpu, v_cpu = I.workload_inputs("C4")
    q, k, v = q_cpu.to(dev), k_cpu.to(dev), v_cpu.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    sl_cpu, qd_cpu, kc_cpu, vc_cpu = I.workload_inputs("C5")
    qd, sl = qd_cpu.to(dev), sl_cpu.to(dev)
    caches = [(kc_cpu.to(dev), vc_cpu.to(dev)) for _ in range(N_REPLICAS)]
    od = torch.empty_like(qd)
    lsed = torch.empty(qd.shape[:2], dtype=torch.float32, device=dev)
    ws = torch.empty(E.attn_decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.Lmax, wd.d), dtype=torch.uint8,
                     device=dev)

    p_flops = A.prefill_flops(wp.B, wp.Hq, wp.N, wp.N, wp.d, wp.causal)
    p_bytes = A.prefill_bytes(wp.B, wp.Hq, wp.Hkv, wp.N, wp.N, wp.d, wp.dtype)
    d_bytes = A.decode_bytes(sl_cpu.tolist(), wd.Hq, wd.Hkv, wd.d, wd.dtype)
    d_flops = A.decode_flops(sl_cpu.tolist(), wd.Hq, wd.d)

    def prefill():
        E.attn_fwd(q, k, v, scale=wp.scale, causal=wp.causal, o=o, lse=lse)

    def decode(r):
        kc, vc = caches[r % N_REPLICAS]
        E.attn_decode(qd, kc, vc, sl, scale=wd.scale, o=od, lse=lsed, workspace=ws)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for name, fn, on in (("first_prefill_ms", prefill, run_p), ("first_decode_ms", lambda: decode(0), run_d)):
        if on:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            startup[name] = round((time.perf_counter() - t0) * 1e3, 3)

    # The measurements reported beside the main line run before the main
    # loop, each with its own warm-up and timing.  The main steps then start
    # on a chip that has been under load for a while: its engine clock takes
    # some 50 ms of load to settle, longer than a few warm-up steps last.
    side = {}
    if run_d and not args.no_graph:
        side["decode_graph"] = decode_graph_line(E, A, I, dev, qd, sl, caches, od, lsed, ws)
    if run_d and not args.no_paged:
        side["decode_paged"] = paged_decode_line(E, A, I, dev, args.paged_block_size)
    if run_b:
        prefill()  # o and lse for the backward pass
        torch.cuda.synchronize()
        side["backward"] = backward_line(E, A, I, dev, q, k, v, o, lse, wp)
    if run_8:
        side["fp8_prefill"] = fp8_prefill_line(E, A, I, dev)
    config_outputs = None
    if run_p and not args.no_configs:
        side["other_configs"], config_outputs = other_configs_line(E, A, I, dev)
    if run_p and not args.no_rect:
        side["chunked_prefill"] = rect_prefill_line(E, A, I, dev, "X1")
        side["cross_attention"] = rect_prefill_line(E, A, I, dev, "X2")

    for i in range(args.warmup):
        if run_p:
            prefill()
        if run_d:
            decode(i)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        if run_p:
            prefill()
        ev[i][1].record(stream)
        if run_d:
            decode(i)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    p_all = [e[0].elapsed_time(e[1]) for e in ev]
    d_all = [e[1].elapsed_time(e[2]) for e in ev]
    p_ms, d_ms = sum(p_all) / K, sum(d_all) / K
    p_med, d_med = statistics.median(p_all), statistics.median(d_all)
    ms_per_step = wall * 1e3 / K
    # the timed calls' outputs (every step writes the same values), for the
    # parity check against the oracle after the other measurements
    timed_prefill = (o.cpu(), lse.cpu()) if run_p else None
    timed_decode = (od.cpu(), lsed.cpu()) if run_d else None

    p_tflops = p_flops / (p_ms * 1e-3) / 1e12 if run_p else None
    d_gbs = d_bytes / (d_ms * 1e-3) / 1e9 if run_d else None

    out = {
        "metric": METRIC,
        "value": round(p_tflops, 2) if run_p else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) from seeded CPU generators, rounded to bf16",
        "config": {
            "workload": "GQA causal prefill B=1 Hq=64 Hkv=8 N=8192 d=128 bf16 + KV-cache decode B=16 "
                        "Hq=32 Hkv=8 d=128 bf16 L~U[512,4096]",
            "prefill": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "N": wp.N, "d": wp.d, "causal": wp.causal,
                        "seed": wp.seed, "flops_per_launch": p_flops, "bytes_per_launch": p_bytes},
            "decode": {"B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "Lmax": wd.Lmax, "d": wd.d, "seed": wd.seed,
                       "sum_seq_len": int(sl_cpu.sum()), "bytes_per_launch": d_bytes,
                       "flops_per_launch": d_flops, "cache_replicas": N_REPLICAS},
            "parallelism": "single GPU",
        },
    }
    if run_p:
        tr = stored_traffic("prefill")
        clk = stored_clock("prefill")
        out["roofline"] = {
            "bound": "mfma", "achieved": round(p_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4), "traffic": tr,
            "kernel": "prefill_bf16_kernel<128,true,8,8>", "avg_launch_ms": round(p_ms, 5),
            "median_launch_ms": round(p_med, 5),
            "median_tflops": round(p_flops / (p_med * 1e-3) / 1e12, 2),
            "sclk_ghz_counters": clk,
            # the same rate against the dense peak scaled to that observed clock
            "frac_at_sclk": round(p_tflops / (PEAK_BF16_TFLOPS * clk / PEAK_SCLK_GHZ), 4) if clk else None,
        }
    if run_d:
        tr = stored_traffic("decode")
        out["decode"] = {"value": round(d_gbs, 1), "unit": "GB/s", "frac_hbm": round(d_gbs / PEAK_HBM_GBS, 4),
                         "avg_launch_ms": round(d_ms, 5), "median_launch_ms": round(d_med, 5),
                         "median_gbs": round(d_bytes / (d_med * 1e-3) / 1e9, 1),
                         "tflops": round(d_flops / (d_ms * 1e-3) / 1e12, 2)}
        out["roofline_decode"] = {
            "bound": "hbm", "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(d_gbs / PEAK_HBM_GBS, 4), "traffic": tr,
            "kernel": "decode_chunk_kernel<__bf16,128,4,3> + decode_merge_kernel<__bf16,128>", "avg_launch_ms": round(d_ms, 5),
            "median_launch_ms": round(d_med, 5),
        }
    out["startup"] = dict(startup, note="library load and the first call of each kernel (code-object load "
                          "included), against the warm per-call times above; compilation happens at build time")
    out.update(side)
    if not args.no_cpu_baseline and run_d:
        out["decode"]["parity"] = decode_parity(sl_cpu, qd_cpu, kc_cpu, vc_cpu, *timed_decode, wd)
    if not args.no_cpu_baseline and run_p:
        out["cpu_baseline"] = cpu_baseline(q_cpu, k_cpu, v_cpu, wp, args.cpu_seconds,
                                           per_config=() if args.no_configs else OTHER_CONFIGS,
                                           gpu_out=timed_prefill, gpu_config_out=config_outputs)
        out["parity"] = dict(out["cpu_baseline"]["parity"], config="C4")
        for name, rec in out["cpu_baseline"].get("per_config", {}).items():
            if name in out.get("other_configs", {}):
                rec["gpu_us"] = out["other_configs"][name]["us"]
                rec["gpu_speedup"] = round(rec["seconds"] / (rec["gpu_us"] * 1e-6), 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
