"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with something independent of the oracle's own code: a
high-precision brute force of the definition, a library routine
(torch's CPU scaled_dot_product_attention and logsumexp in fp64), a closed
form, or an invariant the pages state.  ``tests/test_oracle_mutants.py`` runs
every pin against deliberately broken copies of the oracle to show that each
plausible mistake is caught by at least one pin.

Pages (cited by title and section):
  [R]  "Transformer 架构的数学与计算深度解析：注意力机制的详尽研究报告":
       sec. 2.4 (rows of weights sum to one; output is a convex combination of
       value rows), sec. 4.1 (causal: token t sees positions 1..t),
       sec. 6.3 (the online recurrence reaches exactly the standard result).
  [IO] "从注意力到 IO 感知执行": sec. 8 (subtracting the max leaves the
       probabilities unchanged; recurrence eqs. (1)-(2)).
  [N]  "Transformer 笔记：注意力机制为什么会变成系统问题": KV-cache section
       (a decode query reads the cached K/V of all earlier tokens).
  [E]  pwwt.cn engineering blog: sec. 2.3 (GQA: a group of query heads shares
       one K/V head), sec. 5.1 (attention is order-insensitive: shuffling the
       sequence only shuffles the output).
  [M]  "Transformer 深度进阶：从矩阵视角到 FlashAttention 工程优化": the
       FlashAttention section (the backward pass recomputes instead of storing
       the score matrix).
"""
from decimal import Decimal, getcontext

import numpy as np
import torch

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _randn(rng, *shape):
    return rng.standard_normal(shape)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(both_inf, 0.0, np.abs(a - b))
    err = float(np.nanmax(diff)) if diff.size else 0.0
    assert not np.isnan(diff).any(), "%s: NaN" % what
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


# ---------------------------------------------------------------------------
# 1. brute force in 50-digit decimal arithmetic, softmax written as
#    exp(s_j) / sum_k exp(s_k) with no max subtraction ([R] sec. 2.4).
# ---------------------------------------------------------------------------
def _decimal_attention(q, k, v, scale, causal):
    getcontext().prec = 50
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    sc = Decimal(repr(float(scale)))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i in range(Nq):
                es = []
                for j in range(Nk):
                    if causal and j > i:  # square case only: token i sees 0..i
                        continue
                    s = sum(Decimal(repr(float(q[b, h, i, c]))) * Decimal(repr(float(k[b, hk, j, c])))
                            for c in range(d)) * sc
                    es.append((j, s.exp()))
                z = sum(e for _, e in es)
                for c in range(d):
                    acc = sum(e * Decimal(repr(float(v[b, hk, j, c]))) for j, e in es)
                    o[b, h, i, c] = float(acc / z)
                lse[b, h, i] = float(z.ln())
    return o, lse


def pin_decimal_bruteforce(orc):
    rng = _rng(1)
    cases = [
        (2, 4, 2, 5, 7, 3, False),   # GQA, rectangular (cross-attention shape)
        (1, 2, 1, 6, 6, 4, True),    # GQA, causal square
        (1, 3, 3, 4, 2, 2, False),   # Nq > Nk, non-causal
        (1, 1, 1, 1, 1, 5, True),    # single token
    ]
    for (B, Hq, Hkv, Nq, Nk, d, causal) in cases:
        q = _randn(rng, B, Hq, Nq, d)
        k = _randn(rng, B, Hkv, Nk, d)
        v = _randn(rng, B, Hkv, Nk, d)
        scale = 1.0 / np.sqrt(d)
        o, lse = orc.attn(q, k, v, scale, causal)
        o_ref, lse_ref = _decimal_attention(q, k, v, scale, causal)
        _close(o, o_ref, TOL, "decimal brute force O %s" % ((B, Hq, Hkv, Nq, Nk, d, causal),))
        _close(lse, lse_ref, TOL, "decimal brute force LSE")


# ---------------------------------------------------------------------------
# 2. library special case: torch's CPU SDPA and logsumexp in fp64.
# ---------------------------------------------------------------------------
def _torch_ref(q, k, v, scale, causal):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, scale=scale, is_causal=causal, enable_gqa=(G > 1))
    kk = tk.repeat_interleave(G, dim=1)
    s = (tq @ kk.transpose(-1, -2)) * scale
    if causal:
        Nq, Nk = s.shape[-2], s.shape[-1]
        mask = torch.ones(Nq, Nk, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def pin_torch_sdpa(orc):
    rng = _rng(2)
    cases = [
        (1, 1, 1, 128, 128, 64, False),
        (1, 1, 1, 128, 128, 64, True),
        (2, 8, 2, 33, 33, 16, True),   # GQA, causal, square
        (2, 6, 3, 17, 40, 8, False),   # GQA, cross-attention (Nq != Nk)
    ]
    for (B, Hq, Hkv, Nq, Nk, d, causal) in cases:
        q = _randn(rng, B, Hq, Nq, d)
        k = _randn(rng, B, Hkv, Nk, d)
        v = _randn(rng, B, Hkv, Nk, d)
        scale = 1.0 / np.sqrt(d)
        o, lse = orc.attn(q, k, v, scale, causal)
        o_ref, lse_ref = _torch_ref(q, k, v, scale, causal)
        _close(o, o_ref, 1e-11, "torch SDPA O %s" % ((B, Hq, Hkv, Nq, Nk, d, causal),))
        _close(lse, lse_ref, 1e-11, "torch logsumexp LSE")


# ---------------------------------------------------------------------------
# 3. invariants and closed forms ([R] sec. 2.4, 4.1; [IO] sec. 8)
# ---------------------------------------------------------------------------
def pin_rows_sum_to_one(orc):
    rng = _rng(3)
    for causal in (False, True):
        q = _randn(rng, 1, 2, 24, 8)
        k = _randn(rng, 1, 2, 24, 8)
        v = _randn(rng, 1, 2, 24, 8)
        o, lse, w = orc.attn(q, k, v, 0.35, causal, weights=True)
        _close(w.sum(-1), np.ones(w.shape[:3]), TOL, "weight rows sum to 1")
        assert (w >= 0).all(), "negative weight"
        if causal:
            upper = np.triu(np.ones((24, 24), dtype=bool), 1)
            assert (w[..., upper] == 0).all(), "masked weight not exactly 0"
        _close(o, w @ v, TOL, "O = A V")


def pin_values_ones(orc):
    rng = _rng(4)
    for causal in (False, True):
        q = _randn(rng, 2, 4, 19, 16) * 3
        k = _randn(rng, 2, 2, 19, 16) * 3
        v = np.ones((2, 2, 19, 16))
        o, _ = orc.attn(q, k, v, 0.25, causal)
        _close(o, np.ones_like(o), 1e-14, "V = ones gives O = ones")


def _prefix_mean(v, causal, Nq):
    # mean of the visible value rows; square causal: rows 0..i
    if causal:
        cs = np.cumsum(v, axis=-2)
        cnt = np.arange(1, v.shape[-2] + 1)[:, None]
        return (cs / cnt)[..., :Nq, :]
    return np.broadcast_to(v.mean(axis=-2, keepdims=True), v.shape[:-2] + (Nq, v.shape[-1]))


def pin_identical_keys(orc):
    rng = _rng(5)
    N, d = 21, 8
    for causal in (False, True):
        q = _randn(rng, 1, 1, N, d)
        kap = _randn(rng, d)
        k = np.broadcast_to(kap, (1, 1, N, d)).copy()
        v = _randn(rng, 1, 1, N, d)
        scale = 0.4
        o, lse = orc.attn(q, k, v, scale, causal)
        _close(o, _prefix_mean(v, causal, N), 1e-13, "identical keys: O = mean of visible V")
        nvis = np.arange(1, N + 1) if causal else np.full(N, N)
        s = scale * (q[0, 0] @ kap)
        _close(lse[0, 0], s + np.log(nvis), 1e-12, "identical keys: lse = s + ln n")


def pin_zero_keys(orc):
    rng = _rng(6)
    N, d = 13, 4
    for causal in (False, True):
        q = _randn(rng, 1, 1, N, d)
        k = np.zeros((1, 1, N, d))
        v = _randn(rng, 1, 1, N, d)
        o, lse = orc.attn(q, k, v, 1.0, causal)
        nvis = np.arange(1, N + 1) if causal else np.full(N, N)
        assert np.array_equal(lse[0, 0], np.log(nvis.astype(np.float64))), "K = 0: lse = ln n exactly"
        _close(o, _prefix_mean(v, causal, N), 1e-14, "K = 0: O = mean of visible V")


def pin_causal_row0(orc):
    rng = _rng(7)
    q = _randn(rng, 2, 3, 9, 8)
    k = _randn(rng, 2, 3, 9, 8)
    v = _randn(rng, 2, 3, 9, 8)
    o, lse = orc.attn(q, k, v, 0.3, True)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :]), "causal row 0 must return v_0 exactly"
    _close(lse[:, :, 0], 0.3 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0]), 1e-14,
           "causal row 0: lse = s_00")


def pin_shift_invariance(orc):
    """K' = K + 1 w^T adds scale * q_i.w to every score of row i: O is
    unchanged and lse shifts by that amount ([IO] sec. 8).  Shifts reach
    +-1000, far beyond exp's fp64 range, so a softmax without the max
    subtraction overflows."""
    rng = _rng(8)
    B, H, N, d = 1, 2, 16, 8
    q = _randn(rng, B, H, N, d)
    k = _randn(rng, B, H, N, d)
    v = _randn(rng, B, H, N, d)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        o, lse = orc.attn(q, k, v, scale, causal)
        for mag in (3.0, 1000.0):
            w = _randn(rng, d)
            w = w / np.linalg.norm(w)
            # scale the shift so that max_i |scale * q_i . w| = mag
            qs = scale * (q[0] @ w)
            w = w * (mag / np.abs(qs).max())
            k2 = k + w
            o2, lse2 = orc.attn(q, k2, v, scale, causal)
            shift = scale * (q @ w)
            _close(o2, o, 1e-10 if mag < 100 else 1e-8, "shift invariance O (|c| <= %g)" % mag)
            _close(lse2, lse + shift, 1e-9 * max(1.0, mag), "shift: lse + c (|c| <= %g)" % mag)


def pin_permutation(orc):
    """[E] sec. 5.1: without a mask, permuting the sequence permutes the
    output; permuting K and V rows jointly changes nothing."""
    rng = _rng(9)
    q = _randn(rng, 1, 2, 11, 6)
    k = _randn(rng, 1, 2, 15, 6)
    v = _randn(rng, 1, 2, 15, 6)
    o, lse = orc.attn(q, k, v, 0.5, False)
    pk = rng.permutation(15)
    o2, lse2 = orc.attn(q, k[:, :, pk], v[:, :, pk], 0.5, False)
    _close(o2, o, 1e-13, "K/V permutation")
    _close(lse2, lse, 1e-13, "K/V permutation lse")
    pq = rng.permutation(11)
    o3, lse3 = orc.attn(q[:, :, pq], k, v, 0.5, False)
    _close(o3, o[:, :, pq], 0.0, "Q permutation")
    _close(lse3, lse[:, :, pq], 0.0, "Q permutation lse")


def pin_gqa_repeat(orc):
    """[E] sec. 2.3, contiguous grouping: GQA equals MHA with each K/V head
    repeated for the G query heads of its group."""
    rng = _rng(10)
    for (Hq, Hkv) in ((6, 3), (8, 2), (4, 1)):
        G = Hq // Hkv
        q = _randn(rng, 2, Hq, 10, 4)
        k = _randn(rng, 2, Hkv, 12, 4)
        v = _randn(rng, 2, Hkv, 12, 4)
        for causal in (False, True):
            o, lse = orc.attn(q, k, v, 0.5, causal)
            o2, lse2 = orc.attn(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.5, causal)
            _close(o, o2, 0.0, "GQA == repeated MHA")
            _close(lse, lse2, 0.0, "GQA == repeated MHA lse")


def pin_chunked_prefill_alignment(orc):
    """Causal with Nq < Nk: the Nq queries are the LAST Nq positions, so their
    rows equal the last Nq rows of square causal attention over all Nk
    positions ([R] sec. 4.1 defines the square case)."""
    rng = _rng(11)
    Nk, d = 23, 8
    qf = _randn(rng, 1, 2, Nk, d)
    k = _randn(rng, 1, 2, Nk, d)
    v = _randn(rng, 1, 2, Nk, d)
    of, lf = orc.attn(qf, k, v, 0.3, True)
    for Nq in (1, 5, 22, 23):
        o, lse = orc.attn(qf[:, :, Nk - Nq:], k, v, 0.3, True)
        _close(o, of[:, :, Nk - Nq:], 0.0, "chunked prefill == last rows of full causal (Nq=%d)" % Nq)
        _close(lse, lf[:, :, Nk - Nq:], 0.0, "chunked prefill lse")


def pin_decode_is_last_row(orc):
    """[N]: a decode query attends to every cached row; it equals the last row
    of causal attention over the sequence so far."""
    rng = _rng(12)
    B, Hq, Hkv, Lmax, d = 3, 4, 2, 20, 8
    kc = _randn(rng, B, Hkv, Lmax, d)
    vc = _randn(rng, B, Hkv, Lmax, d)
    q = _randn(rng, B, Hq, d)
    sl = np.array([20, 7, 1], dtype=np.int32)
    o, lse = orc.decode(q, kc, vc, sl, 0.35)
    for b in range(B):
        L = int(sl[b])
        qf = _randn(rng, 1, Hq, L, d)
        qf[0, :, L - 1] = q[b]
        of, lf = orc.attn(qf, kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], 0.35, True)
        _close(o[b], of[0, :, L - 1], 0.0, "decode == last causal row (b=%d)" % b)
        _close(lse[b], lf[0, :, L - 1], 0.0, "decode lse == last causal row")
    # padding rows are never read: poison them
    kp, vp = kc.copy(), vc.copy()
    for b in range(B):
        kp[b, :, sl[b]:] = np.nan
        vp[b, :, sl[b]:] = np.nan
    o2, lse2 = orc.decode(q, kp, vp, sl, 0.35)
    _close(o2, o, 0.0, "decode ignores rows beyond seq_len")
    # empty and over-long sequences
    o3, lse3 = orc.decode(q, kc, vc, np.array([0, 99, -5], dtype=np.int32), 0.35)
    assert (o3[0] == 0).all() and np.isneginf(lse3[0]).all(), "seq_len 0: O = 0, lse = -inf"
    assert (o3[2] == 0).all() and np.isneginf(lse3[2]).all(), "negative seq_len clamps to 0"
    o4, lse4 = orc.decode(q[1:2], kc[1:2], vc[1:2], np.array([Lmax], dtype=np.int32), 0.35)
    _close(o3[1], o4[0], 0.0, "seq_len above Lmax clamps to Lmax")


def pin_paged_decode(orc):
    """[N] (FlashAttention / PagedAttention section) and [E] sec. 3.3: a paged
    cache stores each sequence's K/V in fixed-size blocks anywhere in a pool,
    found through a block table.  Decode over the pages must equal decode
    over the same rows laid out contiguously, whatever the block order;
    sequences may share prefix blocks; unused blocks are never read; table
    entries and lengths are clamped as documented."""
    rng = _rng(13)
    B, Hq, Hkv, d, bs, nblk, maxb = 4, 6, 2, 8, 4, 24, 5
    kp = _randn(rng, nblk, Hkv, bs, d)
    vp = _randn(rng, nblk, Hkv, bs, d)
    q = _randn(rng, B, Hq, d)
    bt = rng.permutation(nblk)[:B * maxb].reshape(B, maxb).astype(np.int32)
    bt[1, :2] = bt[0, :2]  # sequence 1 shares its first two blocks with sequence 0
    sl = np.array([20, 9, 1, 0], dtype=np.int32)

    def contiguous(table):
        Lmax = maxb * bs
        kc = np.zeros((B, Hkv, Lmax, d))
        vc = np.zeros((B, Hkv, Lmax, d))
        for b in range(B):
            for j in range(Lmax):
                blk = min(max(int(table[b, j // bs]), 0), nblk - 1)
                kc[b, :, j] = kp[blk, :, j % bs]
                vc[b, :, j] = vp[blk, :, j % bs]
        return kc, vc

    o, lse = orc.decode_paged(q, kp, vp, bt, sl, 0.4)
    kc, vc = contiguous(bt)
    oc, lc = orc.decode(q, kc, vc, sl, 0.4)
    _close(o, oc, 0.0, "paged decode == contiguous decode")
    _close(lse, lc, 0.0, "paged decode lse == contiguous decode lse")
    # blocks no valid row lives in are never read
    used = {int(bt[b, j // bs]) for b in range(B) for j in range(int(sl[b]))}
    kpp, vpp = kp.copy(), vp.copy()
    for blk in range(nblk):
        if blk not in used:
            kpp[blk] = np.nan
            vpp[blk] = np.nan
    o2, l2 = orc.decode_paged(q, kpp, vpp, bt, sl, 0.4)
    _close(o2, o, 0.0, "paged decode ignores unused blocks")
    # a different physical placement of the same rows gives the same result
    perm = rng.permutation(nblk)
    inv = np.argsort(perm)
    o3, l3 = orc.decode_paged(q, kp[perm], vp[perm], inv[bt].astype(np.int32), sl, 0.4)
    _close(o3, o, 0.0, "paged decode independent of block placement")
    # clamping: lengths above max_blocks * bs, table entries out of range
    bt2 = bt.copy()
    bt2[0, 1] = -3
    bt2[2, 0] = nblk + 7
    sl2 = np.array([99, 9, 1, 0], dtype=np.int32)
    o4, l4 = orc.decode_paged(q, kp, vp, bt2, sl2, 0.4)
    kc4, vc4 = contiguous(bt2)
    oc4, lc4 = orc.decode(q, kc4, vc4, np.minimum(sl2, maxb * bs), 0.4)
    _close(o4, oc4, 0.0, "paged decode clamps lengths and table entries")
    _close(l4, lc4, 0.0, "paged decode clamps (lse)")


def pin_blockwise_equals_direct(orc):
    """[R] sec. 6.3 / [IO] eqs. (1)-(2): the blockwise recurrence reaches the
    direct result, for any block size, dividing or not."""
    rng = _rng(13)
    N = 37
    q = _randn(rng, 1, 2, N, 8) * 2
    k = _randn(rng, 1, 2, N, 8) * 2
    v = _randn(rng, 1, 2, N, 8)
    for causal in (False, True):
        o, lse = orc.attn(q, k, v, 0.5, causal)
        for beta in (1, 3, 16, 64, N):
            ob, lb = orc.blockwise(q, k, v, 0.5, causal, beta)
            _close(ob, o, TOL, "blockwise beta=%d causal=%s" % (beta, causal))
            _close(lb, lse, TOL, "blockwise lse beta=%d" % beta)


def pin_rows_entry_matches_full(orc):
    rng = _rng(14)
    q = _randn(rng, 2, 4, 30, 8)
    k = _randn(rng, 2, 2, 30, 8)
    v = _randn(rng, 2, 2, 30, 8)
    for causal in (False, True):
        o, lse = orc.attn(q, k, v, 0.3, causal)
        rows = np.array([[0, 0, 0], [1, 3, 29], [0, 2, 17], [1, 1, 5]], dtype=np.int32)
        orr, lr = orc.attn_rows(q, k, v, 0.3, causal, rows)
        _close(orr, o[rows[:, 0], rows[:, 1], rows[:, 2]], 0.0, "attn_rows == attn")
        _close(lr, lse[rows[:, 0], rows[:, 1], rows[:, 2]], 0.0, "attn_rows lse")


# ---------------------------------------------------------------------------
# 4. backward pass: gradients of the forward definition ([R] sec. 3.3 and
#    [M]'s FlashAttention section: training needs them; [IO], the evaluation
#    protocol: compare gradients with a higher-precision reference).
# ---------------------------------------------------------------------------
def _bottom_right_mask(Nq, Nk):
    """True where key j is hidden from query row i (j > i + Nk - Nq)."""
    i = torch.arange(Nq).unsqueeze(1)
    j = torch.arange(Nk).unsqueeze(0)
    return j > i + (Nk - Nq)


def pin_bwd_finite_differences(orc):
    """Central differences of the scalar L = sum(do * o(q, k, v)), with o from
    the oracle's forward (itself pinned above), against every element of
    dq, dk, dv.  Independent of the gradient formulas: a dropped term, a sign,
    a transposed operand, a missing scale or a GQA head summed wrongly each
    moves some element by far more than the O(h^2) difference error."""
    rng = _rng(20)
    cases = [
        (1, 2, 1, 5, 7, 3, True),    # GQA, chunked (bottom-right)
        (1, 2, 2, 6, 6, 4, False),
        (2, 3, 1, 4, 4, 2, True),    # MQA, square causal
        (1, 2, 1, 6, 3, 3, False),   # cross-attention, Nq > Nk
    ]
    h = 1e-5
    for (B, Hq, Hkv, Nq, Nk, d, causal) in cases:
        q = _randn(rng, B, Hq, Nq, d)
        k = _randn(rng, B, Hkv, Nk, d)
        v = _randn(rng, B, Hkv, Nk, d)
        do = _randn(rng, B, Hq, Nq, d)
        scale = 0.7
        dq, dk, dv = orc.attn_bwd(q, k, v, do, scale, causal)

        def loss(q_, k_, v_):
            return float(np.sum(do * orc.attn(q_, k_, v_, scale, causal)[0]))

        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                slot = {"dq": 0, "dk": 1, "dv": 2}[name]
                args_p[slot] = xp
                args_m[slot] = xm
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(g, fd, 1e-7, "%s vs finite differences %s" % (name, (B, Hq, Hkv, Nq, Nk, d, causal)))


def pin_bwd_torch_autograd(orc):
    """Library special case: torch autograd through the fp64 CPU
    scaled_dot_product_attention, with an explicit bottom-right mask and the
    K/V heads repeated for their query heads (autograd sums the repeats)."""
    rng = _rng(21)
    cases = [
        (2, 4, 2, 33, 47, 16, True),
        (2, 4, 2, 33, 47, 16, False),
        (1, 6, 1, 40, 40, 8, True),
        (1, 2, 2, 64, 128, 32, True),
    ]
    for (B, Hq, Hkv, Nq, Nk, d, causal) in cases:
        q = _randn(rng, B, Hq, Nq, d)
        k = _randn(rng, B, Hkv, Nk, d)
        v = _randn(rng, B, Hkv, Nk, d)
        do = _randn(rng, B, Hq, Nq, d)
        scale = 1.0 / np.sqrt(d)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        G = Hq // Hkv
        mask = ~_bottom_right_mask(Nq, Nk) if causal else None
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), attn_mask=mask, scale=scale)
        o.backward(torch.from_numpy(do))
        dq, dk, dv = orc.attn_bwd(q, k, v, do, scale, causal)
        tag = (B, Hq, Hkv, Nq, Nk, d, causal)
        _close(dq, tq.grad.numpy(), 1e-10, "dq vs torch autograd %s" % (tag,))
        _close(dk, tk.grad.numpy(), 1e-10, "dk vs torch autograd %s" % (tag,))
        _close(dv, tv.grad.numpy(), 1e-10, "dv vs torch autograd %s" % (tag,))


def pin_bwd_closed_forms(orc):
    """Facts of the definition that hold for any inputs:
      * each row of weights sums to one, so sum_j dv_j = sum of do_i over the
        group's rows that see some key, and the softmax Jacobian's rows sum to
        zero, so sum_j dk_j = 0 ([R] sec. 2.4);
      * with one key the weights are constant (= 1): dq = 0, dk = 0 and
        dv_0 = sum of every do_i of the group;
      * square causal row 0 sees only key 0 ([R] sec. 4.1): its dq is 0;
      * the gradients are linear in do, and do = 0 gives zeros."""
    rng = _rng(22)
    B, Hq, Hkv, d = 2, 6, 2, 5
    G = Hq // Hkv
    for (Nq, Nk, causal) in ((9, 9, True), (9, 9, False), (4, 11, True), (7, 3, False)):
        q = _randn(rng, B, Hq, Nq, d)
        k = _randn(rng, B, Hkv, Nk, d)
        v = _randn(rng, B, Hkv, Nk, d)
        do = _randn(rng, B, Hq, Nq, d)
        dq, dk, dv = orc.attn_bwd(q, k, v, do, 0.4, causal)
        do_g = do.reshape(B, Hkv, G, Nq, d).sum(axis=(2, 3))
        _close(dv.sum(axis=2), do_g, 1e-12, "sum_j dv_j = sum_i do_i")
        _close(dk.sum(axis=2), np.zeros((B, Hkv, d)), 1e-12, "sum_j dk_j = 0")
        if causal and Nq == Nk:
            _close(dq[:, :, 0], np.zeros((B, Hq, d)), 0.0, "causal row 0: dq = 0")
        dq2, dk2, dv2 = orc.attn_bwd(q, k, v, -2.5 * do, 0.4, causal)
        _close(dq2, -2.5 * dq, 1e-12, "dq linear in do")
        _close(dk2, -2.5 * dk, 1e-12, "dk linear in do")
        _close(dv2, -2.5 * dv, 1e-12, "dv linear in do")
        z = orc.attn_bwd(q, k, v, np.zeros_like(do), 0.4, causal)
        for t in z:
            _close(t, np.zeros_like(t), 0.0, "do = 0")
    q = _randn(rng, B, Hq, 5, d)
    k = _randn(rng, B, Hkv, 1, d)
    v = _randn(rng, B, Hkv, 1, d)
    do = _randn(rng, B, Hq, 5, d)
    dq, dk, dv = orc.attn_bwd(q, k, v, do, 0.4, False)
    _close(dq, np.zeros_like(dq), 0.0, "one key: dq = 0")
    _close(dk, np.zeros_like(dk), 1e-12, "one key: dk = 0")
    _close(dv[:, :, 0], do.reshape(B, Hkv, G, 5, d).sum(axis=(2, 3)), 1e-12, "one key: dv = sum do")


def pin_bwd_rows_match_full(orc):
    """The selected-rows entry (weights from the log-sum-exp) equals the full
    backward on the rows it names."""
    rng = _rng(23)
    B, Hq, Hkv, d = 2, 4, 2, 6
    for (Nq, Nk, causal) in ((20, 20, True), (13, 29, True), (17, 9, False)):
        q = _randn(rng, B, Hq, Nq, d)
        k = _randn(rng, B, Hkv, Nk, d)
        v = _randn(rng, B, Hkv, Nk, d)
        do = _randn(rng, B, Hq, Nq, d)
        dq, dk, dv = orc.attn_bwd(q, k, v, do, 0.5, causal)
        qr = np.array([[0, 0, 0], [1, 3, Nq - 1], [0, 2, Nq // 2], [1, 1, 3]], dtype=np.int32)
        kr = np.array([[0, 0, 0], [1, 1, Nk - 1], [0, 1, Nk // 2], [1, 0, 2]], dtype=np.int32)
        gq, gk, gv = orc.attn_bwd_rows(q, k, v, do, 0.5, causal, qr, kr)
        _close(gq, dq[qr[:, 0], qr[:, 1], qr[:, 2]], 1e-12, "bwd rows dq")
        _close(gk, dk[kr[:, 0], kr[:, 1], kr[:, 2]], 1e-12, "bwd rows dk")
        _close(gv, dv[kr[:, 0], kr[:, 1], kr[:, 2]], 1e-12, "bwd rows dv")


ALL_PINS = [
    pin_decimal_bruteforce,
    pin_torch_sdpa,
    pin_rows_sum_to_one,
    pin_values_ones,
    pin_identical_keys,
    pin_zero_keys,
    pin_causal_row0,
    pin_shift_invariance,
    pin_permutation,
    pin_gqa_repeat,
    pin_chunked_prefill_alignment,
    pin_decode_is_last_row,
    pin_paged_decode,
    pin_blockwise_equals_direct,
    pin_rows_entry_matches_full,
    pin_bwd_finite_differences,
    pin_bwd_torch_autograd,
    pin_bwd_closed_forms,
    pin_bwd_rows_match_full,
]
