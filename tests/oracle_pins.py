"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something other than itself: the worked example of page
"Attention Kernel" (section "Blockwise reference"), closed forms, invariants,
library routines on special cases, an independent blockwise recurrence, and
brute force with ``math.fsum`` on tiny inputs.  The same battery runs against
mutated copies of the oracle (tests/test_oracle_mutants.py) to show that a
plausible mistake in the oracle fails at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit, logsumexp, softmax

from oracle import blockwise
from synth import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _row_problem(scores, values):
    """Dense f32 problem whose single query row has exactly the given scores.

    q = e_0 and k_j = scores_j * e_0 (scale 1), so q.k_j = scores_j; entries
    equal to -inf are produced by k_keep = 0 instead.
    """
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n, d = values.shape
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, n, d), np.float32)
    fin = np.isfinite(scores)
    k[0, 0, fin, 0] = scores[fin]
    keep = fin.astype(np.uint8).reshape(1, n)
    v = _f32(values).reshape(1, 1, n, d)
    return q, k, v, keep


# --- the page's worked example --------------------------------------------------

def pin_worked_example(orc):
    fx = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    scores = np.array([float(s) for s in fx["scores"]])
    values = np.arange(15, dtype=np.float64).reshape(fx["values_rows"], fx["values_cols"])
    q, k, v, keep = _row_problem(scores, values)
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=1.0, k_keep=keep)
    want = softmax(scores) @ values
    assert np.allclose(o[0, 0, 0], want, rtol=0, atol=1e-12), (o[0, 0, 0], want)
    assert abs(lse[0, 0, 0] - logsumexp(scores)) < 1e-12
    # sum(P) = 1 and value columns differ by exactly 1, so consecutive outputs do too
    assert abs((o[0, 0, 0, 1] - o[0, 0, 0, 0]) - 1.0) < 1e-12
    assert abs((o[0, 0, 0, 2] - o[0, 0, 0, 1]) - 1.0) < 1e-12
    # the page's blockwise procedure with block size 2 agrees
    ob, lb = blockwise.online_attention_row(scores, values, block_size=fx["block_size"])
    assert np.allclose(ob, want, rtol=0, atol=1e-12) and abs(lb - lse[0, 0, 0]) < 1e-12


def pin_all_masked_row(orc):
    values = np.arange(15, dtype=np.float64).reshape(5, 3)
    q, k, v, keep = _row_problem(np.full(5, -np.inf), values)
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=1.0, k_keep=keep)
    assert np.array_equal(o[0, 0, 0], np.zeros(3)) and not np.isnan(o).any()
    assert lse[0, 0, 0] == -np.inf
    ob, lb = blockwise.online_attention_row(np.full(5, -np.inf), values, block_size=2)
    assert np.array_equal(ob, np.zeros(3)) and lb == -np.inf
    # S_k = 0: every row is fully masked
    o0, l0 = orc.attn_fwd(np.ones((1, 2, 3, 4), np.float32), np.ones((1, 1, 0, 4), np.float32),
                          np.ones((1, 1, 0, 4), np.float32), dtype="f32", scale=0.5)
    assert np.array_equal(o0, np.zeros_like(o0)) and np.all(l0 == -np.inf)


def pin_shape_rejection(orc):
    values = np.zeros((6, 3))
    for bad in (
        lambda: orc.attn_fwd(np.zeros((1, 1, 1, 3), np.float32), np.zeros((1, 1, 5, 3), np.float32),
                             _f32(values).reshape(1, 1, 6, 3), dtype="f32", scale=1.0),
        lambda: blockwise.online_attention_row(np.zeros(5), values, block_size=2),
        lambda: orc.attn_fwd(np.zeros((1, 3, 1, 3), np.float32), np.zeros((1, 2, 5, 3), np.float32),
                             np.zeros((1, 2, 5, 3), np.float32), dtype="f32", scale=1.0),
    ):
        try:
            bad()
        except ValueError:
            continue
        raise AssertionError("misaligned inputs must be rejected")


# --- closed forms -----------------------------------------------------------------

def pin_single_key(orc):
    rng = np.random.default_rng(11)
    q = _f32(rng.standard_normal((2, 3, 4, 16)))
    k = _f32(rng.standard_normal((2, 3, 1, 16)))
    v = _f32(rng.standard_normal((2, 3, 1, 16)))
    scale = 0.3125
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=scale)
    for b in range(2):
        for h in range(3):
            for i in range(4):
                assert np.array_equal(o[b, h, i], v[b, h, 0].astype(np.float64))
                s = scale * math.fsum(float(a) * float(c) for a, c in zip(q[b, h, i], k[b, h, 0]))
                assert abs(lse[b, h, i] - s) < 1e-12


def pin_causal_first_row(orc):
    """Causal row 0 sees key 0 only, so O = v_0 exactly, for every head (GQA)."""
    p = gen.make_dense(2, 4, 2, 9, 9, 8, dtype="bf16", causal=True, seed=5)
    o, lse = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True)
    vf = gen.as_f32(p.v, "bf16")
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, h, 0], vf[b, h // 2, 0].astype(np.float64))


def pin_two_keys(orc):
    rng = np.random.default_rng(12)
    q = _f32(rng.standard_normal((1, 1, 5, 8)))
    k = _f32(rng.standard_normal((1, 1, 2, 8)))
    v = _f32(rng.standard_normal((1, 1, 2, 8)))
    scale = 0.6875
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=scale)
    for i in range(5):
        s1 = scale * math.fsum(float(a) * float(c) for a, c in zip(q[0, 0, i], k[0, 0, 0]))
        s2 = scale * math.fsum(float(a) * float(c) for a, c in zip(q[0, 0, i], k[0, 0, 1]))
        want = expit(s1 - s2) * v[0, 0, 0].astype(np.float64) + expit(s2 - s1) * v[0, 0, 1].astype(np.float64)
        assert np.allclose(o[0, 0, i], want, rtol=0, atol=1e-12)
        assert abs(lse[0, 0, i] - np.logaddexp(s1, s2)) < 1e-12


def pin_uniform_scores(orc):
    """q = 0 makes every score 0: O = mean of the visible values, LSE = ln n."""
    rng = np.random.default_rng(13)
    n, d = 37, 16
    q = np.zeros((1, 2, 3, d), np.float32)
    k = _f32(rng.standard_normal((1, 2, n, d)))
    v = _f32(rng.standard_normal((1, 2, n, d)))
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=1.0)
    for h in range(2):
        for i in range(3):
            assert np.allclose(o[0, h, i], v[0, h].astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)
            assert abs(lse[0, h, i] - math.log(n)) < 1e-12


def pin_rows_are_distributions(orc):
    """With V = identity (S_k = d), O is the probability row itself."""
    rng = np.random.default_rng(14)
    n = 24
    q = _f32(rng.standard_normal((1, 1, 6, n)) * 2)
    k = _f32(rng.standard_normal((1, 1, n, n)))
    v = np.eye(n, dtype=np.float32).reshape(1, 1, n, n)
    keep = np.ones((1, n), np.uint8)
    keep[0, [3, 7, 20]] = 0
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.25, k_keep=keep)
    s = 0.25 * (q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T)
    s[:, keep[0] == 0] = -np.inf
    for i in range(6):
        assert abs(math.fsum(o[0, 0, i]) - 1.0) < 1e-12 and np.all(o[0, 0, i] >= 0)
        assert np.allclose(o[0, 0, i], softmax(s[i]), rtol=0, atol=1e-12)
        assert np.all(o[0, 0, i, keep[0] == 0] == 0)
        assert abs(lse[0, 0, i] - logsumexp(s[i])) < 1e-12


# --- invariants -----------------------------------------------------------------------

def pin_masked_keys_inert(orc):
    p = gen.make_dense(1, 2, 2, 10, 30, 8, dtype="f32", causal=True, seed=15, k_masked=9)
    o1, l1 = orc.attn_fwd(p.q, p.k, p.v, dtype="f32", scale=p.scale, causal=True, k_keep=p.k_keep)
    k2, v2 = p.k.copy(), p.v.copy()
    dead = p.k_keep[0] == 0
    k2[:, :, dead] = 1e30
    v2[:, :, dead] = -7e29
    o2, l2 = orc.attn_fwd(p.q, k2, v2, dtype="f32", scale=p.scale, causal=True, k_keep=p.k_keep)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_shift_invariance(orc):
    """Adding c to every score leaves O unchanged and shifts LSE by c (|c| up to 1e4)."""
    rng = np.random.default_rng(16)
    n = 19
    x = rng.standard_normal(4)
    y = rng.standard_normal(n)
    v = _f32(rng.standard_normal((1, 1, n, 2)))
    base = None
    for c in (0.0, 1e4, -1e4, 37.5):
        q = np.zeros((1, 1, 4, 2), np.float32)
        q[0, 0, :, 0] = x
        q[0, 0, :, 1] = 1.0
        k = np.zeros((1, 1, n, 2), np.float32)
        k[0, 0, :, 0] = y
        k[0, 0, :, 1] = c
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=1.0)
        if base is None:
            base = (o, lse)
            continue
        assert np.allclose(o, base[0], rtol=0, atol=1e-10)
        assert np.allclose(lse - base[1], c, rtol=0, atol=1e-9)


def pin_gqa_equals_repeated_heads(orc):
    p = gen.make_dense(2, 8, 2, 7, 11, 16, dtype="bf16", causal=True, seed=17)
    o, lse = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True)
    kr = np.repeat(p.k, 4, axis=1)
    vr = np.repeat(p.v, 4, axis=1)
    o2, l2 = orc.attn_fwd(p.q, kr, vr, dtype="bf16", scale=p.scale, causal=True)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def pin_varlen_equals_separate(orc):
    lens = [5, 0, 13, 1, 8]
    p = gen.make_varlen(lens, 4, 2, 8, dtype="bf16", causal=True, seed=18, q_mask_frac=0.1, k_mask_frac=0.1)
    o, lse = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=True,
                                 q_keep=p.q_keep, k_keep=p.k_keep)
    for s, n in enumerate(lens):
        a, b = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
        if n == 0:
            continue
        qs = p.q[:, a:b][None]
        ks = p.k[:, a:b][None]
        vs = p.v[:, a:b][None]
        o1, l1 = orc.attn_fwd(qs, ks, vs, dtype="bf16", scale=p.scale, causal=True,
                              q_keep=p.q_keep[a:b][None], k_keep=p.k_keep[a:b][None])
        assert np.array_equal(o[:, a:b], o1[0]) and np.array_equal(lse[:, a:b], l1[0])


def pin_decode_is_last_causal_row(orc):
    n, d = 23, 16
    p = gen.make_dense(1, 4, 2, n, n, d, dtype="bf16", causal=True, seed=19)
    o, lse = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True)
    # S_q = 1 < S_k: bottom-right alignment lets the single query see every key
    o1, l1 = orc.attn_fwd(p.q[:, :, n - 1:], p.k, p.v, dtype="bf16", scale=p.scale, causal=True)
    assert np.array_equal(o1[:, :, 0], o[:, :, n - 1]) and np.array_equal(l1[:, :, 0], lse[:, :, n - 1])
    # the same through a paged cache (page size 4, identity page order)
    ps = 4
    npg = (n + ps - 1) // ps
    kc = np.zeros((npg, ps, 2, d), np.uint16)
    vc = np.zeros((npg, ps, 2, d), np.uint16)
    for t in range(n):
        kc[t // ps, t % ps] = p.k[0, :, t]
        vc[t // ps, t % ps] = p.v[0, :, t]
    bt = np.arange(npg, dtype=np.int32)[None]
    o2, l2 = orc.decode_paged(p.q[:, :, n - 1], kc, vc, bt, np.array([n], np.int32), dtype="bf16",
                              scale=p.scale)
    assert np.array_equal(o2[0], o[0, :, n - 1]) and np.array_equal(l2[0], lse[0, :, n - 1])


def pin_paged_equals_contiguous(orc):
    lens = [1, 16, 17, 40, 0, 33]
    p = gen.make_paged(lens, 8, 2, 16, 16, dtype="bf16", seed=20, extra_pages=3)
    o, lse = orc.decode_paged(p.q, p.k_cache, p.v_cache, p.block_table, p.seq_lens, dtype="bf16",
                              scale=p.scale)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(o[b], np.zeros_like(o[b])) and np.all(lse[b] == -np.inf)
            continue
        t = np.arange(n)
        pages = p.block_table[b, t // 16]
        kc = p.k_cache[pages, t % 16].transpose(1, 0, 2)[None]  # [1, A_kv, n, d]
        vc = p.v_cache[pages, t % 16].transpose(1, 0, 2)[None]
        o1, l1 = orc.attn_fwd(p.q[b][None, :, None], np.ascontiguousarray(kc), np.ascontiguousarray(vc),
                              dtype="bf16", scale=p.scale)
        assert np.array_equal(o1[0, :, 0], o[b]) and np.array_equal(l1[0, :, 0], lse[b])
    # cache rows no sequence owns (page tails past seq_len, spare pages) are never read
    kc, vc = p.k_cache.copy(), p.v_cache.copy()
    owned = np.zeros(p.k_cache.shape[:2], bool)
    for b, n in enumerate(lens):
        for t in range(n):
            owned[p.block_table[b, t // 16], t % 16] = True
    kc[~owned] = 0x7FC0  # bf16 NaN
    vc[~owned] = 0x7FC0
    o3, l3 = orc.decode_paged(p.q, kc, vc, p.block_table, p.seq_lens, dtype="bf16", scale=p.scale)
    assert np.array_equal(o3, o) and np.array_equal(l3, lse)


def pin_causal_offset(orc):
    """Bottom-right alignment: S_q > S_k masks the leading S_q - S_k rows entirely;
    S_q < S_k lets row i see keys 0 .. i + S_k - S_q."""
    p = gen.make_dense(1, 1, 1, 9, 5, 8, dtype="f32", causal=True, seed=21)
    o, lse = orc.attn_fwd(p.q, p.k, p.v, dtype="f32", scale=p.scale, causal=True)
    assert np.array_equal(o[0, 0, :4], np.zeros((4, 8))) and np.all(lse[0, 0, :4] == -np.inf)
    assert np.all(np.isfinite(lse[0, 0, 4:]))
    p = gen.make_dense(1, 1, 1, 4, 10, 8, dtype="f32", causal=True, seed=22)
    o, lse = orc.attn_fwd(p.q, p.k, p.v, dtype="f32", scale=p.scale, causal=True)
    for i in range(4):
        n = i + 10 - 4 + 1
        o1, l1 = orc.attn_fwd(p.q[:, :, i:i + 1], p.k[:, :, :n], p.v[:, :, :n], dtype="f32", scale=p.scale)
        assert np.array_equal(o1[0, 0, 0], o[0, 0, i]) and l1[0, 0, 0] == lse[0, 0, i]


def pin_bf16_widening(orc):
    """bf16 bits are widened exactly: same result as feeding the widened fp32 values."""
    p = gen.make_dense(1, 2, 1, 6, 9, 8, dtype="bf16", causal=False, seed=23)
    o, lse = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale)
    o2, l2 = orc.attn_fwd(gen.as_f32(p.q, "bf16"), gen.as_f32(p.k, "bf16"), gen.as_f32(p.v, "bf16"),
                          dtype="f32", scale=p.scale)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # and the widening is the textbook one: 1.0 = 0x3f80, -2.0 = 0xc000, 0.5 = 0x3f00
    q = np.array([0x3F80, 0, 0, 0], np.uint16).reshape(1, 1, 1, 4)
    k = np.array([[0xC000, 0, 0, 0], [0x3F00, 0, 0, 0]], np.uint16).reshape(1, 1, 2, 4)
    v = np.array([[0x3F80, 0, 0, 0], [0, 0x3F80, 0, 0]], np.uint16).reshape(1, 1, 2, 4)
    o3, l3 = orc.attn_fwd(q, k, v, dtype="bf16", scale=1.0)
    assert abs(l3[0, 0, 0] - np.logaddexp(-2.0, 0.5)) < 1e-12
    assert abs(o3[0, 0, 0, 0] - expit(-2.5)) < 1e-12


# --- independent recurrence and brute force ---------------------------------------

def pin_blockwise_recurrence(orc):
    rng = np.random.default_rng(24)
    for trial in range(4):
        S_q, S_k, d = 6, int(rng.integers(1, 60)), 8
        causal = bool(trial % 2)
        p = gen.make_dense(1, 2, 1, S_q, S_k, d, dtype="bf16", causal=causal, seed=100 + trial, k_masked=S_k // 5)
        o, lse = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=causal, k_keep=p.k_keep)
        qf, kf, vf = (gen.as_f32(x, "bf16").astype(np.float64) for x in (p.q, p.k, p.v))
        for h in range(2):
            s = blockwise.dense_scores(qf[0, h], kf[0, 0], p.scale)
            s[:, p.k_keep[0] == 0] = -np.inf
            if causal:
                for i in range(S_q):
                    s[i, np.arange(S_k) > i + S_k - S_q] = -np.inf
            for i in range(S_q):
                cuts = sorted(set([0, S_k] + list(rng.integers(0, S_k + 1, size=int(rng.integers(0, 6))))))
                order = list(rng.permutation(len(cuts) - 1))
                ob, lb = blockwise.online_attention_row(s[i], vf[0, 0], bounds=cuts, order=order)
                assert np.allclose(ob, o[0, h, i], rtol=1e-12, atol=1e-12)
                assert (lb == -np.inf and lse[0, h, i] == -np.inf) or abs(lb - lse[0, h, i]) < 1e-12


def _brute(q, k, v, scale, vis):
    """Pure-Python softmax attention for one row with math.fsum."""
    s = [scale * math.fsum(a * b for a, b in zip(q, kj)) if ok else -math.inf for kj, ok in zip(k, vis)]
    m = max(s) if s else -math.inf
    if m == -math.inf:
        return [0.0] * len(q), -math.inf
    w = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
    lsum = math.fsum(w)
    out = [math.fsum(wj * vj[e] for wj, vj in zip(w, v)) / lsum for e in range(len(v[0]) if v else len(q))]
    return out, m + math.log(lsum)


def pin_brute_force(orc):
    rng = np.random.default_rng(25)
    for S_q, S_k, d, A, A_kv, causal in [(3, 5, 4, 2, 1, True), (5, 3, 2, 4, 2, True), (4, 4, 3, 3, 3, False),
                                         (1, 8, 4, 2, 2, True), (6, 7, 1, 2, 1, False)]:
        q = _f32(rng.standard_normal((2, A, S_q, d)))
        k = _f32(rng.standard_normal((2, A_kv, S_k, d)))
        v = _f32(rng.standard_normal((2, A_kv, S_k, d)))
        qk = (rng.random((2, S_q)) > 0.2).astype(np.uint8)
        kk = (rng.random((2, S_k)) > 0.2).astype(np.uint8)
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.875, causal=causal, q_keep=qk, k_keep=kk)
        G = A // A_kv
        for b in range(2):
            for h in range(A):
                for i in range(S_q):
                    vis = [bool(qk[b, i]) and bool(kk[b, j]) and (not causal or j <= i + S_k - S_q)
                           for j in range(S_k)]
                    want, wl = _brute([float(x) for x in q[b, h, i]],
                                      [[float(x) for x in row] for row in k[b, h // G]],
                                      [[float(x) for x in row] for row in v[b, h // G]], 0.875, vis)
                    assert np.allclose(o[b, h, i], want, rtol=0, atol=1e-13), (S_q, S_k, b, h, i)
                    assert (wl == -math.inf and lse[b, h, i] == -np.inf) or abs(lse[b, h, i] - wl) < 1e-13


def pin_varlen_brute_force(orc):
    rng = np.random.default_rng(26)
    lens = [3, 0, 5, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, A, A_kv, d = int(cu[-1]), 2, 1, 3
    q = _f32(rng.standard_normal((A, T, d)))
    k = _f32(rng.standard_normal((A_kv, T, d)))
    v = _f32(rng.standard_normal((A_kv, T, d)))
    kk = (rng.random(T) > 0.25).astype(np.uint8)
    o, lse = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=1.125, causal=True, k_keep=kk)
    for h in range(A):
        for t in range(T):
            s = int(np.searchsorted(cu, t, side="right") - 1)
            a = int(cu[s])
            vis = [bool(kk[j]) and cu[s] <= j < cu[s + 1] and j <= t for j in range(T)]
            want, wl = _brute([float(x) for x in q[h, t]], [[float(x) for x in r] for r in k[0]],
                              [[float(x) for x in r] for r in v[0]], 1.125, vis)
            assert np.allclose(o[h, t], want, rtol=0, atol=1e-13), (h, t, a)
            assert (wl == -math.inf and lse[h, t] == -np.inf) or abs(lse[h, t] - wl) < 1e-13


def pin_paged_brute_force(orc):
    rng = np.random.default_rng(27)
    lens = [5, 0, 9]
    p = gen.make_paged(lens, 4, 2, 3, 4, dtype="f32", seed=28, extra_pages=2)
    o, lse = orc.decode_paged(p.q, p.k_cache, p.v_cache, p.block_table, p.seq_lens, dtype="f32", scale=p.scale)
    for b, n in enumerate(lens):
        for h in range(4):
            ks = [[float(x) for x in p.k_cache[p.block_table[b, t // 4], t % 4, h // 2]] for t in range(n)]
            vs = [[float(x) for x in p.v_cache[p.block_table[b, t // 4], t % 4, h // 2]] for t in range(n)]
            want, wl = _brute([float(x) for x in p.q[b, h]], ks, vs, p.scale, [True] * n)
            if n == 0:
                want = [0.0] * 3
            assert np.allclose(o[b, h], want, rtol=0, atol=1e-13)
            assert (wl == -math.inf and lse[b, h] == -np.inf) or abs(lse[b, h] - wl) < 1e-13
    del rng


# ---- dense keep matrix and sliding windows (page "Attention Kernel", section
# "可编程 mask": element rules given to the oracle as a keep matrix)

def pin_dense_keep_brute_force(orc):
    rng = np.random.default_rng(41)
    for S_q, S_k, d, A, A_kv, causal in [(4, 6, 3, 2, 1, True), (5, 5, 2, 2, 2, False), (6, 4, 2, 2, 1, True)]:
        q = _f32(rng.standard_normal((2, A, S_q, d)))
        k = _f32(rng.standard_normal((2, A_kv, S_k, d)))
        v = _f32(rng.standard_normal((2, A_kv, S_k, d)))
        kk = (rng.random((2, S_k)) > 0.2).astype(np.uint8)
        mk = (rng.random((2, S_q, S_k)) > 0.35).astype(np.uint8)
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.75, causal=causal, k_keep=kk, m_keep=mk)
        G = A // A_kv
        for b in range(2):
            for h in range(A):
                for i in range(S_q):
                    vis = [bool(kk[b, j]) and bool(mk[b, i, j]) and (not causal or j <= i + S_k - S_q)
                           for j in range(S_k)]
                    want, wl = _brute([float(x) for x in q[b, h, i]],
                                      [[float(x) for x in row] for row in k[b, h // G]],
                                      [[float(x) for x in row] for row in v[b, h // G]], 0.75, vis)
                    assert np.allclose(o[b, h, i], want, rtol=0, atol=1e-13), (S_q, S_k, b, h, i)
                    assert (wl == -math.inf and lse[b, h, i] == -np.inf) or abs(lse[b, h, i] - wl) < 1e-13


def pin_dense_keep_matches_flag_masks(orc):
    """The causal pattern, and the outer product of q_keep and k_keep, given as
    a keep matrix reproduce the flags bit for bit."""
    rng = np.random.default_rng(42)
    B, A, A_kv, S_q, S_k, d = 2, 2, 1, 5, 7, 3
    q = _f32(rng.standard_normal((B, A, S_q, d)))
    k = _f32(rng.standard_normal((B, A_kv, S_k, d)))
    v = _f32(rng.standard_normal((B, A_kv, S_k, d)))
    o1, l1 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, causal=True)
    causal_pattern = np.tril(np.ones((S_q, S_k), np.uint8), S_k - S_q)
    o2, l2 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, m_keep=np.broadcast_to(causal_pattern, (B, S_q, S_k)))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    qk = (rng.random((B, S_q)) > 0.3).astype(np.uint8)
    kk = (rng.random((B, S_k)) > 0.3).astype(np.uint8)
    o3, l3 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, q_keep=qk, k_keep=kk)
    o4, l4 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, m_keep=qk[:, :, None] * kk[:, None, :])
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


# ---- general dense M (page "Attention Kernel", section "可编程 mask"; the
# definition P = softmax(Q K^T / sqrt(d_h) + M) of section "问题与成本"): an
# additive fp32 term per (row, key), finite or -inf

def _brute_bias(q, k, v, scale, bias_row, vis):
    """Pure-Python softmax attention for one row with an additive term."""
    s = [scale * math.fsum(a * b for a, b in zip(q, kj)) + mj if ok else -math.inf
         for kj, mj, ok in zip(k, bias_row, vis)]
    m = max(s) if s else -math.inf
    if m == -math.inf:
        return [0.0] * len(q), -math.inf
    w = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
    lsum = math.fsum(w)
    out = [math.fsum(wj * vj[e] for wj, vj in zip(w, v)) / lsum for e in range(len(v[0]))]
    return out, m + math.log(lsum)


def pin_bias_brute_force(orc):
    rng = np.random.default_rng(61)
    for S_q, S_k, d, A, A_kv, causal, heads in [(4, 6, 3, 2, 1, True, 1), (5, 5, 2, 2, 2, False, 2),
                                                (3, 7, 2, 4, 2, True, 4)]:
        q = _f32(rng.standard_normal((2, A, S_q, d)))
        k = _f32(rng.standard_normal((2, A_kv, S_k, d)))
        v = _f32(rng.standard_normal((2, A_kv, S_k, d)))
        bias = _f32(3.0 * rng.standard_normal((2, heads, S_q, S_k)))
        bias[rng.random(bias.shape) < 0.25] = -np.inf
        bias[1, 0, 0, :] = -np.inf  # a row with every key masked by the term alone
        kk = (rng.random((2, S_k)) > 0.2).astype(np.uint8)
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.625, causal=causal, k_keep=kk, bias=bias)
        G = A // A_kv
        for b in range(2):
            for h in range(A):
                for i in range(S_q):
                    vis = [bool(kk[b, j]) and (not causal or j <= i + S_k - S_q) for j in range(S_k)]
                    row = [float(x) for x in bias[b, h if heads > 1 else 0, i]]
                    want, wl = _brute_bias([float(x) for x in q[b, h, i]],
                                           [[float(x) for x in r] for r in k[b, h // G]],
                                           [[float(x) for x in r] for r in v[b, h // G]], 0.625, row, vis)
                    assert np.allclose(o[b, h, i], want, rtol=0, atol=1e-13), (S_q, S_k, b, h, i)
                    assert (wl == -math.inf and lse[b, h, i] == -np.inf) or abs(lse[b, h, i] - wl) < 1e-13


def pin_bias_zero_and_keep(orc):
    """M = 0 is no mask, and M in {0, -inf} is the keep matrix of the same
    pattern, bit for bit."""
    rng = np.random.default_rng(62)
    B, A, A_kv, S_q, S_k, d = 2, 2, 1, 5, 6, 3
    q = _f32(rng.standard_normal((B, A, S_q, d)))
    k = _f32(rng.standard_normal((B, A_kv, S_k, d)))
    v = _f32(rng.standard_normal((B, A_kv, S_k, d)))
    o0, l0 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, causal=True)
    o1, l1 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, causal=True, bias=np.zeros((B, 1, S_q, S_k), np.float32))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    mk = (rng.random((B, S_q, S_k)) > 0.4).astype(np.uint8)
    o2, l2 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, m_keep=mk)
    bias = np.where(mk[:, None] != 0, 0.0, -np.inf).astype(np.float32)
    o3, l3 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, bias=bias)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


def pin_bias_row_shift(orc):
    """Softmax ignores a constant added to a whole row: O is unchanged and the
    log-sum-exp moves by exactly that constant."""
    rng = np.random.default_rng(63)
    B, A, S_q, S_k, d = 2, 3, 4, 9, 5
    q = _f32(rng.standard_normal((B, A, S_q, d)))
    k = _f32(rng.standard_normal((B, A, S_k, d)))
    v = _f32(rng.standard_normal((B, A, S_k, d)))
    c = _f32(rng.uniform(-20, 20, (B, A, S_q, 1)))
    o0, l0 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.4)
    o1, l1 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.4, bias=np.broadcast_to(c, (B, A, S_q, S_k)))
    assert np.allclose(o0, o1, rtol=0, atol=1e-12)
    assert np.allclose(l1 - l0, c[..., 0].astype(np.float64), rtol=0, atol=1e-12)


def pin_bias_log_weights(orc):
    """M = ln w weights each key's exponential by w: O_i = sum_j w_ij e^{s_ij} v_j
    / sum_j w_ij e^{s_ij}, evaluated directly in numpy."""
    rng = np.random.default_rng(64)
    B, A, S_q, S_k, d, scale = 1, 2, 3, 8, 4, 0.7
    q = _f32(rng.standard_normal((B, A, S_q, d)))
    k = _f32(rng.standard_normal((B, A, S_k, d)))
    v = _f32(rng.standard_normal((B, A, S_k, d)))
    w = _f32(rng.uniform(0.05, 4.0, (B, A, S_q, S_k)))
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=scale, bias=np.log(w.astype(np.float64)).astype(np.float32))
    lw = np.log(w.astype(np.float64)).astype(np.float32).astype(np.float64)  # the term as the oracle reads it
    sc = float(np.float32(scale))  # the scale is an fp32 argument
    s = sc * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
    e = np.exp(s) * np.exp(lw)
    want = np.einsum("bhij,bhjd->bhid", e, v.astype(np.float64)) / e.sum(-1, keepdims=True)
    assert np.allclose(o, want, rtol=0, atol=1e-12)
    assert np.allclose(lse, np.log(e.sum(-1)), rtol=0, atol=1e-12)


def pin_window_equals_key_slice(orc):
    """A sliding-window row equals plain attention over the contiguous slice of
    keys the window keeps (same keys in the same order: bit for bit); a row
    whose window holds no key is fully masked."""
    import oracle as oracle_pkg
    rng = np.random.default_rng(43)
    for S_q, S_k, left, right in [(6, 9, 2, 1), (7, 7, 3, 0), (5, 8, 0, 0), (4, 6, -1, 1), (6, 6, 2, -1),
                                  (8, 5, 1, 0)]:
        q = _f32(rng.standard_normal((1, 2, S_q, 4)))
        k = _f32(rng.standard_normal((1, 1, S_k, 4)))
        v = _f32(rng.standard_normal((1, 1, S_k, 4)))
        mk = oracle_pkg.window_keep(1, S_q, S_k, left, right)
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.625, m_keep=mk)
        off = S_k - S_q
        for i in range(S_q):
            lo = max(0, i + off - left) if left >= 0 else 0
            hi = min(S_k - 1, i + off + right) if right >= 0 else S_k - 1
            if lo > hi:
                assert np.all(o[0, :, i] == 0) and np.all(np.isneginf(lse[0, :, i])), (S_q, S_k, left, right, i)
                continue
            os_, ls = orc.attn_fwd(q[:, :, i:i + 1], k[:, :, lo:hi + 1], v[:, :, lo:hi + 1], dtype="f32", scale=0.625)
            assert np.array_equal(o[0, :, i], os_[0, :, 0]), (S_q, S_k, left, right, i)
            assert np.array_equal(lse[0, :, i], ls[0, :, 0]), (S_q, S_k, left, right, i)


# ---- per-row key ranges (document boundaries, prefix-LM)

def pin_key_range_equals_key_slice(orc):
    """A row with key range [first, last] equals plain attention over the
    contiguous slice of keys max(first, 0) .. min(last, S_k - 1) (cut at the
    causal diagonal when causal; same keys in the same order: bit for bit); a
    row whose range holds no key is fully masked."""
    from synth import gen
    rng = np.random.default_rng(44)
    for S_q, S_k, causal in [(9, 12, False), (12, 12, True), (7, 10, True), (10, 6, False)]:
        q = _f32(rng.standard_normal((1, 2, S_q, 4)))
        k = _f32(rng.standard_normal((1, 1, S_k, 4)))
        v = _f32(rng.standard_normal((1, 1, S_k, 4)))
        kr = gen.make_key_ranges(1, S_q, S_k, "random", 5 + S_q)
        kr[0, 0] = (-3, S_k + 5)   # both ends past the keys
        kr[0, 1] = (4, 3)          # empty
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.625, causal=causal, key_range=kr)
        off = S_k - S_q
        for i in range(S_q):
            lo = max(int(kr[0, i, 0]), 0)
            hi = min(int(kr[0, i, 1]), S_k - 1, i + off if causal else S_k - 1)
            if lo > hi:
                assert np.all(o[0, :, i] == 0) and np.all(np.isneginf(lse[0, :, i])), (S_q, S_k, i)
                continue
            os_, ls = orc.attn_fwd(q[:, :, i:i + 1], k[:, :, lo:hi + 1], v[:, :, lo:hi + 1], dtype="f32",
                                   scale=0.625)
            assert np.array_equal(o[0, :, i], os_[0, :, 0]), (S_q, S_k, causal, i)
            assert np.array_equal(lse[0, :, i], ls[0, :, 0]), (S_q, S_k, causal, i)


def pin_key_range_documents_are_varlen(orc):
    """Packed documents as key ranges (each row keeps its own document, cut at
    the causal diagonal) equal the packed-sequence attention with the
    documents as sequences: the same rows see the same keys."""
    from synth import gen
    rng = np.random.default_rng(45)
    S, A, A_kv, d = 300, 2, 1, 4
    kr = gen.make_key_ranges(1, S, S, "document", 3, doc_median=40)
    doc = gen.document_ids(S, 3, 0, 40)
    cu = np.concatenate([[0], np.cumsum(np.bincount(doc))]).astype(np.int32)
    cu = np.unique(cu)
    assert cu.size > 4
    q = _f32(rng.standard_normal((1, A, S, d)))
    k = _f32(rng.standard_normal((1, A_kv, S, d)))
    v = _f32(rng.standard_normal((1, A_kv, S, d)))
    for causal in (True, False):
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, causal=causal, key_range=kr)
        ov, lv = orc.attn_fwd_varlen(q[0], k[0], v[0], cu, dtype="f32", scale=0.5, causal=causal)
        assert np.allclose(o[0], ov, rtol=0, atol=1e-12) and np.allclose(lse[0], lv, rtol=0, atol=1e-12), causal


def pin_key_range_prefix_lm(orc):
    """Prefix-LM ranges: prefix 0 or 1 is causal attention, a prefix covering
    every key is full (non-causal) attention, and a row inside a prefix of P
    keys attends to exactly the first P keys."""
    from synth import gen
    rng = np.random.default_rng(46)
    S, d = 40, 4
    q = _f32(rng.standard_normal((1, 1, S, d)))
    k = _f32(rng.standard_normal((1, 1, S, d)))
    v = _f32(rng.standard_normal((1, 1, S, d)))
    causal = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, causal=True)
    full = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5)
    for P, want in ((0, causal), (1, causal), (S, full), (S + 7, full)):
        got = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, key_range=gen.make_key_ranges(1, S, S, "prefix", 0, prefix=P))
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), P
    P = 13
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, key_range=gen.make_key_ranges(1, S, S, "prefix", 0, prefix=P))
    pre = orc.attn_fwd(q[:, :, :P], k[:, :, :P], v[:, :, :P], dtype="f32", scale=0.5)
    assert np.array_equal(o[:, :, :P], pre[0]) and np.array_equal(lse[:, :, :P], pre[1])
    assert np.array_equal(o[:, :, P:], causal[0][:, :, P:])


def _window_ranges(positions, left, right):
    first = positions - left if left >= 0 else np.full_like(positions, -1)
    last = positions + right if right >= 0 else np.full_like(positions, 1 << 30)
    return np.stack([first, last], axis=-1).astype(np.int32)


def pin_key_range_packed_paths_equal_windows(orc):
    """Key ranges that describe a sliding window give the window's result in
    the packed prefill, the paged prefill (whose window is applied inside the
    C oracle) and the packed gradient (likewise): the ranges are indexed by
    token and read as positions within each sequence."""
    lens = [70, 0, 33, 101]
    A, A_kv, d = 2, 1, 4
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(47)
    q = _f32(rng.standard_normal((A, T, d)))
    k = _f32(rng.standard_normal((A_kv, T, d)))
    v = _f32(rng.standard_normal((A_kv, T, d)))
    do = _f32(rng.standard_normal((A, T, d)))
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int64)
    for left, right, causal in ((9, 3, False), (20, -1, True), (-1, 5, False)):
        kr = _window_ranges(pos, left, right)
        a = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=0.5, causal=causal, key_range=kr)
        b = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=0.5, causal=causal, window=(left, right))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), (left, right)
        ga = orc.attn_bwd_varlen(q, k, v, do, cu, dtype="f32", scale=0.5, causal=causal, key_range=kr)
        gb = orc.attn_bwd_varlen(q, k, v, do, cu, dtype="f32", scale=0.5, causal=causal, window=(left, right))
        for x, y in zip(ga, gb):
            assert np.allclose(x, y, rtol=0, atol=1e-12), (left, right)
    # ranges together with a window: the intersection of the two intervals
    from synth import gen
    kr2 = gen.make_key_ranges(1, T, max(lens), "random", 8)[0]
    win = _window_ranges(pos, 9, 3)
    both = np.stack([np.maximum(kr2[:, 0], win[:, 0]), np.minimum(kr2[:, 1], win[:, 1])], axis=-1)
    a = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=0.5, causal=False, key_range=kr2, window=(9, 3))
    b = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=0.5, causal=False, key_range=both)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q_lens = [5, 0, 17, 30]
    qp, kc, vc, bt, sl, cuq = _paged_problem([40, 9, 64, 77], q_lens, A, A_kv, d, 16, 48)
    posq = np.concatenate([np.arange(int(L) - ql, int(L)) for L, ql in zip(sl, q_lens)]).astype(np.int64)
    for left, right in ((6, 0), (-1, 0), (12, -1)):
        kr = _window_ranges(posq, left, right)
        a = orc.prefill_paged(qp, kc, vc, bt, sl, cuq, dtype="f32", scale=0.5, causal=False, key_range=kr)
        b = orc.prefill_paged(qp, kc, vc, bt, sl, cuq, dtype="f32", scale=0.5, causal=False, window=(left, right))
        assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], rtol=0, atol=1e-12)


def pin_bwd_key_range_finite_differences(orc):
    """The gradient under document key ranges against central differences of
    the loss sum(O * dO) (fp64 inputs)."""
    from synth import gen
    B, A, A_kv, S_q, S_k, d = 1, 2, 1, 24, 24, 3
    q, k, v, do = _bwd_problem(B, A, A_kv, S_q, S_k, d, 49)
    kr = gen.make_key_ranges(B, S_q, S_k, "document", 9, doc_median=6)
    kr[0, 5] = (7, 2)   # a row that keeps nothing
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.7, causal=True, key_range=kr)
    assert np.all(dq[0, :, 5] == 0)

    def loss(qq, kk, vv):
        o, _ = orc.attn_fwd(qq, kk, vv, dtype="f64", scale=0.7, causal=True, key_range=kr)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            am = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-7, name


# ---- ALiBi (a per-head linear distance penalty as the additive term)

def pin_alibi_causal_is_a_per_key_term(orc):
    """Under causal masking row i's ALiBi term -s (p_i - j) is s j plus a row
    constant, so O equals attention with the per-key term s j alone and the
    LSE moves by -s p_i (softmax shift invariance); per head, its own slope."""
    rng = np.random.default_rng(81)
    B, A, S_q, S_k, d = 1, 3, 7, 11, 4
    slopes = np.array([0.5, 0.125, 2.0])
    q = _f32(rng.standard_normal((B, A, S_q, d)))
    k = _f32(rng.standard_normal((B, A, S_k, d)))
    v = _f32(rng.standard_normal((B, A, S_k, d)))
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, causal=True, alibi_slopes=slopes)
    p = np.arange(S_q) + (S_k - S_q)
    for h, sl in enumerate(slopes):
        term = np.broadcast_to((sl * np.arange(S_k))[None, None, None, :], (B, 1, S_q, S_k)).astype(np.float32)
        o2, l2 = orc.attn_fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], dtype="f32", scale=0.5, causal=True,
                              bias=term)
        assert np.allclose(o[:, h], o2[:, 0], rtol=0, atol=1e-10), h
        assert np.allclose(lse[:, h], l2[:, 0] - sl * p, rtol=0, atol=1e-9), h


def pin_alibi_closed_forms(orc):
    """Slope 0 is no term (bitwise); two keys give the logistic of the logit
    difference including the distance penalty; a huge slope leaves only the
    key at the query's own position (O = that value row); non-causal ALiBi is
    mirror-symmetric: row i over keys reversed = row S - 1 - i over the
    original keys."""
    rng = np.random.default_rng(82)
    S, d = 9, 4
    q = _f32(rng.standard_normal((1, 1, S, d)))
    k = _f32(rng.standard_normal((1, 1, S, d)))
    v = _f32(rng.standard_normal((1, 1, S, d)))
    a = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, alibi_slopes=[0.0])
    b = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # two keys at positions 0 and 1, query rows at positions 0 and 1 (S_q = S_k = 2)
    s2 = 0.75
    o, lse = orc.attn_fwd(q[:, :, :2], k[:, :, :2], v[:, :, :2], dtype="f32", scale=0.5, alibi_slopes=[s2])
    qq, kk, vv = (x[0, 0, :2].astype(np.float64) for x in (q, k, v))
    for i in range(2):
        z = 0.5 * (qq[i] @ kk.T) - s2 * np.abs(i - np.arange(2))
        w = expit(z[0] - z[1])
        assert np.allclose(o[0, 0, i], w * vv[0] + (1 - w) * vv[1], rtol=0, atol=1e-12)
        assert abs(lse[0, 0, i] - np.logaddexp(z[0], z[1])) < 1e-12
    o, _ = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, alibi_slopes=[1e4])
    assert np.array_equal(o[0, 0], v[0, 0].astype(np.float64))
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, alibi_slopes=[0.3])
    om, lm = orc.attn_fwd(q[:, :, ::-1], k[:, :, ::-1], v[:, :, ::-1], dtype="f32", scale=0.5, alibi_slopes=[0.3])
    assert np.allclose(o[0, 0], om[0, 0, ::-1], rtol=0, atol=1e-12)
    assert np.allclose(lse[0, 0], lm[0, 0, ::-1], rtol=0, atol=1e-12)


def pin_alibi_packed_and_paged_positions(orc):
    """Packed sequences measure distances within each sequence (one sequence
    = the dense call, bitwise), and a paged chunk's rows sit at the bottom of
    their sequence: they equal the last rows of the dense call over the whole
    sequence, ALiBi included."""
    rng = np.random.default_rng(83)
    A, A_kv, d = 2, 1, 4
    slopes = np.array([0.25, 1.0])
    lens = [9, 0, 14]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = _f32(rng.standard_normal((A, T, d)))
    k = _f32(rng.standard_normal((A_kv, T, d)))
    v = _f32(rng.standard_normal((A_kv, T, d)))
    o, lse = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=0.5, causal=False, alibi_slopes=slopes)
    for s0, s1 in ((0, 9), (9, 23)):
        o2, l2 = orc.attn_fwd(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], dtype="f32", scale=0.5,
                              alibi_slopes=slopes)
        assert np.array_equal(o[:, s0:s1], o2[0]) and np.array_equal(lse[:, s0:s1], l2[0])
    q_lens = [3, 0, 5]
    qp, kc, vc, bt, sl, cuq = _paged_problem([20, 4, 33], q_lens, A, A_kv, d, 16, 84)
    for causal in (True, False):
        op, lp = orc.prefill_paged(qp, kc, vc, bt, sl, cuq, dtype="f32", scale=0.5, causal=causal,
                                   alibi_slopes=slopes)
        for sidx, (L, ql) in enumerate(zip(sl, q_lens)):
            if ql == 0:
                continue
            c0 = int(cuq[sidx])
            kk = _contiguous(kc, bt[sidx], int(L), 16)[None]
            vv = _contiguous(vc, bt[sidx], int(L), 16)[None]
            # the chunk's rows are the last ql of a dense call with S_q = S_k = L
            qfull = np.zeros((1, A, int(L), d), np.float32)
            qfull[0, :, L - ql:] = qp[:, c0:c0 + ql]
            o2, l2 = orc.attn_fwd(qfull, kk, vv, dtype="f32", scale=0.5, causal=causal, alibi_slopes=slopes)
            assert np.allclose(op[:, c0:c0 + ql], o2[0, :, L - ql:], rtol=0, atol=1e-12), (sidx, causal)
            assert np.allclose(lp[:, c0:c0 + ql], l2[0, :, L - ql:], rtol=0, atol=1e-12), (sidx, causal)


def pin_bwd_alibi_finite_differences(orc):
    """The gradient with ALiBi (non-causal, two heads with their own slopes,
    packed and dense) against central differences of the loss sum(O * dO)."""
    B, A, A_kv, S_q, S_k, d = 1, 2, 1, 6, 9, 3
    q, k, v, do = _bwd_problem(B, A, A_kv, S_q, S_k, d, 85)
    slopes = [0.4, 1.5]
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.7, alibi_slopes=slopes)

    def loss(qq, kk, vv):
        o, _ = orc.attn_fwd(qq, kk, vv, dtype="f64", scale=0.7, alibi_slopes=slopes)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            am = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-7, name
    # packed: one sequence's gradient is the dense gradient of that sequence
    cu = np.array([0, 4, 9], np.int32)
    qp, kp, vp, dop = q[0, :, :S_q], k[0, :, :S_k], v[0, :, :S_k], do[0, :, :S_q]
    qp = np.concatenate([qp, qp[:, :3]], axis=1)[:, :9]
    dop = np.concatenate([dop, dop[:, :3]], axis=1)[:, :9]
    g = orc.attn_bwd_varlen(qp, kp, vp, dop, cu, dtype="f64", scale=0.7, causal=True, alibi_slopes=slopes)
    for s0, s1 in ((0, 4), (4, 9)):
        r = orc.attn_bwd(qp[None, :, s0:s1], kp[None, :, s0:s1], vp[None, :, s0:s1], dop[None, :, s0:s1],
                         dtype="f64", scale=0.7, causal=True, alibi_slopes=slopes)
        for x, y in zip(g, r):
            assert np.array_equal(x[:, s0:s1], y[0])


def pin_decode_alibi_is_last_dense_row(orc):
    """Paged decode with ALiBi (and with a window) = the last row of the
    dense causal prefill with ALiBi over the sequence's keys gathered token by
    token; an empty sequence is a fully masked row; the FP8-cache decode
    takes the same slopes."""
    rng = np.random.default_rng(86)
    lens, A, A_kv, d, ps = [40, 0, 17, 33], 4, 2, 4, 16
    slopes = np.array([0.5, 0.25, 1.0, 0.0])
    q, kc, vc, bt, sl, _ = _paged_problem(lens, [0] * len(lens), A, A_kv, d, ps, 87)
    qd = _f32(rng.standard_normal((len(lens), A, d)))
    for wl in (None, 5):
        o, lse = orc.decode_paged(qd, kc, vc, bt, sl, dtype="f32", scale=0.5, alibi_slopes=slopes, window_left=wl)
        for b, L in enumerate(lens):
            if L == 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
                continue
            kk = _contiguous(kc, bt[b], L, ps)[None]
            vv = _contiguous(vc, bt[b], L, ps)[None]
            qq = np.zeros((1, A, L, d), np.float32)
            qq[0, :, L - 1] = qd[b]
            mk = None if wl is None else oracle_window(L, wl)
            o2, l2 = orc.attn_fwd(qq, kk, vv, dtype="f32", scale=0.5, causal=True, alibi_slopes=slopes, m_keep=mk)
            assert np.allclose(o[b], o2[0, :, L - 1], rtol=0, atol=1e-12), (b, wl)
            assert np.allclose(lse[b], l2[0, :, L - 1], rtol=0, atol=1e-12), (b, wl)
    # FP8 caches: the same decode over the dequantised pages
    import oracle as oracle_pkg
    codes = lambda shape: (rng.integers(0, 0x7E, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    k8, v8 = codes(kc.shape), codes(vc.shape)
    ks, vs = rng.uniform(0.01, 0.1, kc.shape[::2]), rng.uniform(0.01, 0.1, kc.shape[::2])
    qb = gen.f32_to_bf16_bits(qd)
    o8, l8 = orc.decode_paged_fp8(qb, k8, v8, ks, vs, bt, sl, scale=0.5, alibi_slopes=slopes)
    kd = oracle_pkg.fp8_e4m3_value(k8) * ks[:, None, :, None]
    vd = oracle_pkg.fp8_e4m3_value(v8) * vs[:, None, :, None]
    qf = gen.bf16_bits_to_f32(qb).astype(np.float64)
    o9, l9 = orc.decode_paged(qf, kd, vd, bt, sl, dtype="f64", scale=0.5, alibi_slopes=slopes)
    assert np.allclose(o8, o9, rtol=0, atol=1e-12) and np.allclose(l8[np.isfinite(l9)], l9[np.isfinite(l9)], atol=1e-12)


def oracle_window(L, wl):
    import oracle as oracle_pkg
    return oracle_pkg.window_keep(1, L, L, wl, 0)


# ---- FP8 (OCP E4M3) caches: code values, and decode over dequantised pages

def pin_fp8_e4m3_published_values(orc):
    """Values the OCP FP8 specification lists for E4M3: zero, the smallest
    subnormal 2^-9, the largest subnormal 7 * 2^-9, the smallest normal 2^-6,
    one, the largest finite 448, negative zero, and NaN at S.1111.111."""
    import oracle as oracle_pkg
    v = oracle_pkg.fp8_e4m3_value
    assert v(0x00) == 0.0 and v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9 and v(0x08) == 2.0 ** -6
    assert v(0x38) == 1.0 and v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x80) == 0.0 and np.signbit(v(0x80))
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    vals = v(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)                         # codes 0..126 increase strictly
    assert np.array_equal(v(np.arange(0x80, 0xFF)), -vals)   # the sign bit only negates


def pin_fp8_decode_brute_force(orc):
    """Tiny FP8 paged decode against math.fsum over K = code value * k_scale and
    V = code value * v_scale, scales per (page, KV head)."""
    import oracle as oracle_pkg
    rng = np.random.default_rng(51)
    ps, A, A_kv, d = 4, 4, 2, 3
    lens = np.array([6, 1, 0], np.int32)
    bt = np.array([[2, 0], [1, -1], [-1, -1]], np.int32)
    kc = rng.integers(0, 0x7F, size=(3, ps, A_kv, d)).astype(np.uint8) | (rng.integers(0, 2, size=(3, ps, A_kv, d)) * 0x80).astype(np.uint8)
    vc = rng.integers(0, 0x7F, size=(3, ps, A_kv, d)).astype(np.uint8)
    ksc = rng.uniform(0.001, 0.01, size=(3, A_kv)).astype(np.float32)
    vsc = rng.uniform(0.001, 0.01, size=(3, A_kv)).astype(np.float32)
    q = gen.f32_to_bf16_bits(rng.standard_normal((3, A, d)).astype(np.float32))
    o, lse = orc.decode_paged_fp8(q, kc, vc, ksc, vsc, bt, lens, scale=0.75)
    qv = gen.bf16_bits_to_f32(q).astype(np.float64)
    G = A // A_kv
    for b in range(3):
        for h in range(A):
            hk = h // G
            keys, vals = [], []
            for t in range(int(lens[b])):
                pg, off = int(bt[b, t // ps]), t % ps
                keys.append([float(x) * float(ksc[pg, hk]) for x in oracle_pkg.fp8_e4m3_value(kc[pg, off, hk])])
                vals.append([float(x) * float(vsc[pg, hk]) for x in oracle_pkg.fp8_e4m3_value(vc[pg, off, hk])])
            want, wl = _brute([float(x) for x in qv[b, h]], keys, vals, 0.75, [True] * len(keys))
            if not keys:
                want = [0.0] * d
            assert np.allclose(o[b, h], want, rtol=0, atol=1e-13), (b, h)
            assert (wl == -math.inf and lse[b, h] == -np.inf) or abs(lse[b, h] - wl) < 1e-13


def pin_fp8_decode_window_brute_force(orc):
    """FP8 paged decode under a sliding window ("Attention Kernel", 可编程 mask:
    the query at position len - 1 sees the keys t >= len - 1 - w) against
    math.fsum over the visible dequantised keys alone, for windows of 0, 2
    and 9 keys and one reaching past the first token."""
    import oracle as oracle_pkg
    rng = np.random.default_rng(52)
    ps, A, A_kv, d = 4, 4, 2, 3
    lens = np.array([11, 1, 0, 6], np.int32)
    bt = np.array([[3, 0, 5], [1, -1, -1], [-1, -1, -1], [2, 4, -1]], np.int32)
    kc = rng.integers(0, 0x7F, size=(6, ps, A_kv, d)).astype(np.uint8) | (rng.integers(0, 2, size=(6, ps, A_kv, d)) * 0x80).astype(np.uint8)
    vc = rng.integers(0, 0x7F, size=(6, ps, A_kv, d)).astype(np.uint8)
    ksc = rng.uniform(0.001, 0.01, size=(6, A_kv)).astype(np.float32)
    vsc = rng.uniform(0.001, 0.01, size=(6, A_kv)).astype(np.float32)
    q = gen.f32_to_bf16_bits(rng.standard_normal((4, A, d)).astype(np.float32))
    qv = gen.bf16_bits_to_f32(q).astype(np.float64)
    G = A // A_kv
    for w in (0, 2, 9, 50):
        o, lse = orc.decode_paged_fp8(q, kc, vc, ksc, vsc, bt, lens, scale=0.75, window_left=w)
        for b in range(4):
            L = int(lens[b])
            for h in range(A):
                hk = h // G
                keys, vals = [], []
                for t in range(max(0, L - 1 - w), L):
                    pg, off = int(bt[b, t // ps]), t % ps
                    keys.append([float(x) * float(ksc[pg, hk]) for x in oracle_pkg.fp8_e4m3_value(kc[pg, off, hk])])
                    vals.append([float(x) * float(vsc[pg, hk]) for x in oracle_pkg.fp8_e4m3_value(vc[pg, off, hk])])
                want, wl = _brute([float(x) for x in qv[b, h]], keys, vals, 0.75, [True] * len(keys))
                if not keys:
                    want = [0.0] * d
                assert np.allclose(o[b, h], want, rtol=0, atol=1e-13), (w, b, h)
                assert (wl == -math.inf and lse[b, h] == -np.inf) or abs(lse[b, h] - wl) < 1e-13, (w, b, h)


def pin_fp8_prefill_brute_force(orc):
    """FP8 dense prefill (E4M3 codes, one scale per 128 tokens of each head)
    against math.fsum over the dequantised rows: S = 300 queries and keys span
    three scale blocks, each with its own scale, so a block size or index
    mistake moves rows of the later blocks."""
    import oracle as oracle_pkg
    rng = np.random.default_rng(52)
    B, A, A_kv, S_q, S_k, d = 1, 2, 1, 300, 280, 4
    qc = rng.integers(0, 0x7F, size=(B, A, S_q, d)).astype(np.uint8) | (rng.integers(0, 2, size=(B, A, S_q, d)) * 0x80).astype(np.uint8)
    kc = rng.integers(0, 0x7F, size=(B, A_kv, S_k, d)).astype(np.uint8) | (rng.integers(0, 2, size=(B, A_kv, S_k, d)) * 0x80).astype(np.uint8)
    qs = rng.uniform(0.001, 0.004, size=(B, A, 3)).astype(np.float32)
    ks = rng.uniform(0.001, 0.004, size=(B, A_kv, 3)).astype(np.float32)
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, A_kv, S_k, d)).astype(np.float32))
    o, lse = orc.attn_fwd_fp8(qc, kc, v, qs, ks, scale=0.5, causal=True)
    vv = gen.bf16_bits_to_f32(v).astype(np.float64)
    off = S_k - S_q
    for h in range(A):
        for i in (0, 21, 127, 128, 200, 255, 256, 299):
            qrow = [float(x) * float(qs[0, h, i // 128]) for x in oracle_pkg.fp8_e4m3_value(qc[0, h, i])]
            keys, vals, vis = [], [], []
            for j in range(S_k):
                keys.append([float(x) * float(ks[0, 0, j // 128]) for x in oracle_pkg.fp8_e4m3_value(kc[0, 0, j])])
                vals.append([float(x) for x in vv[0, 0, j]])
                vis.append(j <= i + off)
            want, wl = _brute(qrow, keys, vals, 0.5, vis)
            if wl == -math.inf:
                assert np.all(o[0, h, i] == 0) and np.isneginf(lse[0, h, i]), (h, i)
                continue
            assert np.allclose(o[0, h, i], want, rtol=0, atol=1e-12), (h, i)
            assert abs(lse[0, h, i] - wl) < 1e-12, (h, i)


# ---- gradient (oracle_attn_bwd): the exact derivative of the forward above.
# Pinned against central finite differences of the (already pinned) forward
# in fp64, closed forms and invariants of the softmax Jacobian.

def _bwd_problem(B, A, A_kv, S_q, S_k, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, A, S_q, d))
    k = rng.standard_normal((B, A_kv, S_k, d))
    v = rng.standard_normal((B, A_kv, S_k, d))
    do = rng.standard_normal((B, A, S_q, d))
    return q, k, v, do


def _loss(orc, q, k, v, do, scale, causal, q_keep=None, k_keep=None, m_keep=None):
    o, _ = orc.attn_fwd(q, k, v, dtype="f64", scale=scale, causal=causal, q_keep=q_keep, k_keep=k_keep,
                        m_keep=m_keep)
    return float(np.sum(o.reshape(do.shape) * do))


def pin_bwd_finite_differences(orc):
    """Every entry of dQ, dK, dV equals the central difference of
    L = sum(O * dO) computed with the forward oracle (h = 1e-6, fp64)."""
    cases = [  # B, A, A_kv, S_q, S_k, d, causal, masks (1: keep flags, 2: a dense keep matrix)
        (1, 2, 1, 3, 4, 3, True, 0),
        (1, 2, 2, 4, 3, 2, False, 1),
        (2, 2, 1, 3, 3, 2, True, 1),
        (1, 2, 1, 4, 5, 2, False, 2),
    ]
    h = 1e-6
    for n, (B, A, A_kv, S_q, S_k, d, causal, masks) in enumerate(cases):
        q, k, v, do = _bwd_problem(B, A, A_kv, S_q, S_k, d, 100 + n)
        scale = 0.6875  # exact in fp32
        qk = kk = mk = None
        if masks == 1:
            qk = np.ones((B, S_q), np.uint8)
            qk[0, 1] = 0
            kk = np.ones((B, S_k), np.uint8)
            kk[-1, 0] = 0
        elif masks == 2:
            mk = (np.random.default_rng(200 + n).random((B, S_q, S_k)) > 0.4).astype(np.uint8)
            mk[0, 2, :] = 0  # one row fully masked
        dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=scale, causal=causal, q_keep=qk, k_keep=kk,
                                  m_keep=mk)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (_loss(orc, *args_p, do, scale, causal, qk, kk, mk) -
                            _loss(orc, *args_m, do, scale, causal, qk, kk, mk)) / (2 * h)
            err = np.max(np.abs(num - g))
            assert err <= 1e-7, (n, name, err)


def pin_bwd_two_keys(orc):
    """One query, two keys: with a = s_1 - s_2, dS_1 = -dS_2 =
    sigmoid(a) sigmoid(-a) (dP_1 - dP_2), dV_1 = sigmoid(a) dO, dV_2 = sigmoid(-a) dO."""
    q, k, v, do = _bwd_problem(1, 1, 1, 1, 2, 3, 7)
    scale = 0.875  # exact in fp32, the oracle's scale type
    s = scale * (k[0, 0] @ q[0, 0, 0])
    a = s[0] - s[1]
    p1, p2 = expit(a), expit(-a)
    dp = v[0, 0] @ do[0, 0, 0]
    ds1 = p1 * p2 * (dp[0] - dp[1])
    dq_ref = scale * (ds1 * k[0, 0, 0] - ds1 * k[0, 0, 1])
    dk_ref = np.stack([scale * ds1 * q[0, 0, 0], -scale * ds1 * q[0, 0, 0]])
    dv_ref = np.stack([p1 * do[0, 0, 0], p2 * do[0, 0, 0]])
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=scale)
    assert np.allclose(dq[0, 0, 0], dq_ref, rtol=0, atol=1e-13)
    assert np.allclose(dk[0, 0], dk_ref, rtol=0, atol=1e-13)
    assert np.allclose(dv[0, 0], dv_ref, rtol=0, atol=1e-13)


def pin_bwd_single_key(orc):
    """A single visible key: O = v, so dV = dO and dQ = dK = 0."""
    q, k, v, do = _bwd_problem(1, 2, 1, 1, 1, 4, 8)
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.5)
    assert np.all(dq == 0) and np.all(dk == 0)
    assert np.allclose(dv[0, 0, 0], do[0, 0, 0] + do[0, 1, 0], rtol=0, atol=1e-15)


def pin_bwd_uniform_values(orc):
    """All value rows equal: O does not depend on the scores, so dQ = dK = 0,
    and dV_j = sum_i P_ij dO_i with P from a library softmax."""
    q, k, v, do = _bwd_problem(1, 1, 1, 3, 5, 2, 9)
    v[:] = v[0, 0, 0]
    scale = 0.625  # exact in fp32, the oracle's scale type
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=scale)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14
    P = softmax(scale * q[0, 0] @ k[0, 0].T, axis=1)
    assert np.allclose(dv[0, 0], P.T @ do[0, 0], rtol=0, atol=1e-13)


def pin_bwd_key_gradients_sum_to_zero(orc):
    """Each row of dS sums to zero (softmax Jacobian), so sum_j dK_j = 0 for
    every (batch, KV head), with masks too."""
    q, k, v, do = _bwd_problem(2, 4, 2, 6, 7, 3, 10)
    kk = np.ones((2, 7), np.uint8)
    kk[1, 3] = 0
    _, dk, _ = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.8, causal=True, k_keep=kk)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
    assert np.max(np.abs(dk)) > 1e-3


def pin_bwd_gqa_equals_repeated_heads(orc):
    """GQA gradients equal those of the MHA problem with each KV head repeated
    G times, dK and dV summed over the repeats."""
    q, k, v, do = _bwd_problem(1, 4, 2, 5, 6, 3, 11)
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.7, causal=True)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = orc.attn_bwd(q, kr, vr, do, dtype="f64", scale=0.7, causal=True)
    assert np.allclose(dq, dq2, rtol=0, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(1, 2, 2, 6, 3).sum(axis=2), rtol=0, atol=1e-13)
    assert np.allclose(dv, dv2.reshape(1, 2, 2, 6, 3).sum(axis=2), rtol=0, atol=1e-13)


def pin_bwd_masked_row_inert(orc):
    """A query row whose keep flag is 0 has dQ = 0 and its dO moves nothing."""
    q, k, v, do = _bwd_problem(1, 2, 2, 4, 4, 3, 12)
    qk = np.ones((1, 4), np.uint8)
    qk[0, 2] = 0
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.5, q_keep=qk)
    assert np.all(dq[:, :, 2] == 0)
    do2 = do.copy()
    do2[:, :, 2] += 5.0
    _, dk2, dv2 = orc.attn_bwd(q, k, v, do2, dtype="f64", scale=0.5, q_keep=qk)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


# ---- block masks (page "Attention Kernel", section "可编程 mask": one flag per
# 128 x 128 block of (row, key) pairs), the block mask of an additive term,
# and the masking fill value of a finite term

def _expand_blocks_by_loops(bk_bh, S_q, S_k):
    """The element rule keep[i][j] = block flag (i // 128, j // 128), one
    element at a time."""
    keep = np.zeros((S_q, S_k), np.uint8)
    for i in range(S_q):
        for j in range(S_k):
            keep[i, j] = 1 if bk_bh[i // 128][j // 128] else 0
    return keep


def pin_block_keep_element_rule(orc):
    """A block mask equals, bit for bit, the dense keep matrix its element rule
    defines (built here element by element), per head and per batch row, on
    ragged sizes with more key blocks than row blocks; with causal and key
    flags combined."""
    rng = np.random.default_rng(61)
    B, A, A_kv, S_q, S_k, d = 2, 2, 1, 300, 420, 4
    q = _f32(rng.standard_normal((B, A, S_q, d)))
    k = _f32(rng.standard_normal((B, A_kv, S_k, d)))
    v = _f32(rng.standard_normal((B, A_kv, S_k, d)))
    kk = (rng.random((B, S_k)) > 0.1).astype(np.uint8)
    bk = (rng.random((B, A, 3, 4)) < 0.6).astype(np.uint8)
    bk[0, 0, 0, :] = 1
    bk[1, 1, 2, :] = 0                     # a row block with no key block kept
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, causal=causal, k_keep=kk, block_keep=bk)
        for h in range(A):
            mk = np.stack([_expand_blocks_by_loops(bk[b, h], S_q, S_k) for b in range(B)])
            o2, l2 = orc.attn_fwd(q[:, h:h + 1], k, v, dtype="f32", scale=0.5, causal=causal, k_keep=kk, m_keep=mk)
            assert np.array_equal(o[:, h:h + 1], o2) and np.array_equal(lse[:, h:h + 1], l2), (causal, h)
    assert np.all(np.isneginf(lse[1, 1, 256:]))
    # one mask shared by the heads
    o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, block_keep=bk[:, :1])
    mk = np.stack([_expand_blocks_by_loops(bk[b, 0], S_q, S_k) for b in range(B)])
    o2, l2 = orc.attn_fwd(q, k, v, dtype="f32", scale=0.5, m_keep=mk)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def pin_block_keep_of_bias_brute_force(orc):
    """The block mask of an additive term: 1 exactly where some entry of the
    block (clipped to the matrix) exceeds -inf, checked block by block and
    element by element."""
    rng = np.random.default_rng(62)
    B, H, S_q, S_k = 2, 2, 260, 300
    bias = rng.standard_normal((B, H, S_q, S_k)).astype(np.float32)
    bias[rng.random(bias.shape) < 0.97] = -np.inf
    bias[0, 0, :128, :] = -np.inf            # a whole row of blocks masked
    bias[1, 1, 200:, 256:] = -np.inf         # the ragged corner block masked
    bias[1, 0, 259, 299] = np.float32(-3e38)  # a finite entry keeps its block
    bias[1, 0, 256:259, 256:] = -np.inf
    bias[1, 0, 259, 256:299] = -np.inf
    got = orc.block_keep_of_bias(bias)
    assert got.shape == (B, H, 3, 3)
    for b in range(B):
        for h in range(H):
            for qb in range(3):
                for kb in range(3):
                    kept = 0
                    for i in range(128 * qb, min(128 * qb + 128, S_q)):
                        for j in range(128 * kb, min(128 * kb + 128, S_k)):
                            if bias[b, h, i, j] > -np.inf:
                                kept = 1
                                break
                        if kept:
                            break
                    assert got[b, h, qb, kb] == kept, (b, h, qb, kb)
    assert got[0, 0, 0].sum() == 0 and got[1, 1, 2, 2] == 0 and got[1, 0, 2, 2] == 1


def pin_bias_fill_value(orc):
    """A finite term below -FLT_MAX * min(scale, ln 2) is a masking fill value:
    a row filled with the float32 minimum is fully masked (O = 0, LSE = -inf);
    with one key left at 0 the row sees that key alone (O = v_j exactly,
    LSE = s_j); a large but representable term (-1e30 on every key) is an
    ordinary constant shift (mean of V, LSE = -1e30 + ln n)."""
    rng = np.random.default_rng(63)
    S_k, d = 6, 3
    q = _f32(rng.standard_normal((1, 1, 3, d)))
    k = _f32(rng.standard_normal((1, 1, S_k, d)))
    v = _f32(rng.standard_normal((1, 1, S_k, d)))
    fmin = np.finfo(np.float32).min
    bias = np.zeros((1, 1, 3, S_k), np.float32)
    bias[0, 0, 0, :] = fmin
    bias[0, 0, 1, :] = fmin
    bias[0, 0, 1, 4] = 0.0
    bias[0, 0, 2, :] = np.float32(-1e30)
    for scale in (0.125, 2.0):
        o, lse = orc.attn_fwd(q, k, v, dtype="f32", scale=scale, bias=bias)
        assert np.all(o[0, 0, 0] == 0) and np.isneginf(lse[0, 0, 0])
        assert np.array_equal(o[0, 0, 1], v[0, 0, 4].astype(np.float64))
        s4 = float(np.float32(scale)) * float(np.dot(q[0, 0, 1].astype(np.float64), k[0, 0, 4].astype(np.float64)))
        assert abs(lse[0, 0, 1] - s4) < 1e-12
        assert np.allclose(o[0, 0, 2], v[0, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)
        m = float(np.float32(-1e30))  # the term as stored (fp32)
        assert abs(lse[0, 0, 2] / m - 1) < 1e-15


# ---- prefill of query chunks over a paged cache: each chunk is the tail of
# its sequence (bottom-right positions); keys through the block table

def _paged_problem(lens, q_lens, A, A_kv, d, ps, seed):
    rng = np.random.default_rng(seed)
    npg = [(L + ps - 1) // ps for L in lens]
    pool = sum(npg) + 2
    perm = rng.permutation(pool)
    bt = np.full((len(lens), max(max(npg), 1)), -1, np.int32)
    at = 0
    for s, n in enumerate(npg):
        bt[s, :n] = perm[at:at + n]
        at += n
    kc = _f32(rng.standard_normal((pool, ps, A_kv, d)))
    vc = _f32(rng.standard_normal((pool, ps, A_kv, d)))
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = _f32(rng.standard_normal((A, int(cu[-1]), d)))
    return q, kc, vc, bt, np.array(lens, np.int32), cu


def _contiguous(cache, bt_row, L, ps):
    """Tokens 0..L-1 of one sequence as [A_kv, L, d], token by token: token t
    is row t % ps of page bt_row[t // ps]."""
    out = np.zeros((cache.shape[2], L, cache.shape[3]), cache.dtype)
    for t in range(L):
        out[:, t] = cache[bt_row[t // ps], t % ps]
    return out


def pin_prefill_paged_decode_rows(orc):
    """Chunks of one row are decode steps: bit for bit the paged decode of the
    same sequences (causal changes nothing for the last position)."""
    lens = [9, 1, 23, 16]
    A, A_kv, d, ps = 4, 2, 3, 4
    q, kc, vc, bt, sl, cu = _paged_problem(lens, [1, 1, 1, 1], A, A_kv, d, ps, 64)
    for causal in (True, False):
        o, lse = orc.prefill_paged(q, kc, vc, bt, sl, cu, dtype="f32", scale=0.75, causal=causal)
        od, ld = orc.decode_paged(np.ascontiguousarray(q.transpose(1, 0, 2)), kc, vc, bt, sl, dtype="f32",
                                  scale=0.75)
        assert np.array_equal(o.transpose(1, 0, 2), od) and np.array_equal(lse.T, ld)


def pin_decode_window_rows(orc):
    """A decode step with a sliding window of w keys before the query is the
    one-row chunk of the paged prefill under the window (w, unbounded right),
    bit for bit ("Attention Kernel", 可编程 mask: sliding window), for windows
    shorter and longer than the sequences."""
    lens = [9, 1, 23, 16, 5]
    A, A_kv, d, ps = 4, 2, 3, 4
    q, kc, vc, bt, sl, cu = _paged_problem(lens, [1] * len(lens), A, A_kv, d, ps, 66)
    qd = np.ascontiguousarray(q.transpose(1, 0, 2))
    for w in (0, 3, 8, 40):
        o, lse = orc.prefill_paged(q, kc, vc, bt, sl, cu, dtype="f32", scale=0.75, causal=True, window=(w, -1))
        od, ld = orc.decode_paged(qd, kc, vc, bt, sl, dtype="f32", scale=0.75, window_left=w)
        assert np.array_equal(o.transpose(1, 0, 2), od) and np.array_equal(lse.T, ld), w


def pin_decode_window_closed_forms(orc):
    """Window 0: the query sees only itself, O = v of the last token exactly and
    LSE = scale q . k_last.  Window 1: the two-key softmax written out.  A
    window reaching the first token: the decode without a window, bit for bit."""
    lens = [7, 12, 2]
    A, A_kv, d, ps = 2, 1, 5, 4
    q, kc, vc, bt, sl, cu = _paged_problem(lens, [1] * len(lens), A, A_kv, d, ps, 67)
    qd = np.ascontiguousarray(q.transpose(1, 0, 2)).astype(np.float64)
    o0, l0 = orc.decode_paged(qd.astype(np.float32), kc, vc, bt, sl, dtype="f32", scale=0.5, window_left=0)
    o1, l1 = orc.decode_paged(qd.astype(np.float32), kc, vc, bt, sl, dtype="f32", scale=0.5, window_left=1)
    for b, L in enumerate(lens):
        kk = _contiguous(kc, bt[b], L, ps).astype(np.float64)
        vv = _contiguous(vc, bt[b], L, ps).astype(np.float64)
        for h in range(A):
            s_last = 0.5 * float(qd[b, h] @ kk[0, L - 1])
            assert np.array_equal(o0[b, h], vv[0, L - 1]) and abs(l0[b, h] - s_last) < 1e-12
            s_prev = 0.5 * float(qd[b, h] @ kk[0, L - 2])
            m = max(s_last, s_prev)
            e1, e2 = math.exp(s_prev - m), math.exp(s_last - m)
            want = (e1 * vv[0, L - 2] + e2 * vv[0, L - 1]) / (e1 + e2)
            assert np.allclose(o1[b, h], want, rtol=0, atol=1e-12)
            assert abs(l1[b, h] - (m + math.log(e1 + e2))) < 1e-12
    on, ln = orc.decode_paged(qd.astype(np.float32), kc, vc, bt, sl, dtype="f32", scale=0.5)
    ow, lw = orc.decode_paged(qd.astype(np.float32), kc, vc, bt, sl, dtype="f32", scale=0.5, window_left=11)
    assert np.array_equal(on, ow) and np.array_equal(ln, lw)


def pin_varlen_masks_brute_force(orc):
    """Packed sequences with a per-token additive term, per-sequence block
    masks and a window, against a direct fp64 softmax of each sequence's own
    score matrix (tiny sizes; the term's row t and column j are token t and the
    key at position j of t's sequence; block (qb, kb) of sequence s covers its
    rows and keys 128 qb.., 128 kb..)."""
    rng = np.random.default_rng(68)
    lens = [130, 0, 200, 7]
    A, A_kv, d, scale = 2, 1, 4, 0.625   # (a float32 value: the oracle takes the scale as float)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, nb = int(cu[-1]), 2
    q = _f32(rng.standard_normal((A, T, d)))
    k = _f32(rng.standard_normal((A_kv, T, d)))
    v = _f32(rng.standard_normal((A_kv, T, d)))
    bias = _f32(rng.standard_normal((A, T, 204)))
    bias[rng.random(bias.shape) < 0.1] = -np.inf
    bk = (rng.random((len(lens), A, nb, nb)) < 0.7).astype(np.uint8)
    bk[0, :, 1, 0] = 1
    for causal, window in ((True, None), (False, (50, 20)), (True, (90, -1))):
        o, lse = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=scale, causal=causal, bias=bias,
                                     block_keep=bk, window=window)
        ids = np.array([0 * T + 3, 1 * T + 140, 0 * T + T - 1, 1 * T + 131], np.int64)
        o_r, l_r = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=scale, causal=causal, bias=bias,
                                       block_keep=bk, window=window, rows=ids)
        assert np.array_equal(o_r, o.reshape(-1, d)[ids]) and np.array_equal(l_r, lse.reshape(-1)[ids])
        for s, L in enumerate(lens):
            s0 = int(cu[s])
            for h in range(A):
                qq = q[h, s0:s0 + L].astype(np.float64)
                kk = k[h // (A // A_kv), s0:s0 + L].astype(np.float64)
                vv = v[h // (A // A_kv), s0:s0 + L].astype(np.float64)
                sc = scale * qq @ kk.T + bias[h, s0:s0 + L, :L].astype(np.float64)
                i = np.arange(L)[:, None]
                j = np.arange(L)[None, :]
                keep = bk[s, h][i // 128, j // 128] != 0
                if causal:
                    keep &= j <= i
                if window is not None:
                    if window[0] >= 0:
                        keep &= j >= i - window[0]
                    if window[1] >= 0:
                        keep &= j <= i + window[1]
                sc = np.where(keep, sc, -np.inf)
                for r in range(L):
                    row = sc[r]
                    if not np.isfinite(row).any():
                        assert np.all(o[h, s0 + r] == 0) and np.isneginf(lse[h, s0 + r])
                        continue
                    m = row[np.isfinite(row)].max()
                    e = np.exp(row - m)
                    want = e @ vv / e.sum()
                    assert np.allclose(o[h, s0 + r], want, rtol=0, atol=1e-12), (s, h, r)
                    assert abs(lse[h, s0 + r] - (m + math.log(e.sum()))) < 1e-12


def pin_prefill_paged_masks_neutral(orc):
    """A zero term and an all-ones block mask change nothing: the masked paged
    prefill (keys gathered per sequence, the dense definition per chunk) is the
    paged prefill bit for bit, with and without a window."""
    lens, q_lens = [9, 130, 23, 260], [3, 130, 1, 129]
    A, A_kv, d, ps = 4, 2, 3, 4
    q, kc, vc, bt, sl, cu = _paged_problem(lens, q_lens, A, A_kv, d, ps, 69)
    T_q = int(cu[-1])
    zero = np.zeros((A, T_q, max(lens)), np.float32)
    ones = np.ones((len(lens), 1, 2, 3), np.uint8)
    for causal, window in ((True, None), (False, None), (True, (40, -1))):
        o, lse = orc.prefill_paged(q, kc, vc, bt, sl, cu, dtype="f32", scale=0.75, causal=causal, window=window)
        o2, l2 = orc.prefill_paged(q, kc, vc, bt, sl, cu, dtype="f32", scale=0.75, causal=causal, window=window,
                                   bias=zero, block_keep=ones)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2), (causal, window)


def pin_prefill_paged_masks_brute_force(orc):
    """Chunks with a per-token term and per-sequence block masks against a
    direct fp64 softmax over keys read token by token from the pages."""
    rng = np.random.default_rng(70)
    lens, q_lens = [150, 20, 300], [140, 1, 150]
    A, A_kv, d, ps, scale = 2, 1, 4, 8, 0.625
    q, kc, vc, bt, sl, cu = _paged_problem(lens, q_lens, A, A_kv, d, ps, 71)
    T_q = int(cu[-1])
    bias = _f32(rng.standard_normal((A, T_q, 304)))
    bias[rng.random(bias.shape) < 0.1] = -np.inf
    bk = (rng.random((len(lens), A, 2, 3)) < 0.7).astype(np.uint8)
    ids = np.array([0 * T_q + 5, 1 * T_q + T_q - 1, 1 * T_q + 141], np.int64)
    for causal in (True, False):
        o, lse = orc.prefill_paged(q, kc, vc, bt, sl, cu, dtype="f32", scale=scale, causal=causal, bias=bias,
                                   block_keep=bk)
        o_r, l_r = orc.prefill_paged(q, kc, vc, bt, sl, cu, dtype="f32", scale=scale, causal=causal, bias=bias,
                                     block_keep=bk, rows=ids)
        assert np.array_equal(o_r, o.reshape(-1, d)[ids]) and np.array_equal(l_r, lse.reshape(-1)[ids])
        for s, (L, ql) in enumerate(zip(lens, q_lens)):
            s0 = int(cu[s])
            kk = _contiguous(kc, bt[s], L, ps).astype(np.float64)
            vv = _contiguous(vc, bt[s], L, ps).astype(np.float64)
            for h in range(A):
                qq = q[h, s0:s0 + ql].astype(np.float64)
                sc = scale * qq @ kk[0].T + bias[h, s0:s0 + ql, :L].astype(np.float64)
                i = np.arange(ql)[:, None]
                j = np.arange(L)[None, :]
                keep = bk[s, h][i // 128, j // 128] != 0
                if causal:
                    keep &= j <= i + (L - ql)
                sc = np.where(keep, sc, -np.inf)
                for r in range(ql):
                    row = sc[r]
                    if not np.isfinite(row).any():
                        assert np.all(o[h, s0 + r] == 0) and np.isneginf(lse[h, s0 + r])
                        continue
                    m = row[np.isfinite(row)].max()
                    e = np.exp(row - m)
                    assert np.allclose(o[h, s0 + r], e @ vv[0] / e.sum(), rtol=0, atol=1e-12), (s, h, r)
                    assert abs(lse[h, s0 + r] - (m + math.log(e.sum()))) < 1e-12


def pin_prefill_paged_identity_is_varlen(orc):
    """With pages laid out in order and each whole sequence as its chunk, the
    paged prefill is the packed varlen prefill, bit for bit."""
    rng = np.random.default_rng(65)
    lens = [7, 0, 12, 5]
    A, A_kv, d, ps = 4, 2, 3, 4
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = _f32(rng.standard_normal((A, T, d)))
    k = _f32(rng.standard_normal((A_kv, T, d)))
    v = _f32(rng.standard_normal((A_kv, T, d)))
    npg = [(L + ps - 1) // ps for L in lens]
    kc = np.zeros((sum(npg), ps, A_kv, d), np.float32)
    vc = np.zeros_like(kc)
    bt = np.full((len(lens), max(npg)), -1, np.int32)
    page = 0
    for s, L in enumerate(lens):
        for t in range(L):
            if t % ps == 0:
                bt[s, t // ps] = page
                page += 1
            kc[page - 1, t % ps] = k[:, cu[s] + t]
            vc[page - 1, t % ps] = v[:, cu[s] + t]
    for causal in (True, False):
        o, lse = orc.prefill_paged(q, kc, vc, bt, np.array(lens, np.int32), cu, dtype="f32", scale=0.5,
                                   causal=causal)
        o2, l2 = orc.attn_fwd_varlen(q, k, v, cu, dtype="f32", scale=0.5, causal=causal)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2), causal


def pin_prefill_paged_chunk_tail(orc):
    """A chunk of q_s < L rows (scattered pages) equals the last q_s rows of the
    dense bottom-right-aligned prefill over the sequence's contiguous keys,
    causal and with a two-sided window; an empty chunk computes nothing."""
    import oracle as oracle_pkg
    lens, q_lens = [13, 6, 20], [5, 0, 20]
    A, A_kv, d, ps = 2, 1, 3, 4
    q, kc, vc, bt, sl, cu = _paged_problem(lens, q_lens, A, A_kv, d, ps, 66)
    for causal, window in ((True, None), (False, None), (True, (3, -1)), (False, (2, 4))):
        o, lse = orc.prefill_paged(q, kc, vc, bt, sl, cu, dtype="f32", scale=0.625, causal=causal, window=window)
        for s, (L, n) in enumerate(zip(lens, q_lens)):
            if n == 0:
                continue
            k = _contiguous(kc, bt[s], L, ps)[None]
            v = _contiguous(vc, bt[s], L, ps)[None]
            qs = q[None, :, cu[s]:cu[s + 1]]
            mk = None if window is None else oracle_pkg.window_keep(1, n, L, window[0], window[1])
            o2, l2 = orc.attn_fwd(qs, k, v, dtype="f32", scale=0.625, causal=causal, m_keep=mk)
            assert np.array_equal(o[:, cu[s]:cu[s + 1]], o2[0]), (s, causal, window)
            assert np.array_equal(lse[:, cu[s]:cu[s + 1]], l2[0]), (s, causal, window)


def pin_prefill_paged_fp8(orc):
    """Over FP8 caches: one-row chunks equal the FP8 paged decode (bit for
    bit), and a chunk of 5 rows matches math.fsum over the dequantised keys
    (code value x its page's scale) at the bottom-right positions."""
    import oracle as oracle_pkg
    rng = np.random.default_rng(72)
    ps, A, A_kv, d = 4, 4, 2, 3
    lens = np.array([9, 6, 1], np.int32)
    bt = np.array([[3, 0, 5], [1, 4, -1], [2, -1, -1]], np.int32)
    kc = rng.integers(0, 0x7F, size=(6, ps, A_kv, d)).astype(np.uint8) | (rng.integers(0, 2, size=(6, ps, A_kv, d)) * 0x80).astype(np.uint8)
    vc = rng.integers(0, 0x7F, size=(6, ps, A_kv, d)).astype(np.uint8)
    ksc = rng.uniform(0.001, 0.01, size=(6, A_kv)).astype(np.float32)
    vsc = rng.uniform(0.001, 0.01, size=(6, A_kv)).astype(np.float32)
    q1 = gen.f32_to_bf16_bits(rng.standard_normal((A, 3, d)).astype(np.float32))
    cu1 = np.array([0, 1, 2, 3], np.int32)
    o, lse = orc.prefill_paged_fp8(q1, kc, vc, ksc, vsc, bt, lens, cu1, scale=0.75)
    od, ld = orc.decode_paged_fp8(np.ascontiguousarray(q1.transpose(1, 0, 2)), kc, vc, ksc, vsc, bt, lens,
                                  scale=0.75)
    assert np.array_equal(o.transpose(1, 0, 2), od) and np.array_equal(lse.T, ld)
    q5 = gen.f32_to_bf16_bits(rng.standard_normal((A, 5, d)).astype(np.float32))
    cu5 = np.array([0, 5, 5, 5], np.int32)
    o, lse = orc.prefill_paged_fp8(q5, kc, vc, ksc, vsc, bt, lens, cu5, scale=0.75)
    qv = gen.bf16_bits_to_f32(q5).astype(np.float64)
    G = A // A_kv
    for h in range(A):
        hk = h // G
        keys = [[float(x) * float(ksc[bt[0, t // ps], hk]) for x in oracle_pkg.fp8_e4m3_value(kc[bt[0, t // ps], t % ps, hk])]
                for t in range(9)]
        vals = [[float(x) * float(vsc[bt[0, t // ps], hk]) for x in oracle_pkg.fp8_e4m3_value(vc[bt[0, t // ps], t % ps, hk])]
                for t in range(9)]
        for i in range(5):
            pos = 9 - 5 + i
            want, wl = _brute([float(x) for x in qv[h, i]], keys, vals, 0.75, [t <= pos for t in range(9)])
            assert np.allclose(o[h, i], want, rtol=0, atol=1e-13) and abs(lse[h, i] - wl) < 1e-13, (h, i)


# ---- gradient of the packed varlen prefill, and of block / additive masks

def pin_bwd_varlen_equals_separate(orc):
    """The varlen gradient is the dense gradient of each sequence on its own
    (bit for bit), with keep flags, GQA, causal or not, and a window given as
    the dense keep matrix of its definition; tokens of empty or fully masked
    rows receive exactly zero."""
    import oracle as oracle_pkg
    rng = np.random.default_rng(67)
    lens = [5, 0, 9, 1, 7]
    A, A_kv, d = 4, 2, 3
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, do = rng.standard_normal((A, T, d)), rng.standard_normal((A, T, d))
    k, v = rng.standard_normal((A_kv, T, d)), rng.standard_normal((A_kv, T, d))
    qk = np.ones(T, np.uint8)
    kk = np.ones(T, np.uint8)
    qk[[3, 10]] = 0
    kk[[2, 8, 15, 21]] = 0
    for causal, window in ((True, None), (False, None), (True, (2, -1)), (False, (1, 3))):
        dq, dk, dv = orc.attn_bwd_varlen(q, k, v, do, cu, dtype="f64", scale=0.8, causal=causal, q_keep=qk,
                                         k_keep=kk, window=window)
        for s, L in enumerate(lens):
            a, b = cu[s], cu[s + 1]
            if L == 0:
                continue
            mk = None if window is None else oracle_pkg.window_keep(1, L, L, window[0], window[1])
            r = orc.attn_bwd(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], do[None, :, a:b], dtype="f64",
                             scale=0.8, causal=causal, q_keep=qk[None, a:b], k_keep=kk[None, a:b], m_keep=mk)
            for g, want in zip((dq, dk, dv), r):
                assert np.array_equal(g[:, a:b], want[0]), (causal, window, s)


def pin_bwd_varlen_masks(orc):
    """The packed-sequence gradient with per-sequence blocks and per-token
    terms: neutral masks give the unmasked packed gradient bit for bit, and
    with real masks it matches central differences of the packed forward under
    the same masks (the forward's and the backward's slicing are separate
    code)."""
    rng = np.random.default_rng(72)
    lens = [4, 0, 6, 3]
    A, A_kv, d, scale = 2, 1, 3, 0.7
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, do = rng.standard_normal((A, T, d)), rng.standard_normal((A, T, d))
    k, v = rng.standard_normal((A_kv, T, d)), rng.standard_normal((A_kv, T, d))
    zero = np.zeros((A, T, 8), np.float32)
    ones = np.ones((len(lens), 1, 1, 1), np.uint8)
    ref = orc.attn_bwd_varlen(q, k, v, do, cu, dtype="f64", scale=scale, causal=True)
    neu = orc.attn_bwd_varlen(q, k, v, do, cu, dtype="f64", scale=scale, causal=True, bias=zero, block_keep=ones)
    for g, want in zip(neu, ref):
        assert np.array_equal(g, want)
    bias = (0.5 * rng.standard_normal((A, T, 6))).astype(np.float32)
    bias[0, 5, 1] = -np.inf
    bias[1, 11, 0] = -np.inf
    bk = np.ones((len(lens), A, 1, 1), np.uint8)
    bk[3, 1] = 0                     # head 1 of the last sequence fully masked
    dq, dk, dv = orc.attn_bwd_varlen(q, k, v, do, cu, dtype="f64", scale=scale, causal=False, bias=bias,
                                     block_keep=bk)

    def loss(qq, kk, vv):
        o, _ = orc.attn_fwd_varlen(qq, kk, vv, cu, dtype="f64", scale=scale, causal=False, bias=bias, block_keep=bk)
        return float(np.sum(o * do))
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for h, t, e in [(0, 0, 0), (1, 5, 2), (0, 9, 1), (1, T - 1, 0), (0, 12, 2)]:
            idx = (h % arr.shape[0], t, e)
            saved = arr[idx]
            arr[idx] = saved + eps
            lp = loss(q, k, v)
            arr[idx] = saved - eps
            lm = loss(q, k, v)
            arr[idx] = saved
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (idx, fd, grad[idx])
    assert np.all(dq[1, 10:13] == 0)  # the fully masked head and sequence


def pin_bwd_masks_finite_differences(orc):
    """Gradients with a block mask, an additive term (finite values and -inf)
    and both: central differences of L = sum(O * dO) through the forward."""
    rng = np.random.default_rng(68)
    B, A, A_kv, S_q, S_k, d = 1, 2, 1, 3, 4, 2
    q, k, v, do = _bwd_problem(B, A, A_kv, S_q, S_k, d, 69)
    bias = rng.standard_normal((B, A, S_q, S_k)).astype(np.float32)
    bias[0, 0, 1, 2] = -np.inf
    bias[0, 1, 0, :] = -np.inf
    bk = np.ones((B, 1, 1, 1), np.uint8)
    h = 1e-6
    for kw in ({"bias": bias}, {"block_keep": bk}, {"bias": bias[:, :1], "block_keep": bk}):
        dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.6875, causal=True, **kw)

        def loss(qq, kk_, vv):
            o, _ = orc.attn_fwd(qq, kk_, vv, dtype="f64", scale=0.6875, causal=True, **kw)
            return float(np.sum(o * do))
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                ap = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                am = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
            assert np.max(np.abs(num - g)) <= 1e-7, (list(kw), name)
        if "bias" in kw and kw["bias"].shape[1] == A:
            assert np.all(dq[0, 1, 0] == 0)  # the row the term masks whole has no gradient


def pin_bwd_block_mask_is_keep_matrix(orc):
    """A block mask in the gradient equals its dense keep matrix (element rule,
    built element by element), bit for bit, per head."""
    rng = np.random.default_rng(70)
    B, A, A_kv, S_q, S_k, d = 1, 2, 2, 200, 300, 2
    q, k, v, do = _bwd_problem(B, A, A_kv, S_q, S_k, d, 71)
    bk = (rng.random((B, A, 2, 3)) < 0.6).astype(np.uint8)
    bk[0, 0, 1, 0] = 1
    bk[0, 1, 0, 2] = 0
    dq, dk, dv = orc.attn_bwd(q, k, v, do, dtype="f64", scale=0.5, causal=False, block_keep=bk)
    for h in range(A):
        mk = _expand_blocks_by_loops(bk[0, h], S_q, S_k)[None]
        r = orc.attn_bwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], do[:, h:h + 1], dtype="f64", scale=0.5,
                         m_keep=mk)
        for g, want in zip((dq, dk, dv), r):
            assert np.array_equal(g[:, h:h + 1], want), h


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
