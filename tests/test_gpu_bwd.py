"""GPU parity: the backward pass (dQ, dK, dV recomputed from the forward's LSE)
against the fp64 oracle's exact gradient.

The GPU side runs its own forward first (O and LSE are the backward's inputs),
the oracle differentiates the same bf16 Q, K, V for the same dO.  Small cases
are compared over every element; the full-size causal workload on sampled
(batch, head) slices plus properties that hold at any size.
"""
import sys

import numpy as np
import pytest

import oracle
from synth import gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ea():
    import exact_attention_108_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def run_bwd(ea, p, dout, q_keep=None, k_keep=None, window=None):
    """GPU forward then backward; returns (dq, dk, dv) as float64 arrays."""
    t = gu.torch()
    q, k, v = gu.dev(p.q, "bf16"), gu.dev(p.k, "bf16"), gu.dev(p.v, "bf16")
    do = gu.dev(dout, "bf16")
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    qk = None if q_keep is None else gu.dev(q_keep, "u8")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk, window=window)
    dq, dk, dv = (gu.empty_out(x.shape, "bf16") for x in (q, k, v))
    for x in (dq, dk, dv):
        x.fill_(float("nan"))
    ws = t.empty(max(ea.attn_bwd_workspace_bytes(p.B, p.A, p.S_q), 1), dtype=t.uint8, device="cuda")
    ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk,
                window=window)
    t.cuda.synchronize()
    return gu.host_f64(dq), gu.host_f64(dk), gu.host_f64(dv)


def visibility(B, S_q, S_k, causal, q_keep=None, k_keep=None):
    """[B, S_q, S_k] bool: which (row, key) pairs the mask leaves in."""
    i = np.arange(S_q)[:, None]
    j = np.arange(S_k)[None, :]
    vis = np.ones((B, S_q, S_k), bool)
    if causal:
        vis &= (j <= i + (S_k - S_q))[None]
    if q_keep is not None:
        vis &= (np.asarray(q_keep) != 0)[:, :, None]
    if k_keep is not None:
        vis &= (np.asarray(k_keep) != 0)[:, None, :]
    return vis


def compare(got, ref, what, vis=None, A=1, A_kv=1):
    """Element-wise check of (dq, dk, dv); with ``vis`` also that rows of dq and
    keys of dk/dv that see nothing are exactly zero."""
    zq = zk = None
    if vis is not None:
        zq = np.repeat(~vis.any(axis=2)[:, None, :], A, axis=1)       # [B, A, S_q]
        zk = np.repeat(~vis.any(axis=1)[:, None, :], A_kv, axis=1)    # [B, A_kv, S_k]
    out = {}
    for name, g, r, z in zip(("dq", "dk", "dv"), got, ref, (zq, zk, zk)):
        out[name] = gu.check_grad(g, r, f"{what} {name}", zero_rows=z)
    return out


BWD_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal
    (1, 1, 1, 1, 1, 128, False),
    (1, 2, 1, 17, 17, 128, True),
    (2, 4, 4, 64, 64, 128, True),
    (1, 2, 2, 127, 129, 128, True),
    (1, 2, 2, 129, 127, 128, True),     # the first two rows see no key
    (2, 8, 2, 200, 200, 128, True),     # GQA 4:1
    (1, 4, 1, 300, 300, 64, True),      # GQA 4:1, d = 64
    (1, 3, 3, 128, 1000, 64, False),
    (1, 2, 2, 300, 300, 128, False),
    (2, 4, 2, 257, 384, 64, True),
    (1, 1, 1, 1, 700, 128, True),
    (1, 2, 1, 5, 0, 128, True),         # no key: dQ = 0
    (1, 2, 1, 0, 5, 128, True),         # no query: dK = dV = 0
    (1, 16, 1, 130, 130, 128, True),    # 16 query heads summed into one KV head
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n"))
def test_bwd_small(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal = case
    _say("bwd bf16", case)
    seed = 500 + sum(case[:6])
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=seed)
    dout = gen.make_dout(p, seed)
    got = run_bwd(ea, p, dout)
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=causal)
    vis = visibility(B, S_q, S_k, causal)
    _say(compare(got, ref, str(case), vis, A, A_kv))


def test_bwd_keep_masks(ea, orc):
    _say("bwd keep masks")
    p = gen.make_dense(2, 4, 2, 150, 190, 128, dtype="bf16", causal=True, seed=77, q_masked=30, k_masked=60)
    kk = p.k_keep.copy()
    kk[1, :] = 0                        # batch row 1: every key masked
    dout = gen.make_dout(p, 77)
    got = run_bwd(ea, p, dout, q_keep=p.q_keep, k_keep=kk)
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=True, q_keep=p.q_keep, k_keep=kk)
    vis = visibility(p.B, p.S_q, p.S_k, True, p.q_keep, kk)
    _say(compare(got, ref, "keep masks", vis, p.A, p.A_kv))
    dq, dk, dv = got
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)
    assert np.all(dq[0][:, p.q_keep[0] == 0] == 0)
    assert np.all(dk[0][:, kk[0] == 0] == 0) and np.all(dv[0][:, kk[0] == 0] == 0)


def test_bwd_deterministic(ea):
    _say("bwd determinism")
    p = gen.make_dense(1, 8, 2, 300, 300, 128, dtype="bf16", causal=True, seed=91)
    dout = gen.make_dout(p, 91)
    a = run_bwd(ea, p, dout)
    b = run_bwd(ea, p, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _slice(p, b, hk):
    """The independent sub-problem of batch b, KV head hk and its query heads."""
    G = p.A // p.A_kv
    hs = slice(hk * G, (hk + 1) * G)
    return (p.q[b:b + 1, hs], p.k[b:b + 1, hk:hk + 1], p.v[b:b + 1, hk:hk + 1]), hs


@pytest.mark.parametrize("shape", [(4, 32, 32, 2048, 128), (1, 32, 8, 2048, 128)],
                         ids=["mha-4x32x2048x128", "gqa-1x32:8x2048x128"])
def test_bwd_full_size_sampled(ea, orc, shape):
    B, A, A_kv, S, d = shape
    _say("bwd full size", shape)
    p = gen.make_dense(B, A, A_kv, S, S, d, dtype="bf16", causal=True, seed=1002)
    dout = gen.make_dout(p, 1002)
    dq, dk, dv = run_bwd(ea, p, dout)
    # any size: finite, and the key gradients of every head sum to zero (each
    # row of dS sums to zero, so sum_j dK_j = scale sum_i (sum_j dS_ij) q_i = 0)
    for x in (dq, dk, dv):
        assert np.all(np.isfinite(x))
    col_sum = np.abs(dk.sum(axis=2))
    col_norm = np.sqrt((dk ** 2).sum(axis=2))
    assert np.all(col_sum <= 2.0 ** -5 * col_norm + 1e-6), float((col_sum / (col_norm + 1e-30)).max())
    # sampled (batch, KV head) slices against the oracle, element by element
    rng = np.random.default_rng(11)
    picks = [(0, 0), (B - 1, A_kv - 1), (int(rng.integers(B)), int(rng.integers(A_kv)))]
    for b, hk in picks:
        (qs, ks, vs), hs = _slice(p, b, hk)
        ref = orc.attn_bwd(qs, ks, vs, dout[b:b + 1, hs], dtype="bf16", scale=p.scale, causal=True)
        got = (dq[b:b + 1, hs], dk[b:b + 1, hk:hk + 1], dv[b:b + 1, hk:hk + 1])
        _say("slice", (b, hk), compare(got, ref, f"{shape} slice {(b, hk)}"))


def run_bwd_window(ea, p, dout, window, k_keep=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, "bf16"), gu.dev(p.k, "bf16"), gu.dev(p.v, "bf16")
    do = gu.dev(dout, "bf16")
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, k_keep=kk, window=window)
    dq, dk, dv = (gu.empty_out(x.shape, "bf16") for x in (q, k, v))
    for x in (dq, dk, dv):
        x.fill_(float("nan"))
    ws = t.empty(max(ea.attn_bwd_workspace_bytes(p.B, p.A, p.S_q), 1), dtype=t.uint8, device="cuda")
    ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p.scale, causal=p.causal, k_keep=kk, window=window)
    t.cuda.synchronize()
    return gu.host_f64(dq), gu.host_f64(dk), gu.host_f64(dv)


BWD_WINDOW_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, (left, right)
    (1, 2, 1, 300, 300, 128, True, (0, -1)),
    (2, 4, 2, 500, 500, 128, True, (100, -1)),
    (1, 2, 2, 300, 420, 128, True, (63, -1)),
    (1, 2, 2, 420, 300, 128, True, (200, -1)),
    (1, 2, 2, 400, 400, 128, False, (40, 90)),
    (1, 4, 1, 350, 350, 64, True, (129, -1)),
    (1, 2, 1, 300, 300, 128, True, (2147483647, -1)),     # the widest edge: the causal gradient
    (1, 2, 2, 260, 300, 64, False, (2147483647, 2147483647)),
]


@pytest.mark.parametrize("case", BWD_WINDOW_CASES,
                         ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n") + f"w{c[7][0]}_{c[7][1]}")
def test_bwd_window(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, (left, right) = case
    _say("bwd window", case)
    seed = 800 + S_q + left
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=seed)
    dout = gen.make_dout(p, seed)
    got = run_bwd_window(ea, p, dout, (left, right))
    mk = oracle.window_keep(B, S_q, S_k, left, 0 if causal else right)
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=causal, m_keep=mk)
    vis = visibility(B, S_q, S_k, causal) & (mk != 0)
    if left == 0 and causal:
        # every row sees one key: p = 1 and dS = dP - D = 0 exactly, so the
        # exact dQ and dK vanish by cancellation.  The GPU's dS is the
        # rounding difference of two fp32 sums (dP by MFMA, D from the bf16
        # O = v): |dS_i| <= 2 u sum_e |dO_ie v_ie| with u = 2^-8 (bounding both
        # sums' fp32 errors generously); dQ_i = scale dS_i k_i and
        # dK_i = scale sum over the query heads of dS_i q_i
        assert S_q == S_k and np.all(ref[0] == 0) and np.all(ref[1] == 0)
        q_, k_, v_ = (gen.as_f32(x, "bf16").astype(np.float64) for x in (p.q, p.k, p.v))
        do_ = gen.as_f32(dout, "bf16").astype(np.float64)
        G = A // A_kv
        kv, vv = np.repeat(k_, G, axis=1), np.repeat(v_, G, axis=1)
        ds_bound = 2 * 2.0 ** -8 * np.abs(do_ * vv).sum(axis=-1, keepdims=True)   # [B, A, S, 1]
        assert np.all(np.abs(got[0]) <= 1.01 * p.scale * ds_bound * np.abs(kv))
        dk_bound = (p.scale * ds_bound * np.abs(q_)).reshape(B, A_kv, G, S_q, d).sum(axis=2)
        assert np.all(np.abs(got[1]) <= 1.01 * dk_bound)
        _say({"dv": gu.check_grad(got[2], ref[2], f"{case} dv"), "dq_max": float(np.abs(got[0]).max()),
              "dk_max": float(np.abs(got[1]).max())})
        return
    _say(compare(got, ref, str(case), vis, A, A_kv))


# Grids of at least 2048 dK/dV workgroups (key tiles x KV heads x batch) at
# d = 128 run the form of the dK/dV pass that keeps the workgroup's K rows in
# LDS; these cases give it ragged key tiles, keep masks, GQA sums and both
# window shapes, checked on sampled (batch, KV head) slices.
MANY_WG_CASES = [
    # B, A, A_kv, S_q, S_k, causal, window, masked
    (4, 256, 256, 200, 200, True, None, True),         # 2 key tiles (one ragged): 2048 workgroups
    (4, 512, 256, 300, 300, True, (100, -1), False),   # GQA 2:1, 3 key tiles: 3072
    (4, 128, 128, 130, 390, False, (40, 90), False),   # 4 key tiles: 2048
]


@pytest.mark.parametrize("case", MANY_WG_CASES, ids=["mha-masks", "gqa-window", "noncausal-window"])
def test_bwd_many_workgroups_sampled(ea, orc, case):
    B, A, A_kv, S_q, S_k, causal, window, masked = case
    _say("bwd many workgroups", case)
    seed = 900 + S_q + A
    p = gen.make_dense(B, A, A_kv, S_q, S_k, 128, dtype="bf16", causal=causal, seed=seed,
                       q_masked=20 if masked else 0, k_masked=40 if masked else 0)
    dout = gen.make_dout(p, seed)
    q_keep = p.q_keep if masked else None
    k_keep = p.k_keep if masked else None
    dq, dk, dv = run_bwd(ea, p, dout, q_keep=q_keep, k_keep=k_keep, window=window)
    for x in (dq, dk, dv):
        assert np.all(np.isfinite(x))
    mk = None
    vis = visibility(B, S_q, S_k, causal, q_keep, k_keep)
    if window is not None:
        mk = oracle.window_keep(B, S_q, S_k, window[0], 0 if causal else window[1])
        vis &= mk != 0
    G = A // A_kv
    rng = np.random.default_rng(seed)
    picks = [(0, 0), (B - 1, A_kv - 1), (int(rng.integers(B)), int(rng.integers(A_kv)))]
    for b, hk in picks:
        (qs, ks, vs), hs = _slice(p, b, hk)
        kw = {}
        if masked:
            kw.update(q_keep=q_keep[b:b + 1], k_keep=k_keep[b:b + 1])
        if mk is not None:
            kw.update(m_keep=mk[b:b + 1])
        ref = orc.attn_bwd(qs, ks, vs, dout[b:b + 1, hs], dtype="bf16", scale=p.scale, causal=causal, **kw)
        got = (dq[b:b + 1, hs], dk[b:b + 1, hk:hk + 1], dv[b:b + 1, hk:hk + 1])
        _say("slice", (b, hk), compare(got, ref, f"{case} slice {(b, hk)}", vis[b:b + 1], G, 1))
