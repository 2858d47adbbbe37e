"""GPU parity of the backward pass for packed sequences (attn_bwd_varlen) and
for the forward's block and additive masks in attn_bwd, against the fp64
oracle's exact gradient (oracle_attn_bwd_varlen, oracle_attn_bwd with
block_keep / bias).  Page "Attention Kernel", section "Backward 与重计算":
packed-sequence boundaries and the mask must be the forward's.

Each case prints its parameters before it runs.  The GPU side runs its own
forward first (O and LSE are the backward's inputs); the oracle differentiates
the same bf16 inputs for the same dO.
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


# ---- packed sequences

def run_bwd_varlen(ea, p, dout, q_keep=None, k_keep=None, window=None, bias_np=None, bk_np=None):
    t = gu.torch()
    q, k, v, do = (gu.dev(x, "bf16") for x in (p.q, p.k, p.v, dout))
    cu = gu.dev(p.cu_seqlens, "i32")
    qk = None if q_keep is None else gu.dev(q_keep, "u8")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    bias = None
    if bias_np is not None:
        H, T, L = bias_np.shape
        ld = max(4, (L + 3) // 4 * 4)
        full = t.zeros((H, T, ld), dtype=t.float32, device="cuda")
        full[..., :L] = t.from_numpy(bias_np).cuda()
        bias = full[..., :L]
    bk = None if bk_np is None else t.from_numpy(bk_np).cuda()
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.A, p.T), dtype=t.float32, device="cuda")
    ea.attn_fwd_varlen(q, k, v, o, lse, cu, p.cu_seqlens, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk,
                       window=window, block_keep=bk, bias=bias)
    dq, dk, dv = (gu.empty_out(x.shape, "bf16") for x in (q, k, v))
    for x in (dq, dk, dv):
        x.fill_(float("nan"))
    ws = t.empty(max(ea.attn_bwd_workspace_bytes(1, p.A, p.T), 1), dtype=t.uint8, device="cuda")
    ea.attn_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, cu, p.cu_seqlens, ws, scale=p.scale, causal=p.causal,
                       q_keep=qk, k_keep=kk, window=window, block_keep=bk, bias=bias)
    t.cuda.synchronize()
    return gu.host_f64(dq), gu.host_f64(dk), gu.host_f64(dv)


VARLEN_CASES = [
    # lens, A, A_kv, d, causal, window, masked
    ([1, 0, 130, 17, 400, 64, 300], 4, 2, 128, True, None, False),
    ([257, 1, 128, 129, 5], 2, 2, 128, True, None, True),
    ([300, 77, 513], 4, 1, 64, True, (70, -1), False),
    ([200, 0, 333], 2, 2, 128, False, None, False),
    ([190, 260], 2, 1, 64, False, (40, 30), True),
    ([0, 0, 3], 2, 2, 128, True, None, False),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"n{len(c[0])}A{c[1]}:{c[2]}d{c[3]}"
                         + ("c" if c[4] else "n") + ("w" if c[5] else "") + ("m" if c[6] else ""))
def test_bwd_varlen(ea, orc, case):
    lens, A, A_kv, d, causal, window, masked = case
    _say("bwd varlen", case)
    seed = 1400 + sum(lens) + A + d
    p = gen.make_varlen(lens, A, A_kv, d, dtype="bf16", causal=causal, seed=seed,
                        q_mask_frac=0.05 if masked else 0.0, k_mask_frac=0.1 if masked else 0.0)
    dout = gen.draw((A, p.T, d), seed, gen.S_DOUT, "normal", "bf16")
    got = run_bwd_varlen(ea, p, dout, p.q_keep, p.k_keep, window)
    w = None if window is None else (window[0], 0 if causal else window[1])
    ref = orc.attn_bwd_varlen(p.q, p.k, p.v, dout, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=causal,
                              q_keep=p.q_keep, k_keep=p.k_keep, window=w)
    out = {n: gu.check_grad(g, r, f"{case} {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)}
    _say(out)


def test_bwd_varlen_workload_sampled(ea, orc):
    """The packed varlen workload's shape (16 log-normal sequences, A = 16,
    d = 64, causal, 5% of query rows fully masked): every gradient finite, and
    the longest, the shortest and one drawn sequence against the oracle (each
    sequence is an independent problem)."""
    p = gen.make_config(5)
    dout = gen.draw((p.A, p.T, p.d), 1005, gen.S_DOUT, "normal", "bf16")
    _say("bwd varlen workload", p.T)
    dq, dk, dv = run_bwd_varlen(ea, p, dout, p.q_keep)
    for x in (dq, dk, dv):
        assert np.all(np.isfinite(x))
    assert np.all(dq[:, p.q_keep == 0] == 0)
    lens = np.diff(p.cu_seqlens)
    rng = np.random.default_rng(1405)
    for s in sorted({int(np.argmax(lens)), int(np.argmin(lens)), int(rng.integers(lens.size))}):
        a, b = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
        ref = orc.attn_bwd(p.q[None, :, a:b], p.k[None, :, a:b], p.v[None, :, a:b], dout[None, :, a:b], dtype="bf16",
                           scale=p.scale, causal=True, q_keep=p.q_keep[None, a:b])
        got = (dq[None, :, a:b], dk[None, :, a:b], dv[None, :, a:b])
        _say("sequence", s, b - a, {n: gu.check_grad(g, r, f"workload seq {s} {n}")
                                    for n, g, r in zip(("dq", "dk", "dv"), got, ref)})


# ---- block masks and the additive term

def run_bwd_masked(ea, p, dout, *, block_keep=None, bias=None, q_keep=None, k_keep=None, window=None):
    t = gu.torch()
    q, k, v, do = (gu.dev(x, "bf16") for x in (p.q, p.k, p.v, dout))
    bk = None if block_keep is None else gu.dev(block_keep, "u8")
    bs = None if bias is None else ea.pad_bias(t.from_numpy(bias).cuda())
    qk = None if q_keep is None else gu.dev(q_keep, "u8")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk, window=window,
                block_keep=bk, bias=bs)
    dq, dk, dv = (gu.empty_out(x.shape, "bf16") for x in (q, k, v))
    for x in (dq, dk, dv):
        x.fill_(float("nan"))
    ws = t.empty(max(ea.attn_bwd_workspace_bytes(p.B, p.A, p.S_q), 1), dtype=t.uint8, device="cuda")
    ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk,
                window=window, block_keep=bk, bias=bs)
    t.cuda.synchronize()
    return gu.host_f64(dq), gu.host_f64(dk), gu.host_f64(dv)


MASK_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, block_heads (0 = none), bias kind (None = none), bias heads, window, keeps
    (2, 4, 2, 700, 700, 128, True, 1, None, 0, None, False),
    (1, 4, 4, 513, 900, 128, False, 4, None, 0, None, False),
    (1, 2, 1, 640, 640, 64, True, 2, None, 0, (200, -1), True),
    (2, 4, 2, 300, 300, 128, True, 0, "document", 1, None, False),
    (1, 4, 4, 257, 390, 64, False, 0, "alibi", 4, None, False),
    (2, 2, 1, 200, 333, 128, True, 0, "random", 2, None, True),
    (1, 8, 2, 500, 500, 128, True, 1, "document", 1, None, False),
    (1, 2, 2, 130, 130, 128, True, 2, "random", 1, (40, -1), False),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n")
                         + f"_b{c[7]}" + (f"_{c[8]}{c[9]}" if c[8] else "") + ("_w" if c[10] else "")
                         + ("_keep" if c[11] else ""))
def test_bwd_block_and_bias(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, bh, kind, heads, window, keeps = case
    _say("bwd masks", case)
    seed = 1600 + S_q + S_k + d
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=seed,
                       q_masked=S_q // 10 if keeps else 0, k_masked=S_k // 8 if keeps else 0)
    dout = gen.make_dout(p, seed)
    bk = None
    if bh:
        rng = np.random.default_rng(seed)
        bk = (rng.random((B, bh, (S_q + 127) // 128, (S_k + 127) // 128)) < 0.6).astype(np.uint8)
        # diagonal blocks kept, so that every row block sees keys; then one row
        # block with every block off (a row that sees one key has an exact
        # gradient of 0 that rounding cannot reproduce relative to the scale)
        for i in range(min(bk.shape[2], bk.shape[3])):
            bk[:, :, i, i] = 1
        bk[0, 0, min(1, bk.shape[2] - 1), :] = 0
    bias = None if kind is None else gen.make_bias(B, heads, S_q, S_k, kind, seed)
    qk = p.q_keep if keeps else None
    kk = p.k_keep if keeps else None
    got = run_bwd_masked(ea, p, dout, block_keep=bk, bias=bias, q_keep=qk, k_keep=kk, window=window)
    mk = None if window is None else oracle.window_keep(B, S_q, S_k, window[0], 0 if causal else window[1])
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=causal, q_keep=qk, k_keep=kk,
                       m_keep=mk, bias=bias, block_keep=bk)
    out = {n: gu.check_grad(g, r, f"{case} {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)}
    _say(out)


def test_bwd_bias_fill_value_rows(ea, orc):
    """Rows of the additive term filled with the float32 minimum are fully
    masked in the forward and pass no gradient."""
    p = gen.make_dense(1, 2, 1, 150, 200, 128, dtype="bf16", causal=False, seed=1650)
    dout = gen.make_dout(p, 1650)
    bias = gen.make_bias(1, 2, 150, 200, "random", 1650)
    fmin = np.finfo(np.float32).min
    bias[0, 0, 3, :] = fmin
    bias[0, 1, 7:20, :] = fmin
    bias[0, 1, 9, 55] = 0.0
    _say("bwd fill value rows")
    got = run_bwd_masked(ea, p, dout, bias=bias)
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=False, bias=bias)
    assert np.all(got[0][0, 0, 3] == 0) and np.all(got[0][0, 1, 7:9] == 0)
    _say({n: gu.check_grad(g, r, f"fill {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)})


def test_bwd_block_mask_all_on_equals_dense_bitwise(ea):
    """Every block kept: the masked backward computes exactly the unmasked one."""
    t = gu.torch()
    p = gen.make_dense(1, 4, 2, 300, 300, 128, dtype="bf16", causal=True, seed=1660)
    dout = gen.make_dout(p, 1660)
    _say("bwd block mask all on")
    a = run_bwd_masked(ea, p, dout)
    b = run_bwd_masked(ea, p, dout, block_keep=np.ones((1, 1, 3, 3), np.uint8))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


VARLEN_MASK_CASES = [
    # lens, A, A_kv, d, causal, window, term heads (0 = none), block heads (0 = none)
    ([1, 0, 130, 17, 400, 64, 300], 4, 2, 128, True, None, 1, 1),
    ([257, 1, 128, 129, 5], 2, 2, 128, False, None, 2, 0),
    ([300, 77, 513], 4, 1, 64, True, (70, -1), 0, 4),
    ([190, 260], 2, 1, 64, False, (40, 30), 1, 2),
]


@pytest.mark.parametrize("case", VARLEN_MASK_CASES, ids=lambda c: f"n{len(c[0])}A{c[1]}:{c[2]}d{c[3]}"
                         + ("c" if c[4] else "n") + ("w" if c[5] else "") + f"t{c[6]}b{c[7]}")
def test_bwd_varlen_block_mask_and_term(ea, orc, case):
    """Gradient of packed sequences under the forward's per-sequence block
    masks and per-token terms ("Attention Kernel", Backward 与重计算: the
    backward uses the forward's mask) against the oracle's."""
    lens, A, A_kv, d, causal, window, th, bh = case
    _say("bwd varlen block mask + term", case)
    seed = 1500 + sum(lens) + A + d
    p = gen.make_varlen(lens, A, A_kv, d, dtype="bf16", causal=causal, seed=seed)
    dout = gen.draw((A, p.T, d), seed, gen.S_DOUT, "normal", "bf16")
    rng = np.random.default_rng(seed)
    L = max(lens)
    nb = (L + 127) // 128
    bias = None
    if th:
        bias = (0.5 * rng.standard_normal((th, p.T, L))).astype(np.float32)
        bias[rng.random(bias.shape) < 0.05] = -np.inf
    bk = None
    if bh:
        bk = (rng.random((len(lens), bh, nb, nb)) < 0.6).astype(np.uint8)
        for s_ in range(len(lens)):
            for h_ in range(bh):
                np.fill_diagonal(bk[s_, h_], 1)   # keep rows that see more than a key or two
    got = run_bwd_varlen(ea, p, dout, window=window, bias_np=bias, bk_np=bk)
    w = None if window is None else (window[0], 0 if causal else window[1])
    ref = orc.attn_bwd_varlen(p.q, p.k, p.v, dout, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=causal,
                              window=w, bias=bias, block_keep=bk)
    out = {n: gu.check_grad(g, r, f"{case} {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)}
    _say(out)
