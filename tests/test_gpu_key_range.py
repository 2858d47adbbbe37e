"""GPU parity of per-row key ranges (document boundaries, prefix-LM and
arbitrary intervals; page "Attention Kernel", section "可编程 mask") in every
prefill path and in the gradient, against the fp64 oracle.

Each case prints its parameters before it runs.  Ranges are drawn by
synth.gen.make_key_ranges: "document" (each row keeps its own document),
"prefix" (prefix-LM) and "random" (seeded intervals, some empty, some past the
key range on either side).
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


def ranges(B, S_q, S_k, kind, seed, **kw):
    return gen.make_key_ranges(B, S_q, S_k, kind, seed, **kw)


def run_dense(ea, p, kr, *, window=None, q_keep=None, k_keep=None, bk=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, p.dtype), gu.dev(p.k, p.dtype), gu.dev(p.v, p.dtype)
    o = gu.empty_out(q.shape, p.dtype)
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, window=window,
                key_range=None if kr is None else gu.dev(kr, "i32"),
                q_keep=None if q_keep is None else gu.dev(q_keep, "u8"),
                k_keep=None if k_keep is None else gu.dev(k_keep, "u8"),
                block_keep=None if bk is None else t.from_numpy(bk).cuda())
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


DENSE_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, kind, extra
    (2, 4, 2, 300, 300, 128, True, "document", {"doc_median": 40}),
    (1, 4, 4, 257, 257, 64, False, "document", {"doc_median": 60}),
    (2, 2, 1, 200, 333, 128, False, "random", {}),
    (1, 2, 2, 384, 384, 64, False, "prefix", {"prefix": 150}),
    (1, 4, 2, 130, 130, 128, True, "random", {}),
    (1, 2, 1, 700, 400, 64, True, "random", {}),          # S_q > S_k: leading rows at negative positions
    (1, 2, 2, 1, 1, 128, False, "prefix", {"prefix": 1}),
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: f"{c[0]}x{c[1]}:{c[2]}x{c[3]}x{c[4]}d{c[5]}"
                         + ("c" if c[6] else "n") + c[7])
def test_dense_key_ranges(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, kind, extra = case
    _say("dense key ranges", case)
    seed = 2100 + S_q + S_k + d
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=seed)
    kr = ranges(B, S_q, S_k, kind, seed, **extra)
    o, lse = run_dense(ea, p, kr)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=causal, key_range=kr)
    _say(gu.check(o, lse, o_ref, l_ref, "bf16", f"dense {case}"))


def test_dense_key_ranges_with_other_masks(ea, orc):
    """Ranges together with a window, keep masks and a block mask."""
    B, A, A_kv, S, d = 2, 4, 2, 400, 128
    _say("key ranges + window + keep masks + block mask", B, A, S, d)
    p = gen.make_dense(B, A, A_kv, S, S, d, dtype="bf16", causal=True, seed=2201, q_masked=9, k_masked=17)
    kr = ranges(B, S, S, "document", 2201, doc_median=90)
    o, lse = run_dense(ea, p, kr, window=(120, -1), q_keep=p.q_keep, k_keep=p.k_keep)
    mk = oracle.window_keep(B, S, S, 120, 0)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True, q_keep=p.q_keep,
                                k_keep=p.k_keep, m_keep=mk, key_range=kr)
    _say(gu.check(o, lse, o_ref, l_ref, "bf16", "ranges + window + keeps"))
    rng = np.random.default_rng(2202)
    bk = (rng.random((B, A, 4, 4)) < 0.7).astype(np.uint8)
    o, lse = run_dense(ea, p, kr, bk=bk)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True, key_range=kr, block_keep=bk)
    _say(gu.check(o, lse, o_ref, l_ref, "bf16", "ranges + block mask"))


@pytest.mark.parametrize("varlen", [False, True])
def test_covering_ranges_are_bitwise_neutral(ea, varlen):
    """Ranges that hold every key give the unmasked call's bits (the same tiles
    in the same order, with no per-element step on whole tiles)."""
    t = gu.torch()
    if not varlen:
        B, A, S, d = 2, 4, 333, 128
        _say("covering ranges neutral (dense)", B, A, S, d)
        p = gen.make_dense(B, A, 2, S, S, d, dtype="bf16", causal=True, seed=2301)
        kr = np.zeros((B, S, 2), np.int32)
        kr[..., 0] = -5
        kr[..., 1] = 1 << 30
        a = run_dense(ea, p, kr)
        b = run_dense(ea, p, None)
    else:
        lens = [300, 0, 77, 513]
        _say("covering ranges neutral (packed)", lens)
        p = gen.make_varlen(lens, 4, 2, 64, dtype="bf16", causal=True, seed=2302)
        kr = np.zeros((p.T, 2), np.int32)
        kr[:, 0] = -1
        kr[:, 1] = 100000
        a = run_varlen(ea, p, kr)
        b = run_varlen(ea, p, None)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_f32_key_ranges(ea, orc):
    for (B, A, S_q, S_k, d, causal, kind) in [(1, 2, 100, 100, 64, True, "document"),
                                              (2, 2, 70, 150, 33, False, "random")]:
        _say("fp32 key ranges", B, A, S_q, S_k, d, causal, kind)
        p = gen.make_dense(B, A, 1, S_q, S_k, d, dtype="f32", causal=causal, seed=2400 + d)
        kr = ranges(B, S_q, S_k, kind, 2400 + d, doc_median=20)
        o, lse = run_dense(ea, p, kr)
        o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="f32", scale=p.scale, causal=causal, key_range=kr)
        _say(gu.check(o, lse, o_ref, l_ref, "f32", f"fp32 {kind}"))


def test_fp8_key_ranges(ea, orc):
    t = gu.torch()
    B, A, A_kv, S = 2, 4, 2, 300
    _say("fp8 prefill key ranges", B, A, S)
    p = gen.make_dense_fp8(B, A, A_kv, S, S, 128, causal=True, seed=2501)
    kr = ranges(B, S, S, "document", 2501, doc_median=50)
    q, k = t.from_numpy(p.q_codes).cuda(), t.from_numpy(p.k_codes).cuda()
    v = gu.dev(p.v, "bf16")
    qs, ks = t.from_numpy(p.q_scale).cuda(), t.from_numpy(p.k_scale).cuda()
    o = t.empty((B, A, S, 128), dtype=t.bfloat16, device="cuda")
    lse = t.empty((B, A, S), dtype=t.float32, device="cuda")
    ea.attn_fwd_fp8(q, k, v, o, lse, qs, ks, scale=p.scale, causal=True, key_range=gu.dev(kr, "i32"))
    t.cuda.synchronize()
    o_ref, l_ref = orc.attn_fwd_fp8(p.q_codes, p.k_codes, p.v, p.q_scale, p.k_scale, scale=p.scale, causal=True,
                                    key_range=kr)
    _say(gu.check(gu.host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, "bf16", "fp8 ranges"))


# ---- packed sequences and paged chunks

def packed_ranges(lens, kind, seed, **kw):
    """[T, 2]: each sequence's rows with ranges over its own positions."""
    parts = [ranges(1, L, L, kind, seed + s, **kw)[0] for s, L in enumerate(lens)]
    return np.concatenate(parts).astype(np.int32) if parts else np.zeros((0, 2), np.int32)


def run_varlen(ea, p, kr, window=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, p.dtype), gu.dev(p.k, p.dtype), gu.dev(p.v, p.dtype)
    cu = gu.dev(p.cu_seqlens, "i32")
    o = gu.empty_out(q.shape, p.dtype)
    lse = t.empty((p.A, p.T), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ea.attn_fwd_varlen(q, k, v, o, lse, cu, p.cu_seqlens, scale=p.scale, causal=p.causal, window=window,
                       key_range=None if kr is None else gu.dev(kr, "i32"))
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,d,causal,kind", [("bf16", 128, True, "document"), ("bf16", 64, False, "random"),
                                                 ("bf16", 64, True, "prefix"), ("f32", 64, True, "document")])
def test_varlen_key_ranges(ea, orc, dtype, d, causal, kind):
    lens = [300, 0, 77, 513, 1, 129]
    _say("varlen key ranges", dtype, d, causal, kind, lens)
    p = gen.make_varlen(lens, 4, 2, d, dtype=dtype, causal=causal, seed=2600 + d)
    kr = packed_ranges(lens, kind, 2600, doc_median=40, prefix=100)
    o, lse = run_varlen(ea, p, kr)
    o_ref, l_ref = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype=dtype, scale=p.scale, causal=causal,
                                       key_range=kr)
    _say(gu.check(o, lse, o_ref, l_ref, dtype, f"varlen {kind}"))


def test_varlen_key_ranges_with_window(ea, orc):
    lens = [260, 31, 400]
    _say("varlen key ranges + window", lens)
    p = gen.make_varlen(lens, 4, 4, 128, dtype="bf16", causal=True, seed=2611)
    kr = packed_ranges(lens, "random", 2611)
    o, lse = run_varlen(ea, p, kr, window=(90, -1))
    o_ref, l_ref = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=True,
                                       key_range=kr, window=(90, 0))
    _say(gu.check(o, lse, o_ref, l_ref, "bf16", "varlen ranges + window"))


@pytest.mark.parametrize("d,ps", [(128, 16), (64, 32)])
def test_paged_prefill_key_ranges(ea, orc, d, ps):
    t = gu.torch()
    lens = [300, 1, 129, 700, 64, 1000]
    q_lens = [300, 1, 1, 200, 64, 129]
    _say("paged prefill key ranges", d, ps, lens, q_lens)
    pg, q, cu = gen.make_paged_prefill(lens, q_lens, 8, 2, d, ps, seed=2700 + d, extra_pages=2)
    kr = np.concatenate([ranges(1, ql, L, "document", 2700 + s, doc_median=60)[0]
                         for s, (L, ql) in enumerate(zip(lens, q_lens))]).astype(np.int32)
    qd = gu.dev(q, pg.dtype)
    kc, vc = gu.dev(pg.k_cache, pg.dtype), gu.dev(pg.v_cache, pg.dtype)
    bt, sl, cud = gu.dev(pg.block_table, "i32"), gu.dev(pg.seq_lens, "i32"), gu.dev(cu, "i32")
    o = gu.empty_out(qd.shape, pg.dtype)
    lse = t.empty((qd.shape[0], qd.shape[1]), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    ea.attn_prefill_paged_masked(qd, kc, vc, bt, sl, pg.seq_lens, cud, cu, o, lse, scale=pg.scale, causal=True,
                                 key_range=gu.dev(kr, "i32"))
    t.cuda.synchronize()
    o_ref, l_ref = orc.prefill_paged(q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, cu, dtype=pg.dtype,
                                     scale=pg.scale, causal=True, key_range=kr)
    _say(gu.check(gu.host_f64(o)[None], lse.cpu().numpy()[None].astype(np.float64), o_ref[None], l_ref[None],
                  "bf16", f"paged ranges d={d}"))


def test_documents_full_size_sampled(ea, orc):
    """The MHA causal workload's shape (B = 4, A = 32, S = 2048, d = 128) with
    packed documents (median 200 tokens) as key ranges; sampled rows against
    the oracle, and row 0 of every document equals its first value row."""
    B, A, S, d = 4, 32, 2048, 128
    _say("documents as key ranges, full size (sampled rows)", B, A, S, d)
    p = gen.make_dense(B, A, A, S, S, d, dtype="bf16", causal=True, seed=1002)
    kr = ranges(B, S, S, "document", 1002)
    o, lse = run_dense(ea, p, kr)
    rng = np.random.default_rng(2801)
    rows = np.unique(rng.choice(B * A * S, size=600, replace=False))
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True, key_range=kr, rows=rows)
    _say(gu.check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", "documents full size"))
    # a document's first row sees only itself: O equals that value row (bf16-exact)
    v = gu.host_f64(gu.dev(p.v, "bf16"))
    firsts = np.flatnonzero(kr[0, :, 0] == np.arange(S))
    for i in firsts[:20]:
        assert np.array_equal(o[0, 0, i], v[0, 0, i]), i


# ---- gradients

def run_bwd_dense(ea, p, dout, kr, bk=None):
    t = gu.torch()
    q, k, v, do = (gu.dev(x, "bf16") for x in (p.q, p.k, p.v, dout))
    krd = gu.dev(kr, "i32")
    bkd = None if bk is None else t.from_numpy(bk).cuda()
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, key_range=krd, block_keep=bkd)
    dq, dk, dv = (gu.empty_out(x.shape, "bf16") for x in (q, k, v))
    for x in (dq, dk, dv):
        x.fill_(float("nan"))
    ws = t.empty(max(ea.attn_bwd_workspace_bytes(p.B, p.A, p.S_q), 1), dtype=t.uint8, device="cuda")
    ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p.scale, causal=p.causal, key_range=krd, block_keep=bkd)
    t.cuda.synchronize()
    return gu.host_f64(dq), gu.host_f64(dk), gu.host_f64(dv)


BWD_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, kind
    (1, 4, 2, 300, 300, 128, True, "document"),
    (2, 2, 2, 257, 257, 64, True, "document"),
    (1, 2, 1, 200, 333, 128, False, "random"),
    (1, 4, 4, 384, 384, 64, False, "prefix"),
    (1, 2, 2, 130, 70, 128, True, "random"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"{c[0]}x{c[1]}:{c[2]}x{c[3]}x{c[4]}d{c[5]}"
                         + ("c" if c[6] else "n") + c[7])
def test_bwd_key_ranges(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, kind = case
    _say("bwd key ranges", case)
    seed = 2900 + S_q + S_k + d
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=seed)
    kr = ranges(B, S_q, S_k, kind, seed, doc_median=50, prefix=120)
    dout = gen.make_dout(p, seed)
    got = run_bwd_dense(ea, p, dout, kr)
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=causal, key_range=kr)
    _say({n: gu.check_grad(g, r, f"{case} {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)})


@pytest.mark.parametrize("case", [
    # B, A, A_kv, S, d, causal, window (left, right), kind
    (1, 4, 2, 320, 128, True, (100, -1), "document"),
    (2, 2, 1, 290, 64, False, (60, 40), "random"),
], ids=lambda c: f"{c[3]}d{c[4]}" + ("c" if c[5] else "n") + c[7])
def test_bwd_key_ranges_with_window_and_keeps(ea, orc, case):
    """Key ranges beside a window and both keep masks: forward and
    gradients against the oracle (the window as its keep matrix)."""
    t = gu.torch()
    B, A, A_kv, S, d, causal, window, kind = case
    _say("bwd key ranges + window + keeps", case)
    seed = 2970 + S + d
    p = gen.make_dense(B, A, A_kv, S, S, d, dtype="bf16", causal=causal, seed=seed)
    kr = ranges(B, S, S, kind, seed, doc_median=60)
    rng = np.random.default_rng(seed)
    qk = (rng.random((B, S)) > 0.1).astype(np.uint8)
    kk = (rng.random((B, S)) > 0.1).astype(np.uint8)
    dout = gen.make_dout(p, seed)
    q, k, v, do = (gu.dev(x, "bf16") for x in (p.q, p.k, p.v, dout))
    krd, qkd, kkd = gu.dev(kr, "i32"), gu.dev(qk, "u8"), gu.dev(kk, "u8")
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((B, A, S), dtype=t.float32, device="cuda")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=causal, window=window, q_keep=qkd, k_keep=kkd, key_range=krd)
    dq, dk, dv = (gu.empty_out(x.shape, "bf16") for x in (q, k, v))
    ws = t.empty(max(ea.attn_bwd_workspace_bytes(B, A, S), 1), dtype=t.uint8, device="cuda")
    ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p.scale, causal=causal, window=window, q_keep=qkd,
                k_keep=kkd, key_range=krd)
    t.cuda.synchronize()
    mk = oracle.window_keep(B, S, S, window[0], 0 if causal else window[1])
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=causal, q_keep=qk, k_keep=kk,
                                m_keep=mk, key_range=kr)
    _say(gu.check(gu.host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, "bf16", f"{case} fwd"))
    got = (gu.host_f64(dq), gu.host_f64(dk), gu.host_f64(dv))
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=causal, q_keep=qk, k_keep=kk,
                       m_keep=mk, key_range=kr)
    _say({n: gu.check_grad(g, r, f"{case} {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)})


def test_bwd_key_ranges_with_block_mask(ea, orc):
    B, A, A_kv, S, d = 1, 4, 2, 400, 128
    _say("bwd key ranges + block mask", B, A, S, d)
    p = gen.make_dense(B, A, A_kv, S, S, d, dtype="bf16", causal=True, seed=2951)
    kr = ranges(B, S, S, "document", 2951, doc_median=80)
    bk = (np.random.default_rng(2952).random((B, A, 4, 4)) < 0.7).astype(np.uint8)
    dout = gen.make_dout(p, 2951)
    got = run_bwd_dense(ea, p, dout, kr, bk)
    ref = orc.attn_bwd(p.q, p.k, p.v, dout, dtype="bf16", scale=p.scale, causal=True, key_range=kr, block_keep=bk)
    _say({n: gu.check_grad(g, r, f"ranges+blocks {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)})


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_varlen_key_ranges(ea, orc, d):
    t = gu.torch()
    lens = [300, 0, 77, 260, 1]
    _say("bwd varlen key ranges", d, lens)
    p = gen.make_varlen(lens, 4, 2, d, dtype="bf16", causal=True, seed=3000 + d)
    kr = packed_ranges(lens, "document", 3000, doc_median=40)
    dout = gen.draw((p.A, p.T, d), 3000 + d, gen.S_DOUT, "normal", "bf16")
    q, k, v, do = (gu.dev(x, "bf16") for x in (p.q, p.k, p.v, dout))
    cu, krd = gu.dev(p.cu_seqlens, "i32"), gu.dev(kr, "i32")
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.A, p.T), dtype=t.float32, device="cuda")
    ea.attn_fwd_varlen(q, k, v, o, lse, cu, p.cu_seqlens, scale=p.scale, causal=True, key_range=krd)
    dq, dk, dv = (gu.empty_out(x.shape, "bf16") for x in (q, k, v))
    ws = t.empty(max(ea.attn_bwd_workspace_bytes(1, p.A, p.T), 1), dtype=t.uint8, device="cuda")
    ea.attn_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, cu, p.cu_seqlens, ws, scale=p.scale, causal=True,
                       key_range=krd)
    t.cuda.synchronize()
    got = (gu.host_f64(dq), gu.host_f64(dk), gu.host_f64(dv))
    ref = orc.attn_bwd_varlen(p.q, p.k, p.v, dout, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=True,
                              key_range=kr)
    _say({n: gu.check_grad(g, r, f"varlen ranges {n}") for n, g, r in zip(("dq", "dk", "dv"), got, ref)})
