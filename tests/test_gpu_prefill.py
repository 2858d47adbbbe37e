"""GPU parity: prefill kernels (dense, GQA, causal, masks, varlen) vs the fp64 oracle.

Small cases are compared element by element over every row; the full-size
workloads are compared on sampled rows plus properties that hold at any size.
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


def run_dense(ea, p, q_keep=None, k_keep=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, p.dtype), gu.dev(p.k, p.dtype), gu.dev(p.v, p.dtype)
    o = gu.empty_out(q.shape, p.dtype)
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    qk = None if q_keep is None else gu.dev(q_keep, "u8")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


DENSE_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal
    (1, 1, 1, 1, 1, 128, False),
    (1, 2, 1, 17, 17, 128, True),
    (2, 4, 4, 64, 64, 128, True),
    (1, 2, 2, 65, 65, 128, True),
    (1, 2, 2, 127, 129, 128, True),
    (1, 2, 2, 129, 127, 128, True),
    (2, 8, 2, 200, 200, 128, True),
    (1, 4, 1, 300, 300, 64, True),
    (1, 3, 3, 128, 1000, 64, False),
    (1, 2, 2, 1000, 1000, 128, False),
    (2, 4, 2, 257, 384, 64, True),
    (1, 1, 1, 1, 700, 128, True),
    (1, 2, 1, 5, 0, 128, True),
    # B*A a multiple of 8: each XCD gets a contiguous block of (batch, head)
    # pairs, taken in head groups of 8 (first), 2 (with 16 query heads per KV
    # head) and 1 (three heads per XCD)
    (2, 32, 8, 200, 200, 128, True),
    (1, 16, 1, 130, 130, 128, True),
    (3, 8, 8, 150, 150, 64, True),
]


# Grids of more query tiles than one resident round of workgroups holds (512
# at d = 128, 768 at d = 64 on 256 CUs), compared over every row: with and
# without the XCD-blocked order (B*A a multiple of 8 or not), GQA, ragged row
# tiles, non-causal, and keep masks on both sides.
MULTI_ROUND_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, keep masks
    (16, 8, 2, 1024, 1024, 128, True, False),
    (4, 16, 16, 1100, 1100, 128, False, False),
    (4, 16, 4, 2048, 2048, 64, True, False),
    (12, 7, 7, 1300, 1300, 64, True, False),
    (9, 8, 4, 1000, 1030, 128, True, True),
]


@pytest.mark.parametrize("case", MULTI_ROUND_CASES,
                         ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n") + ("k" if c[7] else ""))
def test_dense_bf16_multi_round(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, keep = case
    _say("dense bf16 multi-round grid", case)
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=hash(case) % 10000)
    qk = kk = None
    if keep:
        rng = np.random.default_rng(77)
        qk = (rng.random((B, S_q)) >= 0.05).astype(np.uint8)
        kk = (rng.random((B, S_k)) >= 0.2).astype(np.uint8)
    o, lse = run_dense(ea, p, q_keep=qk, k_keep=kk)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=causal, q_keep=qk, k_keep=kk)
    gu.check(o, lse, o_ref, l_ref, "bf16", str(case))


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n"))
def test_dense_bf16_small(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal = case
    _say("dense bf16", case)
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=hash(case) % 10000)
    o, lse = run_dense(ea, p)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=causal)
    gu.check(o, lse, o_ref, l_ref, "bf16", str(case))


@pytest.mark.parametrize("case", [(1, 1, 1, 128, 128, 64, False), (2, 4, 2, 33, 70, 128, True),
                                  (1, 2, 2, 100, 100, 37, False), (1, 2, 1, 48, 16, 64, True)],
                         ids=lambda c: "x".join(map(str, c)))
def test_dense_f32_small(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal = case
    _say("dense f32", case)
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="f32", causal=causal, seed=7 + S_q)
    o, lse = run_dense(ea, p)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="f32", scale=p.scale, causal=causal)
    gu.check(o, lse, o_ref, l_ref, "f32", str(case))


def test_config1_fp32(ea, orc):
    _say("config 1 fp32 full")
    p = gen.make_config(1)
    o, lse = run_dense(ea, p)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="f32", scale=p.scale, causal=False)
    gu.check(o, lse, o_ref, l_ref, "f32", "config1")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_keep_masks(ea, orc, dtype):
    _say("keep masks", dtype)
    p = gen.make_dense(2, 4, 2, 150, 190, 128 if dtype == "bf16" else 64, dtype=dtype, causal=True, seed=31,
                       q_masked=30, k_masked=60)
    # one batch row with every key masked
    kk = p.k_keep.copy()
    kk[1, :] = 0
    o, lse = run_dense(ea, p, q_keep=p.q_keep, k_keep=kk)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype=dtype, scale=p.scale, causal=True, q_keep=p.q_keep,
                                k_keep=kk)
    assert np.all(np.isneginf(l_ref[1]))
    gu.check(o, lse, o_ref, l_ref, dtype, "keep masks")


def _sample_rows(rng, B, A, S_q, n):
    ids = rng.choice(B * A * S_q, size=n, replace=False)
    # always include the first and last row of a few heads
    extra = [(b * A + h) * S_q + i for b in range(B) for h in range(0, A, max(1, A // 4)) for i in (0, S_q - 1)]
    return np.unique(np.concatenate([ids, np.array(extra, np.int64)]))


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_configs(ea, orc, cfg):
    _say("config", cfg, "full size (sampled rows)")
    p = gen.make_config(cfg)
    o, lse = run_dense(ea, p)
    rng = np.random.default_rng(cfg)
    rows = _sample_rows(rng, p.B, p.A, p.S_q, 1500 if cfg == 2 else 600)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True, rows=rows)
    o_flat = o.reshape(-1, p.d)[rows]
    l_flat = lse.reshape(-1)[rows]
    stats = gu.check(o_flat, l_flat, o_ref, l_ref, "bf16", f"config{cfg}")
    _say("config", cfg, stats)
    # any size: outputs finite, every LSE finite (no row is masked)
    assert np.all(np.isfinite(lse)) and np.all(np.isfinite(o))
    # causal row 0 sees only key 0: O equals V[b, h_kv, 0] bit for bit
    vf = gen.as_f32(p.v, "bf16").astype(np.float64)
    G = p.A // p.A_kv
    for b in range(p.B):
        for h in range(p.A):
            assert np.array_equal(o[b, h, 0], vf[b, h // G, 0]), (b, h)


def run_varlen(ea, p, k_keep=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, p.dtype), gu.dev(p.k, p.dtype), gu.dev(p.v, p.dtype)
    o = gu.empty_out(q.shape, p.dtype)
    lse = t.empty((p.A, p.T), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    cu = gu.dev(p.cu_seqlens, "i32")
    qk = None if p.q_keep is None else gu.dev(p.q_keep, "u8")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    ea.attn_fwd_varlen(q, k, v, o, lse, cu, p.cu_seqlens, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_varlen_small(ea, orc, dtype, d):
    lens = [1, 0, 130, 17, 256, 0, 64, 300, 5]
    _say("varlen small", dtype, d, lens)
    p = gen.make_varlen(lens, 4, 2, d, dtype=dtype, causal=True, seed=41, q_mask_frac=0.05, k_mask_frac=0.1)
    o, lse = run_varlen(ea, p, k_keep=p.k_keep)
    o_ref, l_ref = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype=dtype, scale=p.scale, causal=True,
                                       q_keep=p.q_keep, k_keep=p.k_keep)
    gu.check(o, lse, o_ref, l_ref, dtype, "varlen small")


def test_varlen_noncausal_small(ea, orc):
    lens = [70, 129, 3]
    _say("varlen non-causal", lens)
    p = gen.make_varlen(lens, 2, 1, 128, dtype="bf16", causal=False, seed=43)
    o, lse = run_varlen(ea, p)
    o_ref, l_ref = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=False)
    gu.check(o, lse, o_ref, l_ref, "bf16", "varlen non-causal")


def test_config5_full(ea, orc):
    _say("config 5 varlen full size (sampled rows)")
    p = gen.make_config(5)
    o, lse = run_varlen(ea, p)
    # every query row the keep-mask drops: exactly zero output and -inf LSE, in every head
    dead = p.q_keep == 0
    assert dead.sum() == round(0.05 * p.T)
    assert np.all(o[:, dead] == 0) and np.all(np.isneginf(lse[:, dead]))
    assert np.all(np.isfinite(lse[:, ~dead]))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(p.A * p.T, size=1500, replace=False),
                                     np.nonzero(np.tile(dead, p.A))[0][:50]]))
    o_ref, l_ref = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=True,
                                       q_keep=p.q_keep, rows=rows)
    stats = gu.check(o.reshape(-1, p.d)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", "config5")
    _say("config 5", stats)


# ---- sliding windows (page "Attention Kernel", section "可编程 mask"): the
# oracle takes the window as a dense keep matrix built from its definition

def run_dense_window(ea, p, window, k_keep=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, p.dtype), gu.dev(p.k, p.dtype), gu.dev(p.v, p.dtype)
    o = gu.empty_out(q.shape, p.dtype)
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, k_keep=kk, window=window)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


WINDOW_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, (left, right)
    (1, 2, 1, 300, 300, 128, True, (0, -1)),       # each row sees only its own key
    (1, 2, 2, 300, 300, 128, True, (37, -1)),      # window inside one tile
    (2, 4, 2, 700, 700, 128, True, (255, -1)),     # several tiles, masked edges on both sides
    (1, 4, 1, 513, 700, 128, True, (100, -1)),     # S_q < S_k (bottom-right alignment)
    (1, 2, 2, 700, 400, 128, True, (64, -1)),      # S_q > S_k: leading rows see nothing
    (1, 2, 2, 600, 600, 128, False, (50, 70)),     # two-sided, non-causal
    (1, 2, 2, 600, 600, 128, False, (-1, 0)),      # right edge only = causal
    (1, 2, 2, 600, 600, 128, False, (200, -1)),    # left edge only
    (2, 4, 4, 400, 400, 64, True, (129, -1)),      # d = 64
    (1, 2, 1, 300, 300, 128, True, (5000, -1)),    # window wider than the sequence = causal
    (1, 2, 1, 300, 300, 128, True, (2147483647, -1)),   # the widest edge the header accepts (no int32 wrap)
    (1, 2, 2, 300, 260, 128, False, (-1, 2147483647)),
    (1, 2, 2, 260, 300, 64, False, (2147483647, 2147483647)),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n")
                         + f"w{c[7][0]}_{c[7][1]}")
def test_window_bf16(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, (left, right) = case
    _say("window bf16", case)
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=700 + S_q + left)
    o, lse = run_dense_window(ea, p, (left, right))
    mk = oracle.window_keep(B, S_q, S_k, left, 0 if causal else right)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=causal, m_keep=mk)
    gu.check(o, lse, o_ref, l_ref, "bf16", str(case))


def test_window_key_mask_and_f32(ea, orc):
    _say("window + key mask (bf16) and fp32 window")
    p = gen.make_dense(2, 4, 2, 333, 333, 128, dtype="bf16", causal=True, seed=771, k_masked=50)
    o, lse = run_dense_window(ea, p, (90, -1), k_keep=p.k_keep)
    mk = oracle.window_keep(2, 333, 333, 90, 0)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True, k_keep=p.k_keep, m_keep=mk)
    gu.check(o, lse, o_ref, l_ref, "bf16", "window + key mask")
    p = gen.make_dense(1, 2, 1, 150, 170, 64, dtype="f32", causal=False, seed=772)
    o, lse = run_dense_window(ea, p, (20, 9))
    mk = oracle.window_keep(1, 150, 170, 20, 9)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="f32", scale=p.scale, m_keep=mk)
    gu.check(o, lse, o_ref, l_ref, "f32", "fp32 window")


def test_window_varlen(ea, orc):
    lens = [1, 0, 130, 17, 400, 64, 300]
    left = 70
    _say("varlen window", lens, left)
    p = gen.make_varlen(lens, 4, 2, 128, dtype="bf16", causal=True, seed=773)
    t = gu.torch()
    q, k, v = gu.dev(p.q, "bf16"), gu.dev(p.k, "bf16"), gu.dev(p.v, "bf16")
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.A, p.T), dtype=t.float32, device="cuda")
    cu = gu.dev(p.cu_seqlens, "i32")
    ea.attn_fwd_varlen(q, k, v, o, lse, cu, p.cu_seqlens, scale=p.scale, causal=True, window=(left, -1))
    t.cuda.synchronize()
    o, lse = gu.host_f64(o), lse.cpu().numpy().astype(np.float64)
    # a packed sequence is an independent dense problem (pinned for the oracle)
    for s in range(len(lens)):
        a, b = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
        if a == b:
            continue
        L = b - a
        mk = oracle.window_keep(1, L, L, left, 0)
        o_ref, l_ref = orc.attn_fwd(p.q[None, :, a:b], p.k[None, :, a:b], p.v[None, :, a:b], dtype="bf16",
                                    scale=p.scale, causal=True, m_keep=mk)
        gu.check(o[None, :, a:b], lse[None, :, a:b], o_ref, l_ref, "bf16", f"varlen window seq {s}")


def test_window_full_size_sampled(ea, orc):
    """The MHA workload's shape with a 512-key causal window, sampled rows."""
    _say("window full size 4x32x2048x128, left 511")
    p = gen.make_dense(4, 32, 32, 2048, 2048, 128, dtype="bf16", causal=True, seed=774)
    o, lse = run_dense_window(ea, p, (511, -1))
    rng = np.random.default_rng(774)
    rows = _sample_rows(rng, p.B, p.A, p.S_q, 1000)
    mk = oracle.window_keep(p.B, p.S_q, p.S_k, 511, 0)
    o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True, m_keep=mk, rows=rows)
    stats = gu.check(o.reshape(-1, p.d)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", "window full size")
    _say(stats)
    assert np.all(np.isfinite(lse)) and np.all(np.isfinite(o))


# ---- prefill of query chunks over a paged KV cache, mixing prefill chunks
# and single-row decode steps in one call (the reference gathers each
# sequence's tokens through the block table and runs the dense oracle with the
# bottom-right causal alignment)

def run_paged_prefill(ea, pg, q, cu, window=None, causal=True):
    t = gu.torch()
    qd = gu.dev(q, pg.dtype)
    kc, vc = gu.dev(pg.k_cache, pg.dtype), gu.dev(pg.v_cache, pg.dtype)
    bt, sl, cud = gu.dev(pg.block_table, "i32"), gu.dev(pg.seq_lens, "i32"), gu.dev(cu, "i32")
    o = gu.empty_out(qd.shape, pg.dtype)
    lse = t.empty((qd.shape[0], qd.shape[1]), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ea.attn_prefill_paged(qd, kc, vc, bt, sl, pg.seq_lens, cud, cu, o, lse, scale=pg.scale, causal=causal,
                          window=window)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


def check_paged_prefill(orc, pg, q, cu, o, lse, what, window=None, causal=True):
    w = None if window is None else (window[0], 0 if causal else window[1])
    o_ref, l_ref = orc.prefill_paged(q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, cu, dtype=pg.dtype,
                                     scale=pg.scale, causal=causal, window=w)
    gu.check(o[None], lse[None], o_ref[None], l_ref[None], pg.dtype, what)


@pytest.mark.parametrize("d,ps", [(128, 16), (128, 64), (64, 32)])
def test_paged_prefill_mixed(ea, orc, d, ps):
    lens = [300, 1, 129, 700, 64, 5, 1000, 17]       # KV length per sequence (chunk included)
    q_lens = [300, 1, 1, 200, 64, 5, 129, 0]         # full prefill, decode rows, chunks, an empty chunk
    _say("paged prefill", d, ps, lens, q_lens)
    pg, q, cu = gen.make_paged_prefill(lens, q_lens, 8, 2, d, ps, seed=900 + d + ps, extra_pages=3)
    o, lse = run_paged_prefill(ea, pg, q, cu)
    check_paged_prefill(orc, pg, q, cu, o, lse, f"paged d={d} ps={ps}")


def test_paged_prefill_window_and_noncausal(ea, orc):
    lens = [400, 260, 33]
    q_lens = [150, 260, 3]
    _say("paged prefill window / non-causal", lens, q_lens)
    pg, q, cu = gen.make_paged_prefill(lens, q_lens, 4, 4, 128, 16, seed=931)
    o, lse = run_paged_prefill(ea, pg, q, cu, window=(77, -1))
    check_paged_prefill(orc, pg, q, cu, o, lse, "paged window", window=(77, -1))
    o, lse = run_paged_prefill(ea, pg, q, cu, causal=False)
    check_paged_prefill(orc, pg, q, cu, o, lse, "paged non-causal", causal=False)


def run_paged_prefill_fp8(ea, pf, q, cu, window=None, causal=True):
    t = gu.torch()
    p = pf.base
    qd = gu.dev(q, "bf16")
    kc, vc = t.from_numpy(pf.k_codes).cuda(), t.from_numpy(pf.v_codes).cuda()
    ks, vs = t.from_numpy(pf.k_scale).cuda(), t.from_numpy(pf.v_scale).cuda()
    bt, sl, cud = gu.dev(p.block_table, "i32"), gu.dev(p.seq_lens, "i32"), gu.dev(cu, "i32")
    o = gu.empty_out(qd.shape, "bf16")
    lse = t.empty((qd.shape[0], qd.shape[1]), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ea.attn_prefill_paged_fp8(qd, kc, vc, ks, vs, bt, sl, p.seq_lens, cud, cu, o, lse, scale=p.scale, causal=causal,
                              window=window)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d,ps", [(128, 16), (128, 64), (64, 32)])
def test_paged_prefill_fp8_cache(ea, orc, d, ps):
    """Prefill chunks and decode rows over E4M3 caches with per-(page, KV head)
    scales; causal, then a window and non-causal (the bf16 tolerances: the
    codes widen exactly and the scales stay fp32)."""
    lens = [300, 1, 129, 700, 64, 5, 1000, 17]
    q_lens = [300, 1, 1, 200, 64, 5, 129, 0]
    _say("paged prefill fp8 cache", d, ps)
    pf, q, cu = gen.make_paged_prefill_fp8(lens, q_lens, 8, 2, d, ps, seed=1900 + d + ps, extra_pages=3)
    p = pf.base
    for causal, window in ((True, None), (True, (77, -1)), (False, None)):
        o, lse = run_paged_prefill_fp8(ea, pf, q, cu, window=window, causal=causal)
        w = None if window is None else (window[0], 0 if causal else window[1])
        o_ref, l_ref = orc.prefill_paged_fp8(q, pf.k_codes, pf.v_codes, pf.k_scale, pf.v_scale, p.block_table,
                                             p.seq_lens, cu, scale=p.scale, causal=causal, window=w)
        _say(gu.check(o[None], lse[None], o_ref[None], l_ref[None], "bf16", f"fp8 cache d={d} ps={ps} {causal} {window}"))


def test_paged_prefill_fp8_cache_full_size_sampled(ea, orc):
    """The decode workload's FP8 cache (64 sequences, lengths ~U{512..32768},
    A = 32, A_kv = 8, page 16) with each sequence's last 256 tokens as the
    chunk: sampled rows against the oracle, all outputs finite."""
    lens = gen.make_config(4).seq_lens
    q_lens = np.full(lens.size, 256, np.int32)
    _say("paged prefill fp8 cache full size", int(lens.sum()))
    pf, q, cu = gen.make_paged_prefill_fp8(lens, q_lens, 32, 8, 128, 16, seed=1950)
    o, lse = run_paged_prefill_fp8(ea, pf, q, cu)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(1951)
    rows = np.unique(rng.integers(0, 32 * int(cu[-1]), size=300))
    o_ref, l_ref = orc.prefill_paged_fp8(q, pf.k_codes, pf.v_codes, pf.k_scale, pf.v_scale, pf.base.block_table,
                                         lens, cu, scale=pf.base.scale, rows=rows)
    _say(gu.check(o.reshape(-1, 128)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", "fp8 cache full size"))


def test_paged_prefill_equals_varlen_bitwise(ea):
    """With identity pages and the whole sequence as the chunk, the paged call
    computes exactly the packed varlen prefill (same tiles, same order)."""
    t = gu.torch()
    lens = [256, 77, 513]
    _say("paged == varlen", lens)
    pv = gen.make_varlen(lens, 4, 2, 128, dtype="bf16", causal=True, seed=932)
    ps = 16
    npg = [(L + ps - 1) // ps for L in lens]
    pool = sum(npg)
    kc = np.zeros((pool, ps, 2, 128), np.uint16)
    vc = np.zeros_like(kc)
    bt = np.full((len(lens), max(npg)), -1, np.int32)
    page = 0
    for s, L in enumerate(lens):
        a = int(pv.cu_seqlens[s])
        for j in range(npg[s]):
            n = min(ps, L - j * ps)
            kc[page, :n] = pv.k[:, a + j * ps: a + j * ps + n].transpose(1, 0, 2)
            vc[page, :n] = pv.v[:, a + j * ps: a + j * ps + n].transpose(1, 0, 2)
            bt[s, j] = page
            page += 1
    qd = gu.dev(pv.q, "bf16")
    o1 = gu.empty_out(qd.shape, "bf16")
    l1 = t.empty((4, pv.T), dtype=t.float32, device="cuda")
    cu = gu.dev(pv.cu_seqlens, "i32")
    ea.attn_fwd_varlen(qd, gu.dev(pv.k, "bf16"), gu.dev(pv.v, "bf16"), o1, l1, cu, pv.cu_seqlens, scale=pv.scale,
                       causal=True)
    o2 = gu.empty_out(qd.shape, "bf16")
    l2 = t.empty((4, pv.T), dtype=t.float32, device="cuda")
    sl = np.array(lens, np.int32)
    ea.attn_prefill_paged(qd, gu.dev(kc, "bf16"), gu.dev(vc, "bf16"), gu.dev(bt, "i32"), gu.dev(sl, "i32"), sl,
                          cu, pv.cu_seqlens, o2, l2, scale=pv.scale, causal=True)
    t.cuda.synchronize()
    assert t.equal(o1.view(t.int16), o2.view(t.int16)) and t.equal(l1, l2)


# ---- block sparsity (page "Attention Kernel", section "可编程 mask"): the
# oracle receives the block mask expanded to the dense keep matrix it defines

def run_block_sparse(ea, p, bk, window=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, "bf16"), gu.dev(p.k, "bf16"), gu.dev(p.v, "bf16")
    o = gu.empty_out(q.shape, "bf16")
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, window=window, block_keep=gu.dev(bk, "u8"))
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


def check_block_sparse(orc, p, bk, o, lse, what, window=None, heads=None):
    mk = None
    if window is not None:
        mk = oracle.window_keep(p.B, p.S_q, p.S_k, window[0], 0 if p.causal else window[1])
    if heads is None:
        o_ref, l_ref = orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=p.causal, m_keep=mk,
                                    block_keep=bk)
        gu.check(o, lse, o_ref, l_ref, "bf16", what)
        return
    G = p.A // p.A_kv
    for h in heads:
        hm = 0 if bk.shape[1] == 1 else h
        o_ref, l_ref = orc.attn_fwd(p.q[:, h:h + 1], p.k[:, h // G:h // G + 1], p.v[:, h // G:h // G + 1],
                                    dtype="bf16", scale=p.scale, causal=p.causal, m_keep=mk,
                                    block_keep=bk[:, hm:hm + 1])
        gu.check(o[:, h:h + 1], lse[:, h:h + 1], o_ref, l_ref, "bf16", f"{what} head {h}")


BLOCK_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, block_heads, density, window
    (2, 4, 2, 700, 700, 128, True, 1, 0.5, None),
    (1, 4, 4, 513, 900, 128, False, 4, 0.4, None),     # a different mask per head, ragged sizes
    (1, 2, 1, 640, 640, 64, True, 2, 0.6, None),
    (1, 2, 2, 600, 600, 128, True, 1, 0.7, (200, -1)),  # with a sliding window
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n")
                         + f"h{c[7]}d{c[8]}" + ("w" if c[9] else ""))
def test_block_sparse(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, bh, dens, window = case
    _say("block sparse", case)
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=950 + S_q)
    rng = np.random.default_rng(S_q + S_k)
    bk = (rng.random((B, bh, (S_q + 127) // 128, (S_k + 127) // 128)) < dens).astype(np.uint8)
    bk[0, 0, 1, :] = 0                                   # a row block with every block off
    o, lse = run_block_sparse(ea, p, bk, window)
    check_block_sparse(orc, p, bk, o, lse, str(case), window)


def test_block_sparse_all_on_equals_dense_bitwise(ea):
    """Every block kept: the listed tiles are the plain tile range in the same
    order, so the output equals the plain causal call bit for bit."""
    t = gu.torch()
    p = gen.make_dense(1, 4, 2, 777, 777, 128, dtype="bf16", causal=True, seed=960)
    q, k, v = gu.dev(p.q, "bf16"), gu.dev(p.k, "bf16"), gu.dev(p.v, "bf16")
    o1, o2 = gu.empty_out(q.shape, "bf16"), gu.empty_out(q.shape, "bf16")
    l1 = t.empty((1, 4, 777), dtype=t.float32, device="cuda")
    l2 = t.empty_like(l1)
    ea.attn_fwd(q, k, v, o1, l1, scale=p.scale, causal=True)
    bk = t.ones((1, 1, 7, 7), dtype=t.uint8, device="cuda")
    ea.attn_fwd(q, k, v, o2, l2, scale=p.scale, causal=True, block_keep=bk)
    t.cuda.synchronize()
    assert t.equal(o1.view(t.int16), o2.view(t.int16)) and t.equal(l1, l2)


def test_block_sparse_full_size_sampled(ea, orc):
    """The MHA workload's shape, causal, half of the blocks kept (per batch row),
    sampled heads against the oracle."""
    p = gen.make_dense(4, 32, 32, 2048, 2048, 128, dtype="bf16", causal=True, seed=961)
    rng = np.random.default_rng(961)
    bk = (rng.random((4, 1, 16, 16)) < 0.5).astype(np.uint8)
    _say("block sparse full size", int(bk.sum()), "blocks kept")
    o, lse = run_block_sparse(ea, p, bk)
    # a row is empty when no kept block of its row block reaches the causal diagonal
    kept_upto = np.array([[[bk[b, 0, i // 128, :(i // 128) + 1].any()] for i in range(2048)] for b in range(4)])[..., 0]
    assert np.all(np.isneginf(lse[~kept_upto[:, None, :].repeat(32, 1)]))
    check_block_sparse(orc, p, bk, o, lse, "block sparse full size", heads=[0, 17, 31])


# ---- general dense additive mask M (page "Attention Kernel", section "可编程
# mask"): fp32 [B, 1 or A, S_q, S_k], alone or with the flag masks, windows and
# the block mask attn_block_keep_from_bias derives from it

def run_bias(ea, p, bias_np, *, window=None, blocks=False, q_keep=None, k_keep=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, p.dtype), gu.dev(p.k, p.dtype), gu.dev(p.v, p.dtype)
    o = gu.empty_out(q.shape, p.dtype)
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    bias = ea.pad_bias(t.from_numpy(bias_np).cuda())
    bk = None
    if blocks:
        bk = t.full((p.B, bias_np.shape[1], (p.S_q + 127) // 128, (p.S_k + 127) // 128), 7, dtype=t.uint8,
                    device="cuda")
        ea.attn_block_keep_from_bias(bias, bk)
    qk = None if q_keep is None else gu.dev(q_keep, "u8")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk, window=window,
                block_keep=bk, bias=bias)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64), None if bk is None else bk.cpu().numpy()


def bias_oracle(orc, p, bias_np, *, window=None, q_keep=None, k_keep=None, rows=None):
    mk = None
    if window is not None:
        mk = oracle.window_keep(p.B, p.S_q, p.S_k, window[0], 0 if p.causal else window[1])
    return orc.attn_fwd(p.q, p.k, p.v, dtype=p.dtype, scale=p.scale, causal=p.causal, q_keep=q_keep,
                        k_keep=k_keep, m_keep=mk, bias=bias_np, rows=rows)


BIAS_CASES = [
    # B, A, A_kv, S_q, S_k, d, causal, window, heads, kind, blocks, keep masks
    (2, 4, 2, 300, 300, 128, True, None, 1, "document", True, False),
    (1, 4, 4, 257, 390, 64, False, None, 4, "alibi", False, False),
    (2, 2, 1, 200, 333, 128, True, None, 2, "random", True, True),
    (1, 2, 2, 130, 130, 128, True, (40, -1), 1, "random", False, False),
    (1, 8, 2, 500, 500, 64, True, None, 1, "document", True, True),
    (2, 2, 2, 1, 70, 128, False, None, 1, "random", False, False),
    (1, 2, 1, 64, 1000, 128, False, (100, 100), 2, "alibi", True, False),
]


@pytest.mark.parametrize("case", BIAS_CASES, ids=lambda c: "x".join(map(str, c[:6])) + ("c" if c[6] else "n")
                         + f"_{c[9]}{c[8]}" + ("_blk" if c[10] else "") + ("_keep" if c[11] else "")
                         + ("" if c[7] is None else f"_w{c[7][0]}_{c[7][1]}"))
def test_bias_bf16(ea, orc, case):
    B, A, A_kv, S_q, S_k, d, causal, window, heads, kind, blocks, keeps = case
    _say("dense additive mask", case)
    seed = 1100 + S_q + S_k
    p = gen.make_dense(B, A, A_kv, S_q, S_k, d, dtype="bf16", causal=causal, seed=seed,
                       q_masked=S_q // 10 if keeps else 0, k_masked=S_k // 8 if keeps else 0)
    bias = gen.make_bias(B, heads, S_q, S_k, kind, seed)
    qk = p.q_keep if keeps else None
    kk = p.k_keep if keeps else None
    o, lse, bk = run_bias(ea, p, bias, window=window, blocks=blocks, q_keep=qk, k_keep=kk)
    if blocks:
        assert np.array_equal(bk, orc.block_keep_of_bias(bias))
    o_ref, l_ref = bias_oracle(orc, p, bias, window=window, q_keep=qk, k_keep=kk)
    _say(gu.check(o, lse, o_ref, l_ref, "bf16", str(case)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bias_fill_value_rows(ea, orc, dtype):
    """Rows of the additive term filled with the float32 minimum (the usual
    fill value of additive masks) are fully masked: O = 0, LSE = -inf; a row
    with the fill value everywhere but one key sees that key alone; other rows
    mix the fill value with finite terms."""
    d = 128 if dtype == "bf16" else 64
    p = gen.make_dense(1, 2, 1, 150, 200, d, dtype=dtype, causal=False, seed=1210)
    bias = gen.make_bias(1, 2, 150, 200, "random", 1210)
    fmin = np.finfo(np.float32).min
    bias[0, 0, 3, :] = fmin
    bias[0, 1, 7:20, :] = fmin
    bias[0, 1, 9, 55] = 0.0
    bias[0, 0, 40:, 100:] = fmin
    _say("fill value rows", dtype)
    o, lse, _ = run_bias(ea, p, bias)
    o_ref, l_ref = bias_oracle(orc, p, bias)
    assert np.all(o[0, 0, 3] == 0) and np.isneginf(lse[0, 0, 3]) and np.isneginf(lse[0, 1, 8])
    _say(gu.check(o, lse, o_ref, l_ref, dtype, f"fill value rows {dtype}"))


def test_bias_f32(ea, orc):
    """The fp32 path with a per-head distance penalty (the single-head fp32
    workload's shape) and with a random term plus keep masks on a ragged shape."""
    p = gen.make_config(1)
    bias = gen.make_bias(p.B, p.A, p.S_q, p.S_k, "alibi", 1200)
    o, lse, _ = run_bias(ea, p, bias)
    o_ref, l_ref = bias_oracle(orc, p, bias)
    _say("f32 alibi", gu.check(o, lse, o_ref, l_ref, "f32", "f32 alibi"))
    p = gen.make_dense(2, 3, 1, 45, 77, 40, dtype="f32", causal=True, seed=1201, q_masked=4, k_masked=9)
    bias = gen.make_bias(2, 1, 45, 77, "random", 1201)
    o, lse, _ = run_bias(ea, p, bias, q_keep=p.q_keep, k_keep=p.k_keep)
    o_ref, l_ref = bias_oracle(orc, p, bias, q_keep=p.q_keep, k_keep=p.k_keep)
    _say("f32 random", gu.check(o, lse, o_ref, l_ref, "f32", "f32 random"))


def test_bias_block_skip_bitwise(ea):
    """The block mask derived from the bias skips only tiles the bias masks
    whole: with and without it the outputs agree bit for bit."""
    t = gu.torch()
    p = gen.make_dense(2, 4, 2, 700, 900, 128, dtype="bf16", causal=True, seed=1202)
    bias_np = gen.make_bias(2, 1, 700, 900, "document", 1202, doc_median=150)
    q, k, v = gu.dev(p.q, "bf16"), gu.dev(p.k, "bf16"), gu.dev(p.v, "bf16")
    bias = ea.pad_bias(t.from_numpy(bias_np).cuda())
    bk = t.empty((2, 1, 6, 8), dtype=t.uint8, device="cuda")
    ea.attn_block_keep_from_bias(bias, bk)
    o1, o2 = gu.empty_out(q.shape, "bf16"), gu.empty_out(q.shape, "bf16")
    l1 = t.empty((2, 4, 700), dtype=t.float32, device="cuda")
    l2 = t.empty_like(l1)
    ea.attn_fwd(q, k, v, o1, l1, scale=p.scale, causal=True, bias=bias)
    ea.attn_fwd(q, k, v, o2, l2, scale=p.scale, causal=True, bias=bias, block_keep=bk)
    t.cuda.synchronize()
    kept = int(bk.sum().item())
    _say("blocks kept", kept, "of", bk.numel())
    assert kept < bk.numel()
    assert t.equal(o1.view(t.int16), o2.view(t.int16)) and t.equal(l1, l2)


# More dense-term shapes without block or key masks: one, two and three key
# tiles, long key ranges, rows and keys past the last full tile, shared and
# per-head terms, GQA and windows.
TERM_CASES = [
    # B, A, A_kv, S_q, S_k, causal, window, heads, kind
    (1, 4, 4, 1000, 1000, True, None, 4, "alibi"),
    (2, 4, 1, 300, 777, False, None, 1, "random"),
    (1, 2, 2, 129, 50, False, None, 2, "random"),
    (1, 2, 2, 64, 130, True, None, 2, "random"),
    (1, 2, 2, 100, 190, False, None, 1, "alibi"),
    (1, 2, 1, 700, 1300, True, (200, -1), 2, "alibi"),
    (1, 2, 2, 256, 640, False, (100, 100), 1, "random"),
]


@pytest.mark.parametrize("case", TERM_CASES, ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else "n")
                         + f"_{c[8]}{c[7]}" + ("" if c[6] is None else f"_w{c[6][0]}_{c[6][1]}"))
def test_bias_shapes(ea, orc, case):
    B, A, A_kv, S_q, S_k, causal, window, heads, kind = case
    _say("dense additive term", case)
    seed = 1400 + S_q + S_k
    p = gen.make_dense(B, A, A_kv, S_q, S_k, 128, dtype="bf16", causal=causal, seed=seed)
    bias = gen.make_bias(B, heads, S_q, S_k, kind, seed)
    o, lse, _ = run_bias(ea, p, bias, window=window)
    o_ref, l_ref = bias_oracle(orc, p, bias, window=window)
    _say(gu.check(o, lse, o_ref, l_ref, "bf16", str(case)))


@pytest.mark.parametrize("shape", [(1, 4, 2, 300, 512), (2, 2, 2, 128, 1024), (1, 2, 1, 77, 64)])
def test_bias_all_kept_key_mask_bitwise(ea, shape):
    """A key mask that keeps every key changes nothing: non-causal with whole
    key tiles, the call with it (every tile through the masked body) and the
    call without it (every tile predicate-free) visit the tiles in the same
    order and agree bit for bit."""
    t = gu.torch()
    B, A, A_kv, S_q, S_k = shape
    p = gen.make_dense(B, A, A_kv, S_q, S_k, 128, dtype="bf16", causal=False, seed=1450 + S_k)
    bias = ea.pad_bias(t.from_numpy(gen.make_bias(B, A, S_q, S_k, "random", 1450 + S_k)).cuda())
    q, k, v = gu.dev(p.q, "bf16"), gu.dev(p.k, "bf16"), gu.dev(p.v, "bf16")
    ones = t.ones((B, S_k), dtype=t.uint8, device="cuda")
    o1, o2 = gu.empty_out(q.shape, "bf16"), gu.empty_out(q.shape, "bf16")
    l1 = t.empty((B, A, S_q), dtype=t.float32, device="cuda")
    l2 = t.empty_like(l1)
    _say("all-kept key mask bitwise", shape)
    ea.attn_fwd(q, k, v, o1, l1, scale=p.scale, causal=False, bias=bias)
    ea.attn_fwd(q, k, v, o2, l2, scale=p.scale, causal=False, bias=bias, k_keep=ones)
    t.cuda.synchronize()
    assert t.equal(o1.view(t.int16), o2.view(t.int16))
    assert t.equal(l1.isneginf(), l2.isneginf())
    fin = l1.isfinite()
    assert t.equal(l1[fin], l2[fin])


def test_bias_penalty_full_size_sampled(ea, orc):
    """The MHA workload's shape, causal, with a per-head distance penalty
    [4, 32, 2048, 2048] (the timed additive-term launch), sampled rows against
    the oracle."""
    p = gen.make_config(2)
    bias = gen.make_bias(p.B, p.A, p.S_q, p.S_k, "alibi", 1460)
    _say("per-head penalty full size")
    o, lse, _ = run_bias(ea, p, bias)
    rng = np.random.default_rng(1460)
    rows = _sample_rows(rng, p.B, p.A, p.S_q, 1200)
    o_ref, l_ref = bias_oracle(orc, p, bias, rows=rows)
    _say("per-head penalty full size",
         gu.check(o.reshape(-1, p.d)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", "penalty full size"))


def test_bias_full_size_sampled(ea, orc):
    """The MHA workload's shape, causal, with a packed-document mask given as
    the additive term (and its block mask), sampled rows against the oracle."""
    p = gen.make_config(2)
    bias = gen.make_bias(p.B, 1, p.S_q, p.S_k, "document", 1203)
    o, lse, bk = run_bias(ea, p, bias, blocks=True)
    assert np.array_equal(bk, orc.block_keep_of_bias(bias))
    rng = np.random.default_rng(1203)
    rows = _sample_rows(rng, p.B, p.A, p.S_q, 1200)
    o_ref, l_ref = bias_oracle(orc, p, bias, rows=rows)
    _say("bias full size", int(bk.sum()), "blocks kept",
         gu.check(o.reshape(-1, p.d)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", "bias full size"))


def test_block_sparse_longest_key_range(ea, orc):
    """The largest key range a block mask accepts (S_k = 262144: 4096 listed
    64-key tiles per workgroup at most), non-causal, one block in ten kept per
    row block; every row checked against the oracle."""
    S_q, S_k = 200, 262144
    p = gen.make_dense(1, 2, 1, S_q, S_k, 128, dtype="bf16", causal=False, seed=1300)
    rng = np.random.default_rng(1300)
    bk = (rng.random((1, 1, 2, S_k // 128)) < 0.1).astype(np.uint8)
    bk[0, 0, 0, -1] = 1                                   # the last block of the range
    bk[0, 0, 1, :] = 0                                    # a row block with nothing kept
    _say("block sparse longest range", int(bk.sum()), "blocks kept")
    o, lse = run_block_sparse(ea, p, bk)
    assert np.all(np.isneginf(lse[:, :, 128:])) and np.all(o[:, :, 128:] == 0)
    check_block_sparse(orc, p, bk, o, lse, "block sparse longest range")


# ---------------------------------------------------------------- packed sequences with block masks and terms
def _varlen_term(rng, A_heads, T, L, p_inf=0.1):
    """fp32 [heads, T, L] term: N(0, 1/2) with a fraction of -inf entries."""
    b = (0.5 * rng.standard_normal((A_heads, T, L))).astype(np.float32)
    b[rng.random(b.shape) < p_inf] = -np.inf
    return b


def run_varlen_masks(ea, p, *, bias_np=None, bk_np=None, window=None, k_keep=None):
    t = gu.torch()
    q, k, v = gu.dev(p.q, p.dtype), gu.dev(p.k, p.dtype), gu.dev(p.v, p.dtype)
    o = gu.empty_out(q.shape, p.dtype)
    lse = t.empty((p.A, p.T), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    cu = gu.dev(p.cu_seqlens, "i32")
    bias = None
    if bias_np is not None:
        H, T, L = bias_np.shape
        ld = max(4, (L + 3) // 4 * 4)
        full = t.full((H, T, ld), float("nan"), dtype=t.float32, device="cuda")   # padding is never used
        full[..., :L] = t.from_numpy(bias_np).cuda()
        bias = full[..., :L]
    bk = None if bk_np is None else t.from_numpy(bk_np).cuda()
    qk = None if p.q_keep is None else gu.dev(p.q_keep, "u8")
    kk = None if k_keep is None else gu.dev(k_keep, "u8")
    ea.attn_fwd_varlen(q, k, v, o, lse, cu, p.cu_seqlens, scale=p.scale, causal=p.causal, q_keep=qk, k_keep=kk,
                       window=window, block_keep=bk, bias=bias)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


VARLEN_MASK_CASES = [
    # lens, A, A_kv, d, causal, window, term heads (0 = none), block heads (0 = none), keep masks
    ([1, 0, 130, 17, 256, 0, 64, 300, 5], 4, 2, 128, True, None, 1, 0, False),
    ([300, 129, 7], 4, 4, 64, False, None, 4, 4, True),
    ([500, 40, 260], 8, 2, 128, True, (100, -1), 0, 1, False),
    ([257, 0, 513], 2, 1, 128, True, None, 2, 2, True),
    ([70, 700], 4, 2, 64, True, None, 1, 1, False),
    ([129, 384, 1], 4, 1, 128, False, (60, 30), 1, 0, False),
]


@pytest.mark.parametrize("case", VARLEN_MASK_CASES,
                         ids=lambda c: f"{len(c[0])}seq-A{c[1]}-kv{c[2]}-d{c[3]}-{'c' if c[4] else 'n'}"
                                       f"-t{c[6]}-b{c[7]}" + ("-keep" if c[8] else "")
                                       + ("" if c[5] is None else f"-w{c[5][0]}_{c[5][1]}"))
def test_varlen_block_mask_and_term(ea, orc, case):
    """Packed sequences with per-sequence block masks [n_seq, heads, nb, nb] and
    per-token terms [heads, T, longest] ("Attention Kernel", 可编程 mask, over
    the ragged batches of Paged 与 ragged KV) against the oracle."""
    lens, A, A_kv, d, causal, window, th, bh, keeps = case
    _say("varlen block mask + term", case)
    p = gen.make_varlen(lens, A, A_kv, d, dtype="bf16", causal=causal, seed=sum(lens) + A,
                        q_mask_frac=0.05 if keeps else 0.0, k_mask_frac=0.1 if keeps else 0.0)
    rng = np.random.default_rng(sum(lens) + 7)
    L = max(lens)
    nb = (L + 127) // 128
    bias = _varlen_term(rng, th, p.T, L) if th else None
    if bias is not None and th == 1:
        bias[0, int(p.cu_seqlens[np.argmax(lens)]) + 3, :] = np.finfo(np.float32).min   # a fully filled row
    bk = (rng.random((len(lens), bh, nb, nb)) < 0.6).astype(np.uint8) if bh else None
    k_keep = p.k_keep if keeps else None
    o, lse = run_varlen_masks(ea, p, bias_np=bias, bk_np=bk, window=window, k_keep=k_keep)
    o_ref, l_ref = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=causal,
                                       q_keep=p.q_keep, k_keep=k_keep, bias=bias, block_keep=bk, window=window)
    gu.check(o, lse, o_ref, l_ref, "bf16", str(case))


def test_varlen_masks_one_sequence_is_dense_bitwise(ea):
    """One packed sequence with a block mask and a term gives the dense call's
    bits (same arithmetic; only the workgroup-to-tile map differs)."""
    t = gu.torch()
    L, A, A_kv, d = 333, 4, 2, 128
    _say("varlen masks one sequence == dense", L)
    p = gen.make_varlen([L], A, A_kv, d, dtype="bf16", causal=True, seed=511)
    rng = np.random.default_rng(512)
    bias = _varlen_term(rng, A, L, L)
    bk = (rng.random((1, A, 3, 3)) < 0.7).astype(np.uint8)
    o1, l1 = run_varlen_masks(ea, p, bias_np=bias, bk_np=bk)
    q = gu.dev(p.q, "bf16")[None]
    k = gu.dev(p.k, "bf16")[None]
    v = gu.dev(p.v, "bf16")[None]
    o = t.empty_like(q)
    lse = t.empty((1, A, L), dtype=t.float32, device="cuda")
    ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=True, bias=ea.pad_bias(t.from_numpy(bias[None]).cuda()),
                block_keep=t.from_numpy(bk).cuda())
    t.cuda.synchronize()
    assert np.array_equal(o1, gu.host_f64(o)[0]) and np.array_equal(l1, lse.cpu().numpy()[0].astype(np.float64))


def test_config5_block_mask_full_size_sampled(ea, orc):
    """The varlen workload (16 sequences, A = 16, d = 64) with a seeded block
    mask per sequence and a per-token term shared by the heads; sampled rows."""
    _say("config 5 with block mask and term (sampled rows)")
    p = gen.make_config(5)
    rng = np.random.default_rng(555)
    L = int(np.diff(p.cu_seqlens).max())
    nb = (L + 127) // 128
    bk = (rng.random((p.n_seq, 1, nb, nb)) < 0.5).astype(np.uint8)
    for s in range(p.n_seq):
        np.fill_diagonal(bk[s, 0], 1)
    bias = _varlen_term(rng, 1, p.T, L, p_inf=0.05)
    o, lse = run_varlen_masks(ea, p, bias_np=bias, bk_np=bk)
    rows = np.unique(np.concatenate([rng.choice(p.A * p.T, size=300, replace=False),
                                     [int(p.cu_seqlens[-1]) - 1, p.T + int(p.cu_seqlens[1])]]))
    o_ref, l_ref = orc.attn_fwd_varlen(p.q, p.k, p.v, p.cu_seqlens, dtype="bf16", scale=p.scale, causal=True,
                                       q_keep=p.q_keep, bias=bias, block_keep=bk, rows=rows)
    stats = gu.check(o.reshape(-1, p.d)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", "config5 masks")
    _say("config 5 masks", stats)


# ---------------------------------------------------------------- paged chunks with block masks and terms
def run_paged_masked(ea, pg, q, cu, *, bias_np=None, bk_np=None, window=None, causal=True):
    t = gu.torch()
    qd = gu.dev(q, pg.dtype)
    kc, vc = gu.dev(pg.k_cache, pg.dtype), gu.dev(pg.v_cache, pg.dtype)
    bt, sl, cud = gu.dev(pg.block_table, "i32"), gu.dev(pg.seq_lens, "i32"), gu.dev(cu, "i32")
    o = gu.empty_out(qd.shape, pg.dtype)
    lse = t.empty((qd.shape[0], qd.shape[1]), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    bias = None
    if bias_np is not None:
        H, T, L = bias_np.shape
        ld = max(4, (L + 3) // 4 * 4)
        full = t.full((H, T, ld), float("nan"), dtype=t.float32, device="cuda")
        full[..., :L] = t.from_numpy(bias_np).cuda()
        bias = full[..., :L]
    bk = None if bk_np is None else t.from_numpy(bk_np).cuda()
    ea.attn_prefill_paged_masked(qd, kc, vc, bt, sl, pg.seq_lens, cud, cu, o, lse, scale=pg.scale, causal=causal,
                                 window=window, block_keep=bk, bias=bias)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


PAGED_MASK_CASES = [
    # KV lengths, chunk lengths, A, A_kv, d, page size, causal, window, term heads, block heads
    ([300, 1, 129, 700, 64, 5, 1000, 17], [300, 1, 1, 200, 64, 5, 129, 0], 8, 2, 128, 16, True, None, 1, 1),
    ([400, 260, 33], [150, 260, 3], 4, 4, 128, 64, True, (77, -1), 4, 0),
    ([520, 90], [260, 90], 4, 2, 64, 32, False, None, 0, 4),
    ([1000, 300], [129, 300], 8, 1, 128, 16, True, None, 1, 8),
]


@pytest.mark.parametrize("case", PAGED_MASK_CASES,
                         ids=lambda c: f"{len(c[0])}seq-A{c[2]}-kv{c[3]}-d{c[4]}-ps{c[5]}-{'c' if c[6] else 'n'}"
                                       f"-t{c[8]}-b{c[9]}" + ("" if c[7] is None else f"-w{c[7][0]}"))
def test_paged_prefill_block_mask_and_term(ea, orc, case):
    """Paged chunks with per-sequence block masks over (chunk row, key
    position) and per-token terms ("Attention Kernel", 可编程 mask over Paged 与
    ragged KV) against the oracle, mixed with decode rows and an empty chunk."""
    lens, q_lens, A, A_kv, d, ps, causal, window, th, bh = case
    _say("paged prefill block mask + term", case)
    pg, q, cu = gen.make_paged_prefill(lens, q_lens, A, A_kv, d, ps, seed=sum(lens) + A, extra_pages=3)
    rng = np.random.default_rng(sum(q_lens) + 11)
    T_q, L = int(cu[-1]), max(lens)
    nqb, nkb = (max(q_lens) + 127) // 128, (L + 127) // 128
    bias = None
    if th:
        bias = (0.5 * rng.standard_normal((th, T_q, L))).astype(np.float32)
        bias[rng.random(bias.shape) < 0.1] = -np.inf
    bk = (rng.random((len(lens), bh, nqb, nkb)) < 0.6).astype(np.uint8) if bh else None
    w = None if window is None else (window[0], 0 if causal else window[1])
    o, lse = run_paged_masked(ea, pg, q, cu, bias_np=bias, bk_np=bk, window=window, causal=causal)
    o_ref, l_ref = orc.prefill_paged(q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, cu, dtype=pg.dtype,
                                     scale=pg.scale, causal=causal, window=w, bias=bias, block_keep=bk)
    gu.check(o[None], lse[None], o_ref[None], l_ref[None], pg.dtype, str(case))


def test_paged_masked_neutral_is_paged_bitwise(ea):
    """An all-ones block mask gives attn_prefill_paged's bits (the listed tiles
    are all the tiles; a zero term differs only by the term's path)."""
    lens, q_lens = [700, 33, 260], [200, 3, 260]
    _say("paged masked, all-ones blocks == paged", lens, q_lens)
    pg, q, cu = gen.make_paged_prefill(lens, q_lens, 8, 2, 128, 16, seed=977)
    bk = np.ones((3, 1, 3, 6), np.uint8)
    o1, l1 = run_paged_prefill(ea, pg, q, cu)
    o2, l2 = run_paged_masked(ea, pg, q, cu, bk_np=bk)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
