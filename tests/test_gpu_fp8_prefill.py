"""GPU parity of attn_fwd_fp8 (E4M3 queries and keys with one scale per 128
tokens, QK^T on the FP8 matrix cores, bf16 values) against the fp64 oracle
over the dequantised inputs (oracle.attn_fwd_fp8).  The scores are exact
products of the FP8 codes accumulated in fp32 and the probabilities are
rounded to bf16 as in the bf16 path, so the bf16 tolerances apply.
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


def run_fp8(ea, p, q_keep=None, k_keep=None, window=None):
    t = gu.torch()
    q, k = t.from_numpy(p.q_codes).cuda(), t.from_numpy(p.k_codes).cuda()
    v = gu.dev(p.v, "bf16")
    qs, ks = t.from_numpy(p.q_scale).cuda(), t.from_numpy(p.k_scale).cuda()
    o = t.empty((p.B, p.A, p.S_q, p.d), dtype=t.bfloat16, device="cuda")
    lse = t.empty((p.B, p.A, p.S_q), dtype=t.float32, device="cuda")
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ea.attn_fwd_fp8(q, k, v, o, lse, qs, ks, scale=p.scale, causal=p.causal,
                    q_keep=None if q_keep is None else gu.dev(q_keep, "u8"),
                    k_keep=None if k_keep is None else gu.dev(k_keep, "u8"), window=window)
    t.cuda.synchronize()
    return gu.host_f64(o), lse.cpu().numpy().astype(np.float64)


FP8_CASES = [
    # B, A, A_kv, S_q, S_k, causal, window, keeps
    (1, 2, 1, 1, 1, False, None, False),
    (2, 4, 2, 300, 300, True, None, False),
    (1, 4, 4, 513, 900, False, None, False),      # ragged tiles, S_q < S_k, several key scale blocks
    (1, 2, 2, 700, 400, True, None, False),       # S_q > S_k: leading rows masked
    (2, 8, 2, 256, 256, True, (100, -1), True),   # GQA, window, keep masks
    (1, 2, 1, 130, 1000, False, (200, 300), False),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else "n")
                         + ("w" if c[6] else "") + ("k" if c[7] else ""))
def test_fp8_prefill_small(ea, orc, case):
    B, A, A_kv, S_q, S_k, causal, window, keeps = case
    _say("fp8 prefill", case)
    seed = 1700 + S_q + S_k + A
    p = gen.make_dense_fp8(B, A, A_kv, S_q, S_k, 128, causal=causal, seed=seed)
    qk = kk = None
    if keeps:
        qk = gen.keep_mask(B * S_q, S_q // 10, seed, gen.S_QKEEP).reshape(B, S_q)
        kk = gen.keep_mask(B * S_k, S_k // 8, seed, gen.S_KKEEP).reshape(B, S_k)
    o, lse = run_fp8(ea, p, qk, kk, window)
    mk = None if window is None else oracle.window_keep(B, S_q, S_k, window[0], 0 if causal else window[1])
    o_ref, l_ref = orc.attn_fwd_fp8(p.q_codes, p.k_codes, p.v, p.q_scale, p.k_scale, scale=p.scale, causal=causal,
                                    q_keep=qk, k_keep=kk, m_keep=mk)
    _say(gu.check(o, lse, o_ref, l_ref, "bf16", str(case)))


@pytest.mark.parametrize("shape", [(4, 32, 32, 2048), (1, 32, 8, 16384)], ids=["mha-4x32x2048", "gqa-1x32:8x16384"])
def test_fp8_prefill_full_size_sampled(ea, orc, shape):
    """The MHA and the long GQA causal workloads' shapes with FP8 queries and
    keys: sampled rows against the oracle, causal row 0 of every head equal
    to V's first row exactly, all outputs finite."""
    B, A, A_kv, S = shape
    _say("fp8 prefill full size", shape)
    p = gen.make_dense_fp8(B, A, A_kv, S, S, 128, causal=True, seed=1800 + S,
                           v_kind="uniform" if A_kv != A else "normal")
    o, lse = run_fp8(ea, p)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    v0 = gen.as_f32(p.v, "bf16")[:, :, 0].astype(np.float64)               # [B, A_kv, d]
    assert np.array_equal(o[:, :, 0], np.repeat(v0, A // A_kv, axis=1))
    rng = np.random.default_rng(1801)
    n = 600
    rows = np.unique(rng.integers(0, B * A * S, size=n))
    o_ref, l_ref = orc.attn_fwd_fp8(p.q_codes, p.k_codes, p.v, p.q_scale, p.k_scale, scale=p.scale, causal=True,
                                    rows=rows)
    _say(gu.check(o.reshape(-1, 128)[rows], lse.reshape(-1)[rows], o_ref, l_ref, "bf16", f"fp8 full {shape}"))
