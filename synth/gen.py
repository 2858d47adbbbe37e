"""Seeded synthetic inputs for fused exact attention (prefill, varlen, paged decode).

Nothing here computes attention.  The module draws numbers, rounds them to the
storage dtype once, and builds the index structures (cu_seqlens, block tables)
that describe where each sequence lives.  Both sides of a parity check read the
same arrays: the CPU oracle widens the stored bf16 bits to fp64, the GPU reads
the bits.

Random streams.  Every tensor is drawn from its own stream, identified by
``(seed, stream)``; a tensor is filled in chunks of ``CHUNK`` elements and chunk
``c`` comes from ``PCG64(SeedSequence([seed, stream, c]))``.  The values are
therefore fixed by (seed, stream, position) and do not depend on how many
threads fill the array.

Workload shapes follow the pages' workloads (dense causal prefill, GQA prefill,
long-context paged decode, ragged packed prefill); the five named recipes are in
``CONFIGS``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22

# stream ids, in drawing order
S_Q, S_K, S_V, S_LENS, S_PERM, S_QKEEP, S_KKEEP, S_DOUT, S_BIAS = 0, 1, 2, 3, 4, 5, 6, 7, 8


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(out: np.ndarray, seed: int, stream: int, kind: str, lo: float = 0.0, hi: float = 1.0) -> None:
    flat = out.reshape(-1)
    n = flat.size
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        view = flat[c * CHUNK: min(n, (c + 1) * CHUNK)]
        if kind == "normal":
            rng.standard_normal(out=view, dtype=np.float32)
        elif kind == "uniform":
            rng.random(out=view, dtype=np.float32)
            view *= np.float32(hi - lo)
            view += np.float32(lo)
        else:  # pragma: no cover
            raise ValueError(kind)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, round-to-nearest-even, returned as uint16 bits.

    Inputs are finite draws, so the NaN special case is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    src = x.reshape(-1).view(np.uint32)
    dst = out.reshape(-1)
    n = src.size

    def work(c: int) -> None:
        s = src[c * CHUNK: min(n, (c + 1) * CHUNK)]
        lsb = (s >> np.uint32(16)) & np.uint32(1)
        dst[c * CHUNK: min(n, (c + 1) * CHUNK)] = ((s + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(shape, seed: int, stream: int, kind: str = "normal", dtype: str = "bf16",
         lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Draw a tensor; bf16 tensors are returned as uint16 bits, fp32 as float32."""
    x = np.empty(shape, dtype=np.float32)
    _fill(x, seed, stream, kind, lo, hi)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (bits or float32) as float32 values."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def keep_mask(n: int, n_masked: int, seed: int, stream: int) -> np.ndarray:
    """uint8 keep vector with exactly ``n_masked`` zeros at seeded positions."""
    keep = np.ones(n, dtype=np.uint8)
    if n_masked > 0:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))
        keep[rng.choice(n, size=n_masked, replace=False)] = 0
    return keep


@dataclass
class Dense:
    """Batched prefill problem: q/o [B, A, S_q, d], k/v [B, A_kv, S_k, d]."""
    B: int
    A: int
    A_kv: int
    S_q: int
    S_k: int
    d: int
    dtype: str
    causal: bool
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_keep: np.ndarray | None = None   # [B, S_q] uint8
    k_keep: np.ndarray | None = None   # [B, S_k] uint8

    def flops(self) -> float:
        """Algorithmic FLOPs, 4*B*A*S_q*S_k*d, halved when causal."""
        f = 4.0 * self.B * self.A * self.S_q * self.S_k * self.d
        return f / 2 if self.causal else f

    def io_bytes(self) -> int:
        """Bytes each launch must move at least once: Q, K, V read, O written
        (element size of `dtype`) and the fp32 LSE written."""
        e = 2 if self.dtype == "bf16" else 4
        return (e * self.d * (2 * self.B * self.A * self.S_q + 2 * self.B * self.A_kv * self.S_k)
                + 4 * self.B * self.A * self.S_q)


@dataclass
class Varlen:
    """Packed ragged prefill: q/o [A, T, d], k/v [A_kv, T, d], sequences by cu_seqlens."""
    lens: np.ndarray
    cu_seqlens: np.ndarray     # int32 [n_seq + 1]
    A: int
    A_kv: int
    d: int
    dtype: str
    causal: bool
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_keep: np.ndarray | None = None   # [T]
    k_keep: np.ndarray | None = None   # [T]

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_seq(self) -> int:
        return int(self.lens.size)

    def flops(self) -> float:
        f = float(np.sum(4.0 * self.A * self.lens.astype(np.float64) ** 2 * self.d))
        return f / 2 if self.causal else f


@dataclass
class Paged:
    """Single-query decode over a paged KV cache.

    q/o [B, A, d]; k_cache/v_cache [num_pages, page_size, A_kv, d];
    block_table int32 [B, max_pages] (-1 past a sequence's last page);
    seq_lens int32 [B].
    """
    B: int
    A: int
    A_kv: int
    d: int
    page_size: int
    dtype: str
    scale: float
    seq_lens: np.ndarray
    block_table: np.ndarray
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    num_pages: int = field(default=0)

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def kv_bytes(self) -> float:
        """Algorithmic KV bytes: every valid token's K and V row of every KV head."""
        esz = 2 if self.dtype == "bf16" else 4
        return float(2 * self.A_kv * self.d * esz * int(np.sum(self.seq_lens, dtype=np.int64)))


def make_dense(B, A, A_kv, S_q, S_k, d, *, dtype="bf16", causal=False, seed=0,
               v_kind="normal", scale=None, q_masked=0, k_masked=0) -> Dense:
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    q = draw((B, A, S_q, d), seed, S_Q, "normal", dtype)
    k = draw((B, A_kv, S_k, d), seed, S_K, "normal", dtype)
    if v_kind == "uniform":
        v = draw((B, A_kv, S_k, d), seed, S_V, "uniform", dtype, -1.0, 1.0)
    else:
        v = draw((B, A_kv, S_k, d), seed, S_V, "normal", dtype)
    qk = keep_mask(B * S_q, q_masked, seed, S_QKEEP).reshape(B, S_q) if q_masked else None
    kk = keep_mask(B * S_k, k_masked, seed, S_KKEEP).reshape(B, S_k) if k_masked else None
    return Dense(B, A, A_kv, S_q, S_k, d, dtype, causal, scale, q, k, v, qk, kk)


def make_dout(p: Dense, seed: int) -> np.ndarray:
    """Incoming output gradient dO for a dense problem: N(0, 1), shaped like Q."""
    return draw((p.B, p.A, p.S_q, p.d), seed, S_DOUT, "normal", p.dtype)


def lognormal_lengths(n: int, median: float, sigma: float, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, S_LENS])))
    x = np.exp(rng.normal(math.log(median), sigma, size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def make_varlen(lens, A, A_kv, d, *, dtype="bf16", causal=True, seed=0, q_mask_frac=0.0,
                k_mask_frac=0.0, scale=None) -> Varlen:
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(lens.size + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    q = draw((A, T, d), seed, S_Q, "normal", dtype)
    k = draw((A_kv, T, d), seed, S_K, "normal", dtype)
    v = draw((A_kv, T, d), seed, S_V, "normal", dtype)
    qk = keep_mask(T, int(round(q_mask_frac * T)), seed, S_QKEEP) if q_mask_frac > 0 else None
    kk = keep_mask(T, int(round(k_mask_frac * T)), seed, S_KKEEP) if k_mask_frac > 0 else None
    return Varlen(lens, cu, A, A_kv, d, dtype, causal, scale, q, k, v, qk, kk)


def make_paged(lens, A, A_kv, d, page_size, *, dtype="bf16", seed=0, scale=None,
               max_pages=None, extra_pages=0) -> Paged:
    """Paged KV cache whose physical pages are a seeded permutation of the pool.

    The pool holds exactly sum(ceil(len/page_size)) pages (plus ``extra_pages``
    spare ones), assigned to (sequence, logical page) in order through the
    permutation.  Unused block-table entries are -1.
    """
    lens = np.asarray(lens, dtype=np.int32)
    B = lens.size
    npg = (lens.astype(np.int64) + page_size - 1) // page_size
    pool = int(npg.sum()) + int(extra_pages)
    if max_pages is None:
        max_pages = max(1, int(npg.max()) if B else 1)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, S_PERM])))
    perm = rng.permutation(pool).astype(np.int32)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(npg[b])
        bt[b, :n] = perm[off: off + n]
        off += n
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    q = draw((B, A, d), seed, S_Q, "normal", dtype)
    kc = draw((pool, page_size, A_kv, d), seed, S_K, "normal", dtype)
    vc = draw((pool, page_size, A_kv, d), seed, S_V, "normal", dtype)
    return Paged(B, A, A_kv, d, page_size, dtype, scale, lens, bt, q, kc, vc, pool)


def make_paged_prefill(lens, q_lens, A, A_kv, d, page_size, *, dtype="bf16", seed=0, extra_pages=0):
    """Query chunks over a paged cache: the cache, block table and lengths of
    make_paged (``lens`` = KV length per sequence, chunk included) plus packed
    chunk queries q [A, sum(q_lens), d] and cu_seqlens_q [n_seq + 1]."""
    pg = make_paged(lens, A, A_kv, d, page_size, dtype=dtype, seed=seed, extra_pages=extra_pages)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    cu = np.zeros(q_lens.size + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    q = draw((A, int(cu[-1]), d), seed, S_DOUT + 1, "normal", dtype)
    return pg, q, cu


def _e4m3_positive_values() -> np.ndarray:
    """Values of the E4M3 codes 0x00..0x7E (sign bit clear, NaN excluded), by
    the OCP FP8 definition: bias 7, 3 mantissa bits, subnormals at exponent 0."""
    c = np.arange(0x7F)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


def quantize_e4m3_reference(y: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 code (ties to the even code), saturating at
    448, by searching the table of code values; returns uint8 codes."""
    tab = _e4m3_positive_values()
    a = np.minimum(np.abs(np.asarray(y, dtype=np.float64)), tab[-1])
    hi = np.clip(np.searchsorted(tab, a), 1, tab.size - 1)
    lo = hi - 1
    dl, dh = a - tab[lo], tab[hi] - a
    pick_hi = (dh < dl) | ((dh == dl) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y) & (code != 0), code | 0x80, code).astype(np.uint8)


def quantize_e4m3(y: np.ndarray) -> np.ndarray:
    """quantize_e4m3_reference for fp32 input, with integer arithmetic: below
    2^-6 the code is round-half-even(|y| * 2^9); above, the fp32 mantissa is
    rounded to 3 bits (ties to even) and the exponent rebiased from 127 to 7.
    Runs in chunks on a thread pool (the FP8 decode workload has 1e9 values)."""
    y = np.ascontiguousarray(y, dtype=np.float32).reshape(-1)
    out = np.empty(y.size, dtype=np.uint8)
    step = CHUNK

    def work(c: int) -> None:
        v = y[c * step: (c + 1) * step]
        a = np.minimum(np.abs(v), np.float32(448.0))
        bits = a.view(np.uint32)
        lsb = (bits >> np.uint32(20)) & np.uint32(1)
        normal = ((bits + np.uint32(0x7FFFF) + lsb) >> np.uint32(20)).astype(np.int64) - 960
        sub = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)
        code = np.where(a < np.float32(2.0 ** -6), sub, normal).astype(np.uint8)
        out[c * step: (c + 1) * step] = np.where((v < 0) & (code != 0), code | np.uint8(0x80), code)

    n = (y.size + step - 1) // step
    if n <= 1:
        for c in range(n):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n)))
    return out


@dataclass
class PagedFp8:
    """Paged decode over FP8 caches: ``base`` holds q, block table and lengths
    (its bf16 caches are not used); k/v_codes uint8 [num_pages, page_size,
    A_kv, d]; k/v_scale fp32 [num_pages, A_kv]."""
    base: Paged
    k_codes: np.ndarray
    v_codes: np.ndarray
    k_scale: np.ndarray
    v_scale: np.ndarray


def make_paged_fp8(lens, A, A_kv, d, page_size, *, seed=0, extra_pages=0) -> PagedFp8:
    """FP8 caches quantised per (page, KV head): N(0, 1) values drawn in fp32,
    scale = max |x| / 448 over the page's tokens and dims, codes =
    round-to-nearest-even of x / scale."""
    lens = np.asarray(lens, dtype=np.int32)
    npg = (lens.astype(np.int64) + page_size - 1) // page_size
    pool = int(npg.sum()) + int(extra_pages)
    # block table, q and lengths exactly as make_paged draws them (caches drawn below in fp32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, S_PERM])))
    perm = rng.permutation(pool).astype(np.int32)
    max_pages = max(1, int(npg.max()) if lens.size else 1)
    bt = np.full((lens.size, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(lens.size):
        n = int(npg[b])
        bt[b, :n] = perm[off: off + n]
        off += n
    q = draw((lens.size, A, d), seed, S_Q, "normal", "bf16")
    base = Paged(lens.size, A, A_kv, d, page_size, "bf16", float(np.float32(1.0 / math.sqrt(d))), lens, bt, q,
                 np.zeros((0,), np.uint16), np.zeros((0,), np.uint16), pool)
    out = []
    for stream in (S_K, S_V):
        x = draw((pool, page_size, A_kv, d), seed, stream, "normal", "f32")
        amax = np.abs(x).max(axis=(1, 3))                              # [pool, A_kv]
        sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        x /= sc[:, None, :, None]
        codes = quantize_e4m3(x).reshape(x.shape)
        del x
        out += [codes, sc]
    return PagedFp8(base, out[0], out[2], out[1], out[3])


@dataclass
class DenseFp8:
    """Dense prefill with FP8 queries and keys: q/k_codes uint8 E4M3 [B, A or
    A_kv, S, d]; q/k_scale fp32 [B, A or A_kv, ceil(S / 128)] (one scale per 128
    tokens); v bf16 bits [B, A_kv, S_k, d]."""
    B: int
    A: int
    A_kv: int
    S_q: int
    S_k: int
    d: int
    causal: bool
    scale: float
    q_codes: np.ndarray
    k_codes: np.ndarray
    q_scale: np.ndarray
    k_scale: np.ndarray
    v: np.ndarray

    def flops(self) -> float:
        f = 4.0 * self.B * self.A * self.S_q * self.S_k * self.d
        return f / 2 if self.causal else f


def _quantise_blocks(x: np.ndarray) -> tuple:
    """E4M3 codes of x [B, H, S, d] (fp32) with one scale per 128 rows of each
    (batch, head): scale = max |x| / 448 over the block (1 for an all-zero
    block), codes = round-to-nearest-even of x / scale."""
    B, H, S, d = x.shape
    nb = (S + 127) // 128
    pad = np.zeros((B, H, nb * 128, d), np.float32)
    pad[:, :, :S] = x
    amax = np.abs(pad.reshape(B, H, nb, 128 * d)).max(axis=3)
    sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = x / np.repeat(sc, 128, axis=2)[:, :, :S, None]
    return quantize_e4m3(y).reshape(x.shape), sc


def make_dense_fp8(B, A, A_kv, S_q, S_k, d, *, causal=False, seed=0, v_kind="normal") -> DenseFp8:
    """Q, K ~ N(0, 1) drawn in fp32 and quantised to E4M3 per 128-token block;
    V ~ N(0, 1) (or U(-1, 1)) rounded to bf16; scale = fp32(1 / sqrt(d))."""
    q = draw((B, A, S_q, d), seed, S_Q, "normal", "f32")
    k = draw((B, A_kv, S_k, d), seed, S_K, "normal", "f32")
    if v_kind == "uniform":
        v = draw((B, A_kv, S_k, d), seed, S_V, "uniform", "bf16", -1.0, 1.0)
    else:
        v = draw((B, A_kv, S_k, d), seed, S_V, "normal", "bf16")
    qc, qs = _quantise_blocks(q)
    kc, ks = _quantise_blocks(k)
    return DenseFp8(B, A, A_kv, S_q, S_k, d, causal, float(np.float32(1.0 / math.sqrt(d))), qc, kc, qs, ks, v)


def make_paged_prefill_fp8(lens, q_lens, A, A_kv, d, page_size, *, seed=0, extra_pages=0):
    """Query chunks over FP8 caches: make_paged_fp8's caches, scales, block
    table and lengths (``lens`` = KV length per sequence, chunk included) plus
    packed bf16 chunk queries q [A, sum(q_lens), d] and cu_seqlens_q."""
    pf = make_paged_fp8(lens, A, A_kv, d, page_size, seed=seed, extra_pages=extra_pages)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    cu = np.zeros(q_lens.size + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    q = draw((A, int(cu[-1]), d), seed, S_DOUT + 1, "normal", "bf16")
    return pf, q, cu


# --- the five named workloads -------------------------------------------------

CONFIG_SEEDS = {1: 1001, 2: 1002, 3: 1003, 4: 1004, 5: 1005}

CONFIGS = {
    1: "fp32 single head, B=1 A=A_kv=1 S_q=S_k=128 d=64, non-causal, no mask",
    2: "bf16 MHA causal prefill, B=4 A=A_kv=32 S_q=S_k=2048 d=128",
    3: "bf16 GQA causal prefill, B=1 A=32 A_kv=8 S_q=S_k=16384 d=128, V~U(-1,1)",
    4: "bf16 paged decode, 64 seqs, A=32 A_kv=8 d=128, lens~U{512..32768}, page 16",
    5: "bf16 varlen causal, 16 seqs log-normal(median 1024, sigma 1, clip [64,8192]), A=A_kv=16 d=64, 5% rows fully masked",
}


def config_lengths_decode(seed: int = CONFIG_SEEDS[4], n: int = 64) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, S_LENS])))
    return rng.integers(512, 32768, size=n, endpoint=True).astype(np.int32)


def make_config(k: int, seed: int | None = None):
    seed = CONFIG_SEEDS[k] if seed is None else seed
    if k == 1:
        return make_dense(1, 1, 1, 128, 128, 64, dtype="f32", causal=False, seed=seed)
    if k == 2:
        return make_dense(4, 32, 32, 2048, 2048, 128, dtype="bf16", causal=True, seed=seed)
    if k == 3:
        return make_dense(1, 32, 8, 16384, 16384, 128, dtype="bf16", causal=True, seed=seed,
                          v_kind="uniform")
    if k == 4:
        return make_paged(config_lengths_decode(seed), 32, 8, 128, 16, dtype="bf16", seed=seed)
    if k == 5:
        lens = lognormal_lengths(16, 1024.0, 1.0, 64, 8192, seed)
        return make_varlen(lens, 16, 16, 64, dtype="bf16", causal=True, seed=seed, q_mask_frac=0.05)
    raise ValueError(f"no config {k}")


def document_ids(S: int, seed: int, b: int, doc_median: int = 200) -> np.ndarray:
    """Document index of each of S packed positions of batch row b: documents
    with log-normal lengths (median doc_median, sigma 0.8) laid end to end."""
    lens = lognormal_lengths(max(1, S // max(doc_median // 4, 1)) + 1, doc_median, 0.8, 1, max(S, 1), seed * 1000 + b)
    return np.searchsorted(np.cumsum(lens), np.arange(S), side="right")


def make_key_ranges(B: int, S_q: int, S_k: int, kind: str, seed: int, *, doc_median: int = 200,
                    prefix: int = 0) -> np.ndarray:
    """Per-row key ranges int32 [B, S_q, 2]: query i (at position i + S_k - S_q)
    keeps keys first..last (both included).

    kind "document": the keys of the query's own document, the documents of
        document_ids (the same ones make_bias "document" draws for this seed);
        rows at negative positions keep none (first > last).
    kind "prefix": prefix-LM, 0..max(position, prefix - 1).
    kind "random": seeded intervals, some empty, some with first < 0 or last
        >= S_k.
    """
    off = S_k - S_q
    pos = np.arange(S_q, dtype=np.int64) + off
    out = np.empty((B, S_q, 2), np.int64)
    if kind == "document":
        for b in range(B):
            doc = document_ids(S_k, seed, b, doc_median)
            first = np.searchsorted(doc, doc, side="left")
            last = np.searchsorted(doc, doc, side="right") - 1
            p = np.clip(pos, 0, max(S_k - 1, 0))
            ok = (pos >= 0) & (S_k > 0)
            out[b, :, 0] = np.where(ok, first[p] if S_k else 0, 1)
            out[b, :, 1] = np.where(ok, last[p] if S_k else 0, 0)
    elif kind == "prefix":
        out[:, :, 0] = 0
        out[:, :, 1] = np.maximum(pos, prefix - 1)[None]
    elif kind == "random":
        u = draw((B, S_q, 3), seed, S_BIAS + 200, "uniform", "f32").astype(np.float64)
        a = np.floor(u[..., 0] * (S_k + 8)).astype(np.int64) - 4
        w = np.floor(u[..., 1] * (S_k // 2 + 2)).astype(np.int64)
        out[..., 0] = a
        out[..., 1] = np.where(u[..., 2] < 0.05, a - 1, a + w)   # about 5% of the rows keep nothing
    else:
        raise ValueError(kind)
    return out.astype(np.int32)


def make_bias(B: int, H: int, S_q: int, S_k: int, kind: str, seed: int, *, doc_median: int = 200) -> np.ndarray:
    """A dense additive mask M, fp32 [B, H, S_q, S_k] (query i at position
    i + S_k - S_q, as for causal alignment).

    kind "document": packed documents with log-normal lengths (median
        doc_median) drawn per batch row; 0 inside a document, -inf across
        (H must be 1).
    kind "alibi": a linear distance penalty -slope_h |pos_i - j| with
        slope_h = 2^(-8 (h + 1) / H) (finite everywhere).
    kind "random": N(0, 2^2) entries, a seeded quarter of them -inf, and query
        row 0 of batch row 0 all -inf (a row the term alone masks).
    """
    off = S_k - S_q
    pos = np.arange(S_q)[:, None] + off
    j = np.arange(S_k)[None, :]
    out = np.empty((B, H, S_q, S_k), np.float32)
    if kind == "document":
        assert H == 1
        for b in range(B):
            doc = document_ids(S_k, seed, b, doc_median)
            same = doc[np.clip(pos, 0, S_k - 1)] == doc[j]
            same &= (pos >= 0)
            out[b, 0] = np.where(same, 0.0, -np.inf).astype(np.float32)
    elif kind == "alibi":
        for h in range(H):
            slope = 2.0 ** (-8.0 * (h + 1) / H)
            out[:, h] = (-slope * np.abs(pos - j)).astype(np.float32)
    elif kind == "random":
        x = draw((B, H, S_q, S_k), seed, S_BIAS, "normal", "f32").astype(np.float32) * 2.0
        u = draw((B, H, S_q, S_k), seed, S_BIAS + 100, "uniform", "f32")
        x[u < 0.25] = -np.inf
        if S_q > 0:
            x[0, :, 0, :] = -np.inf
        out[...] = x
    else:
        raise ValueError(kind)
    return out
