"""fp64 CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  It shares no code with the GPU library
(``exact_attention_108_amd``) and neither imports the other.

* ``attn_oracle.c``  -- the plain definition (scores and probabilities
  materialised per row, fp64), built into ``liboracle.so`` with gcc + OpenMP.
* ``blockwise.py``   -- an independent numpy fp64 re-statement of the
  two-state online-softmax merge, used only to pin the C oracle.

Every function follows page "Attention Kernel" (sections "问题与成本",
"Online softmax", "Paged 与 ragged KV") and page "Attention 算子加速史"
(section 1.1 for the materialised S and P, 1.2 for the safe softmax).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_DT = {"f32": 0, "bf16": 1, "f64": 2}  # f64: test inputs for the finite-difference gradient pins


def build(src: str = SRC, out: str = LIB, werror: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-fno-fast-math", src, "-o", out + ".tmp", "-lm"] + (["-Werror"] if werror else [])
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes view of one build of ``attn_oracle.c``."""

    def __init__(self, lib_path: str = LIB):
        if not os.path.exists(lib_path):
            build(out=lib_path)
        self.lib = ctypes.CDLL(lib_path)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        self.lib.oracle_attn_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                             vp, vp, vp, vp, i32, vp, i32, vp, i64, vp, vp]
        self.lib.oracle_attn_fwd_varlen.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, f32,
                                                    i32, vp, vp, vp, i64, vp, vp]
        self.lib.oracle_decode_paged.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                                 i32, f32, i32, vp, i64, vp, vp]
        self.lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                             vp, vp, vp, vp, i32, vp, i32, vp, vp, vp]
        self.lib.oracle_attn_bwd_varlen.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, f32, i32,
                                                    vp, vp, i32, i32, vp, vp, vp]
        self.lib.oracle_prefill_paged.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                  i32, f32, i32, i32, i32, vp, i64, vp, vp]
        self.lib.oracle_block_keep_of_bias.argtypes = [vp, i32, i32, i32, i32, vp]
        for f in (self.lib.oracle_attn_fwd, self.lib.oracle_attn_fwd_varlen, self.lib.oracle_decode_paged,
                  self.lib.oracle_attn_bwd, self.lib.oracle_attn_bwd_varlen, self.lib.oracle_prefill_paged,
                  self.lib.oracle_block_keep_of_bias):
            f.restype = ctypes.c_int
        self.lib.oracle_num_threads.restype = ctypes.c_int

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    @staticmethod
    def _arr(x, dtype):
        if dtype == "bf16":
            return np.ascontiguousarray(x, dtype=np.uint16)
        if dtype == "f32":
            return np.ascontiguousarray(x, dtype=np.float32)
        if dtype == "f64":
            return np.ascontiguousarray(x, dtype=np.float64)
        raise ValueError(f"unknown dtype {dtype!r}")

    @staticmethod
    def _blocks(block_keep, B, A, S_q, S_k):
        if block_keep is None:
            return None, 0
        bk = np.ascontiguousarray(block_keep, dtype=np.uint8)
        want = ((S_q + 127) // 128, (S_k + 127) // 128)
        if bk.ndim != 4 or bk.shape[0] != B or bk.shape[1] not in (1, A) or bk.shape[2:] != want:
            raise ValueError(f"block_keep must be [B, 1 or A, {want[0]}, {want[1]}]")
        return bk, bk.shape[1]

    @staticmethod
    def _bias(bias, B, A, S_q, S_k):
        if bias is None:
            return None, 0
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.ndim != 4 or bias.shape[0] != B or bias.shape[1] not in (1, A) or bias.shape[2:] != (S_q, S_k):
            raise ValueError("bias must be [B, 1 or A, S_q, S_k]")
        return bias, bias.shape[1]

    @staticmethod
    def _with_alibi(bias, alibi_slopes, B, A, S_q, S_k):
        if alibi_slopes is None:
            return bias
        if np.asarray(alibi_slopes).reshape(-1).size != A:
            raise ValueError("alibi_slopes must hold one slope per query head")
        a = alibi_term(alibi_slopes, B, S_q, S_k)
        return a if bias is None else (np.asarray(bias, np.float32) + a).astype(np.float32)

    @staticmethod
    def _keep_matrix(m_keep, key_range, B, S_q, S_k):
        mk = None if m_keep is None else np.ascontiguousarray(m_keep, dtype=np.uint8).reshape(B, S_q, S_k)
        if key_range is not None:
            kr = np.asarray(key_range)
            if kr.shape != (B, S_q, 2):
                raise ValueError("key_range must be [B, S_q, 2]")
            rk = key_range_keep(kr, S_k)
            mk = rk if mk is None else mk & rk
        return mk

    @staticmethod
    def _rows(rows):
        if rows is None:
            return None, 0
        r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        return r, r.size

    def attn_fwd(self, q, k, v, *, dtype, scale, causal=False, q_keep=None, k_keep=None, m_keep=None, bias=None,
                 block_keep=None, rows=None, key_range=None, alibi_slopes=None):
        """Dense batched attention.  q [B,A,S_q,d], k/v [B,A_kv,S_k,d]; alibi_slopes
        optional per-head ALiBi slopes [A] (see alibi_term), added to bias; m_keep an
        optional dense keep matrix [B,S_q,S_k] (see window_keep); key_range
        optional per-row key ranges int [B,S_q,2] (see key_range_keep), applied
        together with m_keep; bias an optional
        dense additive term M, fp32 [B,1,S_q,S_k] (every head) or [B,A,S_q,S_k],
        finite or -inf; block_keep an optional block mask uint8
        [B, 1 or A, ceil(S_q/128), ceil(S_k/128)] (0 masks the 128 x 128 block).

        Returns (o, lse): o [B,A,S_q,d] / lse [B,A,S_q] in fp64, or [n,d] / [n]
        for the flattened row ids ``rows`` = (b*A + h)*S_q + i.
        """
        q, k, v = self._arr(q, dtype), self._arr(k, dtype), self._arr(v, dtype)
        if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
            raise ValueError("q, k, v must be 4-D [B, heads, S, d]")
        B, A, S_q, d = q.shape
        if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
            raise ValueError("k and v must be [B, A_kv, S_k, d] matching q")
        A_kv, S_k = k.shape[1], k.shape[2]
        if A % A_kv:
            raise ValueError("A must be a multiple of A_kv")
        qk = None if q_keep is None else np.ascontiguousarray(q_keep, dtype=np.uint8).reshape(B, S_q)
        kk = None if k_keep is None else np.ascontiguousarray(k_keep, dtype=np.uint8).reshape(B, S_k)
        mk = self._keep_matrix(m_keep, key_range, B, S_q, S_k)
        bias = self._with_alibi(bias, alibi_slopes, B, A, S_q, S_k)
        bias, bh = self._bias(bias, B, A, S_q, S_k)
        bk, bkh = self._blocks(block_keep, B, A, S_q, S_k)
        r, n = self._rows(rows)
        n_out = B * A * S_q if r is None else n
        o = np.empty((n_out, d), dtype=np.float64)
        lse = np.empty(n_out, dtype=np.float64)
        rc = self.lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[dtype], B, A, A_kv, S_q, S_k, d,
                                      float(scale), int(bool(causal)), _ptr(qk), _ptr(kk), _ptr(mk), _ptr(bias),
                                      bh, _ptr(bk), bkh, _ptr(r), n, _ptr(o), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle_attn_fwd rejected its arguments")
        if r is None:
            return o.reshape(B, A, S_q, d), lse.reshape(B, A, S_q)
        return o, lse

    def attn_fwd_varlen(self, q, k, v, cu_seqlens, *, dtype, scale, causal=True, q_keep=None,
                        k_keep=None, rows=None, bias=None, block_keep=None, window=None, key_range=None,
                        alibi_slopes=None):
        """Packed varlen attention.  q [A,T,d], k/v [A_kv,T,d]; rows = h*T + t.

        bias: fp32 [1 or A, T, ld] -- row t (token i of its sequence) holds the
        additive term of its keys j < len at columns j (positions within the
        sequence); block_keep: uint8 [n_seq, 1 or A, nb, nb], nb = ceil(longest
        length / 128), the 128 x 128 block flags of each sequence's own
        (row, key) grid; window: (left, right) around each row's position in
        its sequence; key_range: int [T, 2], token t's key range as positions
        within its sequence; alibi_slopes: [A], distances within each sequence.
        With any of these, each sequence is its own dense problem
        ("Attention Kernel", Paged 与 ragged KV: packed sequences never attend
        across boundaries) and goes through attn_fwd with its slices."""
        if bias is not None or block_keep is not None or window is not None or key_range is not None or \
                alibi_slopes is not None:
            return self._varlen_by_sequence(q, k, v, cu_seqlens, dtype=dtype, scale=scale, causal=causal,
                                            q_keep=q_keep, k_keep=k_keep, bias=bias, block_keep=block_keep,
                                            window=window, rows=rows, key_range=key_range, alibi_slopes=alibi_slopes)
        q, k, v = self._arr(q, dtype), self._arr(k, dtype), self._arr(v, dtype)
        if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or k.shape != v.shape:
            raise ValueError("q [A,T,d], k/v [A_kv,T,d]")
        A, T, d = q.shape
        A_kv = k.shape[0]
        if k.shape[1] != T or k.shape[2] != d or A % A_kv:
            raise ValueError("k/v must be [A_kv, T, d] with A % A_kv == 0")
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        n_seq = cu.size - 1
        qk = None if q_keep is None else np.ascontiguousarray(q_keep, dtype=np.uint8).reshape(T)
        kk = None if k_keep is None else np.ascontiguousarray(k_keep, dtype=np.uint8).reshape(T)
        r, n = self._rows(rows)
        n_out = A * T if r is None else n
        o = np.empty((n_out, d), dtype=np.float64)
        lse = np.empty(n_out, dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _DT[dtype], _ptr(cu), n_seq, T, A,
                                             A_kv, d, float(scale), int(bool(causal)), _ptr(qk), _ptr(kk),
                                             _ptr(r), n, _ptr(o), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle_attn_fwd_varlen rejected its arguments")
        if r is None:
            return o.reshape(A, T, d), lse.reshape(A, T)
        return o, lse

    def _varlen_by_sequence(self, q, k, v, cu_seqlens, *, dtype, scale, causal, q_keep, k_keep, bias, block_keep,
                            window, rows=None, key_range=None, alibi_slopes=None):
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        A, T, d = q.shape
        n_seq = cu.size - 1
        lens = np.diff(cu)
        nb = int((lens.max() + 127) // 128) if n_seq else 0
        if bias is not None:
            bias = np.asarray(bias, dtype=np.float32)
            if bias.ndim != 3 or bias.shape[0] not in (1, A) or bias.shape[1] != T or bias.shape[2] < lens.max(initial=0):
                raise ValueError("bias must be [1 or A, T, ld >= longest length]")
        if block_keep is not None:
            block_keep = np.asarray(block_keep, dtype=np.uint8)
            if block_keep.ndim != 4 or block_keep.shape[0] != n_seq or block_keep.shape[1] not in (1, A) or \
                    block_keep.shape[2:] != (nb, nb):
                raise ValueError(f"block_keep must be [n_seq, 1 or A, {nb}, {nb}]")
        o = np.zeros((A, T, d), dtype=np.float64)
        lse = np.full((A, T), -np.inf, dtype=np.float64)
        want = None
        if rows is not None:  # flattened ids h*T + t: only those rows are formed
            r = np.asarray(rows, dtype=np.int64).reshape(-1)
            want = (r // T, r % T)
        for s in range(n_seq):
            s0, s1 = int(cu[s]), int(cu[s + 1])
            L = s1 - s0
            if L == 0:
                continue
            kw = {}
            if want is not None:
                sel = (want[1] >= s0) & (want[1] < s1)
                if not sel.any():
                    continue
                kw["rows"] = want[0][sel] * L + (want[1][sel] - s0)   # (b = 0, h, i) of the one-sequence call
            if q_keep is not None:
                kw["q_keep"] = np.asarray(q_keep).reshape(T)[s0:s1][None]
            if k_keep is not None:
                kw["k_keep"] = np.asarray(k_keep).reshape(T)[s0:s1][None]
            if window is not None:
                kw["m_keep"] = window_keep(1, L, L, int(window[0]), int(window[1]))
            if key_range is not None:
                kw["key_range"] = np.asarray(key_range).reshape(T, 2)[s0:s1][None]
            if alibi_slopes is not None:
                kw["alibi_slopes"] = alibi_slopes
            if bias is not None:
                kw["bias"] = bias[:, s0:s1, :L][None]
            if block_keep is not None:
                nbs = (L + 127) // 128
                kw["block_keep"] = block_keep[s][None, :, :nbs, :nbs]
            os_, ls_ = self.attn_fwd(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], dtype=dtype,
                                     scale=scale, causal=causal, **kw)
            if want is not None:
                o[want[0][sel], want[1][sel]] = os_
                lse[want[0][sel], want[1][sel]] = ls_
            else:
                o[:, s0:s1] = os_[0]
                lse[:, s0:s1] = ls_[0]
        if want is not None:
            return o[want], lse[want]
        return o, lse

    def attn_bwd(self, q, k, v, do, *, dtype, scale, causal=False, q_keep=None, k_keep=None, m_keep=None,
                 bias=None, block_keep=None, key_range=None, alibi_slopes=None):
        """Gradient of attn_fwd: q, do [B,A,S_q,d]; k, v [B,A_kv,S_k,d]; masks
        and ALiBi slopes as attn_fwd takes them.  Returns (dq, dk, dv) in fp64 with the shapes of
        q, k and v."""
        q, k, v, do = self._arr(q, dtype), self._arr(k, dtype), self._arr(v, dtype), self._arr(do, dtype)
        if q.ndim != 4 or k.shape != v.shape or do.shape != q.shape:
            raise ValueError("q, do [B,A,S_q,d]; k, v [B,A_kv,S_k,d]")
        B, A, S_q, d = q.shape
        A_kv, S_k = k.shape[1], k.shape[2]
        if k.shape[0] != B or k.shape[3] != d or A % A_kv:
            raise ValueError("k/v must be [B, A_kv, S_k, d] with A % A_kv == 0")
        qk = None if q_keep is None else np.ascontiguousarray(q_keep, dtype=np.uint8).reshape(B, S_q)
        kk = None if k_keep is None else np.ascontiguousarray(k_keep, dtype=np.uint8).reshape(B, S_k)
        mk = self._keep_matrix(m_keep, key_range, B, S_q, S_k)
        bias = self._with_alibi(bias, alibi_slopes, B, A, S_q, S_k)
        bias, bh = self._bias(bias, B, A, S_q, S_k)
        bk, bkh = self._blocks(block_keep, B, A, S_q, S_k)
        dq = np.empty((B, A, S_q, d), dtype=np.float64)
        dk = np.empty((B, A_kv, S_k, d), dtype=np.float64)
        dv = np.empty((B, A_kv, S_k, d), dtype=np.float64)
        rc = self.lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _DT[dtype], B, A, A_kv, S_q, S_k, d,
                                      float(scale), int(bool(causal)), _ptr(qk), _ptr(kk), _ptr(mk), _ptr(bias), bh,
                                      _ptr(bk), bkh, _ptr(dq), _ptr(dk), _ptr(dv))
        if rc != 0:
            raise ValueError("oracle_attn_bwd rejected its arguments")
        return dq, dk, dv

    def attn_bwd_varlen(self, q, k, v, do, cu_seqlens, *, dtype, scale, causal=True, q_keep=None, k_keep=None,
                        window=None, bias=None, block_keep=None, key_range=None, alibi_slopes=None):
        """Gradient of the packed varlen prefill: q, do [A,T,d]; k, v [A_kv,T,d];
        cu_seqlens [n_seq+1]; keep masks [T]; window (left, right) within each
        sequence (-1 = unbounded).  Returns (dq, dk, dv) in fp64.  bias,
        block_keep and key_range as attn_fwd_varlen takes them; with any, each sequence's
        gradient is the dense gradient of its own problem (its slices of the
        masks) -- the backward uses the forward's mask ("Attention Kernel",
        Backward 与重计算)."""
        if bias is not None or block_keep is not None or key_range is not None or alibi_slopes is not None:
            return self._bwd_varlen_by_sequence(q, k, v, do, cu_seqlens, dtype=dtype, scale=scale, causal=causal,
                                                q_keep=q_keep, k_keep=k_keep, window=window, bias=bias,
                                                block_keep=block_keep, key_range=key_range,
                                                alibi_slopes=alibi_slopes)
        q, k, v, do = self._arr(q, dtype), self._arr(k, dtype), self._arr(v, dtype), self._arr(do, dtype)
        if q.ndim != 3 or k.shape != v.shape or do.shape != q.shape:
            raise ValueError("q, do [A,T,d]; k, v [A_kv,T,d]")
        A, T, d = q.shape
        A_kv = k.shape[0]
        if k.shape[1] != T or k.shape[2] != d or A % A_kv:
            raise ValueError("k/v must be [A_kv, T, d] with A % A_kv == 0")
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        qk = None if q_keep is None else np.ascontiguousarray(q_keep, dtype=np.uint8).reshape(T)
        kk = None if k_keep is None else np.ascontiguousarray(k_keep, dtype=np.uint8).reshape(T)
        wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
        dq = np.empty((A, T, d), dtype=np.float64)
        dk = np.empty((A_kv, T, d), dtype=np.float64)
        dv = np.empty((A_kv, T, d), dtype=np.float64)
        rc = self.lib.oracle_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _DT[dtype], _ptr(cu), cu.size - 1,
                                             T, A, A_kv, d, float(scale), int(bool(causal)), _ptr(qk), _ptr(kk), wl,
                                             wr, _ptr(dq), _ptr(dk), _ptr(dv))
        if rc != 0:
            raise ValueError("oracle_attn_bwd_varlen rejected its arguments")
        return dq, dk, dv

    def _bwd_varlen_by_sequence(self, q, k, v, do, cu_seqlens, *, dtype, scale, causal, q_keep, k_keep, window, bias,
                                block_keep, key_range=None, alibi_slopes=None):
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        A, T, d = q.shape
        A_kv = k.shape[0]
        n_seq = cu.size - 1
        lens = np.diff(cu)
        nb = int((lens.max(initial=0) + 127) // 128)
        if bias is not None:
            bias = np.asarray(bias, dtype=np.float32)
            if bias.ndim != 3 or bias.shape[0] not in (1, A) or bias.shape[1] != T or bias.shape[2] < lens.max(initial=0):
                raise ValueError("bias must be [1 or A, T, ld >= longest length]")
        if block_keep is not None:
            block_keep = np.asarray(block_keep, dtype=np.uint8)
            if block_keep.ndim != 4 or block_keep.shape[0] != n_seq or block_keep.shape[1] not in (1, A) or \
                    block_keep.shape[2:] != (nb, nb):
                raise ValueError(f"block_keep must be [n_seq, 1 or A, {nb}, {nb}]")
        dq = np.zeros((A, T, d), dtype=np.float64)
        dk = np.zeros((A_kv, T, d), dtype=np.float64)
        dv = np.zeros((A_kv, T, d), dtype=np.float64)
        for s in range(n_seq):
            s0, s1 = int(cu[s]), int(cu[s + 1])
            L = s1 - s0
            if L == 0:
                continue
            kw = {}
            if q_keep is not None:
                kw["q_keep"] = np.asarray(q_keep).reshape(T)[s0:s1][None]
            if k_keep is not None:
                kw["k_keep"] = np.asarray(k_keep).reshape(T)[s0:s1][None]
            if window is not None:
                kw["m_keep"] = window_keep(1, L, L, int(window[0]), int(window[1]))
            if key_range is not None:
                kw["key_range"] = np.asarray(key_range).reshape(T, 2)[s0:s1][None]
            if alibi_slopes is not None:
                kw["alibi_slopes"] = alibi_slopes
            if bias is not None:
                kw["bias"] = bias[:, s0:s1, :L][None]
            if block_keep is not None:
                nbs = (L + 127) // 128
                kw["block_keep"] = block_keep[s][None, :, :nbs, :nbs]
            g = self.attn_bwd(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], do[None, :, s0:s1],
                              dtype=dtype, scale=scale, causal=causal, **kw)
            dq[:, s0:s1], dk[:, s0:s1], dv[:, s0:s1] = g[0][0], g[1][0], g[2][0]
        return dq, dk, dv

    def prefill_paged(self, q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, *, dtype, scale, causal=True,
                      window=None, rows=None, bias=None, block_keep=None, key_range=None, alibi_slopes=None):
        """Query chunks over a paged cache: q [A,T_q,d] packed chunks (cu_seqlens_q
        [n_seq+1]); caches [P, page_size, A_kv, d]; block_table [n_seq, max_pages];
        seq_lens [n_seq] (chunk included).  Chunk row i of sequence s sits at
        position seq_lens[s] - q_s + i.  Returns (o [A,T_q,d], lse [A,T_q]) in
        fp64, or [n,d] / [n] for the flattened ids ``rows`` = h*T_q + r.

        bias: fp32 [1 or A, T_q, ld] -- row t (a chunk token) holds the term of
        the keys at positions j < seq_lens of its sequence; block_keep: uint8
        [n_seq, 1 or A, ceil(longest chunk/128), ceil(longest seq_lens/128)] over
        (chunk row, key position); key_range: int [T_q, 2], chunk token t's key
        range as positions in its sequence; alibi_slopes: [A], chunk row i at
        position seq_lens - q_s + i.  With any of these, each sequence's keys are
        gathered token by token through its block table (token t: row t %
        page_size of page block_table[s][t // page_size]) and the chunk is the
        dense problem of its rows against them ("Attention Kernel", Paged 与
        ragged KV and 可编程 mask)."""
        if bias is not None or block_keep is not None or key_range is not None or alibi_slopes is not None:
            return self._paged_by_sequence(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, dtype=dtype,
                                           scale=scale, causal=causal, window=window, rows=rows, bias=bias,
                                           block_keep=block_keep, key_range=key_range, alibi_slopes=alibi_slopes)
        q, kc, vc = self._arr(q, dtype), self._arr(k_cache, dtype), self._arr(v_cache, dtype)
        if q.ndim != 3 or kc.ndim != 4 or kc.shape != vc.shape:
            raise ValueError("q [A,T_q,d]; caches [num_pages, page_size, A_kv, d]")
        A, T_q, d = q.shape
        num_pages, page_size, A_kv, dk = kc.shape
        if dk != d or A % A_kv:
            raise ValueError("cache head dim / head count mismatch")
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
        n_seq = cu.size - 1
        if bt.ndim != 2 or bt.shape[0] != n_seq or sl.shape != (n_seq,):
            raise ValueError("block_table [n_seq, max_pages], seq_lens [n_seq]")
        wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
        r, n = self._rows(rows)
        n_out = A * T_q if r is None else n
        o = np.empty((n_out, d), dtype=np.float64)
        lse = np.empty(n_out, dtype=np.float64)
        rc = self.lib.oracle_prefill_paged(_ptr(q), _ptr(kc), _ptr(vc), _DT[dtype], _ptr(bt), _ptr(sl), _ptr(cu),
                                           n_seq, T_q, A, A_kv, d, page_size, bt.shape[1], num_pages, float(scale),
                                           int(bool(causal)), wl, wr, _ptr(r), n, _ptr(o), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle_prefill_paged rejected its arguments")
        if r is None:
            return o.reshape(A, T_q, d), lse.reshape(A, T_q)
        return o, lse

    def _paged_by_sequence(self, q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, *, dtype, scale, causal,
                           window, rows, bias, block_keep, key_range=None, alibi_slopes=None):
        A, T_q, d = q.shape
        page_size, A_kv = k_cache.shape[1], k_cache.shape[2]
        cu = np.asarray(cu_seqlens_q, dtype=np.int64)
        sl = np.asarray(seq_lens, dtype=np.int64)
        bt = np.asarray(block_table)
        n_seq = cu.size - 1
        qlens = np.diff(cu)
        nqb = int((qlens.max(initial=0) + 127) // 128)
        nkb = int((sl.max(initial=0) + 127) // 128)
        if bias is not None:
            bias = np.asarray(bias, dtype=np.float32)
            if bias.ndim != 3 or bias.shape[0] not in (1, A) or bias.shape[1] != T_q or bias.shape[2] < sl.max(initial=0):
                raise ValueError("bias must be [1 or A, T_q, ld >= longest seq_lens]")
        if block_keep is not None:
            block_keep = np.asarray(block_keep, dtype=np.uint8)
            if block_keep.ndim != 4 or block_keep.shape[0] != n_seq or block_keep.shape[1] not in (1, A) or \
                    block_keep.shape[2:] != (nqb, nkb):
                raise ValueError(f"block_keep must be [n_seq, 1 or A, {nqb}, {nkb}]")
        o = np.zeros((A, T_q, d), dtype=np.float64)
        lse = np.full((A, T_q), -np.inf, dtype=np.float64)
        want = None
        if rows is not None:
            r = np.asarray(rows, dtype=np.int64).reshape(-1)
            want = (r // T_q, r % T_q)
        for s in range(n_seq):
            s0, s1, L = int(cu[s]), int(cu[s + 1]), int(sl[s])
            ql = s1 - s0
            if ql == 0:
                continue
            kw = {}
            if want is not None:
                sel = (want[1] >= s0) & (want[1] < s1)
                if not sel.any():
                    continue
                kw["rows"] = want[0][sel] * ql + (want[1][sel] - s0)
            pages = bt[s, np.arange(L) // page_size]
            offs = np.arange(L) % page_size
            ks = np.ascontiguousarray(np.asarray(k_cache)[pages, offs].transpose(1, 0, 2))   # [A_kv, L, d]
            vs = np.ascontiguousarray(np.asarray(v_cache)[pages, offs].transpose(1, 0, 2))
            if window is not None:
                kw["m_keep"] = window_keep(1, ql, L, int(window[0]), int(window[1]))
            if key_range is not None:
                kw["key_range"] = np.asarray(key_range).reshape(T_q, 2)[s0:s1][None]
            if alibi_slopes is not None:
                kw["alibi_slopes"] = alibi_slopes
            if bias is not None:
                kw["bias"] = bias[:, s0:s1, :L][None]
            if block_keep is not None:
                kw["block_keep"] = block_keep[s][None, :, :(ql + 127) // 128, :(L + 127) // 128]
            os_, ls_ = self.attn_fwd(q[None, :, s0:s1], ks[None], vs[None], dtype=dtype, scale=scale, causal=causal,
                                     **kw)
            if want is not None:
                o[want[0][sel], want[1][sel]] = os_
                lse[want[0][sel], want[1][sel]] = ls_
            else:
                o[:, s0:s1] = os_[0]
                lse[:, s0:s1] = ls_[0]
        if want is not None:
            return o[want], lse[want]
        return o, lse

    def block_keep_of_bias(self, bias):
        """[B, H, ceil(S_q/128), ceil(S_k/128)] uint8: 1 where some entry of the
        128 x 128 block of the additive term bias [B, H, S_q, S_k] exceeds -inf."""
        b = np.ascontiguousarray(bias, dtype=np.float32)
        if b.ndim != 4:
            raise ValueError("bias must be [B, H, S_q, S_k]")
        B, H, S_q, S_k = b.shape
        out = np.empty((B, H, (S_q + 127) // 128, (S_k + 127) // 128), dtype=np.uint8)
        if self.lib.oracle_block_keep_of_bias(_ptr(b), B, H, S_q, S_k, _ptr(out)) != 0:
            raise ValueError("oracle_block_keep_of_bias rejected its arguments")
        return out

    def attn_fwd_fp8(self, q_codes, k_codes, v, q_scale, k_scale, *, scale, causal=False, q_keep=None,
                     k_keep=None, m_keep=None, rows=None, key_range=None):
        """Dense prefill with FP8 (E4M3) queries and keys: q_codes [B,A,S_q,d],
        k_codes [B,A_kv,S_k,d] (uint8 codes), one fp32 scale per 128 consecutive
        tokens of each (batch, head): q_scale [B,A,ceil(S_q/128)], k_scale
        [B,A_kv,ceil(S_k/128)]; v bf16 bits [B,A_kv,S_k,d].  Query row i's
        value is code value * q_scale[.., i // 128], key j's code value *
        k_scale[.., j // 128] (formed in fp64); the attention is attn_fwd's."""
        qc, kc = np.asarray(q_codes), np.asarray(k_codes)
        B, A, S_q, d = qc.shape
        A_kv, S_k = kc.shape[1], kc.shape[2]
        qs = np.asarray(q_scale, np.float64)
        ks = np.asarray(k_scale, np.float64)
        if qs.shape != (B, A, (S_q + 127) // 128) or ks.shape != (B, A_kv, (S_k + 127) // 128):
            raise ValueError("q_scale [B, A, ceil(S_q/128)], k_scale [B, A_kv, ceil(S_k/128)]")
        qv = fp8_e4m3_value(qc) * np.repeat(qs, 128, axis=2)[:, :, :S_q, None]
        kv = fp8_e4m3_value(kc) * np.repeat(ks, 128, axis=2)[:, :, :S_k, None]
        vb = self._arr(v, "bf16").astype(np.uint32) << np.uint32(16)   # bf16 bits -> fp32 bits
        vv = vb.view(np.float32).astype(np.float64)
        return self.attn_fwd(qv, kv, vv, dtype="f64", scale=scale, causal=causal, q_keep=q_keep, k_keep=k_keep,
                             m_keep=m_keep, rows=rows, key_range=key_range)

    def prefill_paged_fp8(self, q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, cu_seqlens_q, *,
                          scale, causal=True, window=None, rows=None, key_range=None):
        """prefill_paged over FP8 caches: E4M3 codes [P, page_size, A_kv, d]
        with per-(page, KV head) scales [P, A_kv]; q bf16 bits [A, T_q, d].  The
        cache values code value * scale are formed in fp64 and the chunks run
        through prefill_paged."""
        kc = fp8_e4m3_value(k_codes) * np.asarray(k_scale, np.float64)[:, None, :, None]
        vc = fp8_e4m3_value(v_codes) * np.asarray(v_scale, np.float64)[:, None, :, None]
        qb = self._arr(q, "bf16").astype(np.uint32) << np.uint32(16)   # bf16 bits -> fp32 bits
        qf = qb.view(np.float32).astype(np.float64)
        return self.prefill_paged(qf, kc, vc, block_table, seq_lens, cu_seqlens_q, dtype="f64", scale=scale,
                                  causal=causal, window=window, rows=rows, key_range=key_range)

    def decode_paged_fp8(self, q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, *, scale,
                         seqs=None, window_left=None, alibi_slopes=None):
        """Paged decode over FP8 caches (E4M3 codes [P, page_size, A_kv, d] with
        per-(page, KV head) scales [P, A_kv]); q bf16 bits [B, A, d].  The cache
        values code value * scale are formed in fp64 for the pages each sequence
        uses, and the sequence runs through decode_paged (with its window,
        window_left as there).  Returns (o [n, A, d], lse [n, A]) for the
        sequences ``seqs`` (default: all)."""
        B, A, d = q.shape
        bt = np.asarray(block_table)
        sl = np.asarray(seq_lens)
        ps = k_codes.shape[1]
        seqs = range(B) if seqs is None else list(seqs)
        qb = self._arr(q, "bf16").astype(np.uint32) << np.uint32(16)   # bf16 bits -> fp32 bits
        qf = qb.view(np.float32).astype(np.float64)
        outs, lses = [], []
        for b in seqs:
            n = int((int(sl[b]) + ps - 1) // ps)
            pages = bt[b, :max(n, 1)].astype(np.int64) if n else np.zeros(1, np.int64)
            kc = fp8_e4m3_value(k_codes[pages]) * np.asarray(k_scale, np.float64)[pages][:, None, :, None]
            vc = fp8_e4m3_value(v_codes[pages]) * np.asarray(v_scale, np.float64)[pages][:, None, :, None]
            o, lse = self.decode_paged(qf[b:b + 1], kc, vc, np.arange(pages.size, dtype=np.int32)[None],
                                       np.array([sl[b]], np.int32), dtype="f64", scale=scale,
                                       window_left=window_left, alibi_slopes=alibi_slopes)
            outs.append(o.reshape(A, d))
            lses.append(lse.reshape(A))
        return np.stack(outs), np.stack(lses)

    def decode_paged(self, q, k_cache, v_cache, block_table, seq_lens, *, dtype, scale, rows=None, window_left=None,
                     alibi_slopes=None):
        """Paged decode.  q [B,A,d]; caches [P, page_size, A_kv, d]; rows = b*A + h.
        window_left: the query (position seq_lens[b] - 1) sees keys t >=
        seq_lens[b] - 1 - window_left; None = every key.  alibi_slopes: [A]; the
        decode row is then the one-row chunk of each sequence in prefill_paged
        (the query at position seq_lens[b] - 1)."""
        if alibi_slopes is not None:
            return self._decode_as_chunks(q, k_cache, v_cache, block_table, seq_lens, dtype=dtype, scale=scale,
                                          rows=rows, window_left=window_left, alibi_slopes=alibi_slopes)
        q, kc, vc = self._arr(q, dtype), self._arr(k_cache, dtype), self._arr(v_cache, dtype)
        if q.ndim != 3 or kc.ndim != 4 or kc.shape != vc.shape:
            raise ValueError("q [B,A,d]; caches [num_pages, page_size, A_kv, d]")
        B, A, d = q.shape
        num_pages, page_size, A_kv, dk = kc.shape
        if dk != d or A % A_kv:
            raise ValueError("cache head dim / head count mismatch")
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if bt.ndim != 2 or bt.shape[0] != B or sl.shape != (B,):
            raise ValueError("block_table [B, max_pages], seq_lens [B]")
        r, n = self._rows(rows)
        n_out = B * A if r is None else n
        o = np.empty((n_out, d), dtype=np.float64)
        lse = np.empty(n_out, dtype=np.float64)
        wl = -1 if window_left is None else int(window_left)
        rc = self.lib.oracle_decode_paged(_ptr(q), _ptr(kc), _ptr(vc), _DT[dtype], _ptr(bt), _ptr(sl), B, A,
                                          A_kv, d, page_size, bt.shape[1], num_pages, float(scale), wl, _ptr(r), n,
                                          _ptr(o), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle_decode_paged rejected its arguments")
        if r is None:
            return o.reshape(B, A, d), lse.reshape(B, A)
        return o, lse


    def _decode_as_chunks(self, q, k_cache, v_cache, block_table, seq_lens, *, dtype, scale, rows, window_left,
                          alibi_slopes):
        B, A, d = np.asarray(q).shape
        sl = np.asarray(seq_lens, dtype=np.int32)
        live = sl > 0
        cu = np.concatenate([[0], np.cumsum(live.astype(np.int32))]).astype(np.int32)
        qc = np.ascontiguousarray(np.asarray(q)[live].transpose(1, 0, 2))   # [A, chunk rows, d]
        window = None if window_left is None else (int(window_left), 0)
        o = np.zeros((B, A, d), np.float64)
        lse = np.full((B, A), -np.inf, np.float64)
        if qc.shape[1]:
            oc, lc = self.prefill_paged(qc, k_cache, v_cache, block_table, sl, cu, dtype=dtype, scale=scale,
                                        causal=True, window=window, alibi_slopes=alibi_slopes)
            o[live] = oc.transpose(1, 0, 2)
            lse[live] = lc.T
        if rows is not None:
            r = np.asarray(rows, np.int64).reshape(-1)
            return o.reshape(B * A, d)[r], lse.reshape(-1)[r]
        return o, lse


_default = None


def fp8_e4m3_value(codes) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes (uint8) in fp64: sign bit 7, exponent bits
    6..3 with bias 7, mantissa bits 2..0; exponent 0 is subnormal
    (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def window_keep(B: int, S_q: int, S_k: int, left: int, right: int) -> np.ndarray:
    """Dense keep matrix [B, S_q, S_k] of a sliding window around each query's
    position i + (S_k - S_q) (bottom-right alignment, as for causal): key j is
    kept when i + off - left <= j <= i + off + right; -1 leaves that side
    unbounded.  Page "Attention Kernel", section "可编程 mask" (sliding window
    as an element rule)."""
    off = S_k - S_q
    i = np.arange(S_q, dtype=np.int64)[:, None] + off
    j = np.arange(S_k, dtype=np.int64)[None, :]
    keep = np.ones((S_q, S_k), dtype=bool)
    if left >= 0:
        keep &= j >= i - left
    if right >= 0:
        keep &= j <= i + right
    return np.broadcast_to(keep.astype(np.uint8), (B, S_q, S_k)).copy()


def alibi_term(slopes, B: int, S_q: int, S_k: int, positions=None) -> np.ndarray:
    """ALiBi as the additive term M, fp32 [B, A, S_q, S_k]: M[b, h, i, j] =
    -slopes[h] * |p_i - j|, with query i at the bottom-right aligned position
    p_i = i + S_k - S_q (as for causal), or at positions[i] when given (a
    packed chunk's positions in its sequence).  Page "Attention Kernel",
    section "正确性契约": ALiBi is one of the transforms fused into the score
    (a linear penalty on the query-key distance, per head); it enters the
    score like any additive term, after the scaling of q . k."""
    sl = np.asarray(slopes, dtype=np.float64).reshape(-1)
    p = (np.arange(S_q, dtype=np.int64) + (S_k - S_q)) if positions is None else np.asarray(positions, np.int64)
    dist = np.abs(p[:, None] - np.arange(S_k, dtype=np.int64)[None, :]).astype(np.float64)
    m = -sl[:, None, None] * dist[None]
    return np.broadcast_to(m.astype(np.float32)[None], (B, sl.size, S_q, S_k)).copy()


def key_range_keep(key_range, S_k: int) -> np.ndarray:
    """Dense keep matrix [..., S_q, S_k] of per-row key ranges: row i keeps
    key j when key_range[..., i, 0] <= j <= key_range[..., i, 1] (both ends
    included; a first end past the last keeps no key).  Page "Attention
    Kernel", section "可编程 mask": document boundaries (a row keeps the keys
    of its own document) and prefix-LM (rows of the prefix see the whole
    prefix) are element rules of this form."""
    r = np.asarray(key_range, dtype=np.int64)
    j = np.arange(S_k, dtype=np.int64)
    return ((j >= r[..., 0:1]) & (j <= r[..., 1:2])).astype(np.uint8)


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
