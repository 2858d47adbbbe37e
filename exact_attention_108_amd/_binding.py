"""ctypes marshalling for libattn_mi355x.so (argument checks + pointers only)."""
from __future__ import annotations

import ctypes
import os

import numpy as np
# torch first: its wheel carries its own libamdhip64.so.7.  Loading torch before
# the library makes the library's libamdhip64.so.7 dependency resolve to that
# same, already-loaded runtime, so device pointers and streams handed over from
# torch belong to the runtime that launches the kernels.  Loading the library
# first would bring in a second HIP runtime for torch.
import torch  # noqa: F401

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python exact_attention_108_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

ATTN_OK, ATTN_ERR_INVAL, ATTN_ERR_UNSUPPORTED, ATTN_ERR_LAUNCH = 0, 1, 2, 3
ATTN_F32, ATTN_BF16 = 0, 1


class _Mask(ctypes.Structure):
    _fields_ = [("q_keep", ctypes.c_void_p), ("k_keep", ctypes.c_void_p), ("block_keep", ctypes.c_void_p),
                ("block_heads", ctypes.c_int), ("bias", ctypes.c_void_p), ("bias_heads", ctypes.c_int),
                ("bias_ld", ctypes.c_int), ("key_range", ctypes.c_void_p), ("alibi_slopes", ctypes.c_void_p)]


class _Window(ctypes.Structure):
    _fields_ = [("left", ctypes.c_int), ("right", ctypes.c_int)]


_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_WP = ctypes.POINTER(_Window)
_lib.attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, ctypes.POINTER(_Mask), _WP, _i,
                          _vp]
_lib.attn_fwd.restype = _i
_lib.attn_fwd_fp8.argtypes = [_vp] * 7 + [_i] * 6 + [_f, _i, ctypes.POINTER(_Mask), _WP, _vp]
_lib.attn_fwd_fp8.restype = _i
_lib.attn_fwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                 ctypes.POINTER(_Mask), _WP, _i, _vp]
_lib.attn_fwd_varlen.restype = _i
_lib.attn_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                                   _vp, _sz, _vp]
_lib.attn_decode_paged.restype = _i
_lib.attn_decode_paged_window.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                          _i, _i, _vp, _sz, _vp]
_lib.attn_decode_paged_window.restype = _i
_lib.attn_decode_paged_alibi.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                         _i, _vp, _i, _vp, _sz, _vp]
_lib.attn_decode_paged_alibi.restype = _i
_lib.attn_decode_paged_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                           _i, _vp]
_lib.attn_decode_paged_noalloc.restype = _i
_lib.attn_decode_paged_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _vp]
_lib.attn_decode_paged_workspace_bytes.restype = _sz
_lib.attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                          ctypes.POINTER(_Mask), _WP, _i, _vp, _sz, _vp]
_lib.attn_bwd.restype = _i
_lib.attn_bwd_varlen.argtypes = [_vp] * 11 + [_i] * 5 + [_f, _i, ctypes.POINTER(_Mask), _WP, _i, _vp, _sz, _vp]
_lib.attn_bwd_varlen.restype = _i
_lib.attn_bwd_workspace_bytes.argtypes = [_i, _i, _i]
_lib.attn_prefill_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                    _f, _i, _WP, _i, _vp]
_lib.attn_prefill_paged.restype = _i
_lib.attn_prefill_paged_masked.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i,
                                           _i, _i, _f, _i, ctypes.POINTER(_Mask), _WP, _i, _vp]
_lib.attn_prefill_paged_masked.restype = _i
_lib.attn_prefill_paged_fp8.argtypes = [_vp] * 10 + [_i, _vp, _vp] + [_i] * 7 + [_f, _i, _WP, _vp]
_lib.attn_prefill_paged_fp8.restype = _i
_lib.attn_bwd_workspace_bytes.restype = _sz
_lib.attn_decode_paged_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                       _f, _vp, _sz, _vp]
_lib.attn_decode_paged_fp8.restype = _i
_lib.attn_decode_paged_fp8_window.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i,
                                              _i, _f, _i, _vp, _sz, _vp]
_lib.attn_decode_paged_fp8_window.restype = _i
_lib.attn_decode_paged_fp8_alibi.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i,
                                             _i, _f, _i, _vp, _vp, _sz, _vp]
_lib.attn_decode_paged_fp8_alibi.restype = _i
_lib.attn_status_string.argtypes = [_i]
_lib.attn_status_string.restype = ctypes.c_char_p
_lib.attn_abi_version.argtypes = []
_lib.attn_abi_version.restype = _i
_lib.attn_block_keep_from_bias.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp]
_lib.attn_block_keep_from_bias.restype = _i


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")
        self.status = status


def attn_status_string(status: int) -> str:
    return _lib.attn_status_string(int(status)).decode()


def attn_abi_version() -> int:
    return int(_lib.attn_abi_version())


def exported_symbols():
    """Names of the C entry points this binding resolves (one per header declaration)."""
    return ["attn_fwd", "attn_fwd_fp8", "attn_fwd_varlen", "attn_decode_paged", "attn_decode_paged_noalloc",
            "attn_decode_paged_window", "attn_prefill_paged_masked",
            "attn_decode_paged_workspace_bytes",
            "attn_bwd", "attn_bwd_varlen", "attn_bwd_workspace_bytes", "attn_prefill_paged", "attn_prefill_paged_fp8", "attn_decode_paged_fp8",
            "attn_decode_paged_fp8_window", "attn_decode_paged_alibi", "attn_decode_paged_fp8_alibi",
            "attn_block_keep_from_bias", "attn_status_string", "attn_abi_version"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else None


def _view_ptr(t):
    """Data pointer of a strided view whose layout the caller has checked."""
    if t is None or t.numel() == 0:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must share one device")
    return dev


def _stream(stream, dev):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream)


def _bias_view(bias, B, A, S_q, S_k):
    """(heads, row stride) of a dense additive mask: an fp32 [B, 1 or A, S_q, S_k]
    tensor whose rows are unit-stride and ld elements apart (ld a multiple of
    4, e.g. a [..., :S_k] slice of a padded tensor) and whose heads and batch
    rows are packed at that stride."""
    torch = _torch()
    if bias.dtype != torch.float32 or bias.dim() != 4:
        raise ValueError("bias must be fp32 [B, 1 or A, S_q, S_k]")
    if bias.shape[0] != B or bias.shape[1] not in (1, A) or tuple(bias.shape[2:]) != (S_q, S_k):
        raise ValueError("bias must be [B, 1 or A, S_q, S_k]")
    heads = int(bias.shape[1])
    ld = int(bias.stride(2))
    if (S_k > 1 and bias.stride(3) != 1) or ld % 4 or ld < S_k:
        raise ValueError("bias rows must be unit-stride, ld >= S_k apart with ld a multiple of 4")
    if (heads > 1 and bias.stride(1) != S_q * ld) or (B > 1 and bias.stride(0) != heads * S_q * ld):
        raise ValueError("bias heads and batch rows must be packed at the row stride")
    return heads, ld


def _mask(q_keep, k_keep, block_keep=None, bias=None, bias_heads=0, bias_ld=0, key_range=None, alibi_slopes=None):
    torch = _torch()
    for t in (q_keep, k_keep, block_keep):
        if t is not None and t.dtype != torch.uint8:
            raise ValueError("keep-masks must be uint8")
    if key_range is not None and key_range.dtype != torch.int32:
        raise ValueError("key_range must be int32 (first, last) pairs")
    if alibi_slopes is not None and alibi_slopes.dtype != torch.float32:
        raise ValueError("alibi_slopes must be fp32 [A]")
    if q_keep is None and k_keep is None and block_keep is None and bias is None and key_range is None and \
            alibi_slopes is None:
        return None
    heads = 0 if block_keep is None else int(block_keep.shape[1])
    return ctypes.byref(_Mask(_ptr(q_keep), _ptr(k_keep), _ptr(block_keep), heads, _view_ptr(bias), bias_heads,
                             bias_ld, _ptr(key_range), _ptr(alibi_slopes)))


def _check_slopes(alibi_slopes, A):
    if alibi_slopes is not None and tuple(alibi_slopes.shape) != (A,):
        raise ValueError(f"alibi_slopes must be fp32 [{A}]")


def _check_key_range(key_range, shape):
    if key_range is not None and tuple(key_range.shape) != tuple(shape):
        raise ValueError(f"key_range must be int32 {list(shape)}")


def _window(window):
    """None, or (left, right) with -1 for an unbounded side."""
    if window is None:
        return None
    left, right = window
    return ctypes.byref(_Window(int(left), int(right)))


def _check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)


def attn_fwd(q, k, v, o, lse, *, scale: float, causal: bool = False, q_keep=None, k_keep=None, window=None,
             block_keep=None, bias=None, key_range=None, alibi_slopes=None, stream=None):
    """O, LSE of softmax(Q K^T * scale + M) V.  q/o [B,A,S_q,d], k/v [B,A_kv,S_k,d], lse [B,A,S_q] fp32;
    window = (left, right) sliding window around each query's position, -1 = unbounded side;
    key_range = int32 [B, S_q, 2]: row i keeps keys first..last only (documents, prefix-LM);
    alibi_slopes = fp32 [A]: ALiBi, -slope_h |p_i - j| joins M;
    block_keep = uint8 [B, 1 or A, ceil(S_q/128), ceil(S_k/128)] block mask (bf16 only);
    bias = the dense additive term M, fp32 [B, 1 or A, S_q, S_k] (finite or -inf; rows unit-stride and
    a multiple of 4 elements apart, see pad_bias)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, heads, S, d]")
    B, A, S_q, d = q.shape
    _, A_kv, S_k, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k, v must be [B, A_kv, S_k, d]")
    if o.shape != q.shape or o.dtype != q.dtype or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("o must match q; k, v must share q's dtype")
    if lse.shape != (B, A, S_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, A, S_q]")
    if q_keep is not None and q_keep.shape != (B, S_q):
        raise ValueError("q_keep must be [B, S_q]")
    if k_keep is not None and k_keep.shape != (B, S_k):
        raise ValueError("k_keep must be [B, S_k]")
    if block_keep is not None and (block_keep.dim() != 4 or block_keep.shape[0] != B or
                                   block_keep.shape[1] not in (1, A) or
                                   tuple(block_keep.shape[2:]) != ((S_q + 127) // 128, (S_k + 127) // 128)):
        raise ValueError("block_keep must be [B, 1 or A, ceil(S_q/128), ceil(S_k/128)]")
    bh, ld = _bias_view(bias, B, A, S_q, S_k) if bias is not None else (0, 0)
    _check_key_range(key_range, (B, S_q, 2))
    _check_slopes(alibi_slopes, A)
    dev = _dev(q, k, v, o, lse, q_keep, k_keep, block_keep, bias, key_range, alibi_slopes)
    st = _lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, A, A_kv, S_q, S_k, d, float(scale),
                       int(bool(causal)), _mask(q_keep, k_keep, block_keep, bias, bh, ld, key_range, alibi_slopes),
                       _window(window), _dtype_code(q), _stream(stream, dev))
    _check(st, "attn_fwd")


def attn_fwd_fp8(q, k, v, o, lse, q_scale, k_scale, *, scale: float, causal: bool = False, q_keep=None,
                 k_keep=None, window=None, key_range=None, stream=None):
    """attn_fwd with E4M3 queries and keys: q uint8 [B,A,S_q,128], k uint8 [B,A_kv,S_k,128] (code bytes),
    q_scale fp32 [B,A,ceil(S_q/128)], k_scale fp32 [B,A_kv,ceil(S_k/128)] (one scale per 128 tokens);
    v bf16 [B,A_kv,S_k,128]; o bf16 like q; lse fp32 [B,A,S_q]."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, heads, S, d]")
    B, A, S_q, d = q.shape
    _, A_kv, S_k, _ = k.shape
    if q.dtype != torch.uint8 or k.dtype != torch.uint8 or v.dtype != torch.bfloat16 or o.dtype != torch.bfloat16:
        raise ValueError("q, k: uint8 E4M3 codes; v, o: bf16")
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape or tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    if lse.shape != (B, A, S_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, A, S_q]")
    if q_scale.dtype != torch.float32 or tuple(q_scale.shape) != (B, A, (S_q + 127) // 128):
        raise ValueError("q_scale must be fp32 [B, A, ceil(S_q/128)]")
    if k_scale.dtype != torch.float32 or tuple(k_scale.shape) != (B, A_kv, (S_k + 127) // 128):
        raise ValueError("k_scale must be fp32 [B, A_kv, ceil(S_k/128)]")
    if q_keep is not None and q_keep.shape != (B, S_q):
        raise ValueError("q_keep must be [B, S_q]")
    if k_keep is not None and k_keep.shape != (B, S_k):
        raise ValueError("k_keep must be [B, S_k]")
    _check_key_range(key_range, (B, S_q, 2))
    dev = _dev(q, k, v, o, lse, q_scale, k_scale, q_keep, k_keep, key_range)
    st = _lib.attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(q_scale), _ptr(k_scale), B, A, A_kv,
                           S_q, S_k, d, float(scale), int(bool(causal)),
                           _mask(q_keep, k_keep, key_range=key_range), _window(window), _stream(stream, dev))
    _check(st, "attn_fwd_fp8")


def pad_bias(bias):
    """An fp32 [B, H, S_q, S_k] tensor as the [..., :S_k] view of a zero-padded copy whose rows are a
    multiple of 4 elements long (the layout attn_fwd and attn_block_keep_from_bias read)."""
    torch = _torch()
    B, H, S_q, S_k = bias.shape
    ld = max(4, (S_k + 3) // 4 * 4)
    out = torch.zeros((B, H, S_q, ld), dtype=torch.float32, device=bias.device)
    out[..., :S_k] = bias
    return out[..., :S_k]


def attn_block_keep_from_bias(bias, block_keep, *, stream=None):
    """block_keep uint8 [B, H, ceil(S_q/128), ceil(S_k/128)] = whether each 128 x 128 block of the fp32
    bias [B, H, S_q, S_k] (layout as attn_fwd's bias) holds an entry greater than -inf."""
    torch = _torch()
    if bias.dim() != 4:
        raise ValueError("bias must be [B, H, S_q, S_k]")
    B, H, S_q, S_k = bias.shape
    bh, ld = _bias_view(bias, B, H, S_q, S_k)
    if block_keep.dtype != torch.uint8 or tuple(block_keep.shape) != (B, bh, (S_q + 127) // 128,
                                                                      (S_k + 127) // 128):
        raise ValueError("block_keep must be uint8 [B, H, ceil(S_q/128), ceil(S_k/128)]")
    if not block_keep.is_contiguous():
        raise ValueError("block_keep must be contiguous")
    dev = _dev(bias, block_keep)
    st = _lib.attn_block_keep_from_bias(_view_ptr(bias), B, bh, S_q, S_k, ld, _ptr(block_keep), _stream(stream, dev))
    _check(st, "attn_block_keep_from_bias")


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, cu_seqlens_host, *, scale: float, causal: bool = True,
                    q_keep=None, k_keep=None, window=None, block_keep=None, bias=None, key_range=None,
                    alibi_slopes=None, stream=None):
    """Packed varlen prefill.  q/o [A,T,d], k/v [A_kv,T,d], lse [A,T]; cu_seqlens int32 device,
    cu_seqlens_host the same values on the host (numpy int32).  bf16 only: block_keep uint8
    [n_seq, 1 or A, nb, nb] (nb = ceil(longest length / 128)), each sequence's own 128 x 128 blocks;
    bias fp32 [1 or A, T, L] (L = the longest length; row t = token t against the keys at positions
    j < len of its sequence; rows unit-stride and a multiple of 4 elements apart); key_range int32
    [T, 2], token t's (first, last) key positions within its sequence."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("q [A,T,d], k/v [A_kv,T,d]")
    A, T, d = q.shape
    A_kv = k.shape[0]
    if k.shape[1] != T or k.shape[2] != d or o.shape != q.shape or lse.shape != (A, T):
        raise ValueError("shape mismatch")
    if lse.dtype != torch.float32 or o.dtype != q.dtype or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    cu_host = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    n_seq = cu_host.size - 1
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.numel() != cu_host.size:
        raise ValueError("cu_seqlens must be int32 [n_seq + 1] matching cu_seqlens_host")
    for t in (q_keep, k_keep):
        if t is not None and t.shape != (T,):
            raise ValueError("keep-masks must be [T]")
    bh, ld = _packed_masks(block_keep, bias, cu_host, A, T)
    _check_key_range(key_range, (T, 2))
    _check_slopes(alibi_slopes, A)
    dev = _dev(q, k, v, o, lse, cu_seqlens, q_keep, k_keep, block_keep, bias, key_range, alibi_slopes)
    st = _lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                              cu_host.ctypes.data_as(_vp), n_seq, T, A, A_kv, d, float(scale), int(bool(causal)),
                              _mask(q_keep, k_keep, block_keep, bias, bh, ld, key_range, alibi_slopes),
                              _window(window), _dtype_code(q), _stream(stream, dev))
    _check(st, "attn_fwd_varlen")


def _packed_masks(block_keep, bias, cu_host, A, T):
    """Checks the packed-sequence block mask [n_seq, 1 or A, nb, nb] and term
    [1 or A, T, longest length]; returns the term's (heads, row stride)."""
    torch = _torch()
    n_seq = cu_host.size - 1
    max_len = int(np.diff(cu_host).max()) if n_seq > 0 else 0
    nb = (max_len + 127) // 128
    if block_keep is not None and (block_keep.dim() != 4 or block_keep.shape[0] != n_seq or
                                   block_keep.shape[1] not in (1, A) or tuple(block_keep.shape[2:]) != (nb, nb)):
        raise ValueError(f"block_keep must be [n_seq, 1 or A, {nb}, {nb}]")
    bh, ld = 0, 0
    if bias is not None:
        if bias.dtype != torch.float32 or bias.dim() != 3 or bias.shape[0] not in (1, A) or \
                tuple(bias.shape[1:]) != (T, max_len):
            raise ValueError(f"bias must be fp32 [1 or A, T, {max_len}]")
        bh, ld = int(bias.shape[0]), int(bias.stride(1))
        if (max_len > 1 and bias.stride(2) != 1) or ld % 4 or ld < max_len or (bh > 1 and bias.stride(0) != T * ld):
            raise ValueError("bias rows must be unit-stride, a multiple of 4 elements apart, heads packed")
    return bh, ld


def attn_decode_paged_workspace_bytes(B: int, A: int, A_kv: int, d: int, page_size: int, seq_lens_host) -> int:
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if sl.shape != (B,):
        raise ValueError("seq_lens_host must be [B]")
    return int(_lib.attn_decode_paged_workspace_bytes(B, A, A_kv, d, page_size, sl.ctypes.data_as(_vp)))


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse, workspace, *,
                      scale: float, stream=None):
    """Paged decode.  q/o [B,A,d]; caches [num_pages, page_size, A_kv, d]; block_table int32 [B, max_pages];
    seq_lens int32 [B] (device) and seq_lens_host (numpy); workspace a uint8 device tensor of at least
    attn_decode_paged_workspace_bytes(...) bytes."""
    _decode_call("attn_decode_paged", q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse, workspace,
                 scale, None, stream)


def attn_decode_paged_window(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse, workspace, *,
                             scale: float, window_left: int, stream=None):
    """attn_decode_paged where the query (position seq_lens[b] - 1) sees the keys t >= seq_lens[b] - 1 -
    window_left; window_left = -1 sees every key."""
    _decode_call("attn_decode_paged_window", q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse,
                 workspace, scale, int(window_left), stream)


def attn_decode_paged_alibi(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse, workspace, *,
                            scale: float, alibi_slopes, window_left: int = -1, stream=None):
    """attn_decode_paged_window with ALiBi: alibi_slopes fp32 [A]; key t of sequence b gets
    -slope_h (seq_lens[b] - 1 - t) on its score."""
    _decode_call("attn_decode_paged_alibi", q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse,
                 workspace, scale, int(window_left), stream, alibi_slopes)


def _decode_call(name, q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse, workspace, scale,
                 window_left, stream, alibi_slopes=None):
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [B,A,d]; caches [num_pages, page_size, A_kv, d]")
    B, A, d = q.shape
    num_pages, page_size, A_kv, dk = k_cache.shape
    if dk != d or o.shape != q.shape or lse.shape != (B, A) or lse.dtype != torch.float32:
        raise ValueError("shape mismatch")
    if o.dtype != q.dtype or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if sl.shape != (B,):
        raise ValueError("seq_lens_host must be [B]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (A,)):
        raise ValueError(f"alibi_slopes must be fp32 [{A}]")
    dev = _dev(q, k_cache, v_cache, block_table, seq_lens, o, lse, workspace, alibi_slopes)
    args = [_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), sl.ctypes.data_as(_vp),
            page_size, _ptr(o), _ptr(lse), B, A, A_kv, d, block_table.shape[1], num_pages, float(scale)]
    if window_left is not None:
        args.append(window_left)
    if alibi_slopes is not None:
        args.append(_ptr(alibi_slopes))
    st = getattr(_lib, name)(*args, _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream, dev))
    _check(st, name)


DECODE_NOALLOC_MAX_BYTES = 48 << 20


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, o, lse, *, scale: float,
                              stream=None):
    """attn_decode_paged with the split partials in the library's static per-device array (no allocation;
    calls that overlap on one device race).  Raises AttnError (unsupported) when the workspace the call needs,
    attn_decode_paged_workspace_bytes(...), exceeds DECODE_NOALLOC_MAX_BYTES."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [B,A,d]; caches [num_pages, page_size, A_kv, d]")
    B, A, d = q.shape
    num_pages, page_size, A_kv, dk = k_cache.shape
    if dk != d or o.shape != q.shape or lse.shape != (B, A) or lse.dtype != torch.float32:
        raise ValueError("shape mismatch")
    if o.dtype != q.dtype or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if sl.shape != (B,):
        raise ValueError("seq_lens_host must be [B]")
    dev = _dev(q, k_cache, v_cache, block_table, seq_lens, o, lse)
    st = _lib.attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                        sl.ctypes.data_as(_vp), page_size, _ptr(o), _ptr(lse), B, A, A_kv, d,
                                        block_table.shape[1], num_pages, float(scale), _dtype_code(q),
                                        _stream(stream, dev))
    if st == ATTN_ERR_UNSUPPORTED:
        need = attn_decode_paged_workspace_bytes(B, A, A_kv, d, page_size, sl)
        if need > DECODE_NOALLOC_MAX_BYTES:
            raise AttnError(st, f"attn_decode_paged_noalloc: needs {need} bytes of split workspace, more than the "
                                f"static {DECODE_NOALLOC_MAX_BYTES}")
    _check(st, "attn_decode_paged_noalloc")


def attn_bwd_workspace_bytes(B: int, A: int, S_q: int) -> int:
    return int(_lib.attn_bwd_workspace_bytes(B, A, S_q))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, *, scale: float, causal: bool = False, q_keep=None,
             k_keep=None, window=None, block_keep=None, bias=None, key_range=None, alibi_slopes=None, stream=None):
    """dQ, dK, dV of attn_fwd.  q/o/dout/dq [B,A,S_q,d], k/v/dk/dv [B,A_kv,S_k,d], lse [B,A,S_q] fp32 (the
    forward's); workspace a uint8 device tensor of at least attn_bwd_workspace_bytes(B, A, S_q) bytes; masks as
    given to attn_fwd."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, heads, S, d]")
    B, A, S_q, d = q.shape
    _, A_kv, S_k, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k, v must be [B, A_kv, S_k, d]")
    for t in (o, dout, dq):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("o, dout, dq must match q")
    for t in (dk, dv):
        if t.shape != k.shape or t.dtype != q.dtype:
            raise ValueError("dk, dv must match k")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k, v must share q's dtype")
    if lse.shape != (B, A, S_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, A, S_q]")
    if q_keep is not None and q_keep.shape != (B, S_q):
        raise ValueError("q_keep must be [B, S_q]")
    if k_keep is not None and k_keep.shape != (B, S_k):
        raise ValueError("k_keep must be [B, S_k]")
    if block_keep is not None and (block_keep.dim() != 4 or block_keep.shape[0] != B or
                                   block_keep.shape[1] not in (1, A) or
                                   tuple(block_keep.shape[2:]) != ((S_q + 127) // 128, (S_k + 127) // 128)):
        raise ValueError("block_keep must be [B, 1 or A, ceil(S_q/128), ceil(S_k/128)]")
    bh, ld = _bias_view(bias, B, A, S_q, S_k) if bias is not None else (0, 0)
    _check_key_range(key_range, (B, S_q, 2))
    _check_slopes(alibi_slopes, A)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dev = _dev(q, k, v, o, dout, lse, dq, dk, dv, workspace, q_keep, k_keep, block_keep, bias, key_range, alibi_slopes)
    st = _lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                       B, A, A_kv, S_q, S_k, d, float(scale), int(bool(causal)),
                       _mask(q_keep, k_keep, block_keep, bias, bh, ld, key_range, alibi_slopes), _window(window),
                       _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream, dev))
    _check(st, "attn_bwd")


def attn_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, cu_seqlens_host, workspace, *, scale: float,
                    causal: bool = True, q_keep=None, k_keep=None, window=None, block_keep=None, bias=None,
                    key_range=None, alibi_slopes=None, stream=None):
    """dQ, dK, dV of attn_fwd_varlen.  q/o/dout/dq [A,T,d], k/v/dk/dv [A_kv,T,d], lse [A,T] fp32 (the
    forward's); cu_seqlens int32 device with cu_seqlens_host (numpy); workspace a uint8 device tensor of at
    least attn_bwd_workspace_bytes(1, A, T) bytes; block_keep, bias and key_range as attn_fwd_varlen takes
    them."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("q [A,T,d], k/v [A_kv,T,d]")
    A, T, d = q.shape
    A_kv = k.shape[0]
    if k.shape[1] != T or k.shape[2] != d:
        raise ValueError("k/v must be [A_kv, T, d]")
    for t in (o, dout, dq):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("o, dout, dq must match q")
    for t in (dk, dv):
        if t.shape != k.shape or t.dtype != q.dtype:
            raise ValueError("dk, dv must match k")
    if k.dtype != q.dtype or v.dtype != q.dtype or lse.shape != (A, T) or lse.dtype != torch.float32:
        raise ValueError("dtype / lse mismatch")
    cu_host = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    n_seq = cu_host.size - 1
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.numel() != cu_host.size:
        raise ValueError("cu_seqlens must be int32 [n_seq + 1] matching cu_seqlens_host")
    for t in (q_keep, k_keep):
        if t is not None and t.shape != (T,):
            raise ValueError("keep-masks must be [T]")
    bh, ld = _packed_masks(block_keep, bias, cu_host, A, T)
    _check_key_range(key_range, (T, 2))
    _check_slopes(alibi_slopes, A)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dev = _dev(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, workspace, q_keep, k_keep, block_keep, bias, key_range,
               alibi_slopes)
    st = _lib.attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(cu_seqlens), cu_host.ctypes.data_as(_vp), n_seq, T, A, A_kv, d,
                              float(scale), int(bool(causal)),
                              _mask(q_keep, k_keep, block_keep, bias, bh, ld, key_range, alibi_slopes),
                              _window(window),
                              _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream, dev))
    _check(st, "attn_bwd_varlen")


def attn_prefill_paged(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, cu_seqlens_q, cu_seqlens_q_host,
                       o, lse, *, scale: float, causal: bool = True, window=None, stream=None):
    """Prefill of packed query chunks q/o [A,T_q,d] (lse [A,T_q]) over a paged cache [num_pages, page_size,
    A_kv, d]; block_table int32 [n_seq, max_pages]; seq_lens int32 [n_seq] (device) with seq_lens_host; chunk
    boundaries cu_seqlens_q int32 [n_seq+1] (device) with cu_seqlens_q_host."""
    _paged_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, cu_seqlens_q, cu_seqlens_q_host, o, lse,
                scale, causal, window, stream, None, None)


def attn_prefill_paged_masked(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, cu_seqlens_q,
                              cu_seqlens_q_host, o, lse, *, scale: float, causal: bool = True, window=None,
                              block_keep=None, bias=None, key_range=None, alibi_slopes=None, stream=None):
    """attn_prefill_paged with block_keep uint8 [n_seq, 1 or A, ceil(longest chunk/128), ceil(longest
    seq_len/128)] over (chunk rows, key positions) and bias fp32 [1 or A, T_q, L] (L = the longest
    seq_len; row t = chunk token t against the key positions of its sequence; rows unit-stride and a
    multiple of 4 elements apart); key_range int32 [T_q, 2], chunk token t's (first, last) key positions
    in its sequence's cache; alibi_slopes fp32 [A] (chunk rows at the bottom of their sequence)."""
    _paged_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, cu_seqlens_q, cu_seqlens_q_host, o, lse,
                scale, causal, window, stream, block_keep, bias, key_range, alibi_slopes)


def _paged_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, cu_seqlens_q, cu_seqlens_q_host, o, lse,
                scale, causal, window, stream, block_keep, bias, key_range=None, alibi_slopes=None):
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [A,T_q,d]; caches [num_pages, page_size, A_kv, d]")
    A, T_q, d = q.shape
    num_pages, page_size, A_kv, dk = k_cache.shape
    if dk != d or o.shape != q.shape or lse.shape != (A, T_q) or lse.dtype != torch.float32:
        raise ValueError("shape mismatch")
    if o.dtype != q.dtype or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    cu_host = np.ascontiguousarray(cu_seqlens_q_host, dtype=np.int32)
    n_seq = cu_host.size - 1
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if sl.shape != (n_seq,) or seq_lens.dtype != torch.int32 or seq_lens.shape != (n_seq,):
        raise ValueError("seq_lens must be int32 [n_seq]")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_q.numel() != cu_host.size:
        raise ValueError("cu_seqlens_q must be int32 [n_seq + 1]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != n_seq:
        raise ValueError("block_table must be int32 [n_seq, max_pages]")
    _check_key_range(key_range, (T_q, 2))
    _check_slopes(alibi_slopes, A)
    dev = _dev(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, o, lse, block_keep, bias, key_range,
               alibi_slopes)
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), sl.ctypes.data_as(_vp),
            _ptr(cu_seqlens_q), cu_host.ctypes.data_as(_vp), page_size, _ptr(o), _ptr(lse), n_seq, T_q, A, A_kv, d,
            block_table.shape[1], num_pages, float(scale), int(bool(causal)))
    if block_keep is None and bias is None and key_range is None and alibi_slopes is None:
        st = _lib.attn_prefill_paged(*head, _window(window), _dtype_code(q), _stream(stream, dev))
        _check(st, "attn_prefill_paged")
        return
    max_q = int(np.diff(cu_host).max()) if n_seq > 0 else 0
    max_l = int(sl.max()) if n_seq > 0 else 0
    want = (n_seq, (max_q + 127) // 128, (max_l + 127) // 128)
    if block_keep is not None and (block_keep.dim() != 4 or block_keep.shape[0] != n_seq or
                                   block_keep.shape[1] not in (1, A) or tuple(block_keep.shape[2:]) != want[1:]):
        raise ValueError(f"block_keep must be [n_seq, 1 or A, {want[1]}, {want[2]}]")
    bh, ld = 0, 0
    if bias is not None:
        if bias.dtype != torch.float32 or bias.dim() != 3 or bias.shape[0] not in (1, A) or \
                tuple(bias.shape[1:]) != (T_q, max_l):
            raise ValueError(f"bias must be fp32 [1 or A, T_q, {max_l}]")
        bh, ld = int(bias.shape[0]), int(bias.stride(1))
        if (max_l > 1 and bias.stride(2) != 1) or ld % 4 or ld < max_l or (bh > 1 and bias.stride(0) != T_q * ld):
            raise ValueError("bias rows must be unit-stride, a multiple of 4 elements apart, heads packed")
    st = _lib.attn_prefill_paged_masked(*head, _mask(None, None, block_keep, bias, bh, ld, key_range, alibi_slopes),
                                        _window(window),
                                        _dtype_code(q), _stream(stream, dev))
    _check(st, "attn_prefill_paged_masked")


def attn_prefill_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host,
                           cu_seqlens_q, cu_seqlens_q_host, o, lse, *, scale: float, causal: bool = True, window=None,
                           stream=None):
    """attn_prefill_paged over E4M3 caches: caches uint8 [num_pages, page_size, A_kv, d] of code bytes,
    k_scale/v_scale fp32 [num_pages, A_kv]; q/o bf16 [A,T_q,d]; the rest as attn_prefill_paged."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [A,T_q,d]; caches [num_pages, page_size, A_kv, d]")
    A, T_q, d = q.shape
    num_pages, page_size, A_kv, dk = k_cache.shape
    if dk != d or o.shape != q.shape or lse.shape != (A, T_q) or lse.dtype != torch.float32:
        raise ValueError("shape mismatch")
    if q.dtype != torch.bfloat16 or o.dtype != torch.bfloat16:
        raise ValueError("q and o must be bf16")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("fp8 caches are passed as uint8 tensors of E4M3 bytes")
    for sc in (k_scale, v_scale):
        if sc.dtype != torch.float32 or sc.shape != (num_pages, A_kv):
            raise ValueError("scales must be fp32 [num_pages, A_kv]")
    cu_host = np.ascontiguousarray(cu_seqlens_q_host, dtype=np.int32)
    n_seq = cu_host.size - 1
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if sl.shape != (n_seq,) or seq_lens.dtype != torch.int32 or seq_lens.shape != (n_seq,):
        raise ValueError("seq_lens must be int32 [n_seq]")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_q.numel() != cu_host.size:
        raise ValueError("cu_seqlens_q must be int32 [n_seq + 1]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != n_seq:
        raise ValueError("block_table must be int32 [n_seq, max_pages]")
    dev = _dev(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, cu_seqlens_q, o, lse)
    st = _lib.attn_prefill_paged_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                     _ptr(block_table), _ptr(seq_lens), sl.ctypes.data_as(_vp), _ptr(cu_seqlens_q),
                                     cu_host.ctypes.data_as(_vp), page_size, _ptr(o), _ptr(lse), n_seq, T_q, A, A_kv,
                                     d, block_table.shape[1], num_pages, float(scale), int(bool(causal)),
                                     _window(window), _stream(stream, dev))
    _check(st, "attn_prefill_paged_fp8")


def attn_decode_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, o, lse,
                          workspace, *, scale: float, stream=None):
    """Paged decode over FP8 (E4M3) caches: q/o bf16 [B,A,d]; caches uint8 [num_pages, page_size, A_kv, d];
    k_scale/v_scale fp32 [num_pages, A_kv]; the rest as attn_decode_paged."""
    _fp8_decode_call(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, o, lse, workspace,
                     scale, None, stream)


def attn_decode_paged_fp8_window(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, o,
                                 lse, workspace, *, scale: float, window_left: int, stream=None):
    """attn_decode_paged_fp8 where the query of sequence b sees only the keys t >= seq_lens[b] - 1 - window_left
    (-1: every key)."""
    _fp8_decode_call(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, o, lse, workspace,
                     scale, int(window_left), stream)


def attn_decode_paged_fp8_alibi(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, o,
                                lse, workspace, *, scale: float, alibi_slopes, window_left: int = -1, stream=None):
    """attn_decode_paged_fp8_window with ALiBi (alibi_slopes fp32 [A], as attn_decode_paged_alibi)."""
    _fp8_decode_call(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, o, lse, workspace,
                     scale, int(window_left), stream, alibi_slopes)


def _fp8_decode_call(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, o, lse, workspace,
                     scale, window_left, stream, alibi_slopes=None):
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [B,A,d]; caches [num_pages, page_size, A_kv, d]")
    B, A, d = q.shape
    num_pages, page_size, A_kv, dk = k_cache.shape
    if dk != d or o.shape != q.shape or lse.shape != (B, A) or lse.dtype != torch.float32:
        raise ValueError("shape mismatch")
    if q.dtype != torch.bfloat16 or o.dtype != torch.bfloat16:
        raise ValueError("q and o must be bf16")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("fp8 caches are passed as uint8 tensors of E4M3 bytes")
    for sc in (k_scale, v_scale):
        if sc.dtype != torch.float32 or sc.shape != (num_pages, A_kv):
            raise ValueError("scales must be fp32 [num_pages, A_kv]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if sl.shape != (B,):
        raise ValueError("seq_lens_host must be [B]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (A,)):
        raise ValueError(f"alibi_slopes must be fp32 [{A}]")
    dev = _dev(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, o, lse, workspace, alibi_slopes)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
            sl.ctypes.data_as(_vp), page_size, _ptr(o), _ptr(lse), B, A, A_kv, d, block_table.shape[1], num_pages,
            float(scale))
    tail = (_ptr(workspace), ws_bytes, _stream(stream, dev))
    if alibi_slopes is not None:
        _check(_lib.attn_decode_paged_fp8_alibi(*args, window_left, _ptr(alibi_slopes), *tail),
               "attn_decode_paged_fp8_alibi")
    elif window_left is None:
        _check(_lib.attn_decode_paged_fp8(*args, *tail), "attn_decode_paged_fp8")
    else:
        _check(_lib.attn_decode_paged_fp8_window(*args, window_left, *tail), "attn_decode_paged_fp8_window")
