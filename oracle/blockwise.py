"""Independent blockwise online-softmax recurrence (numpy, fp64) -- TEST ONLY.

Restates the two-state merge of page "Attention Kernel", section "Online
softmax": a running state (m, l, o) and a block state (m_b, l_b, o_b) merge as

    m' = max(m, m_b)
    l' = exp(m - m') l + exp(m_b - m') l_b
    o' = exp(m - m') o + exp(m_b - m') o_b

and after the last block O = o / l.  Blocks may be visited in any order and be
of any size; a block whose scores are all -inf is skipped, and a row whose
normaliser stays 0 returns the zero vector (same section, fully-masked-row
contract; section "Blockwise reference" for the per-row interface).

This shares no code with ``attn_oracle.c``; it exists to check it.
"""
from __future__ import annotations

import math

import numpy as np


def _check(scores, values):
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if scores.ndim != 1 or values.ndim != 2 or values.shape[0] != scores.shape[0]:
        raise ValueError("scores [n] and values [n, d] must align")
    return scores, values


def block_state(scores, values):
    """(m_b, l_b, o_b) of one block, relative to the block's own maximum."""
    m_b = float(np.max(scores)) if scores.size else -math.inf
    if m_b == -math.inf:
        return m_b, 0.0, np.zeros(values.shape[1])
    w = np.exp(scores - m_b)          # exp(-inf) = 0 for masked entries
    return m_b, float(np.sum(w)), w @ values


def merge(state, blk):
    """Two-state merge: exact softmax combination of disjoint key sets."""
    m, l, o = state
    m_b, l_b, o_b = blk
    if m_b == -math.inf:
        return state
    if m == -math.inf:
        return blk
    m2 = max(m, m_b)
    a, c = math.exp(m - m2), math.exp(m_b - m2)
    return m2, a * l + c * l_b, a * o + c * o_b


def online_attention_row(scores, values, block_size=None, bounds=None, order=None):
    """Attention output and LSE for one score row, processed block by block.

    ``block_size`` cuts [0, n) into equal blocks; alternatively ``bounds`` lists
    the block edges explicitly (sorted, from 0 to n).  ``order`` permutes the
    blocks.  Returns (o [d], lse) with lse = -inf for a fully masked row.
    """
    scores, values = _check(scores, values)
    n = scores.shape[0]
    if bounds is None:
        if block_size is None or int(block_size) <= 0:
            raise ValueError("block_size must be positive")
        bounds = list(range(0, n, int(block_size))) + [n]
    bounds = list(bounds)
    if bounds[0] != 0 or bounds[-1] != n or any(b > c for b, c in zip(bounds, bounds[1:])):
        raise ValueError("bounds must run from 0 to n")
    blocks = list(zip(bounds[:-1], bounds[1:]))
    if order is not None:
        if sorted(order) != list(range(len(blocks))):
            raise ValueError("order must permute the blocks")
        blocks = [blocks[i] for i in order]
    state = (-math.inf, 0.0, np.zeros(values.shape[1]))
    for a, b in blocks:
        state = merge(state, block_state(scores[a:b], values[a:b]))
    m, l, o = state
    if not l > 0.0:
        return np.zeros(values.shape[1]), -math.inf
    return o / l, m + math.log(l)


def dense_scores(q, k, scale):
    """Score rows scale * q k^T for one head (library matmul as a step)."""
    return float(scale) * (np.asarray(q, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T)
