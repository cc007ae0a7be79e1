"""Algorithmic work of one attention layer, for throughput reporting.

Prefill counts 4*D flops per visible (query head, key) pair: 2*D for the
logit dot product and 2*D for the probability-weighted value sum.  Masked or
skipped pairs, the softmax and the norm/rotation prologue are not counted.
Decode counts the bytes that must cross HBM once: K and V of every visible
key per (sequence, kv head), plus q, o and the new K/V rows.

Visibility per query position i (Gemma 3 Technical Report, sections 1-2;
"Gemma explained" vision section): keys j <= i, or j in the image span that
contains i; local layers also need |i - j| < window.  The visible keys of a
row form the interval [lo(i), hi(i)], which is what is summed here.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


def visible_counts(qpos: np.ndarray, local: bool, window: int, spans: Iterable[Tuple[int, int]] = (),
                   kmin: int = 0) -> np.ndarray:
    """Number of visible keys for each query position (keys below ``kmin``
    do not exist)."""
    qpos = np.asarray(qpos, dtype=np.int64)
    hi = qpos.copy()
    for (s, e) in spans:
        inside = (qpos >= s) & (qpos < e)
        hi = np.where(inside, np.maximum(hi, e - 1), hi)
    lo = np.full_like(qpos, kmin)
    if local:
        lo = np.maximum(lo, qpos - window + 1)
        hi = np.minimum(hi, qpos + window - 1)
    return np.maximum(hi - lo + 1, 0)


def prefill_pairs(B: int, S: int, local: bool, window: int, pos0: Optional[Sequence[int]] = None,
                  spans: Optional[Sequence[Sequence[Tuple[int, int]]]] = None, has_cache: bool = False,
                  ring_capacity: Optional[int] = None) -> int:
    """Visible (query, key) pairs per query head, summed over sequences."""
    total = 0
    for b in range(B):
        p0 = 0 if pos0 is None else int(pos0[b])
        if has_cache:
            kmin = max(0, p0 - ring_capacity) if ring_capacity else 0
        else:
            kmin = p0
        sp = [] if spans is None else spans[b]
        total += int(visible_counts(p0 + np.arange(S), local, window, sp, kmin).sum())
    return total


def prefill_flops(B, S, Hq, D, local, window, **kw) -> float:
    return 4.0 * D * Hq * prefill_pairs(B, S, local, window, **kw)


def decode_bytes(B: int, Hq: int, Hkv: int, D: int, positions: Sequence[int], local: bool, window: int) -> float:
    """HBM bytes of one decode step: K+V of each visible key per (sequence,
    kv head) read once (bf16), plus q, o, k_new, v_new."""
    keys = 0
    for p in positions:
        lo = max(0, p - window + 1) if local else 0
        keys += p - lo + 1
    kv = 2.0 * 2 * D * Hkv * keys
    io = 2.0 * D * (2 * B * Hq + 2 * B * Hkv)
    return kv + io
