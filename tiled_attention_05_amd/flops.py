"""Mask-adjusted work counts for the throughput metric (host logic, closed forms).

FLOP convention: 4 d FLOPs per allowed (query, key) pair -- 2 d for the row of
Q K^T and 2 d for the row of P V -- and nothing for the softmax.  With d = 128
that is 512 matmul FLOPs per exponential, the ratio "FlashAttention-3 : une
attention plus rapide ..." states in section "Chevauchement de GEMM et softmax
grace a l'asynchronisme".

Pair counts are closed forms per query row (no N x N enumeration), vectorised
with numpy so the largest workloads (N = 32768) count instantly.
"""
from __future__ import annotations

import numpy as np

MASK_CAUSAL = 1
MASK_WINDOW = 2
MASK_DOC = 4


def pairs_per_row(Nq: int, Nk: int, mask: int, window: int = 0, doc_row=None) -> np.ndarray:
    """int64 [Nq]: number of keys row i may attend to."""
    i = np.arange(Nq, dtype=np.int64)
    off = Nk - Nq
    hi = np.full(Nq, Nk - 1, dtype=np.int64)          # last allowed key (inclusive)
    lo = np.zeros(Nq, dtype=np.int64)                 # first allowed key
    if mask & MASK_CAUSAL:
        hi = np.minimum(hi, i + off)
    if mask & MASK_WINDOW:
        lo = np.maximum(lo, i + off - window + 1)
    if mask & MASK_DOC:
        doc = np.asarray(doc_row, dtype=np.int64)
        if doc.shape[0] != Nq or Nq != Nk:
            raise ValueError("document mask needs Nq == Nk == len(doc_ids)")
        # contiguous documents: [first index of doc(i), last index of doc(i)]
        starts = np.searchsorted(doc, doc, side="left")
        ends = np.searchsorted(doc, doc, side="right") - 1
        lo = np.maximum(lo, starts)
        hi = np.minimum(hi, ends)
    return np.maximum(hi - lo + 1, 0)


def allowed_pairs(Nq: int, Nk: int, mask: int, window: int = 0, doc_row=None) -> int:
    return int(pairs_per_row(Nq, Nk, mask, window, doc_row).sum())


def attention_flops(B: int, Hq: int, Nq: int, Nk: int, d: int, mask: int, window: int = 0,
                    doc_ids=None) -> int:
    """4 d * sum over (b, h) of allowed pairs."""
    tot = 0
    for b in range(B):
        row = None if doc_ids is None else np.asarray(doc_ids[b])
        tot += allowed_pairs(Nq, Nk, mask, window, row)
    return 4 * d * Hq * tot


def exps(B: int, Hq: int, Nq: int, Nk: int, mask: int, window: int = 0, doc_ids=None) -> int:
    """One exponential per allowed pair."""
    tot = 0
    for b in range(B):
        row = None if doc_ids is None else np.asarray(doc_ids[b])
        tot += allowed_pairs(Nq, Nk, mask, window, row)
    return Hq * tot
