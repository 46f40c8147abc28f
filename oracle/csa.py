"""DeepSeek-V4 compressed sparse attention (CSA) selection: KV compression into blocks and
the indexer + top-k over compressed blocks (oracle; test infrastructure only).

[IDX] §5.1: every m tokens become one compressed entry by a learned gated pooling with an
overlapping window: C^a = H W^a, C^b = H W^b, Z^a = H W_Z^a, Z^b = H W_Z^b; the scores of
rows m i .. m(i+1)-1 of Z^a plus the bias B^a and of rows m(i-1) .. m i - 1 of Z^b plus
B^b are normalised together by a softmax along the row axis (separately for every
feature column), and C_i = sum_j S^a_j * C^a_j + sum_j S^b_j * C^b_j (elementwise).
[IDX] §5.2: the indexer score of a compressed block s for query t is the same ReLU-
weighted head sum as the token indexer, over compressed keys; block s is visible to
query t iff s < floor(t / m); S_t^CSA = TopK_k over the visible blocks.
[IDX] §5.4: a lower-precision selector rounds the index scores to bf16 before the top-k;
its agreement with the fp32 selector is measured as the recall of the fp32 selection.

Readings (listed in the design notes): B^a and B^b are [m, c] (one bias per position
inside the window and per feature column); for block 0 the overlap half (rows -m .. -1)
does not exist and the softmax runs over the m rows of the a-half only; blocks are formed
only from complete groups of m tokens (n // m blocks); an empty visible set (t < m) gives
a row of -1.
"""
from __future__ import annotations

import numpy as np

from .dsa import indexer_row, topk_row


def compress_kv(ca: np.ndarray, cb: np.ndarray, za: np.ndarray, zb: np.ndarray, ba: np.ndarray, bb: np.ndarray,
                m: int) -> np.ndarray:
    """Gated pooling of n tokens into n // m compressed entries (float64).

    ca, cb, za, zb [n, c]; ba, bb [m, c].  Returns C [n // m, c]."""
    n, c = ca.shape
    nb = n // m
    out = np.zeros((nb, c))
    for i in range(nb):
        a_rows = slice(m * i, m * (i + 1))
        logits = [za[a_rows] + ba]
        vals = [ca[a_rows]]
        if i > 0:
            b_rows = slice(m * (i - 1), m * i)
            logits.append(zb[b_rows] + bb)
            vals.append(cb[b_rows])
        lg = np.concatenate(logits, axis=0)            # [m or 2m, c]
        v = np.concatenate(vals, axis=0)
        lg = lg - lg.max(axis=0, keepdims=True)        # softmax along the row axis, per column
        wgt = np.exp(lg)
        wgt /= wgt.sum(axis=0, keepdims=True)
        out[i] = (wgt * v).sum(axis=0)
    return out


def visible_blocks(t: int, m: int) -> int:
    """Number of compressed blocks query t may read: s < floor(t / m)."""
    return t // m


def csa_topk_row(q_t: np.ndarray, w_t: np.ndarray, kcomp: np.ndarray, t: int, m: int, k: int,
                 bf16_scores: bool = False):
    """S_t^CSA of one query: the k best visible compressed blocks by the indexer score
    (ties to the lower block).  With bf16_scores the scores are first rounded to bf16
    (round to nearest even), the lower-precision selector of [IDX] §5.4.
    Returns (row [k] ascending, -1 padded; scores of the visible blocks)."""
    nv = visible_blocks(t, m)
    if nv == 0:
        return np.full(k, -1, dtype=np.int64), np.zeros(0)
    I = indexer_row(q_t, w_t, kcomp[:nv])
    if bf16_scores:
        I = round_bf16(I)
    row, _, _ = topk_row(I, k)
    return row, I


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest fp32 -> nearest-even bf16, back in float64 (finite inputs)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
