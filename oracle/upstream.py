"""Upstream of the indexer: its projections, key LayerNorm, rotary position encoding,
the folded score scales, and the decode-time cache append (oracle; test infrastructure
only, shared with no GPU code).

[IDX] §6.4 ("Transformers 实现里的 GLM Indexer") describes the GLM indexer's own
projections: a query projection from the low-rank query latent, a key projection from
the hidden state followed by a LayerNorm over the head dimension, a head-weight
projection from the hidden state scaled by (H^I)^(-1/2), a score scaled by d_I^(-1/2),
and rotary encoding of the query/key "RoPE part".  [IDX] §4's memory view (the
six-step data flow) writes every new token into the caches before it is read.

Readings where the pages leave a step open (each listed in the design notes):
  * the rotary part is the first `rope_dim` (default 64) of the d_I = 128 dimensions,
    rotated in the half-split form: dimension j pairs with j + rope_dim/2, angle
    pos * base^(-2j/rope_dim), base 10000;
  * the key LayerNorm has a per-dimension weight and bias and eps = 1e-5 (the default of
    the layer named on the page);
  * d_I^(-1/2) multiplies q.k before the ReLU; as a positive factor it is moved into the
    head weight, which therefore carries (H^I)^(-1/2) * d_I^(-1/2);
  * the projections have no bias (the page lists nn.Linear layers without saying; a
    bias-free projection is the plainest reading and a bias would be a per-output add).
Everything is float64.
"""
from __future__ import annotations

import numpy as np


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * gamma + beta,
    var the biased (population) variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def rope(x: np.ndarray, pos: np.ndarray, rope_dim: int = 64, base: float = 10000.0) -> np.ndarray:
    """Rotary encoding of the first rope_dim dimensions of the last axis of x.

    x [..., n, d] with pos [n] (one position per row along axis -2), or x [n, d] with
    pos [n].  Pair (j, j + rope_dim/2) of row i is rotated by pos[i] * base^(-2j/rope_dim);
    dimensions from rope_dim on pass through unchanged."""
    half = rope_dim // 2
    j = np.arange(half, dtype=np.float64)
    inv = base ** (-2.0 * j / rope_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [n, half]
    cos, sin = np.cos(ang), np.sin(ang)
    if x.ndim == 3:                                                        # [n, H, d]
        cos, sin = cos[:, None, :], sin[:, None, :]
    out = np.array(x, dtype=np.float64, copy=True)
    a = x[..., :half]
    b = x[..., half:rope_dim]
    out[..., :half] = a * cos - b * sin
    out[..., half:rope_dim] = a * sin + b * cos
    return out


def indexer_project(q_lat: np.ndarray, h: np.ndarray, wq: np.ndarray, wk: np.ndarray, gamma: np.ndarray,
                    beta: np.ndarray, ww: np.ndarray, pos: np.ndarray, H: int, d: int, rope_dim: int = 64,
                    base: float = 10000.0, eps: float = 1e-5):
    """The indexer inputs of n tokens from their query latent and hidden state.

    q_lat [n, r] (low-rank query latent), h [n, hidden], wq [r, H*d], wk [hidden, d],
    gamma/beta [d], ww [hidden, H], pos [n] (token positions).
    Returns q_idx [n, H, d], k_idx [n, d], w [n, H] with
      q_idx = RoPE(reshape(q_lat wq, [H, d])),  k_idx = RoPE(LayerNorm(h wk)),
      w = (h ww) * H^(-1/2) * d^(-1/2)  (the score's d^(-1/2) folded in)."""
    n = q_lat.shape[0]
    q = (q_lat @ wq).reshape(n, H, d)
    q = rope(q, pos, rope_dim, base)
    k = layer_norm(h @ wk, gamma, beta, eps)
    k = rope(k, pos, rope_dim, base)
    w = (h @ ww) * (H ** -0.5) * (d ** -0.5)
    return q, k, w


def cache_append(cache: np.ndarray, lens: np.ndarray, caps: np.ndarray, rows: np.ndarray):
    """Decode-time write of one new row per sequence into a packed per-sequence cache.

    Sequence b owns cache rows [offset_b, offset_b + caps[b]) (offsets = exclusive prefix
    of caps) and holds lens[b] valid rows; the new row rows[b] goes to row
    offset_b + lens[b].  Returns (the updated cache, lens + 1)."""
    out = np.array(cache, copy=True)
    offs = np.concatenate([[0], np.cumsum(caps)[:-1]])
    for b in range(len(lens)):
        assert lens[b] < caps[b], "sequence %d is full" % b
        out[offs[b] + lens[b]] = rows[b]
    return out, np.asarray(lens) + 1
