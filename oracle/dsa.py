"""The DSA hot path, written out from its definitions (oracle; test infrastructure only).

Conventions (readings of points the pages leave open):
  * visible set of query position t is {s : 0 <= s <= t} (the query sees itself);
  * top-k ranks by score descending, then position ascending (the lower position
    wins a tie); -0.0 and +0.0 compare equal;
  * a row keeps exactly min(k, t+1) positions, sorted ascending, padded with -1;
  * no internal scale inside the indexer score (positive scales commute with ReLU
    and belong in w);
  * attention is MQA over the shared latent: key = latent[s, :576],
    value = latent[s, :d_v], softmax over the selected set only.

Citations: [IDX] = Jerry's Blog, "注意力机制中的 Index：从位置下标到预算检索";
[IC] = "读懂 IndexCache：从 DSA 的选词开销到跨层索引复用".
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np


class RoleError(ValueError):
    pass


# ---------------------------------------------------------------------------
# indexer score  ([IDX] §4, lightning-indexer score equation; restated in §6.4 and §10)
# ---------------------------------------------------------------------------

def indexer_row(q_t: np.ndarray, w_t: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """I[t, s] = sum_j w[t, j] * ReLU(q_idx[t, j, :] . k_idx[s, :]) for every row s of `keys`.

    q_t [H, d] float64, w_t [H] float64, keys [n, d] float64 -> I [n] float64.
    """
    a = q_t @ keys.T                       # [H, n]: per-head dot products
    return w_t @ np.maximum(a, 0.0)        # head-weighted sum of the ReLU'd dots


def indexer_row_int2(q_t: np.ndarray, w2_t: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """2 * I[t, s] in exact int64 arithmetic, for integer-valued q/k and half-integer w
    (w2_t = 2w as integers).  Same definition as indexer_row."""
    a = q_t.astype(np.int64) @ keys.astype(np.int64).T
    return w2_t.astype(np.int64) @ np.maximum(a, 0)


def tolerance_row(scores: np.ndarray, rel: float = 1e-3) -> float:
    """Score tolerance of one row: rel * max_s |I[t, s]| over the visible prefix."""
    return rel * float(np.max(np.abs(scores))) if scores.size else 0.0


# ---------------------------------------------------------------------------
# top-k selection  ([IDX] §2 TopK over the visible set; §6.5 deterministic top-k)
# ---------------------------------------------------------------------------

def topk_row(scores: np.ndarray, k: int):
    """S_t = the k best visible positions of one query row.

    `scores` holds I[t, 0..t].  Order: score descending, then position
    ascending, so the selection is unique.  Returns (row, kth, n_valid):
    row [k] int64 sorted ascending and padded with -1; kth = the score of the
    last selected element in rank order; n_valid = min(k, t+1).
    """
    assert k >= 1
    n = scores.shape[0]
    assert np.all(np.isfinite(scores))
    pos = np.arange(n)
    order = np.lexsort((pos, -scores))     # primary: -score ascending; secondary: position
    m = min(k, n)
    chosen = np.sort(order[:m])
    row = np.full(k, -1, dtype=np.int64)
    row[:m] = chosen
    kth = float(scores[order[m - 1]]) if m else float("nan")
    return row, kth, m


# ---------------------------------------------------------------------------
# attention  ([IDX] §1 dense causal attention; §2 sparse attention over S_t;
#             §4 MLA latent read shared by all query heads)
# ---------------------------------------------------------------------------

def attn_row(q_t: np.ndarray, latent: np.ndarray, idx: np.ndarray, scale: float, d_v: int) -> np.ndarray:
    """o[h, :] = sum_{s in S} softmax_s(scale * q[h] . c[s]) * c[s, :d_v].

    q_t [n_h, D] float64, latent [n, D] float64 (rows indexed by position),
    idx [k] with -1 for unused slots.  A row with no valid index returns zeros.
    """
    sel = np.asarray(idx)
    sel = sel[sel >= 0]
    n_h = q_t.shape[0]
    if sel.size == 0:
        return np.zeros((n_h, d_v))
    c = latent[sel]                        # gathered latent rows [m, D]
    z = scale * (q_t @ c.T)                # [n_h, m]
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p @ c[:, :d_v]


def dense_attn_row(q_t: np.ndarray, latent_prefix: np.ndarray, scale: float, d_v: int):
    """Dense causal attention of query t over rows 0..t (= latent_prefix).

    Returns (o [n_h, d_v], alpha [n_h, t+1])."""
    z = scale * (q_t @ latent_prefix.T)
    z -= z.max(axis=1, keepdims=True)
    a = np.exp(z)
    a /= a.sum(axis=1, keepdims=True)
    return a @ latent_prefix[:, :d_v], a


# ---------------------------------------------------------------------------
# index-quality metrics  ([IDX] §3 residual mass; §8 captured mass and cross-layer overlap)
# ---------------------------------------------------------------------------

def captured_mass(alpha_row: np.ndarray, idx: np.ndarray) -> float:
    """A_t(S) = sum_{s in S} alpha[t, s]; the missed mass R_t = 1 - A_t."""
    sel = np.asarray(idx)
    sel = sel[sel >= 0]
    return float(alpha_row[sel].sum())


def head_mean_distribution(alpha: np.ndarray) -> np.ndarray:
    """The attention distribution of one query aggregated over heads: the per-head
    distributions alpha [n_h, n] summed over heads, then L1-normalised over positions
    ([IDX] §4.1, the dense warm-up target p_t).  Each row of alpha sums to 1, so this is
    the mean over heads."""
    p = alpha.sum(axis=0)
    return p / p.sum()


def captured_mass_at_k(alpha: np.ndarray, idx: np.ndarray):
    """CapturedMass@k of one query ([IDX] §8 item 1): sum over s in S_t of the dense
    attention weight alpha^dense[t, s], per head (alpha [n_h, t+1]) and for the
    head-aggregated distribution p_t.  Returns (per_head [n_h], aggregated); the missed
    mass is 1 minus either."""
    sel = np.asarray(idx)
    sel = sel[sel >= 0]
    per_head = alpha[:, sel].sum(axis=1)
    return per_head, float(head_mean_distribution(alpha)[sel].sum())


def recall_at_k(alpha: np.ndarray, idx_model: np.ndarray, k: int):
    """Recall@k of one query ([IDX] §8 item 2): the oracle selection S^oracle = the k
    positions of largest head-aggregated dense weight p_t (same total order as the
    indexer's top-k: weight descending, position ascending), against the model's
    selection S^model (valid entries of idx_model).  Returns
    (|S^oracle ∩ S^model| / |S^oracle|, S^oracle row as topk_row returns it)."""
    p = head_mean_distribution(alpha)
    row, _, m = topk_row(p, k)
    oracle_set = set(int(x) for x in row[:m])
    model_set = set(int(x) for x in np.asarray(idx_model) if x >= 0)
    return len(oracle_set & model_set) / float(m), row


# ---------------------------------------------------------------------------
# sparse-training indexer loss  ([IDX] §4.2 KL over S_t; [IC] §3.1 multi-layer form)
# ---------------------------------------------------------------------------

def sparse_attention_weights(q_t: np.ndarray, latent: np.ndarray, idx: np.ndarray, scale: float):
    """The main attention's weights over the selected set: per head, softmax over
    s in S_t of scale * q[h] . c[s] ([IDX] §2).  Returns (alpha_hat [n_h, |S|], sel)."""
    sel = np.asarray(idx)
    sel = sel[sel >= 0]
    z = scale * (q_t @ latent[sel].T)
    z -= z.max(axis=1, keepdims=True)
    a = np.exp(z)
    return a / a.sum(axis=1, keepdims=True), sel


def indexer_kl_row(q_t: np.ndarray, latent: np.ndarray, idx: np.ndarray, scores: np.ndarray, scale: float) -> float:
    """D_KL(p_{t,S_t} || Softmax(I_{t,S_t})) of one query ([IDX] §4.2).

    p_{t,S_t}: the main attention's weights over S_t (sparse attention, softmax over S_t
    per head), summed over heads and L1-normalised; Softmax(I_{t,S_t}): the indexer
    scores of the same positions, softmax over S_t.  `scores[j]` is the indexer score of
    position idx[j] (slots with idx < 0 ignored).  Terms with p = 0 contribute 0."""
    ii = np.asarray(idx)
    ok = ii >= 0
    alpha, _ = sparse_attention_weights(q_t, latent, ii, scale)
    p = head_mean_distribution(alpha)
    I = np.asarray(scores, dtype=np.float64)[ok]
    logpi = I - I.max()
    logpi = logpi - np.log(np.exp(logpi).sum())
    nz = p > 0
    return float(np.sum(p[nz] * (np.log(p[nz]) - logpi[nz])))


def multilayer_kl(layers, idx: np.ndarray, scores: np.ndarray, scale: float) -> float:
    """The multi-layer distillation loss of one F layer that serves m S layers
    ([IC] §3.1): (1/(m+1)) sum_{j=0..m} sum_t D_KL(p_t^{(l+j)} || q_t^{(l)}), where
    q_t^{(l)} = Softmax(I_{t,S_t}) is the F layer's indexer distribution and p^{(l+j)}
    the attention distribution of layer l+j over the same S_t.

    layers: m+1 dicts with 'q' [n, n_h, D] (the checked rows) and 'latent' [n_k, D];
    idx, scores [n, k] (the F layer's selection and indexer scores)."""
    tot = 0.0
    for L in layers:
        for i in range(idx.shape[0]):
            tot += indexer_kl_row(L["q"][i], L["latent"], idx[i], scores[i], scale)
    return tot / len(layers)


def overlap(idx_a: np.ndarray, idx_b: np.ndarray, k: int) -> float:
    """|S^(l) intersect S^(l+1)| / k for one query row."""
    a = set(int(x) for x in idx_a if x >= 0)
    b = set(int(x) for x in idx_b if x >= 0)
    return len(a & b) / float(k)


# ---------------------------------------------------------------------------
# IndexCache  ([IC] §1.1 F/S roles, first layer must be F; §1.2 the cache loop)
# ---------------------------------------------------------------------------

def indexcache_plan(roles: str):
    """src_layer[l] = the nearest layer l' <= l with role F; n_calls = number of F layers.

    Raises RoleError for an empty string, a character outside {F, S}, or a
    first layer that is not F (an S layer needs an earlier F layer's indices).
    """
    if not isinstance(roles, str) or len(roles) == 0:
        raise RoleError("empty role string")
    bad = [c for c in roles if c not in "FS"]
    if bad:
        raise RoleError("role must be F or S, got %r" % bad[0])
    if roles[0] != "F":
        raise RoleError("first layer must be F")
    src: List[int] = []
    last = -1
    for l, r in enumerate(roles):
        if r == "F":
            last = l
        src.append(last)
    return src, roles.count("F")


def indexcache_forward(roles: str, layers: Sequence[Dict[str, np.ndarray]], positions: Sequence[int],
                       k: int, scale: float, d_v: int, index_override: Optional[Dict[int, np.ndarray]] = None):
    """The IndexCache inference loop over the query rows at `positions`.

    layers[l] holds float64 arrays: 'q_idx' [n, H, d], 'w' [n, H], 'q' [n, n_h, D]
    for the n checked rows (aligned with `positions`), and 'k_idx' [n_k, d],
    'latent' [n_k, D] over the whole prefix.  'q_idx'/'w'/'k_idx' are read only
    for F layers.  T_cache starts empty; an F layer scores and selects, then
    overwrites it; every layer attends with its own q and latent over T_cache.

    index_override[l] (optional) replaces the selection of F layer l by given
    rows (used to evaluate attention on another implementation's indices).
    Returns a dict: calls, src_layer, index (per layer, the rows attended),
    out (per layer [n, n_h, d_v]), scores (per F layer: list of I rows).
    """
    src, _ = indexcache_plan(roles)
    positions = [int(p) for p in positions]
    t_cache: Optional[np.ndarray] = None
    calls = 0
    index_used, outs, scores = [], [], {}
    for l, role in enumerate(roles):
        L = layers[l]
        if role == "F":
            rows, srows = [], []
            for i, t in enumerate(positions):
                I = indexer_row(L["q_idx"][i], L["w"][i], L["k_idx"][: t + 1])
                srows.append(I)
                rows.append(topk_row(I, k)[0])
            t_cache = np.stack(rows)
            if index_override is not None and l in index_override:
                t_cache = np.asarray(index_override[l])
            scores[l] = srows
            calls += 1
        assert t_cache is not None
        index_used.append(t_cache)
        outs.append(np.stack([attn_row(L["q"][i], L["latent"], t_cache[i], scale, d_v)
                              for i in range(len(positions))]))
    return {"calls": calls, "src_layer": src, "index": index_used, "out": outs, "scores": scores}
