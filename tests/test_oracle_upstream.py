"""Pins for the oracle's upstream, diagnostics, sparse-training loss and compressed-block
functions: hand values, closed forms, invariances, planted mistakes and library routines
(torch's float64 layer_norm and bf16 cast, scipy's relative entropy), never a retyped copy
of the oracle's own formula."""
import math

import numpy as np
import pytest
import torch
from scipy.special import rel_entr

import oracle
from oracle import csa, upstream


# ----------------------------------------------------------------------------- LayerNorm

def test_layer_norm_hand_values():
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    got = upstream.layer_norm(x, np.ones(4), np.zeros(4), eps=0.0)
    want = np.array([-1.5, -0.5, 0.5, 1.5]) / math.sqrt(1.25)      # mean 2.5, population variance 1.25
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-15)
    got = upstream.layer_norm(x, np.array([1.0, 2.0, 1.0, 1.0]), np.array([0.0, 0.0, 1.0, 0.0]), eps=0.0)
    np.testing.assert_allclose(got[0], [want[0], 2 * want[1], want[2] + 1, want[3]], rtol=0, atol=1e-15)
    # the sample variance (n - 1) would give a different value
    assert not np.allclose(got[0, 0], -1.5 / math.sqrt(5.0 / 3.0))


def test_layer_norm_matches_library_and_is_affine_invariant():
    g = np.random.default_rng(0)
    x = g.standard_normal((50, 128)) * 3 + 1
    gamma, beta = g.standard_normal(128), g.standard_normal(128)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), torch.from_numpy(gamma),
                                         torch.from_numpy(beta), eps=1e-5).numpy()
    np.testing.assert_allclose(upstream.layer_norm(x, gamma, beta), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(upstream.layer_norm(4.0 * x - 7.0, gamma, beta, eps=0.0),
                               upstream.layer_norm(x, gamma, beta, eps=0.0), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- RoPE

def test_rope_hand_values_and_pairing():
    # rope_dim 2: the single pair (0, 1) turns by pos * base^0 = pos radians
    x = np.array([[1.0, 0.0, 5.0]])
    for p in (0.0, 1.0, math.pi / 2, 3.0):
        got = upstream.rope(x, np.array([p]), rope_dim=2)
        np.testing.assert_allclose(got[0], [math.cos(p), math.sin(p), 5.0], rtol=0, atol=1e-15)
    # rope_dim 4, base 100: pairs (0, 2) at angle p and (1, 3) at angle p / 10 (half-split pairing)
    x = np.array([[1.0, 0.0, 0.0, 1.0]])
    got = upstream.rope(x, np.array([2.0]), rope_dim=4, base=100.0)
    want = [math.cos(2.0), -math.sin(0.2), math.sin(2.0), math.cos(0.2)]
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-15)
    # an interleaved pairing (2j, 2j+1) would rotate (0, 1) together instead
    interleaved = [math.cos(2.0), math.sin(2.0), -math.sin(0.2), math.cos(0.2)]
    assert not np.allclose(got[0], interleaved)


def test_rope_is_a_rotation_with_relative_positions():
    """Per pair a plane rotation: norms are kept, position 0 is the identity, and the
    dot product of a query at t with a key at s depends on t - s only; checked against
    complex multiplication z_j * exp(i pos theta_j) (an independent formulation)."""
    g = np.random.default_rng(1)
    d, r = 128, 64
    q = g.standard_normal((1, d))
    k = g.standard_normal((1, d))
    np.testing.assert_array_equal(upstream.rope(q, np.array([0]), r), q)
    for t, s in ((5, 2), (1000, 997), (40000, 39997)):
        a = upstream.rope(q, np.array([t]), r) @ upstream.rope(k, np.array([s]), r).T
        b = upstream.rope(q, np.array([t - s]), r) @ k.T
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)
    pos = np.array([0.0, 3.0, 12345.0])
    x = g.standard_normal((3, d))
    got = upstream.rope(x, pos, r)
    theta = 10000.0 ** (-2.0 * np.arange(r // 2) / r)
    z = (x[:, :r // 2] + 1j * x[:, r // 2:r]) * np.exp(1j * pos[:, None] * theta[None, :])
    np.testing.assert_allclose(got[:, :r // 2], z.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(got[:, r // 2:r], z.imag, rtol=0, atol=1e-9)
    np.testing.assert_array_equal(got[:, r:], x[:, r:])
    np.testing.assert_allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    # [n, H, d] input: every head of a row turns by that row's position
    xh = g.standard_normal((3, 4, d))
    gh = upstream.rope(xh, pos, r)
    for h in range(4):
        np.testing.assert_array_equal(gh[:, h], upstream.rope(xh[:, h], pos, r))


# ----------------------------------------------------------------------------- projections

def test_indexer_project_folds_the_score_scales_into_w():
    """[IDX] §6.4: score = ReLU(q.k * d^-1/2) weighted by w = (h W_w)_h * H^-1/2.  With the
    positive d^-1/2 moved into w the indexer score is the same (ReLU is positively
    homogeneous), so the folded projection feeds the unscaled score definition."""
    g = np.random.default_rng(2)
    n, r, hid, H, d = 9, 16, 12, 4, 8
    q_lat, h = g.standard_normal((n, r)), g.standard_normal((n, hid))
    wq, wk, ww = g.standard_normal((r, H * d)), g.standard_normal((hid, d)), g.standard_normal((hid, H))
    gamma, beta = g.standard_normal(d), g.standard_normal(d)
    pos = np.arange(n) + 3
    q, k, w = upstream.indexer_project(q_lat, h, wq, wk, gamma, beta, ww, pos, H, d, rope_dim=4)
    t = n - 1
    w_unfolded = (h[t] @ ww) * H ** -0.5
    explicit = np.array([np.sum(w_unfolded * np.maximum(q[t] @ k[s] * d ** -0.5, 0.0)) for s in range(n)])
    np.testing.assert_allclose(oracle.indexer_row(q[t], w[t], k), explicit, rtol=1e-12, atol=1e-12)
    # shapes and the pieces taken apart: q is RoPE of the reshaped projection, k of the LayerNorm
    np.testing.assert_allclose(q, upstream.rope((q_lat @ wq).reshape(n, H, d), pos, 4), rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, upstream.rope(upstream.layer_norm(h @ wk, gamma, beta), pos, 4), rtol=0,
                               atol=1e-12)
    assert q.shape == (n, H, d) and k.shape == (n, d) and w.shape == (n, H)


def test_cache_append_hand_example():
    cache = np.arange(12.0).reshape(6, 2)          # two sequences of capacity 4 and 2
    new, lens = upstream.cache_append(cache, np.array([2, 1]), np.array([4, 2]), np.array([[-1.0, -2.0],
                                                                                          [-3.0, -4.0]]))
    want = cache.copy()
    want[2] = [-1.0, -2.0]
    want[5] = [-3.0, -4.0]
    np.testing.assert_array_equal(new, want)
    assert lens.tolist() == [3, 2]
    with pytest.raises(AssertionError):
        upstream.cache_append(cache, np.array([4, 1]), np.array([4, 2]), np.zeros((2, 2)))


# ----------------------------------------------------------------------------- diagnostics

def test_captured_mass_and_head_aggregate_hand_values():
    alpha = np.array([[0.5, 0.3, 0.2], [0.1, 0.1, 0.8]])
    p = oracle.head_mean_distribution(alpha)
    np.testing.assert_allclose(p, [0.3, 0.2, 0.5], rtol=0, atol=1e-15)
    per_head, agg = oracle.captured_mass_at_k(alpha, np.array([0, 2, -1]))
    np.testing.assert_allclose(per_head, [0.7, 0.9], rtol=0, atol=1e-15)
    assert agg == pytest.approx(0.8, abs=1e-15)
    # the whole prefix captures all mass; a set and its complement add up to one
    assert oracle.captured_mass_at_k(alpha, np.array([0, 1, 2]))[1] == pytest.approx(1.0, abs=1e-15)
    c1 = oracle.captured_mass_at_k(alpha, np.array([1]))[1]
    assert agg + c1 == pytest.approx(1.0, abs=1e-15)


def test_recall_at_k_hand_values():
    alpha = np.array([[0.5, 0.3, 0.2], [0.5, 0.3, 0.2]])
    r, row = oracle.recall_at_k(alpha, np.array([0, 2]), 2)
    assert row.tolist() == [0, 1] and r == 0.5
    assert oracle.recall_at_k(alpha, np.array([1, 0, -1]), 2)[0] == 1.0
    assert oracle.recall_at_k(alpha, np.array([2]), 2)[0] == 0.0
    # ties in the aggregated weight go to the lower position
    tie = np.array([[0.25, 0.25, 0.25, 0.25]])
    r, row = oracle.recall_at_k(tie, np.array([0, 1]), 2)
    assert r == 1.0 and row.tolist() == [0, 1]
    assert oracle.recall_at_k(tie, np.array([2, 3]), 2)[0] == 0.0
    # the budget beyond the prefix: all positions, recall over t + 1
    assert oracle.recall_at_k(alpha, np.array([0, 1, 2]), 5)[0] == 1.0


# ----------------------------------------------------------------------------- sparse-training KL

def test_indexer_kl_hand_value():
    """One head, two selected keys with attention weights 3/4, 1/4 (score gap ln 3) against
    equal indexer scores (uniform softmax): KL = 3/4 ln(3/2) + 1/4 ln(1/2)."""
    q = np.array([[math.log(3.0), 0.0]])
    lat = np.array([[1.0, 0.0], [0.0, 0.0], [9.0, 9.0]])
    kl = oracle.indexer_kl_row(q, lat, np.array([0, 1, -1]), np.array([2.5, 2.5, 0.0]), 1.0)
    assert kl == pytest.approx(0.75 * math.log(1.5) + 0.25 * math.log(0.5), abs=1e-14)
    # swapped roles (KL(pi || p)) would give a different number
    assert not math.isclose(kl, 0.5 * math.log(0.5 / 0.75) + 0.5 * math.log(0.5 / 0.25))


def test_indexer_kl_library_gibbs_and_zero():
    g = np.random.default_rng(3)
    n_h, D, n, k = 8, 24, 60, 17
    lat = g.standard_normal((n, D))
    q = g.standard_normal((n_h, D))
    idx = np.sort(g.choice(n, size=k, replace=False))
    scores = g.standard_normal(k) * 2
    kl = oracle.indexer_kl_row(q, lat, idx, scores, 0.3)
    alpha, _ = oracle.sparse_attention_weights(q, lat, idx, 0.3)
    p = alpha.mean(axis=0)
    pi = np.exp(scores - scores.max())
    pi /= pi.sum()
    assert kl == pytest.approx(float(rel_entr(p, pi).sum()), rel=1e-12)
    assert kl > 0
    # indexer scores equal to log p (+ any constant) make the distributions equal
    assert oracle.indexer_kl_row(q, lat, idx, np.log(p) + 7.0, 0.3) == pytest.approx(0.0, abs=1e-13)
    # -1 padding slots are ignored
    pad = np.concatenate([idx, [-1, -1]])
    assert oracle.indexer_kl_row(q, lat, pad, np.concatenate([scores, [50.0, -50.0]]), 0.3) == pytest.approx(kl)


def test_multilayer_kl_averages_the_served_layers():
    g = np.random.default_rng(4)
    n_h, D, n, k, rows = 4, 16, 40, 9, 3
    layers = [{"q": g.standard_normal((rows, n_h, D)), "latent": g.standard_normal((n, D))} for _ in range(4)]
    idx = np.stack([np.sort(g.choice(n, size=k, replace=False)) for _ in range(rows)])
    sc = g.standard_normal((rows, k))
    per = [sum(oracle.indexer_kl_row(L["q"][i], L["latent"], idx[i], sc[i], 0.25) for i in range(rows))
           for L in layers]
    assert oracle.multilayer_kl(layers, idx, sc, 0.25) == pytest.approx(np.mean(per), rel=1e-13)
    assert oracle.multilayer_kl(layers[:1], idx, sc, 0.25) == pytest.approx(per[0], rel=1e-13)


# ----------------------------------------------------------------------------- compressed blocks (CSA)

def test_compress_kv_hand_values_and_convexity():
    g = np.random.default_rng(5)
    n, c, m = 12, 5, 4
    ca, cb = g.standard_normal((n, c)), g.standard_normal((n, c))
    zero_z, zero_b = np.zeros((n, c)), np.zeros((m, c))
    out = csa.compress_kv(ca, cb, zero_z, zero_z, zero_b, zero_b, m)
    assert out.shape == (3, c)
    # equal logits: block 0 is the mean of its m a-rows; block i > 0 the mean of m a-rows and
    # the m b-rows of the previous window (the overlap)
    np.testing.assert_allclose(out[0], ca[0:4].mean(axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[1], np.concatenate([ca[4:8], cb[0:4]]).mean(axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[2], np.concatenate([ca[8:12], cb[4:8]]).mean(axis=0), rtol=0, atol=1e-15)
    # a dominant logit (through the bias) selects one row per column
    big = np.zeros((m, c))
    big[2, :] = 200.0
    out = csa.compress_kv(ca, cb, zero_z, zero_z, big, zero_b, m)
    np.testing.assert_allclose(out[1], ca[6], rtol=0, atol=1e-12)
    # random logits: every column is a convex combination of its window
    za, zb = g.standard_normal((n, c)), g.standard_normal((n, c))
    out = csa.compress_kv(ca, cb, za, zb, g.standard_normal((m, c)), g.standard_normal((m, c)), m)
    win = np.concatenate([ca[4:8], cb[0:4]])
    assert np.all(out[1] <= win.max(axis=0) + 1e-12) and np.all(out[1] >= win.min(axis=0) - 1e-12)
    # the trailing incomplete group (n % m tokens) forms no block
    assert csa.compress_kv(ca[:11], cb[:11], za[:11], zb[:11], zero_b, zero_b, m).shape == (2, c)


def test_csa_visibility_and_selection():
    assert [csa.visible_blocks(t, 4) for t in (0, 3, 4, 7, 8, 9)] == [0, 0, 1, 1, 2, 2]
    g = np.random.default_rng(6)
    H, d, nb = 4, 8, 30
    q, w, kc = g.standard_normal((H, d)), g.standard_normal(H), g.standard_normal((nb, d))
    row, I = csa.csa_topk_row(q, w, kc, 3, 4, 5)
    assert np.all(row == -1) and I.size == 0                     # t < m: nothing visible
    row, I = csa.csa_topk_row(q, w, kc, 50, 4, 5)
    assert I.size == 12 and np.all((row[:5] >= 0) & (row[:5] < 12))
    ref = oracle.indexer_row(q, w, kc[:12])
    assert row.tolist() == sorted(np.lexsort((np.arange(12), -ref))[:5].tolist())
    # m = 1 is the token indexer with a strict visible set s < t
    row1, _ = csa.csa_topk_row(q, w, kc, 10, 1, 3)
    assert row1.tolist() == oracle.topk_row(oracle.indexer_row(q, w, kc[:10]), 3)[0].tolist()


def test_round_bf16_hand_values_and_library():
    v = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.0 * 2.0 ** -130, 0.0])
    np.testing.assert_array_equal(csa.round_bf16(v), [1.0, 1.0, 1 + 2.0 ** -6, -1.0,
                                                      float(torch.tensor(3.0 * 2.0 ** -130, dtype=torch.float32)
                                                            .to(torch.bfloat16).double()), 0.0])
    g = np.random.default_rng(7)
    x = (g.standard_normal(5000) * 10.0 ** g.uniform(-5, 5, 5000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(csa.round_bf16(x.astype(np.float64)), ref)
