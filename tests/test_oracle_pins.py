"""Pins for the CPU oracle: what the pages and mathematics fix, independent of the oracle itself.

Each test targets a plausible mistake (dropped ReLU, wrong sign, transposed operand,
off-by-one visibility, wrong tie order, wrong value slice, wrong cache source layer):
hand-derived fixtures (tests/golden/hand_examples.json), closed forms, brute force,
library routines (torch CPU float64 attention, torch's fp8/bf16 casts) and the
top-k error identity and bound of the index blog's §3.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import (attn_row, decode_bf16, decode_e4m3fn, dense_attn_row, indexcache_forward,
                    indexcache_plan, indexer_row, indexer_row_int2, topk_row, RoleError)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


# ----------------------------------------------------------------------------- formats

def test_bf16_decode_known_values():
    cases = {0x3F80: 1.0, 0xC040: -3.0, 0x3F00: 0.5, 0x0001: 2.0 ** -133,
             0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x4049: 3.140625}
    for code, val in cases.items():
        assert decode_bf16(np.array([code], np.uint16))[0] == val
    neg0 = decode_bf16(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0


def test_bf16_decode_matches_library_cast():
    g = np.random.default_rng(1)
    codes = g.integers(0, 1 << 16, size=4096).astype(np.uint16)
    codes = codes[(codes & 0x7F80) != 0x7F80]          # drop inf/nan patterns
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(decode_bf16(codes), ref)


def test_e4m3fn_known_values():
    v = lambda c: decode_e4m3fn(np.array([c], np.uint8))[0]
    assert v(0x38) == 1.0           # exponent 7 = bias, mantissa 0
    assert v(0x7E) == 448.0         # largest finite
    assert v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6     # smallest normal
    assert v(0x01) == 2.0 ** -9     # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9
    assert v(0x3C) == 1.5
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert v(0x80) == 0.0 and math.copysign(1, v(0x80)) == -1


def test_e4m3fn_matches_library_cast():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = decode_e4m3fn(codes)
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])


def test_dequant_rows_fp8_scale():
    payload = np.array([[0x38, 0xB8, 0x7E]], np.uint8)   # 1, -1, 448
    s = np.array([0.25], np.float32)
    np.testing.assert_array_equal(oracle.dequant_rows(payload, s, "fp8"), [[0.25, -0.25, 112.0]])


# ----------------------------------------------------------------------------- hand fixtures

def _hand_indexer():
    g = GOLD["indexer_topk"]
    q = np.array(g["q_t"], float)
    w = np.array(g["w_t"], float)
    keys = np.array(g["keys"], float)
    return g, q, w, keys


def test_hand_indexer_scores_and_visibility():
    g, q, w, keys = _hand_indexer()
    t = g["t"]
    I = indexer_row(q, w, keys[: t + 1])
    np.testing.assert_array_equal(I, g["scores_visible"])
    for k, expect in g["topk"].items():
        row, kth, m = topk_row(I, int(k))
        assert row.tolist() == expect
        assert m == min(int(k), t + 1)


def test_hand_fixture_rejects_planted_mistakes():
    """Plausible wrong versions of the score and selection fail the hand fixture."""
    g, q, w, keys = _hand_indexer()
    t = g["t"]
    good = np.array(g["scores_visible"])
    no_relu = w @ (q @ keys[: t + 1].T)
    flipped_w = (-w) @ np.maximum(q @ keys[: t + 1].T, 0)
    transposed = w @ np.maximum(q.T @ keys[: t + 1].T, 0)
    for bad in (no_relu, flipped_w, transposed):
        assert not np.array_equal(bad, good)
    # strict causality (s < t) would lose position 3, which is in the top-2
    strict = indexer_row(q, w, keys[:t])
    assert topk_row(strict, 2)[0].tolist() != g["topk"]["2"]
    # upper-position tie break would pick 3 instead of 1 for k=1
    order_hi = np.lexsort((-np.arange(t + 1), -good))
    assert [int(order_hi[0])] != g["topk"]["1"]


def test_hand_attention():
    g = GOLD["attention"]
    o = attn_row(np.array(g["q_t"]), np.array(g["latent"], float), np.array(g["idx"]), g["scale"], g["d_v"])
    np.testing.assert_allclose(o, g["out"], rtol=0, atol=1e-15)


def test_hand_indexcache_plan():
    g = GOLD["indexcache_fsss"]
    src, n = indexcache_plan(g["roles"])
    assert src == g["src_layer"] and n == g["n_calls"]
    assert indexcache_plan(g["roles_all_f"])[1] == g["n_calls_all_f"]
    for bad in g["invalid"]:
        with pytest.raises(RoleError):
            indexcache_plan(bad)


# ----------------------------------------------------------------------------- acceptance tolerance

def test_tolerance_row_hand_values():
    """The float acceptance threshold is 1e-3 times the largest |I[t, s]| over the visible
    prefix (the score tolerance the parity rules state).  Hand rows separate it from the
    plausible wrong forms: max(I) instead of max|I| (all-negative row), sum|I| or the
    mean (mixed row), and a relative factor other than 1e-3 (single element)."""
    assert oracle.tolerance_row(np.array([-3.0, -1.0, -2.0])) == pytest.approx(3e-3, rel=0, abs=1e-18)
    assert oracle.tolerance_row(np.array([2.0, -5.0, 1.0])) == pytest.approx(5e-3, rel=0, abs=1e-18)
    assert oracle.tolerance_row(np.array([7.0])) == pytest.approx(7e-3, rel=0, abs=1e-18)
    assert oracle.tolerance_row(np.array([0.0, -0.0])) == 0.0
    assert oracle.tolerance_row(np.array([])) == 0.0
    assert oracle.tolerance_row(np.array([2.0, -5.0, 1.0]), rel=0.5) == 2.5


def test_parity_rules_use_the_stated_thresholds():
    """The thresholds every float parity test applies: scores within 1e-3 x row max |I|,
    mean recall >= 0.999, attention max abs error <= 1e-2."""
    import parity
    assert parity.SCORE_REL == 1e-3
    assert parity.RECALL_MIN == 0.999
    assert parity.ATTN_ATOL == 1e-2


# ----------------------------------------------------------------------------- exactness (C6)

def test_integer_indexer_is_exact_in_fp64():
    g = np.random.default_rng(7)
    H, d, n = 8, 64, 300
    q = g.integers(-4, 5, size=(H, d))
    k = g.integers(-4, 5, size=(n, d))
    w2 = g.choice([-2, -1, 1, 2], size=H)
    I = indexer_row(q.astype(float), w2 / 2.0, k.astype(float))
    I2 = indexer_row_int2(q, w2, k)
    np.testing.assert_array_equal(I * 2, I2.astype(float))
    assert np.all(I * 2 == np.round(I * 2))


# ----------------------------------------------------------------------------- brute force (C5)

def _rank_count_topk(I, k):
    """Selected iff fewer than k positions beat it under (score desc, position asc)."""
    n = len(I)
    sel = []
    for s in range(n):
        beats = sum(1 for s2 in range(n) if I[s2] > I[s] or (I[s2] == I[s] and s2 < s))
        if beats < k:
            sel.append(s)
    return sel


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_rank_counting_brute_force(seed):
    g = np.random.default_rng(100 + seed)
    for L in range(1, 13):
        for t in range(L):
            I = g.integers(-3, 4, size=t + 1).astype(float) * 0.5   # many ties
            if seed % 2:
                I = I + g.standard_normal(t + 1) * (seed > 2)
            for k in range(1, L + 2):
                row, kth, m = topk_row(I, k)
                assert row[:m].tolist() == _rank_count_topk(I, k)
                assert np.all(row[m:] == -1)


def test_attention_matches_index_mask_formulation():
    """[IDX] §6.4: scores + index mask (-inf outside S_t) + causal mask, softmax over all columns."""
    g = np.random.default_rng(3)
    n_h, D, dv, L = 3, 9, 5, 12
    lat = g.standard_normal((L, D))
    for t in range(L):
        q = g.standard_normal((n_h, D))
        for k in range(1, L + 2):
            I = g.standard_normal(t + 1)
            row, _, m = topk_row(I, k)
            e = 0.7 * (q @ lat.T)                                   # all L columns
            mask = np.full(L, -np.inf)
            mask[row[:m]] = 0.0
            causal = np.where(np.arange(L) <= t, 0.0, -np.inf)
            e = e + mask + causal
            a = np.exp(e - e.max(axis=1, keepdims=True))
            a /= a.sum(axis=1, keepdims=True)
            ref = a @ lat[:, :dv]
            np.testing.assert_allclose(attn_row(q, lat, row, 0.7, dv), ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- sparse == dense (C3)

def test_sparse_equals_dense_when_budget_covers_prefix():
    g = np.random.default_rng(11)
    n_h, D, dv, L = 4, 16, 12, 20
    lat = g.standard_normal((L, D))
    for t in range(L):
        q = g.standard_normal((n_h, D))
        I = g.standard_normal(t + 1)
        row, _, m = topk_row(I, t + 1 + (t % 3))
        assert m == t + 1 and row[:m].tolist() == list(range(t + 1))
        o_dense, _ = dense_attn_row(q, lat[: t + 1], 0.3, dv)
        np.testing.assert_allclose(attn_row(q, lat, row, 0.3, dv), o_dense, rtol=0, atol=1e-12)


def test_dense_attention_matches_library_sdpa():
    g = np.random.default_rng(12)
    n_h, D, dv, L = 4, 24, 16, 33
    q = g.standard_normal((n_h, L, D))
    lat = g.standard_normal((L, D))
    scale = 1 / math.sqrt(D)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(lat)[None].expand(n_h, L, D),
        torch.from_numpy(lat[:, :dv])[None].expand(n_h, L, dv), is_causal=True, scale=scale).numpy()
    for t in range(L):
        o, _ = dense_attn_row(q[:, t], lat[: t + 1], scale, dv)
        np.testing.assert_allclose(o, ref[:, t], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- error identity and bound (C4)

def test_topk_error_identity_and_bound():
    """[IDX] §3: ||o - o_hat|| = R_t ||o_Sbar - o_S|| <= 2 V R_t, per query and head."""
    g = np.random.default_rng(21)
    n_h, D, dv, L = 4, 12, 8, 40
    lat = g.standard_normal((L, D)) * 1.5
    worst = 0.0
    for t in range(2, L):
        q = g.standard_normal((n_h, D))
        I = g.standard_normal(t + 1)
        for k in (1, 3, max(1, t // 2), t):
            row, _, m = topk_row(I, k)
            sel = row[:m]
            o, alpha = dense_attn_row(q, lat[: t + 1], 0.5, dv)
            o_hat = attn_row(q, lat, row, 0.5, dv)
            V = np.max(np.linalg.norm(lat[: t + 1, :dv], axis=1))
            rest = np.setdiff1d(np.arange(t + 1), sel)
            for h in range(n_h):
                A = oracle.captured_mass(alpha[h], row)
                R = 1.0 - A
                o_S = (alpha[h, sel] @ lat[sel, :dv]) / A
                np.testing.assert_allclose(o_hat[h], o_S, rtol=1e-10, atol=1e-12)
                err = np.linalg.norm(o[h] - o_hat[h])
                if rest.size:
                    o_Sb = (alpha[h, rest] @ lat[rest, :dv]) / R
                    np.testing.assert_allclose(err, R * np.linalg.norm(o_Sb - o_S), rtol=1e-9, atol=1e-13)
                assert err <= 2 * V * R + 1e-12
                worst = max(worst, err / max(2 * V * R, 1e-300))
    assert worst > 0.0


# ----------------------------------------------------------------------------- invariances (C7)

def test_indexer_invariances():
    g = np.random.default_rng(5)
    H, d, n = 16, 32, 500
    q = g.standard_normal((H, d))
    w = g.standard_normal(H) / 8
    k = g.standard_normal((n, d))
    I = indexer_row(q, w, k)
    np.testing.assert_array_equal(indexer_row(q, 2 * w, k), 2 * I)          # exact: power-of-two scale
    assert topk_row(2 * I, 37)[0].tolist() == topk_row(I, 37)[0].tolist()
    perm = g.permutation(H)
    np.testing.assert_allclose(indexer_row(q[perm], w[perm], k), I, rtol=1e-13, atol=1e-13)
    # a positive per-head scale on q can be folded into w (ReLU is positively homogeneous)
    sq = np.abs(g.standard_normal(H)) + 0.1
    np.testing.assert_allclose(indexer_row(q * sq[:, None], w, k), indexer_row(q, w * sq, k),
                               rtol=1e-12, atol=1e-12)
    # ReLU matters: a negative head scale cannot be folded
    assert not np.allclose(indexer_row(-q, w, k), indexer_row(q, -w, k))


# ----------------------------------------------------------------------------- ties and signed zero (C8)

def test_ties_constant_row_and_signed_zero():
    for n, k in ((10, 3), (5000, 2048), (7, 7), (7, 9)):
        row, kth, m = topk_row(np.full(n, 0.25), k)
        assert row[:m].tolist() == list(range(min(n, k)))
    I = np.array([0.0, -0.0, 1.0, -0.0, 0.0, -1.0])
    row, kth, m = topk_row(I, 3)
    assert row.tolist() == [0, 1, 2]      # zeros tie regardless of sign; lower positions win
    row, _, _ = topk_row(I, 5)
    assert row.tolist() == [0, 1, 2, 3, 4]


# ----------------------------------------------------------------------------- IndexCache loop (C1, C2, C9)

def _random_layers(n_layers, L, H, d, n_h, D, seed):
    g = np.random.default_rng(seed)
    layers = []
    for _ in range(n_layers):
        layers.append({"q_idx": g.standard_normal((L, H, d)), "w": g.standard_normal((L, H)),
                       "k_idx": g.standard_normal((L, d)), "q": g.standard_normal((L, n_h, D)),
                       "latent": g.standard_normal((L, D))})
    return layers


def test_indexcache_fsss_semantics():
    L, k = 24, 5
    layers = _random_layers(8, L, 4, 8, 2, 10, 9)
    pos = list(range(L))
    r = indexcache_forward("FSSSFSSS", layers, pos, k, 0.4, 6)
    assert r["calls"] == 2 and r["src_layer"] == [0, 0, 0, 0, 4, 4, 4, 4]
    rf = indexcache_forward("FFFFFFFF", layers, pos, k, 0.4, 6)
    assert rf["calls"] == 8
    T0, T4 = r["index"][0], r["index"][4]
    assert not np.array_equal(T0, T4)
    for l in range(8):
        own = T0 if l < 4 else T4
        other = T4 if l < 4 else T0
        np.testing.assert_array_equal(r["index"][l], own)
        expect = np.stack([attn_row(layers[l]["q"][i], layers[l]["latent"], own[i], 0.4, 6) for i in pos])
        np.testing.assert_allclose(r["out"][l], expect, rtol=0, atol=0)
        wrong = np.stack([attn_row(layers[l]["q"][i], layers[l]["latent"], other[i], 0.4, 6) for i in pos])
        assert not np.allclose(r["out"][l][k + 2:], wrong[k + 2:])
        # F layers agree with the all-F run; S layers generally do not
        if l in (0, 4):
            np.testing.assert_array_equal(r["out"][l], rf["out"][l])


def test_first_layer_must_be_f():
    layers = _random_layers(4, 6, 2, 4, 1, 6, 1)
    for roles in ("SFFF", "", "FX"):
        with pytest.raises(RoleError):
            indexcache_forward(roles, layers, [0, 1], 2, 1.0, 3)


def test_index_258_toy():
    """[IC] §1.2: layer 1 picks {2, 5, 8}; layers 2-3 attend over {2, 5, 8} with their OWN latents."""
    L, H, d, n_h, D, dv = 12, 2, 4, 2, 6, 4
    layers = _random_layers(3, L, H, d, n_h, D, 4)
    t = 10
    big = {2, 5, 8}
    k_idx = np.zeros((L, d))
    for s in range(L):
        k_idx[s] = (5.0 if s in big else -1.0) * np.ones(d) + 0.01 * s
    layers[0]["k_idx"] = k_idx
    layers[0]["q_idx"][:] = 1.0
    layers[0]["w"][:] = 1.0
    r = indexcache_forward("FSS", layers, [t], 3, 0.5, dv)
    assert r["index"][0][0].tolist() == [2, 5, 8]
    for l in (1, 2):
        np.testing.assert_array_equal(r["index"][l][0], [2, 5, 8])
        own = attn_row(layers[l]["q"][0], layers[l]["latent"], np.array([2, 5, 8]), 0.5, dv)
        np.testing.assert_array_equal(r["out"][l][0], own)
        borrowed = attn_row(layers[l]["q"][0], layers[0]["latent"], np.array([2, 5, 8]), 0.5, dv)
        assert not np.allclose(own, borrowed)


def test_index_override_and_overlap_metric():
    L, k = 10, 3
    layers = _random_layers(2, L, 2, 4, 1, 6, 2)
    forced = np.tile(np.array([0, 1, -1]), (L, 1))
    r = indexcache_forward("FS", layers, list(range(L)), k, 1.0, 4, index_override={0: forced})
    np.testing.assert_array_equal(r["index"][1], forced)
    assert oracle.overlap([0, 1, -1], [1, 2, 0], 3) == 2 / 3


def test_overlap_special_cases():
    """Overlap = |A ∩ B| / k over valid entries: identical full rows give 1, disjoint rows 0,
    order and -1 padding do not matter, and a short row (fewer than k valid) stays below 1."""
    a = np.arange(8)
    assert oracle.overlap(a, a[::-1], 8) == 1.0
    assert oracle.overlap(a, a + 8, 8) == 0.0
    assert oracle.overlap([3, 1, -1, -1], [1, -1, 3, -1], 4) == 0.5
    assert oracle.overlap([0, 1, 2, -1], [2, 1, 0, -1], 4) == 0.75


def test_e4m3fn_encoder_round_trip_and_hand_values():
    """Every finite code decodes and re-encodes to itself (signed zero included); values
    worked out by hand from the format: the maximum, a power of two, ties to the even
    mantissa in the normal and subnormal ranges, and signed zero."""
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_e4m3fn(codes)
    ok = ~np.isnan(vals)
    assert np.array_equal(oracle.encode_e4m3fn(vals[ok]), codes[ok])
    cases = [(448.0, 0x7E), (-448.0, 0xFE), (0.5, 0x30), (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -9, 0x01),
             (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (-0.0, 0x80), (0.0, 0x00), (440.0, 0x7E)]
    for v, c in cases:
        assert int(oracle.encode_e4m3fn(v)) == c, (v, c)


def test_e4m3fn_encoder_matches_torch_cast():
    """An independent implementation: torch's CPU float8_e4m3fn cast (round to nearest
    even) on values spread over the whole range, subnormals included."""
    g = np.random.default_rng(5)
    v = (g.standard_normal(20000) * np.exp2(g.integers(-12, 9, 20000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3fn(v), want)


def test_quantize_rows_definition():
    """Zero rows get scale 1 and zero codes; each row's largest magnitude lands on +-448;
    the result equals the seeded generators' torch-based quantiser."""
    g = np.random.default_rng(6)
    x = (g.standard_normal((64, 128)) * np.exp2(g.integers(-6, 6, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    codes, scales = oracle.quantize_fp8_rows(x)
    assert scales[3] == 1.0 and np.all(codes[3] == 0)
    big = np.abs(x).argmax(axis=1)
    top = codes[np.arange(64), big]
    assert np.all((top[np.arange(64) != 3] & 0x7F) == 0x7E)
    tq, ts = synth.quantize_fp8_rows(torch.from_numpy(x))
    assert np.array_equal(codes, tq.view(torch.uint8).numpy())
    assert np.array_equal(scales, ts.numpy())
