"""GPU parity of the attention statistics against the oracle: CapturedMass@k /
MissedMass@k and Recall@k ([IDX] §8 items 1-2) and the sparse-training indexer KL with its
multi-layer average ([IDX] §4.2, [IC] §3.1).

Tolerances: the GPU evaluates scores in fp32 from bf16 inputs (exact products, fp32
sums over 576 columns: a relative error of a few 1e-7 of |z|) and softmax sums in fp32,
so a captured mass (a ratio of such sums) is within 1e-4 of the fp64 oracle, and a KL
(sums of p ln p and p I of size up to ln k plus the indexer scores' log-sum-exp) within
1e-3 x max(1, |KL|).  Recall: the oracle's top-k of the dense distribution may differ from
the GPU's at near-ties; the GPU's set must satisfy the top-k tolerance rule on the oracle's
distribution, and the GPU recall must equal its own set's overlap with the selection.
"""
import numpy as np
import pytest
import torch

import dsa_indexer_indexcache_amd as dsa
import oracle
import synth
from parity import OracleView, row_geometry

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print("[case] " + msg, flush=True)


def _dense_alpha(view, seqs, i, scale):
    p, k0 = row_geometry(seqs, i)
    q = view.q_rows([i])[0]
    lat = view.latent_rows(np.arange(k0, k0 + p + 1))
    _, alpha = oracle.dense_attn_row(q, lat, scale, 512)
    return alpha, p


@pytest.mark.parametrize("L,k,n_h", [(700, 64, 128), (1500, 256, 64), (300, 300, 16)])
def test_attention_mass_and_recall(L, k, n_h):
    announce("attention mass / recall L=%d k=%d n_h=%d" % (L, k, n_h))
    li = synth.make_layer(L, L, 64, 128, n_h, wid=1, layer=2).to(DEV)
    seqs = dsa.Seqs.prefill(L)
    idx, _ = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs)
    mass_head, mass, recall = dsa.attention_mass(li.q, li.latent, idx, seqs)
    torch.cuda.synchronize()
    view = OracleView(li)
    rows = sorted({0, 1, k - 1, k, L - 1, *np.random.default_rng(L).integers(0, L, 24).tolist()} - {-1})
    rows = [r for r in rows if 0 <= r < L]
    ig, mh, mm, rc = idx.cpu().numpy(), mass_head.cpu().numpy(), mass.cpu().numpy(), recall.cpu().numpy()
    scale = 576 ** -0.5
    worst = 0.0
    for i in rows:
        alpha, p = _dense_alpha(view, seqs, i, scale)
        ph, agg = oracle.captured_mass_at_k(alpha, ig[i])
        worst = max(worst, float(np.abs(mh[i] - ph).max()), abs(float(mm[i]) - agg))
        assert np.all(np.abs(mh[i] - ph) <= 1e-4) and abs(float(mm[i]) - agg) <= 1e-4, i
        r_or, row = oracle.recall_at_k(alpha, ig[i], k)
        assert abs(float(rc[i]) - r_or) <= 2.0 / min(k, p + 1) + 1e-6, (i, rc[i], r_or)
    print("rows %d, worst mass error %.2e" % (len(rows), worst), flush=True)
    if k >= L:   # the budget covers every prefix: everything is captured, recall is 1
        assert torch.allclose(mass, torch.ones_like(mass), atol=1e-5)
        assert torch.all(recall == 1.0)


def test_recall_set_is_a_valid_top_k():
    """Recall computed from the GPU's own oracle set: a selection equal to the dense top-k
    (taken from the oracle) gives recall 1 except at near-ties; a disjoint one gives 0."""
    announce("recall against the dense top-k itself")
    L, k, n_h = 600, 32, 32
    li = synth.make_layer(L, L, 64, 128, n_h, wid=1, layer=3).to(DEV)
    seqs = dsa.Seqs.prefill(L)
    view = OracleView(li)
    rows = [40, 123, 599]
    best = np.full((L, k), -1, dtype=np.int32)
    for i in range(L):
        best[i, :min(k, i + 1)] = np.arange(min(k, i + 1))   # a fixed low-position selection elsewhere
    for i in rows:
        alpha, _ = _dense_alpha(view, seqs, i, 576 ** -0.5)
        best[i] = oracle.recall_at_k(alpha, np.arange(i + 1), k)[1]
    _, _, rc = dsa.attention_mass(li.q, li.latent, torch.from_numpy(best).to(DEV), seqs)
    torch.cuda.synchronize()
    for i in rows:
        assert float(rc[i]) >= 1.0 - 2.0 / k
    assert float(rc[0]) == 1.0   # one visible key


@pytest.mark.parametrize("L,k,n_h", [(900, 128, 128), (400, 512, 16)])
def test_indexer_kl_and_multilayer_average(L, k, n_h):
    announce("indexer KL L=%d k=%d n_h=%d" % (L, k, n_h))
    layers = [synth.make_layer(L, L, 64, 128, n_h, wid=2, layer=l).to(DEV) for l in range(3)]
    seqs = dsa.Seqs.prefill(L)
    f = layers[0]
    idx, sc = dsa.indexer_topk(f.q_idx, f.k_idx, f.w, k, seqs, want_scores=True)
    kl1, loss1 = dsa.indexer_kl(f.q, f.latent, idx, sc, seqs, want_loss=True)
    kl = None
    for j, lj in enumerate(layers):   # one F layer serving two S layers: (1/3) sum_j KL_j
        kl, loss = dsa.indexer_kl(lj.q, lj.latent, idx, sc, seqs, weight=1.0 / 3, kl=kl, accumulate=j > 0,
                                  want_loss=True)
    torch.cuda.synchronize()
    ig, sg = idx.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    views = [OracleView(x) for x in layers]
    rows = sorted(r for r in {0, 1, k - 1, L - 1, *np.random.default_rng(k).integers(0, L, 20).tolist()} if r < L)
    k1, km = kl1.cpu().numpy(), kl.cpu().numpy()
    worst = 0.0
    for i in rows:
        p, _ = row_geometry(seqs, i)
        sel = ig[i][(ig[i] >= 0) & (ig[i] <= p)]
        vals = []
        for v in views:
            q = v.q_rows([i])[0]
            lat = np.zeros((p + 1, 576))
            lat[sel] = v.latent_rows(sel)
            vals.append(oracle.indexer_kl_row(q, lat, ig[i], sg[i], 576 ** -0.5))
        for got, want in ((k1[i], vals[0]), (km[i], float(np.mean(vals)))):
            err = abs(float(got) - want)
            worst = max(worst, err / max(1.0, abs(want)))
            assert err <= 1e-3 * max(1.0, abs(want)), (i, got, want)
    assert abs(float(loss1[0]) - float(kl1.double().sum())) <= 1e-4 * max(1.0, float(kl1.abs().sum()))
    assert abs(float(loss[0]) - float(kl.double().sum())) <= 1e-4 * max(1.0, float(kl.abs().sum()))
    assert torch.all(kl1 >= -1e-4)
    print("rows %d, worst KL error %.2e" % (len(rows), worst), flush=True)
