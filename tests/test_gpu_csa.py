"""GPU parity of compressed sparse attention (DeepSeek-V4 CSA) selection against the oracle
(oracle/csa.py): the gated-pooling KV compression, the indexer + top-k over compressed
blocks (block s visible to query t iff s < t // m), the bf16-score selector and its recall
against the fp32 selector, and the IndexCache loop over compressed keys.

Compression tolerance: the output is a convex combination of the window's values
(softmax weights), computed in fp32 with a running max: each of the 2m weights carries a
few fp32 rounding steps (exp, rescale, fma), so |gpu - oracle| <= (2m + 8) 2^-21 max|v| over
the window's values of that column; a bf16 output adds half a bf16 step, at most 2^-8 |out|
(8 significand bits).
"""
import numpy as np
import pytest
import torch

import dsa_indexer_indexcache_amd as dsa
import oracle
import synth
from oracle import csa as ocsa
from parity import OracleView, check_attention, check_indexer, check_indexer_bf16, row_geometry, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print("[case] " + msg, flush=True)


def _f64(t):
    return oracle.decode_bf16(synth.bits(t))


def _window_absmax(ca, cb, m):
    """max |value| over each entry's pooling window, per column (float64 [n // m, c])."""
    n, c = ca.shape
    nb = n // m
    a = np.abs(ca[:nb * m]).reshape(nb, m, c).max(axis=1)
    b = np.zeros_like(a)
    if nb > 1:
        b[1:] = np.abs(cb[:(nb - 1) * m]).reshape(nb - 1, m, c).max(axis=1)
    return np.maximum(a, b)


def _compress_case(n, c, m, seed=0):
    ins = synth.csa_inputs(n, c, m, seed)
    host = [_f64(t) for t in ins[:4]] + [t.numpy().astype(np.float64) for t in ins[4:]]
    want = ocsa.compress_kv(*host, m)
    return [t.to(DEV) for t in ins], host, want


@pytest.mark.parametrize("n,c,m", [(1003, 128, 4), (4096 + 77, 512, 128), (7, 128, 4), (96, 64, 1)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_compress_matches_oracle(n, c, m, out_dtype):
    announce("csa compress n=%d c=%d m=%d %s" % (n, c, m, out_dtype))
    dev_in, host, want = _compress_case(n, c, m)
    out = dsa.csa_compress(*dev_in, m, out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert got.shape == want.shape == (n // m, c)
    tol = (2 * m + 8) * 2.0 ** -21 * _window_absmax(host[0], host[1], m)
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(want)
    err = np.abs(got - want)
    assert np.all(err <= tol), "worst error %.3g of the tolerance" % float((err / np.maximum(tol, 1e-300)).max())
    print("entries %d, worst error / tolerance %.3f" % (n // m, float((err / np.maximum(tol, 1e-300)).max())),
          flush=True)


def test_compress_incremental_entries_are_bit_identical():
    """A decode step that completes a group writes one entry (block0 = n // m - 1) from all n rows:
    it equals the same entry of the one-shot compression bit for bit; n // m <= block0 is a no-op."""
    announce("csa compress incremental")
    n, c, m = 4 * 333 + 2, 128, 4
    dev_in, _, _ = _compress_case(n, c, m, seed=3)
    full = dsa.csa_compress(*dev_in, m, out_dtype=torch.float32)
    for b0 in (0, 1, n // m - 1):
        part = dsa.csa_compress(*dev_in, m, block0=b0, out_dtype=torch.float32)
        assert torch.equal(part, full[b0:])
    sentinel = torch.full((0, c), 7.0, device=DEV)
    assert dsa.csa_compress(*dev_in, m, block0=n // m, out=sentinel, out_dtype=torch.float32).shape == (0, c)


def _csa_layer(n_tok, m, H, d, n_h, wid, layer, qk_dtype="bf16"):
    """Indexer queries and head weights of n_tok tokens over n_tok // m compressed keys."""
    return synth.make_layer(n_tok, n_tok // m, H, d, n_h, wid=wid, layer=layer, qk_dtype=qk_dtype).to(DEV)


@pytest.mark.parametrize("qk_dtype", ["bf16", "fp8"])
def test_csa_topk_prefill(qk_dtype):
    """One sequence, 4096 query tokens over 1024 blocks of 4 (the one-pass fused path):
    rows with t < 4 see nothing, rows with fewer than k visible blocks are padded."""
    announce("csa top-k prefill %s" % qk_dtype)
    n_tok, m, k = 4096, 4, 128
    li = _csa_layer(n_tok, m, 64, 128, 16, wid=11, layer=0, qk_dtype=qk_dtype)
    seqs = dsa.Seqs.compressed(n_tok, m)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, q_scale=li.q_scale, k_scale=li.k_scale,
                               want_scores=True)
    torch.cuda.synchronize()
    rows = sample_rows(n_tok, k, n=24, seed=5, extra=(0, 3, 4, 5, 7, 8, 4 * k - 1, 4 * k, 4 * k + 4))
    st = check_indexer(OracleView(li), seqs, rows, k, idx, sc, exact=False)
    ig = idx.cpu()
    assert torch.all(ig[:4] == -1)
    print("rows %d, recall %.5f" % (st["rows"], st["recall_mean"]), flush=True)


def test_csa_topk_chunked_and_packed_batch():
    """Chunked prefill (q_pos0 > 0) and a packed batch of 3 sequences (the slab path) over
    compressed keys agree with the oracle; a chunk of the one-sequence call is bit-identical."""
    announce("csa top-k chunk and batch")
    m, k = 4, 64
    n_tok = 2048
    li = _csa_layer(n_tok, m, 32, 128, 16, wid=11, layer=1)
    full, _ = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, dsa.Seqs.compressed(n_tok, m))
    c0 = 1000
    seqs_c = dsa.Seqs.compressed(n_tok - c0, m, q_pos0=c0, n_k=n_tok // m)
    part, _ = dsa.indexer_topk(li.q_idx[c0:], li.k_idx, li.w[c0:], k, seqs_c)
    torch.cuda.synchronize()
    assert torch.equal(part, full[c0:])
    # three sequences of 300, 700 and 1048 tokens with their own compressed caches
    lens = [300, 700, 1048]
    seqs_b = dsa.Seqs.varlen(lens, [L // m for L in lens], [0, 0, 0], block=m)
    k_packed = torch.cat([li.k_idx[:L // m] for L in lens])
    idx_b, sc_b = dsa.indexer_topk(li.q_idx, k_packed, li.w, k, seqs_b, want_scores=True)
    torch.cuda.synchronize()

    class View(OracleView):
        def keys(self):
            return _f64(k_packed)

    rows = sorted({0, 3, 4, 299, 300, 303, 304, 999, 1000, 1500, 2047})
    st = check_indexer(View(li), seqs_b, rows, k, idx_b, sc_b, exact=False)
    print("rows %d, recall %.5f" % (st["rows"], st["recall_mean"]), flush=True)


def test_csa_topk_decode_wide():
    """Decode over long compressed caches (4 sequences of 150K-200K tokens, m = 4: 37K-50K
    blocks per row, the chunked wide selection), fp32 and bf16-score selectors."""
    announce("csa top-k decode wide")
    m, k = 4, 2048
    lens = synth.decode_lengths()[:4]
    n_blk = [int(L) // m for L in lens]
    li = synth.make_layer(4, int(np.sum(n_blk)), 64, 128, 16, wid=12, layer=0, device=DEV)
    seqs = dsa.Seqs.varlen([1] * 4, n_blk, [int(L) - 1 for L in lens], block=m)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    idx_b, sc_b = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True, bf16_scores=True)
    torch.cuda.synchronize()
    view = OracleView(li)
    st = check_indexer(view, seqs, range(4), k, idx, sc, exact=False)
    st_b = check_indexer_bf16(view, seqs, range(4), k, idx_b, sc_b)
    print("fp32 recall %.5f, bf16 recall %.5f" % (st["recall_mean"], st_b["recall_mean"]), flush=True)


@pytest.mark.parametrize("n_tok,k", [(4096, 128), (2000, 600)])
def test_csa_bf16_selector_and_its_recall(n_tok, k):
    """The bf16-score selector agrees with the oracle's (fp32 -> bf16 rounded scores, ties to
    the lower block), and the recall of the fp32 selection by the bf16 one (the per-row overlap
    counted by dsa_index_overlap) matches the oracle's on the same rows."""
    announce("csa bf16 selector n=%d k=%d" % (n_tok, k))
    m = 4
    li = _csa_layer(n_tok, m, 64, 128, 16, wid=11, layer=2)
    seqs = dsa.Seqs.compressed(n_tok, m)
    i32, s32 = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    i16, s16 = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True, bf16_scores=True)
    counts = dsa.index_overlap(i16, i32)
    torch.cuda.synchronize()
    view = OracleView(li)
    rows = sample_rows(n_tok, k, n=20, seed=9, extra=(3, 4, 4 * k, 4 * k + 3))
    check_indexer_bf16(view, seqs, rows, k, i16, s16)
    qv, wv, keys = view.q_idx_rows(rows), view.w_rows(rows), view.keys()
    cg = counts.cpu().numpy()
    got, want = [], []
    for n, i in enumerate(rows):
        p, _ = row_geometry(seqs, i)
        if p < 0:
            assert cg[i] == 0
            continue
        r32, _ = ocsa.csa_topk_row(qv[n], wv[n], keys, i, m, k)
        r16, _ = ocsa.csa_topk_row(qv[n], wv[n], keys, i, m, k, bf16_scores=True)
        v = r32[r32 >= 0]
        want.append(len(set(v.tolist()) & set(r16[r16 >= 0].tolist())) / len(v))
        got.append(cg[i] / len(v))
    gm, wm = float(np.mean(got)), float(np.mean(want))
    assert abs(gm - wm) <= 0.01, (gm, wm)
    print("rows %d, recall of the fp32 selection: gpu %.4f oracle %.4f" % (len(got), gm, wm), flush=True)


def test_indexcache_loop_over_compressed_keys():
    """FSSS over compressed keys: the F layer's selection equals dsa_indexer_topk with the same
    block table bit for bit, and every layer's attention over the compressed latent rows agrees
    with the oracle on the GPU's own index rows (causal: no block at or past t // m)."""
    announce("indexcache FSSS over compressed keys")
    n_tok, m, k, n_h = 1536, 4, 64, 16
    layers = [_csa_layer(n_tok, m, 32, 128, n_h, wid=13, layer=l) for l in range(4)]
    seqs = dsa.Seqs.compressed(n_tok, m)
    res = dsa.indexcache_forward("FSSS", [dsa.layer_dict(x) for x in layers], k, seqs, q_chunk=512,
                                 bf16_scores=True)
    ref, _ = dsa.indexer_topk(layers[0].q_idx, layers[0].k_idx, layers[0].w, k, seqs, bf16_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(res.index_cache, ref)
    rows = sorted({0, 3, 4, 5, 100, 511, 512, 1000, 1535})
    worst = 0.0
    for l, x in enumerate(layers):
        worst = max(worst, check_attention(OracleView(x), seqs, rows, res.index_cache, res.outs[l], 576 ** -0.5))
    print("worst attention error %.2e" % worst, flush=True)


def test_csa_decode_rows_with_nothing_visible():
    """Decode over compressed caches where some queries see no block yet (t < m) and one sees
    two: the wide select and the attention handle empty and short rows (all -1, zero output)."""
    announce("csa decode with empty rows")
    m, k = 4, 1024
    lens = [3, 4, 50000, 9]                    # t = 2, 3 -> no block; t = 49999 -> 12499; t = 8 -> 2
    nb = [L // m for L in lens]
    li = synth.make_layer(4, int(np.sum(nb)), 64, 128, 16, wid=18, layer=0, device=DEV)
    seqs = dsa.Seqs.varlen([1] * 4, nb, [L - 1 for L in lens], block=m)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    out = dsa.sparse_attn(li.q, li.latent, idx, seqs)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    assert np.all(ig[0] == -1) and np.all(ig[1] == -1)
    assert list(ig[3][:2]) == [0, 1] and np.all(ig[3][2:] == -1)
    assert float(out[0].abs().max()) == 0.0 and float(out[1].abs().max()) == 0.0
    view = OracleView(li)
    st = check_indexer(view, seqs, [0, 1, 2, 3], k, idx, sc, exact=False)
    worst = check_attention(view, seqs, [2, 3], idx, out, 576 ** -0.5)
    print(st, "attention error %.2e" % worst, flush=True)
