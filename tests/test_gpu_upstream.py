"""GPU parity of the indexer projections and the decode-time cache append against the
oracle (oracle/upstream.py).

Tolerance of the projections: the GPU multiplies bf16 inputs with fp32 accumulation
(every bf16 x bf16 product is exact in fp32; summing K <= 4096 terms moves a result by
about K * 2^-24 of its partial sums, below 1e-4 of the row's scale), runs the LayerNorm
and the rotation in fp32 (angles in fp64) and rounds each output once to bf16 (half an
ulp: 2^-9 relative).  Each element must satisfy |gpu - oracle| <= 2^-8 |oracle| +
1e-4 max|oracle row|, the oracle evaluated in fp64 on the same bf16 inputs.
"""
import numpy as np
import pytest
import torch

import dsa_indexer_indexcache_amd as dsa
import oracle
import synth
from oracle import upstream
from parity import OracleView, check_indexer, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print("[case] " + msg, flush=True)


def _bf(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _f64(t):
    return oracle.decode_bf16(synth.bits(t))


def _inputs(n, r, hidden, H, d, seed, pos0):
    g = np.random.default_rng(seed)
    q_lat = _bf(g.standard_normal((n, r)))
    h = _bf(g.standard_normal((n, hidden)))
    wq = _bf(g.standard_normal((H * d, r)) / np.sqrt(r))
    wk = _bf(g.standard_normal((d, hidden)) / np.sqrt(hidden))
    ww = _bf(g.standard_normal((H, hidden)) / np.sqrt(hidden))
    gamma = torch.from_numpy((1.0 + 0.1 * g.standard_normal(d)).astype(np.float32))
    beta = torch.from_numpy((0.1 * g.standard_normal(d)).astype(np.float32))
    pos = torch.from_numpy((pos0 + g.permutation(n)).astype(np.int32))
    return q_lat, h, wq, wk, ww, gamma, beta, pos


def _check_close(got, want, what):
    got = got.float().cpu().numpy().astype(np.float64)
    scale = np.abs(want).reshape(want.shape[0], -1).max(axis=1)
    scale = scale.reshape((-1,) + (1,) * (want.ndim - 1))
    tol = 2.0 ** -8 * np.abs(want) + 1e-4 * scale
    err = np.abs(got - want)
    worst = float((err / tol).max())
    assert np.all(err <= tol), "%s: worst error %.3g of the tolerance" % (what, worst)
    return worst


@pytest.mark.parametrize("n,r,hidden,rope,pos0", [(700, 512, 768, 64, 190000), (129, 64, 128, 32, 0),
                                                  (256, 128, 192, 0, 5)])
def test_indexer_project_against_oracle(n, r, hidden, rope, pos0):
    announce("indexer projection n=%d r=%d hidden=%d rope=%d" % (n, r, hidden, rope))
    H, d = 64, 128
    q_lat, h, wq, wk, ww, gamma, beta, pos = _inputs(n, r, hidden, H, d, seed=n + r, pos0=pos0)
    q_idx, k_idx, w = dsa.indexer_project(q_lat.to(DEV), h.to(DEV), wq.to(DEV), wk.to(DEV), gamma.to(DEV),
                                          beta.to(DEV), ww.to(DEV), pos.to(DEV), H, rope_dim=rope)
    torch.cuda.synchronize()
    # rope_dim 0 (no rotation): the oracle's rotation at position 0 is the identity
    opos, ord_ = (pos.numpy(), rope) if rope else (np.zeros(n, dtype=np.int64), 2)
    rq, rk, rw = upstream.indexer_project(_f64(q_lat), _f64(h), _f64(wq).T, _f64(wk).T, gamma.double().numpy(),
                                          beta.double().numpy(), _f64(ww).T, opos, H, d, rope_dim=ord_, base=10000.0)
    print("q", _check_close(q_idx, rq, "q_idx"), "k", _check_close(k_idx, rk, "k_idx"), "w",
          _check_close(w, rw, "w"), flush=True)


def test_projected_inputs_feed_the_indexer():
    """Projection -> (bf16) indexer + top-k: the selection matches the oracle's on the
    projected tensors, and after per-row fp8 quantisation on the device too."""
    announce("projection -> indexer")
    n, r, hidden, H, d, k = 1200, 256, 512, 64, 128, 200
    q_lat, h, wq, wk, ww, gamma, beta, _ = _inputs(n, r, hidden, H, d, seed=3, pos0=0)
    pos = torch.arange(n, dtype=torch.int32)
    q_idx, k_idx, w = dsa.indexer_project(q_lat.to(DEV), h.to(DEV), wq.to(DEV), wk.to(DEV), gamma.to(DEV),
                                          beta.to(DEV), ww.to(DEV), pos.to(DEV), H)
    seqs = dsa.Seqs.prefill(n)
    idx, sc = dsa.indexer_topk(q_idx, k_idx, w, k, seqs, want_scores=True)
    torch.cuda.synchronize()
    li = synth.LayerInputs(q_idx, None, k_idx, None, w, None, None)
    print(check_indexer(OracleView(li), seqs, sample_rows(n, k, 150, seed=4), k, idx, sc, exact=False))
    qc, qs = dsa.quantize_fp8_rows(q_idx)
    kc, ks = dsa.quantize_fp8_rows(k_idx)
    idx8, sc8 = dsa.indexer_topk(qc, kc, w, k, seqs, q_scale=qs, k_scale=ks, want_scores=True)
    torch.cuda.synchronize()
    l8 = synth.LayerInputs(qc, qs, kc, ks, w, None, None)
    print(check_indexer(OracleView(l8), seqs, sample_rows(n, k, 150, seed=5), k, idx8, sc8, exact=False))


def test_indexer_project_chunk_size():
    """One 8192-token prefill chunk at the GLM-5 query latent width (2048) and a hidden
    size of 4096: sampled rows against the oracle."""
    announce("indexer projection 8192 x (2048, 4096)")
    n, r, hidden, H, d = 8192, 2048, 4096, 64, 128
    q_lat, h, wq, wk, ww, gamma, beta, pos = _inputs(n, r, hidden, H, d, seed=11, pos0=100000)
    q_idx, k_idx, w = dsa.indexer_project(q_lat.to(DEV), h.to(DEV), wq.to(DEV), wk.to(DEV), gamma.to(DEV),
                                          beta.to(DEV), ww.to(DEV), pos.to(DEV), H)
    torch.cuda.synchronize()
    rows = np.array(sample_rows(n, 128, 60, seed=12))
    rq, rk, rw = upstream.indexer_project(_f64(q_lat[rows]), _f64(h[rows]), _f64(wq).T, _f64(wk).T,
                                          gamma.double().numpy(), beta.double().numpy(), _f64(ww).T,
                                          pos.numpy()[rows], H, d)
    r_t = torch.as_tensor(rows, device=DEV)
    print(len(rows), _check_close(q_idx[r_t], rq, "q_idx"), _check_close(k_idx[r_t], rk, "k_idx"),
          _check_close(w[r_t], rw, "w"), flush=True)


@pytest.mark.parametrize("width,dtype", [(576, torch.bfloat16), (128, torch.uint8), (1, torch.float32),
                                         (3, torch.bfloat16)])
def test_cache_append_against_oracle(width, dtype):
    """New rows of 5 sequences written at k_start + len (the last one out of range: skipped);
    16-byte rows (latent, fp8 keys) and unaligned widths (scales, 6-byte rows)."""
    announce("cache append width=%d %s" % (width, dtype))
    caps = np.array([7, 3, 12, 1, 5])
    lens = np.array([2, 0, 11, 0, 4])
    g = np.random.default_rng(width)
    cache_np = g.integers(0, 200, size=(int(caps.sum()), width)).astype(np.float32)
    rows_np = g.integers(0, 200, size=(5, width)).astype(np.float32)
    cache = torch.from_numpy(cache_np).to(dtype).to(DEV)
    rows = torch.from_numpy(rows_np).to(dtype).to(DEV)
    offs = np.concatenate([[0], np.cumsum(caps)[:-1]])
    dst = offs + lens
    dst[4] = caps.sum() + 3                        # outside the cache: skipped
    dsa.cache_append(cache, torch.from_numpy(dst.astype(np.int64)).to(DEV), rows)
    torch.cuda.synchronize()
    want, new_lens = upstream.cache_append(torch.from_numpy(cache_np).to(dtype).float().numpy(), lens[:4], caps[:4],
                                           torch.from_numpy(rows_np).to(dtype).float().numpy()[:4])
    np.testing.assert_array_equal(cache.float().cpu().numpy(), want)
    assert new_lens.tolist() == [3, 1, 12, 1]
