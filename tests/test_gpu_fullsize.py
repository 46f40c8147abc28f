"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Every query row is independent, so checking a stratified sample of rows (chunk and
budget edges, the last rows, seeded uniform draws) is exact parity for those rows.
Inputs are generated on the device from the seeded generators; the oracle reads back
the exact device bytes it needs (the key rows of a sequence, the sampled query rows,
the latent rows a sampled query selected).
"""
import numpy as np
import pytest
import torch

import dsa_indexer_indexcache_amd as dsa
import synth
from parity import OracleView, check_attention, check_indexer, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print("[case] " + msg, flush=True)


@pytest.fixture(autouse=True)
def _release_memory():
    """Each case holds up to ~120 GB of inputs; hand it back before the next one."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _layers(wid, roles, L, indexer_roles="F"):
    return [synth.workload_layer(wid, l, device=DEV, L=L, with_indexer=roles[l] in indexer_roles)
            for l in range(len(roles))]


def test_cfg1_prefill_L32768_bf16():
    """One F layer at L = 32768, H^I = 64, d_I = 128, k = 2048, 128 heads (one chunk)."""
    announce("full size: prefill L=32768 bf16")
    wl = synth.WORKLOADS[1]
    L, k = wl.L, wl.k
    layers = _layers(1, "F", L)
    res = dsa.indexcache_forward("F", [dsa.layer_dict(x) for x in layers], k, want_scores=True)
    torch.cuda.synchronize()
    seqs = dsa.Seqs.prefill(L)
    view = OracleView(layers[0])
    rows = sample_rows(L, k, 96, seed=1)
    print(check_indexer(view, seqs, rows, k, res.index_cache, res.score_cache, exact=False))
    print(check_attention(view, seqs, rows[::2], res.index_cache, res.outs[0], wl.scale))


def test_cfg4_prefill_L200000_fp8_fsss():
    """The benchmark's stack: FSSS at L = 200000, fp8 indexer, 8192-query chunks, a
    one-chunk output ring.  The index cache is kept whole so that rows of every chunk
    can be checked; the last chunk's attention is checked on all four layers."""
    announce("full size: prefill L=200000 fp8 FSSS")
    wl = synth.WORKLOADS[4]
    L, k, chunk = wl.L, wl.k, wl.q_chunk
    layers = _layers(4, wl.roles, L)
    res = dsa.indexcache_forward(wl.roles, [dsa.layer_dict(x) for x in layers], k, q_chunk=chunk,
                                 index_rows=L, out_rows=chunk, want_scores=True)
    torch.cuda.synchronize()
    assert res.n_indexer_calls == 1 and res.n_chunks == (L + chunk - 1) // chunk and res.src_layer == [0, 0, 0, 0]
    seqs = dsa.Seqs.prefill(L)
    rows = sample_rows(L, k, 16, seed=2, extra=(16383, 16384, 98303, 98304, L - chunk // 2))
    print(check_indexer(OracleView(layers[0]), seqs, rows, k, res.index_cache, res.score_cache, exact=False))
    last0 = (L - 1) // chunk * chunk
    arows = [r for r in sample_rows(L, k, 64, seed=3) if r >= last0][:12] + [last0, L - 1]
    for l in range(len(wl.roles)):
        print(l, check_attention(OracleView(layers[l]), seqs, arows, res.index_cache, res.outs[l], wl.scale,
                                 out_row_of=lambda i: i % chunk))


def test_cfg3_decode_full_lengths():
    """Decode: 8 sequences of 150K-200K keys, one query each, through an FSSS stack."""
    announce("full size: decode B=8")
    wl = synth.WORKLOADS[3]
    lens = synth.decode_lengths(3)
    seqs = dsa.Seqs.decode(lens)
    roles, k = "FSSS", wl.k
    layers = [synth.decode_layer(l, lens, device=DEV) for l in range(len(roles))]
    res = dsa.indexcache_forward(roles, [dsa.layer_dict(x) for x in layers], k, seqs=seqs, want_scores=True)
    torch.cuda.synchronize()
    rows = list(range(len(lens)))
    print(check_indexer(OracleView(layers[0]), seqs, rows, k, res.index_cache, res.score_cache, exact=False))
    for l in range(len(roles)):
        print(l, check_attention(OracleView(layers[l]), seqs, rows, res.index_cache, res.outs[l], wl.scale))


def test_cfg2_prefill_L65536_fsssfsss():
    """Eight layers FSSSFSSS at L = 65536 in 8192-query chunks with a one-chunk output
    ring: after the loop the cache holds layer 4's selection, which layers 4-7 used."""
    announce("full size: prefill L=65536 FSSSFSSS")
    wl = synth.WORKLOADS[2]
    L, k, chunk = wl.L, wl.k, 8192
    layers = _layers(2, wl.roles, L)
    res = dsa.indexcache_forward(wl.roles, [dsa.layer_dict(x) for x in layers], k, q_chunk=chunk,
                                 index_rows=L, out_rows=chunk, want_scores=True)
    torch.cuda.synchronize()
    assert res.n_indexer_calls == 2 and res.n_chunks == L // chunk
    assert res.src_layer == [0, 0, 0, 0, 4, 4, 4, 4]
    seqs = dsa.Seqs.prefill(L)
    rows = sample_rows(L, k, 24, seed=4)
    print(check_indexer(OracleView(layers[4]), seqs, rows, k, res.index_cache, res.score_cache, exact=False))
    last0 = L - chunk
    arows = [r for r in sample_rows(L, k, 64, seed=5) if r >= last0][:8] + [last0, L - 1]
    for l in range(4, 8):
        print(l, check_attention(OracleView(layers[l]), seqs, arows, res.index_cache, res.outs[l], wl.scale,
                                 out_row_of=lambda i: i % chunk))
