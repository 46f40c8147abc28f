"""The allocation-free entry point (indexcache_forward_noalloc) against indexcache_forward.

Both run the same kernels on the same inputs, so their outputs must be identical bit
for bit.  The decode shapes use every kernel that needs workspace (score slab, the
multi-workgroup top-k state, split attention partials).  Two calls in a row, the second
smaller, check that nothing a call leaves in the shared scratch array leaks into the next.
"""
import numpy as np
import pytest
import torch

import dsa_indexer_indexcache_amd as dsa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print("[case] " + msg, flush=True)


def _decode_case(lens, roles, layer0):
    lens = [int(x) for x in lens]
    seqs = dsa.Seqs.decode(lens)
    layers = [dsa.layer_dict(synth.decode_layer(layer0 + l, lens, device=DEV)) for l in range(len(roles))]
    return seqs, layers


def _compare(roles, layers, seqs, k, n_h=128):
    B = seqs.n_q
    ref = dsa.indexcache_forward(roles, layers, k, seqs=seqs, want_scores=True)
    outs = [torch.full((B, n_h, 512), float("nan"), dtype=torch.float32, device=DEV) for _ in roles]
    icache = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    scache = torch.full((B, k), float("nan"), dtype=torch.float32, device=DEV)
    got = dsa.indexcache_forward_noalloc(roles, layers, k, outs, icache, seqs=seqs, score_cache=scache)
    torch.cuda.synchronize()
    assert got.n_indexer_calls == ref.n_indexer_calls and got.src_layer == ref.src_layer
    assert torch.equal(got.index_cache, ref.index_cache)
    assert torch.equal(got.score_cache, ref.score_cache)
    for l in range(len(roles)):
        assert torch.equal(got.outs[l], ref.outs[l]), "layer %d output differs" % l


def test_noalloc_matches_forward_twice_second_smaller():
    announce("noalloc: decode B=4 long rows, then B=2 shorter rows")
    k = 2048
    seqs, layers = _decode_case([70001, 41000, 36000, 52000], "FSF", 0)
    _compare("FSF", layers, seqs, k)
    del layers
    seqs, layers = _decode_case([33000, 9000], "FS", 5)
    _compare("FS", layers, seqs, k)


def test_noalloc_prefill_chunks():
    announce("noalloc: prefill L=3000 in 1024-row chunks")
    L, k = 3000, 256
    layers = [dsa.layer_dict(synth.make_layer(L, L, 64, 128, 128, wid=1, layer=l, device=DEV)) for l in range(2)]
    ref = dsa.indexcache_forward("FS", layers, k, q_chunk=1024)
    outs = [torch.empty((L, 128, 512), dtype=torch.float32, device=DEV) for _ in range(2)]
    icache = torch.empty((L, k), dtype=torch.int32, device=DEV)
    got = dsa.indexcache_forward_noalloc("FS", layers, k, outs, icache, q_chunk=1024)
    torch.cuda.synchronize()
    assert torch.equal(got.index_cache, ref.index_cache)
    for l in range(2):
        assert torch.equal(got.outs[l], ref.outs[l])
