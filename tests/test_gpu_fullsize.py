"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Every query row is independent, so checking a stratified sample of rows (chunk and
budget edges, the last rows, seeded uniform draws) is exact parity for those rows.
Inputs are generated on the device from the seeded generators; the oracle reads back
the exact device bytes it needs (the key rows of a sequence, the sampled query rows,
the latent rows a sampled query selected).

Attention rows of early chunks are checked by calling dsa_sparse_attn on that chunk's
query rows with the index cache the loop wrote (the loop's own output buffer is a ring
of one chunk, as in the benchmark); the same call on the last chunk must reproduce the
loop's output bit for bit, which ties the two together.
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


def _chunk_rows(L, chunk, chunks, per, seed):
    """`per` stratified rows from each listed chunk (its first and last row included)."""
    g = np.random.default_rng(seed)
    rows = []
    for c in chunks:
        r0, r1 = c * chunk, min(L, (c + 1) * chunk)
        rows += sorted({r0, r1 - 1, *g.integers(r0, r1, size=per - 2).tolist()})
    return rows


def _attention_by_chunk(layer, seqs, icache, rows, chunk, L, scale):
    """Attention of the given rows recomputed chunk by chunk through dsa_sparse_attn with
    the loop's index cache, checked against the oracle; returns (rows, worst error)."""
    worst = 0.0
    by_chunk = {}
    for r in rows:
        by_chunk.setdefault(r // chunk, []).append(r)
    for c, rs in sorted(by_chunk.items()):
        r0, r1 = c * chunk, min(L, (c + 1) * chunk)
        s = dsa.Seqs.prefill(r1 - r0, n_k=L, q_pos0=r0)
        out = dsa.sparse_attn(layer.q[r0:r1], layer.latent, icache[r0:r1].contiguous(), s)
        torch.cuda.synchronize()
        worst = max(worst, check_attention(OracleView(layer), seqs, rs, icache, out, 576 ** -0.5,
                                           out_row_of=lambda i, r0=r0: i - r0))
    return len(rows), worst


def test_cfg1_prefill_L32768_bf16():
    """One F layer at L = 32768, H^I = 64, d_I = 128, k = 2048, 128 heads (one chunk):
    1,056 indexer rows and 264 attention rows."""
    announce("full size: prefill L=32768 bf16")
    wl = synth.WORKLOADS[1]
    L, k = wl.L, wl.k
    layers = _layers(1, "F", L)
    res = dsa.indexcache_forward("F", [dsa.layer_dict(x) for x in layers], k, want_scores=True)
    torch.cuda.synchronize()
    seqs = dsa.Seqs.prefill(L)
    view = OracleView(layers[0])
    rows = sample_rows(L, k, 1040, seed=1)
    assert len(rows) >= 1024
    st = check_indexer(view, seqs, rows, k, res.index_cache, res.score_cache, exact=False)
    print("indexer", st, flush=True)
    arows = rows[::4]
    assert len(arows) >= 256
    err = check_attention(view, seqs, arows, res.index_cache, res.outs[0], wl.scale)
    print("attention rows %d, max abs error %.2e" % (len(arows), err), flush=True)


def test_cfg4_prefill_L200000_fp8_fsss():
    """The benchmark's stack: FSSS at L = 200000, fp8 indexer, 8192-query chunks, a
    one-chunk output ring; the index cache is kept whole.  >= 256 indexer rows; attention
    of all four layers on rows of chunks 0, 6, 12, 18 and 24 (the last)."""
    announce("full size: prefill L=200000 fp8 FSSS")
    wl = synth.WORKLOADS[4]
    L, k, chunk = wl.L, wl.k, wl.q_chunk
    layers = _layers(4, wl.roles, L)
    res = dsa.indexcache_forward(wl.roles, [dsa.layer_dict(x) for x in layers], k, q_chunk=chunk,
                                 index_rows=L, out_rows=chunk, want_scores=True)
    torch.cuda.synchronize()
    assert res.n_indexer_calls == 1 and res.n_chunks == (L + chunk - 1) // chunk and res.src_layer == [0, 0, 0, 0]
    seqs = dsa.Seqs.prefill(L)
    rows = sample_rows(L, k, 250, seed=2, extra=(16383, 16384, 98303, 98304, L - chunk // 2))
    assert len(rows) >= 256
    announce("indexer rows %d" % len(rows))
    print("indexer", check_indexer(OracleView(layers[0]), seqs, rows, k, res.index_cache, res.score_cache,
                                   exact=False), flush=True)
    last = (L - 1) // chunk
    arows = _chunk_rows(L, chunk, [0, 6, 12, 18, last], 8, seed=3)
    for l in range(len(wl.roles)):
        announce("attention layer %d" % l)
        print(l, _attention_by_chunk(layers[l], seqs, res.index_cache, arows, chunk, L, wl.scale), flush=True)
        # the loop's ring holds the last chunk: the separate call reproduces it exactly
        r0 = last * chunk
        again = dsa.sparse_attn(layers[l].q[r0:], layers[l].latent, res.index_cache[r0:].contiguous(),
                                dsa.Seqs.prefill(L - r0, n_k=L, q_pos0=r0))
        torch.cuda.synchronize()
        assert torch.equal(again, res.outs[l][: L - r0])


def test_cfg3_decode_all_47_layers():
    """Decode as the benchmark runs it: 8 sequences of 150K-200K keys, one query each,
    through the 47-layer stack (F every fourth layer).  Every F layer's selection (computed
    again by dsa_indexer_topk; the last one must equal the loop's final index cache) is
    checked against the oracle, and every layer's output on its F layer's rows."""
    announce("full size: decode B=8, 47 layers")
    wl = synth.WORKLOADS[3]
    lens = synth.decode_lengths(3)
    seqs = dsa.Seqs.decode(lens)
    roles, k = wl.roles, wl.k
    layers = [synth.decode_layer(l, lens, device=DEV) for l in range(len(roles))]
    res = dsa.indexcache_forward(roles, [dsa.layer_dict(x) for x in layers], k, seqs=seqs)
    torch.cuda.synchronize()
    assert res.n_indexer_calls == 12
    rows = list(range(len(lens)))
    sel = {}
    for f in [l for l, r in enumerate(roles) if r == "F"]:
        li = layers[f]
        sel[f], sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
        torch.cuda.synchronize()
        announce("decode F layer %d" % f)
        print(f, check_indexer(OracleView(li), seqs, rows, k, sel[f], sc, exact=False), flush=True)
    assert torch.equal(sel[max(sel)], res.index_cache)
    worst = 0.0
    for l in range(len(roles)):
        worst = max(worst, check_attention(OracleView(layers[l]), seqs, rows, sel[res.src_layer[l]], res.outs[l],
                                           wl.scale))
    print("attention: 47 layers x 8 rows, max abs error %.2e" % worst, flush=True)


def test_cfg2_prefill_L65536_fsssfsss():
    """Eight layers FSSSFSSS at L = 65536 in 8192-query chunks with a one-chunk output
    ring.  The loop's cache ends with layer 4's selection; layer 0's comes from the same
    loop over layers 0-3 alone (FSSS, identical launches).  512 indexer rows of each F
    layer; attention of all eight layers on rows of chunks 0, 3, 5 and 7."""
    announce("full size: prefill L=65536 FSSSFSSS")
    wl = synth.WORKLOADS[2]
    L, k, chunk = wl.L, wl.k, 8192
    layers = _layers(2, wl.roles, L)
    ld = [dsa.layer_dict(x) for x in layers]
    res = dsa.indexcache_forward(wl.roles, ld, k, q_chunk=chunk, index_rows=L, out_rows=chunk, want_scores=True)
    torch.cuda.synchronize()
    assert res.n_indexer_calls == 2 and res.n_chunks == L // chunk
    assert res.src_layer == [0, 0, 0, 0, 4, 4, 4, 4]
    first = dsa.indexcache_forward("FSSS", ld[:4], k, q_chunk=chunk, index_rows=L, out_rows=chunk,
                                   want_scores=True)
    torch.cuda.synchronize()
    caches = {0: (first.index_cache, first.score_cache), 4: (res.index_cache, res.score_cache)}
    seqs = dsa.Seqs.prefill(L)
    rows = sample_rows(L, k, 520, seed=4)
    assert len(rows) >= 512
    for f in (0, 4):
        announce("indexer layer %d, rows %d" % (f, len(rows)))
        print(f, check_indexer(OracleView(layers[f]), seqs, rows, k, caches[f][0], caches[f][1], exact=False),
              flush=True)
    arows = _chunk_rows(L, chunk, [0, 3, 5, 7], 6, seed=5)
    for l in range(8):
        announce("attention layer %d" % l)
        print(l, _attention_by_chunk(layers[l], seqs, caches[res.src_layer[l]][0], arows, chunk, L, wl.scale),
              flush=True)
    for l in range(4):           # both loops end on the last chunk: layers 0-3 agree exactly
        assert torch.equal(first.outs[l], res.outs[l])
