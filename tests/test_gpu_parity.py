"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Small shapes span several key tiles and ragged tails; edge cases cover one-row
inputs, budgets larger than the prefix, all-equal scores and signed zeros,
out-of-range index entries, empty batches and the decode (split) attention path.
"""
import numpy as np
import pytest
import torch

import dsa_indexer_indexcache_amd as dsa
import oracle
import synth
from parity import (ATTN_ATOL, OracleView, check_attention, check_indexer, check_valid_row, row_geometry,
                    sample_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print("[case] " + msg, flush=True)


def layer(L, H, d, n_h, wid=9, layer_id=0, dtype="bf16", integer=False, n_k=None):
    li = synth.make_layer(L, L if n_k is None else n_k, H, d, n_h, wid=wid, layer=layer_id, qk_dtype=dtype,
                          integer_indexer=integer)
    return li.to(DEV)


# --------------------------------------------------------------------------- integer-valued: bit-exact

def test_integer_workload_bit_exact():
    announce("integer L=1024 H=8 d=64 k=128 n_h=16")
    li = synth.workload_layer(0, 0).to(DEV)
    seqs = dsa.Seqs.prefill(1024)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, 128, seqs, want_scores=True)
    torch.cuda.synchronize()
    view = OracleView(li)
    st = check_indexer(view, seqs, range(1024), 128, idx, sc, exact=True)
    assert st["rows"] == 1024
    out = dsa.sparse_attn(li.q, li.latent, idx, seqs)
    torch.cuda.synchronize()
    check_attention(view, seqs, range(0, 1024, 3), idx, out, synth.WORKLOADS[0].scale)


@pytest.mark.parametrize("H,d", [(16, 64), (32, 128), (64, 64)])
def test_integer_other_head_shapes(H, d):
    announce("integer H=%d d=%d" % (H, d))
    li = layer(700, H, d, 16, integer=True)
    seqs = dsa.Seqs.prefill(700)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, 97, seqs, want_scores=True)
    torch.cuda.synchronize()
    check_indexer(OracleView(li), seqs, range(700), 97, idx, sc, exact=True)


# --------------------------------------------------------------------------- float inputs

@pytest.mark.parametrize("L,k", [(2500, 256), (2500, 2048), (513, 7)])
def test_bf16_indexer(L, k):
    announce("bf16 indexer L=%d k=%d" % (L, k))
    li = layer(L, 64, 128, 16, wid=1)
    seqs = dsa.Seqs.prefill(L)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    torch.cuda.synchronize()
    st = check_indexer(OracleView(li), seqs, sample_rows(L, k, 96), k, idx, sc, exact=False)
    print(st)


def test_fp8_indexer():
    announce("fp8 indexer L=3000 k=512")
    li = layer(3000, 64, 128, 16, wid=4, dtype="fp8")
    seqs = dsa.Seqs.prefill(3000)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, 512, seqs, q_scale=li.q_scale, k_scale=li.k_scale,
                               want_scores=True)
    torch.cuda.synchronize()
    print(check_indexer(OracleView(li), seqs, sample_rows(3000, 512, 96), 512, idx, sc, exact=False))


@pytest.mark.parametrize("H", [16, 32])
def test_fp8_indexer_fewer_heads(H):
    """The fused fp8 kernel with one and two 16-head blocks."""
    announce("fp8 indexer H=%d" % H)
    li = layer(2100, H, 128, 16, wid=4, layer_id=3, dtype="fp8")
    seqs = dsa.Seqs.prefill(2100)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, 300, seqs, q_scale=li.q_scale, k_scale=li.k_scale,
                               want_scores=True)
    torch.cuda.synchronize()
    print(check_indexer(OracleView(li), seqs, sample_rows(2100, 300, 64), 300, idx, sc, exact=False))


def test_fp8_decode_wide_select():
    """fp8 decode: the fp8 score slab (per-row scales) and the chunked select."""
    announce("fp8 decode")
    lens = [40000, 33000, 500]
    li = synth.make_layer(len(lens), sum(lens), 64, 128, 16, wid=4, layer=9, qk_dtype="fp8",
                          with_attention=False).to(DEV)
    seqs = dsa.Seqs.decode(lens)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, 2048, seqs, q_scale=li.q_scale, k_scale=li.k_scale,
                               want_scores=True)
    torch.cuda.synchronize()
    print(check_indexer(OracleView(li), seqs, range(len(lens)), 2048, idx, sc, exact=False))


def test_chunk_offsets_match_one_call():
    """Queries scored in chunks (q_pos0 > 0, full key prefix) give the same rows as one call."""
    announce("chunked indexer")
    L, k = 1500, 300
    li = layer(L, 64, 128, 16, wid=1, layer_id=2)
    full, fs = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, dsa.Seqs.prefill(L), want_scores=True)
    parts = []
    for r0 in range(0, L, 512):
        r1 = min(L, r0 + 512)
        s = dsa.Seqs.prefill(r1 - r0, n_k=L, q_pos0=r0)
        parts.append(dsa.indexer_topk(li.q_idx[r0:r1].contiguous(), li.k_idx, li.w[r0:r1].contiguous(), k, s,
                                      want_scores=True))
    torch.cuda.synchronize()
    assert torch.equal(full, torch.cat([p[0] for p in parts]))
    assert torch.equal(fs, torch.cat([p[1] for p in parts]))


# --------------------------------------------------------------------------- edge cases

def test_ties_and_signed_zero():
    """All-zero indexer queries: every score is +-0, so the lowest positions win."""
    announce("ties")
    L, k = 600, 50
    li = layer(L, 64, 128, 16, wid=1)
    qz = torch.zeros_like(li.q_idx)
    w = li.w.clone()
    w[:, ::2] = -w[:, ::2].abs()                      # negative weights times ReLU(0) give -0.0 terms
    idx, sc = dsa.indexer_topk(qz, li.k_idx, w, k, dsa.Seqs.prefill(L), want_scores=True)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    for t in range(L):
        m = min(k, t + 1)
        assert ig[t, :m].tolist() == list(range(m)) and np.all(ig[t, m:] == -1)
    assert torch.all(sc == 0)


@pytest.mark.parametrize("L,k", [(1, 1), (1, 5), (17, 1), (64, 64), (65, 64)])
def test_tiny_inputs(L, k):
    announce("tiny L=%d k=%d" % (L, k))
    li = layer(L, 8, 64, 16, integer=True)
    seqs = dsa.Seqs.prefill(L)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    out = dsa.sparse_attn(li.q, li.latent, idx, seqs)
    torch.cuda.synchronize()
    view = OracleView(li)
    check_indexer(view, seqs, range(L), k, idx, sc, exact=True)
    check_attention(view, seqs, range(L), idx, out, 576 ** -0.5)


def test_empty_batch_is_a_no_op():
    announce("empty")
    q = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    kk = torch.empty((5, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((0, 8), dtype=torch.bfloat16, device=DEV)
    idx, _ = dsa.indexer_topk(q, kk, w, 4, dsa.Seqs.prefill(0, n_k=5))
    assert idx.shape == (0, 4)


@pytest.mark.parametrize("n_h", [16, 32, 64, 128])
def test_attention_random_indices(n_h):
    """Index rows with -1 padding, duplicates and out-of-range entries (skipped, never read)."""
    announce("attention n_h=%d" % n_h)
    L, k = 400, 100
    li = layer(L, 8, 64, n_h, wid=1)
    g = np.random.default_rng(n_h)
    idx = np.full((L, k), -1, np.int32)
    for t in range(L):
        m = g.integers(0, k + 1)
        idx[t, :m] = g.integers(-2, t + 3, size=m)     # includes -2, t+1, t+2: not visible
    idx_t = torch.from_numpy(idx).to(DEV)
    seqs = dsa.Seqs.prefill(L)
    out = dsa.sparse_attn(li.q, li.latent, idx_t, seqs)
    torch.cuda.synchronize()
    check_attention(OracleView(li), seqs, range(0, L, 7), idx_t, out, 576 ** -0.5)
    out_bf = dsa.sparse_attn(li.q, li.latent, idx_t, seqs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = out.to(torch.bfloat16)
    assert (out_bf.float() - ref.float()).abs().max().item() <= 2 ** -7 * max(1.0, out.abs().max().item())


@pytest.mark.parametrize("n_h", [32, 64, 128])
def test_attention_many_rows_every_pair_kernel(n_h):
    """At 512 rows or more each row is one workgroup with every head (32 heads per wave pair,
    the softmax split between the pair and PV one block behind QK): 2, 4 and 8 waves.
    601 rows leave a ragged last group of the 8-row grid order; rows mix full, partly
    padded (-1, out of range, invisible) and empty index lists over 7 blocks of 32."""
    announce("attention 601 rows n_h=%d" % n_h)
    L, k = 601, 200
    li = layer(L, 8, 64, n_h, wid=1, layer_id=4)
    g = np.random.default_rng(100 + n_h)
    idx = np.full((L, k), -1, np.int32)
    for t in range(L):
        kind = t % 3
        if kind == 0:
            m = min(k, t + 1)
            idx[t, :m] = np.sort(g.choice(t + 1, size=m, replace=False))
        elif kind == 1:
            m = int(g.integers(0, k + 1))
            idx[t, :m] = g.integers(-2, t + 3, size=m)
    idx_t = torch.from_numpy(idx).to(DEV)
    seqs = dsa.Seqs.prefill(L)
    out = dsa.sparse_attn(li.q, li.latent, idx_t, seqs)
    torch.cuda.synchronize()
    rows = sorted(set(range(0, L, 11)) | {1, 2, 598, 599, 600})
    check_attention(OracleView(li), seqs, rows, idx_t, out, 576 ** -0.5)
    print("checked %d rows" % len(rows), flush=True)


# --------------------------------------------------------------------------- decode (varlen, split attention)

@pytest.mark.parametrize("dtype,integer", [("bf16", True), ("bf16", False), ("fp8", False)])
def test_packed_varlen_prefill(dtype, integer):
    """Three ragged sequences in one prefill call (the fused path with per-sequence row
    groups): a fresh prompt, a chunk continuing at position 500 and a short prompt.  Each
    sequence's rows equal the same sequence called alone bit for bit, and match the oracle
    (exactly on integer inputs)."""
    announce("packed varlen prefill %s%s" % (dtype, " integer" if integer else ""))
    q_lens, q_pos0 = [700, 1300, 333], [0, 500, 0]
    k_lens = [p + n for p, n in zip(q_pos0, q_lens)]
    H, d, k = (16, 64, 97) if integer else (64, 128, 256)
    li = synth.make_layer(sum(q_lens), sum(k_lens), H, d, 16, wid=15, layer=0, qk_dtype=dtype,
                          integer_indexer=integer).to(DEV)
    seqs = dsa.Seqs.varlen(q_lens, k_lens, q_pos0)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, q_scale=li.q_scale, k_scale=li.k_scale,
                               want_scores=True)
    torch.cuda.synchronize()
    qa = ka = 0
    for nq, nk, p0 in zip(q_lens, k_lens, q_pos0):
        qs = li.q_scale[qa:qa + nq] if li.q_scale is not None else None
        ks = li.k_scale[ka:ka + nk] if li.k_scale is not None else None
        one, one_sc = dsa.indexer_topk(li.q_idx[qa:qa + nq], li.k_idx[ka:ka + nk], li.w[qa:qa + nq], k,
                                       dsa.Seqs.prefill(nq, nk, q_pos0=p0), q_scale=qs, k_scale=ks, want_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(one, idx[qa:qa + nq]) and torch.equal(one_sc, sc[qa:qa + nq])
        qa, ka = qa + nq, ka + nk
    rows = sorted({0, 1, 7, 8, 96, 699, 700, 701, 1000, 1999, 2000, 2001, 2332} |
                  set(np.random.default_rng(4).integers(0, sum(q_lens), 40).tolist()))
    st = check_indexer(OracleView(li), seqs, rows, k, idx, sc, exact=integer)
    print(st, flush=True)


def test_row_order_past_the_bitmap_range():
    """Rows whose selected positions reach past 2^18 are put in order by the bitonic fallback
    instead of the bitmap rank (a 512-row chunk at positions 400000..; checked against the
    oracle, scores following their positions)."""
    announce("row order past position 2^18")
    n_q, p0, k = 512, 400000, 64
    li = synth.make_layer(n_q, p0 + n_q, 16, 128, 16, wid=16, layer=0, with_attention=False).to(DEV)
    seqs = dsa.Seqs.prefill(n_q, p0 + n_q, q_pos0=p0)
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    torch.cuda.synchronize()
    rows = [0, 200, 511]
    st = check_indexer(OracleView(li), seqs, rows, k, idx, sc, exact=False)
    print(st, flush=True)


def test_decode_varlen():
    announce("decode varlen")
    lens = [3000, 5000, 4097, 1]
    li = synth.make_layer(len(lens), sum(lens), 64, 128, 128, wid=3, layer=7).to(DEV)
    seqs = dsa.Seqs.decode(lens)
    k = 2048
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    out = dsa.sparse_attn(li.q, li.latent, idx, seqs)
    torch.cuda.synchronize()
    view = OracleView(li)
    check_indexer(view, seqs, range(len(lens)), k, idx, sc, exact=False)
    check_attention(view, seqs, range(len(lens)), idx, out, 576 ** -0.5)


@pytest.mark.parametrize("lens,n_h,k", [([5000], 128, 2048), ([5000], 32, 2048), ([3001, 700], 128, 2048),
                                        ([3001, 700], 64, 512), ([40], 128, 2048), ([5000], 128, 100),
                                        ([3001, 700], 32, 1000)])
def test_decode_attention_few_rows(lens, n_h, k):
    """One or two decode rows: the index list is cut into at most 8 splits of whole blocks
    (a lone 2048-entry row: 8 splits of 8 blocks over 4 head groups), merged by the combine;
    a 40-key row leaves most of its 2048 slots -1; k = 100 and 1000 end in a partly filled
    block that falls in the last split.  Every row against the oracle."""
    announce("decode attention lens=%s n_h=%d k=%d" % (lens, n_h, k))
    g = np.random.default_rng(sum(lens) + n_h + k)
    li = synth.make_layer(len(lens), sum(lens), 64, 128, n_h, wid=5, layer=2).to(DEV)
    idx = np.full((len(lens), k), -1, np.int32)
    for b, n in enumerate(lens):
        m = min(k, n)
        idx[b, :m] = np.sort(g.choice(n, size=m, replace=False))
    idx_t = torch.from_numpy(idx).to(DEV)
    seqs = dsa.Seqs.decode(lens)
    out = dsa.sparse_attn(li.q, li.latent, idx_t, seqs)
    torch.cuda.synchronize()
    worst = check_attention(OracleView(li), seqs, range(len(lens)), idx_t, out, 576 ** -0.5)
    print("attention error %.2e" % worst, flush=True)


def test_decode_at_the_sequence_limit():
    """64 sequences (the table's maximum) in one decode call: lengths from 1 to 40000 (the
    longest take the chunked wide select), k = 2048; selection and attention against the
    oracle on a sample of rows, every row valid."""
    announce("decode B=64")
    g = np.random.default_rng(64)
    lens = g.integers(1, 12000, size=64)
    lens[[5, 17, 40]] = [40000, 36000, 33000]
    lens[9] = 1
    li = synth.make_layer(64, int(lens.sum()), 64, 128, 128, wid=17, layer=0).to(DEV)
    seqs = dsa.Seqs.decode(lens)
    k = 2048
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    out = dsa.sparse_attn(li.q, li.latent, idx, seqs)
    torch.cuda.synchronize()
    view = OracleView(li)
    rows = [0, 5, 9, 17, 33, 40, 63]
    st = check_indexer(view, seqs, rows, k, idx, sc, exact=False)
    ig = idx.cpu().numpy()
    for i in range(64):
        check_valid_row(ig[i], int(lens[i]) - 1, k)
    worst = check_attention(view, seqs, rows, idx, out, 576 ** -0.5)
    print(st, "attention error %.2e" % worst, flush=True)


def test_decode_wide_select_bf16():
    """Few long rows: the (chunk, row) multi-workgroup select; one row shorter than k."""
    announce("decode wide select bf16")
    lens = [40000, 65537, 1000, 33000]
    li = synth.make_layer(len(lens), sum(lens), 64, 128, 16, wid=3, layer=11, with_attention=False).to(DEV)
    seqs = dsa.Seqs.decode(lens)
    k = 2048
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    torch.cuda.synchronize()
    print(check_indexer(OracleView(li), seqs, range(len(lens)), k, idx, sc, exact=False))


def test_decode_wide_select_integer_exact():
    """Integer-valued inputs (many equal scores): sets and scores bit-exact, ties to lower positions."""
    announce("decode wide select integer")
    lens = [50000, 36000, 2047]
    li = synth.make_layer(len(lens), sum(lens), 8, 64, 16, wid=0, layer=5, integer_indexer=True,
                          with_attention=False).to(DEV)
    seqs = dsa.Seqs.decode(lens)
    k = 2048
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    torch.cuda.synchronize()
    check_indexer(OracleView(li), seqs, range(len(lens)), k, idx, sc, exact=True)


def test_decode_wide_select_all_ties():
    """Every score +-0: the threshold bin overflows the candidate list; the lowest positions win."""
    announce("decode wide select all ties")
    lens = [40000, 70001]
    li = synth.make_layer(len(lens), sum(lens), 64, 128, 16, wid=3, layer=12, with_attention=False).to(DEV)
    li.q_idx.zero_()
    seqs = dsa.Seqs.decode(lens)
    k = 2048
    idx, sc = dsa.indexer_topk(li.q_idx, li.k_idx, li.w, k, seqs, want_scores=True)
    torch.cuda.synchronize()
    want = torch.arange(k, dtype=torch.int32, device=DEV).expand(len(lens), k)
    assert torch.equal(idx, want)
    assert torch.all(sc == 0)


# --------------------------------------------------------------------------- IndexCache loop

def _stack(roles, L, k, wid=2, chunk=None, n_h=16):
    layers = [synth.make_layer(L, L, 64, 128, n_h, wid=wid, layer=l).to(DEV) for l in range(len(roles))]
    res = dsa.indexcache_forward(roles, [dsa.layer_dict(x) for x in layers], k, q_chunk=chunk)
    torch.cuda.synchronize()
    return layers, res


def test_indexcache_fsss_against_oracle():
    announce("FSSSFSSS")
    L, k = 600, 64
    layers, res = _stack("FSSSFSSS", L, k)
    assert res.n_indexer_calls == 2 and res.src_layer == [0, 0, 0, 0, 4, 4, 4, 4]
    rows = sample_rows(L, k, 24)
    seqs = dsa.Seqs.prefill(L)
    # the cache after the loop holds layer 5's selection (the last F layer)
    check_indexer(OracleView(layers[4]), seqs, rows, k, res.index_cache, None, exact=False)
    # every layer attends with its own q/latent over its F layer's rows
    idx_f = {}
    for f in (0, 4):
        idx_f[f], _ = dsa.indexer_topk(layers[f].q_idx, layers[f].k_idx, layers[f].w, k, seqs)
    torch.cuda.synchronize()
    assert torch.equal(idx_f[4], res.index_cache)
    for l in range(8):
        src = res.src_layer[l]
        check_attention(OracleView(layers[l]), seqs, rows, idx_f[src], res.outs[l], 576 ** -0.5)
        if l not in (0, 4):
            own = dsa.sparse_attn(layers[l].q, layers[l].latent, idx_f[src], seqs)
            torch.cuda.synchronize()
            assert torch.equal(own, res.outs[l])


def test_all_f_runs_every_indexer_and_chunking_is_invisible():
    announce("FFFF / chunks")
    L, k = 700, 100
    layers, a = _stack("FFFF", L, k)
    assert a.n_indexer_calls == 4
    _, b = _stack("FFFF", L, k, chunk=256)
    assert b.n_chunks == 3
    assert torch.equal(a.index_cache, b.index_cache)
    # 256-row chunks take the split-combine attention path: P is rounded to bf16 against a
    # different running max there, so the two agree to bf16 resolution (both are checked
    # against the oracle elsewhere)
    for l in range(4):
        assert torch.allclose(a.outs[l], b.outs[l], rtol=0, atol=5e-3)
    # ring-buffered outputs hold the last chunk
    res = dsa.indexcache_forward("FS", [dsa.layer_dict(x) for x in layers[:2]], k, q_chunk=256, out_rows=256,
                                 index_rows=256)
    torch.cuda.synchronize()
    last = slice(512, 700)
    full = dsa.indexcache_forward("FS", [dsa.layer_dict(x) for x in layers[:2]], k)
    torch.cuda.synchronize()
    assert torch.allclose(res.outs[1][: 700 - 512], full.outs[1][last], rtol=0, atol=5e-3)
    assert torch.equal(res.index_cache[: 700 - 512], full.index_cache[last])


def test_attention_large_budget_fallback():
    """k above the paired kernel's LDS index capacity takes the 16-heads-per-wave kernel."""
    announce("attention k=2100")
    L, k = 2300, 2100
    li = layer(L, 8, 64, 32, wid=1, layer_id=5)
    g = np.random.default_rng(5)
    idx = np.full((L, k), -1, np.int32)
    for t in range(L):
        m = min(k, t + 1)
        idx[t, :m] = np.sort(g.choice(t + 1, size=m, replace=False))
    idx_t = torch.from_numpy(idx).to(DEV)
    seqs = dsa.Seqs.prefill(L)
    out = dsa.sparse_attn(li.q, li.latent, idx_t, seqs)
    torch.cuda.synchronize()
    check_attention(OracleView(li), seqs, [0, 5, 2047, 2048, 2099, 2100, 2299], idx_t, out, 576 ** -0.5)


# --------------------------------------------------------------------------- diagnostics

def _overlap_rows(n, k, seed):
    """Index rows with every overlap from none to all, shuffled order and -1 padding."""
    g = np.random.default_rng(seed)
    a = np.full((n, k), -1, dtype=np.int32)
    b = np.full((n, k), -1, dtype=np.int32)
    for i in range(n):
        va = int(g.integers(0, k + 1))
        vb = int(g.integers(0, k + 1))
        pool = g.permutation(4 * k + 7)
        common = int(g.integers(0, min(va, vb) + 1))
        sa = pool[:va]
        sb = np.concatenate([sa[:common], pool[va:va + vb - common]])
        a[i, :va] = g.permutation(sa)
        b[i, :vb] = g.permutation(sb)
        a[i] = g.permutation(a[i])
        b[i] = g.permutation(b[i])
    return a, b


@pytest.mark.parametrize("n,k", [(700, 2048), (300, 7), (40, 16384)])
def test_index_overlap_exact(n, k):
    announce("index overlap n=%d k=%d" % (n, k))
    a, b = _overlap_rows(n, k, seed=k)
    got = dsa.index_overlap(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    want = np.array([round(oracle.overlap(a[i], b[i], k) * k) for i in range(n)], dtype=np.int32)
    assert np.array_equal(got.cpu().numpy(), want)


def test_index_overlap_bitmap_and_hash_rows():
    """Rows whose valid entries of B span fewer than 2^18 positions take the bitmap, wider
    rows the hash table: both in one call, at the span boundary (2^18 - 1 and 2^18), near
    INT32_MAX, and with B empty or a single entry."""
    announce("index overlap bitmap and hash rows")
    n, k = 60, 2048
    g = np.random.default_rng(77)
    a = np.full((n, k), -1, dtype=np.int32)
    b = np.full((n, k), -1, dtype=np.int32)
    for i in range(n):
        mode = i % 5
        base = 2 ** 31 - 1_000_000 if mode == 3 else 1000
        span = {0: 4 * k + 7, 1: 2 ** 18, 2: 2 ** 18 + 1, 3: 1_000_000, 4: 4 * k}[mode]
        pool = base + g.choice(span, size=4 * k, replace=False)
        if mode in (1, 2):   # B holds both ends: hi - lo = span - 1
            pool = np.concatenate([[base, base + span - 1], pool[(pool != base) & (pool != base + span - 1)]])
        va = int(g.integers(0, k + 1))
        vb = int(g.integers(0, 2)) if mode == 4 else int(g.integers(2, k + 1))
        common = int(g.integers(0, min(va, vb) + 1))
        sb = pool[:vb]
        sa = np.concatenate([sb[:common], pool[vb:vb + va - common]])
        a[i, :va] = g.permutation(sa)
        b[i, :vb] = sb if mode in (1, 2) else g.permutation(sb)
        a[i] = g.permutation(a[i])
        b[i] = g.permutation(b[i])
    got = dsa.index_overlap(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    want = np.array([round(oracle.overlap(a[i], b[i], k) * k) for i in range(n)], dtype=np.int32)
    assert np.array_equal(got.cpu().numpy(), want)


def test_index_overlap_between_two_f_layers():
    """Cross-layer overlap of two F layers' own selections (FF stack), against the oracle."""
    announce("index overlap of two F layers")
    L, k = 1500, 128
    layers = [synth.make_layer(L, L, 64, 128, 16, wid=2, layer=l).to(DEV) for l in range(2)]
    seqs = dsa.Seqs.prefill(L)
    i0, _ = dsa.indexer_topk(layers[0].q_idx, layers[0].k_idx, layers[0].w, k, seqs)
    i1, _ = dsa.indexer_topk(layers[1].q_idx, layers[1].k_idx, layers[1].w, k, seqs)
    got = dsa.index_overlap(i0, i1)
    torch.cuda.synchronize()
    a, b = i0.cpu().numpy(), i1.cpu().numpy()
    want = np.array([round(oracle.overlap(a[i], b[i], k) * k) for i in range(L)], dtype=np.int32)
    assert np.array_equal(got.cpu().numpy(), want)
    assert got[:k].eq(torch.arange(1, k + 1, device=DEV, dtype=torch.int32)).all()   # t < k: all rows visible


# --------------------------------------------------------------------------- device fp8 quantisation

def _quant_rows(rows, cols, seed):
    """bf16 rows of mixed magnitude; row 0 is all zero, row 1 holds exact e4m3 ties at
    scale 1 (normal and subnormal midpoints, both signs, a negative that rounds to zero),
    row 2 is tiny (codes in the subnormal range), row 3 has a single non-zero entry."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32) * (2.0 ** g.integers(-12, 12, (rows, 1)))
    x[0] = 0.0
    ties = np.array([448.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -(2.0 ** -10), 0.0, -0.0,
                     240.0 + 8.0, 13.0, -416.0 - 16.0], dtype=np.float32)
    x[1] = np.resize(ties, cols)
    x[1, 0] = 448.0
    x[2] *= 2.0 ** -20
    x[3] = 0.0
    x[3, cols // 2] = -3.5
    xb = torch.from_numpy(x).to(torch.bfloat16)
    return xb, xb.to(torch.float32).numpy()


@pytest.mark.parametrize("rows,cols", [(1001, 128), (37, 100), (9, 577), (4, 1), (33, 1024), (17, 24), (9, 40)])
def test_quantize_fp8_rows_bit_exact(rows, cols):
    announce("fp8 quantisation rows=%d cols=%d" % (rows, cols))
    xb, xf = _quant_rows(rows, cols, seed=rows + cols)
    codes, scales = dsa.quantize_fp8_rows(xb.to(DEV))
    torch.cuda.synchronize()
    want_codes, want_scales = oracle.quantize_fp8_rows(xf)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), want_scales.view(np.uint32))
    np.testing.assert_array_equal(codes.view(torch.uint8).cpu().numpy(), want_codes)


def test_quantize_fp8_rows_misaligned_view():
    """A bf16 view one element past an aligned base (rows of a multiple of 8 elements):
    the 16-byte vector path does not apply, the per-element path must give the same codes."""
    announce("fp8 quantisation misaligned view")
    rows, cols = 21, 128
    xb, xf = _quant_rows(rows, cols, seed=77)
    buf = torch.empty(rows * cols + 1, dtype=torch.bfloat16, device=DEV)
    buf[1:] = xb.reshape(-1).to(DEV)
    x = buf[1:].view(rows, cols)
    assert x.data_ptr() % 16 != 0
    codes, scales = dsa.quantize_fp8_rows(x)
    torch.cuda.synchronize()
    want_codes, want_scales = oracle.quantize_fp8_rows(xf)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), want_scales.view(np.uint32))
    np.testing.assert_array_equal(codes.view(torch.uint8).cpu().numpy(), want_codes)


def test_quantize_fp8_rows_feeds_the_indexer():
    """The fp8 indexer path end to end from bf16 inputs: q_idx / k_idx quantised on the
    device (codes and scales equal to the oracle's quantisation of the same bf16
    values), then indexer + top-k checked against the oracle on those inputs."""
    announce("fp8 quantisation -> indexer")
    L, H, d, k = 1500, 16, 128, 256
    li = layer(L, H, d, 16)
    seqs = dsa.Seqs.prefill(L)
    qc, qs = dsa.quantize_fp8_rows(li.q_idx.contiguous())
    kc, ks = dsa.quantize_fp8_rows(li.k_idx.contiguous())
    torch.cuda.synchronize()
    for codes, scales, src in ((qc, qs, li.q_idx), (kc, ks, li.k_idx)):
        want_c, want_s = oracle.quantize_fp8_rows(src.float().cpu().numpy())
        np.testing.assert_array_equal(codes.view(torch.uint8).cpu().numpy(), want_c)
        np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    idx, sc = dsa.indexer_topk(qc, kc, li.w, k, seqs, q_scale=qs, k_scale=ks, want_scores=True)
    torch.cuda.synchronize()
    q8 = synth.LayerInputs(qc, qs, kc, ks, li.w, li.q, li.latent)
    check_indexer(OracleView(q8), seqs, sample_rows(L, k, 200, seed=11), k, idx, sc, exact=False)
