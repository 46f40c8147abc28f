"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-only logic (role planning, argument validation, workspace queries) behaves as
include/dsa.h states.  No compute entry point reaches a kernel here: every call
below is rejected by validation before any launch, or is host-only."""
import ctypes
import os
import random
import re

import pytest

import oracle
import dsa_indexer_indexcache_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="HIP library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(dsa.EXPORTS), names
    L = dsa.lib()
    for n in names:
        assert hasattr(L, n)
    assert L.dsa_version() == 101


def test_status_strings():
    L = dsa.lib()
    for code in dsa.STATUS:
        assert L.dsa_status_string(code)
    assert L.dsa_status_string(-99) == b"unknown status"


def test_plan_matches_oracle_on_random_roles():
    rnd = random.Random(0)
    for _ in range(500):
        n = rnd.randint(1, 60)
        roles = "F" + "".join(rnd.choice("FS") for _ in range(n - 1))
        assert dsa.indexcache_plan(roles) == oracle.indexcache_plan(roles)
    assert dsa.indexcache_plan("FSSSFSSS") == ([0, 0, 0, 0, 4, 4, 4, 4], 2)
    assert dsa.indexcache_plan("FSSS" * 11 + "FSS")[1] == 12


@pytest.mark.parametrize("roles,code", [("", -2), ("FX", -2), ("fS", -2), ("SFFF", -3), ("S", -3)])
def test_plan_rejects(roles, code):
    with pytest.raises(dsa.DsaError) as e:
        dsa.indexcache_plan(roles)
    assert e.value.status == code
    with pytest.raises(oracle.RoleError):
        oracle.indexcache_plan(roles)


FAKE = 1 << 40   # never dereferenced: every call below fails validation first


def _topk(**kw):
    a = dict(q_idx=FAKE, q_scale=None, k_idx=FAKE, k_scale=None, w=FAKE, dt=0, H=64, d=128, k=2048,
             seqs=dsa.Seqs.prefill(100), idx=FAKE, sc=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return dsa.lib().dsa_indexer_topk(a["q_idx"], a["q_scale"], a["k_idx"], a["k_scale"], a["w"], a["dt"], a["H"],
                                      a["d"], a["k"], ctypes.byref(a["seqs"]), a["idx"], a["sc"], a["ws"], a["wsb"],
                                      None)


def test_indexer_validation():
    assert _topk(k=0) == -1
    assert _topk(H=65) == -4
    assert _topk(d=96) == -4
    assert _topk(dt=1, d=64, q_scale=FAKE, k_scale=FAKE) == -4       # fp8 needs d=128
    assert _topk(dt=1) == -1                                        # fp8 without scales
    assert _topk(q_scale=FAKE) == -1                                # bf16 with scales
    assert _topk(q_idx=FAKE + 8) == -5
    assert _topk(idx=None) == -1
    assert _topk(wsb=16) == -6
    bad = dsa.Seqs.prefill(100, n_k=50)                              # positions beyond the keys
    assert _topk(seqs=bad) == -1
    s = dsa.Seqs.prefill(4)
    s.B = 0
    assert _topk(seqs=s) == -1
    assert dsa.lib().dsa_last_error()


def _attn(**kw):
    a = dict(q=FAKE, lat=FAKE, idx=FAKE, n_h=128, dqk=576, dv=512, k=2048, scale=0.04,
             seqs=dsa.Seqs.prefill(100), out=FAKE, odt=2, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return dsa.lib().dsa_sparse_attn(a["q"], a["lat"], a["idx"], a["n_h"], a["dqk"], a["dv"], a["k"], a["scale"],
                                     ctypes.byref(a["seqs"]), a["out"], a["odt"], a["ws"], a["wsb"], None)


def test_attention_validation():
    assert _attn(n_h=48) == -4
    assert _attn(dqk=512) == -4
    assert _attn(dv=600) == -1
    assert _attn(k=0) == -1
    assert _attn(odt=1) == -4
    assert _attn(q=None) == -1
    assert _attn(out=FAKE + 4) == -5
    dec = dsa.Seqs.decode([100, 200])
    need = dsa.lib().dsa_sparse_attn_ws(128, 576, 512, 2048, ctypes.byref(dec))
    assert need > 0                                                # few rows -> split partials
    assert _attn(seqs=dec, wsb=need - 1) == -6


def test_workspace_queries():
    L = dsa.lib()
    s = dsa.Seqs.prefill(1000)
    # one-sequence prefill with >= 256 rows takes the fused indexer: no workspace
    assert L.dsa_indexer_topk_ws(0, 64, 128, 2048, ctypes.byref(s)) == 0
    assert L.dsa_indexer_topk_ws(1, 64, 128, 2048, ctypes.byref(s)) == 0
    # decode (many sequences) and short prefill keep a score slab
    dec = dsa.Seqs.decode([1000, 3000])
    assert L.dsa_indexer_topk_ws(0, 64, 128, 2048, ctypes.byref(dec)) >= 2 * 3000 * 4
    short = dsa.Seqs.prefill(100)
    assert L.dsa_indexer_topk_ws(0, 64, 128, 2048, ctypes.byref(short)) >= 100 * 100 * 4
    # k above the fused kernel's 2048-slot state falls back to the slab
    assert L.dsa_indexer_topk_ws(0, 64, 128, 4096, ctypes.byref(s)) >= 1000 * 1000 * 4
    assert L.dsa_sparse_attn_ws(128, 576, 512, 2048, ctypes.byref(s)) == 0
    sh = dsa.Shape(H=64, d=128, k=2048, n_h=128, d_qk=576, d_v=512, scale=0.04, qk_dtype=0, out_dtype=2,
                   q_chunk=256, index_rows=1000, out_rows=256)
    assert L.indexcache_forward_ws(b"FSSS", ctypes.byref(sh), ctypes.byref(s)) > 0   # 256-row chunks split attention


def test_decode_attention_split_plan_every_head_count():
    """The few-row plan (head groups x index-list splits) for every supported head count and
    batch: the workspace holds a whole number of fp32 split partials (O, max, sum per head)."""
    L = dsa.lib()
    for n_h in (16, 32, 64, 128):
        for B in (1, 3, 8, 64):
            dec = dsa.Seqs.decode([5000 + 17 * b for b in range(B)])
            need = L.dsa_sparse_attn_ws(n_h, 576, 512, 2048, ctypes.byref(dec))
            per_split = B * n_h * (512 + 2) * 4
            if need == 0:
                continue
            assert (need - 256) % per_split == 0, (n_h, B, need)
            assert 1 <= (need - 256) // per_split <= 8, (n_h, B, need)  # the combine takes 8 at once


def test_forward_validation():
    L = dsa.lib()
    s = dsa.Seqs.prefill(64)
    sh = dsa.Shape(H=64, d=128, k=16, n_h=16, d_qk=576, d_v=512, scale=0.04, qk_dtype=0, out_dtype=2,
                   q_chunk=32, index_rows=64, out_rows=64)
    layers = (dsa.Layer * 2)()
    for l in layers:
        l.q_idx = l.k_idx = l.w = l.q = l.latent = l.out = FAKE
    st = dsa.Stats()
    call = lambda roles, shape=sh, ic=FAKE: L.indexcache_forward(roles, layers, ctypes.byref(shape), ctypes.byref(s),
                                                                 ic, None, FAKE, 0, ctypes.byref(st), None)
    assert call(b"SF") == -3
    assert call(b"FQ") == -2
    assert call(b"FS", ic=None) == -1
    bad = dsa.Shape(**{f: getattr(sh, f) for f, _ in dsa.Shape._fields_})
    bad.out_rows = 48                                              # neither >= n_q nor a multiple of q_chunk
    assert call(b"FS", shape=bad) == -1
    bad.out_rows, bad.n_h = 64, 20
    assert call(b"FS", shape=bad) == -4
    assert call(b"FS") == -6                                       # workspace 0 bytes


def test_index_overlap_validation():
    """Argument checks of dsa_index_overlap run before any launch (no GPU needed)."""
    L = dsa.lib()
    assert L.dsa_index_overlap(None, None, 0, 2048, None, None) == 0          # no rows: a no-op
    assert L.dsa_index_overlap(None, None, 4, 0, None, None) == -4            # k < 1
    assert L.dsa_index_overlap(None, None, 4, 16385, None, None) == -4        # k too large
    assert L.dsa_index_overlap(None, None, -1, 16, None, None) == -1          # negative row count
    assert L.dsa_index_overlap(None, None, 4, 16, None, None) == -1           # null pointers
    assert L.dsa_index_overlap(None, None, 2 ** 31, 16, None, None) == -4     # rows beyond int32


def test_quantize_fp8_rows_validation():
    L = dsa.lib()
    assert L.dsa_quantize_fp8_rows(None, 0, 128, None, None, None) == 0      # no rows: a no-op
    assert L.dsa_quantize_fp8_rows(None, 4, 0, None, None, None) == -4       # cols < 1
    assert L.dsa_quantize_fp8_rows(None, 4, 65537, None, None, None) == -4   # cols too large
    assert L.dsa_quantize_fp8_rows(None, 4, 128, None, None, None) == -1     # null pointers
    assert L.dsa_quantize_fp8_rows(None, 2 ** 31, 128, None, None, None) == -4  # too many rows


def test_binding_rejects_bad_tensors_before_the_library():
    """The Python binding checks dtype, shape, contiguity and device of every tensor it
    turns into a raw pointer (an int64 index tensor, as torch.topk returns, would otherwise
    be read as int32; a short counts tensor would be written out of bounds)."""
    import torch
    cpu32 = torch.zeros((4, 16), dtype=torch.int32)
    with pytest.raises(ValueError, match="int32"):
        dsa.index_overlap(cpu32.to(torch.int64), cpu32)
    with pytest.raises(ValueError, match="GPU"):
        dsa.index_overlap(cpu32, cpu32)
    with pytest.raises(ValueError, match="shape"):
        dsa.index_overlap(torch.zeros((4, 16, 1), dtype=torch.int32), cpu32)
    with pytest.raises(ValueError, match="int32"):
        dsa.sparse_attn(torch.zeros((4, 16, 576), dtype=torch.bfloat16),
                        torch.zeros((8, 576), dtype=torch.bfloat16), cpu32.to(torch.int64))
    with pytest.raises(ValueError, match="GPU"):
        dsa.sparse_attn(torch.zeros((4, 16, 576), dtype=torch.bfloat16),
                        torch.zeros((8, 576), dtype=torch.bfloat16), cpu32)
    with pytest.raises(ValueError, match="contiguous"):
        dsa.sparse_attn(torch.zeros((16, 4, 576), dtype=torch.bfloat16).transpose(0, 1),
                        torch.zeros((8, 576), dtype=torch.bfloat16), cpu32)
    q = torch.zeros((4, 8, 64), dtype=torch.bfloat16)
    kk = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="w must"):
        dsa.indexer_topk(q, kk, torch.zeros((4, 8), dtype=torch.float32), 2)
    with pytest.raises(ValueError, match="k_idx must"):
        dsa.indexer_topk(q, kk.to(torch.float32), torch.zeros((4, 8), dtype=torch.bfloat16), 2)
    with pytest.raises(ValueError, match="x must"):
        dsa.quantize_fp8_rows(torch.zeros((4, 8), dtype=torch.float32))


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """indexcache_forward_noalloc refuses a call whose workspace exceeds its fixed
    per-GPU array, before any launch: 64 decode rows over 400K keys need a 102 MB slab."""
    L = dsa.lib()
    seqs = dsa.Seqs.decode([400000] * 64)
    shape = dsa.Shape()
    shape.H, shape.d, shape.k, shape.n_h, shape.d_qk, shape.d_v = 64, 128, 2048, 128, 576, 512
    shape.scale, shape.qk_dtype, shape.out_dtype = 576 ** -0.5, dsa.DSA_BF16, dsa.DSA_FP32
    shape.q_chunk, shape.index_rows, shape.out_rows = 64, 64, 64
    need = L.indexcache_forward_ws(b"F", ctypes.byref(shape), ctypes.byref(seqs))
    assert need > dsa.NOALLOC_SCRATCH_BYTES
    layers = (dsa.Layer * 1)()
    rc = L.indexcache_forward_noalloc(b"F", layers, ctypes.byref(shape), ctypes.byref(seqs), None, None, None, None)
    assert rc == -6
    assert b"scratch" in L.dsa_last_error()
    assert L.indexcache_forward_noalloc(b"SF", layers, ctypes.byref(shape), ctypes.byref(seqs), None, None, None,
                                        None) == -3


def test_indexer_project_validation():
    """Argument checks of dsa_indexer_project run before any launch."""
    L = dsa.lib()
    z = [None] * 8
    ok = dict(n=4, r=128, hidden=256, H=64, d=128, rope=64)

    def call(n=4, r=128, hidden=256, H=64, d=128, rope=64, base=10000.0, eps=1e-5):
        return L.dsa_indexer_project(*z, n, r, hidden, H, d, rope, base, eps, None, None, None, None)
    assert call(n=0) == 0                        # no tokens: a no-op
    assert call(n=-1) == -1
    assert call(d=64) == -4                      # only d = 128 is compiled
    assert call(H=0) == -4 and call(H=129) == -4
    assert call(rope=48) == -4
    assert call(r=100) == -4 and call(hidden=32) == -4
    assert call(base=1.0) == -1 and call(eps=-1.0) == -1
    assert call() == -1                          # null pointers
    assert ok


def test_cache_append_validation():
    L = dsa.lib()
    assert L.dsa_cache_append(None, 10, None, None, 0, 16, None) == 0      # no rows: a no-op
    assert L.dsa_cache_append(None, 10, None, None, -1, 16, None) == -1
    assert L.dsa_cache_append(None, 10, None, None, 2, 0, None) == -1
    assert L.dsa_cache_append(None, 10, None, None, 2, 16, None) == -1     # null pointers
    assert L.dsa_cache_append(None, 10, None, None, 2 ** 31, 16, None) == -4


def test_compressed_block_table_validation():
    """seqs->block: a negative ratio is rejected; with block m the last query t needs t // m keys."""
    ok = dsa.Seqs.compressed(100, 4)                                 # t = 99 needs 24 blocks, has 25
    assert ok.block == 4 and ok.n_k == 25
    short = dsa.Seqs.compressed(100, 4, n_k=23)                      # t = 99 needs 24
    assert _topk(seqs=short) == -1
    assert b"needs 24 keys" in dsa.lib().dsa_last_error()
    neg = dsa.Seqs.compressed(100, 4)
    neg.block = -2
    assert _topk(seqs=neg) == -1


def test_topk_ex_rejects_unknown_flags():
    L = dsa.lib()
    s = dsa.Seqs.prefill(100)
    rc = L.dsa_indexer_topk_ex(FAKE, None, FAKE, None, FAKE, 0, 64, 128, 2048, ctypes.byref(s), FAKE, None, FAKE,
                               1 << 40, 6, None)
    assert rc == -1 and b"flags" in L.dsa_last_error()


def test_csa_compress_validation():
    L = dsa.lib()
    f = lambda **kw: L.dsa_csa_compress(*[kw.get(n, FAKE) for n in ("ca", "cb", "za", "zb", "ba", "bb")],
                                        kw.get("n", 64), kw.get("c", 128), kw.get("m", 4), kw.get("b0", 0),
                                        kw.get("out", FAKE), kw.get("odt", 0), None)
    assert f(m=0) == -4 and f(m=5000) == -4
    assert f(c=100) == -4 and f(c=0) == -4
    assert f(n=-1) == -1 and f(b0=-1) == -1
    assert f(odt=1) == -1                                            # fp8 output is not offered
    assert f(n=3, ca=None) == 0                                      # fewer than m tokens: no entry, a no-op
    assert f(n=64, b0=16, ca=None) == 0                              # block0 past the last entry: a no-op
    assert f(ca=None) == -1
    assert f(ca=FAKE + 8) == -5


def test_attention_rejects_sequences_past_the_latent_offset_range():
    """Latent rows are addressed by a 32-bit byte offset per sequence: at most
    (2^32 - 4096) / 1152 rows per sequence."""
    L = dsa.lib()
    lim = (2 ** 32 - 4096) // 1152
    s = dsa.Seqs.decode([lim + 1])
    rc = L.dsa_sparse_attn(FAKE, FAKE, FAKE, 128, 576, 512, 2048, 0.04, ctypes.byref(s), FAKE, 2, FAKE, 1 << 40,
                           None)
    assert rc == -4 and b"latent rows" in L.dsa_last_error()
