"""MI355X (gfx950) DSA hot path: lightning indexer + top-k + sparse MLA attention under IndexCache.

Thin Python binding over the C ABI in include/dsa.h (libdsa_mi355x.so, built
in-tree by build.py).  This module only marshals arguments: torch supplies
device memory and the stream; every step of the path runs in the HIP kernels.
There is no CPU or eager fallback: if the library is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_mi355x.so")

DSA_BF16, DSA_FP8_E4M3, DSA_FP32 = 0, 1, 2
DSA_MAX_B = 64
DSA_MAX_LAYERS = 256
STATUS = {0: "DSA_OK", -1: "DSA_ERR_INVALID_ARG", -2: "DSA_ERR_ROLES", -3: "DSA_ERR_FIRST_NOT_F",
          -4: "DSA_ERR_UNSUPPORTED", -5: "DSA_ERR_ALIGNMENT", -6: "DSA_ERR_WORKSPACE", -7: "DSA_ERR_HIP"}

EXPORTS = ("dsa_indexer_topk", "dsa_indexer_topk_ws", "dsa_sparse_attn", "dsa_sparse_attn_ws",
           "indexcache_forward", "indexcache_forward_ws", "indexcache_plan", "dsa_status_string",
           "dsa_last_error", "dsa_version", "dsa_index_overlap", "dsa_quantize_fp8_rows",
           "indexcache_forward_noalloc", "dsa_indexer_project", "dsa_cache_append", "dsa_attention_mass",
           "dsa_attention_mass_ws", "dsa_indexer_kl", "dsa_indexer_kl_ws", "dsa_indexer_topk_ex",
           "dsa_csa_compress")
DSA_TOPK_BF16_SCORES = 1
NOALLOC_SCRATCH_BYTES = 64 << 20


class DsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, detail))
        self.status = status


class Seqs(ctypes.Structure):
    """dsa_seqs: packed variable-length batch (see include/dsa.h)."""
    _fields_ = [("B", ctypes.c_int32), ("block", ctypes.c_int32),
                ("q_start", ctypes.c_int64 * (DSA_MAX_B + 1)),
                ("k_start", ctypes.c_int64 * (DSA_MAX_B + 1)),
                ("q_pos0", ctypes.c_int64 * DSA_MAX_B)]

    @classmethod
    def varlen(cls, q_lens: Sequence[int], k_lens: Sequence[int], q_pos0: Sequence[int], block: int = 0) -> "Seqs":
        """block > 1: the key rows are compressed blocks of `block` tokens (query t sees blocks s < t // block)."""
        s = cls()
        B = len(q_lens)
        if not (1 <= B <= DSA_MAX_B) or len(k_lens) != B or len(q_pos0) != B:
            raise ValueError("need 1..%d sequences with matching lengths" % DSA_MAX_B)
        s.B = B
        s.block = int(block)
        qa = ka = 0
        for b in range(B):
            s.q_start[b] = qa
            s.k_start[b] = ka
            s.q_pos0[b] = int(q_pos0[b])
            qa += int(q_lens[b])
            ka += int(k_lens[b])
        s.q_start[B] = qa
        s.k_start[B] = ka
        return s

    @classmethod
    def prefill(cls, n_q: int, n_k: Optional[int] = None, q_pos0: int = 0) -> "Seqs":
        """One sequence: n_q queries at positions q_pos0.. over n_k keys (default n_k = q_pos0 + n_q)."""
        return cls.varlen([n_q], [q_pos0 + n_q if n_k is None else n_k], [q_pos0])

    @classmethod
    def compressed(cls, n_q: int, block: int, q_pos0: int = 0, n_k: Optional[int] = None) -> "Seqs":
        """One sequence of n_q query tokens at positions q_pos0.. over compressed blocks of `block` tokens
        (default n_k = (q_pos0 + n_q) // block, the complete blocks of the tokens so far)."""
        return cls.varlen([n_q], [(q_pos0 + n_q) // block if n_k is None else n_k], [q_pos0], block=block)

    @classmethod
    def decode(cls, lens: Iterable[int]) -> "Seqs":
        """B sequences, one new query each at position len_b - 1 (the caches already hold it)."""
        lens = [int(x) for x in lens]
        return cls.varlen([1] * len(lens), lens, [x - 1 for x in lens])

    @property
    def n_q(self) -> int:
        return int(self.q_start[self.B])

    @property
    def n_k(self) -> int:
        return int(self.k_start[self.B])


class Layer(ctypes.Structure):
    _fields_ = [("q_idx", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k_idx", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("w", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("latent", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class Shape(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("d", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n_h", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("scale", ctypes.c_float), ("qk_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("q_chunk", ctypes.c_int64), ("index_rows", ctypes.c_int64),
                ("out_rows", ctypes.c_int64)]


DSA_MAX_TRACE = 1024


class Stats(ctypes.Structure):
    _fields_ = [("events", ctypes.c_void_p), ("event_cap", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_indexer_calls", ctypes.c_int32), ("n_chunks", ctypes.c_int32), ("n_traced", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("src_layer", ctypes.c_int32 * DSA_MAX_LAYERS),
                ("trace_kind", ctypes.c_int8 * DSA_MAX_TRACE), ("trace_layer", ctypes.c_int16 * DSA_MAX_TRACE),
                ("trace_chunk", ctypes.c_int32 * DSA_MAX_TRACE)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("HIP library %s is missing: run `python -m dsa_indexer_indexcache_amd.build` "
                               "(or __graft_entry__.build())" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
        L.dsa_indexer_topk.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.POINTER(Seqs), vp, vp, vp,
                                       sz, vp]
        L.dsa_indexer_topk.restype = i32
        L.dsa_indexer_topk_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.POINTER(Seqs), vp, vp, vp,
                                          sz, i32, vp]
        L.dsa_indexer_topk_ex.restype = i32
        L.dsa_csa_compress.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64, i32, i32, ctypes.c_int64, vp, i32, vp]
        L.dsa_csa_compress.restype = i32
        L.dsa_indexer_topk_ws.argtypes = [i32, i32, i32, i32, ctypes.POINTER(Seqs)]
        L.dsa_indexer_topk_ws.restype = sz
        L.dsa_sparse_attn.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, ctypes.POINTER(Seqs), vp, i32, vp, sz,
                                      vp]
        L.dsa_sparse_attn.restype = i32
        L.dsa_sparse_attn_ws.argtypes = [i32, i32, i32, i32, ctypes.POINTER(Seqs)]
        L.dsa_sparse_attn_ws.restype = sz
        L.indexcache_forward.argtypes = [ctypes.c_char_p, ctypes.POINTER(Layer), ctypes.POINTER(Shape),
                                         ctypes.POINTER(Seqs), vp, vp, vp, sz, ctypes.POINTER(Stats), vp]
        L.indexcache_forward.restype = i32
        L.indexcache_forward_noalloc.argtypes = [ctypes.c_char_p, ctypes.POINTER(Layer), ctypes.POINTER(Shape),
                                                 ctypes.POINTER(Seqs), vp, vp, ctypes.POINTER(Stats), vp]
        L.indexcache_forward_noalloc.restype = i32
        L.indexcache_forward_ws.argtypes = [ctypes.c_char_p, ctypes.POINTER(Shape), ctypes.POINTER(Seqs)]
        L.indexcache_forward_ws.restype = sz
        L.indexcache_plan.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        L.indexcache_plan.restype = i32
        L.dsa_status_string.argtypes = [i32]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_version.argtypes = []
        L.dsa_version.restype = i32
        L.dsa_index_overlap.argtypes = [vp, vp, ctypes.c_int64, i32, vp, vp]
        L.dsa_index_overlap.restype = i32
        L.dsa_quantize_fp8_rows.argtypes = [vp, ctypes.c_int64, i32, vp, vp, vp]
        L.dsa_quantize_fp8_rows.restype = i32
        L.dsa_indexer_project.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, i32, i32, i32, i32, i32, f32,
                                          f32, vp, vp, vp, vp]
        L.dsa_indexer_project.restype = i32
        L.dsa_cache_append.argtypes = [vp, ctypes.c_int64, vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
        L.dsa_cache_append.restype = i32
        L.dsa_attention_mass_ws.argtypes = [i32, i32, ctypes.POINTER(Seqs), i32]
        L.dsa_attention_mass_ws.restype = sz
        L.dsa_attention_mass.argtypes = [vp, vp, vp, i32, i32, i32, f32, ctypes.POINTER(Seqs), vp, vp, vp, vp, sz, vp]
        L.dsa_attention_mass.restype = i32
        L.dsa_indexer_kl_ws.argtypes = [i32, i32, ctypes.POINTER(Seqs)]
        L.dsa_indexer_kl_ws.restype = sz
        L.dsa_indexer_kl.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, ctypes.POINTER(Seqs), f32, i32, vp, vp, vp,
                                     sz, vp]
        L.dsa_indexer_kl.restype = i32
        _lib_handle = L
    return _lib_handle


def _check(rc: int):
    if rc != 0:
        raise DsaError(rc, lib().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _req(t: Optional[torch.Tensor], name: str, dtypes, shape=None, optional: bool = False):
    """Checks one tensor argument before it is handed to the library as a raw pointer:
    dtype (one of `dtypes`), exact shape (None entries are free) and contiguity.  Where
    the tensors live is checked afterwards, for all of them together (`_on_gpu`).
    Returns the tensor; raises ValueError."""
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if shape is not None:
        if t.dim() != len(shape) or any(want is not None and int(got) != int(want)
                                        for got, want in zip(t.shape, shape)):
            raise ValueError("%s must have shape %s, got %s" % (
                name, tuple("*" if x is None else x for x in shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _on_gpu(**tensors):
    """Every given tensor (None entries skipped) lives on one and the same GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be on a GPU, got %s" % (name, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, dev))


_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_F32 = (torch.float32,)
_QK = (torch.bfloat16, torch.float8_e4m3fn)
_OUT = (torch.float32, torch.bfloat16)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DSA_FP8_E4M3
    raise TypeError("indexer tensors must be bfloat16 or float8_e4m3fn, got %s" % t.dtype)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def indexcache_plan(roles: str):
    """Host-only plan: (src_layer list, number of indexer calls); raises DsaError on a bad role string."""
    n = len(roles)
    src = (ctypes.c_int32 * max(n, 1))()
    calls = ctypes.c_int32(0)
    _check(lib().indexcache_plan(roles.encode(), src, ctypes.byref(calls)))
    return [int(src[i]) for i in range(n)], int(calls.value)


def indexer_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor, k: int, seqs: Optional[Seqs] = None,
                 q_scale: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                 want_scores: bool = False, idx_out: Optional[torch.Tensor] = None,
                 score_out: Optional[torch.Tensor] = None, stream=None, bf16_scores: bool = False):
    """dsa_indexer_topk(_ex): returns (idx int32 [n_q, k], scores fp32 [n_q, k] or None).
    bf16_scores: rank bf16-rounded scores (DSA_TOPK_BF16_SCORES)."""
    _req(q_idx, "q_idx", _QK, (None, None, None))
    n_q, H, d = q_idx.shape
    dev = q_idx.device
    _req(k_idx, "k_idx", (q_idx.dtype,), (None, d))
    _req(w, "w", _BF16, (n_q, H))
    fp8 = q_idx.dtype == torch.float8_e4m3fn
    _req(q_scale, "q_scale", _F32, (n_q, H), optional=not fp8)
    _req(k_scale, "k_scale", _F32, (k_idx.shape[0],), optional=not fp8)
    if not fp8 and (q_scale is not None or k_scale is not None):
        raise ValueError("the bf16 indexer takes no scales")
    if seqs is None:
        seqs = Seqs.prefill(n_q, k_idx.shape[0], q_pos0=k_idx.shape[0] - n_q)
    if seqs.n_q != n_q or seqs.n_k > k_idx.shape[0]:
        raise ValueError("seqs describes %d queries over %d keys; tensors hold %d and %d"
                         % (seqs.n_q, seqs.n_k, n_q, k_idx.shape[0]))
    dt = _dtype_code(q_idx)
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    _req(idx_out, "idx_out", _I32, (n_q, k))
    if want_scores and score_out is None:
        score_out = torch.empty((n_q, k), dtype=torch.float32, device=dev)
    _req(score_out, "score_out", _F32, (n_q, k), optional=True)
    _on_gpu(q_idx=q_idx, k_idx=k_idx, w=w, q_scale=q_scale, k_scale=k_scale, idx_out=idx_out,
            score_out=score_out)
    L = lib()
    nbytes = L.dsa_indexer_topk_ws(dt, H, d, k, ctypes.byref(seqs))
    ws = _workspace(nbytes, dev)
    flags = DSA_TOPK_BF16_SCORES if bf16_scores else 0
    _check(L.dsa_indexer_topk_ex(_ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), dt, H, d, k,
                                 ctypes.byref(seqs), _ptr(idx_out), _ptr(score_out), _ptr(ws), nbytes, flags,
                                 _stream(stream)))
    return idx_out, score_out


def sparse_attn(q: torch.Tensor, latent: torch.Tensor, idx: torch.Tensor, seqs: Optional[Seqs] = None,
                scale: Optional[float] = None, d_v: int = 512, out_dtype=torch.float32,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dsa_sparse_attn: out [n_q, n_h, d_v] (fp32 by default)."""
    _req(q, "q", _BF16, (None, None, None))
    n_q, n_h, d_qk = q.shape
    dev = q.device
    _req(latent, "latent", _BF16, (None, d_qk))
    _req(idx, "idx", _I32, (n_q, None))
    k = idx.shape[1]
    if seqs is None:
        seqs = Seqs.prefill(n_q, latent.shape[0], q_pos0=latent.shape[0] - n_q)
    if seqs.n_q != n_q or seqs.n_k > latent.shape[0]:
        raise ValueError("seqs describes %d queries over %d keys; tensors hold %d and %d"
                         % (seqs.n_q, seqs.n_k, n_q, latent.shape[0]))
    if scale is None:
        scale = d_qk ** -0.5
    if out is None:
        out = torch.empty((n_q, n_h, d_v), dtype=out_dtype, device=q.device)
    _req(out, "out", _OUT, (n_q, n_h, d_v))
    odt = DSA_FP32 if out.dtype == torch.float32 else DSA_BF16
    _on_gpu(q=q, latent=latent, idx=idx, out=out)
    L = lib()
    nbytes = L.dsa_sparse_attn_ws(n_h, d_qk, d_v, k, ctypes.byref(seqs))
    ws = _workspace(nbytes, q.device)
    _check(L.dsa_sparse_attn(_ptr(q), _ptr(latent), _ptr(idx), n_h, d_qk, d_v, k, float(scale), ctypes.byref(seqs),
                             _ptr(out), odt, _ptr(ws), nbytes, _stream(stream)))
    return out


def quantize_fp8_rows(x: torch.Tensor, codes: Optional[torch.Tensor] = None,
                      scales: Optional[torch.Tensor] = None, stream=None):
    """dsa_quantize_fp8_rows over the last dimension of a bf16 tensor: returns
    (codes as float8_e4m3fn of x's shape, fp32 scales of x's shape without the last dim);
    codes (uint8 or float8_e4m3fn) and scales may be passed in preallocated."""
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise ValueError("x must be a bf16 tensor with at least one dimension")
    _req(x, "x", _BF16, tuple(x.shape))
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _req(codes, "codes", (torch.uint8, torch.float8_e4m3fn), tuple(x.shape))
    _req(scales, "scales", _F32, tuple(x.shape[:-1]))
    _on_gpu(x=x, codes=codes, scales=scales)
    _check(lib().dsa_quantize_fp8_rows(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes.view(torch.float8_e4m3fn), scales


def index_overlap(idx_a: torch.Tensor, idx_b: torch.Tensor, counts: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """dsa_index_overlap: counts[i] = |valid(idx_a[i]) ∩ valid(idx_b[i])| (int32); divide by k
    for the overlap fraction."""
    _req(idx_a, "idx_a", _I32, (None, None))
    n_rows, k = idx_a.shape
    _req(idx_b, "idx_b", _I32, (n_rows, k))
    if counts is None:
        counts = torch.empty((n_rows,), dtype=torch.int32, device=idx_a.device)
    _req(counts, "counts", _I32, (n_rows,))
    _on_gpu(idx_a=idx_a, idx_b=idx_b, counts=counts)
    _check(lib().dsa_index_overlap(_ptr(idx_a), _ptr(idx_b), n_rows, k, _ptr(counts), _stream(stream)))
    return counts


def indexer_project(q_lat: torch.Tensor, h: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor,
                    ln_weight: torch.Tensor, ln_bias: torch.Tensor, ww: torch.Tensor, pos: torch.Tensor, H: int,
                    rope_dim: int = 64, rope_base: float = 10000.0, eps: float = 1e-5, q_idx=None, k_idx=None,
                    w=None, stream=None):
    """dsa_indexer_project: (q_idx [n, H, d], k_idx [n, d], w [n, H]) bf16 from the query latent
    q_lat [n, r] and hidden state h [n, hidden] (weights in nn.Linear layout [out, in])."""
    _req(q_lat, "q_lat", _BF16, (None, None))
    n, r = q_lat.shape
    _req(h, "h", _BF16, (n, None))
    hidden = h.shape[1]
    _req(wk, "wk", _BF16, (None, hidden))
    d = wk.shape[0]
    _req(wq, "wq", _BF16, (H * d, r))
    _req(ww, "ww", _BF16, (H, hidden))
    _req(ln_weight, "ln_weight", _F32, (d,))
    _req(ln_bias, "ln_bias", _F32, (d,))
    _req(pos, "pos", _I32, (n,))
    dev = q_lat.device
    if q_idx is None:
        q_idx = torch.empty((n, H, d), dtype=torch.bfloat16, device=dev)
    if k_idx is None:
        k_idx = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    if w is None:
        w = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    _req(q_idx, "q_idx", _BF16, (n, H, d))
    _req(k_idx, "k_idx", _BF16, (n, d))
    _req(w, "w", _BF16, (n, H))
    _on_gpu(q_lat=q_lat, h=h, wq=wq, wk=wk, ln_weight=ln_weight, ln_bias=ln_bias, ww=ww, pos=pos, q_idx=q_idx,
            k_idx=k_idx, w=w)
    _check(lib().dsa_indexer_project(_ptr(q_lat), _ptr(h), _ptr(wq), _ptr(wk), _ptr(ln_weight), _ptr(ln_bias),
                                     _ptr(ww), _ptr(pos), n, r, hidden, H, d, rope_dim, float(rope_base), float(eps),
                                     _ptr(q_idx), _ptr(k_idx), _ptr(w), _stream(stream)))
    return q_idx, k_idx, w


def _stat_inputs(q, latent, idx, seqs):
    _req(q, "q", _BF16, (None, None, None))
    n_q, n_h, d_qk = q.shape
    _req(latent, "latent", _BF16, (None, d_qk))
    _req(idx, "idx", _I32, (n_q, None))
    if seqs is None:
        seqs = Seqs.prefill(n_q, latent.shape[0], q_pos0=latent.shape[0] - n_q)
    if seqs.n_q != n_q or seqs.n_k > latent.shape[0]:
        raise ValueError("seqs describes %d queries over %d keys; tensors hold %d and %d"
                         % (seqs.n_q, seqs.n_k, n_q, latent.shape[0]))
    return n_q, n_h, d_qk, idx.shape[1], seqs


def attention_mass(q: torch.Tensor, latent: torch.Tensor, idx: torch.Tensor, seqs: Optional[Seqs] = None,
                   scale: Optional[float] = None, want_recall: bool = True, stream=None):
    """dsa_attention_mass: (mass_head [n_q, n_h], mass [n_q], recall [n_q] or None), fp32:
    CapturedMass@k per head and for the head-aggregated dense distribution, Recall@k of
    the selection idx against the dense distribution's own top-k."""
    n_q, n_h, d_qk, k, seqs = _stat_inputs(q, latent, idx, seqs)
    dev = q.device
    mass_head = torch.empty((n_q, n_h), dtype=torch.float32, device=dev)
    mass = torch.empty((n_q,), dtype=torch.float32, device=dev)
    recall = torch.empty((n_q,), dtype=torch.float32, device=dev) if want_recall else None
    _on_gpu(q=q, latent=latent, idx=idx)
    L = lib()
    nbytes = L.dsa_attention_mass_ws(n_h, k, ctypes.byref(seqs), int(want_recall))
    ws = _workspace(nbytes, dev)
    _check(L.dsa_attention_mass(_ptr(q), _ptr(latent), _ptr(idx), n_h, d_qk, k,
                                float(d_qk ** -0.5 if scale is None else scale), ctypes.byref(seqs), _ptr(mass_head),
                                _ptr(mass), _ptr(recall), _ptr(ws), nbytes, _stream(stream)))
    return mass_head, mass, recall


def indexer_kl(q: torch.Tensor, latent: torch.Tensor, idx: torch.Tensor, scores: torch.Tensor,
               seqs: Optional[Seqs] = None, scale: Optional[float] = None, weight: float = 1.0,
               kl: Optional[torch.Tensor] = None, accumulate: bool = False, want_loss: bool = False, stream=None):
    """dsa_indexer_kl: per-row KL(p_{t,S_t} || softmax(I_{t,S_t})) (times weight, added to kl
    when accumulate), and optionally the sum over rows (a 1-element tensor)."""
    n_q, n_h, d_qk, k, seqs = _stat_inputs(q, latent, idx, seqs)
    _req(scores, "scores", _F32, (n_q, k))
    dev = q.device
    if kl is None:
        if accumulate:
            raise ValueError("accumulate needs the kl tensor to add to")
        kl = torch.empty((n_q,), dtype=torch.float32, device=dev)
    _req(kl, "kl", _F32, (n_q,))
    loss = torch.empty((1,), dtype=torch.float32, device=dev) if want_loss else None
    _on_gpu(q=q, latent=latent, idx=idx, scores=scores, kl=kl)
    L = lib()
    nbytes = L.dsa_indexer_kl_ws(n_h, k, ctypes.byref(seqs))
    ws = _workspace(nbytes, dev)
    _check(L.dsa_indexer_kl(_ptr(q), _ptr(latent), _ptr(idx), _ptr(scores), n_h, d_qk, k,
                            float(d_qk ** -0.5 if scale is None else scale), ctypes.byref(seqs), float(weight),
                            int(accumulate), _ptr(kl), _ptr(loss), _ptr(ws), nbytes, _stream(stream)))
    return kl, loss


def csa_compress(ca: torch.Tensor, cb: torch.Tensor, za: torch.Tensor, zb: torch.Tensor, ba: torch.Tensor,
                 bb: torch.Tensor, m: int, block0: int = 0, out: Optional[torch.Tensor] = None,
                 out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """dsa_csa_compress: gated pooling of the n token rows into compressed entries block0 .. n // m - 1.
    ca, cb, za, zb [n, c] bf16; ba, bb [m, c] fp32; returns out [n // m - block0, c]."""
    _req(ca, "ca", _BF16, (None, None))
    n, c = ca.shape
    for name, t in (("cb", cb), ("za", za), ("zb", zb)):
        _req(t, name, _BF16, (n, c))
    _req(ba, "ba", _F32, (m, c))
    _req(bb, "bb", _F32, (m, c))
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    n_out = max(n // m - block0, 0) if m >= 1 else 0
    if out is None:
        out = torch.empty((n_out, c), dtype=out_dtype, device=ca.device)
    _req(out, "out", (out_dtype,), (n_out, c))
    _on_gpu(ca=ca, cb=cb, za=za, zb=zb, ba=ba, bb=bb, out=out)
    _check(lib().dsa_csa_compress(_ptr(ca), _ptr(cb), _ptr(za), _ptr(zb), _ptr(ba), _ptr(bb), n, c, m, block0,
                                  _ptr(out), DSA_FP32 if out_dtype == torch.float32 else DSA_BF16,
                                  _stream(stream)))
    return out


def cache_append(cache: torch.Tensor, dst_row: torch.Tensor, rows: torch.Tensor, stream=None) -> torch.Tensor:
    """dsa_cache_append: rows[b] -> cache[dst_row[b]] (2-D tensors of one dtype and row width;
    dst_row int64).  Destinations outside the cache are skipped."""
    if not isinstance(cache, torch.Tensor) or cache.dim() != 2:
        raise ValueError("cache must be a 2-D tensor")
    _req(cache, "cache", (cache.dtype,), tuple(cache.shape))
    _req(rows, "rows", (cache.dtype,), (None, cache.shape[1]))
    _req(dst_row, "dst_row", (torch.int64,), (rows.shape[0],))
    _on_gpu(cache=cache, dst_row=dst_row, rows=rows)
    _check(lib().dsa_cache_append(_ptr(cache), cache.shape[0], _ptr(dst_row), _ptr(rows), rows.shape[0],
                                  cache.shape[1] * cache.element_size(), _stream(stream)))
    return cache


class ForwardResult:
    def __init__(self, outs, index_cache, score_cache, stats: Stats, ws=None):
        self.outs = outs
        self.index_cache = index_cache
        self.score_cache = score_cache
        self.ws = ws          # the workspace used; pass it back to reuse it
        self.n_indexer_calls = int(stats.n_indexer_calls)
        self.n_chunks = int(stats.n_chunks)
        self.src_layer = [int(stats.src_layer[i]) for i in range(stats.n_layers)]
        self.trace = [(int(stats.trace_kind[j]), int(stats.trace_layer[j]), int(stats.trace_chunk[j]))
                      for j in range(stats.n_traced)]


def _forward_args(roles, layers, k, seqs, q_chunk, index_rows, out_rows, scale, d_v, out_dtype, want_scores, outs,
                  index_cache, score_cache, ws, allocate: bool, bf16_scores: bool = False):
    """Validates and marshals the arguments of indexcache_forward(_noalloc).  With
    allocate=False every output must be given (nothing is allocated here)."""
    n_layers = len(roles)
    if len(layers) != n_layers:
        raise ValueError("one layer dict per role")
    l0 = layers[0]
    _req(l0.get("q"), "layers[0].q", _BF16, (None, None, None))
    n_q, n_h, d_qk = l0["q"].shape
    dev = l0["q"].device
    f0 = next(i for i, r in enumerate(roles) if r == "F") if "F" in roles else 0
    qi = layers[f0].get("q_idx")
    n_k = l0["latent"].shape[0] if l0.get("latent") is not None else 0
    for l, d in enumerate(layers):
        _req(d.get("q"), "layers[%d].q" % l, _BF16, (n_q, n_h, d_qk))
        _req(d.get("latent"), "layers[%d].latent" % l, _BF16, (n_k, d_qk))
        if roles[l:l + 1] == "F":
            _req(d.get("q_idx"), "layers[%d].q_idx" % l, _QK, (n_q, None, None))
            H_, d_ = d["q_idx"].shape[1:]
            _req(d.get("k_idx"), "layers[%d].k_idx" % l, (d["q_idx"].dtype,), (n_k, d_))
            _req(d.get("w"), "layers[%d].w" % l, _BF16, (n_q, H_))
            fp8 = d["q_idx"].dtype == torch.float8_e4m3fn
            _req(d.get("q_scale"), "layers[%d].q_scale" % l, _F32, (n_q, H_), optional=not fp8)
            _req(d.get("k_scale"), "layers[%d].k_scale" % l, _F32, (n_k,), optional=not fp8)
    if seqs is None:
        seqs = Seqs.prefill(n_q, l0["latent"].shape[0], q_pos0=l0["latent"].shape[0] - n_q)
    shape = Shape()
    shape.H, shape.d = (qi.shape[1], qi.shape[2]) if qi is not None else (0, 0)
    shape.k, shape.n_h, shape.d_qk, shape.d_v = k, n_h, d_qk, d_v
    shape.scale = float(d_qk ** -0.5 if scale is None else scale)
    shape.qk_dtype = _dtype_code(qi) if qi is not None else DSA_BF16
    shape.out_dtype = DSA_FP32 if out_dtype == torch.float32 else DSA_BF16
    shape.flags = DSA_TOPK_BF16_SCORES if bf16_scores else 0
    shape.q_chunk = int(q_chunk or max(n_q, 1))
    shape.index_rows = int(index_rows or max(n_q, 1))
    shape.out_rows = int(out_rows or max(n_q, 1))
    if outs is None:
        if not allocate:
            raise ValueError("outs are required")
        outs = [torch.empty((shape.out_rows, n_h, d_v), dtype=out_dtype, device=dev) for _ in range(n_layers)]
    if len(outs) != n_layers:
        raise ValueError("one output tensor per layer")
    for l, o in enumerate(outs):
        _req(o, "outs[%d]" % l, (out_dtype,), (shape.out_rows, n_h, d_v))
    if index_cache is None:
        if not allocate:
            raise ValueError("index_cache is required")
        index_cache = torch.empty((shape.index_rows, k), dtype=torch.int32, device=dev)
    _req(index_cache, "index_cache", _I32, (shape.index_rows, k))
    if want_scores and score_cache is None:
        if not allocate:
            raise ValueError("score_cache is required for want_scores")
        score_cache = torch.empty((shape.index_rows, k), dtype=torch.float32, device=dev)
    _req(score_cache, "score_cache", _F32, (shape.index_rows, k), optional=True)
    if ws is not None:
        _req(ws, "ws", (torch.uint8,), (None,))
    named = {"outs[%d]" % l: o for l, o in enumerate(outs)}
    for l, d in enumerate(layers):
        named.update({"layers[%d].%s" % (l, n): t for n, t in d.items() if isinstance(t, torch.Tensor)})
    _on_gpu(index_cache=index_cache, score_cache=score_cache, ws=ws, **named)
    arr = (Layer * n_layers)()
    for l, d in enumerate(layers):
        for name in ("q_idx", "q_scale", "k_idx", "k_scale", "w", "q", "latent"):
            t = d.get(name)
            setattr(arr[l], name, _ptr(t) if t is not None else None)
        arr[l].out = _ptr(outs[l])
    return arr, shape, seqs, outs, index_cache, score_cache, dev


def _stats(events) -> Stats:
    stats = Stats()
    if events is not None:     # ctypes array of hipEvent_t handles created by the caller
        stats.events = ctypes.cast(events, ctypes.c_void_p)
        stats.event_cap = len(events)
    return stats


def indexcache_forward(roles: str, layers: Sequence[dict], k: int, seqs: Optional[Seqs] = None,
                       q_chunk: Optional[int] = None, index_rows: Optional[int] = None,
                       out_rows: Optional[int] = None, scale: Optional[float] = None, d_v: int = 512,
                       out_dtype=torch.float32, want_scores: bool = False, outs: Optional[List[torch.Tensor]] = None,
                       index_cache: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       events=None, stream=None, score_cache: Optional[torch.Tensor] = None,
                       bf16_scores: bool = False) -> ForwardResult:
    """indexcache_forward over layers given as dicts of tensors
    {q_idx, q_scale, k_idx, k_scale, w, q, latent} (indexer tensors needed on F layers only).
    bf16_scores: the F layers rank bf16-rounded scores (DSA_TOPK_BF16_SCORES)."""
    arr, shape, seqs, outs, index_cache, score_cache, dev = _forward_args(
        roles, layers, k, seqs, q_chunk, index_rows, out_rows, scale, d_v, out_dtype, want_scores, outs,
        index_cache, score_cache, ws, allocate=True, bf16_scores=bf16_scores)
    L = lib()
    need = L.indexcache_forward_ws(roles.encode(), ctypes.byref(shape), ctypes.byref(seqs))
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dev)
    stats = _stats(events)
    _check(L.indexcache_forward(roles.encode(), arr, ctypes.byref(shape), ctypes.byref(seqs), _ptr(index_cache),
                                _ptr(score_cache), _ptr(ws), ws.numel() if ws is not None else 0, ctypes.byref(stats),
                                _stream(stream)))
    return ForwardResult(outs, index_cache, score_cache, stats, ws)


def indexcache_forward_noalloc(roles: str, layers: Sequence[dict], k: int, outs: List[torch.Tensor],
                               index_cache: torch.Tensor, seqs: Optional[Seqs] = None, q_chunk: Optional[int] = None,
                               index_rows: Optional[int] = None, out_rows: Optional[int] = None,
                               scale: Optional[float] = None, d_v: int = 512, out_dtype=torch.float32,
                               score_cache: Optional[torch.Tensor] = None, events=None,
                               stream=None, bf16_scores: bool = False) -> ForwardResult:
    """indexcache_forward_noalloc: the same loop with the library's own per-GPU scratch array as
    workspace; every output is passed in and nothing is allocated."""
    arr, shape, seqs, outs, index_cache, score_cache, dev = _forward_args(
        roles, layers, k, seqs, q_chunk, index_rows, out_rows, scale, d_v, out_dtype, score_cache is not None,
        outs, index_cache, score_cache, None, allocate=False, bf16_scores=bf16_scores)
    stats = _stats(events)
    _check(lib().indexcache_forward_noalloc(roles.encode(), arr, ctypes.byref(shape), ctypes.byref(seqs),
                                            _ptr(index_cache), _ptr(score_cache), ctypes.byref(stats),
                                            _stream(stream)))
    return ForwardResult(outs, index_cache, score_cache, stats)


def layer_dict(li) -> dict:
    """Adapter for objects with q_idx/q_scale/k_idx/k_scale/w/q/latent attributes."""
    return {n: getattr(li, n) for n in ("q_idx", "q_scale", "k_idx", "k_scale", "w", "q", "latent")}
