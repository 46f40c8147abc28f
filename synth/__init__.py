"""Seeded synthetic inputs for the DSA indexer / top-k / sparse-MLA-attention path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds *no* arithmetic of the method: it only draws random numbers,
rounds them into the storage formats the path consumes (bf16, OCP fp8 e4m3fn with
a per-row fp32 scale) and describes the five synthetic workloads.  Every tensor is
a pure function of (workload, layer, tensor id, seed).

Workloads (shapes follow the DSA/IndexCache pages: k = 2048 top-k budget, 64
indexer heads x 128, a 576-wide MLA latent whose first 512 columns are values,
47-layer stacks with one F layer in four, contexts up to 200K):

  0  one layer, L=1024, H=8, d=64, k=128, n_h=16, integer-valued indexer inputs
  1  one layer, L=32768, H=64, d=128, k=2048, n_h=128, bf16 N(0,1)
  2  8 layers FSSSFSSS, L=65536, shapes as 1
  3  decode: 8 sequences, len ~ U{150000..200000}, 47 layers (F every 4th)
  4  4 layers FSSS, L=200000, fp8 e4m3fn indexer inputs with per-row scales

Host generation uses NumPy's PCG64 seeded by SeedSequence([0xD5A, workload,
layer, tensor]).  Tensors too large for the host are drawn on the device with a
torch Philox generator seeded from the same tuple (deterministic for a given
device and torch build); any comparison against the oracle reads those bytes back.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional, Sequence

import numpy as np
import torch

# tensor ids inside one layer
T_QIDX, T_KIDX, T_W, T_Q, T_LAT, T_LENS = 1, 2, 3, 4, 5, 6

D_QK = 576   # MLA latent width (512 value columns + 64 rope columns)
D_V = 512


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    L: int                 # prefill length (queries == keys); decode: unused
    H: int                 # indexer heads H^I
    d: int                 # indexer head dim d_I
    k: int                 # top-k budget
    n_h: int               # attention query heads
    roles: str             # F/S role string, one char per layer
    qk_dtype: str          # "bf16" | "fp8"
    q_chunk: int           # prefill query chunk
    integer_indexer: bool = False
    decode_B: int = 0      # decode: number of sequences
    len_lo: int = 0
    len_hi: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(D_QK))

    @property
    def n_layers(self) -> int:
        return len(self.roles)


WORKLOADS: Dict[int, Workload] = {
    0: Workload(0, "prefill L=1024 H=8 d=64 k=128 n_h=16 integer-valued", 1024, 8, 64, 128, 16,
                "F", "bf16", 1024, integer_indexer=True),
    1: Workload(1, "prefill L=32768 H=64 d=128 k=2048 n_h=128 bf16", 32768, 64, 128, 2048, 128,
                "F", "bf16", 32768),
    2: Workload(2, "8-layer FSSSFSSS prefill L=65536 bf16", 65536, 64, 128, 2048, 128,
                "FSSSFSSS", "bf16", 65536),
    3: Workload(3, "decode B=8 len~U[150000,200000] 47 layers", 0, 64, 128, 2048, 128,
                "FSSS" * 11 + "FSS", "bf16", 1, decode_B=8, len_lo=150000, len_hi=200000),
    4: Workload(4, "4-layer FSSS prefill L=200000 fp8 indexer", 200000, 64, 128, 2048, 128,
                "FSSS", "fp8", 8192),
}


def seed_tuple(wid: int, layer: int, tensor: int, salt: int = 0) -> Sequence[int]:
    return [0xD5A, wid, layer, tensor, salt]


def rng(wid: int, layer: int, tensor: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed_tuple(wid, layer, tensor, salt))))


def torch_seed(wid: int, layer: int, tensor: int, salt: int = 0) -> int:
    h = hashlib.sha256(repr(tuple(seed_tuple(wid, layer, tensor, salt))).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


# ---------------------------------------------------------------------------
# storage-format rounding (input preparation, not the method)
# ---------------------------------------------------------------------------

def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 to bf16, nearest-even (torch's cast)."""
    return x.to(torch.float32).to(torch.bfloat16)


FP8_MAX = 448.0


def quantize_fp8_rows(x: torch.Tensor):
    """Per-row OCP e4m3fn quantisation: scale = amax/448 over the last dim,
    payload = RNE(clamp(x/scale, +-448)).  Returns (payload float8_e4m3fn,
    scale fp32 with the last dim dropped).  A zero row gets scale 1."""
    x = x.to(torch.float32)
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn), scale.contiguous()


# ---------------------------------------------------------------------------
# generic random tensors
# ---------------------------------------------------------------------------

def _normal(shape, wid, layer, tensor, device, salt=0, div=1.0) -> torch.Tensor:
    """N(0,1)/div rounded to bf16.  Host: PCG64; device: torch Philox."""
    if device == "cpu" or device is None:
        g = rng(wid, layer, tensor, salt)
        x = torch.from_numpy(g.standard_normal(size=shape, dtype=np.float32))
        if div != 1.0:
            x = x / div
        return to_bf16(x)
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(wid, layer, tensor, salt))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    step = 1 << 28
    for s in range(0, flat.numel(), step):
        n = min(step, flat.numel() - s)
        x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        if div != 1.0:
            x /= div
        flat[s:s + n] = x.to(torch.bfloat16)
        del x
    return out


def _int_uniform(shape, lo, hi, wid, layer, tensor, salt=0) -> torch.Tensor:
    g = rng(wid, layer, tensor, salt)
    return torch.from_numpy(g.integers(lo, hi + 1, size=shape).astype(np.float32)).to(torch.bfloat16)


def _choice(shape, values, wid, layer, tensor, salt=0) -> torch.Tensor:
    g = rng(wid, layer, tensor, salt)
    v = np.asarray(values, dtype=np.float32)
    return torch.from_numpy(v[g.integers(0, len(v), size=shape)]).to(torch.bfloat16)


# ---------------------------------------------------------------------------
# layer inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LayerInputs:
    q_idx: torch.Tensor            # [n_q, H, d] bf16 or float8_e4m3fn
    q_scale: Optional[torch.Tensor]  # [n_q, H] fp32 (fp8 only)
    k_idx: torch.Tensor            # [n_k, d]
    k_scale: Optional[torch.Tensor]  # [n_k] fp32 (fp8 only)
    w: torch.Tensor                # [n_q, H] bf16
    q: torch.Tensor                # [n_q, n_h, 576] bf16
    latent: torch.Tensor           # [n_k, 576] bf16

    def to(self, device) -> "LayerInputs":
        f = lambda t: None if t is None else t.to(device)
        return LayerInputs(*(f(getattr(self, n)) for n in
                             ("q_idx", "q_scale", "k_idx", "k_scale", "w", "q", "latent")))


def make_layer(n_q: int, n_k: int, H: int, d: int, n_h: int, *, wid: int, layer: int,
               qk_dtype: str = "bf16", integer_indexer: bool = False, device: str = "cpu",
               salt: int = 0, with_indexer: bool = True, with_attention: bool = True) -> LayerInputs:
    """Inputs of one DSA layer.  Prefill: n_q == n_k.  Decode: n_q = B and n_k = sum of lens."""
    if integer_indexer:
        assert qk_dtype == "bf16" and device == "cpu"
        q_idx = _int_uniform((n_q, H, d), -4, 4, wid, layer, T_QIDX, salt) if with_indexer else None
        k_idx = _int_uniform((n_k, d), -4, 4, wid, layer, T_KIDX, salt) if with_indexer else None
        w = _choice((n_q, H), (-1.0, -0.5, 0.5, 1.0), wid, layer, T_W, salt) if with_indexer else None
        qs = ks = None
    elif with_indexer:
        qf = _normal((n_q, H, d), wid, layer, T_QIDX, device, salt)
        kf = _normal((n_k, d), wid, layer, T_KIDX, device, salt)
        w = _normal((n_q, H), wid, layer, T_W, device, salt, div=8.0)
        if qk_dtype == "fp8":
            q_idx, qs = quantize_fp8_rows(qf)
            del qf
            k_idx, ks = quantize_fp8_rows(kf)
            del kf
        else:
            q_idx, k_idx, qs, ks = qf, kf, None, None
    else:
        q_idx = k_idx = w = qs = ks = None
    if with_attention:
        q = _normal((n_q, n_h, D_QK), wid, layer, T_Q, device, salt)
        lat = _normal((n_k, D_QK), wid, layer, T_LAT, device, salt)
    else:
        q = lat = None
    return LayerInputs(q_idx, qs, k_idx, ks, w, q, lat)


def workload_layer(wid: int, layer: int, device: str = "cpu", L: Optional[int] = None,
                   with_indexer: bool = True, with_attention: bool = True) -> LayerInputs:
    """Inputs of layer `layer` of prefill workload `wid` (optionally at a reduced L)."""
    w = WORKLOADS[wid]
    assert w.decode_B == 0
    n = w.L if L is None else L
    return make_layer(n, n, w.H, w.d, w.n_h, wid=wid, layer=layer, qk_dtype=w.qk_dtype,
                      integer_indexer=w.integer_indexer, device=device,
                      with_indexer=with_indexer, with_attention=with_attention)


def decode_lengths(wid: int = 3) -> np.ndarray:
    """Context lengths of the decode workload: integers, inclusive range, seeded."""
    w = WORKLOADS[wid]
    g = rng(wid, 0, T_LENS)
    return g.integers(w.len_lo, w.len_hi + 1, size=w.decode_B).astype(np.int64)


def decode_layer(layer: int, lens: Sequence[int], device: str = "cpu", wid: int = 3) -> LayerInputs:
    """One decode layer: B single queries over packed per-sequence caches (sum(lens) rows)."""
    w = WORKLOADS[wid]
    return make_layer(len(lens), int(np.sum(lens)), w.H, w.d, w.n_h, wid=wid, layer=layer,
                      qk_dtype=w.qk_dtype, device=device)


def csa_inputs(n: int, c: int, m: int, seed: int = 0):
    """Token-level inputs of the KV compression of compressed sparse attention: values C^a, C^b
    and gate logits Z^a, Z^b [n, c] bf16 N(0,1); gate biases B^a, B^b [m, c] fp32 N(0, 1/4)."""
    g = np.random.default_rng([0xC5A, n, c, m, seed])
    vals = [to_bf16(torch.from_numpy(g.standard_normal((n, c), dtype=np.float32))) for _ in range(4)]
    biases = [torch.from_numpy((0.5 * g.standard_normal((m, c))).astype(np.float32)) for _ in range(2)]
    ca, cb, za, zb = vals
    return ca, cb, za, zb, biases[0], biases[1]


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a bf16 / fp8 tensor as a NumPy unsigned array (host copy)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)
