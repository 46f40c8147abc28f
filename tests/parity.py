"""Row-wise comparison of the HIP path with the CPU oracle (test infrastructure).

Acceptance rules (per query row; every row is independent, so checking a row is
exact parity for that row):
  * integer-valued inputs: index sets identical, scores bit-identical;
  * float inputs, scores: |I_gpu - I_oracle| <= 1e-3 * max_s |I_oracle[t, s]|;
  * float inputs, top-k: mean recall over checked rows >= 0.999, and every index in
    the symmetric difference has |I_oracle - kth| <= that tolerance;
  * attention, evaluated by the oracle on the GPU's own index rows: max |err| <= 1e-2;
  * every row: min(k, t+1) distinct valid positions in [0, t], the rest -1.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import csa as ocsa
import synth

SCORE_REL = 1e-3
RECALL_MIN = 0.999
ATTN_ATOL = 1e-2


def sample_rows(n_q: int, k: int, n: int = 32, seed: int = 0, extra=()) -> list:
    """Stratified rows: the edges of the top-k budget and of 8192-row chunks, the last row, uniform draws."""
    fixed = {0, 1, k - 2, k - 1, k, k + 1, 8191, 8192, 8193, n_q - 1, n_q - 2, *extra}
    g = np.random.default_rng(seed)
    rnd = set(g.integers(0, n_q, size=n).tolist()) if n_q > 0 else set()
    return sorted(r for r in fixed | rnd if 0 <= r < n_q)


def row_geometry(seqs, i: int):
    """(last visible key p, first key row k0) of packed query row i: its position t over
    token keys; over compressed blocks of m = seqs.block tokens, t // m - 1 (-1: none)."""
    b = 0
    while b + 1 < seqs.B and i >= seqs.q_start[b + 1]:
        b += 1
    t = int(seqs.q_pos0[b] + (i - seqs.q_start[b]))
    if seqs.block > 1:
        t = ocsa.visible_blocks(t, int(seqs.block)) - 1
    return t, int(seqs.k_start[b])


def _deq(t: torch.Tensor, scale) -> np.ndarray:
    if t.dtype == torch.float8_e4m3fn:
        return oracle.dequant_rows(synth.bits(t), synth.bits(scale), "fp8")
    return oracle.dequant_rows(synth.bits(t), None, "bf16")


class OracleView:
    """Host float64 views of one layer's inputs, decoded on demand from the exact device bytes."""

    def __init__(self, li):
        self.li = li
        self._k = None

    def keys(self) -> np.ndarray:
        if self._k is None:
            self._k = _deq(self.li.k_idx, self.li.k_scale)
        return self._k

    def q_idx_rows(self, rows) -> np.ndarray:
        r = torch.as_tensor(rows, device=self.li.q_idx.device)
        qs = self.li.q_scale[r] if self.li.q_scale is not None else None
        return _deq(self.li.q_idx[r], qs)

    def w_rows(self, rows) -> np.ndarray:
        r = torch.as_tensor(rows, device=self.li.w.device)
        return oracle.decode_bf16(synth.bits(self.li.w[r]))

    def q_rows(self, rows) -> np.ndarray:
        r = torch.as_tensor(rows, device=self.li.q.device)
        return oracle.decode_bf16(synth.bits(self.li.q[r]))

    def latent_rows(self, rows) -> np.ndarray:
        r = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=self.li.latent.device)
        return oracle.decode_bf16(synth.bits(self.li.latent[r]))


def check_valid_row(row: np.ndarray, p: int, k: int):
    m = min(k, p + 1)
    v = row[:m]
    assert np.all(row[m:] == -1), "slots past min(k, t+1) must be -1"
    assert np.all((v >= 0) & (v <= p)), "valid positions must lie in [0, t]"
    assert len(np.unique(v)) == m, "positions must be distinct"
    assert np.all(np.diff(v) > 0), "valid positions are written ascending"


def check_indexer(view: OracleView, seqs, rows, k: int, idx_gpu: torch.Tensor, sc_gpu, exact: bool):
    """Checks GPU index rows (and scores) of `rows` against the oracle.  Returns stats."""
    rows = list(rows)
    qv, wv = view.q_idx_rows(rows), view.w_rows(rows)
    keys = view.keys()
    r = torch.as_tensor(rows, device=idx_gpu.device)
    ig = idx_gpu[r].cpu().numpy()
    sg = sc_gpu[r].cpu().numpy() if sc_gpu is not None else None
    recalls, worst_score = [], 0.0
    for n, i in enumerate(rows):
        p, k0 = row_geometry(seqs, i)
        I = oracle.indexer_row(qv[n], wv[n], keys[k0:k0 + p + 1])
        ro, kth, m = oracle.topk_row(I, k)
        check_valid_row(ig[n], p, k)
        got = ig[n][:m]
        if m == 0:
            recalls.append(1.0)
            continue
        if exact:
            assert np.array_equal(got, ro[:m]), "row %d: index set differs" % i
            if sg is not None:
                assert np.array_equal(sg[n][:m], I[got].astype(np.float32)), "row %d: scores differ" % i
                assert np.all(sg[n][m:] == 0)
            recalls.append(1.0)
            continue
        tol = oracle.tolerance_row(I, SCORE_REL)
        if sg is not None:
            err = np.abs(sg[n][:m].astype(np.float64) - I[got])
            worst_score = max(worst_score, float(err.max() / max(tol, 1e-300)))
            assert np.all(err <= tol), "row %d: score error %g > tol %g" % (i, err.max(), tol)
        a, b = set(got.tolist()), set(ro[:m].tolist())
        recalls.append(len(a & b) / m)
        for s in a ^ b:
            assert abs(I[s] - kth) <= tol, "row %d: mismatch at %d is %g from the k-th score (tol %g)" % (
                i, s, abs(I[s] - kth), tol)
    mean = float(np.mean(recalls)) if recalls else 1.0
    assert mean >= RECALL_MIN, "mean recall %.5f < %.3f" % (mean, RECALL_MIN)
    return {"rows": len(rows), "recall_mean": mean, "recall_min": float(np.min(recalls)) if recalls else 1.0,
            "score_err_over_tol": worst_score}


def check_attention(view: OracleView, seqs, rows, idx_gpu: torch.Tensor, out_gpu: torch.Tensor, scale: float,
                    d_v: int = 512, out_row_of=lambda i: i):
    """Oracle attention on the GPU's own index rows vs the GPU output.  Returns the max abs error."""
    rows = list(rows)
    qv = view.q_rows(rows)
    r = torch.as_tensor(rows, device=idx_gpu.device)
    ig = idx_gpu[r].cpu().numpy()
    og = out_gpu[torch.as_tensor([out_row_of(i) for i in rows], device=out_gpu.device)].float().cpu().numpy()
    worst = 0.0
    for n, i in enumerate(rows):
        p, k0 = row_geometry(seqs, i)
        row = ig[n]
        sel = row[(row >= 0) & (row <= p)]
        lat = view.latent_rows(k0 + sel) if sel.size else np.zeros((0, 576))
        o = oracle.attn_row(qv[n], lat, np.arange(sel.size), scale, d_v)
        err = float(np.abs(o - og[n]).max())
        worst = max(worst, err)
        assert err <= ATTN_ATOL, "row %d: attention max abs error %g > %g" % (i, err, ATTN_ATOL)
    return worst


def check_indexer_bf16(view: OracleView, seqs, rows, k: int, idx_gpu: torch.Tensor, sc_gpu: torch.Tensor):
    """Checks a bf16-score selection (scores rounded to bf16 before the ranking).

    The oracle rounds its fp64 score through fp32 to bf16 (nearest even); the GPU rounds
    its fp32 sum, which lies within the fp32 tolerance of the fp64 score, so a score whose
    fp64 value sits within that tolerance of a rounding midpoint may round either way.
    Rules per row: every returned score is a bf16 value and equals the oracle's rounded
    score or, for such a score, its neighbour; the set equals the oracle's selection
    (rounded scores descending, ties to the lower position) except for keys whose rounded
    score is within one bf16 step of the k-th rounded score; mean recall >= 0.995."""
    rows = list(rows)
    qv, wv = view.q_idx_rows(rows), view.w_rows(rows)
    keys = view.keys()
    r = torch.as_tensor(rows, device=idx_gpu.device)
    ig = idx_gpu[r].cpu().numpy()
    sg = sc_gpu[r].cpu().numpy()
    recalls = []
    for n, i in enumerate(rows):
        p, k0 = row_geometry(seqs, i)
        I = oracle.indexer_row(qv[n], wv[n], keys[k0:k0 + p + 1])
        Ib = ocsa.round_bf16(I)
        ro, kth, m = oracle.topk_row(Ib, k)
        check_valid_row(ig[n], p, k)
        got = ig[n][:m]
        if m == 0:
            recalls.append(1.0)
            continue
        tol = oracle.tolerance_row(I, SCORE_REL)
        s = sg[n][:m]
        assert np.all(s.view(np.uint32) & 0xFFFF == 0), "row %d: scores are not bf16 values" % i
        lo, hi = ocsa.round_bf16(I[got] - tol), ocsa.round_bf16(I[got] + tol)
        assert np.all((s >= lo) & (s <= hi)), "row %d: a bf16 score is off its rounding range" % i
        step = 2.0 ** (np.floor(np.log2(max(abs(kth), 1e-30))) - 7)
        a, b = set(got.tolist()), set(ro[:m].tolist())
        recalls.append(len(a & b) / m)
        for x in a ^ b:
            assert abs(Ib[x] - kth) <= step + tol, "row %d: mismatch at %d is %g from the k-th score" % (
                i, x, abs(Ib[x] - kth))
    mean = float(np.mean(recalls)) if recalls else 1.0
    assert mean >= 0.995, "mean recall %.5f" % mean
    return {"rows": len(rows), "recall_mean": mean}
