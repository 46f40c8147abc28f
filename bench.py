"""Benchmark of the DSA hot path on one MI355X.

Default workload: the 4-layer FSSS prefill stack at L = 200,000 (fp8 e4m3 indexer
inputs with per-row scales, H^I = 64 x d_I = 128, k = 2048; sparse MLA attention
with 128 heads over a [L, 576] bf16 latent), processed in 8192-query chunks
(chunked prefill: every layer of a chunk before the next chunk).  One step = one
indexcache_forward call over the whole stack: the F layer scores and selects,
all four layers attend.  Inputs are synthetic, seeded, and already resident in
HBM when the timed region starts; each layer's fp32 output goes to a ring of one
chunk (the next layer of a real model would consume it chunk by chunk).

Prints one JSON line.  `value` = queries per second through the whole step.
Per-launch durations come from HIP events that the library records around each
indexer / attention call on the stream it launches on, inside the timed steps.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "hbm": 8.0e12}   # MI355X dense MFMA, HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=4,
                    help="synthetic workload id (4 = L=200K FSSS fp8; 3 = decode B=8 over 47 layers)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement after the prefill line")
    ap.add_argument("--no-widened", action="store_true",
                    help="skip the projection / statistics / compressed-attention measurements")
    ap.add_argument("--widened-only", action="store_true", help="only print the widened rows' measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the L=32768 single-layer and L=65536 FSSSFSSS measurements after the headline")
    ap.add_argument("--L", type=int, default=None, help="override the context length (development only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-f", action="store_true", help="skip the all-F comparison step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device twice (scale for the HBM byte counters) and exit")
    return ap.parse_args()


class Hip:
    """Minimal HIP event plumbing (timing only)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for j in range(n):
            e = ctypes.c_void_p()
            assert self.h.hipEventCreate(ctypes.byref(e)) == 0
            arr[j] = e
        return arr

    def elapsed_ms(self, a, b) -> float:
        f = ctypes.c_float()
        assert self.h.hipEventSynchronize(b) == 0
        assert self.h.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return float(f.value)


def pairs_in_chunk(r0, r1, k):
    """Visible (query, key) pairs and selected pairs of query rows [r0, r1) of one sequence."""
    t = np.arange(r0, r1, dtype=np.float64)
    return float((t + 1).sum()), float(np.minimum(t + 1, k).sum())


def cpu_baseline(layers_host, roles, L, k, scale, seconds):
    """The oracle as it stands, timed on this host on a bounded sample of rows of the same stack.

    Rows are drawn uniformly over [0, L) so their mean cost matches the full
    workload's (the indexer cost of row t grows with t).  Returns queries/s."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    g = np.random.default_rng(1234)
    done, t0 = 0, time.perf_counter()
    keys = layers_host["keys"]
    while time.perf_counter() - t0 < seconds:
        t = int(g.integers(0, L))
        T = None
        for l, role in enumerate(roles):
            if role == "F":
                I = oracle.indexer_row(layers_host["q_idx"][l](t), layers_host["w"][l](t), keys[l][: t + 1])
                T = oracle.topk_row(I, k)[0]
            sel = T[T >= 0]
            lat = layers_host["latent"][l](sel)
            oracle.attn_row(layers_host["q"][l](t), lat, np.arange(sel.size), scale, 512)
        done += 1
    dt = time.perf_counter() - t0
    return done / dt, done, dt, threads


def blas_name() -> str:
    """The BLAS library NumPy (the oracle's matrix products) was built against."""
    try:
        b = np.__config__.CONFIG["Build Dependencies"]["blas"]
        return "%s %s" % (b.get("name", "?"), b.get("version", ""))
    except Exception:  # noqa: BLE001 (older NumPy: no machine-readable config)
        return "unknown"


def flush_infinity_cache(buf):
    """Read a 512 MiB device buffer: evicts the 256 MB Infinity Cache (and the L2s) so that a
    repetition does not start with the previous one's data cached.  A read leaves the cache
    holding clean lines; overwriting the buffer instead would leave up to 256 MB of dirty
    lines, written back to HBM while the next repetition's first kernels stream their own
    data (about 40 us more for one decode score pass)."""
    import torch

    buf.view(torch.int32).sum()


def run_prefill_config(wid: int, roles: str, steps: int, warmup: int, hip, all_f: bool) -> dict:
    """One prefill configuration timed through indexcache_forward: per-launch indexer and
    attention times from the library's events, fractions of the MFMA peak, and (all_f) the
    same stack with every layer F.  Work per launch as in the headline measurement."""
    import torch

    import dsa_indexer_indexcache_amd as dsa
    import synth

    wl = synth.WORKLOADS[wid]
    L, k, dev = wl.L, wl.k, "cuda"
    chunk = min(wl.q_chunk, 8192) if len(roles) > 1 else L
    need_idx = "F" * len(roles) if all_f else roles
    layers = [dsa.layer_dict(synth.workload_layer(wid, l, device=dev, with_indexer=need_idx[l] == "F"))
              for l in range(len(roles))]
    outs = [torch.empty((chunk, wl.n_h, 512), dtype=torch.float32, device=dev) for _ in roles]
    icache = torch.empty((chunk, k), dtype=torch.int32, device=dev)
    n_chunks = (L + chunk - 1) // chunk
    torch.cuda.synchronize()

    def timed(rl):
        n_calls = n_chunks * (len(rl) + rl.count("F"))
        ev = [hip.events(2 * n_calls) for _ in range(steps)]
        for _ in range(warmup):
            dsa.indexcache_forward(rl, layers, k, q_chunk=chunk, index_rows=chunk, out_rows=chunk, outs=outs,
                                   index_cache=icache)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        traces = [dsa.indexcache_forward(rl, layers, k, q_chunk=chunk, index_rows=chunk, out_rows=chunk, outs=outs,
                                         index_cache=icache, events=ev[s_]).trace for s_ in range(steps)]
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        ms = {0: 0.0, 1: 0.0}
        for s_, tr in enumerate(traces):
            for j, (kd, _, _) in enumerate(tr):
                ms[kd] += hip.elapsed_ms(ev[s_][2 * j], ev[s_][2 * j + 1])
        return 1e3 * wall, ms[0] / steps, ms[1] / steps

    step_ms, idx_ms, attn_ms = timed(roles)
    vis = sel = 0.0
    for c in range(n_chunks):
        v, s_ = pairs_in_chunk(c * chunk, min(L, (c + 1) * chunk), k)
        vis += v
        sel += s_
    idx_flops = 2.0 * wl.H * wl.d * vis * roles.count("F")
    attn_flops = wl.n_h * 2.0 * (576 + 512) * sel * len(roles)
    peak_i = PEAK["fp8" if wl.qk_dtype == "fp8" else "bf16"]
    res = {"workload": wl.name, "roles": roles, "q_chunk": chunk, "steps": steps, "step_ms": step_ms,
           "indexer_topk_ms": idx_ms, "indexer_tflops": idx_flops / (idx_ms * 1e-3) / 1e12,
           "indexer_frac": idx_flops / (idx_ms * 1e-3) / peak_i,
           "indexer_queries_per_s": L * roles.count("F") / (idx_ms * 1e-3),
           "sparse_attn_ms": attn_ms, "sparse_attn_tflops": attn_flops / (attn_ms * 1e-3) / 1e12,
           "sparse_attn_frac": attn_flops / (attn_ms * 1e-3) / PEAK["bf16"],
           "sparse_attn_tok_per_s": L * len(roles) / (attn_ms * 1e-3)}
    if all_f:
        f_step, f_idx, _ = timed("F" * len(roles))
        res.update({"all_f_step_ms": f_step, "all_f_indexer_topk_ms": f_idx,
                    "indexer_time_ratio_allF_over_pattern": f_idx / idx_ms,
                    "step_speedup_pattern_vs_allF": f_step / step_ms,
                    "indexer_work_saved": 1.0 - roles.count("F") / len(roles)})
    del layers, outs, icache
    torch.cuda.empty_cache()
    return res


def traffic_record(kernel_file: str, kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None.

    The summary (profiles/*_traffic.md) holds one JSON object per kernel and
    workload: FETCH_SIZE + WRITE_SIZE per dispatch, scaled by the same counters'
    reading for a plain copy of known size, and the sha256 of the kernel's source
    file at the time of the counter runs.  A changed source voids the figure.
    """
    import glob
    import hashlib
    src = os.path.join(ROOT, "dsa_indexer_indexcache_amd", "csrc", kernel_file)
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        for line in open(path):
            line = line.strip()
            if not line.startswith("{"):
                continue
            rec = json.loads(line)
            if rec.get("kernel") == kernel and rec.get("workload") == workload and rec.get("source_sha256") == digest:
                return rec
    return None


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 2}), flush=True)


def _time_ms(fn, reps: int = 10) -> float:
    """Mean device time of fn() over reps back-to-back calls on torch's current stream
    (the binding enqueues every library call on it)."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_widened_rows() -> dict:
    """The entry points beside the hot path, each at a shape of the pages' setting:
    indexer projections of one 8192-token chunk, the decode cache append, the attention
    statistics and indexer KL of one chunk, and compressed sparse attention (m = 4): the
    KV compression of 65,536 tokens and the compressed-block selection in prefill and decode."""
    import torch

    import dsa_indexer_indexcache_amd as dsa
    import synth
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    rnd = lambda *shape, div=1.0: (torch.randn(*shape, generator=g, device=dev) / div).to(torch.bfloat16)
    out = {}

    # indexer projections: q_lat [n, 1536] -> q [n, 64, 128] (RoPE 64), h [n, 7168] -> key
    # (LayerNorm, RoPE) and head weights; 2 n (r H d + hidden d + hidden H) flops
    n, r, hid, H, d = 8192, 1536, 7168, 64, 128
    q_lat, h = rnd(n, r), rnd(n, hid)
    wq, wk, ww = rnd(H * d, r, div=r ** 0.5), rnd(d, hid, div=hid ** 0.5), rnd(H, hid, div=hid ** 0.5)
    gam, bet = torch.ones(d, device=dev), torch.zeros(d, device=dev)
    pos = torch.arange(n, dtype=torch.int32, device=dev)
    qo = torch.empty((n, H, d), dtype=torch.bfloat16, device=dev)
    ko = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    wo = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    ms = _time_ms(lambda: dsa.indexer_project(q_lat, h, wq, wk, gam, bet, ww, pos, H, rope_dim=64, q_idx=qo,
                                              k_idx=ko, w=wo))
    fl = 2.0 * n * (r * H * d + hid * d + hid * H)
    out["indexer_project"] = {"n": n, "r": r, "hidden": hid, "H": H, "d": d, "rope_dim": 64, "ms": ms,
                              "tflops": fl / (ms * 1e-3) / 1e12, "frac_bf16_peak": fl / (ms * 1e-3) / PEAK["bf16"]}
    del q_lat, h, wq, wk, ww, qo, ko, wo

    # decode cache append: 8 new 1152-byte latent rows into a 1.6M-row packed cache
    cache = torch.empty((1_600_000, 576), dtype=torch.bfloat16, device=dev)
    rows = rnd(8, 576)
    dst = torch.arange(8, dtype=torch.int64, device=dev) * 200_000 + 199_000
    ms = _time_ms(lambda: dsa.cache_append(cache, dst, rows), reps=50)
    out["cache_append"] = {"rows": 8, "row_bytes": 1152, "us_per_launch": 1e3 * ms}
    del cache

    # attention statistics of the last 256 rows of a 32,768-token prefix (128 heads) and the
    # indexer KL of one 8192-row chunk over its selected lists (k = 2048).  A q.c product is
    # 2 x 576 flops per (row, head, key).  Captured mass + Recall@k: the dense log-sum-exp
    # needs one pass over the prefix and the head-aggregated weights p (for the dense top-k)
    # a second one, as p needs the finished log-sum-exp; plus one pass over S_t.  The KL:
    # a log-sum-exp pass and a weight pass over S_t.
    L, k = 32768, 2048
    li = synth.make_layer(L, L, 64, 128, 128, wid=1, layer=0, device=dev)
    rows_m = 256
    sq = dsa.Seqs.prefill(rows_m, n_k=L, q_pos0=L - rows_m)
    idx_m, _ = dsa.indexer_topk(li.q_idx[-rows_m:], li.k_idx, li.w[-rows_m:], k, sq)
    ms = _time_ms(lambda: dsa.attention_mass(li.q[-rows_m:], li.latent, idx_m, sq), reps=3)
    pairs = float(np.arange(L - rows_m + 1, L + 1).sum())
    fl = 2.0 * 576 * 128 * (2 * pairs + rows_m * k)
    out["attention_mass_recall"] = {"rows": rows_m, "prefix": L, "n_h": 128, "k": k, "ms": ms,
                                    "rows_per_s": rows_m / (ms * 1e-3), "tflops": fl / (ms * 1e-3) / 1e12,
                                    "frac_bf16_peak": fl / (ms * 1e-3) / PEAK["bf16"]}
    c0 = L - 8192
    sk = dsa.Seqs.prefill(8192, n_k=L, q_pos0=c0)
    idx_k, sc_k = dsa.indexer_topk(li.q_idx[c0:], li.k_idx, li.w[c0:], k, sk, want_scores=True)
    ms = _time_ms(lambda: dsa.indexer_kl(li.q[c0:], li.latent, idx_k, sc_k, sk), reps=3)
    fl = 2 * 2.0 * 576 * 128 * 8192 * k
    out["indexer_kl"] = {"rows": 8192, "k": k, "n_h": 128, "ms": ms, "tflops": fl / (ms * 1e-3) / 1e12,
                         "frac_bf16_peak": fl / (ms * 1e-3) / PEAK["bf16"]}
    del li, idx_m, idx_k, sc_k

    # CSA KV compression of 65,536 tokens (m = 4) for the 576-wide latent and the 128-wide
    # indexer key: reads C^a, Z^a of every token and C^b, Z^b of all but the last group
    # (2 B each), writes one bf16 entry per group
    m, n = 4, 65536
    csa = {}
    for c in (576, 128):
        ca, cb, za, zb = rnd(n, c), rnd(n, c), rnd(n, c), rnd(n, c)
        ba, bb = torch.zeros((m, c), device=dev), torch.zeros((m, c), device=dev)
        o = torch.empty((n // m, c), dtype=torch.bfloat16, device=dev)
        ms = _time_ms(lambda: dsa.csa_compress(ca, cb, za, zb, ba, bb, m, out=o), reps=20)
        nbytes = 2.0 * c * (2 * n + 2 * (n - m)) + 2.0 * c * (n // m)
        csa["compress_c%d" % c] = {"tokens": n, "m": m, "us": 1e3 * ms, "GBps": nbytes / (ms * 1e-3) / 1e9,
                                   "hbm_frac": nbytes / (ms * 1e-3) / PEAK["hbm"]}
        del ca, cb, za, zb, o

    # compressed-block selection, prefill: 65,536 query tokens over 16,384 blocks (fp8,
    # H = 64, d = 128, the CSA budget k = 1024); flops 2 H d per visible (query, block) pair
    kc = 1024
    li = synth.make_layer(n, n // m, 64, 128, 16, wid=4, layer=0, qk_dtype="fp8", device=dev, with_attention=False)
    sc = dsa.Seqs.compressed(n, m)
    for bf16s in (False, True):
        ms = _time_ms(lambda: dsa.indexer_topk(li.q_idx, li.k_idx, li.w, kc, sc, q_scale=li.q_scale,
                                               k_scale=li.k_scale, bf16_scores=bf16s), reps=3)
        pairs = float((np.arange(n) // m).sum())
        fl = 2.0 * 64 * 128 * pairs
        csa["select_prefill_%s" % ("bf16_scores" if bf16s else "fp32_scores")] = {
            "queries": n, "blocks": n // m, "k": kc, "ms": ms, "queries_per_s": n / (ms * 1e-3),
            "tflops": fl / (ms * 1e-3) / 1e12, "frac_fp8_peak": fl / (ms * 1e-3) / PEAK["fp8"]}
    del li

    # compressed-block selection, decode: B = 8 single queries over 150K-200K-token
    # contexts (37K-50K blocks each), and the recall of the fp32 selection by the bf16 one
    lens = synth.decode_lengths()
    nb = [int(x) // m for x in lens]
    li = synth.make_layer(8, int(np.sum(nb)), 64, 128, 16, wid=3, layer=0, qk_dtype="bf16", device=dev,
                          with_attention=False)
    sd = dsa.Seqs.varlen([1] * 8, nb, [int(x) - 1 for x in lens], block=m)
    kbytes = 2.0 * 128 * float(np.sum(nb))
    for kc in (512, 1024):
        i32 = torch.empty((8, kc), dtype=torch.int32, device=dev)
        i16 = torch.empty_like(i32)
        ms32 = _time_ms(lambda: dsa.indexer_topk(li.q_idx, li.k_idx, li.w, kc, sd, idx_out=i32), reps=20)
        ms16 = _time_ms(lambda: dsa.indexer_topk(li.q_idx, li.k_idx, li.w, kc, sd, idx_out=i16,
                                                 bf16_scores=True), reps=20)
        cnt = dsa.index_overlap(i16, i32).float()
        csa["select_decode_B8_k%d" % kc] = {"blocks": nb, "k": kc, "us_fp32_scores": 1e3 * ms32,
                                           "us_bf16_scores": 1e3 * ms16,
                                           "key_hbm_frac_fp32": kbytes / (ms32 * 1e-3) / PEAK["hbm"],
                                           "recall_of_fp32_selection_by_bf16": float((cnt / kc).mean())}
    out["csa"] = csa
    del li
    torch.cuda.synchronize()
    return out


def run_decode(steps: int, warmup: int, hip, all_f: bool = True) -> dict:
    """Decode step of the 47-layer stack: 8 sequences, one new query each, context
    lengths drawn from [150000, 200000]; every layer's caches resident in HBM."""
    import torch

    import dsa_indexer_indexcache_amd as dsa
    import synth

    wid = 3
    wl = synth.WORKLOADS[wid]
    lens = synth.decode_lengths(wid)
    seqs = dsa.Seqs.decode(lens)
    roles, k, dev = wl.roles, wl.k, "cuda"
    layers = [dsa.layer_dict(synth.decode_layer(l, lens, device=dev)) for l in range(len(roles))]
    B, n_keys = len(lens), int(np.sum(lens))
    outs = [torch.empty((B, wl.n_h, 512), dtype=torch.float32, device=dev) for _ in roles]
    index_cache = torch.empty((B, k), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    ws = None   # the workspace of the first call, reused by every later one

    def step(rl, events=None):
        nonlocal ws
        res = dsa.indexcache_forward(rl, layers, k, seqs=seqs, outs=outs, index_cache=index_cache, ws=ws,
                                     events=events)
        ws = res.ws
        return res

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def timed(rl, n_steps=steps):
        for _ in range(warmup):
            step(rl)
        n_ev = 2 * (len(rl) + rl.count("F"))
        evs = [hip.events(n_ev) for _ in range(n_steps)]
        traces, walls = [], []
        torch.cuda.synchronize()
        for s_ in range(n_steps):    # a decode step is one synchronous latency: time each
            flush_infinity_cache(flush)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            traces.append(step(rl, evs[s_]).trace)
            torch.cuda.synchronize()
            walls.append(1e3 * (time.perf_counter() - t0))
        ms = float(np.median(walls))
        kind = {0: [], 1: []}
        for s_, tr in enumerate(traces):
            for j, (kd, _, _) in enumerate(tr):
                kind[kd].append(hip.elapsed_ms(evs[s_][2 * j], evs[s_][2 * j + 1]))
        return ms, kind

    ms, kind = timed(roles)
    n_f = roles.count("F")
    idx_ms = float(np.mean(kind[0]))                     # one F layer: scores + selection
    attn_ms = float(np.mean(kind[1]))                    # one layer's sparse attention
    sel = int(np.sum(np.minimum(lens, k)))
    idx_bytes = n_keys * (2 * wl.d + 4 + 4) + B * wl.H * (2 * wl.d + 2)   # keys, score write + read, q, w
    attn_bytes = sel * 576 * 2 + B * wl.n_h * 576 * 2 + B * wl.n_h * 512 * 4 + B * k * 4
    res = {"workload": wl.name, "lens": [int(x) for x in lens], "roles": roles,
           "step_ms": ms, "steps": steps,
           "indexer_topk_ms_per_F_layer": idx_ms, "indexer_calls_per_step": len(kind[0]) // steps,
           "indexer_hbm_GBps": idx_bytes / (idx_ms * 1e-3) / 1e9,
           "indexer_hbm_frac": idx_bytes / (idx_ms * 1e-3) / PEAK["hbm"],
           "sparse_attn_ms_per_layer": attn_ms,
           "sparse_attn_hbm_GBps": attn_bytes / (attn_ms * 1e-3) / 1e9,
           "sparse_attn_hbm_frac": attn_bytes / (attn_ms * 1e-3) / PEAK["hbm"],
           "indexer_bytes_per_F_layer": idx_bytes, "attn_bytes_per_layer": attn_bytes,
           "indexer_work_saved": 1.0 - n_f / len(roles)}
    # the same step captured once as a HIP graph (no host work or launch gaps between the
    # 47 layers' kernels) and replayed; the library records no events inside the capture
    step(roles)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(roles)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(roles)
    torch.cuda.synchronize()
    gw = []
    for _ in range(max(steps, 5)):
        flush_infinity_cache(flush)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        gw.append(1e3 * (time.perf_counter() - t0))
    kern_ms = (idx_ms * n_f + attn_ms * len(roles))
    res.update({"graph_step_ms": float(np.median(gw)), "kernel_sum_ms": kern_ms,
                "graph_step_over_kernel_sum": float(np.median(gw)) / kern_ms})
    del graph
    if all_f:
        ms_f, kind_f = timed("F" * len(roles), max(3, min(steps, 5)))
        res.update({"all_f_step_ms": ms_f, "step_speedup_pattern_vs_allF": ms_f / ms,
                    "indexer_time_ratio_allF_over_pattern": float(np.mean(kind_f[0])) * len(roles)
                    / (float(np.mean(kind[0])) * n_f)})
    del layers, outs, flush
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch

    import dsa_indexer_indexcache_amd as dsa
    import synth

    wl = synth.WORKLOADS[args.workload]
    if args.widened_only:
        torch.cuda.init()
        dsa.lib()
        print(json.dumps({"widened": run_widened_rows()}), flush=True)
        return
    if wl.decode_B:
        torch.cuda.init()
        dsa.lib()
        d = run_decode(args.steps, args.warmup, Hip(), all_f=not args.no_all_f)
        print(json.dumps({
            "metric": "decode step latency (47 layers, B=8, 150K-200K context)", "value": d["step_ms"],
            "unit": "ms per decode step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": d["step_ms"], "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16, fp32 accumulate", "data": "synthetic (seeded)",
            "config": {"workload": wl.name, "B": wl.decode_B, "k": wl.k, "roles": wl.roles},
            "decode": d}), flush=True)
        return
    L = wl.L if args.L is None else args.L
    roles, k, dev = wl.roles, wl.k, "cuda"
    chunk = min(wl.q_chunk, L)
    torch.cuda.init()
    dsa.lib()

    layers = []
    for l in range(len(roles)):
        li = synth.workload_layer(args.workload, l, device=dev, L=L)
        layers.append(li)
    torch.cuda.synchronize()
    n_chunks = (L + chunk - 1) // chunk
    outs = [torch.empty((chunk, wl.n_h, 512), dtype=torch.float32, device=dev) for _ in roles]
    index_cache = torch.empty((chunk, k), dtype=torch.int32, device=dev)
    ldicts = [dsa.layer_dict(x) for x in layers]
    hip = Hip()
    n_calls = n_chunks * len(roles) + n_chunks * roles.count("F")
    ev_steps = [hip.events(2 * n_calls) for _ in range(args.steps)]   # read only after the timed region

    def step(rl, events=None):
        return dsa.indexcache_forward(rl, ldicts, k, q_chunk=chunk, index_rows=chunk, out_rows=chunk,
                                      outs=outs, index_cache=index_cache, events=events)

    for _ in range(args.warmup):
        step(roles)
    torch.cuda.synchronize()

    kind_ms = {0: [], 1: []}
    traces = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        traces.append(step(roles, ev_steps[s_]).trace)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    for s_, tr in enumerate(traces):
        evs = ev_steps[s_]
        for j, (kind, layer, ch) in enumerate(tr):
            kind_ms[kind].append((ch, hip.elapsed_ms(evs[2 * j], evs[2 * j + 1])))

    # algorithmic work per chunk
    qk_flops_pair = 2.0 * wl.H * wl.d
    attn_flops_pair = wl.n_h * 2.0 * (576 + 512)
    idx_ms = sum(ms for _, ms in kind_ms[0]) / args.steps
    attn_ms = sum(ms for _, ms in kind_ms[1]) / args.steps
    idx_flops = attn_flops = 0.0
    for c in range(n_chunks):
        vis, sel = pairs_in_chunk(c * chunk, min(L, (c + 1) * chunk), k)
        idx_flops += qk_flops_pair * vis * roles.count("F")
        attn_flops += attn_flops_pair * sel * len(roles)
    idx_peak = PEAK["fp8" if wl.qk_dtype == "fp8" else "bf16"]
    idx_tfs = idx_flops / (idx_ms * 1e-3) / 1e12
    attn_tfs = attn_flops / (attn_ms * 1e-3) / 1e12
    comp = {
        "indexer_topk": {"ms_per_step": idx_ms, "launches_per_step": len(kind_ms[0]) // args.steps,
                         "queries_per_s": L * roles.count("F") / (idx_ms * 1e-3),
                         "achieved_tflops": idx_tfs, "peak_tflops": idx_peak / 1e12,
                         "frac": idx_tfs * 1e12 / idx_peak},
        "sparse_attn": {"ms_per_step": attn_ms, "launches_per_step": len(kind_ms[1]) // args.steps,
                        "tok_per_s": L * len(roles) / (attn_ms * 1e-3),
                        "achieved_tflops": attn_tfs, "peak_tflops": PEAK["bf16"] / 1e12,
                        "frac": attn_tfs * 1e12 / PEAK["bf16"]},
    }
    dom = "sparse_attn" if attn_ms >= idx_ms else "indexer_topk"
    dc = comp[dom]
    launches = dc["launches_per_step"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": dc["achieved_tflops"], "peak": dc["peak_tflops"],
                "unit": "TFLOP/s", "frac": dc["frac"], "traffic": None,
                "avg_launch_ms": dc["ms_per_step"] / max(launches, 1),
                "work_per_launch_tflop": (attn_flops if dom == "sparse_attn" else idx_flops) / max(launches, 1) / 1e12}
    if dom == "sparse_attn" and args.L is None:
        rec = traffic_record("sparse_attn.hip", "sparse_attn_pair2_kernel", wl.name)
        if rec is not None:
            roofline["traffic"] = rec["hbm_bytes_per_launch"]
            roofline["traffic_source"] = rec["summary"]

    # cross-layer overlap diagnostic at the chunk shape: the step's index cache against
    # a row-rotated copy of itself (reads 2 x rows x k x 4 B, writes 4 B per row)
    other = torch.roll(index_cache, 1, dims=0).contiguous()
    counts = dsa.index_overlap(index_cache, other)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dsa.index_overlap(index_cache, other, counts=counts)
    e1.record()
    torch.cuda.synchronize()
    ov_ms = e0.elapsed_time(e1) / reps
    ov_bytes = 2.0 * index_cache.numel() * 4 + index_cache.shape[0] * 4
    overlap_line = {"rows": int(index_cache.shape[0]), "k": k, "us_per_launch": 1e3 * ov_ms,
                    "hbm_GBps": ov_bytes / (ov_ms * 1e-3) / 1e9, "hbm_frac": ov_bytes / (ov_ms * 1e-3) / PEAK["hbm"]}
    del other, counts

    # device fp8 quantisation of one chunk's indexer queries ([chunk, H, d] bf16 ->
    # e4m3fn codes + per-(row, head) scales): reads 2 B and writes 1 B per element,
    # writes 4 B per (row, head)
    qx = torch.randn((chunk, wl.H, wl.d), device=dev).to(torch.bfloat16)
    qc, qsc = dsa.quantize_fp8_rows(qx)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dsa.quantize_fp8_rows(qx, codes=qc, scales=qsc)
    e1.record()
    torch.cuda.synchronize()
    qz_ms = e0.elapsed_time(e1) / reps
    qz_bytes = 3.0 * qx.numel() + 4.0 * qsc.numel()
    quant_line = {"shape": [chunk, wl.H, wl.d], "us_per_launch": 1e3 * qz_ms,
                  "hbm_GBps": qz_bytes / (qz_ms * 1e-3) / 1e9, "hbm_frac": qz_bytes / (qz_ms * 1e-3) / PEAK["hbm"]}
    del qx, qc, qsc

    extra = {}
    if not args.no_all_f and "S" in roles:
        allf = "F" * len(roles)
        step(allf)
        torch.cuda.synchronize()
        walls, idxs = [], []
        for _ in range(3):           # three all-F steps; medians
            ev_allf = hip.events(2 * n_chunks * 2 * len(roles))
            t1 = time.perf_counter()
            res = step(allf, ev_allf)
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t1)
            idxs.append(sum(hip.elapsed_ms(ev_allf[2 * j], ev_allf[2 * j + 1])
                            for j, (kd, _, _) in enumerate(res.trace) if kd == 0))
        t_allf, idx_allf = float(np.median(walls)), float(np.median(idxs))
        extra = {"all_f_ms_per_step": 1e3 * t_allf, "all_f_indexer_ms": idx_allf, "all_f_steps": 3,
                 "indexer_time_ratio_allF_over_pattern": idx_allf / idx_ms,
                 "step_speedup_pattern_vs_allF": 1e3 * t_allf / ms_step,
                 "indexer_work_saved": 1.0 - roles.count("F") / len(roles)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from oracle import formats

        def deq_rows(t, s, rows):
            r = torch.as_tensor(np.atleast_1d(rows), device=dev)
            if t.dtype == torch.float8_e4m3fn:
                return formats.dequant_rows(synth.bits(t[r]), synth.bits(s[r]), "fp8")
            return formats.decode_bf16(synth.bits(t[r]))

        host = {"keys": [], "q_idx": [], "w": [], "q": [], "latent": []}
        for l, li in enumerate(layers):
            if roles[l] == "F":
                kk = li.k_idx
                host["keys"].append(formats.dequant_rows(synth.bits(kk), synth.bits(li.k_scale), "fp8")
                                    if kk.dtype == torch.float8_e4m3fn else formats.decode_bf16(synth.bits(kk)))
            else:
                host["keys"].append(None)
            host["q_idx"].append(lambda t, li=li: deq_rows(li.q_idx, li.q_scale, t)[0])
            host["w"].append(lambda t, li=li: formats.decode_bf16(synth.bits(li.w[t:t + 1]))[0])
            host["q"].append(lambda t, li=li: formats.decode_bf16(synth.bits(li.q[t:t + 1]))[0])
            lat_bits = synth.bits(li.latent)      # host copy before timing: the oracle reads host memory
            host["latent"].append(lambda rows, b=lat_bits: formats.decode_bf16(b[rows]))
        qps, nrows, secs, threads = cpu_baseline(host, roles, L, k, wl.scale, args.cpu_seconds)
        cpu = {"value": qps, "unit": "queries/s", "cores": threads, "kind": "oracle", "blas": blas_name(),
               "sample": "%d query rows drawn uniformly over [0, %d) through the %s stack (fp64 NumPy indexer, "
                         "sort top-k, sparse attention), %.1f s" % (nrows, L, roles, secs)}

    del layers, ldicts, outs, index_cache
    torch.cuda.empty_cache()
    cfg1 = cfg2 = dec = None
    if not args.no_configs and args.L is None:
        cfg1 = run_prefill_config(1, "F", 5, 1, hip, all_f=False)
        cfg2 = run_prefill_config(2, synth.WORKLOADS[2].roles, 3, 1, hip, all_f=not args.no_all_f)
    if not args.no_decode and args.L is None:
        dec = run_decode(max(args.steps, 3), 1, hip, all_f=not args.no_all_f)

    line = {
        "metric": "indexer+top-k queries/s & sparse-attn tok/s at L=200K; % MFMA/HBM peak",
        "value": L / (ms_step * 1e-3),
        "unit": "queries/s (whole %s step)" % roles,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 indexer / bf16 attention, fp32 accumulate" if wl.qk_dtype == "fp8" else "bf16, fp32 accumulate",
        "data": "synthetic (seeded, shapes of the DSA/IndexCache pages' 200K-context setting)",
        "config": {"workload": wl.name, "L": L, "roles": roles, "k": k, "H_idx": wl.H, "d_idx": wl.d,
                   "n_h": wl.n_h, "q_chunk": chunk, "parallelism": "single GPU"},
        "components": comp,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    line.update(extra)
    line["index_overlap"] = overlap_line
    line["quantize_fp8_rows"] = quant_line
    line["prefill_L32768_bf16"] = cfg1
    line["prefill_L65536_fsssfsss"] = cfg2
    line["decode"] = dec
    line["widened"] = None if args.no_widened else run_widened_rows()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
