// C ABI of the DSA hot path: argument validation, workspace sizing, the IndexCache
// layer loop, and dispatch to the kernels.  Host code only (compiled by hipcc).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Checks the sequence table; returns the packed query and key row counts.
int check_seqs(const dsa_seqs* s, int64_t* n_q, int64_t* n_k) {
  if (!s) return fail(DSA_ERR_INVALID_ARG, "seqs is NULL");
  if (s->B < 1 || s->B > DSA_MAX_B) return fail(DSA_ERR_INVALID_ARG, "seqs->B=%d outside [1,%d]", s->B, DSA_MAX_B);
  if (s->q_start[0] != 0) return fail(DSA_ERR_INVALID_ARG, "seqs->q_start[0] must be 0");
  if (s->k_start[0] < 0) return fail(DSA_ERR_INVALID_ARG, "seqs->k_start[0] < 0");
  if (s->block < 0 || s->block > (1 << 20)) return fail(DSA_ERR_INVALID_ARG, "seqs->block=%d", s->block);
  for (int b = 0; b < s->B; ++b) {
    const int64_t nq = s->q_start[b + 1] - s->q_start[b];
    const int64_t nk = s->k_start[b + 1] - s->k_start[b];
    if (nq < 0 || nk < 0) return fail(DSA_ERR_INVALID_ARG, "sequence %d: decreasing row offsets", b);
    if (s->q_pos0[b] < 0) return fail(DSA_ERR_INVALID_ARG, "sequence %d: q_pos0 < 0", b);
    const int64_t need = s->block > 1 ? (s->q_pos0[b] + nq - 1) / s->block : s->q_pos0[b] + nq;
    if (nq > 0 && need > nk)
      return fail(DSA_ERR_INVALID_ARG, "sequence %d: last query position %lld needs %lld keys, has %lld", b,
                  (long long)(s->q_pos0[b] + nq - 1), (long long)need, (long long)nk);
    if (s->q_pos0[b] + nq > (int64_t)INT32_MAX)
      return fail(DSA_ERR_INVALID_ARG, "sequence %d: positions exceed int32", b);
  }
  *n_q = s->q_start[s->B];
  *n_k = s->k_start[s->B];
  return DSA_OK;
}

int heads_supported(int H) { return H >= 1 && H <= 64; }

dsa::IndexerArgs shape_args(int qk_dtype, int H, int d, int k, const dsa_seqs& s) {
  dsa::IndexerArgs a{};
  a.qk_dtype = qk_dtype;
  a.H = H;
  a.d = d;
  a.k = k;
  a.seqs = s;
  return a;
}

// The fused kernel needs no workspace; the slab path keeps one fp32 score per visible pair of a row.
size_t indexer_ws(int64_t n_q, const dsa_seqs& s, int qk_dtype, int H, int d, int k) {
  const dsa::IndexerArgs a = shape_args(qk_dtype, H, d, k, s);
  if (n_q == 0 || dsa::indexer_fused_ok(a)) return 0;
  const size_t slab = (size_t)n_q * (size_t)dsa::slab_ld(s) * sizeof(float) + 256;
  return dsa::wide_select_ok(a) ? slab + dsa::wide_select_ws(a) : slab;
}

int check_indexer(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                  const uint16_t* w, int qk_dtype, int H, int d, int k, int64_t n_q) {
  if (k < 1) return fail(DSA_ERR_INVALID_ARG, "k=%d < 1", k);
  if (qk_dtype != DSA_BF16 && qk_dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "indexer dtype %d not supported", qk_dtype);
  if (!heads_supported(H)) return fail(DSA_ERR_UNSUPPORTED, "indexer heads H=%d not in [1,64]", H);
  if (d != 64 && d != 128) return fail(DSA_ERR_UNSUPPORTED, "indexer head dim d=%d not in {64,128}", d);
  if (qk_dtype == DSA_FP8_E4M3 && d != 128) return fail(DSA_ERR_UNSUPPORTED, "fp8 indexer needs d=128");
  if (n_q == 0) return DSA_OK;
  if (!q_idx || !k_idx || !w) return fail(DSA_ERR_INVALID_ARG, "q_idx, k_idx and w are required");
  if (qk_dtype == DSA_FP8_E4M3 && (!q_scale || !k_scale))
    return fail(DSA_ERR_INVALID_ARG, "fp8 indexer needs q_scale and k_scale");
  if (qk_dtype == DSA_BF16 && (q_scale || k_scale))
    return fail(DSA_ERR_INVALID_ARG, "bf16 indexer takes no scales");
  if (!aligned16(q_idx) || !aligned16(k_idx)) return fail(DSA_ERR_ALIGNMENT, "q_idx/k_idx not 16-byte aligned");
  if (((uintptr_t)w & 1u) || ((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u))
    return fail(DSA_ERR_ALIGNMENT, "w/scales misaligned");
  return DSA_OK;
}

// The attention gather addresses a latent row by a 32-bit byte offset from its sequence's
// first row: at most (2^32 - 4096) / 1152 rows per sequence.
constexpr int64_t kMaxLatentRows = (((int64_t)1 << 32) - 4096) / 1152;

int check_latent_rows(const dsa_seqs* s) {
  for (int b = 0; b < s->B; ++b)
    if (s->k_start[b + 1] - s->k_start[b] > kMaxLatentRows)
      return fail(DSA_ERR_UNSUPPORTED, "sequence %d has %lld latent rows (at most %lld per sequence)", b,
                  (long long)(s->k_start[b + 1] - s->k_start[b]), (long long)kMaxLatentRows);
  return DSA_OK;
}

int check_attn(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int d_qk, int d_v, int k,
               void* out, int out_dtype, int64_t n_q) {
  if (k < 1) return fail(DSA_ERR_INVALID_ARG, "k=%d < 1", k);
  if (d_v > d_qk) return fail(DSA_ERR_INVALID_ARG, "d_v=%d > d_qk=%d", d_v, d_qk);
  if (n_h != 16 && n_h != 32 && n_h != 64 && n_h != 128)
    return fail(DSA_ERR_UNSUPPORTED, "n_h=%d not in {16,32,64,128}", n_h);
  if (d_qk != 576 || d_v != 512) return fail(DSA_ERR_UNSUPPORTED, "needs d_qk=576, d_v=512 (got %d, %d)", d_qk, d_v);
  if (out_dtype != DSA_FP32 && out_dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "out dtype %d not supported", out_dtype);
  if (n_q == 0) return DSA_OK;
  if (!q || !latent || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "q, latent, idx and out are required");
  if (!aligned16(q) || !aligned16(latent) || !aligned16(out) || ((uintptr_t)idx & 3u))
    return fail(DSA_ERR_ALIGNMENT, "q/latent/out not 16-byte aligned or idx misaligned");
  return DSA_OK;
}

dsa::IndexerArgs indexer_args(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                              const uint16_t* w, int qk_dtype, int H, int d, int k, const dsa_seqs& s,
                              int32_t* idx_out, float* score_out) {
  dsa::IndexerArgs a;
  a.q_idx = q_idx;
  a.q_scale = q_scale;
  a.k_idx = k_idx;
  a.k_scale = k_scale;
  a.w = w;
  a.qk_dtype = qk_dtype;
  a.H = H;
  a.d = d;
  a.k = k;
  a.seqs = s;
  a.idx_out = idx_out;
  a.score_out = score_out;
  a.flags = 0;
  return a;
}

int run_indexer(const dsa::IndexerArgs& a, void* ws, hipStream_t st) {
  if (dsa::indexer_fused_ok(a)) {
    hipError_t e = dsa::launch_indexer_fused(a, st);
    if (e != hipSuccess) return hip_fail(e, "fused indexer launch");
    return DSA_OK;
  }
  float* slab = (float*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  const bool wide = dsa::wide_select_ok(a);
  void* state = slab + a.seqs.q_start[a.seqs.B] * dsa::slab_ld(a.seqs);
  uint32_t* zero = nullptr;
  int64_t zero_words = 0;
  if (wide) dsa::wide_select_zero_region(a, state, &zero, &zero_words);
  hipError_t e = dsa::launch_indexer_slab(a, slab, st, zero, zero_words);
  if (e != hipSuccess) return hip_fail(e, "indexer score launch");
  if (wide)
    e = dsa::launch_wide_select(a, slab, state, st);
  else
    e = dsa::launch_topk_select(a, slab, st);
  if (e != hipSuccess) return hip_fail(e, "top-k select launch");
  return DSA_OK;
}

dsa::AttnArgs attn_args(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int d_qk, int d_v,
                        int k, float scale, const dsa_seqs& s, void* out, int out_dtype) {
  dsa::AttnArgs a;
  a.q = q;
  a.latent = latent;
  a.idx = idx;
  a.n_h = n_h;
  a.d_qk = d_qk;
  a.d_v = d_v;
  a.k = k;
  a.scale = scale;
  a.seqs = s;
  a.out = out;
  a.out_dtype = out_dtype;
  return a;
}

// Sequence table of the packed query rows [r0, r1).
dsa_seqs slice_seqs(const dsa_seqs& s, int64_t r0, int64_t r1) {
  dsa_seqs o;
  memset(&o, 0, sizeof o);
  int nb = 0;
  for (int b = 0; b < s.B; ++b) {
    const int64_t a0 = s.q_start[b] > r0 ? s.q_start[b] : r0;
    const int64_t a1 = s.q_start[b + 1] < r1 ? s.q_start[b + 1] : r1;
    if (a1 <= a0) continue;
    o.q_start[nb] = a0 - r0;
    o.q_start[nb + 1] = a1 - r0;
    o.k_start[nb] = s.k_start[b];
    o.k_start[nb + 1] = s.k_start[b + 1];
    o.q_pos0[nb] = s.q_pos0[b] + (a0 - s.q_start[b]);
    ++nb;
  }
  if (nb == 0) {  // empty range: one empty sequence
    o.q_start[0] = o.q_start[1] = 0;
    o.k_start[0] = o.k_start[1] = s.k_start[0];
    nb = 1;
  }
  o.B = nb;
  o.block = s.block;
  return o;
}

size_t elt_size(int dtype) { return dtype == DSA_FP8_E4M3 ? 1 : dtype == DSA_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int dsa_version(void) { return 101; }

int dsa_quantize_fp8_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, float* scales, void* stream) {
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "rows=%lld < 0", (long long)rows);
  if (rows > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "rows=%lld > 2^31 - 1", (long long)rows);
  if (cols < 1 || cols > 65536) return fail(DSA_ERR_UNSUPPORTED, "cols=%d outside [1, 65536]", cols);
  if (rows == 0) return DSA_OK;
  if (!x || !codes || !scales) return fail(DSA_ERR_INVALID_ARG, "null pointer");
  hipError_t e = dsa::launch_quantize_fp8_rows(x, rows, cols, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 quantisation launch");
  return DSA_OK;
}

int dsa_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t n_rows, int k, int32_t* counts,
                      void* stream) {
  if (n_rows < 0) return fail(DSA_ERR_INVALID_ARG, "n_rows=%lld < 0", (long long)n_rows);
  if (k < 1 || k > dsa::kOverlapMaxK) return fail(DSA_ERR_UNSUPPORTED, "k=%d outside [1, %d]", k, dsa::kOverlapMaxK);
  if (n_rows > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "n_rows=%lld > 2^31 - 1", (long long)n_rows);
  if (n_rows == 0) return DSA_OK;
  if (!idx_a || !idx_b || !counts) return fail(DSA_ERR_INVALID_ARG, "null pointer");
  hipError_t e = dsa::launch_index_overlap(idx_a, idx_b, n_rows, k, counts, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "index overlap launch");
  return DSA_OK;
}

int dsa_indexer_project(const uint16_t* q_lat, const uint16_t* h, const uint16_t* wq, const uint16_t* wk,
                        const float* ln_weight, const float* ln_bias, const uint16_t* ww, const int32_t* pos, int64_t n,
                        int r, int hidden, int H, int d, int rope_dim, float rope_base, float eps, uint16_t* q_idx,
                        uint16_t* k_idx, uint16_t* w, void* stream) {
  if (n < 0) return fail(DSA_ERR_INVALID_ARG, "n=%lld < 0", (long long)n);
  if (d != 128) return fail(DSA_ERR_UNSUPPORTED, "indexer head dim d=%d: only 128 is compiled", d);
  if (H < 1 || H > 128) return fail(DSA_ERR_UNSUPPORTED, "indexer heads H=%d outside [1, 128]", H);
  if (rope_dim != 0 && rope_dim != 32 && rope_dim != 64)
    return fail(DSA_ERR_UNSUPPORTED, "rope_dim=%d not in {0, 32, 64}", rope_dim);
  if (r < 64 || r % 64 || hidden < 64 || hidden % 64)
    return fail(DSA_ERR_UNSUPPORTED, "r=%d and hidden=%d must be positive multiples of 64", r, hidden);
  if (!(rope_base > 1.f) || !(eps >= 0.f)) return fail(DSA_ERR_INVALID_ARG, "rope_base must exceed 1, eps >= 0");
  if (n > (int64_t)INT32_MAX * 64) return fail(DSA_ERR_UNSUPPORTED, "n=%lld too large", (long long)n);
  if (n == 0) return DSA_OK;
  if (!q_lat || !h || !wq || !wk || !ln_weight || !ln_bias || !ww || !pos || !q_idx || !k_idx || !w)
    return fail(DSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q_lat) || !aligned16(h) || !aligned16(wq) || !aligned16(wk) || !aligned16(ww) ||
      !aligned16(q_idx) || !aligned16(k_idx))
    return fail(DSA_ERR_ALIGNMENT, "q_lat, h, the weights, q_idx and k_idx must be 16-byte aligned");
  if (((uintptr_t)w & 1u) || ((uintptr_t)pos & 3u) || ((uintptr_t)ln_weight & 3u) || ((uintptr_t)ln_bias & 3u))
    return fail(DSA_ERR_ALIGNMENT, "w, pos or the LayerNorm parameters misaligned");
  dsa::ProjectArgs a{q_lat, h, wq, wk, ln_weight, ln_bias, ww, pos, n, r, hidden, H, rope_dim, rope_base, eps,
                     q_idx, k_idx, w};
  hipError_t e = dsa::launch_indexer_project(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "indexer projection launch");
  return DSA_OK;
}

int dsa_cache_append(void* cache, int64_t cache_rows, const int64_t* dst_row, const void* rows, int64_t n_rows,
                     int64_t row_bytes, void* stream) {
  if (n_rows < 0 || cache_rows < 0 || row_bytes < 1) return fail(DSA_ERR_INVALID_ARG, "negative size");
  if (n_rows > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "n_rows=%lld > 2^31 - 1", (long long)n_rows);
  if (n_rows == 0) return DSA_OK;
  if (!cache || !dst_row || !rows) return fail(DSA_ERR_INVALID_ARG, "null pointer");
  if ((uintptr_t)dst_row & 7u) return fail(DSA_ERR_ALIGNMENT, "dst_row misaligned");
  hipError_t e = dsa::launch_cache_append(cache, cache_rows, dst_row, rows, n_rows, row_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cache append launch");
  return DSA_OK;
}

int dsa_csa_compress(const uint16_t* ca, const uint16_t* cb, const uint16_t* za, const uint16_t* zb,
                     const float* ba, const float* bb, int64_t n, int c, int m, int64_t block0, void* out,
                     int out_dtype, void* stream) {
  if (n < 0 || block0 < 0) return fail(DSA_ERR_INVALID_ARG, "n=%lld block0=%lld", (long long)n, (long long)block0);
  if (c < 8 || c % 8) return fail(DSA_ERR_UNSUPPORTED, "c=%d is not a positive multiple of 8", c);
  if (m < 1 || m > 4096) return fail(DSA_ERR_UNSUPPORTED, "m=%d outside 1..4096", m);
  if (out_dtype != DSA_FP32 && out_dtype != DSA_BF16) return fail(DSA_ERR_INVALID_ARG, "out_dtype=%d", out_dtype);
  const int64_t n_out = n / m - block0;
  if (n_out <= 0) return DSA_OK;
  if (n_out * (c / 8) > ((int64_t)UINT32_MAX) * 256 / 2)
    return fail(DSA_ERR_UNSUPPORTED, "%lld entries of %d columns exceed one launch", (long long)n_out, c);
  if (!ca || !cb || !za || !zb || !ba || !bb || !out) return fail(DSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(ca) || !aligned16(cb) || !aligned16(za) || !aligned16(zb) || !aligned16(ba) || !aligned16(bb) ||
      !aligned16(out))
    return fail(DSA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  dsa::CsaArgs a;
  a.ca = ca;
  a.cb = cb;
  a.za = za;
  a.zb = zb;
  a.ba = ba;
  a.bb = bb;
  a.n = n;
  a.block0 = block0;
  a.c = c;
  a.m = m;
  a.out = out;
  a.out_dtype = out_dtype;
  hipError_t e = dsa::launch_csa_compress(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "csa compress launch");
  return DSA_OK;
}

static int check_stats(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int d_qk, int k,
                       int64_t n_q) {
  if (k < 1) return fail(DSA_ERR_INVALID_ARG, "k=%d < 1", k);
  if (n_h != 16 && n_h != 32 && n_h != 64 && n_h != 128)
    return fail(DSA_ERR_UNSUPPORTED, "n_h=%d not in {16,32,64,128}", n_h);
  if (d_qk != 576) return fail(DSA_ERR_UNSUPPORTED, "needs d_qk=576 (got %d)", d_qk);
  if (k > 2048) return fail(DSA_ERR_UNSUPPORTED, "k=%d > 2048", k);
  if (n_q == 0) return DSA_OK;
  if (!q || !latent || !idx) return fail(DSA_ERR_INVALID_ARG, "q, latent and idx are required");
  if (!aligned16(q) || !aligned16(latent) || ((uintptr_t)idx & 3u))
    return fail(DSA_ERR_ALIGNMENT, "q/latent not 16-byte aligned or idx misaligned");
  return DSA_OK;
}

static dsa::StatArgs stat_args(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int k,
                               float scale, const dsa_seqs& s) {
  dsa::StatArgs a;
  a.q = q;
  a.latent = latent;
  a.idx = idx;
  a.n_h = n_h;
  a.k = k;
  a.scale = scale;
  a.seqs = s;
  return a;
}

size_t dsa_attention_mass_ws(int n_h, int k, const dsa_seqs* seqs, int want_recall) {
  int64_t n_q, n_k;
  if (check_seqs(seqs, &n_q, &n_k) != DSA_OK) return 0;
  return dsa::attn_mass_ws(stat_args(nullptr, nullptr, nullptr, n_h, k, 1.f, *seqs), want_recall != 0);
}

int dsa_attention_mass(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int d_qk, int k,
                       float scale, const dsa_seqs* seqs, float* mass_head, float* mass, float* recall, void* ws,
                       size_t ws_bytes, void* stream) {
  int64_t n_q, n_k;
  int rc = check_seqs(seqs, &n_q, &n_k);
  if (rc) return rc;
  rc = check_stats(q, latent, idx, n_h, d_qk, k, n_q);
  if (rc) return rc;
  if (n_q == 0) return DSA_OK;
  if (!mass) return fail(DSA_ERR_INVALID_ARG, "mass is required");
  if (((uintptr_t)mass & 3u) || ((uintptr_t)mass_head & 3u) || ((uintptr_t)recall & 3u))
    return fail(DSA_ERR_ALIGNMENT, "outputs misaligned");
  const dsa::StatArgs a = stat_args(q, latent, idx, n_h, k, scale, *seqs);
  const size_t need = dsa::attn_mass_ws(a, recall != nullptr);
  if (ws_bytes < need || !ws) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipError_t e = dsa::launch_attention_mass(a, mass_head, mass, recall, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention mass launch");
  return DSA_OK;
}

size_t dsa_indexer_kl_ws(int n_h, int k, const dsa_seqs* seqs) {
  int64_t n_q, n_k;
  if (check_seqs(seqs, &n_q, &n_k) != DSA_OK) return 0;
  return dsa::indexer_kl_ws(stat_args(nullptr, nullptr, nullptr, n_h, k, 1.f, *seqs));
}

int dsa_indexer_kl(const uint16_t* q, const uint16_t* latent, const int32_t* idx, const float* scores, int n_h,
                   int d_qk, int k, float scale, const dsa_seqs* seqs, float weight, int accumulate, float* kl,
                   float* loss, void* ws, size_t ws_bytes, void* stream) {
  int64_t n_q, n_k;
  int rc = check_seqs(seqs, &n_q, &n_k);
  if (rc) return rc;
  rc = check_stats(q, latent, idx, n_h, d_qk, k, n_q);
  if (rc) return rc;
  if (n_q == 0) return DSA_OK;
  if (!scores || !kl) return fail(DSA_ERR_INVALID_ARG, "scores and kl are required");
  if (((uintptr_t)scores & 3u) || ((uintptr_t)kl & 3u) || ((uintptr_t)loss & 3u))
    return fail(DSA_ERR_ALIGNMENT, "scores/kl/loss misaligned");
  const dsa::StatArgs a = stat_args(q, latent, idx, n_h, k, scale, *seqs);
  const size_t need = dsa::indexer_kl_ws(a);
  if (ws_bytes < need || !ws) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipError_t e = dsa::launch_indexer_kl(a, scores, weight, accumulate, kl, loss, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "indexer KL launch");
  return DSA_OK;
}

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_ROLES: return "invalid role string";
    case DSA_ERR_FIRST_NOT_F: return "first layer must be F";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DSA_ERR_ALIGNMENT: return "misaligned pointer";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

int indexcache_plan(const char* roles, int32_t* src_layer, int32_t* n_indexer_calls) {
  if (!roles || roles[0] == '\0') return fail(DSA_ERR_ROLES, "empty role string");
  const size_t n = strlen(roles);
  if (n > DSA_MAX_LAYERS) return fail(DSA_ERR_ROLES, "%zu layers > %d", n, DSA_MAX_LAYERS);
  for (size_t l = 0; l < n; ++l)
    if (roles[l] != 'F' && roles[l] != 'S') return fail(DSA_ERR_ROLES, "role %zu is '%c', not F or S", l, roles[l]);
  if (roles[0] != 'F') return fail(DSA_ERR_FIRST_NOT_F, "first layer is '%c'", roles[0]);
  int32_t last = -1, calls = 0;
  for (size_t l = 0; l < n; ++l) {
    if (roles[l] == 'F') {
      last = (int32_t)l;
      ++calls;
    }
    if (src_layer) src_layer[l] = last;
  }
  if (n_indexer_calls) *n_indexer_calls = calls;
  return DSA_OK;
}

size_t dsa_indexer_topk_ws(int qk_dtype, int H, int d, int k, const dsa_seqs* seqs) {
  int64_t n_q, n_k;
  if (check_seqs(seqs, &n_q, &n_k) != DSA_OK) return 0;
  return indexer_ws(n_q, *seqs, qk_dtype, H, d, k);
}

int dsa_indexer_topk(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                     const uint16_t* w, int qk_dtype, int H, int d, int k, const dsa_seqs* seqs, int32_t* idx_out,
                     float* score_out, void* ws, size_t ws_bytes, void* stream) {
  return dsa_indexer_topk_ex(q_idx, q_scale, k_idx, k_scale, w, qk_dtype, H, d, k, seqs, idx_out, score_out, ws,
                             ws_bytes, 0, stream);
}

int dsa_indexer_topk_ex(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                        const uint16_t* w, int qk_dtype, int H, int d, int k, const dsa_seqs* seqs, int32_t* idx_out,
                        float* score_out, void* ws, size_t ws_bytes, int flags, void* stream) {
  if (flags & ~DSA_TOPK_BF16_SCORES) return fail(DSA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  int64_t n_q, n_k;
  int rc = check_seqs(seqs, &n_q, &n_k);
  if (rc) return rc;
  rc = check_indexer(q_idx, q_scale, k_idx, k_scale, w, qk_dtype, H, d, k, n_q);
  if (rc) return rc;
  if (n_q == 0) return DSA_OK;
  if (!idx_out) return fail(DSA_ERR_INVALID_ARG, "idx_out is required");
  if (((uintptr_t)idx_out & 3u) || ((uintptr_t)score_out & 3u)) return fail(DSA_ERR_ALIGNMENT, "outputs misaligned");
  const size_t need = indexer_ws(n_q, *seqs, qk_dtype, H, d, k);
  if (ws_bytes < need || (need && !ws)) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  dsa::IndexerArgs a = indexer_args(q_idx, q_scale, k_idx, k_scale, w, qk_dtype, H, d, k, *seqs, idx_out, score_out);
  a.flags = flags;
  return run_indexer(a, ws, (hipStream_t)stream);
}

size_t dsa_sparse_attn_ws(int n_h, int d_qk, int d_v, int k, const dsa_seqs* seqs) {
  int64_t n_q, n_k;
  if (check_seqs(seqs, &n_q, &n_k) != DSA_OK) return 0;
  return dsa::attn_ws_bytes(attn_args(nullptr, nullptr, nullptr, n_h, d_qk, d_v, k, 1.f, *seqs, nullptr, DSA_FP32));
}

int dsa_sparse_attn(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int d_qk, int d_v, int k,
                    float scale, const dsa_seqs* seqs, void* out, int out_dtype, void* ws, size_t ws_bytes,
                    void* stream) {
  int64_t n_q, n_k;
  int rc = check_seqs(seqs, &n_q, &n_k);
  if (rc) return rc;
  rc = check_attn(q, latent, idx, n_h, d_qk, d_v, k, out, out_dtype, n_q);
  if (rc) return rc;
  rc = check_latent_rows(seqs);
  if (rc) return rc;
  if (n_q == 0) return DSA_OK;
  dsa::AttnArgs a = attn_args(q, latent, idx, n_h, d_qk, d_v, k, scale, *seqs, out, out_dtype);
  const size_t need = dsa::attn_ws_bytes(a);
  if (ws_bytes < need || (need && !ws)) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  void* wsa = (void*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  hipError_t e = dsa::launch_sparse_attn(a, wsa, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
  return DSA_OK;
}

static int check_ring(int64_t rows, int64_t n_q, int64_t q_chunk, const char* what) {
  if (rows >= n_q) return DSA_OK;
  if (rows < 1 || rows % q_chunk != 0)
    return fail(DSA_ERR_INVALID_ARG, "%s=%lld must be >= n_q=%lld or a multiple of q_chunk=%lld", what,
                (long long)rows, (long long)n_q, (long long)q_chunk);
  return DSA_OK;
}

size_t indexcache_forward_ws(const char* roles, const dsa_shape* shape, const dsa_seqs* seqs) {
  int64_t n_q, n_k;
  if (!shape || check_seqs(seqs, &n_q, &n_k) != DSA_OK || shape->q_chunk < 1) return 0;
  (void)roles;
  size_t mx = 0;
  for (int64_t r0 = 0; r0 < n_q; r0 += shape->q_chunk) {
    const int64_t r1 = r0 + shape->q_chunk < n_q ? r0 + shape->q_chunk : n_q;
    const dsa_seqs cs = slice_seqs(*seqs, r0, r1);
    size_t a = indexer_ws(r1 - r0, cs, shape->qk_dtype, shape->H, shape->d, shape->k);
    size_t b = dsa::attn_ws_bytes(attn_args(nullptr, nullptr, nullptr, shape->n_h, shape->d_qk, shape->d_v,
                                            shape->k, shape->scale, cs, nullptr, shape->out_dtype));
    mx = mx > a ? mx : a;
    mx = mx > b ? mx : b;
  }
  return mx;
}

int indexcache_forward(const char* roles, const dsa_layer* layers, const dsa_shape* shape, const dsa_seqs* seqs,
                       int32_t* index_cache, float* score_cache, void* ws, size_t ws_bytes, dsa_stats* stats,
                       void* stream) {
  int32_t src[DSA_MAX_LAYERS];
  int32_t calls = 0;
  int rc = indexcache_plan(roles, src, &calls);
  if (rc) return rc;
  const int n_layers = (int)strlen(roles);
  if (!layers || !shape) return fail(DSA_ERR_INVALID_ARG, "layers and shape are required");
  int64_t n_q, n_k;
  rc = check_seqs(seqs, &n_q, &n_k);
  if (rc) return rc;
  if (shape->q_chunk < 1) return fail(DSA_ERR_INVALID_ARG, "q_chunk < 1");
  if (shape->flags & ~DSA_TOPK_BF16_SCORES) return fail(DSA_ERR_INVALID_ARG, "unknown flags 0x%x", shape->flags);
  if (n_q > 0 && !index_cache) return fail(DSA_ERR_INVALID_ARG, "index_cache is required");
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer& L = layers[l];
    if (roles[l] == 'F') {
      rc = check_indexer(L.q_idx, L.q_scale, L.k_idx, L.k_scale, L.w, shape->qk_dtype, shape->H, shape->d, shape->k,
                         n_q);
      if (rc) return fail(rc, "layer %d: %s", l, g_last_error.c_str());
    }
    rc = check_attn(L.q, L.latent, index_cache, shape->n_h, shape->d_qk,
                    shape->d_v, shape->k, L.out, shape->out_dtype, n_q);
    if (rc) return fail(rc, "layer %d: %s", l, g_last_error.c_str());
  }
  rc = check_latent_rows(seqs);
  if (rc) return rc;
  if (((uintptr_t)index_cache & 3u) || ((uintptr_t)score_cache & 3u))
    return fail(DSA_ERR_ALIGNMENT, "index/score cache misaligned");
  rc = check_ring(shape->index_rows, n_q, shape->q_chunk, "index_rows");
  if (rc) return rc;
  rc = check_ring(shape->out_rows, n_q, shape->q_chunk, "out_rows");
  if (rc) return rc;
  const size_t need = indexcache_forward_ws(roles, shape, seqs);
  if (ws_bytes < need || (need && !ws)) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

  int n_chunks = 0, n_traced = 0;
  hipStream_t st = (hipStream_t)stream;
  hipEvent_t* ev = stats && stats->events ? (hipEvent_t*)stats->events : nullptr;
  const int ev_pairs = ev ? (stats->event_cap / 2 < DSA_MAX_TRACE ? stats->event_cap / 2 : DSA_MAX_TRACE) : 0;
  auto trace_begin = [&](int kind, int layer, int chunk) -> bool {
    if (n_traced >= ev_pairs) return false;
    stats->trace_kind[n_traced] = (int8_t)kind;
    stats->trace_layer[n_traced] = (int16_t)layer;
    stats->trace_chunk[n_traced] = chunk;
    return hipEventRecord(ev[2 * n_traced], st) == hipSuccess;
  };
  auto trace_end = [&](bool on) {
    if (on && hipEventRecord(ev[2 * n_traced + 1], st) == hipSuccess) ++n_traced;
  };
  const size_t qe = elt_size(shape->qk_dtype), oe = elt_size(shape->out_dtype);
  void* wsa = (void*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  for (int64_t r0 = 0; r0 < n_q; r0 += shape->q_chunk, ++n_chunks) {
    const int64_t r1 = r0 + shape->q_chunk < n_q ? r0 + shape->q_chunk : n_q;
    const dsa_seqs cs = slice_seqs(*seqs, r0, r1);
    const int64_t islot = shape->index_rows >= n_q ? r0 : r0 % shape->index_rows;
    const int64_t oslot = shape->out_rows >= n_q ? r0 : r0 % shape->out_rows;
    int32_t* icache = index_cache + islot * shape->k;
    float* scache = score_cache ? score_cache + islot * shape->k : nullptr;
    for (int l = 0; l < n_layers; ++l) {
      const dsa_layer& L = layers[l];
      if (roles[l] == 'F') {
        dsa::IndexerArgs a = indexer_args((const char*)L.q_idx + (size_t)r0 * shape->H * shape->d * qe,
                                          L.q_scale ? L.q_scale + r0 * shape->H : nullptr, L.k_idx, L.k_scale,
                                          L.w + r0 * shape->H, shape->qk_dtype, shape->H, shape->d, shape->k, cs,
                                          icache, scache);
        a.flags = shape->flags;
        const bool tr = trace_begin(0, l, n_chunks);
        rc = run_indexer(a, ws, st);
        if (rc) return fail(rc, "layer %d chunk %d: %s", l, n_chunks, g_last_error.c_str());
        trace_end(tr);
      }
      dsa::AttnArgs a = attn_args(L.q + (size_t)r0 * shape->n_h * shape->d_qk, L.latent, icache, shape->n_h,
                                  shape->d_qk, shape->d_v, shape->k, shape->scale, cs,
                                  (char*)L.out + (size_t)oslot * shape->n_h * shape->d_v * oe, shape->out_dtype);
      const bool tr = trace_begin(1, l, n_chunks);
      hipError_t e = dsa::launch_sparse_attn(a, wsa, st);
      if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
      trace_end(tr);
    }
  }
  if (stats) {
    stats->n_traced = n_traced;
    stats->n_layers = n_layers;
    stats->n_indexer_calls = calls;
    stats->n_chunks = n_chunks;
    for (int l = 0; l < n_layers; ++l) stats->src_layer[l] = src[l];
  }
  return DSA_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free variant of indexcache_forward.  Its workspace is this file-scope
// device array: every GPU that runs the library holds its own copy (at its own
// address) until the process ends.  In host code the array's name only stands in
// for the symbol; the device address of the current device's copy is looked up
// once per device with hipGetSymbolAddress and used from then on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on first use).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}
}  // namespace

int indexcache_forward_noalloc(const char* roles, const dsa_layer* layers, const dsa_shape* shape,
                               const dsa_seqs* seqs, int32_t* index_cache, float* score_cache, dsa_stats* stats,
                               void* stream) {
  const int prc = indexcache_plan(roles, nullptr, nullptr);
  if (prc) return prc;
  const size_t need = indexcache_forward_ws(roles, shape, seqs);
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_ERR_WORKSPACE, "this shape needs %zu bytes of workspace, above the %zu bytes of the "
                "allocation-free entry point's scratch array", need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  if (need > 0) {
    const int rc = scratch_for_current_device(&ptr);
    if (rc) return rc;
  }
  return indexcache_forward(roles, layers, shape, seqs, index_cache, score_cache, ptr,
                            ptr ? (size_t)DSA_NOALLOC_SCRATCH_BYTES : 0, stats, stream);
}

}  // extern "C"
