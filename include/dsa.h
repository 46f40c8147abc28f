/*
 * dsa.h — C ABI of the MI355X (gfx950) DSA hot path: lightning indexer, per-query
 * top-k, sparse MLA attention, and the IndexCache F/S layer loop.
 *
 * Sources (page titles; sections/equations named at each declaration):
 *   [IDX] Jerry's Blog, "注意力机制中的 Index：从位置下标到预算检索"
 *   [IC]  "读懂 IndexCache：从 DSA 的选词开销到跨层索引复用"
 *
 * Conventions shared by every entry point
 *   - Device pointers are HIP device addresses; host pointers are marked (host).
 *   - All tensors are dense, row-major, with 16-byte aligned base pointers.
 *   - bf16 tensors are passed as uint16_t bit patterns; fp8 tensors are OCP
 *     e4m3fn bytes (max 448) with one positive fp32 scale per row.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are enqueued
 *     asynchronously on it; the library never synchronises, never allocates
 *     device memory and keeps no pointer after it returns.  Device-side faults
 *     surface at the caller's next synchronisation.
 *   - The caller owns every buffer, including the workspace `ws`, whose size is
 *     given by the matching *_ws() query.  Outputs must not alias inputs.
 *   - Validation happens before any launch: on a non-zero status nothing has
 *     been enqueued and outputs are untouched.  No C++ exception crosses the ABI.
 *   - Reentrant: the only global state is per-device properties initialised once
 *     under a lock.
 */
#ifndef DSA_MI355X_H
#define DSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1, /* null required pointer, k < 1, bad sizes, bad sequence table */
  DSA_ERR_ROLES = -2,       /* empty role string or a character outside {F,S}            */
  DSA_ERR_FIRST_NOT_F = -3, /* roles[0] != 'F': S layers would have no indices ([IC] §1.1) */
  DSA_ERR_UNSUPPORTED = -4, /* (H, d, n_h, d_qk, d_v, dtype) combination not compiled       */
  DSA_ERR_ALIGNMENT = -5,   /* a base pointer is not 16-byte aligned                         */
  DSA_ERR_WORKSPACE = -6,   /* ws_bytes smaller than the *_ws() query                        */
  DSA_ERR_HIP = -7          /* a HIP launch failed (detail in dsa_last_error())             */
};

typedef enum {
  DSA_BF16 = 0,     /* uint16 bf16 bit patterns                     */
  DSA_FP8_E4M3 = 1, /* OCP e4m3fn bytes + fp32 per-row scales       */
  DSA_FP32 = 2
} dsa_dtype;

#define DSA_MAX_B 64        /* sequences per call                  */
#define DSA_MAX_LAYERS 256  /* layers per indexcache_forward call  */

/*
 * Packed variable-length batch (host struct, passed to kernels by value).
 * Sequence b owns query rows [q_start[b], q_start[b+1]) and key/latent rows
 * [k_start[b], k_start[b+1]).  Query row i of sequence b sits at absolute
 * position p = q_pos0[b] + (i - q_start[b]) and sees the key rows
 * k_start[b] .. k_start[b] + p inclusive (visible set s <= t, [IDX] §4 memory
 * M_t = {c_s : s <= t}); p must be < k_start[b+1] - k_start[b].
 * Positions written to index outputs are sequence-local (0..p).
 *   prefill chunk: B = 1, q_pos0[0] = position of the chunk's first query;
 *   decode step:   q_start = {0,1,..,B}, q_pos0[b] = len_b - 1 (the new token
 *                  is already in the caches).
 * block (0 or 1: token keys): the key rows are compressed blocks of `block` tokens
 * (the compressed-block selection of [IDX] §5.2): a query at token position t sees
 * blocks s < floor(t / block), i.e. up to s = floor(t / block) - 1 (none while
 * t < block), and floor(t_last / block) <= k_start[b+1] - k_start[b] must hold.
 */
typedef struct {
  int32_t B;
  int32_t block;
  int64_t q_start[DSA_MAX_B + 1];
  int64_t k_start[DSA_MAX_B + 1];
  int64_t q_pos0[DSA_MAX_B];
} dsa_seqs;

/* ---------------------------------------------------------------- indexer + top-k */
/*
 * Lightning indexer score and per-query top-k ([IDX] §4 score equation
 * I[t,s] = sum_j w[t,j] ReLU(q_idx[t,j,:] . k_idx[s,:]); §2 S_t = TopK_k over the
 * visible set; §6.5 the selection must be deterministic).
 *
 *   q_idx   [n_q, H, d]  bf16 or e4m3fn         (device)
 *   q_scale [n_q, H]     fp32 > 0, fp8 only     (device, NULL for bf16)
 *   k_idx   [n_k, d]     bf16 or e4m3fn         (device)
 *   k_scale [n_k]        fp32 > 0, fp8 only     (device, NULL for bf16)
 *   w       [n_q, H]     bf16                   (device)
 *   idx_out [n_q, k]     int32                  (device, written)
 *   score_out [n_q, k]   fp32, optional         (device, written; NULL to skip)
 * For fp8 the dequantised values are scale * code; the score equals the
 * definition applied to them (the positive scales are folded out of the ReLU).
 * Row i receives exactly min(k, p+1) distinct positions in [0, p], ranked by
 * score descending then position ascending (ties go to the lower position;
 * -0.0 == +0.0); the remaining slots are -1.  Valid positions are written in
 * ascending order.  score_out[i, j] is the fp32 score of idx_out[i, j] (0 for
 * -1 slots).  Scores are computed in fp32 from exact input products.
 * Supported: H in {8,16,32,64} (rounded up to 16 internally), d in {64,128};
 * fp8 needs d == 128.  Returns DSA_ERR_UNSUPPORTED otherwise.
 */
int dsa_indexer_topk(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                     const uint16_t* w, int qk_dtype, int H, int d, int k, const dsa_seqs* seqs /* host */,
                     int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_indexer_topk with selection flags.  DSA_TOPK_BF16_SCORES: every score is rounded
 * to bf16 (nearest even) before the ranking, the lower-precision selector of [IDX] §5.4
 * (which quantises index scores from fp32 to bf16); more scores tie, ties still go to the
 * lower position, and score_out holds the rounded values.  flags == 0 is dsa_indexer_topk.
 */
#define DSA_TOPK_BF16_SCORES 1
int dsa_indexer_topk_ex(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                        const uint16_t* w, int qk_dtype, int H, int d, int k, const dsa_seqs* seqs /* host */,
                        int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes, int flags, void* stream);

/* Workspace bytes dsa_indexer_topk needs for this shape: 0 for one-sequence
 * prefill with at least 256 query rows, k <= 2048 and d in {64,128} (scores never
 * leave the chip); otherwise an fp32 score slab of n_q x (longest visible prefix)
 * plus, for at most 64 rows whose prefix reaches 32768 keys (decode), the state of
 * the chunked multi-workgroup select (about 140 KB per row). */
size_t dsa_indexer_topk_ws(int qk_dtype, int H, int d, int k, const dsa_seqs* seqs /* host */);

/* ---------------------------------------------------------------- sparse attention */
/*
 * Sparse MLA attention over the selected latent rows ([IDX] §2 sparse softmax
 * over S_t and o_t = sum alpha_hat v_s; §4 the latent row c_s is shared by all
 * query heads):
 *   out[i,h,:] = sum_{s in S_i} softmax_s(scale * q[i,h,:d_qk] . c[s,:d_qk]) * c[s,:d_v]
 *
 *   q      [n_q, n_h, d_qk] bf16   (device)
 *   latent [n_k, d_qk]      bf16   (device; keys = all d_qk columns, values = first d_v)
 *   idx    [n_q, k]         int32  (device; sequence-local positions, -1 = unused slot;
 *                                   entries outside [0, p] are skipped, never read)
 *   out    [n_q, n_h, d_v]  fp32 or bf16 (out_dtype)  (device, written)
 * A row with no usable index gets out = 0.  Softmax and accumulation are fp32.
 * Supported: n_h in {16,32,64,128}, d_qk == 576, d_v == 512, at most 3,728,266 latent
 * rows per sequence (rows are addressed by a 32-bit byte offset; else DSA_ERR_UNSUPPORTED,
 * also from indexcache_forward).
 */
int dsa_sparse_attn(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int d_qk, int d_v,
                    int k, float scale, const dsa_seqs* seqs /* host */, void* out, int out_dtype, void* ws,
                    size_t ws_bytes, void* stream);

size_t dsa_sparse_attn_ws(int n_h, int d_qk, int d_v, int k, const dsa_seqs* seqs /* host */);

/* ---------------------------------------------------------------- IndexCache */
/* One layer's tensors (device pointers).  q_idx/q_scale/k_idx/k_scale/w are read
 * only when the layer's role is F. */
typedef struct {
  const void* q_idx;
  const float* q_scale;
  const void* k_idx;
  const float* k_scale;
  const uint16_t* w;
  const uint16_t* q;
  const uint16_t* latent;
  void* out;
} dsa_layer;

typedef struct {
  int32_t H, d, k;          /* indexer heads, head dim, top-k budget   */
  int32_t n_h, d_qk, d_v;   /* attention heads, latent width, value width */
  float scale;              /* softmax scale (1/sqrt(d_qk) for MLA)     */
  int32_t qk_dtype;         /* dsa_dtype of q_idx/k_idx                 */
  int32_t out_dtype;        /* dsa_dtype of out (DSA_FP32 or DSA_BF16)  */
  int32_t flags;            /* DSA_TOPK_* flags of the F layers' selection */
  int64_t q_chunk;          /* query rows per chunk (>= 1)               */
  int64_t index_rows;       /* rows of index_cache / score_cache         */
  int64_t out_rows;         /* rows of every layer's out buffer           */
} dsa_shape;

#define DSA_MAX_TRACE 1024 /* traced calls per indexcache_forward call */

typedef struct {
  /* in (optional): launch tracing.  events points to caller-created hipEvent_t
   * handles (host array of event_cap entries, may be NULL).  Call j of the loop
   * (one dsa_indexer_topk or dsa_sparse_attn step) is bracketed by
   * hipEventRecord(events[2j]) and hipEventRecord(events[2j+1]) on the stream;
   * the library records only and never synchronises or queries them. */
  void** events;
  int32_t event_cap;
  /* out */
  int32_t n_layers;
  int32_t n_indexer_calls;          /* = number of F layers (the indexer work kept)  */
  int32_t n_chunks;
  int32_t n_traced;                 /* event pairs recorded                           */
  int32_t reserved;
  int32_t src_layer[DSA_MAX_LAYERS]; /* layer whose indices layer l attends with      */
  int8_t trace_kind[DSA_MAX_TRACE];  /* 0 = indexer + top-k, 1 = sparse attention      */
  int16_t trace_layer[DSA_MAX_TRACE];
  int32_t trace_chunk[DSA_MAX_TRACE];
} dsa_stats;

/*
 * Index-reuse inference loop ([IC] §1.1 F/S roles; §1.2 the loop that keeps one
 * index tensor, overwritten by each F layer and read by every later S layer).
 * roles: NUL-terminated (host), one 'F' or 'S' per layer; n_layers = strlen(roles).
 * For each chunk of shape->q_chunk query rows (chunked prefill order: every
 * layer of chunk c before chunk c+1), for each layer l:
 *   role F: dsa_indexer_topk on layer l's indexer tensors -> index_cache
 *   every layer: dsa_sparse_attn(layer l's q and latent, index_cache) -> layer l's out
 * An S layer therefore attends over the positions chosen by the nearest
 * preceding F layer, with its own q and latent.  Row i of the index cache lives
 * in slot (i mod index_rows) and row i of out in slot (i mod out_rows); each of
 * index_rows / out_rows must be >= n_q, or a multiple of q_chunk (a ring that
 * holds the current chunk).  score_cache (optional) mirrors index_cache.
 * stats (host, optional) receives the plan and call count, and optionally
 * brackets each step with caller-provided events (see dsa_stats).
 */
int indexcache_forward(const char* roles, const dsa_layer* layers /* host array */, const dsa_shape* shape /* host */,
                       const dsa_seqs* seqs /* host */, int32_t* index_cache, float* score_cache, void* ws,
                       size_t ws_bytes, dsa_stats* stats /* host */, void* stream);

size_t indexcache_forward_ws(const char* roles, const dsa_shape* shape, const dsa_seqs* seqs);

/*
 * Allocation-free variant of indexcache_forward, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as indexcache_forward without
 * ws/ws_bytes: the workspace is a file-scope device array of the library of
 * DSA_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use on that
 * GPU until the process ends.  Returns DSA_ERR_WORKSPACE (nothing enqueued) when
 * indexcache_forward_ws() of the call exceeds that size.  The call allocates and
 * frees nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams or threads without ordering) race; calls
 * ordered on one stream do not.  The kernels leave no state in the array that a
 * later call relies on.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB per GPU */
int indexcache_forward_noalloc(const char* roles, const dsa_layer* layers /* host array */,
                               const dsa_shape* shape /* host */, const dsa_seqs* seqs /* host */,
                               int32_t* index_cache, float* score_cache, dsa_stats* stats /* host */,
                               void* stream);

/*
 * Host-only planning of the loop above ([IC] §1.1: the first layer must be F;
 * an S layer uses the nearest preceding F layer).  src_layer (host, n_layers
 * entries, may be NULL) receives max{l' <= l : roles[l'] == 'F'};
 * n_indexer_calls (host, may be NULL) the number of F layers.  Needs no GPU.
 */
int indexcache_plan(const char* roles, int32_t* src_layer, int32_t* n_indexer_calls);

/* ---------------------------------------------------------------- diagnostics */
/*
 * Cross-layer index overlap ([IDX] §8 metrics: the share of one layer's selected
 * set that another layer also selects; [IC] §1 motivates index reuse by this
 * similarity between layers).  For every row i, counts[i] = |A_i ∩ B_i|, where A_i
 * and B_i are the sets of valid (>= 0) entries of idx_a[i, :] and idx_b[i, :]
 * (row order does not matter; valid entries of a row must be distinct, as the
 * indexer writes them).  Overlap^(l,l') of the row = counts[i] / k.
 *   idx_a, idx_b [n_rows, k] int32 (device);  counts [n_rows] int32 (device, written)
 * 1 <= k <= 16384 and n_rows < 2^31 (else DSA_ERR_UNSUPPORTED); n_rows == 0 is a
 * no-op; n_rows < 0 or a null pointer gives DSA_ERR_INVALID_ARG.  Exact (integer) result.
 */
int dsa_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t n_rows, int k, int32_t* counts,
                      void* stream);

/*
 * Per-row fp8 quantisation of indexer inputs on the device (the fp8 setting's
 * per-row scales, upstream of dsa_indexer_topk).  For every row r of x:
 *   scale[r] = max_j |x[r, j]| / 448 (1 for an all-zero row), computed in fp32;
 *   codes[r, j] = e4m3fn(clamp(x[r, j] / scale[r], -448, 448)), fp32 division, round
 *                 to nearest even, sign kept (OCP e4m3fn, max 448).
 *   x [rows, cols] bf16 (device); codes [rows, cols] e4m3fn bytes, scales [rows] fp32
 *   (device, written).  A q_idx [n_q, H, d] tensor is rows = n_q * H, cols = d.
 * 1 <= cols <= 65536 and rows < 2^31 (else DSA_ERR_UNSUPPORTED); rows == 0 is a no-op;
 * rows < 0 or a null pointer gives DSA_ERR_INVALID_ARG.
 */
int dsa_quantize_fp8_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, float* scales, void* stream);

/*
 * Index-quality metrics of one query row ([IDX] §8 items 1 and 2), from the main
 * attention's dense weights alpha[t, h, s] = softmax over s <= t of scale q[t,h].c[s]
 * (the dense attention of [IDX] §1; keys = all d_qk latent columns):
 *   mass_head[i, h] = CapturedMass@k of head h = sum over s in S_i of alpha[t, h, s]
 *   mass[i]         = the same for the head-aggregated distribution p_t (heads summed,
 *                     then L1-normalised: the mean of mass_head over h); MissedMass = 1 - mass
 *   recall[i]       = Recall@k = |S^oracle_i ∩ S_i| / |S^oracle_i|, S^oracle_i the min(k, t+1)
 *                     positions of largest p_t[s] (ties to the lower position)
 * S_i are the valid entries (0 <= s <= t) of idx[i, :] (the model's selection).
 *   q [n_q, n_h, d_qk] bf16, latent [n_k, d_qk] bf16, idx [n_q, k] int32 (device);
 *   mass [n_q] fp32 (required), mass_head [n_q, n_h] fp32 and recall [n_q] fp32 (optional).
 * Scores and sums in fp32.  Supported: n_h in {16,32,64,128}, d_qk == 576, k <= 2048.
 * The dense pass costs O(t n_h d_qk) per row: a metric for short contexts.  The workspace
 * (dsa_attention_mass_ws) holds two per-head log-sum-exp tables and, with recall, an fp32
 * row of p_t per query (n_q x longest prefix).
 */
size_t dsa_attention_mass_ws(int n_h, int k, const dsa_seqs* seqs /* host */, int want_recall);
int dsa_attention_mass(const uint16_t* q, const uint16_t* latent, const int32_t* idx, int n_h, int d_qk, int k,
                       float scale, const dsa_seqs* seqs /* host */, float* mass_head, float* mass, float* recall,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse-training indexer loss ([IDX] §4.2: D_KL(p_{t,S_t} || Softmax(I_{t,S_t})), p the
 * main attention's weights over S_t summed over heads and L1-normalised; [IC] §3.1: an F
 * layer serving m S layers averages the KL against each served layer's p):
 *   kl[i] = (accumulate ? kl[i] : 0) + weight * D_KL(p_i || softmax(scores[i, valid slots]))
 * with the attention over the valid slots of idx[i, :] (this layer's q and latent) and
 * scores[i, j] the indexer score of slot j (as dsa_indexer_topk's score_out).  The
 * multi-layer loss: call once per served layer with weight 1/(m+1), accumulate = 0 for
 * the first.  loss (optional, device fp32 scalar) receives sum_i kl[i] (fixed-order sum).
 * A row with no valid slot contributes 0.  Supported as dsa_attention_mass.
 */
size_t dsa_indexer_kl_ws(int n_h, int k, const dsa_seqs* seqs /* host */);
int dsa_indexer_kl(const uint16_t* q, const uint16_t* latent, const int32_t* idx, const float* scores, int n_h,
                   int d_qk, int k, float scale, const dsa_seqs* seqs /* host */, float weight, int accumulate,
                   float* kl, float* loss, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- upstream of the indexer */
/*
 * The indexer's inputs from the token's low-rank query latent and hidden state
 * ([IDX] §6.4, the GLM indexer: a query projection split into H heads of d, a key
 * projection followed by a LayerNorm over d, head weights from the hidden state times
 * H^-1/2, a score scaled by d^-1/2, rotary encoding of the query/key rotary part):
 *   q_idx[t, j, :] = RoPE(q_lat[t] . wq[j d .. j d + d, :]^T, pos[t])
 *   k_idx[t, :]    = RoPE(LayerNorm(h[t] . wk^T) * ln_weight + ln_bias, pos[t])
 *   w[t, j]        = (h[t] . ww[j, :]^T) * H^-1/2 * d^-1/2
 * RoPE rotates dimension pairs (i, i + rope_dim/2), i < rope_dim/2, by the angle
 * pos * rope_base^(-2i/rope_dim) (angles in fp64); dimensions from rope_dim on pass
 * through.  The score's positive d^-1/2 is folded into w (it commutes with the ReLU),
 * so these outputs feed dsa_indexer_topk unchanged.  LayerNorm: population variance, eps.
 *   q_lat [n, r] bf16; h [n, hidden] bf16; wq [H d, r], wk [d, hidden], ww [H, hidden]
 *   bf16 (nn.Linear layout: [out, in]); ln_weight, ln_bias [d] fp32; pos [n] int32;
 *   outputs q_idx [n, H, d], k_idx [n, d], w [n, H] bf16 (fp32 accumulation, rounded once).
 * Supported: d == 128, 1 <= H <= 128, rope_dim in {0, 32, 64}, r and hidden positive
 * multiples of 64 (else DSA_ERR_UNSUPPORTED).  n == 0 is a no-op.  For the fp8 indexer,
 * dsa_quantize_fp8_rows turns q_idx / k_idx into codes and scales.
 */
int dsa_indexer_project(const uint16_t* q_lat, const uint16_t* h, const uint16_t* wq, const uint16_t* wk,
                        const float* ln_weight, const float* ln_bias, const uint16_t* ww, const int32_t* pos, int64_t n,
                        int r, int hidden, int H, int d, int rope_dim, float rope_base, float eps, uint16_t* q_idx,
                        uint16_t* k_idx, uint16_t* w, void* stream);

/*
 * KV compression of compressed sparse attention ([IDX] §5.1, DeepSeek-V4 CSA): every m
 * tokens become one entry by a gated pooling over an overlapping window of 2m rows.
 * Entry i, for each feature column j separately, weighs the a-half rows m i .. m i + m - 1
 * and the b-half rows m (i-1) .. m i - 1 by one softmax over the 2m gate logits
 *   za[m i + r, j] + ba[r, j]   and   zb[m (i-1) + r, j] + bb[r, j]   (r < m)
 * and writes the weighted sum of ca[m i + r, j] and cb[m (i-1) + r, j].  Entry 0 has no
 * b-half (its window would start before token 0) and pools the a-half alone.  Only
 * complete groups of m tokens form entries: entries block0 .. n / m - 1 are computed,
 * entry block0 + e written to row e of out (a decode step that completes a group passes
 * block0 = n / m - 1 and all n tokens' rows).
 *   ca, cb, za, zb [n, c] bf16 (the projections C^a, C^b, Z^a, Z^b of the tokens);
 *   ba, bb [m, c] fp32 (positional gate biases); out [n / m - block0, c] in out_dtype
 *   (DSA_FP32 or DSA_BF16, rounded to nearest even once).  fp32 arithmetic.
 * Supported: c a positive multiple of 8, 1 <= m <= 4096.  n / m <= block0 is a no-op.
 * The compressed rows are keys of dsa_indexer_topk with seqs->block = m.
 */
int dsa_csa_compress(const uint16_t* ca, const uint16_t* cb, const uint16_t* za, const uint16_t* zb,
                     const float* ba, const float* bb, int64_t n, int c, int m, int64_t block0, void* out,
                     int out_dtype, void* stream);

/*
 * Decode-time cache write ([IDX] §4: every new token is written into the caches before
 * the read of the same step): row b of `rows` (row_bytes bytes) is copied to row
 * dst_row[b] of `cache` (cache_rows rows of row_bytes).  A packed per-sequence cache with
 * sequence b at k_start[b] and len_b tokens takes dst_row[b] = k_start[b] + len_b.
 *   cache (device, written); dst_row [n_rows] int64 (device); rows [n_rows, row_bytes] (device)
 * A destination outside [0, cache_rows) is skipped for that row.  n_rows == 0 is a no-op.
 */
int dsa_cache_append(void* cache, int64_t cache_rows, const int64_t* dst_row, const void* rows, int64_t n_rows,
                     int64_t row_bytes, void* stream);

/* ---------------------------------------------------------------- misc */
const char* dsa_status_string(int status); /* static string                         */
const char* dsa_last_error(void);          /* thread-local detail of the last error */
int dsa_version(void);                     /* ABI version (major*100 + minor)        */

#ifdef __cplusplus
}
#endif
#endif /* DSA_MI355X_H */
