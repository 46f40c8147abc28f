// Internal launcher interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

struct IndexerArgs {
  const void* q_idx;
  const float* q_scale;
  const void* k_idx;
  const float* k_scale;
  const uint16_t* w;
  int qk_dtype, H, d, k;
  dsa_seqs seqs;
  int32_t* idx_out;
  float* score_out;
  int flags;  // DSA_TOPK_* (bf16-rounded scores)
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* latent;
  const int32_t* idx;
  int n_h, d_qk, d_v, k;
  float scale;
  dsa_seqs seqs;
  void* out;
  int out_dtype;
};

// indexer_slab.hip: scores of every visible (row, key) into a [n_q, ld] fp32 slab, then top-k.
int64_t slab_ld(const dsa_seqs& s);
// zero (or null): zero_words 32-bit words that the score kernel clears before its scores are
// read (the wide select's counters and histograms, wide_select_zero_region).
hipError_t launch_indexer_slab(const IndexerArgs& a, float* slab, hipStream_t st, uint32_t* zero = nullptr,
                               int64_t zero_words = 0);
hipError_t launch_topk_select(const IndexerArgs& a, const float* slab, hipStream_t st);

// topk_wide.hip: top-k of few long slab rows spread over (chunk, row) workgroups;
// `state` is wide_select_ws() bytes of workspace.
bool wide_select_ok(const IndexerArgs& a);
size_t wide_select_ws(const IndexerArgs& a);
// The select's per-row counters and histograms: one contiguous range of `state` that must be
// zero when launch_wide_select starts (the score pass clears it, see launch_indexer_slab).
void wide_select_zero_region(const IndexerArgs& a, void* state, uint32_t** begin, int64_t* words);
hipError_t launch_wide_select(const IndexerArgs& a, const float* slab, void* state, hipStream_t st);

// indexer_fused.hip: one-sequence prefill, scores never leave the chip; no workspace.
bool indexer_fused_ok(const IndexerArgs& a);
hipError_t launch_indexer_fused(const IndexerArgs& a, hipStream_t st);

// diagnostics.hip: per-row fp8 quantisation; per-row intersection counts of two index
// tensors (k <= kOverlapMaxK).
hipError_t launch_quantize_fp8_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, float* scales,
                                    hipStream_t st);
constexpr int kOverlapMaxK = 16384;
hipError_t launch_index_overlap(const int32_t* a, const int32_t* b, int64_t n_rows, int k, int32_t* counts,
                                hipStream_t st);

// proj.hip: indexer projections (query with RoPE; key with LayerNorm and RoPE; head weights
// with the folded scales), d = 128; rope_dim in {0, 32, 64}; r and hidden multiples of 64.
struct ProjectArgs {
  const uint16_t* q_lat;
  const uint16_t* h;
  const uint16_t* wq;
  const uint16_t* wk;
  const float* gamma;
  const float* beta;
  const uint16_t* ww;
  const int32_t* pos;
  int64_t n;
  int r, hidden, H, rope_dim;
  float rope_base, eps;
  uint16_t* q_idx;
  uint16_t* k_idx;
  uint16_t* w;
};
hipError_t launch_indexer_project(const ProjectArgs& a, hipStream_t st);
hipError_t launch_cache_append(void* cache, int64_t cache_rows, const int64_t* dst_row, const void* rows,
                               int64_t n_rows, int64_t row_bytes, hipStream_t st);

// attn_stats.hip: attention statistics over a query's key sets (dense prefix / selected list):
// captured mass and Recall@k against the dense top-k, the sparse-training indexer KL.
struct StatArgs {
  const uint16_t* q;
  const uint16_t* latent;
  const int32_t* idx;
  int n_h, k;
  float scale;
  dsa_seqs seqs;
};
size_t attn_mass_ws(const StatArgs& a, bool recall);
hipError_t launch_attention_mass(const StatArgs& a, float* mass_head, float* mass, float* recall, void* ws,
                                 hipStream_t st);
size_t indexer_kl_ws(const StatArgs& a);
hipError_t launch_indexer_kl(const StatArgs& a, const float* scores, float weight, int accumulate, float* kl,
                             float* loss, void* ws, hipStream_t st);

// csa.hip: gated pooling of tokens n / m ... into compressed entries block0 .. n / m - 1;
// c a multiple of 8; out [n / m - block0, c] in out_dtype (DSA_FP32 or DSA_BF16).
struct CsaArgs {
  const uint16_t* ca;
  const uint16_t* cb;
  const uint16_t* za;
  const uint16_t* zb;
  const float* ba;
  const float* bb;
  int64_t n, block0;
  int c, m;
  void* out;
  int out_dtype;
};
hipError_t launch_csa_compress(const CsaArgs& a, hipStream_t st);

// sparse_attn.hip
int attn_splits(const AttnArgs& a);
size_t attn_ws_bytes(const AttnArgs& a);
hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, hipStream_t st);

}  // namespace dsa
