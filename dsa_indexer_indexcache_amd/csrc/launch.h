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
hipError_t launch_indexer_slab(const IndexerArgs& a, float* slab, hipStream_t st);
hipError_t launch_topk_select(const IndexerArgs& a, const float* slab, hipStream_t st);

// topk_wide.hip: top-k of few long slab rows spread over (chunk, row) workgroups;
// `state` is wide_select_ws() bytes of workspace.
bool wide_select_ok(const IndexerArgs& a);
size_t wide_select_ws(const IndexerArgs& a);
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

// sparse_attn.hip
int attn_splits(const AttnArgs& a);
size_t attn_ws_bytes(const AttnArgs& a);
hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, hipStream_t st);

}  // namespace dsa
