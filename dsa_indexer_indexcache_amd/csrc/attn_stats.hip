// Attention statistics beside the hot path: the index-quality metrics of [IDX] §8
// (CapturedMass@k, MissedMass@k, Recall@k against the dense attention's own top-k) and
// the sparse-training indexer loss of [IDX] §4.2 (KL between the main attention's
// head-aggregated distribution over S_t and the softmax of the indexer scores over
// S_t), with the multi-layer average of [IC] §3.1 by accumulation over served layers.
//
// All of them need the main attention's weights alpha[t, h, s] = softmax_s(scale q[t,h].c[s])
// over a key set: the whole causal prefix (dense) or the selected list (sparse).  One
// workgroup per query row, one wave per 16 heads, each wave computing the full QK over
// the 576 latent columns (as the attention kernel, without PV); keys stream through LDS
// in blocks of 32 by direct global->LDS copies one block ahead.
//   lse  : per head the log2-domain log-sum-exp L_h of x = scale log2(e) q.c over the set;
//   p    : per key p_s = (1/n_h) sum_h 2^(x[h,s] - L_h)  (the head-summed, L1-normalised
//          distribution of [IDX] §4.1), written per key (dense) or folded into the KL (sparse).
// Cross-head sums run over the 16 lanes of a wave's row group (xor shuffles) and over the
// waves through per-wave LDS slots read in wave order (deterministic).
#include <math.h>

#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kSD = 576;                 // latent width (keys use every column)
constexpr int kSB = 32;                  // keys per block
constexpr int kSTile = (kSD / 64) * kSB * 128;   // 36864 bytes: 9 column groups x 32 rows x 128 B
constexpr int kSTileIns = kSTile / 1024;         // 36 copies of 64 lanes x 16 B
constexpr int kSIdxMax = 2048;
constexpr int kSPf = 3;                  // K fragments read this many steps ahead

struct StatSmem {
  uint8_t tile[2][kSTile];
  int idx[kSIdxMax];                     // sparse: the row's slots (-1 = skip)
  float sc[kSIdxMax];                    // sparse KL: indexer score of each slot
  float wsum[2][8][kSB];                 // per-wave sums over the wave's heads, by block parity
  float red[8];
};

// Key position of slot j of block blk (dense: the position itself), -1 when the slot is
// not part of the set or not visible (s > p).
template <bool DENSE>
__device__ __forceinline__ int slot_pos(const StatSmem& sm, int blk, int r, int64_t p, int k) {
  if constexpr (DENSE) {
    const int64_t s = (int64_t)blk * kSB + r;
    return s <= p ? (int)s : -1;
  } else {
    const int j = blk * kSB + r;
    return j < k ? sm.idx[j] : -1;
  }
}

// Stages the sparse row (invisible or out-of-range entries become -1) and, for the KL, the
// indexer scores of the slots.
template <bool DENSE>
__device__ __forceinline__ void stage_row(StatSmem& sm, const int32_t* __restrict__ irow,
                                          const float* __restrict__ srow, int k, int64_t p) {
  if constexpr (!DENSE) {
    for (int j = threadIdx.x; j < ((k + kSB - 1) / kSB) * kSB; j += blockDim.x) {
      const int32_t s = j < k ? irow[j] : -1;
      const bool ok = s >= 0 && s <= p;
      sm.idx[j] = ok ? s : -1;
      if (srow) sm.sc[j] = j < k ? srow[j] : 0.f;
    }
  }
}

// direct global->LDS copy of block blk (32 latent rows) into slot si; layout as the
// attention tiles: column group j / 4, rows 8 (j % 4) .., granules XOR-swizzled by row.
// Slots outside the set load row 0 of the sequence (always present) and are masked.
template <bool DENSE, int NW>
__device__ __forceinline__ void stat_gather(StatSmem& sm, const uint16_t* lat, int blk, int si, int64_t p, int k) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lrow = lane >> 3, lpos = lane & 7;
  for (int j = wave; j < kSTileIns; j += NW) {
    const int r = 8 * (j & 3) + lrow;
    const int chunk = 8 * (j >> 2) + (lpos ^ (r & 7));
    const int s = slot_pos<DENSE>(sm, blk, r, p, k);
    dma16(lat + (int64_t)(s >= 0 ? s : 0) * kSD + 8 * chunk, lds_u32(&sm.tile[si][1024 * j]));
  }
}

// S^T[key][head] of one block for the wave's 16 heads over all 576 columns: lane (c, g)
// gets keys 16 kt + 4 g + r of head c.  K fragments are read kSPf steps ahead.
__device__ __forceinline__ void stat_qk(const uint8_t* tile, const i32x4 (&qf)[kSD / 32], f32x4 (&st)[2]) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  st[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  st[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* kb = tile + c * 128;
  auto off = [&](int ks) { return (ks >> 1) * (kSB * 128) + 16 * ((4 * (ks & 1) + g) ^ (c & 7)); };
  i32x4 kf[kSPf + 1][2];
#pragma unroll
  for (int j = 0; j < kSPf; ++j)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) kf[j][kt] = *reinterpret_cast<const i32x4*>(kb + off(j) + kt * 2048);
#pragma unroll
  for (int ks = 0; ks < kSD / 32; ++ks) {
    __builtin_amdgcn_sched_barrier(0);
    if (ks + kSPf < kSD / 32) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        kf[(ks + kSPf) % (kSPf + 1)][kt] = *reinterpret_cast<const i32x4*>(kb + off(ks + kSPf) + kt * 2048);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) st[kt] = mfma_bf16_16x16x32(kf[ks % (kSPf + 1)][kt], qf[ks], st[kt]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Loads the wave's 16 heads of q (B operand: lane -> head c, columns 32 ks + 8 g ..).
__device__ __forceinline__ void stat_q(const uint16_t* __restrict__ q, int64_t i, int n_h, int head0,
                                       i32x4 (&qf)[kSD / 32]) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const uint16_t* qrow = q + (i * n_h + head0 + c) * kSD + 8 * g;
#pragma unroll
  for (int ks = 0; ks < kSD / 32; ++ks) qf[ks] = *reinterpret_cast<const i32x4*>(qrow + 32 * ks);
}

// Number of key blocks of row i and its last visible position p.
template <bool DENSE>
__device__ __forceinline__ int stat_blocks(int64_t p, int k) {
  if constexpr (DENSE) return (int)((p + kSB) / kSB);
  return (k + kSB - 1) / kSB;
}

// Per-head log2-domain log-sum-exp over the key set; with lse_dense (sparse set), also the
// captured mass 2^(L_sparse - L_dense) per head and its mean over the heads.
template <int NW, bool DENSE>
__global__ __launch_bounds__(64 * NW) void attn_lse_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ latent,
                                                           const int32_t* __restrict__ idx, int n_h, int k,
                                                           float scale_log2, dsa_seqs seqs, int64_t n_q,
                                                           float* __restrict__ lse_out,
                                                           const float* __restrict__ lse_dense,
                                                           float* __restrict__ mass_head, float* __restrict__ mass) {
  __shared__ StatSmem sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int64_t i = blockIdx.x;
  if (i >= n_q) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const uint16_t* lat = latent + seqs.k_start[b] * kSD;
  const int head0 = 16 * wave;
  stage_row<DENSE>(sm, idx + i * (int64_t)k, nullptr, k, p);
  i32x4 qf[kSD / 32];
  stat_q(q, i, n_h, head0, qf);
  __syncthreads();
  const int nb = stat_blocks<DENSE>(p, k);
  float m = -INFINITY, l = 0.f;
  stat_gather<DENSE, NW>(sm, lat, 0, 0, p, k);
  for (int blk = 0; blk < nb; ++blk) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's copies of block blk landed
    lds_barrier();                        // every wave's; slot (blk + 1) & 1 is free
    if (blk + 1 < nb) stat_gather<DENSE, NW>(sm, lat, blk + 1, (blk + 1) & 1, p, k);
    f32x4 st[2];
    stat_qk(sm.tile[blk & 1], qf, st);
    float x[8];
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = slot_pos<DENSE>(sm, blk, 16 * kt + 4 * g + r, p, k) >= 0;
        x[4 * kt + r] = ok ? st[kt][r] * scale_log2 : -INFINITY;
        bm = fmaxf(bm, x[4 * kt + r]);
      }
    if (bm > -INFINITY) {
      const float mn = fmaxf(m, bm);
      float acc = m == -INFINITY ? 0.f : l * exp2f(m - mn);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += exp2f(x[e] - mn);
      m = mn;
      l = acc;
    }
  }
  // combine the four row groups of head c
  const float M = max_over_rows(m);
  const float part = (m == -INFINITY) ? 0.f : l * exp2f(m - M);
  const float Ls = sum_over_rows(part);
  const float lse = (M == -INFINITY || !(Ls > 0.f)) ? -INFINITY : M + log2f(Ls);
  const int head = head0 + c;
  if (g == 0) lse_out[i * n_h + head] = lse;
  if (!mass) return;
  const float ld = lse_dense[i * n_h + head];
  const float mh = (lse == -INFINITY) ? 0.f : exp2f(lse - ld);
  if (g == 0 && mass_head) mass_head[i * n_h + head] = mh;
  float sw = g == 0 ? mh : 0.f;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) sw += __shfl_xor(sw, d);
  if (lane == 0) sm.red[wave] = sw;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < NW; ++w) t += sm.red[w];
    mass[i] = t / (float)n_h;
  }
}

// Head-aggregated distribution per key: DENSE writes p[t, s] for s <= t into a slab of
// leading dimension ld; sparse folds it into the KL against the indexer scores:
//   KL_t = sum_s p_s ln p_s - sum_s p_s I_s + ln sum_s e^(I_s)   (sum_s p_s = 1),
// and writes kl[t] = (accumulate ? kl[t] : 0) + weight * KL_t.
template <int NW, bool DENSE>
__global__ __launch_bounds__(64 * NW) void attn_p_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ latent,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ scores, int n_h, int k,
                                                         float scale_log2, dsa_seqs seqs, int64_t n_q,
                                                         const float* __restrict__ lse, float* __restrict__ p_out,
                                                         int64_t ld, float* __restrict__ kl, float weight,
                                                         int accumulate) {
  __shared__ StatSmem sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int64_t i = blockIdx.x;
  if (i >= n_q) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const uint16_t* lat = latent + seqs.k_start[b] * kSD;
  const int head0 = 16 * wave;
  stage_row<DENSE>(sm, idx + (DENSE ? 0 : i * (int64_t)k), DENSE ? nullptr : scores + i * (int64_t)k, k, p);
  i32x4 qf[kSD / 32];
  stat_q(q, i, n_h, head0, qf);
  const float lh = lse[i * n_h + head0 + c];
  const float inv_h = 1.f / (float)n_h;
  __syncthreads();
  // sparse: ln sum_s e^(I_s) over the valid slots (wave 0)
  float lse_i = 0.f;
  if constexpr (!DENSE) {
    if (wave == 0) {
      float mx = -INFINITY;
      for (int j = lane; j < k; j += 64)
        if (sm.idx[j] >= 0) mx = fmaxf(mx, sm.sc[j]);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
      float sum = 0.f;
      for (int j = lane; j < k; j += 64)
        if (sm.idx[j] >= 0) sum += expf(sm.sc[j] - mx);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) sum += __shfl_xor(sum, d);
      lse_i = mx == -INFINITY ? 0.f : mx + logf(sum);
    }
  }
  float a_plogp = 0.f, a_pi = 0.f;  // wave 0, lane j < 32: slot j of each block
  const int nb = stat_blocks<DENSE>(p, k);
  // wave 0 turns the per-wave sums of block pb into p (after the barrier that follows them)
  auto finish_block = [&](int pb) {
    if (wave == 0 && lane < kSB) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += sm.wsum[pb & 1][w][lane];
      const float pv = s * inv_h;
      const int pos = slot_pos<DENSE>(sm, pb, lane, p, k);
      if (pos >= 0) {
        if constexpr (DENSE) {
          p_out[i * ld + pos] = pv;
        } else {
          if (pv > 0.f) a_plogp += pv * logf(pv);
          a_pi += pv * sm.sc[pb * kSB + lane];
        }
      }
    }
  };
  stat_gather<DENSE, NW>(sm, lat, 0, 0, p, k);
  for (int blk = 0; blk < nb; ++blk) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();  // block blk landed everywhere; the sums of block blk - 1 are complete
    if (blk > 0) finish_block(blk - 1);
    if (blk + 1 < nb) stat_gather<DENSE, NW>(sm, lat, blk + 1, (blk + 1) & 1, p, k);
    f32x4 st[2];
    stat_qk(sm.tile[blk & 1], qf, st);
    // lane (c, g): e = 2^(x - L_c) of keys 16 kt + 4 g + r; sum over the 16 heads (lanes c)
    float e[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = slot_pos<DENSE>(sm, blk, 16 * kt + 4 * g + r, p, k) >= 0;
        e[4 * kt + r] = (ok && lh > -INFINITY) ? exp2f(st[kt][r] * scale_log2 - lh) : 0.f;
      }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] += __shfl_xor(e[j], d);
    if (c == 0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.wsum[blk & 1][wave][16 * kt + 4 * g + r] = e[4 * kt + r];
    }
  }
  __syncthreads();
  if (nb > 0) finish_block(nb - 1);
  if constexpr (!DENSE) {
    if (wave == 0) {
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        a_plogp += __shfl_xor(a_plogp, d);
        a_pi += __shfl_xor(a_pi, d);
      }
      if (lane == 0) {
        // no valid slot: every sum is 0 and so is the divergence
        kl[i] = (accumulate ? kl[i] : 0.f) + weight * (a_plogp - a_pi + lse_i);
      }
    }
  }
}

// recall[i] = counts[i] / min(k, t + 1): the share of the dense attention's top-k that the
// model's selection contains.
__global__ void recall_kernel(const int32_t* __restrict__ counts, dsa_seqs seqs, int64_t n_q, int k,
                              float* __restrict__ recall) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_q) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const int64_t m = p + 1 < k ? p + 1 : k;
  recall[i] = (float)counts[i] / (float)m;
}

// Deterministic sum of n floats into out[0] (one workgroup, fixed order).
__global__ __launch_bounds__(256) void row_sum_kernel(const float* __restrict__ x, int64_t n, float* __restrict__ out) {
  __shared__ float part[256];
  float s = 0.f;
  for (int64_t j = threadIdx.x; j < n; j += 256) s += x[j];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int d = 128; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) part[threadIdx.x] += part[threadIdx.x + d];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = part[0];
}

template <bool DENSE>
hipError_t launch_lse(const StatArgs& a, float* lse_out, const float* lse_dense, float* mass_head, float* mass,
                      hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  const float sl2 = a.scale * 1.4426950408889634f;
#define DSA_LSE(NWv)                                                                                         \
  if (a.n_h == 16 * NWv) {                                                                                   \
    hipLaunchKernelGGL((attn_lse_kernel<NWv, DENSE>), dim3((unsigned)n_q), dim3(64 * NWv), 0, st, a.q,       \
                       a.latent, a.idx, a.n_h, a.k, sl2, a.seqs, n_q, lse_out, lse_dense, mass_head, mass); \
    return hipGetLastError();                                                                                \
  }
  DSA_LSE(1) DSA_LSE(2) DSA_LSE(4) DSA_LSE(8)
#undef DSA_LSE
  return hipErrorInvalidValue;
}

template <bool DENSE>
hipError_t launch_p(const StatArgs& a, const float* scores, const float* lse, float* p_out, int64_t ld, float* kl,
                    float weight, int accumulate, hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  const float sl2 = a.scale * 1.4426950408889634f;
#define DSA_P(NWv)                                                                                            \
  if (a.n_h == 16 * NWv) {                                                                                    \
    hipLaunchKernelGGL((attn_p_kernel<NWv, DENSE>), dim3((unsigned)n_q), dim3(64 * NWv), 0, st, a.q, a.latent, \
                       a.idx, scores, a.n_h, a.k, sl2, a.seqs, n_q, lse, p_out, ld, kl, weight, accumulate);   \
    return hipGetLastError();                                                                                 \
  }
  DSA_P(1) DSA_P(2) DSA_P(4) DSA_P(8)
#undef DSA_P
  return hipErrorInvalidValue;
}

}  // namespace

size_t attn_mass_ws(const StatArgs& a, bool recall) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  size_t b = 2 * (size_t)n_q * a.n_h * sizeof(float) + 1024;
  if (recall) b += (size_t)n_q * slab_ld(a.seqs) * sizeof(float) + (size_t)n_q * a.k * 4 + (size_t)n_q * 4 + 1024;
  return b;
}

hipError_t launch_attention_mass(const StatArgs& a, float* mass_head, float* mass, float* recall, void* ws,
                                 hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  if (n_q == 0) return hipSuccess;
  uintptr_t w = ((uintptr_t)ws + 255) & ~(uintptr_t)255;
  float* lse_d = (float*)w;
  float* lse_s = lse_d + n_q * a.n_h;
  hipError_t e = launch_lse<true>(a, lse_d, nullptr, nullptr, nullptr, st);
  if (e != hipSuccess) return e;
  e = launch_lse<false>(a, lse_s, lse_d, mass_head, mass, st);
  if (e != hipSuccess || !recall) return e;
  const int64_t ld = slab_ld(a.seqs);
  uintptr_t w2 = ((uintptr_t)(lse_s + n_q * a.n_h) + 255) & ~(uintptr_t)255;
  float* slab = (float*)w2;
  int32_t* oidx = (int32_t*)(((uintptr_t)(slab + n_q * ld) + 255) & ~(uintptr_t)255);
  int32_t* counts = oidx + n_q * a.k;
  e = launch_p<true>(a, nullptr, lse_d, slab, ld, nullptr, 0.f, 0, st);
  if (e != hipSuccess) return e;
  IndexerArgs ia{};
  ia.k = a.k;
  ia.seqs = a.seqs;
  ia.idx_out = oidx;
  ia.score_out = nullptr;
  e = launch_topk_select(ia, slab, st);
  if (e != hipSuccess) return e;
  e = launch_index_overlap(oidx, a.idx, n_q, a.k, counts, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(recall_kernel, dim3((unsigned)((n_q + 255) / 256)), dim3(256), 0, st, counts, a.seqs, n_q, a.k,
                     recall);
  return hipGetLastError();
}

size_t indexer_kl_ws(const StatArgs& a) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  return (size_t)n_q * a.n_h * sizeof(float) + 256;
}

hipError_t launch_indexer_kl(const StatArgs& a, const float* scores, float weight, int accumulate, float* kl,
                             float* loss, void* ws, hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  if (n_q == 0) return hipSuccess;
  float* lse_s = (float*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  hipError_t e = launch_lse<false>(a, lse_s, nullptr, nullptr, nullptr, st);
  if (e != hipSuccess) return e;
  e = launch_p<false>(a, scores, lse_s, nullptr, 0, kl, weight, accumulate, st);
  if (e != hipSuccess || !loss) return e;
  hipLaunchKernelGGL(row_sum_kernel, dim3(1), dim3(256), 0, st, kl, n_q, loss);
  return hipGetLastError();
}

}  // namespace dsa
