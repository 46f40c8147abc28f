// Lightning-indexer scores into a per-row score slab, then an exact per-row top-k.
//
// Score ([IDX] §4, lightning-indexer equation): I[t,s] = sum_j w[t,j] ReLU(q_idx[t,j,:] . k_idx[s,:])
// over the visible keys s <= t.  Selection ([IDX] §2 TopK; §6.5 deterministic):
// the k largest scores, ties to the lower position, -0.0 == +0.0.
//
// This is the general path (any number of sequences, any query count): it is
// the decode path (one query per sequence, keys split over many workgroups) and
// the reference GPU path for prefill.  Per-row work is independent, so the slab
// is written once and read by the selection kernel.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x128_f8f6f4):
//   rows  (M) = 16 indexer heads of one query, columns (N) = 16 keys,
//   K = the head dimension.  Lane l supplies head/key (l % 16) and the K slice
//   selected by (l / 16); the result puts key (l % 16) and heads 4*(l/16)+r in
//   lane l, so the head-weighted ReLU sum is an in-lane loop plus a reduction
//   across the four 16-lane groups.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

constexpr int kScoreKeysPerWave = 256;

template <int HB, int D>
__global__ __launch_bounds__(256, 4) void idx_score_bf16_kernel(const uint16_t* __restrict__ q_idx,
                                                             const uint16_t* __restrict__ k_idx,
                                                             const uint16_t* __restrict__ w, int H, dsa_seqs seqs,
                                                             int64_t n_q, float* __restrict__ slab, int64_t ld,
                                                             int bf16_scores, uint32_t* __restrict__ zero,
                                                             int64_t zero_words) {
  // workgroup (0, 0) first clears the wide select's counters and histograms when asked
  // (zero != null): they are read by the passes after this kernel, and the stream orders
  // those after every workgroup here (the separate clearing launch is saved)
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int64_t j = threadIdx.x; j < zero_words; j += 256) zero[j] = 0u;
  // the wave index is uniform (a scalar register), so are the row and its key base
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t i = (int64_t)blockIdx.y * 4 + wave;
  if (i >= n_q) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const int64_t s0 = (int64_t)blockIdx.x * kScoreKeysPerWave;
  if (s0 > p) return;
  const int64_t krow0 = seqs.k_start[b];
  const int c = lane & 15, g = lane >> 4;
  constexpr int KS = D / 32;
  // the wave's keys from a uniform base and a 32-bit lane offset (no per-lane 64-bit
  // address arithmetic); the last visible key relative to the base, at most the chunk's last
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k_idx + (krow0 + s0) * D);
  const int rel_last = (int)min<int64_t>(p - s0, kScoreKeysPerWave - 1);

  i32x4 a[HB][KS];
  // head weights of heads 16 hb + 4 g + r kept as bf16 pairs (r = 2 e, 2 e + 1), widened
  // to fp32 (exactly) where used: eight registers fewer, so four waves fit on a SIMD and
  // keep more key loads in flight
  uint32_t wl2[HB][2];
  // Padded heads (H < 16 HB) load a real head's q and weight from a clamped index and are
  // zeroed by a select: no load sits in a branch, so the compiler issues them all before
  // the first wait (a guarded load per weight had cost a memory round trip each).
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 16 * hb + c;
    const int hq = min(head, H - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(q_idx + (i * H + hq) * D + 32 * ks + 8 * g);
      a[hb][ks] = head < H ? v : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int hh = 16 * hb + 4 * g + 2 * e;
      const uint32_t lo = w[i * H + min(hh, H - 1)], hi = w[i * H + min(hh + 1, H - 1)];
      wl2[hb][e] = (hh < H ? lo : 0u) | ((hh + 1 < H ? hi : 0u) << 16);
    }
  }
  auto wl = [&](int hb, int r) {
    const uint32_t x = wl2[hb][r >> 1];
    return __uint_as_float((r & 1) ? (x & 0xFFFF0000u) : (x << 16));
  };

  // 16 keys per step; the keys of step sb + 1 are loaded while step sb is scored.
  // Rows past the visible prefix load row p (in bounds) and are not written.  Scores
  // collect in LDS and leave in one pass at the end: a global store per step would sit
  // in the same in-order memory counter as the key loads, so that every step's wait for
  // its keys also waited for the previous step's store.
  const int nsb = (int)min<int64_t>(kScoreKeysPerWave / 16, (p - s0) / 16 + 1);
  __shared__ float sbuf[4][kScoreKeysPerWave];
  auto load = [&](int sb, i32x4 (&bf)[KS]) {
    const uint32_t off = (uint32_t)min(16 * sb + c, rel_last) * (2 * D) + 16 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bf[ks] = *reinterpret_cast<const i32x4*>(kbase + off + 64 * ks);
  };
  auto score = [&](int sb, const i32x4 (&bf)[KS]) {
    float part = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16_16x16x32(a[hb][ks], bf[ks], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) part += wl(hb, r) * relu_bits(acc[r]);
    }
    // sum over the four 16-lane rows (heads 4g + r) by two permlane swaps
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    part = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    part = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    if (bf16_scores) part = __uint_as_float(f32_to_bf16_bits(part) << 16);
    if (g == 0) sbuf[wave][16 * sb + c] = part;
  };
  i32x4 bfa[KS], bfb[KS];
  load(0, bfa);
  for (int sb = 0; sb < nsb; sb += 2) {
    if (sb + 1 < nsb) load(sb + 1, bfb);
    score(sb, bfa);
    if (sb + 1 >= nsb) break;
    if (sb + 2 < nsb) load(sb + 2, bfa);
    score(sb + 1, bfb);
  }
  // in each group of 256 keys lane l writes the scores of keys 4 l .. + 3 (one 16-byte store
  // where the whole quad is visible and the row start is 16-byte aligned); the wave reads
  // only its own LDS row, which its own earlier writes fill (LDS operations of a wave are
  // ordered)
  static_assert(kScoreKeysPerWave % 256 == 0, "whole groups of 256 keys per wave");
#pragma unroll
  for (int gq = 0; gq < kScoreKeysPerWave / 256; ++gq) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&sbuf[wave][256 * gq + 4 * lane]);
    const int64_t sl = s0 + 256 * gq + 4 * lane;
    float* dst = slab + i * ld + sl;
    if (sl + 3 <= p && (((i * ld) & 3) == 0)) {
      *reinterpret_cast<f32x4*>(dst) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (sl + e <= p) dst[e] = v[e];
    }
  }
}

// fp8 e4m3: d == 128, one K=128 MFMA per (16 heads x 16 keys).  The positive
// per-row scales leave the ReLU: w' = w * q_scale folds in before the head sum
// and k_scale multiplies the finished score.
template <int HB>
__global__ __launch_bounds__(256) void idx_score_fp8_kernel(const uint8_t* __restrict__ q_idx,
                                                            const float* __restrict__ q_scale,
                                                            const uint8_t* __restrict__ k_idx,
                                                            const float* __restrict__ k_scale,
                                                            const uint16_t* __restrict__ w, int H, dsa_seqs seqs,
                                                            int64_t n_q, float* __restrict__ slab, int64_t ld,
                                                            int bf16_scores, uint32_t* __restrict__ zero,
                                                            int64_t zero_words) {
  // workgroup (0, 0) first clears the wide select's counters and histograms when asked
  // (zero != null): they are read by the passes after this kernel, and the stream orders
  // those after every workgroup here (the separate clearing launch is saved)
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int64_t j = threadIdx.x; j < zero_words; j += 256) zero[j] = 0u;
  constexpr int D = 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.y * 4 + wave;
  if (i >= n_q) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const int64_t s0 = (int64_t)blockIdx.x * kScoreKeysPerWave;
  if (s0 > p) return;
  const int64_t krow0 = seqs.k_start[b];
  const int c = lane & 15, g = lane >> 4;

  i32x8 a[HB];
  float wl[HB][4];
  // padded heads: clamped loads and a select, no load in a branch (as in the bf16 kernel)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 16 * hb + c;
    const int hq = min(head, H - 1);
    const i32x4* src = reinterpret_cast<const i32x4*>(q_idx + (i * H + hq) * D + 32 * g);
    const i32x4 lo = src[0], hi = src[1];
    a[hb] = head < H ? i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]} : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 16 * hb + 4 * g + r;
      const int hc = min(hh, H - 1);
      const float wv = bf16_to_f32(w[i * H + hc]) * q_scale[i * H + hc];
      wl[hb][r] = hh < H ? wv : 0.f;
    }
  }

  for (int sb = 0; sb < kScoreKeysPerWave / 16; ++sb) {
    const int64_t sbase = s0 + 16 * sb;
    if (sbase > p) break;
    const int64_t s = sbase + c;
    i32x8 bf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    float ks = 0.f;
    if (s <= p) {
      const i32x4* src = reinterpret_cast<const i32x4*>(k_idx + (krow0 + s) * D + 32 * g);
      i32x4 lo = src[0], hi = src[1];
      bf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      ks = k_scale[krow0 + s];
    }
    float part = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_fp8_16x16x128(a[hb], bf, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) part += wl[hb][r] * relu_bits(acc[r]);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    float sc = part * ks;
    if (bf16_scores) sc = __uint_as_float(f32_to_bf16_bits(sc) << 16);
    if (g == 0 && s <= p) slab[i * ld + s] = sc;
  }
}

// ----------------------------------------------------------------------------
// Exact top-k of one slab row per workgroup (1024 threads).
//
// Radix select on the 32-bit order keys, digits of 11, 11 and 10 bits, finds the
// k-th largest key T and how many keys exceed it; the output pass then walks the
// row in position order, keeping every key > T and the lowest-position keys == T
// until k are taken.  Positions therefore come out ascending.
// ----------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

struct SelShared {
  uint32_t hist[2048];
  uint32_t wave_tot[kSelWaves];
  uint32_t wave_tot2[2][kSelWaves];
  uint32_t digit, above;
};

// Suffix sums over the histogram: thread t owns bins 2t and 2t+1.
__device__ void sel_find_digit(SelShared& sh, int nbins, uint32_t remaining) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int b0 = 2 * t, b1 = 2 * t + 1;
  const uint32_t h0 = b0 < nbins ? sh.hist[b0] : 0u;
  const uint32_t h1 = b1 < nbins ? sh.hist[b1] : 0u;
  uint32_t v = h0 + h1;
  // inclusive suffix scan inside the wave (higher lanes own higher bins)
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t o = __shfl_down(v, d);
    if (lane + d < 64) v += o;
  }
  if (lane == 0) sh.wave_tot[wv] = v;
  __syncthreads();
  uint32_t higher_waves = 0;
  for (int w2 = wv + 1; w2 < kSelWaves; ++w2) higher_waves += sh.wave_tot[w2];
  const uint32_t incl = v + higher_waves;            // sum of bins >= b0
  const uint32_t above1 = incl - (h0 + h1);          // sum of bins > b1
  if (above1 < remaining && remaining <= above1 + h1) {
    sh.digit = b1;
    sh.above = above1;
  } else if (above1 + h1 < remaining && remaining <= incl) {
    sh.digit = b0;
    sh.above = above1 + h1;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const float* __restrict__ slab, int64_t ld,
                                                                  dsa_seqs seqs, int64_t n_q, int k,
                                                                  int32_t* __restrict__ idx_out,
                                                                  float* __restrict__ score_out) {
  __shared__ SelShared sh;
  const int64_t i = blockIdx.x;
  if (i >= n_q) return;
  const int b = seq_of_row(seqs, i);
  const int64_t n = row_last(seqs, b, i) + 1;
  const float* row = slab + i * ld;
  int32_t* orow = idx_out + i * (int64_t)k;
  float* srow = score_out ? score_out + i * (int64_t)k : nullptr;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;

  if (n <= k) {
    for (int64_t j = t; j < k; j += kSelThreads) {
      orow[j] = j < n ? (int32_t)j : -1;
      if (srow) srow[j] = j < n ? row[j] : 0.f;
    }
    return;
  }

  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)k;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int nb = 1 << widths[pass];
    const uint32_t dmask = (uint32_t)(nb - 1);
    for (int j = t; j < 2048; j += kSelThreads) sh.hist[j] = 0u;
    __syncthreads();
    for (int64_t s = t; s < n; s += kSelThreads) {
      const uint32_t key = order_key(row[s]);
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shifts[pass]) & dmask], 1u);
    }
    __syncthreads();
    sel_find_digit(sh, nb, remaining);
    prefix |= sh.digit << shifts[pass];
    pmask |= dmask << shifts[pass];
    remaining -= sh.above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = remaining;  // how many keys equal to T are taken (lowest positions)

  uint32_t eq_before = 0, sel_before = 0;
  int parity = 0;
  for (int64_t base = 0; base < n; base += kSelThreads, parity ^= 1) {
    const int64_t s = base + t;
    const float v = s < n ? row[s] : 0.f;
    const uint32_t key = s < n ? order_key(v) : 0u;
    const bool gt = s < n && key > T;
    const bool eq = s < n && key == T;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t eq_ball = __ballot(eq);
    if (lane == 0) sh.wave_tot[wv] = __popcll(eq_ball);
    __syncthreads();
    uint32_t eq_wave_before = 0, eq_total = 0;
    for (int w2 = 0; w2 < kSelWaves; ++w2) {
      const uint32_t c2 = sh.wave_tot[w2];
      if (w2 < wv) eq_wave_before += c2;
      eq_total += c2;
    }
    const uint32_t eq_rank = eq_before + eq_wave_before + (uint32_t)__popcll(eq_ball & lt_mask);
    const bool sel = gt || (eq && eq_rank < need_eq);
    const uint64_t sel_ball = __ballot(sel);
    if (lane == 0) sh.wave_tot2[parity][wv] = __popcll(sel_ball);
    __syncthreads();
    uint32_t sel_wave_before = 0, sel_total = 0;
    for (int w2 = 0; w2 < kSelWaves; ++w2) {
      const uint32_t c2 = sh.wave_tot2[parity][w2];
      if (w2 < wv) sel_wave_before += c2;
      sel_total += c2;
    }
    if (sel) {
      const uint32_t pos = sel_before + sel_wave_before + (uint32_t)__popcll(sel_ball & lt_mask);
      if (pos < (uint32_t)k) orow[pos] = (int32_t)s;
      if (srow && pos < (uint32_t)k) srow[pos] = v;
    }
    eq_before += eq_total;
    sel_before += sel_total;
    if (sel_before >= (uint32_t)k) break;  // uniform: every thread sees the same totals
  }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
int64_t slab_ld(const dsa_seqs& s) {
  int64_t mx = 1;
  for (int b = 0; b < s.B; ++b) {
    const int64_t nq = s.q_start[b + 1] - s.q_start[b];
    if (nq <= 0) continue;
    const int64_t t = s.q_pos0[b] + nq - 1;                 // the sequence's last query position
    const int64_t n = s.block > 1 ? t / s.block : t + 1;    // keys it sees
    mx = mx > n ? mx : n;
  }
  return (mx + 3) & ~int64_t(3);
}

hipError_t launch_indexer_slab(const IndexerArgs& a, float* slab, hipStream_t st, uint32_t* zero, int64_t zero_words) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  if (n_q == 0) return hipSuccess;
  const int64_t ld = slab_ld(a.seqs);
  dim3 grid((unsigned)((ld + kScoreKeysPerWave - 1) / kScoreKeysPerWave), (unsigned)((n_q + 3) / 4));
  const int HB = (a.H + 15) / 16;
  const int bf16s = a.flags & DSA_TOPK_BF16_SCORES;
  if (a.qk_dtype == DSA_BF16) {
    const uint16_t* q = (const uint16_t*)a.q_idx;
    const uint16_t* kk = (const uint16_t*)a.k_idx;
#define DSA_SCORE_BF16(HBv, Dv)                                                                        \
  if (HB == HBv && a.d == Dv) {                                                                      \
    hipLaunchKernelGGL((idx_score_bf16_kernel<HBv, Dv>), grid, dim3(256), 0, st, q, kk, a.w, a.H, a.seqs, \
                       n_q, slab, ld, bf16s, zero, zero_words);                                             \
    return hipGetLastError();                                                                        \
  }
    DSA_SCORE_BF16(1, 64) DSA_SCORE_BF16(1, 128) DSA_SCORE_BF16(2, 64) DSA_SCORE_BF16(2, 128)
    DSA_SCORE_BF16(4, 64) DSA_SCORE_BF16(4, 128)
#undef DSA_SCORE_BF16
  } else {
    const uint8_t* q = (const uint8_t*)a.q_idx;
    const uint8_t* kk = (const uint8_t*)a.k_idx;
#define DSA_SCORE_FP8(HBv)                                                                                 \
  if (HB == HBv && a.d == 128) {                                                                         \
    hipLaunchKernelGGL((idx_score_fp8_kernel<HBv>), grid, dim3(256), 0, st, q, a.q_scale, kk, a.k_scale, a.w, \
                       a.H, a.seqs, n_q, slab, ld, bf16s, zero, zero_words);                              \
    return hipGetLastError();                                                                            \
  }
    DSA_SCORE_FP8(1) DSA_SCORE_FP8(2) DSA_SCORE_FP8(4)
#undef DSA_SCORE_FP8
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk_select(const IndexerArgs& a, const float* slab, hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  if (n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)n_q), dim3(kSelThreads), 0, st, slab, slab_ld(a.seqs),
                     a.seqs, n_q, a.k, a.idx_out, a.score_out);
  return hipGetLastError();
}

}  // namespace dsa
