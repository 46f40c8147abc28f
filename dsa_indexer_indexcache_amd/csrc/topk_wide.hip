// Exact top-k over few, long score rows (decode: a handful of queries, each over
// its own 10^5-key context) spread over many workgroups.
//
// Selection rule ([IDX] §2 TopK, §6.5 deterministic): the k largest scores of the
// row, ties to the lower position, i.e. the k largest 64-bit keys
// order(score) << 32 | ~position; output positions ascending, scores alongside.
//
// One workgroup per row would leave most of the chip idle and serialise the row's
// passes on one CU.  Instead every row is cut into chunks of kWChunk keys:
//   zero    : per-row counters and histograms, cleared by the score kernel (the first workgroup);
//   hist    : (chunk, row) workgroups histogram the top 11 key bits (2048 bins) in
//             LDS and add them into the row's global histogram;
//   collect : every chunk finds the bin d holding the k-th key from that histogram,
//             counts its keys in bins above d, and appends the keys in bin d to the
//             row's candidate list;
//   resolve : one workgroup per row finishes the radix select over the candidates
//             (bits below the common 11-bit prefix, 8 at a time) and counts, per
//             chunk, how many of them are taken;
//   write   : every chunk writes its selected positions in order at its offset
//             (a prefix over the earlier chunks' counts).
// If the threshold bin holds more keys than the candidate list can take, resolve
// reads the bin's keys back from the score row instead (slower, same result).
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kWChunk = 4096;     // keys per chunk
constexpr int kWThreads = 256;    // chunk workgroups: 16 keys per thread
constexpr int kWPer = kWChunk / kWThreads;
constexpr int kWBins = 2048;      // first level: top 11 bits of the 32-bit order key
constexpr int kWShift1 = 21;
constexpr int kWCandCap = 16384;  // candidates per row
constexpr int kWMaxChunks = 2048; // rows up to 8M keys
constexpr int kWResThreads = 1024;

// per-row state, in 32-bit words
struct RowMeta {
  uint32_t cand_cnt;
  int32_t d1;       // threshold bin, -1 when the row has at most k keys
  uint32_t above1;  // keys in bins above d1
  uint32_t pad;
  uint64_t t64;     // taken from bin d1  <=>  key64 >= t64
};

struct WideWs {
  uint32_t* hist;    // [n_q][kWBins]
  RowMeta* meta;     // [n_q]
  uint32_t* gt;      // [n_q][mc]  keys of chunk c in bins above d1
  uint32_t* eq;      // [n_q][mc]  keys of chunk c taken from bin d1
  uint64_t* cand;    // [n_q][kWCandCap]
};

__device__ __forceinline__ uint64_t wkey64(uint32_t key, uint32_t pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}

__device__ __forceinline__ int64_t row_len(const dsa_seqs& s, int64_t i) {
  const int b = seq_of_row(s, i);
  return row_last(s, b, i) + 1;
}

// Scores of keys sb .. sb + kWPer - 1 of a slab row with n valid keys (0 past the end):
// four 16-byte loads when the group lies inside the row (its start is 16-byte aligned:
// the row pitch and sb are multiples of 4), else scalar loads of clamped, in-row
// positions.  No load sits in a branch of its own, so all are issued before the first
// wait (a guarded load per key had cost a memory round trip each).
__device__ __forceinline__ void load_group(const float* row, int64_t sb, int64_t n, float (&v)[kWPer]) {
  if (sb + kWPer <= n) {
#pragma unroll
    for (int q = 0; q < kWPer / 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(row + sb + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
    }
  } else {
    const int64_t last = n > 0 ? n - 1 : 0;
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const float x = row[min(sb + j, last)];
      v[j] = sb + j < n ? x : 0.f;
    }
  }
}

__global__ __launch_bounds__(kWThreads) void wsel_hist_kernel(const float* __restrict__ slab, int64_t ld,
                                                               dsa_seqs seqs, WideWs w) {
  __shared__ uint32_t lh[kWBins];
  const int64_t i = blockIdx.y;
  const int64_t n = row_len(seqs, i);
  const int64_t s0 = (int64_t)blockIdx.x * kWChunk;
  if (s0 >= n) return;
  for (int j = threadIdx.x; j < kWBins; j += kWThreads) lh[j] = 0u;
  __syncthreads();
  const float* row = slab + i * ld;
  // all loads first (clamped in-row positions, no load in a branch), then the counts
  float x[kWPer];
#pragma unroll
  for (int j = 0; j < kWPer; ++j) x[j] = row[min(s0 + j * kWThreads + threadIdx.x, n - 1)];
#pragma unroll
  for (int j = 0; j < kWPer; ++j)
    if (s0 + j * kWThreads + threadIdx.x < n) atomicAdd(&lh[order_key(x[j]) >> kWShift1], 1u);
  __syncthreads();
  uint32_t* gh = w.hist + i * kWBins;
  for (int j = threadIdx.x; j < kWBins; j += kWThreads)
    if (lh[j]) atomicAdd(&gh[j], lh[j]);
}

// The bin holding the k-th largest key of row i and the count above it, from the
// row's global histogram (every chunk workgroup computes it; same result everywhere).
__device__ void find_bin(const uint32_t* gh, int k, int64_t n, int* d1_out, uint32_t* above_out) {
  __shared__ uint32_t part[kWThreads];
  __shared__ int s_d1;
  __shared__ uint32_t s_above;
  const int t = threadIdx.x;
  constexpr int per = kWBins / kWThreads;  // 8 consecutive bins per thread
  uint32_t h[per];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    h[j] = gh[t * per + j];
    local += h[j];
  }
  part[t] = local;
  if (t == 0) {
    s_d1 = -1;
    s_above = 0u;
  }
  __syncthreads();
  // suffix sums over threads (bins above this thread's range), Hillis-Steele in LDS
  for (int d = 1; d < kWThreads; d <<= 1) {
    const uint32_t o = t + d < kWThreads ? part[t + d] : 0u;
    __syncthreads();
    part[t] += o;
    __syncthreads();
  }
  if (n > k) {
    uint32_t above = part[t] - local;  // keys in bins above 8t + 7
#pragma unroll
    for (int j = per - 1; j >= 0; --j) {
      if (above < (uint32_t)k && (uint32_t)k <= above + h[j]) {
        s_d1 = t * per + j;
        s_above = above;
      }
      above += h[j];
    }
  }
  __syncthreads();
  *d1_out = s_d1;
  *above_out = s_above;
}

__global__ __launch_bounds__(kWThreads) void wsel_collect_kernel(const float* __restrict__ slab, int64_t ld,
                                                                  dsa_seqs seqs, int k, int mc, WideWs w) {
  __shared__ uint32_t scan[kWThreads];
  __shared__ uint32_t s_base;
  const int64_t i = blockIdx.y;
  const int c = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = row_len(seqs, i);
  const int64_t s0 = (int64_t)c * kWChunk;
  int d1;
  uint32_t above1;
  find_bin(w.hist + i * kWBins, k, n, &d1, &above1);
  if (c == 0 && t == 0) {
    w.meta[i].d1 = d1;
    w.meta[i].above1 = above1;
  }
  // thread t owns keys s0 + 16t .. s0 + 16t + 15
  const float* row = slab + i * ld;
  uint32_t key[kWPer];
  uint32_t gt = 0, nc = 0, candm = 0;
  float x[kWPer];
  load_group(row, s0 + (int64_t)t * kWPer, n, x);
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const int64_t s = s0 + (int64_t)t * kWPer + j;
    const bool ok = s < n;
    key[j] = ok ? order_key(x[j]) : 0u;
    const int bin = (int)(key[j] >> kWShift1);
    gt += (ok && bin > d1) ? 1u : 0u;
    const bool cand = ok && bin == d1;
    nc += cand ? 1u : 0u;
    candm |= (cand ? 1u : 0u) << j;
  }
  // candidate slots: exclusive scan of the per-thread counts, one reservation per
  // workgroup (same-address atomics from every wave serialise at L2)
  scan[t] = nc;
  __syncthreads();
  for (int d = 1; d < kWThreads; d <<= 1) {
    const uint32_t o = t >= d ? scan[t - d] : 0u;
    __syncthreads();
    scan[t] += o;
    __syncthreads();
  }
  if (t == kWThreads - 1) s_base = scan[t] ? atomicAdd(&w.meta[i].cand_cnt, scan[t]) : 0u;
  uint32_t mine = scan[t] - nc;
  __syncthreads();
  const uint32_t base = s_base;
  if (candm) {
    uint32_t idx = base + mine;
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      if (candm >> j & 1u) {
        if (idx < (uint32_t)kWCandCap)
          w.cand[i * kWCandCap + idx] = wkey64(key[j], (uint32_t)(s0 + (int64_t)t * kWPer + j));
        ++idx;
      }
    }
  }
  // chunk total of keys above the threshold bin
  scan[t] = gt;
  __syncthreads();
  for (int d = kWThreads / 2; d >= 1; d >>= 1) {
    if (t < d) scan[t] += scan[t + d];
    __syncthreads();
  }
  if (t == 0) w.gt[i * mc + c] = scan[0];
}

// Exact select inside the threshold bin; one workgroup per row.
__global__ __launch_bounds__(kWResThreads) void wsel_resolve_kernel(const float* __restrict__ slab, int64_t ld,
                                                                     dsa_seqs seqs, int k, int mc, WideWs w,
                                                                     int32_t* __restrict__ idx_out,
                                                                     float* __restrict__ score_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t eqc[kWMaxChunks];
  __shared__ uint32_t s_digit, s_above, s_cnt;
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = row_len(seqs, i);
  const RowMeta meta = w.meta[i];
  for (int c = t; c < mc; c += kWResThreads) eqc[c] = 0u;
  if (meta.d1 < 0) {
    // at most k keys: all of them are taken, the rest of the row is padding
    for (int64_t j = n + t; j < k; j += kWResThreads) {
      idx_out[i * (int64_t)k + j] = -1;
      if (score_out) score_out[i * (int64_t)k + j] = 0.f;
    }
    __syncthreads();
    for (int c = t; c < mc; c += kWResThreads) w.eq[i * mc + c] = 0u;
    if (t == 0) w.meta[i].t64 = 0ull;
    return;
  }
  const bool from_list = meta.cand_cnt <= (uint32_t)kWCandCap;
  const int64_t n_items = from_list ? (int64_t)meta.cand_cnt : n;
  const uint64_t* cand = w.cand + i * kWCandCap;
  const float* row = slab + i * ld;
  // item j of the bin: a key64, or 0 (never taken: real keys are > 0) for row
  // entries outside the bin when reading the row back
  auto item = [&](int64_t j) -> uint64_t {
    if (from_list) return cand[j];
    const uint32_t key = order_key(row[j]);
    return (int)(key >> kWShift1) == meta.d1 ? wkey64(key, (uint32_t)j) : 0ull;
  };
  // all items share the top 11 bits; select the remaining k - above1 largest
  uint32_t remaining = (uint32_t)k - meta.above1;
  uint64_t prefix = (uint64_t)meta.d1 << (32 + kWShift1);
  uint64_t pmask = ~0ull << (32 + kWShift1);
  for (int shift = 32 + kWShift1 - 8;; shift -= 8) {
    if (shift < 0) shift = 0;
    for (int b = t; b < 256; b += kWResThreads) hist[b] = 0u;
    __syncthreads();
    for (int64_t j = t; j < n_items; j += kWResThreads) {
      const uint64_t kk = item(j);
      if (kk != 0ull && (kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (t < 64) {
      uint32_t h[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) h[b] = hist[4 * t + b];
      const uint32_t local = h[0] + h[1] + h[2] + h[3];
      uint32_t incl = local;
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_down(incl, d);
        if (t + d < 64) incl += o;
      }
      uint32_t above = incl - local;
      for (int b = 3; b >= 0; --b) {
        if (above < remaining && remaining <= above + h[b]) {
          s_digit = 4 * t + b;
          s_above = above;
          s_cnt = h[b];
        }
        above += h[b];
      }
    }
    __syncthreads();
    const uint32_t digit = s_digit, ab = s_above, cnt = s_cnt;
    __syncthreads();
    prefix |= (uint64_t)digit << shift;
    pmask |= (uint64_t)0xFFu << shift;
    remaining -= ab;
    if (cnt == remaining || shift == 0) break;  // the whole bin is taken
  }
  const uint64_t t64 = prefix;  // taken from bin d1  <=>  key64 >= t64
  for (int64_t j = t; j < n_items; j += kWResThreads) {
    const uint64_t kk = item(j);
    if (kk != 0ull && kk >= t64) {
      const uint32_t pos = 0xFFFFFFFFu - (uint32_t)kk;
      atomicAdd(&eqc[pos / kWChunk], 1u);
    }
  }
  __syncthreads();
  for (int c = t; c < mc; c += kWResThreads) w.eq[i * mc + c] = eqc[c];
  if (t == 0) w.meta[i].t64 = t64;
}

__global__ __launch_bounds__(kWThreads) void wsel_write_kernel(const float* __restrict__ slab, int64_t ld,
                                                                dsa_seqs seqs, int k, int mc, WideWs w,
                                                                int32_t* __restrict__ idx_out,
                                                                float* __restrict__ score_out) {
  __shared__ uint32_t scan[kWThreads];
  __shared__ uint32_t s_base;
  const int64_t i = blockIdx.y;
  const int c = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = row_len(seqs, i);
  const int64_t s0 = (int64_t)c * kWChunk;
  if (s0 >= n) return;
  const RowMeta meta = w.meta[i];
  // output offset of this chunk: keys taken by the chunks before it
  uint32_t pre = 0;
  for (int c2 = t; c2 < c; c2 += kWThreads) pre += w.gt[i * mc + c2] + w.eq[i * mc + c2];
  scan[t] = pre;
  __syncthreads();
  for (int d = kWThreads / 2; d >= 1; d >>= 1) {
    if (t < d) scan[t] += scan[t + d];
    __syncthreads();
  }
  if (t == 0) s_base = scan[0];
  __syncthreads();
  const uint32_t base = s_base;
  __syncthreads();
  // thread t owns keys s0 + 16t .. s0 + 16t + 15 (consecutive: ordered output)
  const float* row = slab + i * ld;
  float v[kWPer];
  uint32_t selm = 0;
  load_group(row, s0 + (int64_t)t * kWPer, n, v);
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const int64_t s = s0 + (int64_t)t * kWPer + j;
    bool sel = false;
    if (s < n) {
      const uint32_t key = order_key(v[j]);
      const int bin = (int)(key >> kWShift1);
      sel = bin > meta.d1 || (bin == meta.d1 && wkey64(key, (uint32_t)s) >= meta.t64);
    }
    selm |= (sel ? 1u : 0u) << j;
  }
  const uint32_t cnt = __popc(selm);
  // exclusive scan of the per-thread counts (Hillis-Steele)
  scan[t] = cnt;
  __syncthreads();
  for (int d = 1; d < kWThreads; d <<= 1) {
    const uint32_t o = t >= d ? scan[t - d] : 0u;
    __syncthreads();
    scan[t] += o;
    __syncthreads();
  }
  uint32_t pos = base + scan[t] - cnt;
  int32_t* orow = idx_out + i * (int64_t)k;
  float* srow = score_out ? score_out + i * (int64_t)k : nullptr;
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    if (selm >> j & 1u) {
      if (pos < (uint32_t)k) {
        orow[pos] = (int32_t)(s0 + (int64_t)t * kWPer + j);
        if (srow) srow[pos] = v[j];
      }
      ++pos;
    }
  }
}

int wide_chunks(const IndexerArgs& a) { return (int)((slab_ld(a.seqs) + kWChunk - 1) / kWChunk); }

WideWs carve(const IndexerArgs& a, void* state) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  const int mc = wide_chunks(a);
  uintptr_t p = ((uintptr_t)state + 255) & ~(uintptr_t)255;
  WideWs w;
  w.cand = (uint64_t*)p;
  p += (size_t)n_q * kWCandCap * sizeof(uint64_t);
  w.meta = (RowMeta*)p;
  p += (size_t)n_q * sizeof(RowMeta);
  w.hist = (uint32_t*)p;
  p += (size_t)n_q * kWBins * sizeof(uint32_t);
  w.gt = (uint32_t*)p;
  p += (size_t)n_q * mc * sizeof(uint32_t);
  w.eq = (uint32_t*)p;
  return w;
}

}  // namespace

bool wide_select_ok(const IndexerArgs& a) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  const int64_t ld = slab_ld(a.seqs);
  return n_q >= 1 && n_q <= 64 && ld >= 8 * kWChunk && wide_chunks(a) <= kWMaxChunks;
}

size_t wide_select_ws(const IndexerArgs& a) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  const size_t mc = (size_t)wide_chunks(a);
  return 256 + (size_t)n_q * (kWCandCap * sizeof(uint64_t) + sizeof(RowMeta) + kWBins * sizeof(uint32_t) +
                              2 * mc * sizeof(uint32_t));
}

void wide_select_zero_region(const IndexerArgs& a, void* state, uint32_t** begin, int64_t* words) {
  // meta and hist are adjacent in the carve: the whole range [meta, hist + n_q bins)
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  const WideWs w = carve(a, state);
  static_assert(sizeof(RowMeta) % 4 == 0, "RowMeta in words");
  *begin = reinterpret_cast<uint32_t*>(w.meta);
  *words = n_q * (int64_t)(sizeof(RowMeta) / 4 + kWBins);
}

hipError_t launch_wide_select(const IndexerArgs& a, const float* slab, void* state, hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  if (n_q == 0) return hipSuccess;
  const int64_t ld = slab_ld(a.seqs);
  const int mc = wide_chunks(a);
  const WideWs w = carve(a, state);
  const dim3 grid((unsigned)mc, (unsigned)n_q);
  hipLaunchKernelGGL(wsel_hist_kernel, grid, dim3(kWThreads), 0, st, slab, ld, a.seqs, w);
  hipLaunchKernelGGL(wsel_collect_kernel, grid, dim3(kWThreads), 0, st, slab, ld, a.seqs, a.k, mc, w);
  hipLaunchKernelGGL(wsel_resolve_kernel, dim3((unsigned)n_q), dim3(kWResThreads), 0, st, slab, ld, a.seqs, a.k, mc,
                     w, a.idx_out, a.score_out);
  hipLaunchKernelGGL(wsel_write_kernel, grid, dim3(kWThreads), 0, st, slab, ld, a.seqs, a.k, mc, w, a.idx_out,
                     a.score_out);
  return hipGetLastError();
}

}  // namespace dsa
