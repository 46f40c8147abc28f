// Kernels beside the hot path: per-row fp8 quantisation of the indexer inputs
// (device side of the fp8 setting) and the cross-layer index overlap ([IDX] §8
// metrics): for every row, the number of valid positions two index tensors share.
//
// One workgroup per row.  When row B's valid positions span fewer than 2^18 values (any
// row over a context of at most 262,144 tokens), they are marked in a bitmap of that
// span in LDS and row A's valid positions test their bits: no probe loops, and the
// inserts are fire-and-forget LDS ORs.  Wider rows go into an open-addressing hash
// table in LDS (linear probing, at least twice as many slots as entries, so every
// probe sequence ends at an empty slot) that A's positions look up.  Valid entries of a
// row are distinct, so either way the hits sum to |A ∩ B|.  Integer work throughout:
// the count is exact.
#include <algorithm>
#include <climits>

#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kOvThreads = 256;
constexpr int kOvBitmapBits = 1 << 18;  // 32 KB of LDS

__device__ __forceinline__ uint32_t ov_hash(uint32_t v, uint32_t mask) { return (v * 2654435761u) >> 7 & mask; }

__global__ __launch_bounds__(kOvThreads) void idx_overlap_kernel(const int32_t* __restrict__ a,
                                                                 const int32_t* __restrict__ b, int k, int slots,
                                                                 int32_t* __restrict__ counts) {
  extern __shared__ int32_t table[];
  __shared__ int32_t wsum[kOvThreads / 64];
  __shared__ int32_t wmin[kOvThreads / 64], wmax[kOvThreads / 64];
  const int64_t row = blockIdx.x;
  const int32_t* rb = b + row * (int64_t)k;
  const int32_t* ra = a + row * (int64_t)k;
  int cnt = 0;

  // rows of at most 8 x 256 entries stay in registers (both rows loaded up front, so their
  // latencies overlap); longer rows are read again per pass
  constexpr int kReg = 8;
  const bool in_regs = k <= kReg * kOvThreads;
  int32_t rvb[kReg], rva[kReg];
  if (in_regs) {
#pragma unroll
    for (int m = 0; m < kReg; ++m) {
      const int j = m * kOvThreads + threadIdx.x;
      rvb[m] = j < k ? rb[j] : -1;
      rva[m] = j < k ? ra[j] : -1;
    }
  }

  // ---- span of B's valid entries (lo > hi: none)
  int lo = INT32_MAX, hi = -1;
  if (in_regs) {
#pragma unroll
    for (int m = 0; m < kReg; ++m)
      if (rvb[m] >= 0) {
        lo = min(lo, rvb[m]);
        hi = max(hi, rvb[m]);
      }
  } else {
    for (int j = threadIdx.x; j < k; j += kOvThreads) {
      const int32_t v = rb[j];
      if (v >= 0) {
        lo = min(lo, v);
        hi = max(hi, v);
      }
    }
  }
  for (int d = 32; d >= 1; d >>= 1) {
    lo = min(lo, __shfl_xor(lo, d));
    hi = max(hi, __shfl_xor(hi, d));
  }
  if ((threadIdx.x & 63) == 0) {
    wmin[threadIdx.x >> 6] = lo;
    wmax[threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  lo = wmin[0];
  hi = wmax[0];
#pragma unroll
  for (int w = 1; w < kOvThreads / 64; ++w) {
    lo = min(lo, wmin[w]);
    hi = max(hi, wmax[w]);
  }
  if (lo > hi) {  // no valid entry in B
    if (threadIdx.x == 0) counts[row] = 0;
    return;
  }
  if ((int64_t)hi - lo < kOvBitmapBits) {
    // ---- bitmap of [lo, hi]: clear, mark B, test A
    const int words = ((hi - lo) >> 5) + 1;
    uint32_t* bm = reinterpret_cast<uint32_t*>(table);
    for (int j = threadIdx.x; j < words; j += kOvThreads) bm[j] = 0u;
    __syncthreads();
    auto mark = [&](int32_t v) {
      if (v >= 0) atomicOr(&bm[(v - lo) >> 5], 1u << ((v - lo) & 31));
    };
    auto test = [&](int32_t v) {
      return (v >= lo && v <= hi) ? (int)((bm[(v - lo) >> 5] >> ((v - lo) & 31)) & 1u) : 0;
    };
    if (in_regs) {
#pragma unroll
      for (int m = 0; m < kReg; ++m) mark(rvb[m]);
    } else {
      for (int j = threadIdx.x; j < k; j += kOvThreads) mark(rb[j]);
    }
    __syncthreads();
    if (in_regs) {
#pragma unroll
      for (int m = 0; m < kReg; ++m) cnt += test(rva[m]);
    } else {
      for (int j = threadIdx.x; j < k; j += kOvThreads) cnt += test(ra[j]);
    }
    for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int w = 0; w < kOvThreads / 64; ++w) tot += wsum[w];
      counts[row] = tot;
    }
    return;
  }

  // ---- hash table
  const uint32_t mask = (uint32_t)slots - 1u;
  for (int j = threadIdx.x; j < slots; j += kOvThreads) table[j] = -1;
  // 8 entries per thread per pass (coalesced, all loads issued before use); A's
  // entries of the pass are loaded together with B's, ahead of the table barrier
  for (int base = 0; base < k; base += 8 * kOvThreads) {
    int32_t vb[8], va[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int j = base + m * kOvThreads + threadIdx.x;
      vb[m] = j < k ? rb[j] : -1;
      va[m] = j < k ? ra[j] : -1;
    }
    if (base == 0) __syncthreads();  // the table was cleared
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (vb[m] < 0) continue;
      uint32_t h = ov_hash((uint32_t)vb[m], mask);
      for (;;) {
        const int32_t old = atomicCAS(&table[h], -1, vb[m]);
        if (old == -1 || old == vb[m]) break;
        h = (h + 1u) & mask;
      }
    }
    if (base + 8 * kOvThreads >= k) {
      __syncthreads();  // every entry of B is in the table
      // A's entries of this (last) pass are already in registers
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (va[m] < 0) continue;
        uint32_t h = ov_hash((uint32_t)va[m], mask);
        for (;;) {
          const int32_t e = table[h];
          if (e == va[m]) {
            ++cnt;
            break;
          }
          if (e == -1) break;
          h = (h + 1u) & mask;
        }
      }
    }
  }
  // rows longer than 8 x 256 entries: A's entries before the last pass are probed
  // from memory, now that every entry of B is in the table
  const int last_pass = ((k - 1) / (8 * kOvThreads)) * (8 * kOvThreads);
  for (int j = threadIdx.x; j < last_pass; j += kOvThreads) {
    const int32_t v = ra[j];
    if (v < 0) continue;
    uint32_t h = ov_hash((uint32_t)v, mask);
    for (;;) {
      const int32_t e = table[h];
      if (e == v) {
        ++cnt;
        break;
      }
      if (e == -1) break;
      h = (h + 1u) & mask;
    }
  }
  for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < kOvThreads / 64; ++w) tot += wsum[w];
    counts[row] = tot;
  }
}

// Per-row e4m3fn quantisation of bf16 indexer inputs.  A group of G = 2^glog lanes
// takes one row: the row's absolute maximum (group reduction), scale = amax / 448 (1
// for an all-zero row), y = clamp(x / scale, +-448) in fp32 (correctly rounded
// division), and the code by the hardware OCP e4m3 conversion (round to nearest
// even, the first operand in the low byte).  VEC: 8 elements (16 B in, 8 B out) per
// lane access, for rows of a multiple of 8 elements on aligned buffers.
__device__ __forceinline__ float q_clamp(float v, float scale) { return fminf(fmaxf(v / scale, -448.f), 448.f); }

template <bool VEC>
__global__ __launch_bounds__(256) void quant_fp8_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int cols,
                                                             int glog, uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
  const int G = 1 << glog;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> glog;
  const int lane = threadIdx.x & (G - 1);
  if (row >= rows) return;  // whole groups leave together: the reduction stays inside a group
  const uint16_t* xr = x + row * (int64_t)cols;
  uint8_t* cr = codes + row * (int64_t)cols;
  constexpr int V = VEC ? 8 : 1;
  // VEC: the lane's first 16 B stay in registers for the second pass, so a row of at
  // most 8 G elements (one access per lane) is read from memory once
  uint4 first = make_uint4(0, 0, 0, 0);
  float amax = 0.f;
  for (int j = lane * V; j < cols; j += G * V) {
    if constexpr (VEC) {
      const uint4 v = *reinterpret_cast<const uint4*>(xr + j);
      if (j == lane * V) first = v;
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xFFFF0000u))));
    } else {
      amax = fmaxf(amax, fabsf(bf16_to_f32(xr[j])));
    }
  }
  for (int d = G >> 1; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  for (int j = lane * V; j < cols; j += G * V) {
    if constexpr (VEC) {
      const uint4 v = j == lane * V ? first : *reinterpret_cast<const uint4*>(xr + j);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t out[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int r = __builtin_amdgcn_cvt_pk_fp8_f32(q_clamp(__uint_as_float(w[2 * h] << 16), scale),
                                                q_clamp(__uint_as_float(w[2 * h] & 0xFFFF0000u), scale), 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(q_clamp(__uint_as_float(w[2 * h + 1] << 16), scale),
                                            q_clamp(__uint_as_float(w[2 * h + 1] & 0xFFFF0000u), scale), r, true);
        out[h] = (uint32_t)r;
      }
      *reinterpret_cast<uint2*>(cr + j) = make_uint2(out[0], out[1]);
    } else {
      cr[j] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(q_clamp(bf16_to_f32(xr[j]), scale), 0.f, 0, false) & 0xFF);
    }
  }
  if (lane == 0) scales[row] = scale;
}

}  // namespace

hipError_t launch_quantize_fp8_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, float* scales,
                                    hipStream_t st) {
  const bool vec = cols % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(codes) % 8 == 0;
  const int per_lane = vec ? 8 : 1;
  int glog = 0;  // lanes per row: enough for one pass over the row, at most a wave
  while (glog < 6 && ((1 << glog) * per_lane) < cols) ++glog;
  const int64_t rows_per_block = 256 >> glog;
  const dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block));
  if (vec)
    hipLaunchKernelGGL(quant_fp8_rows_kernel<true>, grid, dim3(256), 0, st, x, rows, cols, glog, codes, scales);
  else
    hipLaunchKernelGGL(quant_fp8_rows_kernel<false>, grid, dim3(256), 0, st, x, rows, cols, glog, codes, scales);
  return hipGetLastError();
}

hipError_t launch_index_overlap(const int32_t* a, const int32_t* b, int64_t n_rows, int k, int32_t* counts,
                                hipStream_t st) {
  int slots = 64;
  while (slots < 2 * k) slots <<= 1;  // load factor <= 1/2: every probe meets an empty slot
  const size_t lds = std::max((size_t)slots, (size_t)kOvBitmapBits / 32) * sizeof(int32_t);
  hipLaunchKernelGGL(idx_overlap_kernel, dim3((unsigned)n_rows), dim3(kOvThreads), lds, st, a, b, k, slots, counts);
  return hipGetLastError();
}

}  // namespace dsa
