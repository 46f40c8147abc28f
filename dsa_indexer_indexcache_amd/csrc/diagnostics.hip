// Cross-layer index overlap ([IDX] §8 metrics): for every row, the number of valid
// positions that two index tensors have in common.
//
// One workgroup per row.  Row B's valid positions go into an open-addressing hash
// table in LDS (linear probing, at least twice as many slots as entries, so every
// probe sequence ends at an empty slot); row A's valid positions are then looked up
// and the hits are summed.  Integer work throughout: the count is exact.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kOvThreads = 256;

__device__ __forceinline__ uint32_t ov_hash(uint32_t v, uint32_t mask) { return (v * 2654435761u) >> 7 & mask; }

__global__ __launch_bounds__(kOvThreads) void idx_overlap_kernel(const int32_t* __restrict__ a,
                                                                 const int32_t* __restrict__ b, int k, int slots,
                                                                 int32_t* __restrict__ counts) {
  extern __shared__ int32_t table[];
  __shared__ int32_t wsum[kOvThreads / 64];
  const int64_t row = blockIdx.x;
  const uint32_t mask = (uint32_t)slots - 1u;
  for (int j = threadIdx.x; j < slots; j += kOvThreads) table[j] = -1;
  // 8 entries per thread per pass (coalesced, all loads issued before use); A's
  // entries of the pass are loaded together with B's, ahead of the table barrier
  const int32_t* rb = b + row * (int64_t)k;
  const int32_t* ra = a + row * (int64_t)k;
  int cnt = 0;
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

}  // namespace

hipError_t launch_index_overlap(const int32_t* a, const int32_t* b, int64_t n_rows, int k, int32_t* counts,
                                hipStream_t st) {
  int slots = 64;
  while (slots < 2 * k) slots <<= 1;  // load factor <= 1/2: every probe meets an empty slot
  hipLaunchKernelGGL(idx_overlap_kernel, dim3((unsigned)n_rows), dim3(kOvThreads), slots * sizeof(int32_t), st, a, b,
                     k, slots, counts);
  return hipGetLastError();
}

}  // namespace dsa
